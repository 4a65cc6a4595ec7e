"""Throughput of the quantized linear layer on one MI355X.

Primary line (value): qgemv weight GB/s at M = 1 on a Llama-2-7B-shaped decode
step, GPTQ 4-bit, group size 128, act-order. One step = one token through the
linear layers of 32 decoder layers; each layer has q, k, v, o (4096 -> 4096),
gate, up (4096 -> 11008) and down (11008 -> 4096). All 224 packed matrices are
distinct buffers resident in HBM (3.36 GB), so the 256 MB Infinity Cache cannot
serve repeated weights. q, k, v read the same input and so do gate and up
(quantized against the same input, they share the act-order permutation):
each of those sets is one grouped launch, 4 launches per layer (--no-group: 7).
The step is captured in a HIP graph and replayed.

Secondary (qgemm): dequant-GEMM TFLOP/s at M = 2048 on the Llama-2-13B MLP
shape 5120 -> 13824, GPTQ 4-bit, group size 128, act-order.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, decimal GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix throughput
METRIC = "qgemv weight GB/s (% of HBM peak) at M=1; dequant-GEMM TFLOP/s at M=2048"
N_LAYERS = 32
LAYER_MIX = ((0, 4), (1, 2), (2, 1))   # (index into the 7B decode shapes, matrices per layer)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--gemm-iters", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-group", action="store_true", help="one qgemv launch per matrix (no grouped q/k/v, gate/up)")
    ap.add_argument("--no-gemm", action="store_true", help="skip the M = 2048 qgemm measurements")
    ap.add_argument("--no-lora", action="store_true", help="skip the on-the-fly LoRA update timings")
    ap.add_argument("--no-kv", action="store_true", help="skip the KV-cache codec timings")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config decode points (7B at M = 4, 16; EXL2 at M = 1, 8; 70B at M = 1, 16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy a MIB-MiB buffer 3 times (a known-size kernel for HBM counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Call:
    """One C entry point with its arguments marshalled once: layouts become
    struct pointers, tensors device pointers (workspaces add their size)."""

    def __init__(self, fn, *args, ws_last=True):
        self.fn = fn
        self.keep = args  # keeps layouts and tensors alive
        out = []
        for a in args:
            if hasattr(a, "ref"):
                out.append(a.ref)
            elif hasattr(a, "data_ptr"):
                out.append(a.data_ptr())
            else:
                out.append(a)
        if ws_last:  # (..., workspace, stream) -> (..., workspace, workspace bytes, stream)
            out.insert(len(out) - 1, args[-2].numel())
        self.args = tuple(out)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"launch failed with status {st}")


def Launch(fn, layout, x, M, qweight, scales, zeros, perm, y, ws, stream):
    """A qlinear_qgemv / qlinear_qgemm call."""
    return Call(fn, layout, x, M, qweight, scales, zeros, perm, y, ws, stream)


def decode_groups(mats, grouped):
    """The step's launches in layer order: per layer [q, k, v], [o], [gate,
    up], [down] when grouped (the matrices of a launch share x and perm),
    else one launch per matrix."""
    out, i = [], 0
    per_layer = sum(c for _, c in LAYER_MIX)
    while i < len(mats):
        layer = mats[i:i + per_layer]
        parts = [layer[0:3], layer[3:4], layer[4:6], layer[6:7]] if grouped else [[m] for m in layer]
        out += [dict(shape=p[0]["shape"], mats=p) for p in parts]
        i += per_layer
    return out


def group_call(lib, dq, shapes, xs, ys, g, ws, sh):
    """A qlinear_qgemv call for one matrix, a qlinear_qgemv_grouped call for several."""
    import ctypes
    si, ms = g["shape"], g["mats"]
    L = shapes[si]["L"]
    if len(ms) == 1:
        m = ms[0]
        return Call(lib.qlinear_qgemv, L, xs[si], 1, m["qw"], m["sc"], m["zr"], m["pm"], ys[si][0], ws, sh)
    arr = lambda ts: (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    call = Call(lib.qlinear_qgemv_grouped, L, xs[si], 1, len(ms), arr([m["qw"] for m in ms]),
                arr([m["sc"] for m in ms]), arr([m["zr"] for m in ms]), ms[0]["pm"], arr(ys[si][:len(ms)]), ws, sh)
    call.hold = ms
    return call


def spin_cycles(torch, stream, ms):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `ms`."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe = 1 << 22
    torch.cuda._sleep(probe)  # first launch loads the kernel
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(probe)
    b.record(stream)
    torch.cuda.synchronize()
    return int(probe * ms / max(a.elapsed_time(b), 1e-3))


def launch_bytes(layout, M, zeros=True, perm=True, count=1):
    """Algorithmic HBM bytes of one decode launch over `count` matrices of one
    layout, in the byte model of the metric: per matrix its weight bytes
    (codes at b bits, float16 scales, zero points at 4 bits) and its float16
    result; shared by the matrices: the float16 activations and the int32
    act-order permutation. `value` counts the weight bytes alone."""
    bits = layout.bits.astype(np.int64)
    K, N, G = layout.K, layout.N, layout.groups
    codes = int((bits * layout.group_size).sum()) * N // 8
    per = codes + G * N * 2 + (G * N // 2 if zeros else 0) + M * N * 2
    return count * per + M * K * 2 + (K * 4 if perm else 0)


def time_graph(torch, stream, fn, n):
    """Microseconds per call of fn(0 .. n-1), captured back to back in one
    HIP graph on `stream` and replayed (once untimed) between two events on
    that stream, as the decode step itself is replayed."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    del g
    return us


# The kernel that runs every launch of the M = 1 decode step.
DECODE_KERNEL = "qgemv_row_kernel (M=1, 4-bit)"

# Files whose code makes up a measured kernel; recorded counter data is valid
# only for the exact sources it was taken on.
ROW_KERNEL_SOURCES = ("qgemv_m1.hpp", "qgemv_row.hip", "qgemv_stream.hpp", "qlinear_device.hpp")
GEMM_KERNEL_SOURCES = ("qgemm.hip", "mfma_frag.hpp", "qlinear_kernels.hpp", "qlinear_device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemv_row_llama7b_decode_traffic.txt")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemm_llama13b_mlp_prefill_counters.txt")


def sources_digest(sources):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "dequant_matmul_gptq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def row_kernel_digest():
    return sources_digest(ROW_KERNEL_SOURCES)


def gemm_kernel_digest():
    return sources_digest(GEMM_KERNEL_SOURCES)


def _recorded(path, digest):
    """HBM bytes per launch from a committed counter summary (FETCH_SIZE plus
    WRITE_SIZE, each scaled by the copy-kernel calibration); None when the
    file is missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != digest:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def recorded_traffic():
    """Single-row qgemv: HBM bytes per launch averaged over the step's launches."""
    return _recorded(TRAFFIC_FILE, row_kernel_digest())


def recorded_gemm_traffic():
    """qgemm gemm_kernel on the 13B MLP prefill shape: HBM-side bytes per launch."""
    return _recorded(GEMM_TRAFFIC_FILE, gemm_kernel_digest())


def setup_decode(torch, dq, wl, dev):
    """Pack the three 7B decode shapes once, then clone them into 32 layers."""
    shapes = []
    for spec in wl.LLAMA7B_DECODE:
        inp = wl.generate(spec, M=1)
        L = dq.Layout(spec.K, spec.N, spec.group_size, inp.bits)
        qw = dq.pack_weights(L, torch.from_numpy(inp.q).to(dev))
        sc = torch.from_numpy(inp.scales).to(dev)
        zr = torch.from_numpy(inp.zeros).to(dev)
        pm = torch.from_numpy(inp.perm).to(dev)
        shapes.append(dict(spec=spec, inp=inp, L=L, qw=qw, sc=sc, zr=zr, pm=pm))
    torch.cuda.synchronize()
    mats = []
    for _ in range(N_LAYERS):
        for si, count in LAYER_MIX:
            s = shapes[si]
            for _ in range(count):
                mats.append(dict(shape=si, qw=s["qw"].clone(), sc=s["sc"].clone(), zr=s["zr"].clone(),
                                 pm=s["pm"].clone()))
    torch.cuda.synchronize()
    return shapes, mats


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs the layer on one GPU; splitting it across GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_matmul_gptq_amd as dq
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = dq.lib()
    # All work runs on one side stream (default priority): graph capture
    # cannot use the legacy default stream.
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    sh = stream.cuda_stream

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {n} bytes read and written")
        del src, dst

    # ---------------------------------------------------------------- decode setup
    t0 = time.time()
    shapes, mats = setup_decode(torch, dq, wl, dev)
    wbytes = [wl.weight_bytes(s["spec"]) for s in shapes]
    step_bytes = sum(wbytes[m["shape"]] for m in mats)
    ws = dq.qgemv_workspace(shapes[2]["L"], dev)  # K = 11008 covers every shape in the step
    xs = [torch.from_numpy(s["inp"].x[:1].copy()).to(dev) for s in shapes]
    ys = [[torch.empty((1, s["spec"].N), dtype=torch.float16, device=dev) for _ in range(3)] for s in shapes]
    groups = decode_groups(mats, not args.no_group)
    launches = [group_call(lib, dq, shapes, xs, ys, g, ws, sh) for g in groups]
    log(f"decode setup {time.time() - t0:.1f}s: {len(mats)} matrices in {len(launches)} launches, "
        f"{step_bytes / 1e9:.3f} GB per step")

    def step():
        for ln in launches:
            ln()

    # Correctness at timing time: each kind of launch exactly as the step
    # runs it (grouped launches included) against the oracle, with both
    # tolerances of the layer. The matrices of a shape are copies of one
    # packed matrix, so every output of a launch has the same reference.
    import oracle
    checked = set()
    for g, ln in zip(groups, launches):
        kind = (g["shape"], len(g["mats"]))
        if kind in checked:
            continue
        checked.add(kind)
        ln()
        torch.cuda.synchronize()
        s = shapes[g["shape"]]
        inp = s["inp"]
        ref = oracle.qlinear(inp.x[:1], inp.q, inp.scales, inp.zeros, inp.bits, s["spec"].group_size, inp.perm)
        for y in ys[g["shape"]][:len(g["mats"])]:
            d = y.float().cpu().numpy().astype(np.float64) - ref
            rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
            mx = float(np.abs(d).max() / np.abs(ref).max())
            if not (rel <= 1e-3 and mx <= 1e-2):
                raise RuntimeError(f"qgemv disagrees with the oracle on {kind[1]} x {s['spec'].name}: "
                                   f"rel_fro={rel:.2e} max_rel={mx:.2e}")
    log(f"decode outputs of all {len(checked)} launch kinds match the oracle (rel_fro <= 1e-3, max <= 1e-2)")

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us -> {value:.0f} GB/s ({value / HBM_PEAK_GBS:.1%} of HBM peak)")

    # Per-launch duration of each kind of launch in the step: >= 256 launches
    # of that kind (cycling through its distinct matrices, so the weights
    # come from HBM) captured back to back in one HIP graph and replayed
    # between two events on the launch stream, as the step is.
    spin = spin_cycles(torch, stream, 50.0)
    per_kind = []
    tot_bytes, tot_us, n_step = 0, 0.0, 0
    kinds = {}
    for g, ln in zip(groups, launches):
        kinds.setdefault((g["shape"], len(g["mats"])), []).append(ln)
    for (si, cnt), calls in kinds.items():
        n = -(-256 // len(calls)) * len(calls)
        us = time_graph(torch, stream, lambda i: calls[i % len(calls)](), n)
        ab = launch_bytes(shapes[si]["L"], 1, count=cnt)
        gbs = ab / (us * 1e-6) / 1e9
        sp = shapes[si]["spec"]
        per_kind.append(dict(launch=f"{cnt} x {sp.K}x{sp.N}", algorithmic_bytes=ab, launches=n,
                             avg_us=round(us, 3), gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4)))
        # weight the kinds as the step does
        tot_bytes += ab * len(calls)
        tot_us += us * len(calls)
        n_step += len(calls)
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    log(f"{DECODE_KERNEL} per launch: avg {tot_us / n_step:.2f} us, {achieved:.0f} GB/s "
        f"(kinds sum to {tot_us:.0f} us per step vs the step's {ms_step * 1e3:.0f} us); " +
        ", ".join(f"{p['launch']}: {p['avg_us']} us {p['gbs']} GB/s" for p in per_kind))
    traffic = recorded_traffic()
    refs = reference_points(torch, lib, stream, [p["algorithmic_bytes"] for p in per_kind])
    for p, f in zip(per_kind, refs["read_floor"]):
        p["read_floor_us"] = f["best_us"]
        p["frac_of_read_floor"] = round(f["best_us"] / p["avg_us"], 4)
    log(f"reference points: empty kernel {refs['empty_kernel_us']} us; read floor " +
        ", ".join(f"{f['bytes']} B: {f['best_us']} us ({f['read_gbs']} GB/s)" for f in refs["read_floor"]))

    gemm = None if args.no_gemm else bench_gemm(args, torch, dq, wl, oracle, lib, dev, stream)
    gemm_mixed = None if args.no_gemm else bench_gemm_mixed(args, torch, dq, wl, oracle, lib, dev, stream)
    configs = None if args.no_configs else bench_configs(torch, dq, wl, lib, dev, stream, spin)
    lora = None if args.no_lora else bench_lora(torch, lib, dev, stream, spin)
    kv = None if args.no_kv else bench_kv(torch, lib, dev, stream, spin)

    # ---------------------------------------------------------------- oracle on the host
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(shapes[1]["inp"], wbytes[1])
        log(f"oracle on host: {cpu['value']} GB/s with {cpu['cores']} threads, "
            f"{cpu['single_thread_value']} GB/s on one")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-2-7B-shaped decode, GPTQ 4-bit g128 act-order, M=1: 32 layers x "
                        "(4 x 4096->4096, 2 x 4096->11008, 1 x 11008->4096), weights resident in HBM; "
                        + ("q/k/v and gate/up as grouped launches" if not args.no_group else "one launch per matrix"),
            "M": 1,
            "matrices_per_step": len(mats),
            "launches_per_step": len(launches),
            "weight_bytes_per_step": step_bytes,
            "hbm_peak_gbs": HBM_PEAK_GBS,
            "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "launch": "hip_graph" if graph is not None else "eager",
            "accumulate": "fp32",
        },
        "roofline": {
            "kernel": DECODE_KERNEL,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(tot_us / n_step, 3),
            "launch_kinds_us_per_step": round(tot_us, 1),
            "algorithmic_bytes_per_launch": round(tot_bytes / n_step),
            "per_launch_kind": per_kind,
        },
        "reference_points": refs,
        "decode_configs": configs,
        "lora": lora,
        "kv_codec": kv,
        "cpu_baseline": cpu,
        "qgemm": gemm,
        "qgemm_mixed": gemm_mixed,
    }
    print(json.dumps(out), flush=True)


def reference_points(torch, lib, stream, sizes):
    """Two floors that frame the per-launch numbers, timed like the launches
    (>= 256 calls captured in one HIP graph, replayed between two events):
    the back-to-back period of an empty kernel (torch.cuda._sleep(0)), and for
    each launch size S the streaming-read floor: qlinear_read_floor reading S
    bytes, cycling over distinct buffers that total >= 1 GiB (so the
    Infinity Cache cannot serve them), best over a few launch shapes (16-byte
    loads in flight per thread, workgroups). No kernel that must read S
    bytes runs faster than the fastest plain read of them."""
    sh = stream.cuda_stream
    empty = time_graph(torch, stream, lambda i: torch.cuda._sleep(0), 256)
    sink = torch.zeros(4, dtype=torch.int32, device=stream.device)
    floors = []
    for size in sizes:
        nbytes = size // 16 * 16
        nbuf = max(2, -(-(1 << 30) // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=stream.device) for _ in range(nbuf)]
        for b_ in bufs:
            b_.fill_(1)
        shapes_tried = []
        for loads in (4, 8, 16):
            one_pass = -(-nbytes // (256 * 16 * loads))
            for grid in sorted({one_pass, 256, 512, 1024, 2048}):
                if grid > one_pass:
                    continue
                def call(i, loads=loads, grid=grid):
                    st = lib.qlinear_read_floor(bufs[i % nbuf].data_ptr(), nbytes, loads, grid, 0x9E3779B9,
                                                sink.data_ptr(), sh)
                    if st != 0:
                        raise RuntimeError(f"qlinear_read_floor failed with status {st}")
                us = time_graph(torch, stream, call, max(256, nbuf))
                shapes_tried.append({"loads_per_thread": loads, "workgroups": grid, "us": round(us, 3)})
        best = min(shapes_tried, key=lambda t: t["us"])
        floors.append({"bytes": nbytes, "best_us": best["us"], "read_gbs": round(nbytes / (best["us"] * 1e-6) / 1e9, 1),
                       "best_shape": best, "tried": shapes_tried})
        del bufs
    return {"empty_kernel_us": round(empty, 3), "read_floor": floors}


def bench_configs(torch, dq, wl, lib, dev, stream, spin):
    """qgemv on every (layer, M) of the decode configs that the step does not
    cover: the 7B shapes at M = 4 and 16, EXL2 4.0 bpw at M = 1 and 8, the 70B
    EXL2 2.5 bpw pair at M = 1 and 16; and the EXL2 layers again with
    two-level scales (4-bit scale codes and a float16 maximum per output,
    qlinear_qgemv_qscale). Per point, >= 256 calls back to back behind a spin
    kernel, cycling through distinct weight copies totalling >= 1 GiB (so the
    Infinity Cache cannot serve them), between two events on the launch
    stream; GB/s counts the weight bytes (codes, scales, zeros; two-level:
    codes, scale codes, maximum scales)."""
    sh = stream.cuda_stream
    points = []

    def time_point(name, M, wbytes, calls, scales_kind):
        for c in calls[:4]:
            c()
        ncopy = len(calls)
        n = max(256, ncopy)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        e0.record(stream)
        for i in range(n):
            calls[i % ncopy]()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        points.append({"workload": name, "M": M, "scales": scales_kind, "us_per_call": round(us, 2),
                       "weight_bytes": wbytes, "weight_gbs": round(wbytes / (us * 1e-6) / 1e9, 1)})
        log(f"config point {name} M={M} ({scales_kind} scales): {us:.2f} us, {points[-1]['weight_gbs']} GB/s")

    plan = [(s, (4, 16)) for s in wl.LLAMA7B_DECODE] + [(wl.EXL2_MIXED, (1, 8))] + \
        [(s, (1, 16)) for s in wl.LLAMA70B_EXL2]
    for spec, Ms in plan:
        inp = wl.generate(spec, M=max(Ms))
        L = dq.Layout(spec.K, spec.N, spec.group_size, inp.bits)
        qw = dq.pack_weights(L, torch.from_numpy(inp.q).to(dev))
        sc = torch.from_numpy(inp.scales).to(dev)
        zr = None if inp.zeros is None else torch.from_numpy(inp.zeros).to(dev)
        pm = torch.from_numpy(inp.perm).to(dev)
        ws = dq.qgemv_workspace(L, dev)
        wbytes = wl.weight_bytes(spec)
        ncopy = max(2, -(-(1 << 30) // wbytes))
        copies = [(qw.clone(), sc.clone(), None if zr is None else zr.clone()) for _ in range(ncopy)]
        for M in Ms:
            x = torch.from_numpy(inp.x[:M].copy()).to(dev)
            y = torch.empty((M, spec.N), dtype=torch.float16, device=dev)
            time_point(spec.name, M, wbytes,
                       [Launch(lib.qlinear_qgemv, L, x, M, q, c, z, pm, y, ws, sh) for q, c, z in copies], "fp16")
        del copies
        if spec.symmetric:
            codes, smax = wl.two_level_scales(spec)
            qs = dq.pack_qscale(torch.from_numpy(codes).to(dev))
            qsm = torch.from_numpy(smax).to(dev)
            wbytes = wl.weight_bytes_two_level(spec)
            ncopy = max(2, -(-(1 << 30) // wbytes))
            copies = [(qw.clone(), qs.clone(), qsm.clone()) for _ in range(ncopy)]
            for M in Ms:
                x = torch.from_numpy(inp.x[:M].copy()).to(dev)
                y = torch.empty((M, spec.N), dtype=torch.float16, device=dev)
                time_point(spec.name, M, wbytes,
                           [Call(lib.qlinear_qgemv_qscale, L, x, M, q, a, b, pm, None, y, ws, sh) for q, a, b in copies],
                           "two-level")
            del copies
        del qw
    return points


# On-the-fly LoRA update delta = s (x A) B (float32 [M][N]) at rank 16 on the
# 7B decode shapes and the 13B MLP prefill shape.
LORA_POINTS = [(1, 4096, 4096, 16), (1, 4096, 11008, 16), (1, 11008, 4096, 16), (2048, 5120, 13824, 16)]


def lora_bytes(M, K, N, r):
    """Algorithmic HBM bytes of one qlinear_lora_delta call: x, A and B read
    once (float16), delta written once (float32); the partial sums in the
    workspace are the kernels' own traffic."""
    return 2 * M * K + 2 * K * r + 2 * r * N + 4 * M * N


def bench_lora(torch, lib, dev, stream, spin):
    """qlinear_lora_delta (shrink + expand launches) per call, >= 256 calls
    back to back behind a spin kernel (20 at M = 2048) between two events on
    the launch stream, against the HBM roofline of its algorithmic bytes."""
    sh = stream.cuda_stream
    points = []
    for M, K, N, r in LORA_POINTS:
        rng = np.random.default_rng(M + K + N + r)
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float16)).to(dev)
        A = torch.from_numpy((rng.standard_normal((K, r)) / np.sqrt(K)).astype(np.float16)).to(dev)
        B = torch.from_numpy(rng.standard_normal((r, N)).astype(np.float16)).to(dev)
        d = torch.empty((M, N), dtype=torch.float32, device=dev)
        need = ctypes.c_size_t()
        assert lib.qlinear_lora_workspace_bytes(M, K, r, ctypes.byref(need)) == 0
        ws = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)

        def call():
            st = lib.qlinear_lora_delta(x.data_ptr(), M, K, A.data_ptr(), r, B.data_ptr(), N, 0.5, 0, d.data_ptr(),
                                        ws.data_ptr(), ws.numel(), sh)
            if st != 0:
                raise RuntimeError(f"qlinear_lora_delta failed with status {st}")

        for _ in range(4):
            call()
        n = 20 if M > 16 else 256
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin)
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        nb = lora_bytes(M, K, N, r)
        gbs = nb / (us * 1e-6) / 1e9
        points.append({"M": M, "K": K, "N": N, "rank": r, "us_per_call": round(us, 2), "algorithmic_bytes": nb,
                       "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        log(f"lora M={M} {K}->{N} rank {r}: {us:.2f} us, {gbs:.1f} GB/s")
    return points


# KV-cache codec points: one layer's key (or value) cache of a 70B-class
# model at 32K tokens (8 key/value heads x 32768 tokens, head dimension 128),
# per (bits, block size).
KV_ROWS, KV_D = 8 * 32768, 128
KV_POINTS = [(4, 128), (6, 128), (8, 128), (4, 32)]


def kv_bytes(elements, bits, group):
    """Algorithmic HBM bytes of one codec call over `elements` values: the
    float16 values on one side, the codes and block scales on the other."""
    return elements * 2 + elements * bits // 8 + elements // group * 2


def bench_kv(torch, lib, dev, stream, spin):
    """qlinear_kv_quant and qlinear_kv_dequant on KV_ROWS x KV_D values,
    >= 64 calls back to back behind a spin kernel, cycling through distinct
    buffers of >= 1 GiB in all (so the Infinity Cache cannot serve them),
    between two events on the launch stream, against the HBM roofline."""
    sh = stream.cuda_stream
    E = KV_ROWS * KV_D
    rng = np.random.default_rng(21)
    x0 = torch.from_numpy((rng.standard_normal((KV_ROWS, KV_D)) *
                           rng.uniform(0.05, 4.0, size=(KV_ROWS, 1))).astype(np.float16)).to(dev)
    points = []
    for bits, group in KV_POINTS:
        nb = kv_bytes(E, bits, group)
        ncopy = max(2, -(-(1 << 30) // nb))
        xs = [x0.clone() for _ in range(ncopy)]
        cs = [torch.empty(E * bits // 32, dtype=torch.int32, device=dev) for _ in range(ncopy)]
        ss = [torch.empty(E // group, dtype=torch.float16, device=dev) for _ in range(ncopy)]
        for quant in (True, False):
            def call(i):
                j = i % ncopy
                if quant:
                    st = lib.qlinear_kv_quant(xs[j].data_ptr(), KV_ROWS, KV_D, bits, group, cs[j].data_ptr(),
                                              ss[j].data_ptr(), sh)
                else:
                    st = lib.qlinear_kv_dequant(cs[j].data_ptr(), ss[j].data_ptr(), KV_ROWS, KV_D, bits, group,
                                                xs[j].data_ptr(), sh)
                if st != 0:
                    raise RuntimeError(f"kv codec failed with status {st}")

            for i in range(ncopy):
                call(i)
            n = max(64, ncopy)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(spin)
            e0.record(stream)
            for i in range(n):
                call(i)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / n
            gbs = nb / (us * 1e-6) / 1e9
            points.append({"op": "quant" if quant else "dequant", "bits": bits, "group": group, "rows": KV_ROWS,
                           "D": KV_D, "us_per_call": round(us, 2), "algorithmic_bytes": nb, "gbs": round(gbs, 1),
                           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                           "bytes_per_element": bits / 8 + 2 / group})
            log(f"kv {'quant' if quant else 'dequant'} Q{bits} G={group} {KV_ROWS}x{KV_D}: {us:.2f} us, "
                f"{gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
        del xs, cs, ss
    return points


def bench_gemm(args, torch, dq, wl, oracle, lib, dev, stream):
    """qgemm on the Llama-2-13B MLP prefill shape, M = 2048, checked against
    the oracle on sampled rows, then timed over --gemm-iters calls."""
    sh = stream.cuda_stream
    spec = wl.PREFILL_13B
    inp = wl.generate(spec)
    L = dq.Layout(spec.K, spec.N, spec.group_size, inp.bits)
    qw = dq.pack_weights(L, torch.from_numpy(inp.q).to(dev))
    sc = torch.from_numpy(inp.scales).to(dev)
    zr = torch.from_numpy(inp.zeros).to(dev)
    pm = torch.from_numpy(inp.perm).to(dev)
    x = torch.from_numpy(inp.x).to(dev)
    M = x.shape[0]
    y = torch.empty((M, spec.N), dtype=torch.float16, device=dev)
    gws = torch.empty(dq.qgemm_workspace_bytes(L, M), dtype=torch.uint8, device=dev)
    gl = Launch(lib.qlinear_qgemm, L, x, M, qw, sc, zr, pm, y, gws, sh)
    rows = np.arange(0, M, 64)
    gl()
    torch.cuda.synchronize()
    ref = oracle.qlinear(inp.x[rows], inp.q, inp.scales, inp.zeros, inp.bits, spec.group_size, inp.perm)
    d = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy() - ref
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
    if rel > 1e-3:
        raise RuntimeError(f"qgemm disagrees with the oracle: rel_fro={rel:.2e}")
    for _ in range(3):
        gl()
    flops = 2.0 * M * spec.K * spec.N
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for _ in range(args.gemm_iters):
        gl()
    g1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = g0.elapsed_time(g1) / args.gemm_iters
    tflops = flops / (gemm_ms * 1e-3) / 1e12
    log(f"qgemm M={M}: {gemm_ms * 1e3:.1f} us per call -> {tflops:.1f} TFLOP/s "
        f"({tflops / MFMA_F16_PEAK_TFLOPS:.1%} of fp16 MFMA peak), rel_fro={rel:.1e}")
    return {
        "workload": "Llama-2-13B MLP prefill 5120->13824, GPTQ 4-bit g128 act-order, M=2048",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "ms_per_call": round(gemm_ms, 5),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": recorded_gemm_traffic(),
            "timed": "whole qlinear_qgemm call: act-order gather kernel + gemm_kernel",
        },
    }


def bench_gemm_mixed(args, torch, dq, wl, oracle, lib, dev, stream):
    """qgemm on the EXL2 4.0 bpw 4096->11008 layer (four runs of widths 6, 5,
    4 and 3: the kernel that dequantizes into LDS) at M = 2048, with float16
    scales and with two-level scales; each checked against the oracle on
    sampled rows, then timed over --gemm-iters calls."""
    sh = stream.cuda_stream
    spec = wl.EXL2_MIXED
    M = 2048
    inp = wl.generate(spec, M=M)
    L = dq.Layout(spec.K, spec.N, spec.group_size, inp.bits)
    qw = dq.pack_weights(L, torch.from_numpy(inp.q).to(dev))
    pm = torch.from_numpy(inp.perm).to(dev)
    x = torch.from_numpy(inp.x).to(dev)
    y = torch.empty((M, spec.N), dtype=torch.float16, device=dev)
    gws = torch.empty(dq.qgemm_workspace_bytes(L, M), dtype=torch.uint8, device=dev)
    rows = np.arange(0, M, 128)
    codes, smax = wl.two_level_scales(spec)
    sc = torch.from_numpy(inp.scales).to(dev)
    qs = dq.pack_qscale(torch.from_numpy(codes).to(dev))
    qsm = torch.from_numpy(smax).to(dev)
    cases = [
        ("fp16", Launch(lib.qlinear_qgemm, L, x, M, qw, sc, None, pm, y, gws, sh),
         lambda: oracle.qlinear(inp.x[rows], inp.q, inp.scales, None, inp.bits, spec.group_size, inp.perm)),
        ("two-level", Call(lib.qlinear_qgemm_qscale, L, x, M, qw, qs, qsm, pm, None, y, gws, sh),
         lambda: oracle.qlinear_qscale(inp.x[rows], inp.q, oracle.qscale_pack(codes), smax, inp.bits, spec.group_size,
                                       inp.perm)),
    ]
    flops = 2.0 * M * spec.K * spec.N
    out = []
    for kind, gl, ref_fn in cases:
        gl()
        torch.cuda.synchronize()
        ref = ref_fn()
        d = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy() - ref
        rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
        if rel > 1e-3 or float(np.abs(d).max()) > 1e-2 * float(np.abs(ref).max()):
            raise RuntimeError(f"mixed-width qgemm ({kind} scales) disagrees with the oracle: rel_fro={rel:.2e}")
        for _ in range(3):
            gl()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(args.gemm_iters):
            gl()
        g1.record(stream)
        torch.cuda.synchronize()
        ms = g0.elapsed_time(g1) / args.gemm_iters
        tflops = flops / (ms * 1e-3) / 1e12
        log(f"qgemm EXL2 4.0 bpw M={M} ({kind} scales): {ms * 1e3:.1f} us per call -> {tflops:.1f} TFLOP/s "
            f"({tflops / MFMA_F16_PEAK_TFLOPS:.1%} of fp16 MFMA peak), rel_fro={rel:.1e}")
        out.append({"workload": f"{spec.name}, M={M}", "scales": kind, "value": round(tflops, 2),
                    "unit": "TFLOP/s", "ms_per_call": round(ms, 5),
                    "frac_of_mfma_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)})
    return out


def cpu_baseline(inp, wbytes):
    """The float64 oracle timed on the host on one 4096 -> 11008 layer at
    M = 1 (dequantize, gather, matmul): the median of 3 runs of about 3 s on
    all the BLAS threads, then one run on a single thread."""
    import statistics

    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    sp = inp.spec
    x = inp.x[:1]

    def run(seconds):
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.qlinear(x, inp.q, inp.scales, inp.zeros, inp.bits, sp.group_size, inp.perm)
            n += 1
            el = time.perf_counter() - t0
            if el > seconds or n >= 100:
                return wbytes * n / el / 1e9, n, el

    runs = [run(3.0) for _ in range(3)]
    med = statistics.median(r[0] for r in runs)
    with threadpool_limits(limits=1):
        one = run(3.0)
    return {
        "value": round(med, 4),
        "unit": "GB/s",
        "cores": blas_threads,
        "kind": "oracle",
        "single_thread_value": round(one[0], 4),
        "runs_gbs": [round(r[0], 4) for r in runs],
        "sample": f"oracle.qlinear on the {sp.K}x{sp.N} GPTQ-4bit layer at M=1, float64 dequantize + gather + "
                  f"BLAS matmul: median of 3 runs ({', '.join(f'{r[1]} calls in {r[2]:.1f} s' for r in runs)}) "
                  f"with the matmul on {blas_threads} BLAS threads (elementwise steps single-threaded), then "
                  f"{one[1]} calls in {one[2]:.1f} s on 1 thread; host has {os.cpu_count()} logical CPUs, "
                  f"{len(os.sched_getaffinity(0))} in this process's affinity mask",
    }


if __name__ == "__main__":
    main()
