"""Guard bands around outputs and workspaces: every kernel path writes only
inside y (its M x N float16 elements) and inside the workspace size it
reports. Each buffer sits between two 4 KiB bands of a known byte pattern
that must survive the call; y also starts out filled with the pattern, and
every element of it must be overwritten (it is checked against the oracle)."""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import GpuLayer, Guarded, assert_close, say

pytestmark = pytest.mark.gpu

MIXED = [6, 6, 5, 5, 4, 4, 4, 3, 3, 2, 8]


def _inputs(bits, gs, N, M, seed, zeros):
    rng = np.random.default_rng(seed)
    bits = np.asarray(bits, np.uint8)
    K = gs * len(bits)
    spec = wl.LayerSpec(f"guard-{K}x{N}", K, N, gs, ((4, 1.0),), not zeros, True, (M,))
    perm = rng.permutation(K).astype(np.int32)
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    z = rng.integers(0, 16, size=(len(bits), N), dtype=np.uint8) if zeros else None
    s = rng.uniform(0.005, 0.02, size=(len(bits), N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    return wl.LayerInputs(spec, bits, q, z, s, perm, x)


CASES = [
    ("qgemv", [4] * 11, 520, 1),          # single-launch kernel
    ("qgemv", [4] * 11, 520, 4),          # single-launch kernel, 4 rows
    ("qgemv", MIXED, 520, 1),             # several widths at M = 1
    ("qgemv", MIXED, 520, 2),
    ("qgemv", MIXED, 392, 8),             # matrix-core decode, gather kernel + workspace
    ("qgemv", [6, 5, 4, 4, 3, 3], 392, 3),   # matrix-core decode, one launch (gather in LDS)
    ("qgemv", [3] * 40, 776, 16),
    ("qgemm", [4] * 11, 520, 300),        # prefill, one width
    ("qgemm", MIXED, 392, 130),           # prefill, several widths (LDS dequant)
    ("qgemm", [3] * 128 + [2] * 128, 264, 70),   # prefill, two long runs on a small grid (LDS dequant, K in slices)
    ("qgemm", [4] * 128, 392, 40),              # prefill, one width on a small grid (K in 8 slices)
]


@pytest.mark.parametrize("op,bits,N,M", CASES, ids=[f"{c[0]}-{len(c[1])}blk-N{c[2]}-M{c[3]}" for c in CASES])
def test_writes_stay_inside_y_and_workspace(op, bits, N, M):
    say(f"guard bands {op} blocks={len(bits)} N={N} M={M}")
    inp = _inputs(bits, 32, N, M, seed=len(bits) * 13 + N + M, zeros=M % 2 == 0)
    lay = GpuLayer(inp)
    yb = Guarded(M * N * 2, lay.dev)
    y = yb.view(torch.float16, (M, N))
    nws = dq.qgemv_workspace_bytes(lay.layout) if op == "qgemv" else dq.qgemm_workspace_bytes(lay.layout, M)
    wb = Guarded(max(nws, 16), lay.dev, fill=0xFF)   # the workspace starts as garbage (NaN patterns)
    ws = wb.bytes()
    x = lay.x(inp.x)
    if op == "qgemv":
        dq.qgemv(lay.layout, x, lay.qweight, lay.scales, lay.zeros, lay.perm, ws, y=y)
    else:
        dq.qgemm(lay.layout, x, lay.qweight, lay.scales, lay.zeros, lay.perm, ws, y=y)
    assert yb.intact(), "a write landed outside y"
    assert wb.intact(), "a write landed outside the workspace"
    ref = oracle.qlinear(inp.x, inp.q, inp.scales, inp.zeros, inp.bits, 32, inp.perm)
    assert_close(y, ref, f"{op} M={M}")


def test_run_by_run_writes_stay_inside_y_and_workspace():
    """Prefill run by run (two runs of 8192 rows, 16 x 16 tiles of 256 x 256,
    M ragged): the float32 partial sums sit in the workspace after the
    gathered activations. y starts as NaN bytes, so every element must come
    out finite; the oracle checks every 64th row and the last."""
    bits, N, M = [3] * 256 + [2] * 256, 4096, 4000
    say(f"guard bands qgemm run by run blocks={len(bits)} N={N} M={M}")
    inp = _inputs(bits, 32, N, M, seed=91, zeros=False)
    lay = GpuLayer(inp)
    nws = dq.qgemm_workspace_bytes(lay.layout, M)
    assert nws == (M * inp.spec.K * 2 + 255) // 256 * 256 + M * N * 4, "expected the run-by-run path"
    yb = Guarded(M * N * 2, lay.dev, fill=0xFF)
    y = yb.view(torch.float16, (M, N))
    wb = Guarded(nws, lay.dev, fill=0xFF)
    dq.qgemm(lay.layout, lay.x(inp.x), lay.qweight, lay.scales, lay.zeros, lay.perm, wb.bytes(), y=y)
    assert yb.intact(), "a write landed outside y"
    assert wb.intact(), "a write landed outside the workspace"
    assert bool(torch.isfinite(y).all().item()), "an element of y was not written"
    rows = np.unique(np.concatenate([np.arange(0, M, 64), [M - 1]]))
    ref = oracle.qlinear(inp.x[rows], inp.q, inp.scales, inp.zeros, inp.bits, 32, inp.perm)
    assert_close(y[torch.from_numpy(rows).to(y.device)], ref, f"qgemm run by run M={M}")


def test_grouped_full_size_gate_up():
    """The step's gate/up launch at full size: two 4096 -> 11008 GPTQ 4-bit
    g128 act-order matrices in one grouped call, each against the oracle,
    with guard bands around both outputs."""
    say("grouped qgemv 2 x 4096x11008")
    spec = wl.LLAMA7B_DECODE[1]
    inps = [wl.generate(spec, M=1, seed=s) for s in (3, 4)]
    lays = [GpuLayer(i) for i in inps]
    x = lays[0].x(inps[0].x[:1])
    guards = [Guarded(spec.N * 2, lays[0].dev) for _ in lays]
    ys = [g.view(torch.float16, (1, spec.N)) for g in guards]
    dq.qgemv_grouped(lays[0].layout, x, [g.qweight for g in lays], [g.scales for g in lays],
                     [g.zeros for g in lays], lays[0].perm, lays[0].ws, ys=ys)
    for i, (inp, g) in enumerate(zip(inps, guards)):
        assert g.intact(), f"a write landed outside y[{i}]"
        ref = oracle.qlinear(inps[0].x[:1], inp.q, inp.scales, inp.zeros, inp.bits, spec.group_size, inps[0].perm)
        assert_close(ys[i], ref, f"matrix {i}")
