"""Seeded random layouts through every dispatch path, against the CPU oracle.

Each case draws a bit map (runs of random widths in random order, up to 12
runs), a group size, a ragged N, M, act-order or not, zero points or not,
and one of: plain qgemv, qgemv with two-level scales, a grouped qgemv, qgemm
(plain or two-level), or a fused epilogue. A second set holds M = 1 (decode
kinds only). Tolerances as everywhere: relative Frobenius error <= 1e-3 and
max error <= 1e-2 * max|y_ref|."""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import assert_close, device, say

pytestmark = pytest.mark.gpu

WIDTHS = (2, 3, 4, 5, 6, 8)
KINDS = ("qgemv", "qgemv-qscale", "grouped", "qgemm", "qgemm-qscale", "fused")
KINDS_M1 = ("qgemv", "qgemv-qscale", "grouped", "fused")
N_CASES = 72
N_CASES_M1 = 32   # one row: the one-launch several-width kernel (run segments, moved wave splits)


def _case(i):
    rng = np.random.default_rng(1000 + i)
    m1 = i >= N_CASES
    kind = KINDS_M1[i % len(KINDS_M1)] if m1 else KINDS[i % len(KINDS)]
    gs = int(rng.choice((32, 64, 128)))
    nruns = int(rng.integers(1, 13))
    widths = [int(w) for w in rng.choice(WIDTHS, size=nruns)]
    # neighbouring runs of one width merge into one (the layout keeps runs maximal)
    groups = []
    for w in widths:
        groups += [w] * int(rng.integers(1, 4))
    G = len(groups)
    K = G * gs
    N = int(rng.integers(1, 80)) * 8
    if m1:
        M = 1
    else:
        M = int(rng.integers(1, 17)) if kind not in ("qgemm", "qgemm-qscale") else int(rng.integers(1, 300))
    act_order = bool(rng.integers(0, 2))
    two = "qscale" in kind
    zeros = (not two) and bool(rng.integers(0, 2))
    return dict(kind=kind, gs=gs, bits=np.array(groups, np.uint8), K=K, N=N, M=M, act_order=act_order,
                zeros=zeros, seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES + N_CASES_M1))
def test_random_layout(i):
    c = _case(i)
    say(f"random layout {i}: {c['kind']} K={c['K']} N={c['N']} gs={c['gs']} M={c['M']} "
        f"runs={1 + int(np.count_nonzero(np.diff(c['bits'])))} ao={c['act_order']} zeros={c['zeros']}")
    dev = device()
    rng = np.random.default_rng(c["seed"])
    K, N, M, gs, bits = c["K"], c["N"], c["M"], c["gs"], c["bits"]
    G = len(bits)
    L = dq.Layout(K, N, gs, bits)
    perm = rng.permutation(K).astype(np.int32) if c["act_order"] else None
    pm = None if perm is None else torch.from_numpy(perm).to(dev)
    count = 3 if c["kind"] == "grouped" else 1
    qs = [np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
          for _ in range(count)]
    x = rng.standard_normal((M, K)).astype(np.float16)
    xd = torch.from_numpy(x).to(dev)
    qw = [dq.pack_weights(L, torch.from_numpy(q).to(dev)) for q in qs]
    ws = dq.qgemv_workspace(L, dev)
    if "qscale" in c["kind"]:
        codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
        smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
        q_scale = dq.pack_qscale(torch.from_numpy(codes).to(dev))
        q_smax = torch.from_numpy(smax).to(dev)
        ref = oracle.qlinear_qscale(x, qs[0], oracle.qscale_pack(codes), smax, bits, gs, perm)
        if c["kind"] == "qgemv-qscale":
            y = dq.qgemv_qscale(L, xd, qw[0], q_scale, q_smax, pm, ws)
        else:
            y = dq.qgemm_qscale(L, xd, qw[0], q_scale, q_smax, pm)
        assert_close(y, ref, c["kind"])
        return
    scales = [rng.uniform(0.005, 0.02, size=(G, N)).astype(np.float16) for _ in range(count)]
    zs = [rng.integers(0, 16, size=(G, N), dtype=np.uint8) if c["zeros"] else None for _ in range(count)]
    sd = [torch.from_numpy(s).to(dev) for s in scales]
    zd = [None if z is None else torch.from_numpy(z).to(dev) for z in zs]
    refs = [oracle.qlinear(x, qs[j], scales[j], zs[j], bits, gs, perm) for j in range(count)]
    if c["kind"] == "qgemv":
        assert_close(dq.qgemv(L, xd, qw[0], sd[0], zd[0], pm, ws), refs[0], "qgemv")
    elif c["kind"] == "grouped":
        ys = dq.qgemv_grouped(L, xd, qw, sd, None if zd[0] is None else zd, pm, ws)
        for j in range(count):
            assert_close(ys[j], refs[j], f"grouped[{j}]")
    elif c["kind"] == "qgemm":
        assert_close(dq.qgemm(L, xd, qw[0], sd[0], zd[0], pm), refs[0], "qgemm")
    else:   # fused epilogue on decode: bias, residual, SiLU
        bias = rng.standard_normal(N).astype(np.float16)
        resid = rng.standard_normal((M, N)).astype(np.float16)
        want = oracle.apply_epilogue(refs[0], bias=bias, residual=resid, activation=oracle.ACT_SILU)
        y = dq.qgemv(L, xd, qw[0], sd[0], zd[0], pm, ws, bias=torch.from_numpy(bias).to(dev),
                     residual=torch.from_numpy(resid).to(dev), activation=dq.ACT_SILU)
        assert_close(y, want, "fused")
