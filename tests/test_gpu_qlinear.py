"""qgemv / qgemm on the GPU against the CPU oracle.

Bit-exact where one product decides the result (one-hot activations);
otherwise relative Frobenius error <= 1e-3 and max error <= 1e-2 * max|y_ref|.
"""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import GpuLayer, assert_close, device, fp16_bits, say

pytestmark = pytest.mark.gpu


def _mixed_inputs(bits, gs, N, M, seed, zeros, act_order=True):
    rng = np.random.default_rng(seed)
    bits = np.asarray(bits, np.uint8)
    K = gs * len(bits)
    spec = wl.LayerSpec(f"mixed-{K}x{N}", K, N, gs, ((4, 1.0),), not zeros, act_order, (M,))
    perm = rng.permutation(K).astype(np.int32) if act_order else None
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    z = rng.integers(0, 16, size=(len(bits), N), dtype=np.uint8) if zeros else None
    s = rng.uniform(0.005, 0.02, size=(len(bits), N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    return wl.LayerInputs(spec, bits, q, z, s, perm, x)


def _ref(inp, x=None):
    sp = inp.spec
    return oracle.qlinear(inp.x if x is None else x, inp.q, inp.scales, inp.zeros, inp.bits, sp.group_size, inp.perm)


MIXED_BITS = [6, 6, 5, 5, 4, 4, 4, 3, 3, 2, 8]   # 11 blocks of 32 rows, 6 runs
LONG_MIXED = [3] * 528 + [2] * 528              # K = 33792 at 32-row groups: past the one-launch kernel's LDS limit


# ------------------------------------------------------------------ one-hot probes

@pytest.mark.parametrize("op", ("qgemv", "qgemm"))
@pytest.mark.parametrize("zeros", (True, False))
def test_one_hot_rows_are_exact(op, zeros):
    """x = e_k returns the float16 weight row holding feature k, bit for bit.

    A single non-zero product is exact in float32 and the final rounding is
    the only one, so the result must equal the oracle's RNE(s * (q - z))."""
    say(f"one-hot {op} zeros={zeros}")
    inp = _mixed_inputs(MIXED_BITS, 32, 520, 16, seed=5, zeros=zeros)
    K = inp.spec.K
    lay = GpuLayer(inp)
    ks = np.random.default_rng(9).choice(K, 16, replace=False)
    x = np.zeros((16, K), np.float16)
    x[np.arange(16), ks] = 1.0
    y = lay.qgemv(x) if op == "qgemv" else lay.qgemm(x)
    w16 = oracle.dequant_fp16(inp.q, inp.scales, inp.zeros, inp.bits, 32)
    inv = np.argsort(inp.perm)
    want = w16[inv[ks]]
    got = y.cpu().numpy()
    # compare values (+0 and -0 are the same weight)
    assert np.array_equal(got.astype(np.float32), want.astype(np.float32))


@pytest.mark.parametrize("M", (1, 2, 3, 4))
@pytest.mark.parametrize("zeros", (True, False))
def test_one_hot_rows_are_exact_single_row_kernel(M, zeros):
    """The same bit-exact probe through the single-row kernel (one code width,
    1 to 4 rows): its factored form s * (acc - 1024 X' - z X) recovers q - z
    exactly for a single non-zero activation, and rounds s * (q - z) once."""
    say(f"one-hot single-row kernel M={M} zeros={zeros}")
    inp = _mixed_inputs([4] * 11, 32, 520, M, seed=6 + M, zeros=zeros)
    K = inp.spec.K
    lay = GpuLayer(inp)
    ks = np.random.default_rng(10 + M).choice(K, M, replace=False)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    y = lay.qgemv(x)
    w16 = oracle.dequant_fp16(inp.q, inp.scales, inp.zeros, inp.bits, 32)
    want = w16[np.argsort(inp.perm)[ks]]
    assert np.array_equal(y.cpu().numpy().astype(np.float32), want.astype(np.float32))


# ------------------------------------------------------------------ small ragged shapes

@pytest.mark.parametrize("M", (1, 2, 3, 5, 8, 13, 16))
@pytest.mark.parametrize("zeros", (True, False))
def test_qgemv_small_mixed(M, zeros):
    say(f"qgemv small mixed M={M} zeros={zeros}")
    inp = _mixed_inputs(MIXED_BITS, 32, 520, M, seed=100 + M, zeros=zeros)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv M={M}")


@pytest.mark.parametrize("M", (2, 4, 12))   # VALU kernel; single-row kernel; matrix-core kernel
@pytest.mark.parametrize("gs", (32, 64, 128))
@pytest.mark.parametrize("b", (2, 3, 4, 5, 6, 8))
def test_qgemv_uniform_widths(b, gs, M):
    say(f"qgemv uniform b={b} gs={gs} M={M}")
    inp = _mixed_inputs([b] * (1024 // gs), gs, 776, M, seed=b * 31 + gs + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv b={b} gs={gs} M={M}")


@pytest.mark.parametrize("M", (1, 7, 130, 257))
@pytest.mark.parametrize("zeros", (True, False))
def test_qgemm_small_mixed(M, zeros):
    say(f"qgemm small mixed M={M} zeros={zeros}")
    inp = _mixed_inputs(MIXED_BITS, 32, 520, M, seed=200 + M, zeros=zeros)
    y = GpuLayer(inp).qgemm(inp.x)
    assert_close(y, _ref(inp), f"qgemm M={M}")


# Layouts for the kernel that dequantizes each 32-row block into LDS: runs of
# one block each (every K-step of two blocks crosses a run boundary, and the
# run cursor passes several runs at once), an odd block count (the K tail
# step with its zeroed half) and an even one, and more than 8 runs.
LDS_KERNEL_BITS = {
    "1-block-runs-odd": [2, 3, 4, 5, 6, 8, 6, 5, 4, 3, 2, 8, 3],     # 13 blocks, 13 runs
    "1-block-runs-even": [8, 2, 6, 3, 5, 4, 8, 2, 6, 3, 5, 4, 8, 2],  # 14 blocks, 14 runs
    "long-odd": [6] * 7 + [4] * 30 + [3] * 18 + [5] * 3 + [2] * 9,  # 67 blocks, 5 runs
}


# (zero points, two-level scales): two-level scales are defined for symmetric layers only
@pytest.mark.parametrize("zeros,two_level", ((True, False), (False, False), (False, True)))
@pytest.mark.parametrize("name", sorted(LDS_KERNEL_BITS))
def test_qgemm_lds_kernel_edges(name, zeros, two_level):
    """The several-width prefill kernel at its edges: M = 130 and N = 136
    (ragged over its 128 x 128 tiles: rows and columns past the matrix read
    the last valid one and are not stored), odd and even block counts, runs of
    one block, with float16 or two-level scales and with or without zero
    points, against the oracle."""
    say(f"qgemm LDS kernel {name} zeros={zeros} two_level={two_level}")
    M, N = 130, 136
    inp = _mixed_inputs(LDS_KERNEL_BITS[name], 32, N, M, seed=len(name) * 13 + zeros, zeros=zeros)
    lay = GpuLayer(inp)
    if not two_level:
        assert_close(lay.qgemm(inp.x), _ref(inp), f"qgemm {name}")
        return
    rng = np.random.default_rng(77)
    G = len(inp.bits)
    codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
    dev = device()
    y = dq.qgemm_qscale(lay.layout, lay.x(inp.x), lay.qweight, dq.pack_qscale(torch.from_numpy(codes).to(dev)),
                        torch.from_numpy(smax).to(dev), lay.perm)
    ref = oracle.qlinear_qscale(inp.x, inp.q, oracle.qscale_pack(codes), smax, inp.bits, 32, inp.perm)
    assert_close(y, ref, f"qgemm_qscale {name}")


RUN_SPLIT_BITS = {
    "2runs-3b2b": [3] * 512 + [2] * 512,               # K = 32768, one run boundary (70B 2.5 bpw widths)
    "3runs-odd": [6] * 13 + [4] * 700 + [3] * 311,     # K = 32768, runs start at blocks 0, 13 and 713
}


@pytest.mark.parametrize("name,M,zeros", (("2runs-3b2b", 4096, True), ("2runs-3b2b", 4000, False),
                                          ("3runs-odd", 4000, True), ("3runs-odd", 4096, False)))
def test_qgemm_run_by_run(name, M, zeros):
    """Several code widths with K >= 16384 rows per run boundary and a grid
    of 16 x 16 tiles of 256 x 256 (N = 4096): one register-dequant launch
    per run, adding up in float32 partial sums in the workspace (first /
    middle / last launch), M even or ragged over the tiles. The oracle checks
    every 64th row and the last, in full float64."""
    say(f"qgemm run by run {name} M={M} zeros={zeros}")
    N = 4096
    inp = _mixed_inputs(RUN_SPLIT_BITS[name], 32, N, M, seed=len(name) * 7 + M, zeros=zeros)
    lay = GpuLayer(inp)
    assert dq.qgemm_workspace_bytes(lay.layout, M) > M * inp.spec.K * 2, "expected the run-by-run path"
    y = lay.qgemm(inp.x)
    rows = np.unique(np.concatenate([np.arange(0, M, 64), [M - 1]]))
    assert_close(y[torch.from_numpy(rows).to(y.device)], _ref(inp, inp.x[rows]), f"qgemm {name} M={M}")


@pytest.mark.parametrize("gs", (32, 128))
@pytest.mark.parametrize("b", (2, 3, 4, 5, 6, 8))
def test_qgemm_uniform_widths(b, gs):
    say(f"qgemm uniform b={b} gs={gs}")
    inp = _mixed_inputs([b] * (1024 // gs), gs, 392, 100, seed=b * 17 + gs, zeros=True)
    y = GpuLayer(inp).qgemm(inp.x)
    assert_close(y, _ref(inp), f"qgemm b={b} gs={gs}")


@pytest.mark.parametrize("b", (2, 3, 4, 5, 6, 8))
def test_qgemm_uniform_widths_large_grid(b):
    """One code width on a grid of 16 x 9 tiles of 256 x 256 (N = 4096,
    M = 2304): the register-dequant kernel's instance for that width. The
    oracle checks every 32nd row and the last."""
    say(f"qgemm uniform large grid b={b}")
    M = 2304
    inp = _mixed_inputs([b] * 8, 128, 4096, M, seed=b * 23, zeros=True)
    y = GpuLayer(inp).qgemm(inp.x)
    rows = np.unique(np.concatenate([np.arange(0, M, 32), [M - 1]]))
    assert_close(y[torch.from_numpy(rows).to(y.device)], _ref(inp, inp.x[rows]), f"qgemm b={b} large grid")


GATHER_ROW_CASES = [
    # (K, N, M): rows per workgroup of the prefill gather and its thread count
    (4096, 48, 37),       # 4 rows (32 KiB), 256 threads; last workgroup 1 row
    (10240, 48, 37),      # 2 rows (40 KiB), 256 threads
    (11008, 48, 37),      # 2 rows (43 KiB), 1024 threads
    (28672, 48, 37),      # 1 row (56 KiB), 1024 threads
    (32768, 48, 37),      # 1 row of exactly 64 KiB, 1024 threads
    (11008, 4096, 2304),  # 2 rows, 1024 threads, pair order of the register-dequant kernel (144 tiles)
]


@pytest.mark.parametrize("K,N,M", GATHER_ROW_CASES)
def test_qgemm_gather_rows(K, N, M):
    """Act-order prefill across the gather's row and thread configurations;
    the oracle checks every 32nd row and the last on the large grid."""
    say(f"qgemm gather rows K={K} N={N} M={M}")
    inp = _mixed_inputs([4] * (K // 128), 128, N, M, seed=K % 101 + M, zeros=True)
    y = GpuLayer(inp).qgemm(inp.x)
    if M * N > 1 << 20:
        rows = np.unique(np.concatenate([np.arange(0, M, 32), [M - 1]]))
        assert_close(y[torch.from_numpy(rows).to(y.device)], _ref(inp, inp.x[rows]), f"qgemm gather K={K} M={M}")
    else:
        assert_close(y, _ref(inp), f"qgemm gather K={K} M={M}")


SPLIT_K_CASES = [
    # (bits per group, group size, N, M, zero points)
    ([4] * 32, 128, 392, 17, True),                  # one width, K = 4096: 8 slices
    ([4] * 32, 128, 392, 130, False),                # two tile rows
    ([3] * 32, 128, 1040, 64, True),                 # 3-bit, 9 tile columns
    ([6] * 11 + [5] * 40 + [4] * 50 + [3] * 30, 32, 392, 50, False),   # 131 blocks: odd, the tail in the last slice
    ([2, 8] * 20 + [5] * 24, 32, 136, 33, True),     # 40 one-block runs and a long one; N ragged over 128
]


@pytest.mark.parametrize("case", range(len(SPLIT_K_CASES)))
@pytest.mark.parametrize("two_level", (False, True))
def test_qgemm_split_k(case, two_level):
    """Small grids on the LDS-dequant kernel with K cut into slices: each
    slice writes float32 partial sums to the workspace and a second kernel
    adds them in slice order before the epilogue, against the oracle."""
    bits, gs, N, M, zeros = SPLIT_K_CASES[case]
    zeros = zeros and not two_level
    say(f"qgemm split K case {case} two_level={two_level} M={M} N={N}")
    inp = _mixed_inputs(bits, gs, N, M, seed=case * 19 + 7, zeros=zeros)
    lay = GpuLayer(inp)
    K = inp.spec.K
    assert dq.qgemm_workspace_bytes(lay.layout, M) > (M * K * 2 + 255) // 256 * 256, "expected split K"
    if not two_level:
        assert_close(lay.qgemm(inp.x), _ref(inp), f"split K case {case}")
        return
    rng = np.random.default_rng(case)
    G = len(inp.bits)
    codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
    dev = device()
    y = dq.qgemm_qscale(lay.layout, lay.x(inp.x), lay.qweight, dq.pack_qscale(torch.from_numpy(codes).to(dev)),
                        torch.from_numpy(smax).to(dev), lay.perm)
    ref = oracle.qlinear_qscale(inp.x, inp.q, oracle.qscale_pack(codes), smax, inp.bits, gs, inp.perm)
    assert_close(y, ref, f"split K case {case} two-level")


MID_ROW_CASES = [
    # (bits per group, group size, zero points)
    ([4] * 32, 128, True),                               # GPTQ 4-bit g128 (K = 4096)
    ([6] * 13 + [5] * 13 + [4] * 64 + [3] * 38, 32, False),   # the EXL2 4.0 bpw mix
]


@pytest.mark.parametrize("M", (17, 24, 32))
@pytest.mark.parametrize("case", range(len(MID_ROW_CASES)))
@pytest.mark.parametrize("kind", ("plain", "fused", "two-level"))
def test_qgemm_mid_rows(case, M, kind):
    """17..32 rows through qlinear_qgemm run as two decode launches (16 rows,
    then the rest), the second with its rows of the residual and addend;
    against the oracle (with its epilogue, or with two-level scales)."""
    bits, gs, zeros = MID_ROW_CASES[case]
    zeros = zeros and kind != "two-level"
    say(f"qgemm mid rows case {case} M={M} {kind}")
    N = 392
    inp = _mixed_inputs(bits, gs, N, M, seed=case * 5 + M, zeros=zeros)
    lay = GpuLayer(inp)
    assert dq.qgemm_workspace_bytes(lay.layout, M) >= dq.qgemv_workspace_bytes(lay.layout)
    dev = device()
    if kind == "plain":
        assert_close(lay.qgemm(inp.x), _ref(inp), f"mid rows case {case} M={M}")
    elif kind == "fused":
        rng = np.random.default_rng(M)
        bias = rng.standard_normal(N).astype(np.float16)
        resid = rng.standard_normal((M, N)).astype(np.float16)
        addend = (rng.standard_normal((M, N)) * 0.25).astype(np.float32)
        y = dq.qgemm(lay.layout, lay.x(inp.x), lay.qweight, lay.scales, lay.zeros, lay.perm,
                     bias=torch.from_numpy(bias).to(dev), residual=torch.from_numpy(resid).to(dev),
                     activation=dq.ACT_SILU, addend=torch.from_numpy(addend).to(dev))
        ref = oracle.apply_epilogue(_ref(inp), bias, resid, oracle.ACT_SILU, addend=addend)
        assert_close(y, ref, f"mid rows fused case {case} M={M}")
    else:
        rng = np.random.default_rng(M + 1)
        G = len(inp.bits)
        codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
        smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
        y = dq.qgemm_qscale(lay.layout, lay.x(inp.x), lay.qweight, dq.pack_qscale(torch.from_numpy(codes).to(dev)),
                            torch.from_numpy(smax).to(dev), lay.perm)
        ref = oracle.qlinear_qscale(inp.x, inp.q, oracle.qscale_pack(codes), smax, inp.bits, gs, inp.perm)
        assert_close(y, ref, f"mid rows two-level case {case} M={M}")


MX_FEW_ROW_BITS = {
    "mid": [6, 5, 5, 4, 4, 4, 3, 3],     # widths 3-6: one launch, gather in the kernel
    "low": [3, 3, 3, 2, 2],              # widths 2-3
}


@pytest.mark.parametrize("zeros", (True, False))
@pytest.mark.parametrize("M", (3, 4))
@pytest.mark.parametrize("name", sorted(MX_FEW_ROW_BITS))
def test_qgemv_matrix_core_few_rows(name, M, zeros):
    """3-4 rows of a layout with several widths run the matrix-core kernel in
    one launch (x rows and perm staged in LDS, gathered run by run); 520
    columns leave a ragged last strip."""
    say(f"qgemv matrix-core one launch {name} M={M} zeros={zeros}")
    inp = _mixed_inputs(MX_FEW_ROW_BITS[name], 32, 520, M, seed=300 + M + 7 * len(name), zeros=zeros)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv {name} M={M}")


@pytest.mark.parametrize("K,M", [(4096, 5), (4096, 8), (5376, 5), (4608, 8), (4096, 16)])
@pytest.mark.parametrize("b,gs", [(4, 128), (2, 32), (3, 32), (5, 32), (6, 64), (8, 32)])
def test_qgemv_matrix_core_one_width_rows(b, gs, K, M):
    """5-8 rows of a single-width layer run the matrix-core kernel in one
    launch while 8 x rows, perm and fragments fit in LDS (K = 4096 at 8 rows,
    5376 at 5), else with the gather kernel first (4608 at 8 rows; 16 rows
    always); act-order, 520 columns leave a ragged last strip."""
    say(f"qgemv matrix-core one width b={b} gs={gs} K={K} M={M}")
    inp = _mixed_inputs([b] * (K // gs), gs, 520, M, seed=500 + b * 31 + K % 97 + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv one width b={b} K={K} M={M}")


@pytest.mark.parametrize("bits,gs,M", [([4] * 40, 128, 3), ([4] * 40, 128, 4), ([4] * 40, 128, 5),
                                       ([3] * 80 + [2] * 80, 32, 3)],
                         ids=("4bit-M3", "4bit-M4", "4bit-M5", "exl2-low-M3"))
def test_qgemv_matrix_core_one_launch_wide_strips(bits, gs, M):
    """K = 5120 in one launch leaves LDS for one workgroup per CU: 321 panels
    (5128 columns, the last one ragged) then run as 161 workgroups of 2
    columns per lane instead of two rounds of 1."""
    say(f"qgemv matrix-core one launch, wide strips, gs={gs} M={M}")
    inp = _mixed_inputs(bits, gs, 5128, M, seed=600 + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv wide strips gs={gs} M={M}")


@pytest.mark.parametrize("M", (3, 4))
@pytest.mark.parametrize("b", (3, 8))
def test_qgemv_matrix_core_3_4_rows_above_4096_squared(b, M):
    """3-4 rows of a 3- or 8-bit layer above 4096^2 weights (5120 x 5128)
    run the matrix-core kernel: one launch with wide strips at 3 bits, the
    gather kernel first at 8 bits."""
    say(f"qgemv matrix-core b={b} 5120x5128 M={M}")
    inp = _mixed_inputs([b] * 160, 32, 5128, M, seed=650 + b + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv b={b} 5120x5128 M={M}")


@pytest.mark.parametrize("K,gs", [(5120, 128), (8192, 32), (16384, 128)])
@pytest.mark.parametrize("mats", (1, 2))
def test_qgemv_two_rows_matrix_core(K, gs, mats):
    """2 rows of a 4-bit layer with K above 4096 and N >= 8192 run the
    matrix-core kernel (one launch at K = 5120 and 8192, the gather kernel
    first at 16384; 32-row groups: a scale per block), alone and as a grouped
    launch of two matrices; 8200 columns leave a ragged last strip. The oracle
    checks every output."""
    say(f"qgemv matrix-core two rows K={K} gs={gs} mats={mats}")
    inp = _mixed_inputs([4] * (K // gs), gs, 8200, 2, seed=660 + K % 97 + mats, zeros=True)
    lay = GpuLayer(inp)
    ref = _ref(inp)
    if mats == 1:
        assert_close(lay.qgemv(inp.x), ref, f"qgemv two rows K={K}")
        return
    ys = dq.qgemv_grouped(lay.layout, lay.x(inp.x), [lay.qweight, lay.qweight], [lay.scales, lay.scales],
                          [lay.zeros, lay.zeros], lay.perm, lay.ws)
    for y in ys:
        assert_close(y, ref, f"qgemv grouped two rows K={K}")


@pytest.mark.parametrize("M", (3, 4))
def test_qgemv_matrix_core_large_uniform(M):
    """3-4 rows of a single-width layer above 2 * 4096^2 weights run the
    matrix-core kernel (4-bit, 128-row groups: scale units of 4 blocks), with
    2 columns per lane and a ragged last strip (8200 columns)."""
    say(f"qgemv matrix-core 4096x8200 M={M}")
    inp = _mixed_inputs([4] * 32, 128, 8200, M, seed=400 + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv 4096x8200 M={M}")


@pytest.mark.parametrize("nblk", (1, 3, 64, 100, 128, 192, 256, 320, 448))
@pytest.mark.parametrize("b", (2, 3, 4, 5, 6, 8))
def test_qgemv_row_kernel_steps(b, nblk):
    """M = 1 with one code width (the single-row kernel): 32-row blocks split
    over 4 waves, 16 per step, two steps in flight. nblk covers waves with no
    blocks (1, 3), a single step, ragged splits (100), the steady-state loop
    and its tails of 2 and 3 steps (256, 320, 448)."""
    say(f"qgemv row kernel b={b} blocks={nblk}")
    inp = _mixed_inputs([b] * nblk, 32, 48, 1, seed=b * 1000 + nblk, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv row b={b} blocks={nblk}")


@pytest.mark.parametrize("M", (2, 3, 4))
@pytest.mark.parametrize("nblk", (3, 100, 192, 320))
@pytest.mark.parametrize("b", (2, 3, 4, 5, 6, 8))
def test_qgemv_row_kernel_rows(b, nblk, M):
    """2 to 4 rows through the single-row kernel's multi-row instances (2 or
    4 x rows in LDS, 3 rows on the 4-row instance with the last row unused):
    waves without blocks, ragged splits, the steady loop and its tails."""
    say(f"qgemv row kernel b={b} blocks={nblk} M={M}")
    inp = _mixed_inputs([b] * nblk, 32, 48, M, seed=b * 1000 + nblk * 7 + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv row b={b} blocks={nblk} M={M}")


@pytest.mark.parametrize("K", (16384, 16416, 28672, 31744))
def test_qgemv_row_kernel_long_rows(K):
    """The single-row kernel's x row staging at K = 16384 (8 pieces per
    thread), just past it and up to the LDS limit (16 pieces)."""
    say(f"qgemv row kernel long row K={K}")
    inp = _mixed_inputs([4] * (K // 32), 32, 48, 1, seed=K % 89, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv row K={K}")


@pytest.mark.parametrize("K,M", [(31744, 1), (33792, 1), (16416, 2), (33792, 2)])
def test_qgemv_long_rows(K, M):
    """Rows near and past the LDS capacity of the one-launch kernels (past
    it: the gather kernel plus the multi-row kernel, at 1 and 2 rows)."""
    say(f"qgemv long row K={K} M={M}")
    bits = [3] * (K // 64) + [2] * (K // 64)
    inp = _mixed_inputs(bits, 32, 48, M, seed=K % 97 + M, zeros=False)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"qgemv K={K}")


# One row, several widths: the one-launch kernel that runs the single-row
# scheme segment by segment (waves split at run boundaries near the equal
# split points).
ROWMIX_BITS = {
    "exl2-4.0bpw": [6] * 13 + [5] * 13 + [4] * 64 + [3] * 38,   # 4 runs, splits moved to 26 / 64 / 90
    "boundary-in-wave": [4] * 48 + [3] * 80,                    # a wave of two segments of 16 blocks
    "all-widths": [8, 6, 5, 4, 3, 2] * 3,                       # every width, 18 runs
    "low": [3] * 40 + [2] * 24,
    "max-runs": [4, 3] * 32,                                     # 64 runs: one block per segment
    "two-blocks": [4, 3],                                        # waves without blocks
    "three-blocks": [5, 3, 5],
}


@pytest.mark.parametrize("M", (1, 2))
@pytest.mark.parametrize("act_order", (True, False))
@pytest.mark.parametrize("zeros", (True, False))
@pytest.mark.parametrize("name", sorted(ROWMIX_BITS))
def test_qgemv_one_launch_mixed(name, zeros, act_order, M):
    say(f"qgemv one-launch mixed {name} zeros={zeros} act_order={act_order} M={M}")
    inp = _mixed_inputs(ROWMIX_BITS[name], 32, 520, M, seed=len(name) * 31 + 2 * zeros + act_order + 5 * M,
                        zeros=zeros, act_order=act_order)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"one-launch mixed {name} M={M}")


@pytest.mark.parametrize("K,M", [(4128, 1), (8224, 1), (16416, 1), (31744, 1), (4128, 2), (8224, 2), (15872, 2)])
def test_qgemv_one_launch_mixed_row_pieces(K, M):
    """x-row pieces per thread: 4, 8 and 16 at one row (K just past 4096,
    8192 and 16384), 4 and 8 at two rows, and the LDS limit of each."""
    say(f"qgemv one-launch mixed K={K} M={M}")
    nb = K // 32
    inp = _mixed_inputs([5] * (nb // 3) + [4] * (nb - nb // 3), 32, 48, M, seed=K % 101 + M, zeros=True)
    y = GpuLayer(inp).qgemv(inp.x)
    assert_close(y, _ref(inp), f"one-launch mixed K={K} M={M}")


def test_qgemv_one_launch_mixed_one_hot():
    """One-hot rows through the one-launch several-width kernel: exact."""
    say("qgemv one-launch mixed one-hot")
    inp = _mixed_inputs(ROWMIX_BITS["exl2-4.0bpw"], 32, 520, 1, seed=13, zeros=True)
    K = inp.spec.K
    lay = GpuLayer(inp)
    w16 = oracle.dequant_fp16(inp.q, inp.scales, inp.zeros, inp.bits, 32)
    inv = np.argsort(inp.perm)
    for k in np.random.default_rng(3).choice(K, 6, replace=False):
        x = np.zeros((1, K), np.float16)
        x[0, k] = 1.0
        got = lay.qgemv(x).cpu().numpy()[0]
        assert np.array_equal(got.astype(np.float32), w16[inv[k]].astype(np.float32)), k


def test_no_act_order_and_single_group():
    say("no act-order, one group")
    inp = _mixed_inputs([4], 32, 8, 3, seed=1, zeros=True, act_order=False)
    lay = GpuLayer(inp)
    assert_close(lay.qgemv(inp.x), _ref(inp), "qgemv tiny")
    assert_close(lay.qgemm(inp.x), _ref(inp), "qgemm tiny")


def test_empty_batch():
    inp = _mixed_inputs([4, 4], 32, 64, 1, seed=2, zeros=True)
    lay = GpuLayer(inp)
    x0 = np.zeros((0, inp.spec.K), np.float16)
    assert lay.qgemv(x0).shape == (0, 64)
    assert lay.qgemm(x0).shape == (0, 64)


# ------------------------------------------------------------------ invariances

def test_act_order_gather_invariance():
    """(x, perm) gives the same y as (x[:, perm], identity)."""
    say("perm invariance")
    inp = _mixed_inputs(MIXED_BITS, 32, 520, 4, seed=7, zeros=True)
    lay = GpuLayer(inp)
    y1 = lay.qgemv(inp.x).float()
    lay.perm = None
    y2 = lay.qgemv(np.ascontiguousarray(inp.x[:, inp.perm])).float()
    assert torch.allclose(y1, y2, rtol=1e-3, atol=1e-3 * y1.abs().max().item())


def test_rows_are_independent():
    """Row m of an M = 16 call equals the M = 1 call on that row."""
    say("row independence")
    inp = _mixed_inputs(MIXED_BITS, 32, 520, 16, seed=8, zeros=False)
    lay = GpuLayer(inp)
    y16 = lay.qgemv(inp.x).float()
    for m in (0, 5, 15):
        y1 = lay.qgemv(inp.x[m:m + 1]).float()
        assert torch.allclose(y16[m:m + 1], y1, rtol=2e-3, atol=2e-3 * y1.abs().max().item())


def test_workspace_is_scratch_and_shareable():
    """The workspace needs no initialization, and one buffer serves layouts of
    different shapes called one after another on a stream."""
    say("workspace scratch")
    a = _mixed_inputs(MIXED_BITS, 32, 520, 16, seed=10, zeros=True)
    b = _mixed_inputs([3] * 40, 32, 264, 2, seed=11, zeros=False)
    la, lb = GpuLayer(a), GpuLayer(b)
    need = max(dq.qgemv_workspace_bytes(la.layout), dq.qgemv_workspace_bytes(lb.layout))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=la.dev)   # garbage: all-NaN patterns
    la.ws = lb.ws = ws
    for _ in range(3):
        assert_close(la.qgemv(a.x), _ref(a), "a")
        assert_close(lb.qgemv(b.x), _ref(b), "b")
        assert_close(lb.qgemv(b.x[:1]), _ref(b, b.x[:1]), "b M=1")


# ------------------------------------------------------------------ full-size workloads

DECODE_CASES = [(wl.TINY, 1)] + [(s, M) for s in wl.LLAMA7B_DECODE for M in s.Ms] + \
    [(wl.EXL2_MIXED, M) for M in wl.EXL2_MIXED.Ms] + [(s, M) for s in wl.LLAMA70B_EXL2 for M in s.Ms]


@pytest.mark.parametrize("spec,M", DECODE_CASES, ids=lambda v: v.name if hasattr(v, "name") else f"M{v}")
def test_qgemv_workloads(spec, M):
    say(f"qgemv workload {spec.name} M={M}")
    inp = wl.generate(spec)
    x = inp.x[:M]
    y = GpuLayer(inp).qgemv(x)
    assert_close(y, _ref(inp, x), f"{spec.name} M={M}")


@pytest.mark.parametrize("spec", (wl.TINY, wl.LLAMA7B_DECODE[1], wl.EXL2_MIXED), ids=lambda s: s.name)
def test_qgemm_decode_shapes(spec):
    say(f"qgemm on decode shape {spec.name}")
    inp = wl.generate(spec)
    y = GpuLayer(inp).qgemm(inp.x)
    assert_close(y, _ref(inp), spec.name)


def test_qgemm_prefill_workload():
    """Llama-2-13B MLP prefill, M = 2048: the oracle checks sampled token rows
    (every 16th row, plus the last), computed in full float64."""
    spec = wl.PREFILL_13B
    say(f"qgemm workload {spec.name}")
    inp = wl.generate(spec)
    y = GpuLayer(inp).qgemm(inp.x)
    rows = np.unique(np.concatenate([np.arange(0, 2048, 16), [2047]]))
    ref = _ref(inp, inp.x[rows])
    assert_close(y[torch.from_numpy(rows).to(y.device)], ref, spec.name)


@pytest.mark.parametrize("two_level", (False, True))
def test_qgemm_exl2_prefill_full_size(two_level):
    """EXL2 4.0 bpw 4096 -> 11008 (widths 6, 5, 4, 3: the kernel that
    dequantizes into LDS) at M = 2048, as the bench times it, with float16 or
    two-level scales: the oracle checks every 16th row and the last, in full
    float64."""
    spec = wl.EXL2_MIXED
    M = 2048
    say(f"qgemm EXL2 prefill {spec.name} M={M} two_level={two_level}")
    inp = wl.generate(spec, M=M)
    lay = GpuLayer(inp)
    rows = np.unique(np.concatenate([np.arange(0, M, 16), [M - 1]]))
    if two_level:
        dev = device()
        codes, smax = wl.two_level_scales(spec)
        y = dq.qgemm_qscale(lay.layout, lay.x(inp.x), lay.qweight, dq.pack_qscale(torch.from_numpy(codes).to(dev)),
                            torch.from_numpy(smax).to(dev), lay.perm)
        ref = oracle.qlinear_qscale(inp.x[rows], inp.q, oracle.qscale_pack(codes), smax, inp.bits, spec.group_size,
                                    inp.perm)
    else:
        y = lay.qgemm(inp.x)
        ref = _ref(inp, inp.x[rows])
    assert_close(y[torch.from_numpy(rows).to(y.device)], ref, f"{spec.name} two_level={two_level}")


def test_qgemm_row_chunks():
    """Activations of more than 2^31 bytes (M * K * 2): the prefill kernel's
    offsets are 32-bit, so the rows run in chunks (here 32512 + 556 rows).
    Rows on both sides of the chunk boundary against the oracle."""
    K, N, gs, M = 32768, 256, 128, 33068
    say(f"qgemm row chunks K={K} N={N} M={M}")
    inp = _mixed_inputs([4] * (K // gs), gs, N, 1, seed=11, zeros=True)
    layer = GpuLayer(inp)
    gen = torch.Generator(device=layer.dev).manual_seed(11)
    x = torch.randn((M, K), generator=gen, device=layer.dev, dtype=torch.float16)
    y = dq.qgemm(layer.layout, x, layer.qweight, layer.scales, layer.zeros, layer.perm)
    rows = np.array([0, 1, 255, 32511, 32512, 32513, 32767, M - 2, M - 1])
    ridx = torch.from_numpy(rows).to(layer.dev)
    ref = _ref(inp, x[ridx].cpu().numpy())
    assert_close(y[ridx], ref, "row chunks")
    # The epilogue's per-row operands (residual, float32 addend) follow the
    # chunks: rows past the first chunk take their own rows of both.
    resid = torch.randn((M, N), generator=gen, device=layer.dev, dtype=torch.float16)
    addend = torch.randn((M, N), generator=gen, device=layer.dev, dtype=torch.float32) * 4.0
    y2 = dq.qgemm(layer.layout, x, layer.qweight, layer.scales, layer.zeros, layer.perm, residual=resid,
                  addend=addend)
    ref2 = oracle.apply_epilogue(ref, None, resid[ridx].cpu().numpy(), dq.ACT_NONE,
                                 addend=addend[ridx].cpu().numpy().astype(np.float64))
    assert_close(y2[ridx], ref2, "row chunks with residual and addend")


# ------------------------------------------------------------------ grouped launches

@pytest.mark.parametrize("bits,M,zeros", [([4] * 16, 1, True), ([4] * 16, 4, True), ([3] * 16, 1, False),
                                          (MIXED_BITS, 1, False), (MIXED_BITS, 3, True), ([4] * 16, 8, True),
                                          (MIXED_BITS, 16, False)],
                         ids=["4bit-M1", "4bit-M4", "3bit-M1-sym", "mixed-M1", "mixed-M3", "4bit-M8-mfma",
                              "mixed-M16-mfma"])
def test_grouped_qgemv_matches_separate_calls(bits, M, zeros):
    """qlinear_qgemv_grouped over 3 matrices (same layout, x and perm, their
    own codes, scales and zeros) gives each matrix's qlinear_qgemv result,
    bit for bit, and the oracle's within tolerance."""
    say(f"grouped qgemv bits={bits[0]}.. M={M} zeros={zeros}")
    base = _mixed_inputs(bits, 32, 520, M, seed=300 + M, zeros=zeros)
    lays = []
    for i in range(3):
        inp = _mixed_inputs(bits, 32, 520, M, seed=400 + 10 * M + i, zeros=zeros)
        # share x and perm with the first matrix
        inp = wl.LayerInputs(inp.spec, inp.bits, inp.q, inp.zeros, inp.scales, base.perm, base.x)
        lays.append((inp, GpuLayer(inp)))
    L0 = lays[0][1]
    x = L0.x(base.x)
    ys = dq.qgemv_grouped(L0.layout, x, [g.qweight for _, g in lays], [g.scales for _, g in lays],
                          None if not zeros else [g.zeros for _, g in lays], L0.perm, L0.ws)
    for (inp, g), y in zip(lays, ys):
        y1 = dq.qgemv(g.layout, x, g.qweight, g.scales, g.zeros, L0.perm, g.ws)
        assert torch.equal(y, y1)
        assert_close(y, _ref(inp), "grouped")


def test_grouped_qgemv_max_group_full_size():
    """Eight 4096 -> 4096 GPTQ matrices in one launch (the largest group)."""
    say("grouped qgemv 8 x 4096x4096")
    spec = wl.LLAMA7B_DECODE[0]
    inps = [wl.generate(spec, M=1, seed=s) for s in range(8)]
    lays = [GpuLayer(i) for i in inps]
    perm = lays[0].perm
    x = lays[0].x(inps[0].x[:1])
    ys = dq.qgemv_grouped(lays[0].layout, x, [g.qweight for g in lays], [g.scales for g in lays],
                          [g.zeros for g in lays], perm, lays[0].ws)
    for i in (0, 7):
        ref = oracle.qlinear(inps[0].x[:1], inps[i].q, inps[i].scales, inps[i].zeros, inps[i].bits,
                             spec.group_size, inps[0].perm)
        assert_close(ys[i], ref, f"matrix {i}")


# ------------------------------------------------------------------ special values

@pytest.mark.parametrize("op,bits,gs,M,exact", [
    ("qgemv", [4] * 11, 32, 1, False),     # single-row kernel (factored arithmetic)
    ("qgemv", [4] * 11, 32, 4, False),     # single-row kernel, 4 rows
    ("qgemv", MIXED_BITS, 32, 1, False),   # one-launch several-width kernel
    ("qgemv", LONG_MIXED, 32, 1, False),   # gather + multi-row VALU kernel (K past the one-launch LDS limit)
    ("qgemv", MIXED_BITS, 32, 2, False),   # one-launch several-width kernel, 2 rows
    ("qgemv", MIXED_BITS, 32, 8, True),    # matrix-core kernel, exact dequantization (a scale per block)
    ("qgemv", [4] * 6, 128, 8, False),     # matrix-core kernel, factored (4-bit, 128-row groups)
    ("qgemm", MIXED_BITS, 32, 64, True),   # prefill, several widths
    ("qgemm", [4] * 11, 32, 64, True),     # prefill, one width
], ids=["row", "row-M4", "rowmix-M1", "gather-valu-M1", "rowmix-M2", "mfma-exact-M8", "mfma-factored-M8",
        "qgemm-mixed", "qgemm-4bit"])
def test_nonfinite_activations(op, bits, gs, M, exact):
    """A NaN activation makes its whole output row NaN; an Inf activation makes
    every column of its row non-finite (kernels that dequantize exactly: the
    IEEE result of the float64 oracle, +-Inf or NaN where the weight is 0; the
    factored decode kernels subtract 1024 X' + z X and give NaN). Other rows
    are unaffected."""
    say(f"non-finite activations {op} M={M} gs={gs}")
    inp = _mixed_inputs(bits, gs, 520, max(M, 2), seed=77 + M, zeros=True)
    x = inp.x[:M].copy()
    K = inp.spec.K
    x[0, 5] = np.float16(np.nan)
    if M >= 2:
        x[1, K - 3] = np.float16(np.inf)
    lay = GpuLayer(inp)
    y = (lay.qgemv(x) if op == "qgemv" else lay.qgemm(x)).float().cpu().numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        ref = _ref(inp, x)
    assert np.isnan(y[0]).all()
    if M >= 2:
        assert not np.isfinite(y[1]).any()
        if exact:
            assert np.array_equal(np.isnan(y[1]), np.isnan(ref[1]))
            assert np.array_equal(np.sign(y[1][np.isinf(ref[1])]), np.sign(ref[1][np.isinf(ref[1])]))
    if M > 2:
        assert_close(torch.from_numpy(y[2:]), ref[2:], "finite rows")


# ------------------------------------------------------------------ fused epilogue

EPILOGUE_PATHS = [
    ("qgemv", [4] * 11, 1, 520),        # single-row kernel
    ("qgemv", [4] * 11, 2, 520),        # single-row kernel, 2-row instance
    ("qgemv", [4] * 11, 3, 520),        # single-row kernel, 4-row instance
    ("qgemv", MIXED_BITS, 1, 520),      # one-launch several-width kernel (with an addend: gather + multi-row VALU kernel)
    ("qgemv", LONG_MIXED, 1, 520),      # gather + multi-row VALU kernel (K past the one-launch LDS limit)
    ("qgemv", MIXED_BITS, 2, 520),      # one-launch several-width kernel, 2 rows
    ("qgemv", [4] * 11, 5, 520),        # MFMA decode kernel
    ("qgemv", MIXED_BITS, 16, 520),     # MFMA decode kernel, several widths
    ("qgemm", [4] * 11, 2304, 4096),    # prefill, register dequant (144 tiles of 256 x 256)
    ("qgemm", [4] * 11, 100, 520),      # prefill, one width on a small grid: LDS dequant
    ("qgemm", MIXED_BITS, 100, 520),    # prefill, LDS dequant
    ("qgemm", [3] * 128 + [2] * 128, 100, 520),   # prefill, LDS dequant with K in 16 slices
    ("qgemm", [3] * 256 + [2] * 256, 4096, 4096),  # prefill, one launch per run
]


@pytest.mark.parametrize("op,bits,M,N", EPILOGUE_PATHS,
                         ids=["row", "row-M2", "row-M3", "rowmix-M1", "gather-valu-M1", "rowmix-M2", "mfma-M5", "mfma-M16", "qgemm",
                              "qgemm-small-grid", "qgemm-mixed", "qgemm-split-k", "qgemm-runs"])
@pytest.mark.parametrize("terms", ["bias", "residual", "bias-silu-residual", "silu-inplace-residual",
                                   "lora-bias-silu"])
def test_fused_epilogue(op, bits, M, N, terms):
    """y = RNE(act(x W + addend + bias) + residual) on every kernel path,
    against the float64 oracle's layer output followed by its epilogue. The
    addend is an on-the-fly LoRA update (rank 8) from qlinear_lora_delta;
    calls with one do not run the single-launch decode kernel (the "row"
    cases then run the gather and multi-row or MFMA kernels)."""
    say(f"fused epilogue {op} M={M} N={N} {terms}")
    inp = _mixed_inputs(bits, 32, N, M, seed=300 + M, zeros=True)
    lay = GpuLayer(inp)
    rng = np.random.default_rng(41)
    K = inp.spec.K
    bias = rng.standard_normal(N).astype(np.float16) if "bias" in terms else None
    resid = rng.standard_normal((M, N)).astype(np.float16) if "residual" in terms else None
    act = dq.ACT_SILU if "silu" in terms else dq.ACT_NONE
    x = lay.x(inp.x)
    b_t = None if bias is None else torch.from_numpy(bias).to(lay.dev)
    r_t = None if resid is None else torch.from_numpy(resid).to(lay.dev)
    add_t = add_ref = None
    if "lora" in terms:
        A = (rng.standard_normal((K, 8)) * (2.0 / np.sqrt(K))).astype(np.float16)
        B = (rng.standard_normal((8, N)) * 0.5).astype(np.float16)
        add_t = dq.lora_delta(x, lay.x(A), lay.x(B), scale=0.75)
        add_ref = oracle.lora_delta(inp.x, [(A, B, 0.75)])
    y = None
    if "inplace" in terms:
        y = r_t.clone()   # the residual is read from and written to the output
        r_t = y
    call = dq.qgemv if op == "qgemv" else dq.qgemm
    extra = (lay.ws,) if op == "qgemv" else (None,)
    out = call(lay.layout, x, lay.qweight, lay.scales, lay.zeros, lay.perm, *extra, y=y, bias=b_t, residual=r_t,
               activation=act, addend=add_t)
    # Large outputs: every 32nd row and the last, in full float64.
    rows = np.arange(M) if M * N <= 1 << 20 else np.unique(np.concatenate([np.arange(0, M, 32), [M - 1]]))
    sub = (lambda a: None if a is None else a[rows])
    base = _ref(inp, inp.x[rows])
    ref = oracle.apply_epilogue(base, bias, sub(resid), act, addend=sub(add_ref))
    assert_close(out[torch.from_numpy(rows).to(out.device)], ref, f"{op} M={M} {terms}")
    if add_ref is not None:
        # the update is large enough that dropping it would fail the check above
        plain = oracle.apply_epilogue(base, bias, sub(resid), act)
        assert np.linalg.norm(ref - plain) > 0.05 * np.linalg.norm(ref)


SHUFFLED_MAPS = {
    # name: (widths drawn per group, K, group size, N, zero points)
    "2.5bpw-256-groups": ((2, 3), 8192, 32, 520, False),
    "all-widths-128-groups": ((2, 3, 4, 5, 6, 8), 4096, 32, 520, True),
}


@pytest.mark.parametrize("M", (1, 4, 16, 64))
@pytest.mark.parametrize("name", sorted(SHUFFLED_MAPS))
def test_shuffled_width_map_via_group_order(name, M):
    """A per-group width map drawn at random (far more than 64 runs) is
    stored in qlinear_group_order's order with the composed act-order
    permutation; decode and prefill on it match the oracle on the original,
    shuffled layout."""
    widths, K, gs, N, zeros = SHUFFLED_MAPS[name]
    say(f"shuffled width map {name} M={M}")
    rng = np.random.default_rng(700 + M + K)
    bits = rng.choice(np.array(widths, np.uint8), size=K // gs)
    inp = _mixed_inputs(bits, gs, N, M, seed=800 + M, zeros=zeros)
    dev = torch.device("cuda")
    per_group = (torch.from_numpy(inp.scales).to(dev),) + (() if inp.zeros is None else (torch.from_numpy(inp.zeros).to(dev),))
    b2, q2, pg, p2 = dq.reorder_groups(dq.group_order(inp.bits), gs, inp.bits, torch.from_numpy(inp.q).to(dev),
                                       per_group, torch.from_numpy(inp.perm).to(dev))
    L = dq.Layout(K, N, gs, b2)
    assert L.nruns == len(np.unique(bits))
    qw = dq.pack_weights(L, q2)
    z2 = pg[1] if len(pg) > 1 else None
    x = torch.from_numpy(inp.x).to(dev)
    if M <= dq.GEMV_MAX_M:
        y = dq.qgemv(L, x, qw, pg[0], z2, p2, dq.qgemv_workspace(L, dev))
    else:
        y = dq.qgemm(L, x, qw, pg[0], z2, p2)
    assert_close(y, _ref(inp), f"shuffled {name} M={M}")


@pytest.mark.parametrize("M", (1, 8, 64))
def test_shuffled_width_map_two_level_scales(M):
    """Two-level scales on a shuffled 2/3-bit map: the per-group scale codes
    move with their groups before packing; the result matches the oracle on
    the original layout (symmetric codes, as two-level scales require)."""
    say(f"shuffled width map, two-level scales, M={M}")
    rng = np.random.default_rng(900 + M)
    gs, K, N = 32, 4096, 264
    bits = rng.choice(np.array([2, 3], np.uint8), size=K // gs)
    inp = _mixed_inputs(bits, gs, N, M, seed=910 + M, zeros=False)
    codes = rng.integers(0, 16, size=(K // gs, N), dtype=np.uint8)
    smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
    dev = torch.device("cuda")
    b2, q2, (c2,), p2 = dq.reorder_groups(dq.group_order(inp.bits), gs, inp.bits, torch.from_numpy(inp.q).to(dev),
                                          (torch.from_numpy(codes).to(dev),), torch.from_numpy(inp.perm).to(dev))
    L = dq.Layout(K, N, gs, b2)
    qw = dq.pack_weights(L, q2)
    x = torch.from_numpy(inp.x).to(dev)
    qs = dq.pack_qscale(c2.contiguous())
    sm = torch.from_numpy(smax).to(dev)
    if M <= dq.GEMV_MAX_M:
        y = dq.qgemv_qscale(L, x, qw, qs, sm, p2, dq.qgemv_workspace(L, dev))
    else:
        y = dq.qgemm_qscale(L, x, qw, qs, sm, p2)
    ref = oracle.qlinear_qscale(inp.x, inp.q, oracle.qscale_pack(codes), smax, inp.bits, gs, inp.perm)
    assert_close(y, ref, f"shuffled two-level M={M}")
