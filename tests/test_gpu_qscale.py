"""EXL2 two-level scales on the GPU against the CPU oracle: q_scale packing
(bit-exact), the float16 dequantized weights (bit-exact), and the decode and
prefill layers (one-hot probes bit-exact; otherwise relative Frobenius error
<= 1e-3 and max error <= 1e-2 * max|y_ref|)."""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import GpuLayer, assert_close, fp16_bits, say

pytestmark = pytest.mark.gpu


def _inputs(bits, gs, N, M, seed, act_order=True):
    rng = np.random.default_rng(seed)
    bits = np.asarray(bits, np.uint8)
    K = gs * len(bits)
    spec = wl.LayerSpec(f"qscale-{K}x{N}", K, N, gs, ((4, 1.0),), True, act_order, (M,))
    perm = rng.permutation(K).astype(np.int32) if act_order else None
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    x = rng.standard_normal((M, K)).astype(np.float16)
    codes = rng.integers(0, 16, size=(len(bits), N), dtype=np.uint8)
    smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
    inp = wl.LayerInputs(spec, bits, q, None, np.zeros((len(bits), N), np.float16), perm, x)
    return inp, codes, smax


class QscaleLayer(GpuLayer):
    """A layer with two-level scales: q_scale packed by qlinear_pack_qscale."""

    def __init__(self, inp, codes, smax):
        super().__init__(inp)
        self.codes = codes
        self.smax_np = smax
        self.q_scale = dq.pack_qscale(torch.from_numpy(np.ascontiguousarray(codes)).to(self.dev))
        self.q_scale_max = torch.from_numpy(smax).to(self.dev)

    def qgemv(self, x_np, **kw):
        return dq.qgemv_qscale(self.layout, self.x(x_np), self.qweight, self.q_scale, self.q_scale_max, self.perm,
                               self.ws, **kw)

    def qgemm(self, x_np, **kw):
        return dq.qgemm_qscale(self.layout, self.x(x_np), self.qweight, self.q_scale, self.q_scale_max, self.perm,
                               **kw)

    def ref(self, x_np):
        sp = self.inp.spec
        return oracle.qlinear_qscale(x_np, self.inp.q, oracle.qscale_pack(self.codes), self.smax_np, self.inp.bits,
                                     sp.group_size, self.inp.perm)


MIXED = [6, 6, 5, 5, 4, 4, 4, 3, 3, 2, 8]   # 11 blocks, every width
MID = [6, 5, 5, 4, 4, 3, 3]                 # widths 3-6 (one-launch matrix-core mode at 3-4 rows)


@pytest.mark.parametrize("G,N", [(1, 8), (3, 520), (37, 4096)])
def test_pack_qscale_bit_exact(G, N):
    say(f"pack_qscale G={G} N={N}")
    rng = np.random.default_rng(G * 7 + N)
    codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    got = dq.pack_qscale(torch.from_numpy(codes).cuda()).cpu().numpy().view(np.uint32)
    assert np.array_equal(got, oracle.qscale_pack(codes))


@pytest.mark.parametrize("bits", [MIXED, [4] * 8, [3] * 4 + [2] * 4], ids=["mixed", "4bit", "3b2b"])
def test_dequant_qscale_bit_exact(bits):
    say(f"dequant_qscale {bits}")
    inp, codes, smax = _inputs(bits, 32, 520, 1, seed=len(bits) + 3)
    lay = QscaleLayer(inp, codes, smax)
    w = dq.dequant_qscale(lay.layout, lay.qweight, lay.q_scale, lay.q_scale_max)
    want = oracle.dequant_qscale_fp16(inp.q, oracle.qscale_pack(codes), smax, inp.bits, 32)
    assert np.array_equal(fp16_bits(w), want.view(np.uint16))


@pytest.mark.parametrize("op,M", [("qgemv", 1), ("qgemv", 2), ("qgemv", 3), ("qgemv", 16), ("qgemm", 16)])
def test_one_hot_rows_are_exact(op, M):
    """x = e_k gives the two-level float16 weight row of feature k bit for bit:
    (q - z) (c + 1) is exact, and so is its product with scale_max / 16 in
    float32, so the float16 store is the only rounding."""
    say(f"qscale one-hot {op} M={M}")
    bits = MID if M == 3 else MIXED
    inp, codes, smax = _inputs(bits, 32, 520, M, seed=40 + M)
    lay = QscaleLayer(inp, codes, smax)
    K = inp.spec.K
    ks = np.random.default_rng(41 + M).choice(K, M, replace=False)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    y = lay.qgemv(x) if op == "qgemv" else lay.qgemm(x)
    w16 = oracle.dequant_qscale_fp16(inp.q, oracle.qscale_pack(codes), smax, inp.bits, 32)
    want = w16[np.argsort(inp.perm)[ks]]
    assert np.array_equal(y.cpu().numpy().astype(np.float32), want.astype(np.float32))


@pytest.mark.parametrize("M", (1, 2, 3, 4, 5, 8, 16))
@pytest.mark.parametrize("name", ("mixed", "mid", "4bit-g128", "3bit"))
def test_qgemv_qscale_small(name, M):
    """One-launch several-width kernel (1 row), multi-row kernel (2 rows),
    matrix-core kernel in one launch (3-4 rows, widths 3-6) or with the
    gather kernel (8-bit runs, 5+ rows); single widths run the several-width
    instances."""
    say(f"qgemv_qscale {name} M={M}")
    bits, gs = {"mixed": (MIXED, 32), "mid": (MID, 32), "4bit-g128": ([4] * 6, 128), "3bit": ([3] * 9, 32)}[name]
    inp, codes, smax = _inputs(bits, gs, 520, M, seed=60 + M + len(name))
    lay = QscaleLayer(inp, codes, smax)
    assert_close(lay.qgemv(inp.x), lay.ref(inp.x), f"qgemv_qscale {name} M={M}")


@pytest.mark.parametrize("M", (7, 130))
@pytest.mark.parametrize("name", ("mixed", "4bit", "split-3b2b"))
def test_qgemm_qscale_small(name, M):
    say(f"qgemm_qscale {name} M={M}")
    bits = {"mixed": MIXED, "4bit": [4] * 8, "split-3b2b": [3] * 128 + [2] * 128}[name]
    inp, codes, smax = _inputs(bits, 32, 264, M, seed=80 + M + len(name))
    lay = QscaleLayer(inp, codes, smax)
    assert_close(lay.qgemm(inp.x), lay.ref(inp.x), f"qgemm_qscale {name} M={M}")


def test_qscale_epilogue():
    say("qscale epilogue")
    inp, codes, smax = _inputs(MIXED, 32, 520, 5, seed=90)
    lay = QscaleLayer(inp, codes, smax)
    rng = np.random.default_rng(91)
    bias = rng.standard_normal(520).astype(np.float16)
    resid = rng.standard_normal((5, 520)).astype(np.float16)
    ref = oracle.apply_epilogue(lay.ref(inp.x), bias=bias, residual=resid, activation=oracle.ACT_SILU)
    for op in ("qgemv", "qgemm"):
        for M in (1, 2, 5):
            f = lay.qgemv if op == "qgemv" else lay.qgemm
            y = f(inp.x[:M], bias=lay.x(bias), residual=lay.x(resid[:M]), activation=dq.ACT_SILU)
            assert_close(y, ref[:M], f"qscale epilogue {op} M={M}")


def test_qgemv_qscale_long_row():
    """One row past the one-launch kernel's LDS limit (K = 33792): gather
    kernel plus multi-row kernel."""
    say("qgemv_qscale long row")
    inp, codes, smax = _inputs([3] * 528 + [2] * 528, 32, 48, 1, seed=95)
    lay = QscaleLayer(inp, codes, smax)
    assert_close(lay.qgemv(inp.x), lay.ref(inp.x), "qgemv_qscale K=33792")


DECODE_CASES = [(wl.EXL2_MIXED, 1), (wl.EXL2_MIXED, 8)] + [(s, M) for s in wl.LLAMA70B_EXL2 for M in (1, 16)]


@pytest.mark.parametrize("spec,M", DECODE_CASES, ids=lambda v: v.name if hasattr(v, "name") else f"M{v}")
def test_qgemv_qscale_workloads(spec, M):
    """The EXL2 decode layers at full size with two-level scales."""
    say(f"qgemv_qscale workload {spec.name} M={M}")
    inp = wl.generate(spec)
    codes, smax = wl.two_level_scales(spec)
    lay = QscaleLayer(inp, codes, smax)
    x = inp.x[:M]
    assert_close(lay.qgemv(x), lay.ref(x), f"{spec.name} M={M}")


def test_qscale_rejects_missing_operands():
    inp, codes, smax = _inputs([4, 4], 32, 64, 1, seed=3)
    lay = QscaleLayer(inp, codes, smax)
    lib = dq.lib()
    y = torch.empty((1, 64), dtype=torch.float16, device=lay.dev)
    x = lay.x(inp.x)
    st = lib.qlinear_qgemv_qscale(lay.layout.ref, x.data_ptr(), 1, lay.qweight.data_ptr(), lay.q_scale.data_ptr(),
                                  None, None, None, y.data_ptr(), lay.ws.data_ptr(), lay.ws.numel(), None)
    assert st == dq._lib.ERR_INVALID_ARGUMENT
