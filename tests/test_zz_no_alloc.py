"""qlinear_qgemv_noalloc (the library's static device scratch as workspace)
against qlinear_qgemv with a caller workspace, through the C ABI: the same
kernels run, so the outputs must be equal bit for bit; both are also checked
against the float64 oracle. Two calls in a row, the second on a smaller
input, so the second reuses scratch left by the first."""

import ctypes

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import GpuLayer, assert_close, say

pytestmark = pytest.mark.gpu


def _mixed(bits, gs, N, M, seed):
    rng = np.random.default_rng(seed)
    bits = np.asarray(bits, np.uint8)
    K = gs * len(bits)
    spec = wl.LayerSpec(f"noalloc-{K}x{N}", K, N, gs, ((4, 1.0),), True, True, (M,))
    perm = rng.permutation(K).astype(np.int32)
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    s = rng.uniform(0.005, 0.02, size=(len(bits), N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    return wl.LayerInputs(spec, bits, q, None, s, perm, x)


def _call_noalloc(lay, x, y):
    """Through the C entry point itself (ctypes), no Python-side workspace."""
    L = dq.lib()
    st = L.qlinear_qgemv_noalloc(lay.layout.ref, x.data_ptr(), int(x.shape[0]), lay.qweight.data_ptr(),
                                 lay.scales.data_ptr(), None if lay.zeros is None else lay.zeros.data_ptr(),
                                 None if lay.perm is None else lay.perm.data_ptr(), y.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, dq.status_string(st)


def _check(inp, M):
    lay = GpuLayer(inp)
    x = lay.x(inp.x[:M])
    y_na = torch.full((M, inp.spec.N), float("nan"), dtype=torch.float16, device=lay.dev)
    _call_noalloc(lay, x, y_na)
    y_ws = dq.qgemv(lay.layout, x, lay.qweight, lay.scales, lay.zeros, lay.perm, lay.ws)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ws), "no-alloc call differs from the call with a workspace"
    ref = oracle.qlinear(inp.x[:M], inp.q, inp.scales, inp.zeros, inp.bits, inp.spec.group_size, inp.perm)
    assert_close(y_na, ref, f"noalloc {inp.spec.name} M={M}")


def test_noalloc_matches_workspace_call_twice():
    big = wl.generate(wl.LLAMA7B_DECODE[2], M=16)          # 11008 -> 4096, GPTQ 4-bit g128 act-order
    say("noalloc: 11008x4096 M=16, then mixed 352x520 M=3")
    _check(big, 16)
    small = _mixed([6, 5, 4, 4, 3, 3, 2, 8, 4, 4, 4], 32, 520, 3, seed=21)
    _check(small, 3)
    _check(small, 1)


def test_noalloc_rejects_k_beyond_scratch():
    say("noalloc: K beyond the maximum")
    K = dq.NOALLOC_MAX_K + 128
    lay = dq.Layout(K, 64, 128, np.full(K // 128, 4, np.uint8))
    fake = 0x10000
    st = dq.lib().qlinear_qgemv_noalloc(lay.ref, fake, 2, fake, fake, None, None, fake, None)
    assert st == dq._lib.ERR_UNSUPPORTED
