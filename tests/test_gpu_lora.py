"""qlinear_lora_delta on the GPU against the CPU oracle's lora_delta.

The update is float32 throughout (float16 inputs, float32 products and sums:
a product of two float16 values is exact in float32). The kernel sums x A in
chunks of 256 rows of K, then over the chunks; with recursive summation the
error of a K-term float32 sum grows like sqrt(K) * 2^-24 relative to the sum
of magnitudes, so for K <= 11008 a relative Frobenius error of 2e-5 and a
max error of 2e-4 * max|ref| leave a wide margin.
"""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
from gpu_util import device, say

pytestmark = pytest.mark.gpu

REL_FRO = 2e-5
MAX_REL = 2e-4


def _case(M, K, N, r, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    A = (rng.standard_normal((K, r)) / np.sqrt(K)).astype(np.float16)
    B = rng.standard_normal((r, N)).astype(np.float16)
    return x, A, B


def _close(got: torch.Tensor, ref: np.ndarray, what: str):
    g = got.cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, what
    assert np.isfinite(g).all(), what
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-300)
    assert rel <= REL_FRO and mx <= MAX_REL, f"{what}: rel_fro={rel:.3e} max_rel={mx:.3e}"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


# (M, K, N, rank): decode and prefill shapes of the Llama projections, and
# ragged ones: K not a multiple of the 256-row chunk, N not a multiple of the
# 256-column tile, M not a multiple of any row tile, every rank instance
# (8, 16, 32, 64) with ranks below and at its size.
SHAPES = [
    (1, 4096, 4096, 16),
    (1, 11008, 4096, 16),
    (4, 4096, 11008, 8),
    (1, 1000, 1000, 1),
    (3, 257, 300, 5),
    (9, 1000, 777, 24),
    (17, 520, 1030, 33),
    (300, 4096, 520, 64),
    (65, 255, 8, 12),
]


@pytest.mark.parametrize("M,K,N,r", SHAPES, ids=[f"M{m}-K{k}-N{n}-r{r}" for m, k, n, r in SHAPES])
def test_lora_delta_parity(M, K, N, r):
    say(f"lora_delta M={M} K={K} N={N} r={r}")
    x, A, B = _case(M, K, N, r, seed=M * 7 + r)
    got = dq.lora_delta(_dev(x), _dev(A), _dev(B), scale=0.5)
    torch.cuda.synchronize()
    _close(got, oracle.lora_delta(x, [(A, B, 0.5)]), f"M={M} K={K} N={N} r={r}")


@pytest.mark.parametrize("M", [5, 40])
def test_lora_delta_adapters_accumulate(M):
    """Two adapters with weights: the second call adds into the first's
    result, as the oracle's weighted sum (M = 40 takes the four-column
    expand kernel of large M)."""
    say(f"lora_delta accumulate M={M}")
    K, N = 1024, 640
    x, A1, B1 = _case(M, K, N, 8, seed=1)
    _, A2, B2 = _case(M, K, N, 40, seed=2)
    xd = _dev(x)
    d = dq.lora_delta(xd, _dev(A1), _dev(B1), scale=0.25)
    d = dq.lora_delta(xd, _dev(A2), _dev(B2), scale=-1.5, delta=d, accumulate=True)
    torch.cuda.synchronize()
    _close(d, oracle.lora_delta(x, [(A1, B1, 0.25), (A2, B2, -1.5)]), "two adapters")


def test_lora_delta_overwrites_without_accumulate():
    """accumulate=False writes the update whatever delta held (NaN here)."""
    say("lora_delta overwrite")
    x, A, B = _case(2, 300, 264, 4, seed=3)
    d = torch.full((2, 264), float("nan"), dtype=torch.float32, device=device())
    dq.lora_delta(_dev(x), _dev(A), _dev(B), scale=1.0, delta=d)
    torch.cuda.synchronize()
    _close(d, oracle.lora_delta(x, [(A, B, 1.0)]), "overwrite")


def test_lora_delta_one_hot_is_exact():
    """A = e_i, B = one row b, scale 1: each entry is x[m][i] * b[n], one
    float16 product, exact in float32 (the other terms are exact zeros)."""
    say("lora_delta one-hot")
    rng = np.random.default_rng(4)
    M, K, N = 6, 700, 300
    x = rng.standard_normal((M, K)).astype(np.float16)
    b = rng.standard_normal((1, N)).astype(np.float16)
    for i in (0, 255, 256, 699):
        A = np.zeros((K, 1), np.float16)
        A[i, 0] = 1
        got = dq.lora_delta(_dev(x), _dev(A), _dev(b)).cpu().numpy()
        want = np.outer(x[:, i].astype(np.float32), b[0].astype(np.float32))
        assert np.array_equal(got, want), i


def test_lora_delta_empty_rows_is_a_noop():
    x = torch.empty((0, 64), dtype=torch.float16, device=device())
    A = torch.zeros((64, 4), dtype=torch.float16, device=device())
    B = torch.zeros((4, 32), dtype=torch.float16, device=device())
    d = dq.lora_delta(x, A, B)
    assert tuple(d.shape) == (0, 32)
