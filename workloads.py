"""Seeded synthetic inputs for the quantized linear layer.

Shared by the tests, the smoke check and the bench, for both the HIP path and
the CPU oracle. It draws raw inputs only -- codes, zero points, scales,
activations, the act-order permutation and the per-group bit map -- and holds
none of the layer's arithmetic (no packing, no dequantization, no matmul).

Every (workload, shape) draws from a fresh ``numpy.random.default_rng(seed)``
in a fixed order: perm -> q -> zeros -> scales -> x. Smaller M use the first
rows of x. Value distributions follow the workload list: x ~ N(0, 1) rounded to
float16, codes uniform over [0, 2^b - 1], GPTQ zero points uniform over
[0, 15], float16 scales uniform over [0.005, 0.02].
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer: K inputs, N outputs, group size, bit map recipe."""

    name: str
    K: int
    N: int
    group_size: int
    bit_mix: tuple  # ((bits, fraction), ...) in stored order, widest first
    symmetric: bool  # True: no zero points (z = 2^(b-1))
    act_order: bool  # True: random permutation of the K input features
    Ms: tuple = (1,)
    seed: int = 0


@dataclass
class LayerInputs:
    spec: LayerSpec
    bits: np.ndarray      # uint8 [G]
    q: np.ndarray         # uint8 [K][N], stored row order
    zeros: np.ndarray | None  # uint8 [G][N] or None (symmetric)
    scales: np.ndarray    # float16 [G][N]
    perm: np.ndarray | None   # int32 [K] (stored row j holds feature perm[j]) or None
    x: np.ndarray         # float16 [M_max][K]
    extra: dict = field(default_factory=dict)


def group_counts(G: int, bit_mix) -> list[tuple[int, int]]:
    """Split G groups over the bit widths of ``bit_mix`` by largest remainder.

    Each width first gets floor(fraction * G) groups; the groups still missing
    go, one each, to the widths with the largest fractional parts, ties going
    to the wider code. (10 % of 128 groups is 12.8 -> 13.)
    """
    fr = [(int(b), float(f)) for b, f in bit_mix]
    base = [int(np.floor(f * G + 1e-9)) for _, f in fr]
    rem = [f * G - base_i for (_, f), base_i in zip(fr, base)]
    missing = G - sum(base)
    order = sorted(range(len(fr)), key=lambda i: (-round(rem[i], 9), -fr[i][0]))
    for i in order[:missing]:
        base[i] += 1
    return [(fr[i][0], base[i]) for i in range(len(fr)) if base[i] > 0]


def bit_map(spec: LayerSpec) -> np.ndarray:
    """Per-group bit widths in stored order: runs of equal width, widest first."""
    G = spec.K // spec.group_size
    out = []
    for b, c in group_counts(G, spec.bit_mix):
        out += [b] * c
    return np.array(out, dtype=np.uint8)


def generate(spec: LayerSpec, M: int | None = None, seed: int | None = None,
             draw_x: bool = True) -> LayerInputs:
    """Draw one layer's inputs. M defaults to max(spec.Ms)."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    K, N, gs = spec.K, spec.N, spec.group_size
    G = K // gs
    bits = bit_map(spec)
    perm = rng.permutation(K).astype(np.int32) if spec.act_order else None
    high = np.repeat(np.left_shift(1, bits.astype(np.int64)), gs)[:, None]
    q = rng.integers(0, high, size=(K, N), dtype=np.uint8)
    zeros = None if spec.symmetric else rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, size=(G, N)).astype(np.float16)
    Mx = max(spec.Ms) if M is None else M
    x = rng.standard_normal((Mx, K)).astype(np.float16) if draw_x else None
    return LayerInputs(spec, bits, q, zeros, scales, perm, x)


def random_x(M: int, K: int, seed: int) -> np.ndarray:
    """Extra activations (e.g. for M > the workload's rows), float16 N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((M, K)).astype(np.float16)


# The five workloads: shapes, group sizes and bit mixes of the layer list.
GPTQ4 = ((4, 1.0),)
EXL2_40 = ((6, 0.10), (5, 0.10), (4, 0.50), (3, 0.30))
EXL2_25 = ((3, 0.50), (2, 0.50))

TINY = LayerSpec("gptq4-tiny-256x512-g32", 256, 512, 32, GPTQ4, False, False, (1,))

LLAMA7B_DECODE = (
    LayerSpec("llama2-7b-gptq4-g128-ao-4096x4096", 4096, 4096, 128, GPTQ4, False, True, (1, 4, 16)),
    LayerSpec("llama2-7b-gptq4-g128-ao-4096x11008", 4096, 11008, 128, GPTQ4, False, True, (1, 4, 16)),
    LayerSpec("llama2-7b-gptq4-g128-ao-11008x4096", 11008, 4096, 128, GPTQ4, False, True, (1, 4, 16)),
)

EXL2_MIXED = LayerSpec("exl2-4.0bpw-g32-ao-4096x11008", 4096, 11008, 32, EXL2_40, True, True, (1, 8))

PREFILL_13B = LayerSpec("llama2-13b-mlp-gptq4-g128-ao-5120x13824", 5120, 13824, 128, GPTQ4, False, True, (2048,))

LLAMA70B_EXL2 = (
    LayerSpec("llama2-70b-exl2-2.5bpw-g32-ao-8192x28672", 8192, 28672, 32, EXL2_25, True, True, (1, 16)),
    LayerSpec("llama2-70b-exl2-2.5bpw-g32-ao-28672x8192", 28672, 8192, 32, EXL2_25, True, True, (1, 16)),
)

ALL_LAYERS = (TINY,) + LLAMA7B_DECODE + (EXL2_MIXED, PREFILL_13B) + LLAMA70B_EXL2


def weight_bytes(spec: LayerSpec) -> int:
    """Algorithmic weight bytes: codes at b bits, float16 scales, 4-bit zeros."""
    G = spec.K // spec.group_size
    bits = bit_map(spec).astype(np.int64)
    qb = int((bits * spec.group_size).sum()) * spec.N // 8
    sb = G * spec.N * 2
    zb = 0 if spec.symmetric else G * spec.N // 2
    return qb + sb + zb


def two_level_scales(spec: LayerSpec, seed: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """EXL2 two-level scale inputs of a symmetric layer: 4-bit scale codes
    uint8 [G][N], uniform over 0..15, and q_scale_max float16 [N], uniform in
    [0.005, 0.02) like the one-level scales. Drawn from a generator of their
    own (seed + 1), so the layer's other inputs are those of generate()."""
    rng = np.random.default_rng((spec.seed if seed is None else seed) + 1)
    G = spec.K // spec.group_size
    codes = rng.integers(0, 16, size=(G, spec.N), dtype=np.uint8)
    smax = rng.uniform(0.005, 0.02, size=spec.N).astype(np.float16)
    return codes, smax


def weight_bytes_two_level(spec: LayerSpec) -> int:
    """Algorithmic weight bytes with two-level scales: codes at b bits, 4-bit
    scale codes and one float16 maximum scale per output (no zero points)."""
    G = spec.K // spec.group_size
    bits = bit_map(spec).astype(np.int64)
    qb = int((bits * spec.group_size).sum()) * spec.N // 8
    return qb + G * spec.N // 2 + 2 * spec.N
