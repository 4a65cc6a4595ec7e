"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle -- a field at the
wrong bit, a transposed block, a dropped zero point, the wrong act-order
direction, a round-half-up instead of ties-to-even, a scale taken from the
wrong group -- fails at least one test. ``test_planted_mistakes_are_caught``
checks that claim by planting such slips into copies of the oracle functions.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import qlinear_oracle as qo

BITS = (2, 3, 4, 5, 6, 8)


def _block_from_rows(b, rows):
    q = np.zeros((32, 1), dtype=np.uint8)
    for r, v in rows.items():
        q[int(r), 0] = v
    return q


# ---------------------------------------------------------------- format

def test_field_map_is_a_bijection():
    # Every bit of the b words of a block is used by exactly one (row, code bit).
    for b in BITS:
        F = oracle.block_field_map(b)
        assert F.shape == (32, b, 2)
        seen = np.zeros((b, 32), dtype=np.int64)
        for r in range(32):
            for k in range(b):
                t, pos = F[r, k]
                assert 0 <= t < b and 0 <= pos < 32
                seen[t, pos] += 1
        assert (seen == 1).all(), f"bit {b}: some block bit is unused or shared"


def test_fields_stay_inside_a_half_word():
    # Regular rows keep all code bits contiguous, ascending, inside one 16-bit half.
    for b in BITS:
        F = oracle.block_field_map(b)
        regular = 2 * (16 // b) * b
        for r in range(regular):
            ts = set(F[r, :, 0].tolist())
            pos = F[r, :, 1]
            assert len(ts) == 1
            assert (np.diff(pos) == 1).all()
            assert pos[0] // 16 == pos[-1] // 16


def test_hand_derived_words(golden_dir):
    with open(os.path.join(golden_dir, "format_examples.json")) as f:
        ex = json.load(f)["examples"]
    assert len(ex) >= 8
    for e in ex:
        b = e["bits"]
        q = _block_from_rows(b, e["rows"])
        want = np.array([int(w, 16) for w in e["words"]], dtype=np.uint32)[:, None]
        got = oracle.pack(q, [b], 32)
        assert got.dtype == np.uint32
        assert np.array_equal(got, want), (b, e["rows"], [hex(v) for v in got[:, 0]])
        assert np.array_equal(oracle.unpack(want, [b], 32, 32), q)


def test_four_bit_layout_matches_nibble_order():
    # Row i of each word sits at bits 4i..4i+3, least significant first,
    # the order that the blog's kernel sketch reads: (word >> 4i) & 0xF.
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(128, 5), dtype=np.uint8)
    w = oracle.pack(q, [4], 128)
    assert w.shape == (16, 5)
    for row in range(16):
        for i in range(8):
            assert np.array_equal((w[row] >> (4 * i)) & 0xF, q[8 * row + i])


@pytest.mark.parametrize("b", BITS)
@pytest.mark.parametrize("gs", (32, 64, 128))
def test_round_trip_random_and_extreme(b, gs):
    rng = np.random.default_rng(b * 1000 + gs)
    K, N = 2 * gs, 24
    for q in (
        rng.integers(0, 1 << b, size=(K, N), dtype=np.uint8),
        np.zeros((K, N), dtype=np.uint8),
        np.full((K, N), (1 << b) - 1, dtype=np.uint8),
        (np.indices((K, N)).sum(axis=0) % 2 * ((1 << b) - 1)).astype(np.uint8),
    ):
        packed = oracle.pack(q, [b, b], gs)
        assert packed.shape == (2 * gs * b // 32, N)
        assert np.array_equal(oracle.unpack(packed, [b, b], gs, K), q)


def test_round_trip_every_value_every_row():
    # Each row of a block takes every code value (b <= 6) against random neighbours.
    rng = np.random.default_rng(5)
    for b in (2, 3, 4, 5, 6):
        nv = 1 << b
        q = rng.integers(0, nv, size=(32, 32 * nv), dtype=np.uint8)
        for r in range(32):
            q[r, r * nv:(r + 1) * nv] = np.arange(nv)
        assert np.array_equal(oracle.unpack(oracle.pack(q, [b], 32), [b], 32, 32), q)


def test_mixed_bits_group_offsets():
    bits = [6, 6, 5, 4, 4, 3, 2, 8]
    gs = 64
    goff = oracle.group_word_offsets(bits, gs)
    # gs/32 = 2 blocks of b words per group, summed by hand
    assert goff.tolist() == [0, 12, 24, 34, 42, 50, 56, 60, 76]
    assert oracle.packed_rows(bits, gs) == 76
    rng = np.random.default_rng(2)
    K = gs * len(bits)
    q = np.concatenate([rng.integers(0, 1 << b, size=(gs, 9), dtype=np.uint8) for b in bits])
    packed = oracle.pack(q, bits, gs)
    assert packed.shape == (76, 9)
    assert np.array_equal(oracle.unpack(packed, bits, gs, K), q)
    # group 3 (4-bit) starts at row 34; its first word holds rows 3*64 .. 3*64+7
    for i in range(8):
        assert np.array_equal((packed[34] >> (4 * i)) & 0xF, q[192 + i])


def test_panel_layout_hand_example():
    # words[r][n] = 100 r + n, N = 24: panel 0 holds columns 0..15, panel 1
    # columns 16..23 followed by 8 zero slots; rows are contiguous per panel.
    R, N = 3, 24
    words = (100 * np.arange(R)[:, None] + np.arange(N)[None, :]).astype(np.uint32)
    P = oracle.panel_layout(words)
    assert P.shape == (2, 3, 16)
    flat = P.reshape(-1)
    assert flat[0] == 0 and flat[15] == 15 and flat[16] == 100 and flat[47] == 215
    assert flat[48] == 16 and flat[55] == 23 and flat[56] == 0 and flat[63] == 0
    assert flat[64] == 116 and flat[48 + 2 * 16 + 7] == 223
    assert np.array_equal(oracle.panel_unlayout(P, N), words)


def test_pack_rejects_out_of_range_codes():
    q = np.full((32, 3), 8, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.pack(q, [3], 32)
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((32, 3), np.uint8), [7], 32)


# ---------------------------------------------------------------- dequant

def test_dequant_hand_values(golden_dir):
    with open(os.path.join(golden_dir, "dequant_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        s = np.array([[int(e["s_bits"], 16)]], dtype=np.uint16).view(np.float16)
        q = np.full((32, 1), e["q"], dtype=np.uint8)
        z = np.array([[e["z"]]], dtype=np.uint8)
        w16 = oracle.dequant_fp16(q, s, z, [8], 32)
        want = float(e["w16"])
        assert float(w16[0, 0]) == want, (e, float(w16[0, 0]))
        if want == 0.0:
            assert not np.signbit(w16[0, 0])


def test_dequant_special_cases():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(64, 8), dtype=np.uint8)
    one = np.ones((2, 8), dtype=np.float16)
    zero = np.zeros((2, 8), dtype=np.uint8)
    assert np.array_equal(oracle.dequant(q, one, zero, [4, 4], 32), q.astype(np.float64))
    # symmetric 4-bit: (q - 8) * s
    s = np.full((2, 8), 0.25, dtype=np.float16)
    w = oracle.dequant(q, s, None, [4, 4], 32)
    assert np.array_equal(w, (q.astype(np.float64) - 8.0) * 0.25)
    # symmetric zero point is 2^(b-1) per group: 2-bit -> 2, 6-bit -> 32
    q2 = np.zeros((64, 1), dtype=np.uint8)
    w2 = oracle.dequant(q2, np.ones((2, 1), np.float16), None, [2, 6], 32)
    assert w2[:32, 0].tolist() == [-2.0] * 32 and w2[32:, 0].tolist() == [-32.0] * 32


def test_dequant_uses_each_groups_own_scale_and_zero():
    # Group g gets scale 2^g and zero g; code 10 everywhere -> w = 2^g * (10 - g).
    G, gs, N = 4, 32, 3
    q = np.full((G * gs, N), 10, dtype=np.uint8)
    s = np.array([[2.0 ** g] * N for g in range(G)], dtype=np.float16)
    z = np.array([[g] * N for g in range(G)], dtype=np.uint8)
    w = oracle.dequant(q, s, z, [4] * G, gs)
    for g in range(G):
        assert (w[g * gs:(g + 1) * gs] == 2.0 ** g * (10 - g)).all()


def test_dequant_fp16_is_single_rounding():
    # The float64 product is exact (<= 19 significant bits), so rounding it once
    # must equal rounding the exact rational value: compare against Fractions.
    from fractions import Fraction
    rng = np.random.default_rng(4)
    s = rng.uniform(0.005, 0.02, size=(1, 400)).astype(np.float16)
    q = rng.integers(0, 256, size=(32, 400), dtype=np.uint8)
    z = rng.integers(0, 256, size=(1, 400), dtype=np.uint8)
    w16 = oracle.dequant_fp16(q, s, z, [8], 32)
    for n in range(0, 400, 7):
        for j in range(0, 32, 5):
            exact = Fraction(float(s[0, n])) * (int(q[j, n]) - int(z[0, n]))
            # nearest float16 by exhaustive comparison with its neighbours
            cand = np.float16(float(exact))
            best = min((cand, np.nextafter(cand, np.float16(np.inf)), np.nextafter(cand, np.float16(-np.inf))),
                       key=lambda c: (abs(Fraction(float(c)) - exact),
                                      int(np.array([c]).view(np.uint16)[0]) & 1))
            assert w16[j, n] == best


# ---------------------------------------------------------------- the layer

def test_blog_sketch_worked_example():
    # One word 0x76543210 (codes 0..7), the remaining 24 rows at the midpoint 8,
    # symmetric 4-bit, scale 0.5, x = ones: y = 0.5 * sum_i (i - 8) = 0.5 * (28 - 64) = -18.
    q = np.full((32, 1), 8, dtype=np.uint8)
    q[:8, 0] = np.arange(8)
    packed = oracle.pack(q, [4], 32)
    assert packed[0, 0] == 0x76543210
    y = oracle.qlinear(np.ones((1, 32), np.float16), q, np.full((1, 1), 0.5, np.float16), None, [4], 32)
    assert y.shape == (1, 1) and y[0, 0] == -18.0


def test_act_order_direction():
    # perm[j] = (j + 1) % 32: stored row j holds original feature j + 1, so feature 0
    # lives in stored row 31. x = e_0 must return stored row 31 (code 15), not row 1.
    K = 32
    perm = (np.arange(K) + 1) % K
    q = (np.arange(K) % 16).astype(np.uint8)[:, None]
    x = np.zeros((1, K), np.float16)
    x[0, 0] = 1.0
    s = np.ones((1, 1), np.float16)
    z = np.zeros((1, 1), np.uint8)
    assert oracle.qlinear(x, q, s, z, [4], 32, perm)[0, 0] == 15.0
    assert oracle.qlinear_gidx(x, q, s, z, [4], 32, perm)[0, 0] == 15.0
    assert oracle.qlinear_bruteforce(x, q, s, z, [4], 32, perm)[0, 0] == 15.0


def test_closed_form_constant_matrix():
    K, N, gs = 256, 7, 64
    q = np.full((K, N), 11, dtype=np.uint8)
    s = np.full((K // gs, N), 0.125, np.float16)
    z = np.full((K // gs, N), 3, np.uint8)
    x = np.ones((2, K), np.float16)
    x[1] *= -2
    y = oracle.qlinear(x, q, s, z, [4] * 4, gs, np.random.default_rng(0).permutation(K))
    assert np.array_equal(y[0], np.full(N, K * 0.125 * 8))
    assert np.array_equal(y[1], np.full(N, -2 * K * 0.125 * 8))


def test_one_hot_rows_equal_dequantized_rows():
    rng = np.random.default_rng(7)
    K, N, gs = 128, 16, 32
    bits = [6, 4, 3, 2]
    q = np.concatenate([rng.integers(0, 1 << b, size=(gs, N), dtype=np.uint8) for b in bits])
    s = rng.uniform(0.005, 0.02, size=(4, N)).astype(np.float16)
    perm = rng.permutation(K)
    w = oracle.dequant(q, s, None, bits, gs)
    x = np.eye(K, dtype=np.float16)
    y = oracle.qlinear(x, q, s, None, bits, gs, perm)
    inv = np.argsort(perm)
    assert np.array_equal(y, w[inv])


@pytest.mark.parametrize("zeros", (True, False))
def test_three_paths_agree(zeros):
    # vectorised gather form == g_idx (scatter) form == pure-Python triple loop
    rng = np.random.default_rng(21 + zeros)
    K, N, M, gs = 96, 10, 3, 32
    bits = [5, 8, 3]
    q = np.concatenate([rng.integers(0, 1 << b, size=(gs, N), dtype=np.uint8) for b in bits])
    s = rng.uniform(0.005, 0.02, size=(3, N)).astype(np.float16)
    z = rng.integers(0, 16, size=(3, N), dtype=np.uint8) if zeros else None
    perm = rng.permutation(K)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y1 = oracle.qlinear(x, q, s, z, bits, gs, perm)
    y2 = oracle.qlinear_gidx(x, q, s, z, bits, gs, perm)
    y3 = oracle.qlinear_bruteforce(x, q, s, z, bits, gs, perm)
    scale = np.abs(y1).max()
    assert np.abs(y1 - y2).max() <= 1e-12 * scale
    assert np.abs(y1 - y3).max() <= 1e-12 * scale


def test_identity_perm_is_plain_matmul():
    rng = np.random.default_rng(8)
    K, N, gs = 64, 12, 32
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(2, N)).astype(np.float16)
    z = rng.integers(0, 16, size=(2, N), dtype=np.uint8)
    x = rng.standard_normal((2, K)).astype(np.float16)
    w = oracle.dequant(q, s, z, [4, 4], gs)
    assert np.array_equal(oracle.qlinear(x, q, s, z, [4, 4], gs, None),
                          x.astype(np.float64) @ w)
    assert np.array_equal(oracle.qlinear(x, q, s, z, [4, 4], gs, np.arange(K)),
                          x.astype(np.float64) @ w)


def test_rejects_bad_inputs():
    q = np.zeros((64, 4), np.uint8)
    s = np.ones((2, 4), np.float16)
    with pytest.raises(ValueError):
        oracle.qlinear(np.ones((1, 64), np.float16), q, s, None, [4, 4], 32, perm=np.zeros(64, int))
    with pytest.raises(ValueError):
        oracle.qlinear(np.ones((1, 63), np.float16), q, s, None, [4, 4], 32)
    with pytest.raises(ValueError):
        oracle.dequant(q, s, None, [4, 4], 48)


# ---------------------------------------------------------------- the pins catch slips

def test_planted_mistakes_are_caught(golden_dir, monkeypatch):
    """Plant plausible slips into the oracle; at least one pin must fail for each."""
    good_map = qo.block_field_map

    def swapped_halves(b):           # high and low half-word swapped
        F = good_map(b).copy()
        F[:, :, 1] = (F[:, :, 1] + 16) % 32
        return F

    def reversed_code_bits(b):       # code bits stored most-significant first
        return good_map(b)[:, ::-1, :].copy()

    def gather_with_inverse(x, q, scales, zeros, bits, gs, perm=None):
        p = np.argsort(np.asarray(perm)) if perm is not None else None
        return good_qlinear(x, q, scales, zeros, bits, gs, p)

    def dropped_zero(q, scales, zeros, bits, gs):
        return good_dequant(q, scales, np.zeros_like(np.asarray(zeros)) if zeros is not None else None, bits, gs)

    def half_up(q, scales, zeros, bits, gs):
        w = good_dequant(q, scales, zeros, bits, gs)
        lo = w.astype(np.float16)
        hi = np.where(w > lo, np.nextafter(lo, np.float16(np.inf)), lo)
        mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2
        return np.where(w >= mid, hi, lo).astype(np.float16)

    def scale_of_next_group(q, scales, zeros, bits, gs):
        return good_dequant(q, np.roll(np.asarray(scales), 1, axis=0), zeros, bits, gs)

    good_qlinear, good_dequant = qo.qlinear, qo.dequant
    planted = [
        ("block_field_map", swapped_halves),
        ("block_field_map", reversed_code_bits),
        ("qlinear", gather_with_inverse),
        ("dequant", dropped_zero),
        ("dequant_fp16", half_up),
        ("dequant", scale_of_next_group),
    ]
    pins = [
        lambda: test_hand_derived_words(golden_dir),
        test_four_bit_layout_matches_nibble_order,
        lambda: test_dequant_hand_values(golden_dir),
        test_dequant_uses_each_groups_own_scale_and_zero,
        test_act_order_direction,
        test_blog_sketch_worked_example,
        test_closed_form_constant_matrix,
    ]
    for name, bad in planted:
        with monkeypatch.context() as mp:
            mp.setattr(qo, name, bad)
            mp.setattr(oracle, name, bad)
            failed = 0
            for pin in pins:
                try:
                    pin()
                except (AssertionError, ValueError):
                    failed += 1
            assert failed > 0, f"no pin caught the planted slip in {name} ({bad.__name__})"


# ------------------------------------------------------------------ epilogue

def test_silu_closed_form_values():
    """SiLU at points where it is known without the formula: 0 at 0; odd part
    v/2 (silu(v) - silu(-v) = v); sigmoid(1) = e / (1 + e); saturation to v and
    to 0 far out."""
    assert oracle.silu(0.0) == 0.0
    e = np.e
    assert np.isclose(oracle.silu(1.0), e / (1.0 + e), rtol=1e-15)
    v = np.linspace(-6, 6, 25)
    assert np.allclose(oracle.silu(v) - oracle.silu(-v), v, rtol=0, atol=1e-14)
    assert np.isclose(oracle.silu(40.0), 40.0, rtol=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert np.all(np.diff(oracle.silu(np.linspace(0, 10, 101))) > 0)   # increasing for v > 0


def test_epilogue_terms_and_order():
    """Bias and residual add exactly; the activation sits between them:
    acc = 1, bias = 1, residual = 1 gives silu(2) + 1, not silu(3) or silu(1) + 2."""
    acc = np.array([[1.0]])
    got = oracle.apply_epilogue(acc, np.array([1.0]), np.array([[1.0]]), oracle.ACT_SILU)[0, 0]
    assert np.isclose(got, 2.0 / (1.0 + np.exp(-2.0)) + 1.0, rtol=1e-15)
    rng = np.random.default_rng(3)
    a = rng.standard_normal((3, 8))
    b = rng.standard_normal(8).astype(np.float16)
    r = rng.standard_normal((3, 8)).astype(np.float16)
    y = oracle.apply_epilogue(a, b, r, oracle.ACT_NONE)
    # (a + b) + r - a equals b + r up to float64 rounding of the sums
    assert np.allclose(y - a, b.astype(np.float64)[None, :] + r.astype(np.float64), rtol=0, atol=1e-14)
    assert np.array_equal(oracle.apply_epilogue(a), a)
    with pytest.raises(ValueError):
        oracle.apply_epilogue(a, activation=9)



# ------------------------------------------------------------------ LoRA

def _lora_case(rng, M=3, K=64, N=16, r=4):
    x = rng.standard_normal((M, K)).astype(np.float16)
    A = (rng.standard_normal((K, r)) * 0.2).astype(np.float16)
    B = (rng.standard_normal((r, N)) * 0.2).astype(np.float16)
    return x, A, B


def test_lora_rank_one_closed_form():
    """A = e_i (one-hot column), B = one row b: the update is s x[:, i] b,
    an outer product, for every i."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 40)).astype(np.float16)
    b = rng.standard_normal((1, 24)).astype(np.float16)
    for i in (0, 17, 39):
        A = np.zeros((40, 1), np.float16)
        A[i, 0] = 1
        got = oracle.lora_delta(x, [(A, b, -0.75)])
        want = -0.75 * np.outer(x[:, i].astype(np.float64), b[0].astype(np.float64))
        assert np.array_equal(got, want)


def test_lora_zero_adapter_and_zero_weight():
    rng = np.random.default_rng(12)
    x, A, B = _lora_case(rng)
    assert np.array_equal(oracle.lora_delta(x, [(A, np.zeros_like(B), 2.0)]), np.zeros((3, 16)))
    assert np.array_equal(oracle.lora_delta(x, [(A, B, 0.0)]), np.zeros((3, 16)))
    with pytest.raises(ValueError):
        oracle.lora_delta(x, [])


def test_lora_adapters_combine_as_one_of_concatenated_rank():
    """Weighted adapters (A1, B1, s1), (A2, B2, s2) are the single adapter
    A = [A1 | A2], B = [s1 B1 ; s2 B2] of rank r1 + r2 (block products), so a
    weight applied to the wrong adapter, or cross terms, would show."""
    rng = np.random.default_rng(13)
    x, A1, B1 = _lora_case(rng, r=3)
    _, A2, B2 = _lora_case(rng, r=5)
    s1, s2 = 0.5, -2.0
    A = np.concatenate([A1, A2], axis=1).astype(np.float64)
    B = np.concatenate([s1 * B1.astype(np.float64), s2 * B2.astype(np.float64)], axis=0)
    got = oracle.lora_delta(x, [(A1, B1, s1), (A2, B2, s2)])
    assert np.allclose(got, oracle.lora_delta(x, [(A, B, 1.0)]), rtol=1e-13, atol=1e-13)


def test_lora_bruteforce_tiny():
    """Explicit sums over k and j, element by element, on a 2 x 5 x 3 rank-2 case."""
    rng = np.random.default_rng(14)
    x, A, B = _lora_case(rng, M=2, K=5, N=3, r=2)
    got = oracle.lora_delta(x, [(A, B, 1.5)])
    for m in range(2):
        for n in range(3):
            v = 0.0
            for j in range(2):
                t = 0.0
                for k in range(5):
                    t += float(x[m, k]) * float(A[k, j])
                v += t * float(B[j, n])
            assert np.isclose(got[m, n], 1.5 * v, rtol=1e-14, atol=1e-14)


def test_lora_merge_identity_through_the_quantized_layer():
    """On the fly equals merged: with act-order, the layer plus the update
    through the epilogue (addend, bias, SiLU) equals SiLU(x W' + bias) for
    the dense merged matrix W' = W + s A B, W in original feature order
    (stored row j of the quantized matrix holds feature perm[j])."""
    rng = np.random.default_rng(15)
    K, N, gs = 128, 16, 32
    bits = [4, 3, 4, 2]
    q = np.stack([rng.integers(0, 2 ** bits[j // gs], N) for j in range(K)]).astype(np.uint8)
    scales = (rng.random((K // gs, N)) * 0.1 + 0.01).astype(np.float16)
    perm = rng.permutation(K)
    x, A, B = _lora_case(rng, M=3, K=K, N=N, r=6)
    bias = rng.standard_normal(N).astype(np.float16)
    s = 0.8
    acc = oracle.qlinear(x, q, scales, None, bits, gs, perm=perm)
    got = oracle.apply_epilogue(acc, bias, None, oracle.ACT_SILU, addend=oracle.lora_delta(x, [(A, B, s)]))
    w = oracle.dequant(q, scales, None, bits, gs)            # stored order
    W = np.zeros((K, N))
    W[perm] = w                                              # original order
    merged = W + s * (A.astype(np.float64) @ B.astype(np.float64))
    v = x.astype(np.float64) @ merged + bias.astype(np.float64)[None, :]
    want = v / (1.0 + np.exp(-v))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_epilogue_addend_joins_before_the_activation():
    """acc = 1, addend = 1, bias = 1, residual = 1: silu(3) + 1."""
    got = oracle.apply_epilogue(np.array([[1.0]]), np.array([1.0]), np.array([[1.0]]), oracle.ACT_SILU,
                                addend=np.array([[1.0]], np.float32))[0, 0]
    assert np.isclose(got, 3.0 / (1.0 + np.exp(-3.0)) + 1.0, rtol=1e-15)


def test_lora_planted_mistakes_are_caught(monkeypatch):
    """Plausible slips planted into lora_delta; a LoRA pin must fail for each."""
    good = qo.lora_delta

    def ignores_weight(x, adapters):
        return good(x, [(A, B, 1.0) for A, B, _ in adapters])

    def first_adapter_only(x, adapters):
        return good(x, list(adapters)[:1])

    def reversed_features(x, adapters):
        return good(np.asarray(x)[:, ::-1], adapters)

    def weight_twice(x, adapters):
        return good(x, [(A, B, s * s) for A, B, s in adapters])

    pins = [
        test_lora_rank_one_closed_form,
        test_lora_adapters_combine_as_one_of_concatenated_rank,
        test_lora_merge_identity_through_the_quantized_layer,
        test_lora_bruteforce_tiny,
    ]
    for bad in (ignores_weight, first_adapter_only, reversed_features, weight_twice):
        with monkeypatch.context() as mp:
            mp.setattr(qo, "lora_delta", bad)
            mp.setattr(oracle, "lora_delta", bad)
            failed = 0
            for pin in pins:
                try:
                    pin()
                except AssertionError:
                    failed += 1
            assert failed > 0, f"no pin caught {bad.__name__}"


# ------------------------------------------------------------------ two-level scales

def test_qscale_nibble_order_hand_words():
    # Codes 0..7 in columns 0..7 give the word 0x76543210, the nibble order of
    # the blog's kernel sketch; codes 15..8 in columns 8..15 give 0x89ABCDEF.
    c = np.concatenate([np.arange(8), 15 - np.arange(8)]).astype(np.uint8)[None, :]
    w = oracle.qscale_pack(c)
    assert w.shape == (1, 2) and int(w[0, 0]) == 0x76543210 and int(w[0, 1]) == 0x89ABCDEF
    assert np.array_equal(oracle.qscale_unpack(w, 16), c)


def test_qscale_round_trip_and_rejects():
    rng = np.random.default_rng(12)
    c = rng.integers(0, 16, size=(7, 40), dtype=np.uint8)
    assert np.array_equal(oracle.qscale_unpack(oracle.qscale_pack(c), 40), c)
    with pytest.raises(ValueError):
        oracle.qscale_pack(np.full((1, 8), 16, np.uint8))
    with pytest.raises(ValueError):
        oracle.qscale_pack(np.zeros((1, 12), np.uint8))


def test_qscale_dequant_hand_values(golden_dir):
    with open(os.path.join(golden_dir, "qscale_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        b = e["b"]
        q = np.full((32, 8), e["q"], dtype=np.uint8)
        codes = np.full((1, 8), e["c"], dtype=np.uint8)
        smax = np.full(8, int(e["smax_bits"], 16), dtype=np.uint16).view(np.float16)
        w16 = oracle.dequant_qscale_fp16(q, oracle.qscale_pack(codes), smax, [b], 32)
        assert (w16 == np.float16(float(e["w16"]))).all(), (e, float(w16[0, 0]))


def test_qscale_largest_code_is_the_one_level_scale():
    # Every code 15: the group scale is 1 and the weights are those of the
    # one-level definition with scale_max as every group's scale.
    rng = np.random.default_rng(13)
    bits = [6, 5, 4, 3, 2, 8]
    K, N = 32 * len(bits), 24
    q = np.concatenate([rng.integers(0, 1 << b, size=(32, N), dtype=np.uint8) for b in bits])
    smax = rng.uniform(0.005, 0.02, size=N).astype(np.float16)
    words = oracle.qscale_pack(np.full((len(bits), N), 15, np.uint8))
    one = oracle.dequant(q, np.repeat(smax[None, :], len(bits), axis=0), None, bits, 32)
    assert np.array_equal(oracle.dequant_qscale(q, words, smax, bits, 32), one)


def test_qscale_each_group_and_column_its_own_factor():
    # Group g, column n holds code (g + 3n) % 16; column n has scale_max 2^-n;
    # code 12 in every 4-bit row: w = (12 - 8) * ((g + 3n) % 16 + 1)/16 * 2^-n.
    G, N = 4, 16
    q = np.full((32 * G, N), 12, dtype=np.uint8)
    codes = np.array([[(g + 3 * n) % 16 for n in range(N)] for g in range(G)], dtype=np.uint8)
    smax = (2.0 ** -np.arange(N)).astype(np.float16)
    w = oracle.dequant_qscale(q, oracle.qscale_pack(codes), smax, [4] * G, 32)
    for g in range(G):
        for n in range(N):
            assert (w[32 * g:32 * (g + 1), n] == 4.0 * ((g + 3 * n) % 16 + 1) / 16.0 * 2.0 ** -n).all()


def test_qscale_layer_equals_one_level_layer_with_exact_scales():
    # With scale_max a power of two, every effective scale (c + 1)/16 * smax is
    # exact in float16: the two-level layer must equal the one-level layer
    # (independently pinned) fed those scales, act-order included.
    rng = np.random.default_rng(14)
    bits = [5, 4, 4, 3]
    G, N = len(bits), 32
    K = 32 * G
    q = np.concatenate([rng.integers(0, 1 << b, size=(32, N), dtype=np.uint8) for b in bits])
    codes = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    smax = (2.0 ** rng.integers(-9, -5, size=N)).astype(np.float16)
    s1 = ((codes.astype(np.float64) + 1.0) / 16.0 * smax.astype(np.float64)[None, :]).astype(np.float16)
    assert np.array_equal(s1.astype(np.float64), (codes + 1.0) / 16.0 * smax.astype(np.float64)[None, :])
    x = rng.standard_normal((3, K)).astype(np.float16)
    perm = rng.permutation(K)
    y2 = oracle.qlinear_qscale(x, q, oracle.qscale_pack(codes), smax, bits, 32, perm)
    y1 = oracle.qlinear(x, q, s1, None, bits, 32, perm)
    assert np.allclose(y2, y1, rtol=1e-12, atol=0)


def test_qscale_planted_mistakes_are_caught(golden_dir, monkeypatch):
    """Plant plausible slips into the two-level oracle; a pin must fail for each."""
    good_pack, good_unpack, good_scales = qo.qscale_pack, qo.qscale_unpack, qo.two_level_scales

    def msb_first_pack(codes):
        c = np.asarray(codes)
        w = np.zeros((c.shape[0], c.shape[1] // 8), np.uint32)
        for n in range(c.shape[1]):
            w[:, n // 8] |= c[:, n].astype(np.uint32) << np.uint32(4 * (7 - n % 8))
        return w

    def code_over_16(q_scale, q_scale_max, N):
        c = good_unpack(q_scale, N).astype(np.float64)
        return c / 16.0 * np.asarray(q_scale_max, np.float16).astype(np.float64)[None, :]

    def smax_by_group(q_scale, q_scale_max, N):
        s = good_scales(q_scale, q_scale_max, N)
        smax = np.asarray(q_scale_max, np.float16).astype(np.float64)
        return s / smax[None, :] * smax[:s.shape[0], None] if s.shape[0] <= N else s

    def codes_of_next_column(q_scale, q_scale_max, N):
        c = np.roll(good_unpack(q_scale, N).astype(np.float64), 1, axis=1)
        return (c + 1.0) / 16.0 * np.asarray(q_scale_max, np.float16).astype(np.float64)[None, :]

    planted = [("qscale_pack", msb_first_pack), ("two_level_scales", code_over_16),
               ("two_level_scales", smax_by_group), ("two_level_scales", codes_of_next_column)]
    pins = [test_qscale_nibble_order_hand_words, lambda: test_qscale_dequant_hand_values(golden_dir),
            test_qscale_each_group_and_column_its_own_factor, test_qscale_largest_code_is_the_one_level_scale]
    for name, bad in planted:
        with monkeypatch.context() as mp:
            mp.setattr(qo, name, bad)
            mp.setattr(oracle, name, bad)
            failed = 0
            for pin in pins:
                try:
                    pin()
                except (AssertionError, ValueError):
                    failed += 1
            assert failed > 0, f"no pin caught the planted slip in {name} ({bad.__name__})"
