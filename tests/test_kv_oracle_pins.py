"""Pins of the KV-cache codec oracle (oracle/kv_oracle.py) against what
arithmetic fixes: hand-derived blocks, brute force over every code, error
bounds, the byte savings the pages quote, and planted slips."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import kv_oracle as ko


def _block(values, group=32, dtype=np.float16):
    x = np.zeros((1, group), dtype)
    x[0, :len(values)] = values
    return x


def test_hand_blocks(golden_dir):
    with open(os.path.join(golden_dir, "kv_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        b, G = e["bits"], e["group"]
        x = _block(e["x"], G)
        words, s = oracle.kv_quantize(x, b, G)
        assert int(s.view(np.uint16)[0, 0]) == int(e["scale_bits"], 16), e["derivation"]
        for i, w in enumerate(e["words"]):
            assert int(words[0, i]) == int(w, 16), (e["derivation"], i, hex(int(words[0, i])))
        xh = oracle.kv_dequantize(words, s, G, b, G)
        assert np.array_equal(xh[0, :len(e["xhat"])], np.array(e["xhat"], np.float16)), e["derivation"]


def test_pack_hand_words():
    # 4-bit: codes 0..7 give 0x76543210 (the nibble order of the blog's 4-bit weights).
    c = np.zeros((1, 32), np.uint8)
    c[0, :8] = np.arange(8)
    assert int(oracle.kv_pack(c, 4, 32)[0, 0]) == 0x76543210
    # 8-bit: bytes 0x10, 0x32, 0x54, 0x76 give 0x76543210.
    c = np.zeros((1, 32), np.uint8)
    c[0, :4] = [0x10, 0x32, 0x54, 0x76]
    assert int(oracle.kv_pack(c, 8, 32)[0, 0]) == 0x76543210
    # 6-bit: element 5 sits at bits 30..35, across the first word boundary.
    c = np.zeros((1, 32), np.uint8)
    c[0, 5] = 63
    w = oracle.kv_pack(c, 6, 32)
    assert w.shape == (1, 6) and int(w[0, 0]) == 0xC0000000 and int(w[0, 1]) == 0x0000000F
    assert not w[0, 2:].any()
    # a block of G elements is G * b / 32 words, blocks one after another
    c = np.zeros((1, 64), np.uint8)
    c[0, 32] = 5
    assert int(oracle.kv_pack(c, 6, 32)[0, 6]) == 5


@pytest.mark.parametrize("bits", (4, 6, 8))
@pytest.mark.parametrize("group", (32, 64, 128))
def test_pack_round_trip(bits, group):
    rng = np.random.default_rng(bits * group)
    c = rng.integers(0, 1 << bits, size=(3, 2 * group), dtype=np.uint8)
    assert np.array_equal(oracle.kv_unpack(oracle.kv_pack(c, bits, group), 2 * group, bits, group), c)


@pytest.mark.parametrize("bits", (4, 6, 8))
def test_codes_are_the_nearest_with_ties_to_even(bits):
    # Brute force: every code is the one of all 2^b whose value s * (q - z) is
    # nearest to x in exact arithmetic, ties to the even integer q - z. (A
    # float32 division cannot turn a non-tie into a tie here: x and s have
    # 11-bit significands, so x / s misses a half-integer by more than 2^-22
    # relative, above float32's rounding.)
    from fractions import Fraction
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal((6, 32)) * rng.uniform(0.01, 5.0, size=(6, 1))).astype(np.float16)
    x[0, :4] = [1.25, -1.25, 0.75, 3.5]     # exact ties for a scale that divides them
    s = oracle.kv_scales(x, bits, 32)
    q = oracle.kv_codes(x, s, bits, 32)
    z = 1 << (bits - 1)
    for r in range(6):
        sf = Fraction(float(s[r, 0]))
        for i in range(32):
            xf = Fraction(float(x[r, i]))
            best = min(range(1 << bits), key=lambda c: (abs(xf - sf * (c - z)), (c - z) % 2))
            assert int(q[r, i]) == best, (r, i, float(x[r, i]), float(s[r, 0]))


@pytest.mark.parametrize("bits", (4, 6, 8))
@pytest.mark.parametrize("group", (32, 128))
def test_error_bound_and_scale(bits, group):
    rng = np.random.default_rng(100 + bits + group)
    x = (rng.standard_normal((50, 2 * group)) * 3).astype(np.float16)
    words, s = oracle.kv_quantize(x, bits, group)
    xh = oracle.kv_dequantize(words, s, 2 * group, bits, group).astype(np.float64)
    sr = np.repeat(s.astype(np.float64), group, axis=1)
    qmax = (1 << (bits - 1)) - 1
    m = np.abs(x.astype(np.float64)).reshape(50, 2, group).max(axis=2)
    assert np.all(np.abs(s.astype(np.float64) * qmax - m) <= m * 2.0 ** -11 * qmax)   # s within half an fp16 ulp of m / qmax
    ulp = np.spacing(np.abs(xh).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(x.astype(np.float64) - xh) <= sr * (0.5 + 2.0 ** -9) + ulp / 2)


def test_zero_block_and_savings():
    x = np.zeros((2, 64), np.float16)
    x[1, 32:] = 1.0
    for b in (4, 6, 8):
        w, s = oracle.kv_quantize(x, b, 32)
        assert s[0, 0] == 0 and s[0, 1] == 0
        assert (oracle.kv_unpack(w, 64, b, 32)[0] == 1 << (b - 1)).all()
        assert (oracle.kv_dequantize(w, s, 64, b, 32)[0] == 0).all()
        assert (oracle.kv_dequantize(w, s, 64, b, 32)[1, 32:] == 1.0).all()
    # the savings the blog quotes against FP16 (Q4: 75%, Q8: 50%), with the
    # block scales of G = 128 counted
    assert abs(1 - oracle.kv_bytes_per_element(4, 128) / 2 - 0.75) < 0.01
    assert abs(1 - oracle.kv_bytes_per_element(8, 128) / 2 - 0.50) < 0.01


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.kv_quantize(np.zeros((1, 48), np.float16), 4, 32)
    with pytest.raises(ValueError):
        oracle.kv_quantize(np.zeros((1, 32), np.float16), 5, 32)
    with pytest.raises(ValueError):
        oracle.kv_pack(np.full((1, 32), 16, np.uint8), 4, 32)


def test_planted_mistakes_are_caught(golden_dir, monkeypatch):
    good_codes, good_scales, good_pack = ko.kv_codes, ko.kv_scales, ko.kv_pack

    def half_away(x, scales, bits, group):
        s = np.repeat(np.asarray(scales, np.float16).astype(np.float32), group, axis=1)
        xf = np.asarray(x, np.float16).astype(np.float32)
        r = np.where(s > 0, np.sign(xf) * np.floor(np.abs(xf) / np.where(s > 0, s, 1) + 0.5), 0)
        half = 1 << (bits - 1)
        return (np.clip(r, -half, half - 1) + half).astype(np.uint8)

    def scale_by_half_range(x, bits, group):
        x = np.asarray(x, np.float16)
        rows, D = x.shape
        m = np.abs(x.astype(np.float32)).reshape(rows, D // group, group).max(axis=2)
        return (m / np.float32(1 << (bits - 1))).astype(np.float16)

    def msb_first(codes, bits, group):
        c = np.asarray(codes)
        rev = np.zeros_like(c)
        for k in range(bits):
            rev |= ((c >> k) & 1) << (bits - 1 - k)
        return good_pack(rev, bits, group)

    def twos_complement(x, scales, bits, group):
        q = good_codes(x, scales, bits, group).astype(np.int64) - (1 << (bits - 1))
        return (q & ((1 << bits) - 1)).astype(np.uint8)

    planted = [("kv_codes", half_away), ("kv_scales", scale_by_half_range), ("kv_pack", msb_first),
               ("kv_codes", twos_complement)]
    pins = [lambda: test_hand_blocks(golden_dir), test_pack_hand_words,
            lambda: test_codes_are_the_nearest_with_ties_to_even(4)]
    for name, bad in planted:
        with monkeypatch.context() as mp:
            mp.setattr(ko, name, bad)
            failed = 0
            for pin in pins:
                try:
                    pin()
                except (AssertionError, ValueError):
                    failed += 1
            assert failed > 0, f"no pin caught the planted slip in {name} ({bad.__name__})"
