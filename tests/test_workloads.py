"""The seeded input generator: bit maps, shapes, determinism, byte accounting."""

import numpy as np

import workloads as wl


def test_exl2_bit_maps():
    # 10 % of 128 groups is 12.8: largest remainder, ties to the wider code
    assert wl.group_counts(128, wl.EXL2_40) == [(6, 13), (5, 13), (4, 64), (3, 38)]
    assert wl.group_counts(256, wl.EXL2_25) == [(3, 128), (2, 128)]
    assert wl.group_counts(896, wl.EXL2_25) == [(3, 448), (2, 448)]
    bm = wl.bit_map(wl.EXL2_MIXED)
    assert bm.shape == (128,) and bm.dtype == np.uint8
    assert abs(bm.mean() - 4.0078125) < 1e-12
    assert (np.diff(bm.astype(int)) <= 0).all()  # widest first, contiguous runs


def test_generate_tiny_is_deterministic_and_in_range():
    a = wl.generate(wl.TINY)
    b = wl.generate(wl.TINY)
    for f in ("q", "zeros", "scales", "x"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert a.perm is None
    assert a.q.shape == (256, 512) and a.q.max() <= 15
    assert a.zeros.shape == (8, 512) and a.zeros.max() <= 15
    assert a.scales.dtype == np.float16 and 0.0049 < a.scales.min() and a.scales.max() < 0.0201
    assert a.x.shape == (1, 256) and a.x.dtype == np.float16


def test_generate_mixed_codes_respect_group_width():
    inp = wl.generate(wl.EXL2_MIXED, M=1)
    assert inp.zeros is None
    assert sorted(inp.perm.tolist()) == list(range(4096))
    rows_b = np.repeat(inp.bits, 32)
    for b in (3, 4, 5, 6):
        sel = inp.q[rows_b == b]
        assert sel.max() == (1 << b) - 1 and sel.min() == 0


def test_weight_bytes_match_hand_counts():
    # q at b bits + float16 scales + 4-bit zeros
    assert wl.weight_bytes(wl.TINY) == 65536 + 8192 + 2048
    assert wl.weight_bytes(wl.LLAMA7B_DECODE[0]) == 8388608 + 262144 + 65536
    assert wl.weight_bytes(wl.LLAMA7B_DECODE[1]) == 22544384 + 704512 + 176128
    assert wl.weight_bytes(wl.EXL2_MIXED) == 22588416 + 2818048
    assert wl.weight_bytes(wl.LLAMA70B_EXL2[0]) == 73400320 + 14680064
    assert wl.weight_bytes(wl.LLAMA70B_EXL2[1]) == 73400320 + 14680064
