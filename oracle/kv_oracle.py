"""CPU oracle of the quantized KV-cache codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. It shares no code with the HIP path.

The ExLlamaV2 blog lists Q4, Q6 and Q8 cache modes beside FP16 (the
comparison table, and "How to Use Effectively", Step 2: Q8 saves 50% of the
cache memory, Q4 75%), and the artifact page names quantized KV-cache
operations among the kernels. The pages give no block size, scale format,
rounding or bit layout, so the format below is this project's own reading,
chosen so that the savings hold (b bits per element plus one float16 scale
per block of G elements: Q4 at G = 128 keeps 26% of the FP16 bytes, Q8 51%):

* a tensor is rows of D float16 values (a head's key or value vector for one
  token is one row); each row is cut into blocks of G consecutive elements,
  G in {32, 64, 128}, D a multiple of G;
* per block, in float32: m = max |x|, scale s = RNE_fp16(m / qmax) with
  qmax = 2^(b-1) - 1 (7, 31, 127), so that the largest magnitude maps to
  +-qmax;
* code q = clamp(rint(x / s), -2^(b-1), 2^(b-1) - 1) + 2^(b-1), in
  [0, 2^b), rint rounding half to even, x / s a float32 division; a block
  with s = 0 stores the midpoint code for every element;
* the codes of a block form a little-endian bit stream of G b / 32 uint32
  words: element i at bits b i .. b i + b - 1 (the nibble order of the blog's
  4-bit weights for b = 4; a 6-bit code may span two words);
* dequantized value x' = RNE_fp16(s (q - 2^(b-1))) (an exact product, one
  rounding).

Both the kernel and this oracle decide the integer codes in float32 (the
pages fix no precision; float32 is the kernel's), so the codes must agree bit
for bit. Parity unpinned: nothing here; the tests pin the format by hand
examples, brute force over all codes, error bounds and planted slips.
"""

from __future__ import annotations

import numpy as np

KV_BITS = (4, 6, 8)
KV_GROUPS = (32, 64, 128)


def _check(D: int, bits: int, group: int) -> None:
    if bits not in KV_BITS:
        raise ValueError(f"unsupported cache width {bits}")
    if group not in KV_GROUPS or D % group != 0 or D <= 0:
        raise ValueError("D must be a positive multiple of the block size 32, 64 or 128")


def kv_scales(x, bits: int, group: int) -> np.ndarray:
    """Per-block float16 scales [rows][D / G] = RNE_fp16(float32(max|x|) / qmax)."""
    x = np.asarray(x, dtype=np.float16)
    rows, D = x.shape
    _check(D, bits, group)
    qmax = np.float32((1 << (bits - 1)) - 1)
    m = np.abs(x.astype(np.float32)).reshape(rows, D // group, group).max(axis=2)
    return (m / qmax).astype(np.float16)


def kv_codes(x, scales, bits: int, group: int) -> np.ndarray:
    """Integer codes uint8 [rows][D] of x under the given block scales."""
    x = np.asarray(x, dtype=np.float16)
    rows, D = x.shape
    _check(D, bits, group)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float32), group, axis=1)
    xf = x.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s > 0, np.rint(xf / np.where(s > 0, s, np.float32(1))), np.float32(0))
    half = 1 << (bits - 1)
    q = np.clip(r, -half, half - 1) + half
    return q.astype(np.uint8)


def kv_pack(codes, bits: int, group: int) -> np.ndarray:
    """Codes uint8 [rows][D] -> words uint32 [rows][D * bits / 32], block by block."""
    c = np.asarray(codes, dtype=np.uint64)
    rows, D = c.shape
    _check(D, bits, group)
    if c.size and int(c.max()) >= (1 << bits):
        raise ValueError("code out of range")
    wpb = group * bits // 32
    out = np.zeros((rows, D // group * wpb), dtype=np.uint64)
    for i in range(D):
        blk, e = divmod(i, group)
        pos = e * bits
        w, sh = divmod(pos, 32)
        base = blk * wpb + w
        out[:, base] |= (c[:, i] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            out[:, base + 1] |= c[:, i] >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def kv_unpack(words, D: int, bits: int, group: int) -> np.ndarray:
    """Inverse of :func:`kv_pack`."""
    w = np.asarray(words, dtype=np.uint64)
    _check(D, bits, group)
    rows = w.shape[0]
    wpb = group * bits // 32
    if w.shape[1] != D // group * wpb:
        raise ValueError("word count does not match D and the width")
    mask = np.uint64((1 << bits) - 1)
    c = np.zeros((rows, D), dtype=np.uint8)
    for i in range(D):
        blk, e = divmod(i, group)
        pos = e * bits
        wi, sh = divmod(pos, 32)
        base = blk * wpb + wi
        v = w[:, base] >> np.uint64(sh)
        if sh + bits > 32:
            v |= w[:, base + 1] << np.uint64(32 - sh)
        c[:, i] = (v & mask).astype(np.uint8)
    return c


def kv_quantize(x, bits: int, group: int):
    """x float16 [rows][D] -> (words uint32 [rows][D b / 32], scales float16 [rows][D / G])."""
    s = kv_scales(x, bits, group)
    return kv_pack(kv_codes(x, s, bits, group), bits, group), s


def kv_dequantize(words, scales, D: int, bits: int, group: int) -> np.ndarray:
    """float16 [rows][D]: RNE_fp16(s * (q - 2^(b-1))), computed exactly in float64 then rounded once."""
    q = kv_unpack(words, D, bits, group).astype(np.float64) - float(1 << (bits - 1))
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), group, axis=1)
    return (s * q).astype(np.float16)


def kv_bytes_per_element(bits: int, group: int) -> float:
    """Stored bytes per cached element: b / 8 of code plus 2 / G of scale."""
    return bits / 8 + 2 / group
