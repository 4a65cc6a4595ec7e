"""Float64 CPU oracle of the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. It shares no code with the HIP path.

What the layer computes (notation: K input features, N outputs, M tokens,
gs rows per group, G = K / gs groups, b_g the bit width of group g):

1. The weight matrix is stored in *stored row order*: stored row j holds the
   weights of original input feature ``perm[j]`` (the act-order remapping of the
   ExLlamaV2 README, "EXL2 quantization", and the ``q_invperm`` tensor of the
   ExLlamaV2 blog, "How the EXL2 Quantization Pipeline Works", Step 3).
2. Integer codes ``q[j][n]`` in ``[0, 2^b_g)`` are packed into uint32 words
   (``q_weights``: packed variable-bit-width values, same Step 3). The 4-bit
   nibble order -- row i of a word at bits 4*i..4*i+3, least significant first --
   is the one the blog's kernel sketch unpacks ("How the Fused CUDA Kernel
   Works"). The pages give no bit layout for 3-, 5- or 6-bit codes; the layout
   used here is defined in :func:`block_field_map`.
3. Dequantization is ``w = s * (q - z)`` with one float16 scale ``s`` and one
   integer zero point ``z`` per (group, output column); a symmetric group uses
   ``z = 2^(b-1)`` (the blog's sketch subtracts 8 from a 4-bit code and
   multiplies by the scale; the GPTQ paragraph of the artifact page gives
   per-group scaling).
4. ``y[m][n] = sum_j x[m][perm[j]] * w[j][n]``: the fused matmul of the blog's
   sketch, here computed exactly in float64 (no float16 rounding of w or y).
5. Optionally the fused epilogue ``act(y + addend + bias) + residual`` (see
   :func:`apply_epilogue`), where the addend may be the on-the-fly LoRA
   update of :func:`lora_delta`.

6. EXL2 two-level scales (:func:`dequant_qscale`): 4-bit scale codes packed
   into ``q_scale`` and one float16 ``q_scale_max`` per output column.

Parity unpinned: the value (c + 1) / 16 that a two-level scale code c stands
for (a reading; the pages give no mapping). Every function is pinned by tests
that do not re-use its formula (see ``tests/test_oracle_pins.py``).
"""

from __future__ import annotations

import numpy as np

BITS_SUPPORTED = (2, 3, 4, 5, 6, 8)
GROUP_SIZES_SUPPORTED = (32, 64, 128)
BLOCK_ROWS = 32  # rows per packing block; a block of b-bit codes is exactly b words
PANEL = 16       # output columns per storage panel


# --------------------------------------------------------------------------
# Packed format
# --------------------------------------------------------------------------

def block_field_map(b: int) -> np.ndarray:
    """Where each bit of each code of a 32-row block lives.

    Returns an int array ``F`` of shape ``[32, b, 2]``: bit ``k`` (0 = least
    significant) of the code of row ``r`` of the block is stored in word
    ``F[r, k, 0]`` (0..b-1, relative to the block's first word) at bit
    position ``F[r, k, 1]`` (0..31).

    Layout ("half-word fields"). A block of 32 codes of b bits occupies b
    words. Each word is seen as two 16-bit halves, h = 0 (bits 0..15) and
    h = 1 (bits 16..31). With f = floor(16 / b) codes per half:

    * Regular rows r < 2*f*b: word t = r // (2f); inside the word u = r % (2f),
      half h = u // f, slot i = u % f; code bit k is at bit 16*h + b*i + k.
      For b in {2, 4, 8} every row is regular and this is the plain
      least-significant-first stream (4-bit: row i of a word at bits 4i..4i+3).
    * b in {3, 5} (rows 30 and 31 are left over, f*b = 15 leaves bit 15 of each
      half free): row 30 + h keeps its code bit k at word k, bit 16*h + 15.
    * b = 6 (rows 24..31 are left over, bits 12..15 of each half are free):
      row 24 + 4h + v (v = 0..3) keeps code bits 0..3 at word v, bits
      16h + 12 .. 16h + 15, and code bits 4, 5 at word 4 + v // 2, bits
      16h + 12 + 2*(v % 2) and the bit above it.

    Every one of the 32*b bits of the block is used exactly once (a tested
    property), so the map is a bijection between codes and block bits.
    """
    if b not in BITS_SUPPORTED:
        raise ValueError(f"unsupported bit width {b}")
    f = 16 // b
    regular = 2 * f * b
    F = np.zeros((BLOCK_ROWS, b, 2), dtype=np.int64)
    for r in range(BLOCK_ROWS):
        for k in range(b):
            if r < regular:
                t, u = divmod(r, 2 * f)
                h, i = divmod(u, f)
                F[r, k] = (t, 16 * h + b * i + k)
            elif b in (3, 5):
                h = r - 30
                F[r, k] = (k, 16 * h + 15)
            else:  # b == 6, rows 24..31
                h, v = divmod(r - 24, 4)
                if k < 4:
                    F[r, k] = (v, 16 * h + 12 + k)
                else:
                    F[r, k] = (4 + v // 2, 16 * h + 12 + 2 * (v % 2) + (k - 4))
    return F


def _check_bits(bits: np.ndarray, K: int, gs: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.int64).reshape(-1)
    if gs not in GROUP_SIZES_SUPPORTED:
        raise ValueError(f"unsupported group size {gs}")
    if K % gs != 0:
        raise ValueError("K must be a multiple of the group size")
    if bits.shape[0] != K // gs:
        raise ValueError("bits must hold one entry per group")
    for b in np.unique(bits):
        if int(b) not in BITS_SUPPORTED:
            raise ValueError(f"unsupported bit width {b}")
    return bits


def group_word_offsets(bits, gs: int) -> np.ndarray:
    """Word-row offset of each group: goff[g] = sum over g' < g of gs*b_g'/32.

    Group g occupies packed rows goff[g] .. goff[g+1]-1; its 32-row block c
    (c = 0 .. gs/32-1) occupies rows goff[g] + c*b_g .. goff[g] + (c+1)*b_g - 1.
    """
    bits = np.asarray(bits, dtype=np.int64).reshape(-1)
    goff = np.zeros(bits.shape[0] + 1, dtype=np.int64)
    goff[1:] = np.cumsum(bits * (gs // BLOCK_ROWS))
    return goff


def packed_rows(bits, gs: int) -> int:
    """Total number of packed word rows R; the packed matrix is uint32 [R][N]."""
    return int(group_word_offsets(bits, gs)[-1])


def pack(q: np.ndarray, bits, gs: int) -> np.ndarray:
    """Pack codes ``q`` (uint8 [K][N], stored row order) into uint32 [R][N].

    Column n of packed row (goff[g] + c*b + t) holds word t of 32-row block c of
    group g for output column n, laid out by :func:`block_field_map`. Output
    columns are the fastest-varying index, as the blog's kernel sketch indexes
    scales by group then output ("How the Fused CUDA Kernel Works").
    """
    q = np.asarray(q)
    K, N = q.shape
    bits = _check_bits(bits, K, gs)
    for b in np.unique(bits):
        rows = np.repeat(bits == b, gs)
        if rows.any() and int(q[rows].max(initial=0)) >= (1 << int(b)):
            raise ValueError(f"code out of range for {b}-bit group")
    goff = group_word_offsets(bits, gs)
    out = np.zeros((int(goff[-1]), N), dtype=np.uint32)
    nblk = gs // BLOCK_ROWS
    for g in range(bits.shape[0]):
        b = int(bits[g])
        F = block_field_map(b)
        for c in range(nblk):
            blk = q[g * gs + c * BLOCK_ROWS: g * gs + (c + 1) * BLOCK_ROWS].astype(np.uint32)
            words = np.zeros((b, N), dtype=np.uint32)
            for r in range(BLOCK_ROWS):
                for k in range(b):
                    t, pos = F[r, k]
                    words[t] |= ((blk[r] >> np.uint32(k)) & np.uint32(1)) << np.uint32(pos)
            base = int(goff[g]) + c * b
            out[base: base + b] = words
    return out


def unpack(packed: np.ndarray, bits, gs: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack`: uint32 [R][N] -> uint8 codes [K][N]."""
    packed = np.asarray(packed, dtype=np.uint32)
    bits = _check_bits(bits, K, gs)
    goff = group_word_offsets(bits, gs)
    if packed.shape[0] != int(goff[-1]):
        raise ValueError("packed row count does not match the bit map")
    N = packed.shape[1]
    q = np.zeros((K, N), dtype=np.uint8)
    nblk = gs // BLOCK_ROWS
    for g in range(bits.shape[0]):
        b = int(bits[g])
        F = block_field_map(b)
        for c in range(nblk):
            base = int(goff[g]) + c * b
            for r in range(BLOCK_ROWS):
                code = np.zeros(N, dtype=np.uint32)
                for k in range(b):
                    t, pos = F[r, k]
                    code |= ((packed[base + t] >> np.uint32(pos)) & np.uint32(1)) << np.uint32(k)
                q[g * gs + c * BLOCK_ROWS + r] = code.astype(np.uint8)
    return q


def panel_layout(words: np.ndarray) -> np.ndarray:
    """Storage order of the packed words: 16-column panels, one after another.

    ``words`` is the word matrix [R][N] of :func:`pack`. The stored array is
    [ceil(N/16)][R][16]: word (r, n) sits at panel n // 16, row r, slot
    n % 16, and panel columns past N are zero. Each panel's R rows are thus
    contiguous (a reader of 16 columns streams one contiguous region).
    """
    words = np.asarray(words, dtype=np.uint32)
    R, N = words.shape
    npan = (N + PANEL - 1) // PANEL
    out = np.zeros((npan, R, PANEL), dtype=np.uint32)
    for n in range(N):
        out[n // PANEL, :, n % PANEL] = words[:, n]
    return out


def panel_unlayout(panels: np.ndarray, N: int) -> np.ndarray:
    """Inverse of :func:`panel_layout`: [ceil(N/16)][R][16] -> [R][N]."""
    panels = np.asarray(panels, dtype=np.uint32)
    R = panels.shape[1]
    words = np.zeros((R, N), dtype=np.uint32)
    for n in range(N):
        words[:, n] = panels[n // PANEL, :, n % PANEL]
    return words


# --------------------------------------------------------------------------
# Dequantization and the layer
# --------------------------------------------------------------------------

def zero_points(zeros, bits, N: int) -> np.ndarray:
    """Per-(group, column) zero point as float64 [G][N].

    ``zeros`` is an integer array [G][N], or None for symmetric groups, whose
    zero point is the midpoint 2^(b-1) of the code range (8 for 4-bit codes,
    as in the blog's kernel sketch).
    """
    bits = np.asarray(bits, dtype=np.int64).reshape(-1)
    if zeros is None:
        return np.repeat((2.0 ** (bits - 1))[:, None], N, axis=1)
    z = np.asarray(zeros, dtype=np.float64)
    if z.shape != (bits.shape[0], N):
        raise ValueError("zeros must be [G][N]")
    return z


def dequant(q, scales, zeros, bits, gs: int) -> np.ndarray:
    """Dequantized weights w[j][n] = s[g][n] * (q[j][n] - z[g][n]), g = j // gs, in float64.

    Exact: s has 11 significant bits and |q - z| <= 255, so the product needs
    at most 19 bits and float64 holds it without rounding.
    """
    q = np.asarray(q)
    K, N = q.shape
    bits = _check_bits(bits, K, gs)
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape != (bits.shape[0], N):
        raise ValueError("scales must be [G][N]")
    z = zero_points(zeros, bits, N)
    s_rows = np.repeat(s, gs, axis=0)
    z_rows = np.repeat(z, gs, axis=0)
    return s_rows * (q.astype(np.float64) - z_rows)


def dequant_fp16(q, scales, zeros, bits, gs: int) -> np.ndarray:
    """The dequantized weights rounded once to float16 (round to nearest even).

    numpy converts float64 to float16 with a single correctly rounded step.
    """
    return dequant(q, scales, zeros, bits, gs).astype(np.float16)


def _perm_or_identity(perm, K: int) -> np.ndarray:
    if perm is None:
        return np.arange(K, dtype=np.int64)
    p = np.asarray(perm, dtype=np.int64).reshape(-1)
    if p.shape[0] != K or not np.array_equal(np.sort(p), np.arange(K)):
        raise ValueError("perm must be a permutation of 0..K-1")
    return p


def qlinear(x, q, scales, zeros, bits, gs: int, perm=None) -> np.ndarray:
    """y = x[:, perm] @ w in float64, with w unrounded (the layer's exact value).

    ``x`` is [M][K] in original feature order (float16 values); ``q`` is in
    stored row order; ``perm[j]`` is the original feature held by stored row j.
    """
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    q = np.asarray(q)
    K = q.shape[0]
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    p = _perm_or_identity(perm, K)
    w = dequant(q, scales, zeros, bits, gs)
    return x[:, p] @ w


def qlinear_gidx(x, q, scales, zeros, bits, gs: int, perm=None) -> np.ndarray:
    """Second path: scatter the weights back to original feature order.

    The GPTQ view of act-order: original feature k belongs to group
    g_idx[k] = invperm[k] // gs, with invperm the inverse permutation. Build
    W_orig[k][n] = s[g_idx[k]][n] * (q[invperm[k]][n] - z[g_idx[k]][n]) and
    return x @ W_orig. Equal to :func:`qlinear` up to float64 summation order.
    """
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    q = np.asarray(q)
    K, N = q.shape
    bits = _check_bits(bits, K, gs)
    p = _perm_or_identity(perm, K)
    invperm = np.empty(K, dtype=np.int64)
    invperm[p] = np.arange(K)
    g_idx = invperm // gs
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = zero_points(zeros, bits, N)
    w_orig = s[g_idx] * (q[invperm].astype(np.float64) - z[g_idx])
    return x @ w_orig


def qlinear_bruteforce(x, q, scales, zeros, bits, gs: int, perm=None) -> np.ndarray:
    """Pure-Python triple loop of the same definition (tiny inputs only)."""
    x = np.asarray(x, dtype=np.float16)
    q = np.asarray(q)
    K, N = q.shape
    M = x.shape[0]
    bits = [int(b) for b in np.asarray(bits).reshape(-1)]
    p = list(range(K)) if perm is None else [int(v) for v in np.asarray(perm).reshape(-1)]
    s = np.asarray(scales, dtype=np.float16)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for j in range(K):
                g = j // gs
                zz = float(2 ** (bits[g] - 1)) if zeros is None else float(zeros[g][n])
                acc += float(x[m][p[j]]) * (float(s[g][n]) * (float(q[j][n]) - zz))
            y[m][n] = acc
    return np.array(y, dtype=np.float64)


# ---------------------------------------------------------------- epilogue
#
# The artifact page's GPTQ paragraph says the kernels fuse scaling, addition
# and activation into one call. Reading (the pages name neither the terms nor
# the activation): addition is a per-output bias and a residual, the
# activation is SiLU (the Llama MLP's), and the order is that of a layer
# followed by its activation and then the residual stream. A float32 addend
# (the LoRA update below) is part of the layer's own output, so it joins acc
# before the bias:
#   y[m][n] = act(acc[m][n] + addend[m][n] + bias[n]) + residual[m][n]

ACT_NONE = 0
ACT_SILU = 1


def silu(v) -> np.ndarray:
    """SiLU in float64: v * sigmoid(v) = v / (1 + exp(-v))."""
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def apply_epilogue(acc, bias=None, residual=None, activation: int = ACT_NONE, addend=None) -> np.ndarray:
    """The fused epilogue on float64 layer outputs acc [M][N]; bias [N],
    residual [M][N] and addend [M][N] are float16, float32 or float64 (None:
    absent)."""
    y = np.asarray(acc, np.float64).copy()
    if addend is not None:
        y = y + np.asarray(addend, np.float64)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    if activation == ACT_SILU:
        y = silu(y)
    elif activation != ACT_NONE:
        raise ValueError(f"unknown activation {activation}")
    if residual is not None:
        y = y + np.asarray(residual, np.float64)
    return y


# ---------------------------------------------------------------- LoRA
#
# The artifact page lists LoRA adapters among the capabilities: an adapter is
# a low-rank pair A [K][r], B [r][N] whose product updates the layer's
# weights, either merged into them before inference or applied on the fly in
# the forward pass; several adapters combine with weights. Reading: applied
# on the fly, adapter i with weight s_i adds s_i (x A_i) B_i to the layer's
# output, x in its original feature order (the adapter belongs to the
# unquantized layer, which knows nothing of the act-order permutation). Since
# x (W + s A B) = x W + s (x A) B, this is the merged layer's output.

def lora_delta(x, adapters) -> np.ndarray:
    """sum_i s_i (x A_i) B_i in float64. x [M][K]; adapters: a sequence of
    (A [K][r], B [r][N], s)."""
    x = np.asarray(x, np.float64)
    out = None
    for A, B, s in adapters:
        t = x @ np.asarray(A, np.float64)                 # [M][r], the down-projection
        d = float(s) * (t @ np.asarray(B, np.float64))    # [M][N], the up-projection
        out = d if out is None else out + d
    if out is None:
        raise ValueError("at least one adapter")
    return out


# ---------------------------------------------------------------- two-level scales
#
# The EXL2 tensor set (ExLlamaV2 blog, "How the EXL2 Quantization Pipeline
# Works Under the Hood", Step 3) keeps the group scales as 4-bit codes packed
# into uint32 words (q_scale) beside one float16 maximum scale per output
# feature (q_scale_max), and the blog's kernel sketch ("How the Fused CUDA
# Kernel Works") dequantizes a 4-bit weight as (w - 8) * scale * scale_max.
# The pages give neither the value a scale code stands for nor the order of
# the codes in a word. Reading:
#   * code c in [0, 15] stands for the relative scale (c + 1) / 16, so the
#     largest code is the maximum scale itself and no code means zero;
#   * the codes run along the output features, 8 per word, least significant
#     nibble first (the sketch's nibble order for q_weights): column n of
#     group g is nibble n % 8 of word q_scale[g][n // 8];
#   * the groups are symmetric, z = 2^(b-1) (the sketch subtracts the
#     midpoint 8 of a 4-bit code);
#   * w = (q - z) * ((c + 1) / 16) * scale_max[n], in that order (the
#     sketch's product; every factor is exact, so the order does not change
#     the value).
# Parity unpinned: the mapping c -> (c + 1) / 16 itself. No file and no formula
# of the pages fixes it; the tests pin the packing, the indexing and the
# product against the one-level definitions above.

QSCALE_CODES_PER_WORD = 8


def qscale_pack(codes) -> np.ndarray:
    """Scale codes uint8 [G][N] (each < 16, N % 8 == 0) -> q_scale uint32 [G][N/8]."""
    c = np.asarray(codes)
    if c.ndim != 2 or c.shape[1] % QSCALE_CODES_PER_WORD:
        raise ValueError("codes must be [G][N] with N a multiple of 8")
    if c.size and int(c.max()) > 15:
        raise ValueError("scale codes are 4-bit")
    G, N = c.shape
    words = np.zeros((G, N // QSCALE_CODES_PER_WORD), dtype=np.uint32)
    for n in range(N):
        words[:, n // 8] |= c[:, n].astype(np.uint32) << np.uint32(4 * (n % 8))
    return words


def qscale_unpack(words, N: int) -> np.ndarray:
    """Inverse of :func:`qscale_pack`: uint32 [G][N/8] -> uint8 codes [G][N]."""
    w = np.asarray(words, dtype=np.uint32)
    if w.ndim != 2 or w.shape[1] * QSCALE_CODES_PER_WORD != N:
        raise ValueError("q_scale must be [G][N/8]")
    c = np.zeros((w.shape[0], N), dtype=np.uint8)
    for n in range(N):
        c[:, n] = ((w[:, n // 8] >> np.uint32(4 * (n % 8))) & np.uint32(15)).astype(np.uint8)
    return c


def two_level_scales(q_scale, q_scale_max, N: int) -> np.ndarray:
    """The effective group scales scale[g][n] * scale_max[n] in float64 [G][N]."""
    c = qscale_unpack(q_scale, N).astype(np.float64)
    smax = np.asarray(q_scale_max, dtype=np.float16).astype(np.float64).reshape(-1)
    if smax.shape[0] != N:
        raise ValueError("q_scale_max must hold one float16 per output feature")
    return ((c + 1.0) / 16.0) * smax[None, :]


def dequant_qscale(q, q_scale, q_scale_max, bits, gs: int) -> np.ndarray:
    """w[j][n] = (q[j][n] - 2^(b_g - 1)) * scale[g][n] * scale_max[n], g = j // gs, float64.

    Exact: |q - z| <= 128 (8 bits), c + 1 <= 16 and scale_max has 11
    significant bits, so the product needs at most 24 bits.
    """
    q = np.asarray(q)
    K, N = q.shape
    bits = _check_bits(bits, K, gs)
    s = two_level_scales(q_scale, q_scale_max, N)
    if s.shape[0] != bits.shape[0]:
        raise ValueError("q_scale must hold one row per group")
    z = zero_points(None, bits, N)
    return (q.astype(np.float64) - np.repeat(z, gs, axis=0)) * np.repeat(s, gs, axis=0)


def dequant_qscale_fp16(q, q_scale, q_scale_max, bits, gs: int) -> np.ndarray:
    """The two-level dequantized weights rounded once to float16."""
    return dequant_qscale(q, q_scale, q_scale_max, bits, gs).astype(np.float16)


def qlinear_qscale(x, q, q_scale, q_scale_max, bits, gs: int, perm=None) -> np.ndarray:
    """y = x[:, perm] @ w in float64 with the two-level weights of :func:`dequant_qscale`."""
    x = np.asarray(x, dtype=np.float16).astype(np.float64)
    q = np.asarray(q)
    K = q.shape[0]
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [M][K]")
    p = _perm_or_identity(perm, K)
    return x[:, p] @ dequant_qscale(q, q_scale, q_scale_max, bits, gs)
