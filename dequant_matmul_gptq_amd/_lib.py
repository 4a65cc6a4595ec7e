"""ctypes binding of libqlinear.so (argument marshalling only).

Every function here checks tensor devices and shapes, passes raw pointers and
the current HIP stream to the C entry point of the same name, and raises
QlinearError on a non-zero status. All computation happens in the library's
gfx950 kernels; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlinear.so")

MAX_RUNS = 64
GEMV_MAX_M = 16
MAX_GROUP = 8
PANEL = 16

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_MISALIGNED = 3
ERR_WORKSPACE = 4
ERR_HIP = 5

EXPORTS = (
    "qlinear_status_string",
    "qlinear_layout_init",
    "qlinear_group_order",
    "qlinear_pack_weights",
    "qlinear_unpack",
    "qlinear_dequant",
    "qlinear_qgemv_workspace_bytes",
    "qlinear_qgemv",
    "qlinear_qgemv_noalloc",
    "qlinear_qgemv_grouped",
    "qlinear_qgemm_workspace_bytes",
    "qlinear_qgemm",
    "qlinear_qgemv_fused",
    "qlinear_qgemm_fused",
    "qlinear_lora_workspace_bytes",
    "qlinear_lora_delta",
    "qlinear_read_floor",
    "qlinear_pack_qscale",
    "qlinear_dequant_qscale",
    "qlinear_qgemv_qscale",
    "qlinear_qgemm_qscale",
    "qlinear_kv_quant",
    "qlinear_kv_dequant",
)

ACT_NONE = 0
ACT_SILU = 1


class QlinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class qlinear_layout(ctypes.Structure):
    _fields_ = [
        ("K", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("packed_rows", ctypes.c_int32),
        ("nruns", ctypes.c_int32),
        ("run_group", ctypes.c_int32 * (MAX_RUNS + 1)),
        ("run_row", ctypes.c_int32 * (MAX_RUNS + 1)),
        ("run_bits", ctypes.c_int32 * MAX_RUNS),
        ("packed_words", ctypes.c_int64),
    ]


class qlinear_epilogue(ctypes.Structure):
    _fields_ = [
        ("bias", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
        ("activation", ctypes.c_int32),
        ("addend", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqlinear.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m dequant_matmul_gptq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lp = ctypes.POINTER(qlinear_layout)
        L.qlinear_status_string.restype = ctypes.c_char_p
        L.qlinear_status_string.argtypes = [ctypes.c_int]
        L.qlinear_layout_init.argtypes = [lp, i32, i32, i32, vp]
        L.qlinear_group_order.argtypes = [vp, i32, vp]
        L.qlinear_pack_weights.argtypes = [lp, vp, vp, vp]
        L.qlinear_unpack.argtypes = [lp, vp, vp, vp]
        L.qlinear_dequant.argtypes = [lp, vp, vp, vp, vp, vp]
        L.qlinear_qgemv_workspace_bytes.argtypes = [lp, ctypes.POINTER(sz)]
        L.qlinear_qgemv.argtypes = [lp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qlinear_qgemv_noalloc.argtypes = [lp, vp, i32, vp, vp, vp, vp, vp, vp]
        pp = ctypes.POINTER(vp)
        L.qlinear_qgemv_grouped.argtypes = [lp, vp, i32, i32, pp, pp, pp, vp, pp, vp, sz, vp]
        L.qlinear_qgemm_workspace_bytes.argtypes = [lp, i32, ctypes.POINTER(sz)]
        L.qlinear_qgemm.argtypes = [lp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        ep = ctypes.POINTER(qlinear_epilogue)
        L.qlinear_qgemv_fused.argtypes = [lp, vp, i32, vp, vp, vp, vp, ep, vp, vp, sz, vp]
        L.qlinear_qgemm_fused.argtypes = [lp, vp, i32, vp, vp, vp, vp, ep, vp, vp, sz, vp]
        L.qlinear_lora_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.qlinear_lora_delta.argtypes = [vp, i32, i32, vp, i32, vp, i32, ctypes.c_float, i32, vp, vp, sz, vp]
        L.qlinear_read_floor.argtypes = [vp, sz, i32, i32, ctypes.c_uint32, vp, vp]
        L.qlinear_pack_qscale.argtypes = [vp, i32, i32, vp, vp]
        L.qlinear_dequant_qscale.argtypes = [lp, vp, vp, vp, vp, vp]
        L.qlinear_qgemv_qscale.argtypes = [lp, vp, i32, vp, vp, vp, vp, ep, vp, vp, sz, vp]
        L.qlinear_qgemm_qscale.argtypes = [lp, vp, i32, vp, vp, vp, vp, ep, vp, vp, sz, vp]
        i64 = ctypes.c_int64
        L.qlinear_kv_quant.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
        L.qlinear_kv_dequant.argtypes = [vp, vp, i64, i32, i32, i32, vp, vp]
        for name in EXPORTS[1:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qlinear_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise QlinearError(status, what)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple | None = None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Layout:
    """Host description of a packed K x N matrix (wraps qlinear_layout_init)."""

    def __init__(self, K: int, N: int, group_size: int, bits):
        b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8).reshape(-1))
        self.bits = b
        self.c = qlinear_layout()
        _check(lib().qlinear_layout_init(ctypes.byref(self.c), int(K), int(N), int(group_size),
                                         b.ctypes.data_as(ctypes.c_void_p)), "qlinear_layout_init")
        self.K, self.N, self.group_size = int(K), int(N), int(group_size)
        self.groups = int(self.c.groups)
        self.packed_rows = int(self.c.packed_rows)
        self.nruns = int(self.c.nruns)
        self.panels = (self.N + PANEL - 1) // PANEL
        # packed words in storage order: 16-column panels of packed_rows rows
        self.qweight_shape = (self.panels, self.packed_rows, PANEL)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def group_order(bits) -> np.ndarray:
    """qlinear_group_order: the storage order of the groups (int32, original
    index of the group stored i-th) that leaves at most 6 width runs."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8).reshape(-1))
    order = np.empty(b.size, dtype=np.int32)
    _check(lib().qlinear_group_order(b.ctypes.data_as(ctypes.c_void_p), int(b.size),
                                     order.ctypes.data_as(ctypes.c_void_p)), "qlinear_group_order")
    return order


def reorder_groups(order, group_size: int, bits, q: torch.Tensor, per_group=(), perm: torch.Tensor | None = None):
    """Move the groups of a matrix into `order` (from group_order), once, before packing.

    q is uint8 [K][N] in stored row order; each tensor of per_group has one row
    per group (scales, zero points, two-level scale codes); perm is the int32
    act-order permutation or None. Returns (bits, q, per_group, perm): group
    order[i]'s rows at position i, and perm composed with that row move
    (stored row i * group_size + r takes perm[order[i] * group_size + r]), so
    the product is unchanged. Tensors stay on their devices.
    """
    o = np.asarray(order, dtype=np.int64)
    rows = (o[:, None] * int(group_size) + np.arange(int(group_size))).reshape(-1)
    r = torch.from_numpy(rows).to(q.device)
    q2 = q.index_select(0, r)
    pg = tuple(t.index_select(0, torch.from_numpy(o).to(t.device)) for t in per_group)
    if perm is None:
        p2 = r.to(torch.int32)
    else:
        p2 = perm.index_select(0, r.to(perm.device)).to(torch.int32)
    return np.asarray(bits, dtype=np.uint8)[o], q2, pg, p2


def pack_weights(layout: Layout, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """q uint8 [K][N] (stored order) -> packed int32 [ceil(N/16)][packed_rows][16] (uint32 bit patterns)."""
    _dev(q, "q", torch.uint8, (layout.K, layout.N))
    if out is None:
        out = torch.empty(layout.qweight_shape, dtype=torch.int32, device=q.device)
    _dev(out, "qweight", torch.int32, layout.qweight_shape)
    _check(lib().qlinear_pack_weights(layout.ref, _ptr(q), _ptr(out), _stream(q.device)), "qlinear_pack_weights")
    return out


def unpack(layout: Layout, qweight: torch.Tensor) -> torch.Tensor:
    _dev(qweight, "qweight", torch.int32, layout.qweight_shape)
    q = torch.empty((layout.K, layout.N), dtype=torch.uint8, device=qweight.device)
    _check(lib().qlinear_unpack(layout.ref, _ptr(qweight), _ptr(q), _stream(q.device)), "qlinear_unpack")
    return q


def dequant(layout: Layout, qweight: torch.Tensor, scales: torch.Tensor,
            zeros: torch.Tensor | None) -> torch.Tensor:
    _dev(qweight, "qweight", torch.int32, layout.qweight_shape)
    _dev(scales, "scales", torch.float16, (layout.groups, layout.N))
    if zeros is not None:
        _dev(zeros, "zeros", torch.uint8, (layout.groups, layout.N))
    w = torch.empty((layout.K, layout.N), dtype=torch.float16, device=qweight.device)
    _check(lib().qlinear_dequant(layout.ref, _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(w),
                                 _stream(w.device)), "qlinear_dequant")
    return w


def qgemv_workspace_bytes(layout: Layout) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().qlinear_qgemv_workspace_bytes(layout.ref, ctypes.byref(n)), "qlinear_qgemv_workspace_bytes")
    return int(n.value)


def qgemv_workspace(layout: Layout, device) -> torch.Tensor:
    """A qgemv workspace (scratch: needs no initialization)."""
    return torch.empty(qgemv_workspace_bytes(layout), dtype=torch.uint8, device=device)


def qgemm_workspace_bytes(layout: Layout, M: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().qlinear_qgemm_workspace_bytes(layout.ref, int(M), ctypes.byref(n)), "qlinear_qgemm_workspace_bytes")
    return int(n.value)


def _gemm_operands(layout, x, qweight, scales, zeros, perm, y):
    if x.dim() != 2 or x.shape[1] != layout.K:
        raise ValueError(f"x must be [M][{layout.K}]")
    M = int(x.shape[0])
    _dev(x, "x", torch.float16)
    _dev(qweight, "qweight", torch.int32, layout.qweight_shape)
    _dev(scales, "scales", torch.float16, (layout.groups, layout.N))
    if zeros is not None:
        _dev(zeros, "zeros", torch.uint8, (layout.groups, layout.N))
    if perm is not None:
        _dev(perm, "perm", torch.int32, (layout.K,))
    if y is None:
        y = torch.empty((M, layout.N), dtype=torch.float16, device=x.device)
    _dev(y, "y", torch.float16, (M, layout.N))
    return M, y


def _epilogue(layout, M, y, bias, residual, activation, addend=None):
    """The qlinear_epilogue of a fused call, or None for the plain call."""
    if bias is None and residual is None and activation == ACT_NONE and addend is None:
        return None
    if bias is not None:
        _dev(bias, "bias", torch.float16, (layout.N,))
    if residual is not None:
        _dev(residual, "residual", torch.float16, (M, layout.N))
    if addend is not None:
        _dev(addend, "addend", torch.float32, (M, layout.N))
    return qlinear_epilogue(_ptr(bias), _ptr(residual), int(activation), _ptr(addend))


def qgemv(layout: Layout, x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
          zeros: torch.Tensor | None, perm: torch.Tensor | None, workspace: torch.Tensor,
          y: torch.Tensor | None = None, bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
          activation: int = ACT_NONE, addend: torch.Tensor | None = None) -> torch.Tensor:
    """Decode layer, M = x.shape[0] <= 16. Returns y float16 [M][N]. With bias
    [N], residual [M][N] (may be y), activation ACT_SILU or addend float32
    [M][N] (e.g. from lora_delta) the fused call runs:
    y = RNE(act(x W + addend + bias) + residual)."""
    M, y = _gemm_operands(layout, x, qweight, scales, zeros, perm, y)
    _dev(workspace, "workspace", torch.uint8)
    epi = _epilogue(layout, M, y, bias, residual, activation, addend)
    if epi is None:
        _check(lib().qlinear_qgemv(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(perm),
                                   _ptr(y), _ptr(workspace), workspace.numel(), _stream(x.device)), "qlinear_qgemv")
    else:
        _check(lib().qlinear_qgemv_fused(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                         _ptr(perm), ctypes.byref(epi), _ptr(y), _ptr(workspace), workspace.numel(),
                                         _stream(x.device)), "qlinear_qgemv_fused")
    return y


NOALLOC_MAX_K = 65536


def qgemv_noalloc(layout: Layout, x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
                  zeros: torch.Tensor | None, perm: torch.Tensor | None,
                  y: torch.Tensor | None = None) -> torch.Tensor:
    """qgemv with the library's static device scratch as its workspace (no
    allocation by the library; y is allocated here unless given). Calls that
    overlap in time on one GPU race."""
    M, y = _gemm_operands(layout, x, qweight, scales, zeros, perm, y)
    _check(lib().qlinear_qgemv_noalloc(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                       _ptr(perm), _ptr(y), _stream(x.device)), "qlinear_qgemv_noalloc")
    return y


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def qgemv_grouped(layout: Layout, x: torch.Tensor, qweights, scales, zeros, perm: torch.Tensor | None,
                  workspace: torch.Tensor, ys=None) -> list:
    """Decode layer for several matrices that share the layout, x and perm
    (e.g. q, k, v). zeros: None or a list (one per matrix). Returns the list
    of outputs y_i float16 [M][N]."""
    count = len(qweights)
    if len(scales) != count or (zeros is not None and len(zeros) != count):
        raise ValueError("one scales (and zeros) tensor per matrix")
    outs = []
    for i in range(count):
        M, y = _gemm_operands(layout, x, qweights[i], scales[i], None if zeros is None else zeros[i], perm,
                              None if ys is None else ys[i])
        outs.append(y)
    _dev(workspace, "workspace", torch.uint8)
    qa, sa, ya = _ptr_array(qweights), _ptr_array(scales), _ptr_array(outs)
    za = None if zeros is None else _ptr_array(zeros)
    _check(lib().qlinear_qgemv_grouped(layout.ref, _ptr(x), int(x.shape[0]), count, qa, sa, za, _ptr(perm), ya,
                                       _ptr(workspace), workspace.numel(), _stream(x.device)),
           "qlinear_qgemv_grouped")
    return outs


def qgemm(layout: Layout, x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
          zeros: torch.Tensor | None, perm: torch.Tensor | None, workspace: torch.Tensor | None = None,
          y: torch.Tensor | None = None, bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
          activation: int = ACT_NONE, addend: torch.Tensor | None = None) -> torch.Tensor:
    """Prefill layer, any M. Returns y float16 [M][N]; epilogue as for qgemv."""
    M, y = _gemm_operands(layout, x, qweight, scales, zeros, perm, y)
    need = qgemm_workspace_bytes(layout, M)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    epi = _epilogue(layout, M, y, bias, residual, activation, addend)
    if epi is None:
        _check(lib().qlinear_qgemm(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(perm),
                                   _ptr(y), _ptr(workspace), workspace.numel(), _stream(x.device)), "qlinear_qgemm")
    else:
        _check(lib().qlinear_qgemm_fused(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(scales), _ptr(zeros),
                                         _ptr(perm), ctypes.byref(epi), _ptr(y), _ptr(workspace), workspace.numel(),
                                         _stream(x.device)), "qlinear_qgemm_fused")
    return y


def lora_workspace_bytes(M: int, K: int, rank: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().qlinear_lora_workspace_bytes(int(M), int(K), int(rank), ctypes.byref(n)),
           "qlinear_lora_workspace_bytes")
    return n.value


def lora_delta(x: torch.Tensor, lora_a: torch.Tensor, lora_b: torch.Tensor, scale: float = 1.0,
               delta: torch.Tensor | None = None, accumulate: bool = False,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """On-the-fly LoRA update delta (+)= scale (x A) B, float32 [M][N], from x
    float16 [M][K] (original feature order), A float16 [K][r], B float16
    [r][N]. Pass the result as `addend` of qgemv/qgemm; accumulate=True adds
    a further adapter into delta."""
    if x.dim() != 2 or lora_a.dim() != 2 or lora_b.dim() != 2:
        raise ValueError("x, lora_a and lora_b must be 2-D")
    M, K = (int(v) for v in x.shape)
    rank = int(lora_a.shape[1])
    N = int(lora_b.shape[1])
    _dev(x, "x", torch.float16)
    _dev(lora_a, "lora_a", torch.float16, (K, rank))
    _dev(lora_b, "lora_b", torch.float16, (rank, N))
    if delta is None:
        if accumulate:
            raise ValueError("accumulate=True needs the delta to add to")
        delta = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev(delta, "delta", torch.float32, (M, N))
    if workspace is None:
        workspace = torch.empty(max(lora_workspace_bytes(M, K, rank), 256), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    _check(lib().qlinear_lora_delta(_ptr(x), M, K, _ptr(lora_a), rank, _ptr(lora_b), N, float(scale),
                                    1 if accumulate else 0, _ptr(delta), _ptr(workspace), workspace.numel(),
                                    _stream(x.device)), "qlinear_lora_delta")
    return delta


# ---------------------------------------------------------------- two-level scales

def pack_qscale(codes: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """4-bit scale codes uint8 [G][N] -> q_scale int32 [G][N/8] (uint32 bit
    patterns, 8 codes per word, column n at bits 4 (n % 8))."""
    if codes.dim() != 2:
        raise ValueError("codes must be [G][N]")
    G, N = int(codes.shape[0]), int(codes.shape[1])
    _dev(codes, "codes", torch.uint8)
    if out is None:
        out = torch.empty((G, N // 8), dtype=torch.int32, device=codes.device)
    _dev(out, "q_scale", torch.int32, (G, N // 8))
    _check(lib().qlinear_pack_qscale(_ptr(codes), G, N, _ptr(out), _stream(codes.device)), "qlinear_pack_qscale")
    return out


def _qscale_operands(layout, q_scale, q_scale_max):
    _dev(q_scale, "q_scale", torch.int32, (layout.groups, layout.N // 8))
    _dev(q_scale_max, "q_scale_max", torch.float16, (layout.N,))


def dequant_qscale(layout: Layout, qweight: torch.Tensor, q_scale: torch.Tensor,
                   q_scale_max: torch.Tensor) -> torch.Tensor:
    """Two-level dequantized weights float16 [K][N] (stored row order)."""
    _dev(qweight, "qweight", torch.int32, layout.qweight_shape)
    _qscale_operands(layout, q_scale, q_scale_max)
    w = torch.empty((layout.K, layout.N), dtype=torch.float16, device=qweight.device)
    _check(lib().qlinear_dequant_qscale(layout.ref, _ptr(qweight), _ptr(q_scale), _ptr(q_scale_max), _ptr(w),
                                        _stream(w.device)), "qlinear_dequant_qscale")
    return w


def _qscale_gemm_operands(layout, x, qweight, q_scale, q_scale_max, perm, y):
    if x.dim() != 2 or x.shape[1] != layout.K:
        raise ValueError(f"x must be [M][{layout.K}]")
    M = int(x.shape[0])
    _dev(x, "x", torch.float16)
    _dev(qweight, "qweight", torch.int32, layout.qweight_shape)
    _qscale_operands(layout, q_scale, q_scale_max)
    if perm is not None:
        _dev(perm, "perm", torch.int32, (layout.K,))
    if y is None:
        y = torch.empty((M, layout.N), dtype=torch.float16, device=x.device)
    _dev(y, "y", torch.float16, (M, layout.N))
    return M, y


def qgemv_qscale(layout: Layout, x: torch.Tensor, qweight: torch.Tensor, q_scale: torch.Tensor,
                 q_scale_max: torch.Tensor, perm: torch.Tensor | None, workspace: torch.Tensor,
                 y: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                 residual: torch.Tensor | None = None, activation: int = ACT_NONE,
                 addend: torch.Tensor | None = None) -> torch.Tensor:
    """Decode layer with two-level scales (M <= 16); epilogue as for qgemv."""
    M, y = _qscale_gemm_operands(layout, x, qweight, q_scale, q_scale_max, perm, y)
    _dev(workspace, "workspace", torch.uint8)
    epi = _epilogue(layout, M, y, bias, residual, activation, addend)
    _check(lib().qlinear_qgemv_qscale(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(q_scale), _ptr(q_scale_max),
                                      _ptr(perm), None if epi is None else ctypes.byref(epi), _ptr(y),
                                      _ptr(workspace), workspace.numel(), _stream(x.device)), "qlinear_qgemv_qscale")
    return y


def qgemm_qscale(layout: Layout, x: torch.Tensor, qweight: torch.Tensor, q_scale: torch.Tensor,
                 q_scale_max: torch.Tensor, perm: torch.Tensor | None, workspace: torch.Tensor | None = None,
                 y: torch.Tensor | None = None, bias: torch.Tensor | None = None,
                 residual: torch.Tensor | None = None, activation: int = ACT_NONE,
                 addend: torch.Tensor | None = None) -> torch.Tensor:
    """Prefill layer with two-level scales, any M; epilogue as for qgemv."""
    M, y = _qscale_gemm_operands(layout, x, qweight, q_scale, q_scale_max, perm, y)
    need = qgemm_workspace_bytes(layout, M)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    epi = _epilogue(layout, M, y, bias, residual, activation, addend)
    _check(lib().qlinear_qgemm_qscale(layout.ref, _ptr(x), M, _ptr(qweight), _ptr(q_scale), _ptr(q_scale_max),
                                      _ptr(perm), None if epi is None else ctypes.byref(epi), _ptr(y),
                                      _ptr(workspace), workspace.numel(), _stream(x.device)), "qlinear_qgemm_qscale")
    return y


# ---------------------------------------------------------------- KV-cache codec

def kv_quant(x: torch.Tensor, bits: int, group: int, codes: torch.Tensor | None = None,
             scales: torch.Tensor | None = None):
    """x float16 [..., D] -> (codes int32 [..., D * bits / 32] (uint32 bit
    patterns), scales float16 [..., D / group]); leading dimensions are rows."""
    _dev(x, "x", torch.float16)
    D = int(x.shape[-1])
    rows = x.numel() // D if D else 0
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (D * bits // 32,), dtype=torch.int32, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (D // group if group else 0,), dtype=torch.float16, device=x.device)
    _dev(codes, "codes", torch.int32, lead + (D * bits // 32,))
    _dev(scales, "scales", torch.float16, lead + (D // group,))
    _check(lib().qlinear_kv_quant(_ptr(x), rows, D, int(bits), int(group), _ptr(codes), _ptr(scales),
                                  _stream(x.device)), "qlinear_kv_quant")
    return codes, scales


def kv_dequant(codes: torch.Tensor, scales: torch.Tensor, D: int, bits: int, group: int,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """(codes, scales) of kv_quant -> float16 [..., D]."""
    _dev(codes, "codes", torch.int32)
    _dev(scales, "scales", torch.float16)
    lead = tuple(codes.shape[:-1])
    if tuple(codes.shape) != lead + (D * bits // 32,):
        raise ValueError("codes must be [..., D * bits / 32]")
    _dev(scales, "scales", torch.float16, lead + (D // group,))
    rows = int(np.prod(lead)) if lead else 1
    if out is None:
        out = torch.empty(lead + (D,), dtype=torch.float16, device=codes.device)
    _dev(out, "out", torch.float16, lead + (D,))
    _check(lib().qlinear_kv_dequant(_ptr(codes), _ptr(scales), rows, int(D), int(bits), int(group), _ptr(out),
                                    _stream(codes.device)), "qlinear_kv_dequant")
    return out
