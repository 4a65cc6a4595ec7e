"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before launching anything (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import dequant_matmul_gptq_amd as dq
from dequant_matmul_gptq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlinear.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlinear_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dq.lib()
    names = declared_functions()
    assert sorted(names) == sorted(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_struct_size_matches_header():
    # 6 scalars + 2 * (MAX_RUNS + 1) + MAX_RUNS int32, then the int64 word count
    assert ctypes.sizeof(_lib.qlinear_layout) == 4 * (6 + 2 * 65 + 64) + 8


def test_status_strings():
    for s in range(6):
        assert dq.status_string(s)
    assert dq.status_string(99) == "unknown status"


def _layout(K=256, N=512, gs=32, bits=None):
    bits = np.full(K // gs, 4, np.uint8) if bits is None else bits
    return dq.Layout(K, N, gs, bits)


def test_layout_runs_and_rows():
    bits = np.array([6] * 3 + [5] * 2 + [4] * 5 + [3] * 4, np.uint8)
    L = _layout(K=14 * 64, N=64, gs=64, bits=bits)
    assert L.nruns == 4
    c = L.c
    assert list(c.run_group)[:5] == [0, 3, 5, 10, 14]
    assert list(c.run_bits)[:4] == [6, 5, 4, 3]
    # 2 blocks per group, b words per block
    assert list(c.run_row)[:5] == [0, 36, 56, 96, 120]
    assert L.packed_rows == 120
    assert c.packed_words == 4 * 120 * 16       # N = 64: four 16-column panels
    L2 = _layout(K=64, N=24, gs=32, bits=np.array([3, 3], np.uint8))
    assert L2.c.packed_words == 2 * 6 * 16       # N = 24: last panel half padding


@pytest.mark.parametrize("args,status", [
    ((256, 512, 48), _lib.ERR_UNSUPPORTED),      # group size
    ((250, 512, 32), _lib.ERR_UNSUPPORTED),      # K % gs
    ((256, 500, 32), _lib.ERR_UNSUPPORTED),      # N % 8
    ((0, 512, 32), _lib.ERR_INVALID_ARGUMENT),
    ((256, -8, 32), _lib.ERR_INVALID_ARGUMENT),
])
def test_layout_init_rejects_shapes(args, status):
    bits = np.full(64, 4, np.uint8)
    with pytest.raises(dq.QlinearError) as e:
        dq.Layout(*args, bits[: max(1, args[0] // args[2]) if args[2] else 1])
    assert e.value.status == status


def test_layout_init_rejects_bits_and_runs():
    with pytest.raises(dq.QlinearError) as e:
        _layout(bits=np.array([4, 4, 7, 4, 4, 4, 4, 4], np.uint8))
    assert e.value.status == _lib.ERR_UNSUPPORTED
    alt = np.array([4, 3] * 40, np.uint8)   # 80 runs > 64
    with pytest.raises(dq.QlinearError) as e:
        _layout(K=80 * 32, N=64, gs=32, bits=alt)
    assert e.value.status == _lib.ERR_UNSUPPORTED
    ok = np.array([4, 3] * 32, np.uint8)    # exactly 64 runs
    assert _layout(K=64 * 32, N=64, gs=32, bits=ok).nruns == 64


@pytest.mark.parametrize("groups,seed", [(1, 0), (7, 1), (128, 2), (896, 3)])
def test_group_order_leaves_at_most_six_runs(groups, seed):
    """Any per-group width map (here shuffled over all six widths) in the
    returned order: a permutation, widest widths first, original order kept
    within a width, at most 6 runs, so qlinear_layout_init accepts it."""
    rng = np.random.default_rng(seed)
    bits = rng.choice(np.array([2, 3, 4, 5, 6, 8], np.uint8), size=groups)
    order = dq.group_order(bits)
    assert sorted(order.tolist()) == list(range(groups))
    b = bits[order]
    assert np.all(np.diff(b.astype(int)) <= 0)
    for w in np.unique(bits):
        idx = order[b == w]
        assert np.all(np.diff(idx) > 0)
    L = dq.Layout(groups * 32, 64, 32, b)
    assert L.nruns == len(np.unique(bits)) <= 6


def test_group_order_errors():
    L = dq.lib()
    with pytest.raises(dq.QlinearError) as e:
        dq.group_order(np.array([4, 7, 4], np.uint8))
    assert e.value.status == _lib.ERR_UNSUPPORTED
    out = np.full(3, -5, np.int32)
    bits = np.array([4, 3, 4], np.uint8)
    assert L.qlinear_group_order(bits.ctypes.data_as(ctypes.c_void_p), 0,
                                 out.ctypes.data_as(ctypes.c_void_p)) == _lib.ERR_INVALID_ARGUMENT
    assert L.qlinear_group_order(None, 3, out.ctypes.data_as(ctypes.c_void_p)) == _lib.ERR_INVALID_ARGUMENT
    assert L.qlinear_group_order(bits.ctypes.data_as(ctypes.c_void_p), 3, None) == _lib.ERR_INVALID_ARGUMENT
    assert np.all(out == -5)


@pytest.mark.parametrize("act_order", (True, False))
def test_reorder_groups_keeps_the_product(act_order):
    """The oracle's product on a shuffled 80-run map equals its product on the
    groups moved into group_order's order with the composed permutation."""
    import torch
    from oracle import qlinear_oracle as oracle
    rng = np.random.default_rng(11)
    gs, G, N, M = 32, 80, 24, 3
    bits = np.array([4, 3] * 40, np.uint8)
    rng.shuffle(bits)
    K = G * gs
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    s = rng.uniform(0.005, 0.02, size=(G, N)).astype(np.float16)
    z = rng.integers(0, 8, size=(G, N), dtype=np.uint8)
    perm = rng.permutation(K).astype(np.int32) if act_order else None
    x = rng.standard_normal((M, K)).astype(np.float16)
    b2, q2, (s2, z2), p2 = dq.reorder_groups(dq.group_order(bits), gs, bits, torch.from_numpy(q),
                                             (torch.from_numpy(s), torch.from_numpy(z)),
                                             None if perm is None else torch.from_numpy(perm))
    assert dq.Layout(K, N, gs, b2).nruns == 2
    ref = oracle.qlinear(x, q, s, z, bits, gs, perm)
    got = oracle.qlinear(x, q2.numpy(), s2.numpy(), z2.numpy(), b2, gs, p2.numpy())
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layout_init_null():
    L = dq.lib()
    assert L.qlinear_layout_init(None, 256, 512, 32, None) == _lib.ERR_INVALID_ARGUMENT


FAKE = 0x10000  # aligned fake device address: never dereferenced on these paths


def _gemv(L, **kw):
    a = dict(x=FAKE, M=1, qw=FAKE, s=FAKE, z=None, perm=None, y=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return dq.lib().qlinear_qgemv(L.ref, a["x"], a["M"], a["qw"], a["s"], a["z"], a["perm"], a["y"],
                                  a["ws"], a["wsb"], None)


def _gemm(L, **kw):
    a = dict(x=FAKE, M=1, qw=FAKE, s=FAKE, z=None, perm=None, y=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return dq.lib().qlinear_qgemm(L.ref, a["x"], a["M"], a["qw"], a["s"], a["z"], a["perm"], a["y"],
                                  a["ws"], a["wsb"], None)


def test_qgemv_validation_before_launch():
    L = _layout()
    assert _gemv(L, x=None) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L, qw=None) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L, s=None) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L, y=None) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L, ws=None) == _lib.ERR_WORKSPACE
    assert _gemv(L, M=-1) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L, M=17) == _lib.ERR_UNSUPPORTED
    assert _gemv(L, x=FAKE + 2) == _lib.ERR_MISALIGNED
    assert _gemv(L, z=FAKE + 8) == _lib.ERR_MISALIGNED
    assert _gemv(L, perm=FAKE + 4) == _lib.ERR_MISALIGNED
    assert _gemv(L, wsb=dq.qgemv_workspace_bytes(L) - 1) == _lib.ERR_WORKSPACE
    assert _gemv(L, M=0) == _lib.OK   # quick return, nothing launched
    assert _gemv(L, M=0, x=None, y=None, ws=None, wsb=0) == _lib.OK  # empty tensors may be NULL


def test_qgemv_grouped_validation_before_launch():
    L = _layout()
    lib = dq.lib()
    big = 1 << 30
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    ok = dict(q=arr(FAKE, FAKE), s=arr(FAKE, FAKE), z=None, y=arr(FAKE, FAKE))

    def call(count=2, M=1, **kw):
        a = dict(ok)
        a.update(kw)
        return lib.qlinear_qgemv_grouped(L.ref, FAKE, M, count, a["q"], a["s"], a["z"], None, a["y"], FAKE, big,
                                         None)

    assert call(count=0) == _lib.ERR_INVALID_ARGUMENT
    assert call(count=9) == _lib.ERR_UNSUPPORTED
    assert call(q=None) == _lib.ERR_INVALID_ARGUMENT
    assert call(q=arr(FAKE, None)) == _lib.ERR_INVALID_ARGUMENT
    assert call(y=arr(FAKE, FAKE + 2)) == _lib.ERR_MISALIGNED
    assert call(z=arr(FAKE, None)) == _lib.ERR_INVALID_ARGUMENT      # mixed NULL / non-NULL zero points
    assert call(M=17) == _lib.ERR_UNSUPPORTED
    assert call(M=0) == _lib.OK


def test_qgemm_validation_before_launch():
    L = _layout()
    assert _gemm(L, qw=None) == _lib.ERR_INVALID_ARGUMENT
    assert _gemm(L, ws=None) == _lib.ERR_WORKSPACE
    assert _gemm(L, M=64, wsb=dq.qgemm_workspace_bytes(L, 64) - 1) == _lib.ERR_WORKSPACE
    assert _gemm(L, y=FAKE + 1) == _lib.ERR_MISALIGNED
    assert _gemm(L, M=0) == _lib.OK
    assert _gemm(L, M=0, x=None, y=None, ws=None, wsb=0) == _lib.OK


def test_fused_epilogue_validation_before_launch():
    """The fused calls check the epilogue (activation, alignment) before
    launching; M = 0 returns OK only once the epilogue is valid."""
    L = _layout()
    lib = dq.lib()
    for fn in (lib.qlinear_qgemv_fused, lib.qlinear_qgemm_fused):
        def call(epi, M=0, y=FAKE):
            e = None if epi is None else ctypes.byref(epi)
            return fn(L.ref, FAKE, M, FAKE, FAKE, None, None, e, y, FAKE, 1 << 30, None)

        E = _lib.qlinear_epilogue
        assert call(None) == _lib.OK                                     # no epilogue: the plain call
        assert call(E(FAKE, FAKE, _lib.ACT_SILU)) == _lib.OK
        assert call(E(None, None, 7)) == _lib.ERR_UNSUPPORTED               # unknown activation
        assert call(E(FAKE + 2, None, 0)) == _lib.ERR_MISALIGNED             # bias
        assert call(E(None, FAKE + 8, 0)) == _lib.ERR_MISALIGNED             # residual
        assert call(E(None, None, 0, FAKE + 4)) == _lib.ERR_MISALIGNED       # addend
        assert call(E(None, None, 0, FAKE)) == _lib.OK
        assert call(E(None, None, 0), M=1, y=None) == _lib.ERR_INVALID_ARGUMENT   # operands still checked
        assert call(E(None, None, 0), M=17 if fn is lib.qlinear_qgemv_fused else -1) != _lib.OK


def test_epilogue_struct_layout():
    # bias, residual, activation (padded to 8), addend
    assert ctypes.sizeof(_lib.qlinear_epilogue) == 32
    assert _lib.qlinear_epilogue.addend.offset == 24


def test_lora_validation_before_launch():
    lib = dq.lib()
    K, N, r = 4096, 11008, 16
    need = dq.lora_workspace_bytes(5, K, r)
    assert need == 16 * 5 * r * 4                       # float32 partial sums [K / 256][M][rank]
    assert dq.lora_workspace_bytes(0, K, r) == 0

    def call(x=FAKE, M=5, K=K, a=FAKE, rank=r, b=FAKE, N=N, d=FAKE, ws=FAKE, wsb=need):
        return lib.qlinear_lora_delta(x, M, K, a, rank, b, N, 0.5, 0, d, ws, wsb, None)

    # every call below is rejected before any launch (the pointers are fake)
    assert call(M=-1) == _lib.ERR_INVALID_ARGUMENT
    assert call(K=0) == _lib.ERR_INVALID_ARGUMENT
    assert call(N=0) == _lib.ERR_INVALID_ARGUMENT
    assert call(rank=0) == _lib.ERR_INVALID_ARGUMENT
    assert call(rank=65) == _lib.ERR_UNSUPPORTED
    assert call(K=65535 * 256 + 1) == _lib.ERR_UNSUPPORTED
    assert call(N=65535 * 256 + 1) == _lib.ERR_UNSUPPORTED
    assert call(M=0, x=None, a=None, b=None, d=None, ws=None, wsb=0) == _lib.OK
    assert call(a=None) == _lib.ERR_INVALID_ARGUMENT
    assert call(d=None) == _lib.ERR_INVALID_ARGUMENT
    assert call(ws=None) == _lib.ERR_WORKSPACE
    assert call(wsb=need - 1) == _lib.ERR_WORKSPACE
    assert call(b=FAKE + 2) == _lib.ERR_MISALIGNED
    assert call(d=FAKE + 4) == _lib.ERR_MISALIGNED
    n = ctypes.c_size_t()
    assert lib.qlinear_lora_workspace_bytes(1, K, 65, ctypes.byref(n)) == _lib.ERR_UNSUPPORTED
    assert lib.qlinear_lora_workspace_bytes(1, 0, 8, ctypes.byref(n)) == _lib.ERR_INVALID_ARGUMENT


def test_tampered_layout_is_rejected():
    L = _layout()
    L.c.packed_rows += 1
    assert _gemv(L) == _lib.ERR_INVALID_ARGUMENT
    L = _layout()
    L.c.run_bits[0] = 7
    assert _gemv(L) == _lib.ERR_UNSUPPORTED
    L = _layout()
    L.c.packed_words -= 16
    assert _gemv(L) == _lib.ERR_INVALID_ARGUMENT
    L = _layout()
    L.c.nruns = 0
    assert _gemm(L) == _lib.ERR_UNSUPPORTED
    # Two adjacent runs of one width (a split run that qlinear_layout_init
    # never produces): the launchers size workspaces from the run count, so
    # such a layout is refused before any launch.
    L = _layout(K=8192, N=64, gs=32, bits=np.array([4] * 256, np.uint8))
    assert L.nruns == 1
    c = L.c
    c.nruns = 2
    c.run_group[1], c.run_group[2] = 128, 256
    c.run_row[1], c.run_row[2] = 128 * 4, 256 * 4
    c.run_bits[1] = 4
    assert _gemm(L) == _lib.ERR_INVALID_ARGUMENT
    assert _gemv(L) == _lib.ERR_INVALID_ARGUMENT


def test_pack_unpack_dequant_validation():
    L = _layout()
    lib = dq.lib()
    assert lib.qlinear_pack_weights(L.ref, None, FAKE, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.qlinear_pack_weights(L.ref, FAKE + 1, FAKE, None) == _lib.ERR_MISALIGNED
    assert lib.qlinear_unpack(L.ref, FAKE, None, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.qlinear_dequant(L.ref, FAKE, None, None, FAKE, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.qlinear_dequant(L.ref, FAKE, FAKE, FAKE + 3, FAKE, None) == _lib.ERR_MISALIGNED


def test_workspace_sizes():
    L = _layout(N=4096, K=4096, gs=128)
    # gathered activations float16 [16][K] + block sums float2 [16][K/32], 256-byte rounded
    assert dq.qgemv_workspace_bytes(L) == 16 * 4096 * 2 + 16 * 128 * 8
    # One width on a grid of more than 128 tiles of 256 x 256: the gathered
    # activations only.
    assert dq.qgemm_workspace_bytes(L, 4096) == 4096 * 4096 * 2
    # A smaller grid: the LDS-dequant kernel with K in slices, whose float32
    # partial sums [slices][M][N] follow the 256-byte rounded activations:
    # slices = min(16, 1024 // (128 x 128 tiles), K / 32 / 16).
    assert dq.qgemm_workspace_bytes(L, 2048) == 2048 * 4096 * 2 + 2 * 2048 * 4096 * 4   # 512 tiles: 2 slices
    small = _layout(N=512, K=4096, gs=128)
    assert dq.qgemm_workspace_bytes(small, 100) == (100 * 4096 * 2 + 255) // 256 * 256 + 8 * 100 * 512 * 4
    # Several code widths with >= 16384 rows of K per run boundary and at
    # least 256 tiles of 256 x 256: one launch per run, float32 partial sums
    # [M][N].
    few = _layout(K=32768, N=4096, gs=32, bits=np.array([6] * 64 + [4] * 448 + [3] * 512, np.uint8))
    assert few.nruns == 3
    assert dq.qgemm_workspace_bytes(few, 4096) == (4096 * 32768 * 2 + 255) // 256 * 256 + 4096 * 4096 * 4
    # Fewer tiles: the LDS kernel, here in 2 slices.
    assert dq.qgemm_workspace_bytes(few, 2048) == 2048 * 32768 * 2 + 2 * 2048 * 4096 * 4
    # Fewer rows per boundary on a full grid (1024 tiles of 128 x 128): the LDS kernel in one slice.
    short = _layout(K=8192, N=4096, gs=32, bits=np.array([6] * 16 + [4] * 176 + [3] * 64, np.uint8))
    assert dq.qgemm_workspace_bytes(short, 4096) == 4096 * 8192 * 2
    # A small grid of several widths: 8 slices (K / 32 / 16).
    many = _layout(K=4096, N=512, gs=32, bits=np.array([4, 3] * 10 + [4] * 108, np.uint8))
    assert many.nruns == 21
    assert dq.qgemm_workspace_bytes(many, 100) == (100 * 4096 * 2 + 255) // 256 * 256 + 8 * 100 * 512 * 4
    # 17..32 rows run as decode launches: at least the decode workspace.
    for M in (17, 24, 32):
        assert dq.qgemm_workspace_bytes(small, M) >= dq.qgemv_workspace_bytes(small)


def test_two_level_scale_validation_before_launch():
    L = _layout()
    lib = dq.lib()
    E = _lib

    def gemv(qs=FAKE, qsm=FAKE, M=1, wsb=1 << 30, **kw):
        return lib.qlinear_qgemv_qscale(L.ref, FAKE, M, FAKE, qs, qsm, None, None, FAKE, FAKE, wsb, None)

    def gemm(qs=FAKE, qsm=FAKE, M=1, wsb=1 << 30):
        return lib.qlinear_qgemm_qscale(L.ref, FAKE, M, FAKE, qs, qsm, None, None, FAKE, FAKE, wsb, None)

    for f in (gemv, gemm):
        assert f(qsm=None) == E.ERR_INVALID_ARGUMENT
        assert f(qs=None) == E.ERR_INVALID_ARGUMENT
        assert f(qsm=FAKE + 2) == E.ERR_MISALIGNED
        assert f(qs=FAKE + 4) == E.ERR_MISALIGNED
        assert f(M=-1) == E.ERR_INVALID_ARGUMENT
        assert f(M=0, qsm=None) == E.OK          # quick return before the operands are checked
        assert f(wsb=0) == E.ERR_WORKSPACE
    assert gemv(M=17) == E.ERR_UNSUPPORTED
    assert lib.qlinear_dequant_qscale(L.ref, FAKE, FAKE, None, FAKE, None) == E.ERR_INVALID_ARGUMENT
    assert lib.qlinear_dequant_qscale(L.ref, FAKE, FAKE + 4, FAKE, FAKE, None) == E.ERR_MISALIGNED
    assert lib.qlinear_pack_qscale(FAKE, 4, 12, FAKE, None) == E.ERR_UNSUPPORTED
    assert lib.qlinear_pack_qscale(FAKE, -1, 8, FAKE, None) == E.ERR_INVALID_ARGUMENT
    assert lib.qlinear_pack_qscale(None, 4, 8, FAKE, None) == E.ERR_INVALID_ARGUMENT
    assert lib.qlinear_pack_qscale(FAKE + 1, 4, 8, FAKE, None) == E.ERR_MISALIGNED
    assert lib.qlinear_pack_qscale(None, 0, 8, None, None) == E.OK
