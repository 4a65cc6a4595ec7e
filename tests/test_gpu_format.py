"""GPU packing, unpacking and dequantization against the oracle: bit-exact."""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
import workloads as wl
from gpu_util import GpuLayer, device, fp16_bits, say

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)


def _small(bits, gs, N, seed, zeros=True):
    rng = np.random.default_rng(seed)
    bits = np.asarray(bits, np.uint8)
    K = gs * len(bits)
    q = np.concatenate([rng.integers(0, 1 << int(b), size=(gs, N), dtype=np.uint8) for b in bits])
    s = rng.uniform(0.005, 0.02, size=(len(bits), N)).astype(np.float16)
    z = rng.integers(0, 16, size=(len(bits), N), dtype=np.uint8) if zeros else None
    return K, bits, q, s, z


def _run(K, N, gs, bits, q, s, z):
    dev = device()
    L = dq.Layout(K, N, gs, bits)
    qd = torch.from_numpy(q).to(dev)
    packed = dq.pack_weights(L, qd)
    sd = torch.from_numpy(s).to(dev)
    zd = None if z is None else torch.from_numpy(z).to(dev)
    w = dq.dequant(L, packed, sd, zd)
    un = dq.unpack(L, packed)
    torch.cuda.synchronize()
    return packed.cpu().numpy().view(np.uint32), un.cpu().numpy(), fp16_bits(w)


def _oracle_storage(q, bits, gs):
    return oracle.panel_layout(oracle.pack(q, bits, gs))


@pytest.mark.parametrize("b", BITS)
@pytest.mark.parametrize("gs", (32, 64, 128))
def test_small_uniform(b, gs):
    say(f"format uniform b={b} gs={gs}")
    N = 264  # one full 256-column strip plus a ragged one
    K, bits, q, s, z = _small([b] * 3, gs, N, seed=b * 7 + gs)
    packed, un, w = _run(K, N, gs, bits, q, s, z)
    assert np.array_equal(packed, _oracle_storage(q, bits, gs))
    assert np.array_equal(un, q)
    assert np.array_equal(w, oracle.dequant_fp16(q, s, z, bits, gs).view(np.uint16))


@pytest.mark.parametrize("zeros", (True, False))
def test_small_mixed_runs(zeros):
    bits = [6, 6, 5, 4, 4, 3, 2, 8, 8, 3, 5, 2]
    say(f"format mixed zeros={zeros}")
    K, bits, q, s, z = _small(bits, 32, 40, seed=3, zeros=zeros)
    packed, un, w = _run(K, 40, 32, bits, q, s, z)
    assert np.array_equal(packed, _oracle_storage(q, bits, 32))
    assert np.array_equal(un, q)
    assert np.array_equal(w, oracle.dequant_fp16(q, s, z, bits, 32).view(np.uint16))


def test_extreme_codes():
    # all-zero, all-max and alternating codes for every width
    for b in BITS:
        say(f"format extreme b={b}")
        gs, N = 32, 16
        for q1 in (np.zeros((gs, N), np.uint8), np.full((gs, N), (1 << b) - 1, np.uint8),
                   (np.indices((gs, N)).sum(0) % 2 * ((1 << b) - 1)).astype(np.uint8)):
            s = np.full((1, N), 1.0, np.float16)
            packed, un, w = _run(gs, N, gs, np.array([b], np.uint8), q1, s, None)
            assert np.array_equal(packed, _oracle_storage(q1, [b], gs))
            assert np.array_equal(un, q1)
            assert np.array_equal(w, oracle.dequant_fp16(q1, s, None, [b], gs).view(np.uint16))


@pytest.mark.parametrize("spec", wl.ALL_LAYERS, ids=lambda s: s.name)
def test_full_size_layers(spec):
    """Full-size workload matrices: unpack must return every code; packed words
    and float16 weights must match the oracle on sampled columns."""
    say(f"format full {spec.name}")
    inp = wl.generate(spec, draw_x=False)
    lay = GpuLayer(inp)
    un = dq.unpack(lay.layout, lay.qweight)
    assert torch.equal(un, lay.q)
    w = dq.dequant(lay.layout, lay.qweight, lay.scales, lay.zeros)
    rng = np.random.default_rng(1)
    cols = np.unique(np.concatenate([rng.choice(spec.N, 24, replace=False), [0, spec.N - 1]]))
    ci = torch.from_numpy(cols).to(lay.dev)
    panels = lay.qweight.cpu().numpy().view(np.uint32)
    packed = np.stack([panels[n // 16, :, n % 16] for n in cols], axis=1)   # word matrix columns
    assert np.array_equal(packed, oracle.pack(inp.q[:, cols], inp.bits, spec.group_size))
    zc = None if inp.zeros is None else inp.zeros[:, cols]
    want = oracle.dequant_fp16(inp.q[:, cols], inp.scales[:, cols], zc, inp.bits, spec.group_size)
    got = w.index_select(1, ci).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want.view(np.uint16))
