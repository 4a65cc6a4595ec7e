"""The Q4/Q6/Q8 KV-cache codec on the GPU against the CPU oracle: codes and
scales bit for bit (both sides decide the codes in float32), dequantized
values bit for bit (computed from the oracle's own codes)."""

import numpy as np
import pytest
import torch

import dequant_matmul_gptq_amd as dq
import oracle
from gpu_util import Guarded, device, say

pytestmark = pytest.mark.gpu


def _cache_rows(rows, D, seed):
    """Key/value-like rows: N(0, 1) times a per-row magnitude, with a few
    outlier channels ten times larger, and one all-zero row."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, D)) * rng.uniform(0.05, 4.0, size=(rows, 1))
    x[:, rng.choice(D, max(1, D // 32), replace=False)] *= 10.0
    if rows > 2:
        x[2] = 0.0
    return x.astype(np.float16)


def _gpu_quant(x, bits, group):
    codes, scales = dq.kv_quant(torch.from_numpy(x).to(device()), bits, group)
    return codes.cpu().numpy().view(np.uint32), scales.cpu().numpy()


@pytest.mark.parametrize("bits", (4, 6, 8))
@pytest.mark.parametrize("group", (32, 64, 128))
@pytest.mark.parametrize("rows,D", [(1, 128), (3, 256), (1000, 128), (77, 384)])
def test_quant_bit_exact(bits, group, rows, D):
    say(f"kv quant b={bits} G={group} rows={rows} D={D}")
    x = _cache_rows(rows, D, seed=bits * 1000 + group + rows)
    words, scales = _gpu_quant(x, bits, group)
    w_ref, s_ref = oracle.kv_quantize(x, bits, group)
    assert np.array_equal(scales.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(words, w_ref)


@pytest.mark.parametrize("bits", (4, 6, 8))
@pytest.mark.parametrize("group", (32, 128))
def test_dequant_bit_exact(bits, group):
    say(f"kv dequant b={bits} G={group}")
    x = _cache_rows(517, 256, seed=bits + group)
    w_ref, s_ref = oracle.kv_quantize(x, bits, group)
    dev = device()
    out = dq.kv_dequant(torch.from_numpy(w_ref.view(np.int32)).to(dev), torch.from_numpy(s_ref).to(dev), 256, bits,
                        group)
    want = oracle.kv_dequantize(w_ref, s_ref, 256, bits, group)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want.view(np.uint16))


def test_ties_and_exact_values():
    """Blocks whose values are exact multiples of the scale come back exactly;
    half-way values round to the even code."""
    x = np.zeros((2, 32), np.float16)
    x[0, :15] = np.arange(-7, 8) * 0.5
    x[1, :5] = [7.0, 2.5, 3.5, -0.5, -1.5]
    words, scales = _gpu_quant(x, 4, 32)
    assert scales.tolist() == [[0.5], [1.0]]
    out = dq.kv_dequant(torch.from_numpy(words.view(np.int32)).cuda(), torch.from_numpy(scales).cuda(), 32, 4, 32)
    y = out.cpu().numpy()
    assert np.array_equal(y[0], x[0])
    assert y[1, :5].tolist() == [7.0, 2.0, 4.0, 0.0, -2.0]


def test_append_one_token_in_place():
    """Quantizing one token's rows into the middle of a cache touches only
    those rows' codes and scales (guard bands around the whole cache)."""
    say("kv append one token")
    heads, T, D, bits, group = 8, 64, 128, 4, 32
    dev = device()
    x = _cache_rows(heads * T, D, seed=5).reshape(T, heads, D)
    cw = D * bits // 32
    cb = Guarded(T * heads * cw * 4, dev)
    sb = Guarded(T * heads * (D // group) * 2, dev)
    codes = cb.view(torch.int32, (T, heads, cw))
    scales = sb.view(torch.float16, (T, heads, D // group))
    codes.fill_(0x5A5A5A5A)
    scales.fill_(7.0)
    t = 37
    dq.kv_quant(torch.from_numpy(np.ascontiguousarray(x[t])).to(dev), bits, group, codes=codes[t], scales=scales[t])
    torch.cuda.synchronize()
    assert cb.intact() and sb.intact()
    w_ref, s_ref = oracle.kv_quantize(x[t], bits, group)
    c = codes.cpu().numpy().view(np.uint32)
    s = scales.cpu().numpy()
    assert np.array_equal(c[t], w_ref) and np.array_equal(s[t], s_ref)
    others = np.arange(T) != t
    assert (c[others] == 0x5A5A5A5A).all() and (s[others] == 7.0).all()


def test_full_layer_cache():
    """One layer's key cache of a 70B-class model at 32K tokens: 8 key/value
    heads x 32768 tokens x 128 = 33.5 M elements, Q4 with one scale per head
    vector (G = 128), against the oracle on every element."""
    say("kv full layer cache 262144 x 128")
    x = _cache_rows(8 * 32768, 128, seed=11)
    words, scales = _gpu_quant(x, 4, 128)
    w_ref, s_ref = oracle.kv_quantize(x, 4, 128)
    assert np.array_equal(scales.view(np.uint16), s_ref.view(np.uint16))
    assert np.array_equal(words, w_ref)


def test_rejects_before_launch():
    lib = dq.lib()
    E = dq._lib
    FAKE = 0x10000
    assert lib.qlinear_kv_quant(FAKE, 4, 128, 5, 32, FAKE, FAKE, None) == E.ERR_UNSUPPORTED
    assert lib.qlinear_kv_quant(FAKE, 4, 96, 4, 64, FAKE, FAKE, None) == E.ERR_UNSUPPORTED
    assert lib.qlinear_kv_quant(FAKE, -1, 128, 4, 32, FAKE, FAKE, None) == E.ERR_INVALID_ARGUMENT
    assert lib.qlinear_kv_quant(None, 4, 128, 4, 32, FAKE, FAKE, None) == E.ERR_INVALID_ARGUMENT
    assert lib.qlinear_kv_quant(FAKE + 8, 4, 128, 4, 32, FAKE, FAKE, None) == E.ERR_MISALIGNED
    assert lib.qlinear_kv_dequant(FAKE + 2, FAKE, 4, 128, 4, 32, FAKE, None) == E.ERR_MISALIGNED
    assert lib.qlinear_kv_quant(None, 0, 128, 4, 32, None, None, None) == E.OK
