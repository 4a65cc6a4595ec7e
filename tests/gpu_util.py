"""Helpers for the GPU parity tests: move seeded inputs to the device, pack
them with the HIP path, and compare against the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import dequant_matmul_gptq_amd as dq

# Output tolerance of the layer: relative Frobenius error and max error
# relative to the largest reference magnitude.
REL_FRO_TOL = 1e-3
MAX_ABS_TOL = 1e-2


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run them with -m 'not gpu' elsewhere)")
    return torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class GpuLayer:
    """One layer's inputs on the GPU, packed by qlinear_pack_weights."""

    def __init__(self, inp, dev=None):
        dev = dev or device()
        sp = inp.spec
        self.inp = inp
        self.layout = dq.Layout(sp.K, sp.N, sp.group_size, inp.bits)
        self.q = torch.from_numpy(np.ascontiguousarray(inp.q)).to(dev)
        self.qweight = dq.pack_weights(self.layout, self.q)
        self.scales = torch.from_numpy(inp.scales).to(dev)
        self.zeros = None if inp.zeros is None else torch.from_numpy(inp.zeros).to(dev)
        self.perm = None if inp.perm is None else torch.from_numpy(inp.perm.astype(np.int32)).to(dev)
        self.ws = dq.qgemv_workspace(self.layout, dev)
        self.dev = dev

    def x(self, x_np):
        return torch.from_numpy(np.ascontiguousarray(x_np)).to(self.dev)

    def qgemv(self, x_np):
        return dq.qgemv(self.layout, self.x(x_np), self.qweight, self.scales, self.zeros, self.perm, self.ws)

    def qgemm(self, x_np):
        return dq.qgemm(self.layout, self.x(x_np), self.qweight, self.scales, self.zeros, self.perm)


def errors(y_gpu: torch.Tensor, y_ref: np.ndarray):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    d = y - y_ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(y_ref), 1e-300)
    mx = np.abs(d).max() / max(np.abs(y_ref).max(), 1e-300)
    return rel, mx


def assert_close(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str = ""):
    assert tuple(y_gpu.shape) == y_ref.shape, (what, tuple(y_gpu.shape), y_ref.shape)
    y = y_gpu.float().cpu().numpy()
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    rel, mx = errors(y_gpu, y_ref)
    assert rel <= REL_FRO_TOL and mx <= MAX_ABS_TOL, f"{what}: rel_fro={rel:.3e} max_rel={mx:.3e}"
    return rel, mx


def fp16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


GUARD_BYTES = 4096
GUARD_VALUE = 0xA5


class Guarded:
    """A device buffer of `nbytes` between two guard bands of GUARD_BYTES
    filled with GUARD_VALUE; `view(dtype, shape)` is the usable middle (16-byte
    aligned). `intact()` says whether both bands still hold their pattern,
    i.e. nothing wrote past either end."""

    def __init__(self, nbytes: int, dev, fill: int = GUARD_VALUE):
        self.nbytes = int(nbytes)
        self.raw = torch.full((GUARD_BYTES + self.nbytes + GUARD_BYTES,), fill, dtype=torch.uint8, device=dev)
        self.raw[:GUARD_BYTES] = GUARD_VALUE
        self.raw[GUARD_BYTES + self.nbytes:] = GUARD_VALUE

    def view(self, dtype, shape):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        assert n <= self.nbytes
        return self.raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(*shape)

    def bytes(self):
        return self.raw[GUARD_BYTES:GUARD_BYTES + self.nbytes]

    def intact(self) -> bool:
        torch.cuda.synchronize()
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.nbytes:]
        return bool((head == GUARD_VALUE).all().item()) and bool((tail == GUARD_VALUE).all().item())
