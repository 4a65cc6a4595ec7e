"""The kernels' packing and unpacking helpers, compiled for the host, against
the oracle: the kernel packer must write the oracle's words, and every
unpacked pair must hold 1024 + code of the two rows it claims (no GPU)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe_output(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("probe") / "format_probe")
    cmd = [hipcc, "-std=c++20", "-O1", "-x", "hip", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "dequant_matmul_gptq_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "format_probe.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    return subprocess.run([exe], check=True, capture_output=True, text=True).stdout


def _records(text):
    lines = [l for l in text.strip().splitlines() if not l.startswith("POSBAD")]
    for i in range(0, len(lines), 4):
        b = int(lines[i].split()[1])
        codes = np.array([int(v) for v in lines[i + 1].split()[1:]], np.uint8)
        words = np.array([int(v) for v in lines[i + 2].split()[1:]], np.uint32)
        pairs = [tuple(int(t) for t in v.split(":")) for v in lines[i + 3].split()[1:]]
        yield b, codes, words, pairs


def test_kernel_packer_matches_oracle(probe_output):
    n = 0
    for b, codes, words, _ in _records(probe_output):
        assert np.array_equal(oracle.pack(codes[:, None], [b], 32)[:, 0], words), b
        n += 1
    assert n == 24


def test_kernel_pairs_cover_every_row_once(probe_output):
    for b, codes, words, pairs in _records(probe_output):
        rows = sorted([p[0] for p in pairs] + [p[1] for p in pairs])
        assert rows == list(range(32)), b
        q = oracle.unpack(words[:, None], [b], 32, 32)[:, 0]
        for lo, hi, v, vs, e in pairs:
            assert v & 0xFFFF == 0x6400 + int(q[lo]) and v >> 16 == 0x6400 + int(q[hi]), (b, lo, hi, hex(v))
            assert q[lo] == codes[lo] and q[hi] == codes[hi]
            # scaled unpacking: the float16 halves are exactly 1024 + q * 2^e
            assert 0 <= e and e + b <= 10
            for half, row in ((vs & 0xFFFF, lo), (vs >> 16, hi)):
                val = float(np.array([half], np.uint16).view(np.float16)[0])
                assert val == 1024.0 + int(q[row]) * 2.0 ** e, (b, row, e, hex(vs))


def test_pair_position_inverts_pair_rows(probe_output):
    line = [l for l in probe_output.splitlines() if l.startswith("POSBAD")]
    assert line == ["POSBAD 0"]
