"""Host-side checks of bench.py: the one-GPU guard and its byte accounting."""

import os
import subprocess
import sys

import numpy as np

import bench
import dequant_matmul_gptq_amd as dq
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_launch_bytes_count_each_operand_once():
    spec = wl.LLAMA7B_DECODE[0]                     # 4096 -> 4096, 4-bit, g128
    L = dq.Layout(spec.K, spec.N, spec.group_size, wl.bit_map(spec))
    codes = 4096 * 4096 // 2
    scales = 32 * 4096 * 2
    zeros = 32 * 4096 // 2                          # zero points at 4 bits, as in the metric's weight bytes
    act = 4096 * 2 + 4096 * 4 + 4096 * 2            # x, perm, y
    assert bench.launch_bytes(L, 1) == codes + scales + zeros + act
    assert bench.launch_bytes(L, 1, zeros=False) == codes + scales + act
    assert bench.launch_bytes(L, 1, perm=False) == codes + scales + zeros + act - 4096 * 4
    # one byte model: the weight bytes of the metric are the same terms
    assert wl.weight_bytes(spec) == codes + scales + zeros
    assert bench.launch_bytes(L, 1) - act == wl.weight_bytes(spec)


def test_mixed_width_codes_bytes():
    bits = np.array([6, 5, 4, 3, 2, 8], np.uint8)
    L = dq.Layout(6 * 32, 64, 32, bits)
    codes = int(sum(int(b) * 32 * 64 for b in bits)) // 8
    assert bench.launch_bytes(L, 1, zeros=False) == codes + 6 * 64 * 2 + 192 * 2 + 192 * 4 + 64 * 2


def test_recorded_traffic_is_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "t.txt"
    f.write_text(f"# comment\nkernel_sources_sha256_16: {bench.row_kernel_digest()}\nhbm_bytes_per_launch: 123.0\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic() == 123
    f.write_text("kernel_sources_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    assert bench.recorded_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic() is None


def test_gemm_traffic_follows_its_own_sources(tmp_path, monkeypatch):
    """The prefill kernel's recorded traffic is keyed to qgemm.hip and its
    headers, not to the decode kernel's sources."""
    assert bench.gemm_kernel_digest() != bench.row_kernel_digest()
    f = tmp_path / "g.txt"
    f.write_text(f"kernel_sources_sha256_16: {bench.gemm_kernel_digest()}\nhbm_bytes_per_launch: 4.5e8\n")
    monkeypatch.setattr(bench, "GEMM_TRAFFIC_FILE", str(f))
    assert bench.recorded_gemm_traffic() == 450000000
    f.write_text(f"kernel_sources_sha256_16: {bench.row_kernel_digest()}\nhbm_bytes_per_launch: 4.5e8\n")
    assert bench.recorded_gemm_traffic() is None


def test_grouped_launch_bytes_share_x_and_perm():
    spec = wl.LLAMA7B_DECODE[0]
    L = dq.Layout(spec.K, spec.N, spec.group_size, wl.bit_map(spec))
    one = bench.launch_bytes(L, 1)
    shared = 4096 * 2 + 4096 * 4
    assert bench.launch_bytes(L, 1, count=3) == 3 * (one - shared) + shared


def test_decode_groups_layer_order():
    mats = [dict(shape=s, i=i) for i, s in enumerate([0, 0, 0, 0, 1, 1, 2] * 2)]
    g = bench.decode_groups(mats, True)
    assert [len(x["mats"]) for x in g] == [3, 1, 2, 1] * 2
    assert [x["shape"] for x in g] == [0, 0, 1, 2] * 2
    assert [m["i"] for x in g for m in x["mats"]] == list(range(14))
    u = bench.decode_groups(mats, False)
    assert [len(x["mats"]) for x in u] == [1] * 14


def test_lora_bytes_count_each_operand_once():
    # 7B decode 4096 -> 4096 at rank 16: x 8 KiB, A 128 KiB, B 128 KiB, delta 16 KiB
    assert bench.lora_bytes(1, 4096, 4096, 16) == 2 * 4096 + 2 * 4096 * 16 + 2 * 16 * 4096 + 4 * 4096
    assert bench.lora_bytes(0, 4096, 4096, 16) == 2 * 4096 * 16 * 2
