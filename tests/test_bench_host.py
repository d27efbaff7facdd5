"""Host-side logic of bench.py (no GPU): the algorithmic byte counts, the
single-GPU guard and the tie between counter data and the kernel sources."""
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def shape(B, n_k, Hkv=8, d=128):
    return types.SimpleNamespace(B=B, Hkv=Hkv, d=d, n_k=np.asarray(n_k, dtype=np.int64))


def test_llama_layer_bytes():
    # all of K (B H_kv n_k d, 2 bytes each) plus S value rows per KV head
    wl = shape(1, [32768])
    assert bench.algorithmic_bytes(wl, 128) == 67_108_864 + 262_144 == 67_371_008
    assert [bench.algorithmic_bytes(wl, S) for S in (32, 64, 256)] == [67_174_400, 67_239_936, 67_633_152]
    # the dense step reads all of K and all of V
    assert bench.algorithmic_bytes(wl, 128, dense=True) == 134_217_728


def test_sweep_and_ragged_bytes():
    # 8192 n_k + 1,048,576 per sequence batch of 4 at S = 128
    for n in (4096, 16384, 65536, 131072):
        assert bench.algorithmic_bytes(shape(4, [n] * 4), 128) == 8192 * n + 1_048_576
    # ragged lengths count each sequence's own keys, not the padded capacity
    wl = shape(3, [10, 2000, 777])
    assert bench.algorithmic_bytes(wl, 16) == (10 + 2000 + 777) * 8 * 128 * 2 + 3 * 8 * 16 * 128 * 2


def test_fp8_key_bytes():
    # one byte per key element, fp16 value rows
    wl = shape(1, [32768])
    assert bench.fp8k_bytes(wl, 128) == 33_554_432 + 262_144 == 33_816_576


def test_traffic_tied_to_kernel_sources(tmp_path, monkeypatch):
    prof = tmp_path / "traffic.txt"
    prof.write_text("hbm_bytes_per_launch: 123\nkernel_source_sha256: %s\n" % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 123.0
    prof.write_text("hbm_bytes_per_launch: 123\nkernel_source_sha256: %s\n" % ("0" * 64))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    for extra in ([], ["--workload", "layers32"], ["--workload", "ceiling"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"] + extra,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode != 0
        assert "single GPU" in r.stderr
        assert r.stdout.strip() == ""


def test_value_rows_counts_distinct_per_kv_head():
    import torch
    # B=1, H_q=4, H_kv=2 (G=2), S=3; heads 0,1 share KV head 0, heads 2,3 KV head 1
    idx = torch.tensor([[[5, 5, 9], [9, 1, 1], [0, 0, 0], [-1, -1, -1]]], dtype=torch.int32)
    r = bench.value_rows(idx, 2, 64)
    # KV head 0: {1, 5, 9}; KV head 1: {0} (the -1 entries are no rows)
    assert r["distinct_measured"] == 4
    assert r["distinct_bytes"] == 4 * 64 * 2
    assert r["S_per_kv_head"] == 2 * 3 and r["G_S_rows"] == 4 * 3
    # the same key index in different sequences is a different row
    two = torch.stack([idx[0], idx[0]])
    assert bench.value_rows(two, 2, 64)["distinct_measured"] == 8
