"""The figures bench.py divides by, checked on the host: algorithmic bytes
and flops against independent counts on the workloads, and the traffic
record's counter arithmetic on synthetic counter files.  CPU only."""

import csv
import json
import os

import numpy as np

import bench
from paged_kv_cache_326_amd import synth


def test_decode_bytes_of_the_benchmark_layer():
    w = synth.config(2, poison_unused=False)
    # 16 sequences x 4096 tokens x 8 KV heads x 128 dims x 2 bytes, K and V;
    # queries in and outputs out (16 x 64 heads x 128 x 2 bytes each); 256
    # table entries and one length per sequence, 4 bytes each.
    kv = 16 * 4096 * 8 * 128 * 2 * 2
    qo = 2 * 16 * 64 * 128 * 2
    assert bench.algorithmic_decode_bytes(w) == kv + qo + 16 * 256 * 4 + 16 * 4 == 268976192
    assert bench.algorithmic_decode_bytes(w, kv_elem_bytes=1) == kv // 2 + qo + 16 * 256 * 4 + 16 * 4 == 134758464


def test_decode_bytes_count_only_the_blocks_read():
    w = synth.custom(seed=1, dtype="f16", num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                     seq_lens=[1, 16, 17, 0], q_lens=[1, 1, 1, 0], pool_factor=1.5, poison_unused=False)
    tokens = 1 + 16 + 17
    blocks = 1 + 1 + 2
    expect = tokens * 2 * 64 * 2 * 2 + 2 * 4 * 8 * 64 * 2 + blocks * 4 + 4 * 4
    assert bench.algorithmic_decode_bytes(w) == expect


def test_prefill_flops_by_brute_force():
    w = synth.custom(seed=2, dtype="bf16", num_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                     seq_lens=[40, 9, 100], q_lens=[7, 9, 33], poison_unused=False)
    pairs = 0
    for L, q in zip(w.seq_lens.tolist(), w.q_lens.tolist()):
        ctx = L - q
        for i in range(q):
            for k in range(L):
                pairs += k <= ctx + i
    assert bench.prefill_flops(w) == 4 * 64 * 4 * pairs


def test_mixed_batch_prefill_flops():
    w = synth.config(5, poison_unused=False)
    pre, _ = synth.prefill_decode_split(w)
    wp = w.subset(pre)
    # 4 chunks of 512 over 3584 cached tokens: each chunk sees 512 * 3584 +
    # 512 * 513 / 2 (query, key) pairs; 64 heads, 4 * 128 flops a pair.
    assert bench.prefill_flops(wp) == 4 * 128 * 64 * 4 * (512 * 3584 + 512 * 513 // 2) == 257731592192


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, counter, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_scales_the_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    part = "void pa::decode_partition_kernel<8, DF16_Li128ELi16ELi8, ...>"
    merge = "decode_reduce_kernel<...>"
    copy = "__amd_rocclr_copyBuffer"
    n_kib = bench.COPY_CALIBRATION_MIB * 1024
    _counters(tmp_path / "pmc_copy_fetch", [(copy, "FETCH_SIZE", n_kib / 2), (copy, "FETCH_SIZE", n_kib / 2)])
    _counters(tmp_path / "pmc_copy_write", [(copy, "WRITE_SIZE", n_kib)])
    # Two dispatches of each kernel: the record takes the mean.
    _counters(tmp_path / "pmc_fetch", [(part, "FETCH_SIZE", 1000.0), (part, "FETCH_SIZE", 1200.0),
                                       (merge, "FETCH_SIZE", 10.0), (merge, "FETCH_SIZE", 10.0)])
    _counters(tmp_path / "pmc_write", [(part, "WRITE_SIZE", 50.0), (part, "WRITE_SIZE", 50.0),
                                       (merge, "WRITE_SIZE", 4.0), (merge, "WRITE_SIZE", 4.0)])
    out = tmp_path / "record.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(out))
    bench.write_traffic_record(str(tmp_path))
    rec = json.loads(out.read_text())
    # The copy moved n_kib each way but FETCH_SIZE read half of it: fetch x2.
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    assert rec["partition_kernel"]["bytes"] == (1100 * 2 + 50) * 1024
    assert rec["merge_kernel"]["bytes"] == (10 * 2 + 4) * 1024
    assert rec["bytes_per_call"] == (1100 * 2 + 50 + 10 * 2 + 4) * 1024
    assert rec["decode_source_sha256"] == bench.decode_source_digest()
    assert np.isclose(rec["ratio_to_algorithmic"], rec["bytes_per_call"] / rec["algorithmic_bytes_per_call"], atol=1e-4)
