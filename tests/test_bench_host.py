"""CPU checks of bench.py's host side: it refuses more than one GPU, the
algorithmic bytes and FLOPs that the roofline divides by match hand counts
for small batches, and rocprofv3 counters are scaled by the copy calibration
and dropped once the kernel source changes."""
import csv
import json
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


def small(dt=W.BF16, q_len=1, topk=None):
    return W.small_case(seed=5, batch=2, num_heads=16, head_size=576, kv_lora_rank=512,
                        page_size=16, seq_lens=(3, 70), kv_dtype=dt, q_len=q_len, topk=topk)


def test_algorithmic_counts_dense_bf16():
    a = bench.algorithmic(small())
    kv = (3 + 70) * 1152                        # cache rows read once, 576 bf16 each
    table = (1 + 5) * 4                         # ceil(3/16) + ceil(70/16) int32 entries
    stage1 = kv + 2 * 16 * 576 * 2 + table + 2 * 4
    assert a["kv_bytes"] == kv and a["stage1_bytes"] == stage1
    assert a["total_bytes"] == stage1 + 2 * 16 * 512 * 2 + 2 * 16 * 4
    assert a["flops"] == 2 * 16 * 73 * (576 + 512) and a["tokens"] == 73


@pytest.mark.parametrize("dt,row", [(W.FP8_E4M3, 576), (W.FP8_PER_TOKEN, 580),
                                    (W.INT8_PER_TOKEN, 580), (W.INT4_PER_TOKEN, 292)])
def test_algorithmic_row_bytes_of_quantised_caches(dt, row):
    """1-byte codes (per-token: plus the 4-byte scale, not the unused pad);
    int4: 288 code bytes plus the scale."""
    assert bench.algorithmic(small(dt))["kv_bytes"] == 73 * row


def test_algorithmic_flops_of_multi_token_decode():
    """q_len = 2: token 0 sees n - 1 keys, token 1 sees n."""
    a = bench.algorithmic(small(q_len=2))
    assert a["flops"] == 2 * 16 * ((2 + 69) + (3 + 70)) * (576 + 512)
    assert a["stage1_bytes"] == 73 * 1152 + 2 * 2 * 16 * 576 * 2 + 24 + 8


def test_algorithmic_counts_sparse():
    inp = small(topk=32)
    k = int(inp.topk_lens.sum())
    a = bench.algorithmic(inp)
    assert a["kv_bytes"] == k * 1152 and a["flops"] == 2 * 16 * k * (576 + 512)
    assert a["stage1_bytes"] == k * 1152 + 2 * 16 * 576 * 2 + 8 * k + 8


def write_counters(path, counter, stage1_kib, copy_kib):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in stage1_kib:
            w.writerow({"Kernel_Name": "void mla::mla_stage1<32, 4>(Stage1Params)",
                        "Counter_Name": counter, "Counter_Value": v})
        w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": copy_kib})


def test_counters_are_scaled_by_the_copy_and_tied_to_the_source(tmp_path, monkeypatch, capsys):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the 1 GiB copy reads FETCH_SIZE = 512 Mi KiB-units: a scale of 2; WRITE_SIZE reads it exactly
    write_counters(tmp_path / "fetch.csv", "FETCH_SIZE", [100.0, 300.0], 524288.0)
    write_counters(tmp_path / "write.csv", "WRITE_SIZE", [40.0, 60.0], 1048576.0)
    bench.ingest_pmc(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), "wl")
    capsys.readouterr()
    t = json.load(open(tmp_path / "profiles" / "mla_stage1_wl_traffic.json"))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == pytest.approx(200 * 1024 * 2 + 50 * 1024)
    assert bench.load_traffic("wl") == pytest.approx(t["bytes_per_launch"])
    # counters taken on another version of the kernel source are not reported
    t["kernel_sha256_16"] = "0" * 16
    json.dump(t, open(tmp_path / "profiles" / "mla_stage1_wl_traffic.json", "w"))
    assert bench.load_traffic("wl") is None
