"""The benchmark's accounting, on the CPU: algorithmic bytes per call against
the byte formula written out term by term, the counter summary's calibration
scaling and source-hash check, and the refusal of more than one GPU."""

import csv
import importlib.util
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_bytes_term_by_term(bench):
    # 3 sequences, 4 query / 2 KV heads, head_dim 64, blocks of 16, bf16
    c = SimpleNamespace(etype="bf16", num_seqs=3, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16)
    lens = np.array([1, 16, 33], dtype=np.int32)
    got = bench.decode_bytes(c, lens)
    kv = (1 + 16 + 33) * 2 * 64 * 2 * 2        # K and V of every context token
    q = 3 * 4 * 64 * 2
    out = 3 * 4 * 64 * 4                       # fp32 output
    ids = 4 * (1 + 1 + 3)                      # one block id per block touched
    lens_b = 4 * 3
    assert got == {"kv": kv, "q": q, "out": out, "ids": ids, "lens": lens_b,
                   "total": kv + q + out + ids + lens_b}


def test_write_bytes(bench):
    c = SimpleNamespace(etype="f32", num_kv_heads=8, head_dim=128)
    # new K and V read once and stored once; the separate call also reads the slot mapping
    assert bench.write_bytes(c, 5, True) == 2 * 5 * 8 * 128 * 4 * 2
    assert bench.write_bytes(c, 5, False) == 2 * 5 * 8 * 128 * 4 * 2 + 4 * 5


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": value})


def test_counter_summary_scaling_and_hash(bench, tmp_path, monkeypatch):
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    dk = "void pa::(anonymous namespace)::decode_kernel<X, 128>(pa::DecodeParams)"
    mk = "void pa::(anonymous namespace)::merge_kernel<128, unsigned short, 1>(pa::DecodeParams)"
    # a 1 MiB calibration copy whose fetch counter reads half its size (the
    # counter's unit is 64 bytes where the copy moves 128) and whose write
    # counter reads it exactly
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, [("__amd_rocclr_copyBuffer", 512.0), (dk, 100.0), (dk, 300.0), (mk, 10.0)])
    _counter_csv(write, [("__amd_rocclr_copyBuffer", 1024.0), (dk, 40.0), (dk, 40.0), (mk, 6.0)])
    entry = bench.summarize_counters(str(fetch), str(write), "llama3_8b", 1)
    assert entry["fetch_scale"] == 2.0 and entry["write_scale"] == 1.0
    # per launch: mean over dispatches, fetch x2, write x1, KiB -> bytes
    assert entry["kernels"]["decode_kernel"]["traffic_bytes"] == (200.0 * 2 + 40.0) * 1024
    assert entry["kernels"]["merge_kernel"]["traffic_bytes"] == (10.0 * 2 + 6.0) * 1024
    assert json.loads(traffic.read_text())["llama3_8b"]["kernel_hash"] == bench.kernel_hash("llama3_8b")
    assert bench.traffic_for("decode_kernel+merge_kernel", "llama3_8b") == (440.0 + 26.0) * 1024
    assert bench.traffic_for("decode_kernel", "llama3_8b") == 440.0 * 1024
    assert bench.traffic_for("write_kv_kernel+decode_kernel", "llama3_8b") is None  # not in the record
    # a record taken on other kernel sources is not used
    rec = json.loads(traffic.read_text())
    rec["llama3_8b"]["kernel_hash"] = "0" * 16
    traffic.write_text(json.dumps(rec))
    assert bench.traffic_for("decode_kernel+merge_kernel", "llama3_8b") is None


def test_step_kernels_from_launch_counts(bench):
    assert bench.step_kernels(1, True) == "decode_kernel"
    assert bench.step_kernels(2, True) == "decode_kernel+merge_kernel"
    assert bench.step_kernels(4, True) == "link_kernel+plan_kernel+decode_kernel+merge_kernel"
    assert bench.step_kernels(1, False) == "write_kv_kernel+decode_kernel"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
