"""Host logic of bench.py (no GPU): the single-GPU guard, the kernel-source
hash that keys the committed HBM traffic counters, the committed counters
themselves, and the workgroup count it reports."""
import json
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""


def test_code_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no\n overflow check */ }\n"
    b = "int f(int x) {\n    return 2 * x;   // other words\n}"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_kernel_hash_is_stable_and_short():
    h = bench.kernel_hash()
    assert h == bench.kernel_hash()
    assert len(h) == 16 and all(ch in "0123456789abcdef" for ch in h)


def test_committed_traffic_counters_are_plausible():
    """Every committed entry: HBM bytes per split launch between the
    algorithmic K/V bytes (each byte read once) and 10 % above them (the
    partials, q and the counters' rounding), for a workload bench.py knows."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    names = {w.name for w in W.all_workloads()}
    assert t, "no committed traffic counters"
    for name, e in t.items():
        assert name in names
        ratio = e["hbm_bytes_per_launch"] / e["algorithmic_bytes_per_launch"]
        assert 0.99 <= ratio <= 1.10, (name, ratio)
        assert abs(e["fetch_scale"] - 0.5) < 0.05 and abs(e["write_scale"] - 1.0) < 0.05


def test_traffic_is_reported_only_for_the_current_kernel():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for name, e in t.items():
        got = bench.traffic_for(name)
        if e["kernel_hash"] == bench.kernel_hash():
            assert got == e["hbm_bytes_per_launch"]
        else:
            assert got is None
    assert bench.traffic_for("no_such_workload") is None


def test_split_workgroups_counts_row_chunks_and_splits():
    llama = W.llama(16, 8192)             # 8 KV heads, group 4
    assert bench.split_workgroups(llama, 2, 8) == 16 * 8 * 1 * 2
    assert bench.split_workgroups(llama, 2, 1) == 16 * 8 * 4 * 2   # unpacked: one row each
    varlen = W.varlen_qwen()              # 4 KV heads, group 7
    assert bench.split_workgroups(varlen, 8, 8) == 32 * 4 * 8


def test_default_workload_is_the_largest_configuration():
    """The bench line runs the largest single-GPU workload: Llama-3.1-8B
    shape at batch 16 and 131,072 keys (8.59 GB of K/V per call)."""
    def kv_bytes(w):
        assert w.kv_len is not None or w.varlen_range is not None
        keys = w.batch * (w.kv_len if w.kv_len is not None else w.varlen_range[1])
        return keys * w.kv_heads * w.dim * 2 * w.elem_bytes
    biggest = max(W.all_workloads(), key=kv_bytes)
    assert bench.DEFAULT_WORKLOAD == biggest.name == "llama8b_b16_l131072_h32kv8_d128_bf16"
    assert kv_bytes(biggest) == 16 * 131072 * 8 * 128 * 2 * 2


def test_context_points_are_the_other_long_context_and_gqa_workloads():
    """A default bench run also times these workloads briefly: each is a
    known workload with a committed traffic entry, none is the headline,
    and together they cover the flash-decoding 16/2-head shapes, Llama-8B
    at batch 1 and 16, and the varlen batch."""
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    names = bench.CONTEXT_WORKLOADS
    assert len(set(names)) == len(names) and bench.DEFAULT_WORKLOAD not in names
    ws = [bench.workload_by_name(n) for n in names]
    assert all(n in t for n in names)
    assert any(w.heads == 16 and w.kv_heads == 2 for w in ws)
    assert {w.batch for w in ws if w.name.startswith("llama8b")} == {1, 16}
    assert any(w.varlen_range is not None for w in ws)

