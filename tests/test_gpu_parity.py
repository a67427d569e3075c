"""GPU parity: libfd (through its C ABI) against the fp64 CPU oracle on the
seeded workloads of the pages, at the stated max-abs tolerances (fp32 1e-5,
fp16 2e-3, bf16 1e-2), plus the pages' own cases."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_cases.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.empty_cache()


def check_full(inp, ns, tol=None, scale=None):
    w = inp.workload
    out = H.gpu_attention(inp, ns, scale=scale)
    ref = H.oracle_full(inp, ns, scale=scale)
    err = H.max_err(H.host(out), ref)
    print(f"  {w.name} ns={ns} max_abs_err={err:.3e}", flush=True)
    assert err <= (tol if tol is not None else H.TOL[w.dtype]), (w.name, ns, err)
    return out


# ------------------------------------------------------------ workloads --
@pytest.mark.parametrize("ns", [7, 1, 64, 1000])
def test_tiny_exactness_case(ns):
    """fp32, 8 query heads on 1 KV head, d=128, 10,000 keys
    (04_flash_decoding.py demo 1 splits {1, 7, 64, 1000}); the partials of
    every split are checked too."""
    inp = W.make_inputs(W.tiny(), H.DEV)
    check_full(inp, ns)
    ws, opart, lse2 = H.gpu_split(inp, ns)
    q, k, v = H.host(inp.q), H.host(inp.k), H.host(inp.v)
    op_ref, lse_ref = oracle.attention_partials(q, k, v, [0, 10000], 8, 1, ns, W.tiny().sm_scale)
    assert H.max_err(opart, op_ref) <= 1e-5
    assert H.max_err(lse2, lse_ref * H.LOG2E) <= 1e-4


@pytest.mark.parametrize("dim", [16, 32, 64, 128])
def test_mha_head_dims(dim):
    """MHA, batch 4, 32 heads, 4096 keys, fp16, [B,H,S,D], ns=16; the d=128
    case is the benchmark's workload and launch configuration."""
    w = W.mha(dim)
    inp = W.make_inputs(w, H.DEV)
    check_full(inp, w.num_splits)


@pytest.mark.parametrize("batch,kv_len", W.FD_UBENCH_SHAPES)
def test_fd_microbenchmark_shapes(batch, kv_len):
    """16 query heads / 2 KV heads, d=128, fp16, split count from the planner."""
    w = W.fd_ubench(batch, kv_len)
    inp = W.make_inputs(w, H.DEV)
    fd = H.fd()
    ns = fd.fd_plan_splits(w.batch, w.heads, w.kv_heads, w.dim, fd.FD_F16, inp.lengths)
    check_full(inp, ns)


@pytest.mark.parametrize("batch,kv_len", W.FD_UBENCH_SHAPES)
def test_unpacked_comparator_shapes(batch, kv_len):
    """The unpacked comparison path (one query head per workgroup, no split,
    as in 04_flash_decoding.py demos 2-3) on the same shapes gives the
    oracle's result."""
    w = W.fd_ubench(batch, kv_len)
    inp = W.make_inputs(w, H.DEV)
    fd = H.fd()
    prev = fd.fd_set_kernel_path(fd.FD_PATH_UNPACKED)
    try:
        check_full(inp, 1)
    finally:
        fd.fd_set_kernel_path(prev)


@pytest.mark.parametrize("kv_len", W.LLAMA_LENS)
@pytest.mark.parametrize("batch", W.LLAMA_BATCHES)
def test_llama_long_context(batch, kv_len):
    """32/8 heads, d=128, bf16, split count from the planner, in the launch
    configuration the benchmark times. Up to 16 x 8K keys the whole batch is
    compared at once; above that (2.1 and 8.6 GB of KV at batch 16) every
    (sequence, KV head) pair is compared, its K/V rows copied to the host one
    pair at a time."""
    w = W.llama(batch, kv_len)
    inp = W.make_inputs(w, H.DEV)
    fd = H.fd()
    ns = fd.fd_plan_splits(w.batch, w.heads, w.kv_heads, w.dim, fd.FD_BF16, inp.lengths)
    if batch * kv_len <= 16 * 8192:
        check_full(inp, ns)
    else:
        check_every_pair(inp, ns)
    del inp
    torch.cuda.empty_cache()


def check_every_pair(inp, ns):
    """Every (sequence, KV head) pair of a whole call against the oracle, its
    K/V rows copied to the host one pair at a time."""
    w = inp.workload
    G = w.group
    out = H.host(H.gpu_attention(inp, ns))
    assert np.isfinite(out).all()
    pairs = [(b, j) for b in range(w.batch) for j in range(w.kv_heads)]
    refs = H.oracle_pairs(inp, pairs, workers=8)
    worst = 0.0
    for (b, j), ref in refs.items():
        err = H.max_err(out[b, j * G:(j + 1) * G], ref)
        worst = max(worst, err)
        assert err <= H.TOL[w.dtype], (b, j, err)
    print(f"  {w.name} ns={ns}: {len(pairs)} pairs, max_abs_err={worst:.3e}", flush=True)


def test_bench_line_under_the_steal_schedule():
    """The bench line as the benchmark times it: Llama B16 x 131,072 keys
    under the steal schedule, the planner's steal layout (8 slots on 256
    CUs), every (sequence, KV head) pair against the oracle."""
    fd = H.fd()
    w = W.llama(16, 131072)
    inp = W.make_inputs(w, H.DEV)
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    try:
        ns = fd.fd_plan_splits(w.batch, w.heads, w.kv_heads, w.dim, fd.FD_BF16, inp.lengths)
        H.announce("steal layout", ns)
        assert ns > 2
        check_every_pair(inp, ns)
    finally:
        fd.fd_set_schedule(prev)
    del inp
    torch.cuda.empty_cache()


def test_varlen_under_the_queue_schedule():
    """The varlen workload as the benchmark times it: the queue schedule,
    ns=8, against the oracle."""
    fd = H.fd()
    w = W.varlen_qwen()
    inp = W.make_inputs(w, H.DEV)
    prev = fd.fd_set_schedule(fd.FD_SCHED_QUEUE)
    try:
        check_full(inp, W.varlen_splits(w, inp.lengths))
    finally:
        fd.fd_set_schedule(prev)


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_llama_split_sweep(path):
    """batch 1, 64K keys, ns in {1, 2, ..., 128}: every split count gives the
    oracle's result, on both split kernels."""
    fd = H.fd()
    prev = fd.fd_set_kernel_path({"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA}[path])
    try:
        w = W.llama(1, 65536)
        inp = W.make_inputs(w, H.DEV)
        ref = H.oracle_full(inp)
        for ns in W.LLAMA_SWEEP_SPLITS:
            out = H.host(H.gpu_attention(inp, ns))
            err = H.max_err(out, ref)
            print(f"  {path} ns={ns} err={err:.3e}", flush=True)
            assert err <= H.TOL["bf16"], (ns, err)
    finally:
        fd.fd_set_kernel_path(prev)


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_varlen_both_kernels(path):
    """The varlen GQA workload (group 7) on each split kernel explicitly."""
    fd = H.fd()
    prev = fd.fd_set_kernel_path({"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA}[path])
    try:
        w = W.varlen_qwen()
        inp = W.make_inputs(w, H.DEV)
        check_full(inp, W.varlen_splits(w, inp.lengths))
    finally:
        fd.fd_set_kernel_path(prev)


def test_varlen_packed_gqa():
    """28/4 heads (group 7), d=128, fp16, 32 sequences of 64..32768 keys in
    [total_kv, kv_heads, dim] with cu_seqlens_k, ns=8 (1 if min length < 8)."""
    w = W.varlen_qwen()
    inp = W.make_inputs(w, H.DEV)
    ns = W.varlen_splits(w, inp.lengths)
    check_full(inp, ns)


# ------------------------------------------------------- the pages' cases --
def test_page_selftest_case():
    """flash_decode_splitk.py self-test: B2 H4 D64 L256 ns4 fp16; its own
    tolerance (atol=rtol=2e-2) and the tighter fp16 bound both hold."""
    c = json.load(open(GOLDEN))["miniinfer_selftest"]
    w = W.Workload("page_selftest", c["batch"], c["heads"], c["kv_heads"], c["dim"], c["dtype"],
                   kv_len=c["kv_len"], layout=c["layout"], num_splits=c["num_splits"])
    inp = W.make_inputs(w, H.DEV, seed=c["seed"])
    out = check_full(inp, c["num_splits"])
    ref = H.oracle_full(inp, c["num_splits"])
    assert np.all(np.abs(H.host(out) - ref) <= c["page_atol"] + c["page_rtol"] * np.abs(ref))


def test_page_default_shape():
    """decode_attention_splitkv.py DEFAULT_SHAPE: batch 8, 28/4 heads,
    total_kv 65536 (8 x 8192), d=128, ns=8, fp16 packed."""
    c = json.load(open(GOLDEN))["tilelang_default_shape"]
    B = c["batch"]
    w = W.Workload("page_default_shape", B, c["heads"], c["kv_heads"], c["dim"], c["dtype"],
                   kv_len=c["total_kv"] // B, layout=c["layout"], num_splits=c["num_splits"])
    inp = W.make_inputs(w, H.DEV)
    assert sum(inp.lengths) == c["total_kv"] and max(inp.lengths) == c["max_kv"]
    check_full(inp, c["num_splits"])
