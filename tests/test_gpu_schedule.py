"""GPU tests of the two launch variants of the whole call:

  * FD_COMBINE_FUSED -- one launch: the last split workgroup of each
    (sequence, KV head) merges the unit's partials ("04_flash_decoding.py",
    demo 3: flash decoding's time is one KV read plus two kernels' fixed
    costs; this pays one). Checked against the fp64 oracle on every kernel
    path, with empty sequences, empty splits (num_splits > L), groups larger
    than one pass and the largest split count; the arrival counters are zero
    after every call, repeated calls are bitwise identical, and partials
    pre-filled with NaN never reach the output.
  * FD_SCHED_QUEUE -- a device-sized grid that claims segments from a
    counter. The segments and their arithmetic are those of the static
    schedule, so outputs and partials must be bitwise equal to it, whatever
    the counter held before the call.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    fd = H.fd()
    yield
    fd.fd_set_combine(fd.FD_COMBINE_SEPARATE)
    fd.fd_set_schedule(fd.FD_SCHED_AUTO)
    fd.fd_set_kernel_path(fd.FD_PATH_AUTO)


@pytest.fixture(params=["valu", "mfma", "unpacked"])
def kernel_path(request):
    fd = H.fd()
    prev = fd.fd_set_kernel_path({"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA,
                                  "unpacked": fd.FD_PATH_UNPACKED}[request.param])
    H.announce("kernel path", request.param)
    yield request.param
    fd.fd_set_kernel_path(prev)


def _layout_sizes(w, ns):
    """Byte offsets of (LSE, control block, arrival counters) in the
    workspace, per include/fd.h."""
    rows = w.batch * w.heads * ns
    lse_off = (rows * w.dim * 4 + 255) // 256 * 256
    ctl_off = lse_off + (rows * 4 + 255) // 256 * 256
    return lse_off, ctl_off, ctl_off + 256


def fused_call(inp, ns, nan_partials=True, workspace=None):
    """fd_decode_attention in the fused mode on a workspace whose partials
    are NaN and whose control block is zero; returns (out, workspace)."""
    fd = H.fd()
    w = inp.workload
    if workspace is None:
        n = fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim)
        workspace = torch.zeros(n, dtype=torch.uint8, device=H.DEV)
        if nan_partials:
            _, ctl_off, _ = _layout_sizes(w, ns)
            workspace[:ctl_off].view(torch.float32).fill_(float("nan"))
    H.announce("fused", w.name, f"ns={ns}", f"lens[:4]={inp.lengths[:4]}")
    prev = fd.fd_set_combine(fd.FD_COMBINE_FUSED)
    try:
        out = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                     workspace=workspace, layout=w.layout)
        torch.cuda.synchronize()
    finally:
        fd.fd_set_combine(prev)
    return out, workspace


def check_vs_oracle(inp, out):
    """Every output row against the oracle's direct attention; sequences with
    no key must give zero rows (the oracle refuses them)."""
    w = inp.workload
    o = H.host(out)
    G = w.group
    live = [(b, j) for b, L in enumerate(inp.lengths) if L > 0 for j in range(w.kv_heads)]
    for b, L in enumerate(inp.lengths):
        if L == 0:
            assert not o[b].any(), b
    ref = H.oracle_pairs(inp, live)
    err = max(H.max_err(o[b, j * G:(j + 1) * G], ref[(b, j)]) for b, j in live)
    assert err <= H.TOL[w.dtype], err


def arrivals(workspace, w, ns):
    _, _, arr_off = _layout_sizes(w, ns)
    return workspace[arr_off:arr_off + 4 * w.batch * w.heads].view(torch.int32).cpu().numpy()


FUSED_CASES = [  # (name, workload, lengths or None, num_splits)
    ("tiny_ns7", W.tiny(), None, 7),
    ("mha_d128", W.mha(128), None, 16),
    ("mha_d16", W.mha(16), None, 16),
    ("ubench_b8_l8192", W.fd_ubench(8, 8192), None, 16),
    ("ubench_b1_l65536", W.fd_ubench(1, 65536), None, 128),
    ("llama_b1_l8192", W.llama(1, 8192), None, 32),
    ("llama_b16_l1024", W.llama(16, 1024), None, 2),
    ("varlen_g7", W.Workload("v7", 6, 28, 4, 128, "f16", kv_len=None), [3000, 65, 1, 0, 2900, 700], 8),
    ("f32_d64_g3", W.Workload("f32g3", 3, 6, 2, 64, "f32", kv_len=None), [1000, 17, 513], 5),
    ("bf16_d32_g16", W.Workload("g16", 2, 32, 2, 32, "bf16", kv_len=None), [700, 300], 4),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c[0])
def test_fused_matches_oracle(case, kernel_path):
    name, w, lengths, ns = case
    inp = W.make_inputs(w, H.DEV, seed=11, lengths=lengths, pad_rows=4)
    out, ws = fused_call(inp, ns)
    check_vs_oracle(inp, out)
    assert not arrivals(ws, w, ns).any(), "arrival counters not back at zero"


def test_fused_repeated_calls_are_bitwise_identical(kernel_path):
    w = W.llama(1, 8192)
    inp = W.make_inputs(w, H.DEV, seed=3)
    out0, ws = fused_call(inp, 32)
    for _ in range(4):
        out1, ws = fused_call(inp, 32, workspace=ws)
        assert torch.equal(out0, out1)
    assert not arrivals(ws, w, 32).any()


def test_fused_empty_splits_and_sequences():
    # ns > L for some sequences: their tail splits hold no key (LSE -inf, o 0)
    w = W.Workload("empty", 4, 8, 2, 128, "bf16", kv_len=None)
    inp = W.make_inputs(w, H.DEV, seed=5, lengths=[5, 0, 40, 1], pad_rows=4)
    out, ws = fused_call(inp, 16)
    check_vs_oracle(inp, out)
    assert not arrivals(ws, w, 16).any()


def test_fused_maximum_split_count():
    fd = H.fd()
    w = W.Workload("maxns", 1, 4, 1, 64, "f16", kv_len=None)
    inp = W.make_inputs(w, H.DEV, seed=9, lengths=[20000], pad_rows=4)
    out, ws = fused_call(inp, fd.FD_MAX_SPLITS)
    assert H.max_err(H.host(out), H.oracle_full(inp, fd.FD_MAX_SPLITS)) <= H.TOL["f16"]
    assert not arrivals(ws, w, fd.FD_MAX_SPLITS).any()


def test_fused_is_close_to_the_two_launch_call():
    fd = H.fd()
    w = W.fd_ubench(16, 4096)
    inp = W.make_inputs(w, H.DEV, seed=2)
    two = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8)
    one, _ = fused_call(inp, 8)
    # same partials, merged in another order: a few output ulps at most
    assert H.max_err(H.host(one), H.host(two)) <= 2 * 2.0 ** -10


def _bitwise(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


QUEUE_CASES = [  # (workload, lengths, ns): more segments than one device-sized grid
    (W.llama(16, 8192), None, 8),
    (W.mha(128), None, 16),
    (W.varlen_qwen(), None, 8),
    (W.fd_ubench(8, 8192), None, 64),
    (W.Workload("qsmall", 40, 16, 8, 64, "bf16", kv_len=None), [300] * 20 + [1000] * 20, 6),
]


@pytest.mark.parametrize("case", QUEUE_CASES, ids=lambda c: f"{c[0].name}-ns{c[2]}")
def test_queue_schedule_is_bitwise_equal_to_static(case, kernel_path):
    fd = H.fd()
    w, lengths, ns = case
    inp = W.make_inputs(w, H.DEV, seed=1, lengths=lengths)
    n = fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim)
    res = {}
    for sched in (fd.FD_SCHED_STATIC, fd.FD_SCHED_QUEUE):
        ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=H.DEV)  # counter garbage too
        prev = fd.fd_set_schedule(sched)
        try:
            H.announce("schedule", sched, w.name, f"ns={ns}")
            out = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                         workspace=ws, layout=w.layout)
            split_ws = fd.fd_decode_split(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                          layout=w.layout)
            torch.cuda.synchronize()
        finally:
            fd.fd_set_schedule(prev)
        _, ctl_off, _ = _layout_sizes(w, ns)
        res[sched] = (out, ws[:ctl_off].clone(), split_ws[:ctl_off].clone())
    s, q = res[fd.FD_SCHED_STATIC], res[fd.FD_SCHED_QUEUE]
    assert _bitwise(s[0], q[0]), "outputs differ"
    assert _bitwise(s[1], q[1]), "whole-call partials differ"
    assert _bitwise(s[2], q[2]), "split-launch partials differ"
    if kernel_path != "unpacked":
        assert H.max_err(H.host(q[0]), H.oracle_full(inp, ns)) <= H.TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_queue_schedule_with_empty_sequences_and_splits(dtype, kernel_path):
    """Segments of no tile (empty sequences, more splits than keys) and of
    fewer tiles than a workgroup has waves, claimed through the queue: the
    claim of the next segment is then made after the walk. Output and
    partials bitwise equal to the static schedule's."""
    fd = H.fd()
    lengths = [0, 5, 100, 0, 3000, 1, 64, 0, 17, 513, 2, 7000, 33, 0, 250, 16]
    w = W.Workload("qempty", len(lengths), 8, 2, 128, dtype, kv_len=None)
    inp = W.make_inputs(w, H.DEV, seed=6, lengths=lengths)
    ns = 16
    n = fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim)
    _, ctl_off, _ = _layout_sizes(w, ns)
    res = {}
    for sched in (fd.FD_SCHED_STATIC, fd.FD_SCHED_QUEUE):
        ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=H.DEV)
        prev = fd.fd_set_schedule(sched)
        try:
            H.announce("schedule", sched, w.name, dtype, f"ns={ns}")
            out = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                         workspace=ws, layout=w.layout)
            torch.cuda.synchronize()
        finally:
            fd.fd_set_schedule(prev)
        res[sched] = (out, ws[:ctl_off].clone())
    s, q = res[fd.FD_SCHED_STATIC], res[fd.FD_SCHED_QUEUE]
    assert _bitwise(s[0], q[0]), "outputs differ"
    assert _bitwise(s[1], q[1]), "partials differ"
    assert torch.isfinite(q[0]).all()


def test_queue_schedule_under_graph_replay():
    """The counter reset is a kernel node: every replay of a captured queued
    call starts from zero and equals the eager call."""
    fd = H.fd()
    w = W.llama(16, 1024)
    inp = W.make_inputs(w, H.DEV, seed=4)
    ns = 8
    ws = torch.zeros(fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim), dtype=torch.uint8,
                     device=H.DEV)
    prev = fd.fd_set_schedule(fd.FD_SCHED_QUEUE)
    try:
        ref = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, workspace=ws)
        out = torch.empty_like(ref)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, out=out,
                                   workspace=ws, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, out=out,
                                   workspace=ws, stream=torch.cuda.current_stream())
        for _ in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
    finally:
        fd.fd_set_schedule(prev)
