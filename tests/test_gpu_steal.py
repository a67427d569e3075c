"""GPU tests of the steal schedule (FD_SCHED_STEAL): whole calls in which
each workgroup streams one share of a (sequence, KV head) unit in chunks it
claims from the front of the share's word, and workgroups that are done take
the back half of another share's unclaimed chunks.

The runs of a call depend on timing, so results are checked against the
fp64 oracle (to the dtype tolerance), not bitwise, and the workspace is
checked for what must hold after every call whatever the timing:

  * every share with two or more chunks published its chunk count, and its
    front and back counts cover every chunk (no chunk left unclaimed);
  * at most steal_cap steals per share; the steal slots no thief took hold
    LSE -inf and a zero row, the taken ones a finite LSE;
  * shares of one chunk were never claimed (word 0).

Calls that cannot take the schedule (the unnormalised format, the VALU
kernel, the fused combine, split counts with no valid share layout) run the
static schedule and must be bitwise equal to it.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MIN_CHUNK = 512      # keys, the kernel's smallest chunk
KEY_QUANTUM = 64     # chunk keys are a multiple of this
CHUNKS = 32          # the library's target chunks per share
MAX_CAP = 15
MAX_SHARES = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    fd = H.fd()
    yield
    fd.fd_set_schedule(fd.FD_SCHED_AUTO)
    fd.fd_set_kernel_path(fd.FD_PATH_AUTO)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def shares_per_unit(units, ns, cus):
    """The host's layout rule: the largest divisor d of ns (d <= ns/2) with
    units*d <= cus and ns/d - 1 steal slots in 1..15."""
    for d in range(ns // 2, 0, -1):
        if ns % d:
            continue
        cap = ns // d - 1
        if 1 <= cap <= MAX_CAP and units * d <= cus and units * d <= MAX_SHARES:
            return d
    return 0


def share_chunks(L, r, nsh):
    """Chunk count of share r of nsh of L keys (the kernel's rule)."""
    start = L * r // nsh
    n = L * (r + 1) // nsh - start
    per = -(-n // CHUNKS)
    ck = max(MIN_CHUNK, -(-per // KEY_QUANTUM) * KEY_QUANTUM)
    return max(1, -(-n // ck))


def _offsets(w, ns):
    rows = w.batch * w.heads * ns
    lse_off = (rows * w.dim * 4 + 255) // 256 * 256
    ctl_off = lse_off + (rows * 4 + 255) // 256 * 256
    steal_off = ctl_off + 256 + (w.batch * w.heads * 4 + 255) // 256 * 256
    return lse_off, ctl_off, steal_off


def steal_call(inp, ns, workspace=None, path=None):
    fd = H.fd()
    w = inp.workload
    if workspace is None:
        n = fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim)
        workspace = torch.full((n,), 0x7f, dtype=torch.uint8, device=H.DEV)  # NaN partials
        _, ctl_off, _ = _offsets(w, ns)
        workspace[ctl_off:].zero_()
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    prev_path = fd.fd_set_kernel_path(path) if path is not None else None
    try:
        H.announce("steal", w.name, f"ns={ns}", f"lens[:4]={inp.lengths[:4]}")
        out = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                     workspace=workspace, layout=w.layout)
        torch.cuda.synchronize()
    finally:
        fd.fd_set_schedule(prev)
        if prev_path is not None:
            fd.fd_set_kernel_path(prev_path)
    return out, workspace


def check_vs_oracle(inp, out):
    w = inp.workload
    o = H.host(out)
    G = w.group
    for b, L in enumerate(inp.lengths):
        if L == 0:
            assert not o[b].any(), b
    live = [(b, j) for b, L in enumerate(inp.lengths) if L > 0 for j in range(w.kv_heads)]
    ref = H.oracle_pairs(inp, live, workers=8)
    err = max(H.max_err(o[b, j * G:(j + 1) * G], ref[(b, j)]) for b, j in live)
    assert err <= H.TOL[w.dtype], err
    return err


def check_workspace(inp, ns, ws):
    """Share words and steal slots after a steal-scheduled call; returns
    the total number of steals."""
    w = inp.workload
    rows_per_pass = 8
    chunks = -(-w.group // rows_per_pass)
    units = w.batch * w.kv_heads * chunks
    nsh = shares_per_unit(units, ns, _cus())
    assert nsh > 0
    cap = ns // nsh - 1
    lse_off, _, steal_off = _offsets(w, ns)
    words = ws[steal_off:steal_off + 8 * units * nsh].view(torch.int64).cpu().numpy()
    words = words.astype(np.uint64)
    rows = w.batch * w.heads * ns
    opart = ws[:rows * w.dim * 4].view(torch.float32).view(w.batch, w.heads, ns, w.dim)
    opart = opart.cpu().numpy()
    lse = ws[lse_off:lse_off + rows * 4].view(torch.float32).view(w.batch, ns, w.heads)
    lse = lse.cpu().numpy()
    field = np.uint64((1 << 20) - 1)
    total = 0
    for q in range(units * nsh):
        unit, r = divmod(q, nsh)
        b = unit // (w.kv_heads * chunks)
        hc = unit % (w.kv_heads * chunks)
        # the kernel ranks sequences longest first for batches up to 64
        order = sorted(range(w.batch), key=lambda i: (-inp.lengths[i], i))
        seq = order[b] if w.batch <= 64 else b
        kvh, ch = divmod(hc, chunks)
        h0 = kvh * w.group + ch * rows_per_pass
        h1 = min(h0 + rows_per_pass, (kvh + 1) * w.group)
        L = inp.lengths[seq]
        nc = share_chunks(L, r, nsh)
        word = words[q]
        front = int(word & field)
        back = int((word >> np.uint64(20)) & field)
        steals = int((word >> np.uint64(40)) & np.uint64(15))
        count = int(word >> np.uint64(44))
        if nc == 1:
            assert word == 0, (q, hex(int(word)))
        else:
            assert count == nc, (q, count, nc)
            assert front + 1 + back >= nc, (q, front, back, nc)
            assert steals <= cap, (q, steals, cap)
        total += steals
        base = r * (1 + cap)
        for s in range(1, cap + 1):
            lrow = lse[seq, base + s, h0:h1]
            if s <= steals:
                assert np.isfinite(lrow).all(), (q, s, lrow)
            else:
                assert np.isneginf(lrow).all(), (q, s, lrow)
                assert not opart[seq, h0:h1, base + s].any(), (q, s)
    return total


CASES = [  # (name, workload, lengths or None, num_splits)
    ("llama_b16_l8192_ns8", W.llama(16, 8192), None, 8),
    ("llama_b1_l65536_ns128", W.llama(1, 65536), None, 128),
    ("llama_b16_l1024_ns4_one_chunk", W.llama(16, 1024), None, 4),
    ("varlen_g7_ns8", W.Workload("v7", 6, 28, 4, 128, "f16", kv_len=None),
     [30000, 65, 1, 0, 20000, 7000], 8),
    ("g16_ns16", W.Workload("g16", 2, 32, 2, 128, "bf16", kv_len=None), [9000, 4000], 16),
    ("f32_g3_ns6", W.Workload("f32g3", 3, 6, 2, 128, "f32", kv_len=None), [10000, 17, 5000], 6),
    ("prime_ns7", W.Workload("p7", 2, 8, 2, 128, "f16", kv_len=None), [12000, 3001], 7),
    ("bhsd", W.Workload("bhsd", 3, 16, 4, 128, "bf16", kv_len=None, layout="bhsd"),
     [7000, 2500, 9000], 8),
    # 32 units, 128 slots: 8 shares per unit with the largest steal count, 15
    ("cap15", W.llama(4, 40000), None, 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_steal_matches_oracle(case):
    name, w, lengths, ns = case
    inp = W.make_inputs(w, H.DEV, seed=21, lengths=lengths, pad_rows=4)
    out, ws = steal_call(inp, ns)
    check_vs_oracle(inp, out)
    check_workspace(inp, ns, ws)


def _random_case(i):
    """A seeded draw that takes the steal schedule: head dim 128, group
    2..16, ragged lengths up to 40,000 keys (empty ones included), a split
    count with a valid share layout, any dtype and K/V layout."""
    rng = np.random.default_rng(7100 + i)
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    group = int(rng.choice([2, 3, 4, 5, 7, 8, 9, 12, 16]))
    kv_heads = int(rng.integers(1, 9))
    batch = int(rng.integers(1, 9))
    lengths = [0 if rng.random() < 0.1 else int(rng.integers(1, 40001)) for _ in range(batch)]
    if max(lengths) == 0:
        lengths[0] = 20000
    layout = str(rng.choice(["packed", "bhsd"]))
    units = batch * kv_heads * -(-group // 8)
    choices = [ns for ns in range(2, 65) if shares_per_unit(units, ns, _cus()) > 0]
    ns = int(rng.choice(choices))
    w = W.Workload(f"steal_r{i}", batch, group * kv_heads, kv_heads, 128, dtype, kv_len=None,
                   layout=layout)
    return w, lengths, ns


@pytest.mark.parametrize("i", range(24))
def test_steal_random_draws(i):
    w, lengths, ns = _random_case(i)
    inp = W.make_inputs(w, H.DEV, seed=100 + i, lengths=lengths, pad_rows=4)
    out, ws = steal_call(inp, ns)
    check_vs_oracle(inp, out)
    check_workspace(inp, ns, ws)


def test_steal_takes_work_from_long_shares():
    """One long sequence among short ones: the short shares end at once and
    their workgroups take chunks of the long shares."""
    w = W.Workload("skew", 16, 32, 8, 128, "bf16", kv_len=None)
    lengths = [131072] + [64] * 15
    inp = W.make_inputs(w, H.DEV, seed=5, lengths=lengths)
    out, ws = steal_call(inp, 8)
    check_vs_oracle(inp, out)
    steals = check_workspace(inp, 8, ws)
    H.announce("steals", steals)
    assert steals > 0


def test_steal_repeated_calls_and_graph_replay():
    """The share words are zeroed by a kernel before each launch: repeated
    calls and graph replays all give correct results."""
    fd = H.fd()
    w = W.llama(4, 16384)
    inp = W.make_inputs(w, H.DEV, seed=8)
    ns = 8
    out0, ws = steal_call(inp, ns)
    err0 = check_vs_oracle(inp, out0)
    for _ in range(3):
        out1, ws = steal_call(inp, ns, workspace=ws)
        assert H.max_err(H.host(out1), H.host(out0)) <= 2 * H.TOL[w.dtype]
        check_workspace(inp, ns, ws)
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    try:
        out = torch.empty_like(out0)
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
            assert torch.isfinite(out.float()).all()
            assert H.max_err(H.host(out), H.host(out0)) <= 2 * H.TOL[w.dtype]
            check_workspace(inp, ns, ws)
    finally:
        fd.fd_set_schedule(prev)
    assert err0 <= H.TOL[w.dtype]


def _bitwise(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _static_and_steal(fn):
    fd = H.fd()
    res = []
    for sched in (fd.FD_SCHED_STATIC, fd.FD_SCHED_STEAL):
        prev = fd.fd_set_schedule(sched)
        try:
            res.append(fn())
            torch.cuda.synchronize()
        finally:
            fd.fd_set_schedule(prev)
    return res


def test_split_launch_leaves_the_steal_slots():
    """fd_decode_split under the steal setting leaves the steal layout's
    partials; fd_decode_combine merges them into the oracle's output."""
    fd = H.fd()
    w = W.llama(16, 4096)
    inp = W.make_inputs(w, H.DEV, seed=3)
    ns = 8
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    try:
        H.announce("steal split", w.name, f"ns={ns}")
        ws = fd.fd_decode_split(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns)
        out = torch.empty_like(inp.q)
        fd.fd_decode_combine(ws, w.batch, w.heads, w.dim, ns, out)
        torch.cuda.synchronize()
    finally:
        fd.fd_set_schedule(prev)
    check_workspace(inp, ns, ws)
    check_vs_oracle(inp, out)


@pytest.mark.parametrize("kind", ["valu_path", "unnorm", "no_layout", "fused"])
def test_calls_outside_the_schedule_run_static(kind):
    fd = H.fd()
    w = W.llama(16, 4096)
    inp = W.make_inputs(w, H.DEV, seed=4)
    if kind == "valu_path":
        prev = fd.fd_set_kernel_path(fd.FD_PATH_VALU)
        try:
            a, b = _static_and_steal(lambda: fd.fd_decode_attention(
                inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8))
        finally:
            fd.fd_set_kernel_path(prev)
    elif kind == "unnorm":
        a, b = _static_and_steal(lambda: fd.fd_decode_attention_unnorm(
            inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8))
    elif kind == "no_layout":
        # 128 units and 64 splits: every share layout has more than 15 steal slots
        a, b = _static_and_steal(lambda: fd.fd_decode_attention(
            inp.q, inp.k, inp.v, inp.cu_seqlens_k, 64))
    else:
        prev = fd.fd_set_combine(fd.FD_COMBINE_FUSED)
        try:
            a, b = _static_and_steal(lambda: fd.fd_decode_attention(
                inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8))
        finally:
            fd.fd_set_combine(prev)
    assert _bitwise(a, b)


def test_share_layout_rule():
    """The cases above take the schedule on this device (MI355X: 256 CUs)."""
    cus = _cus()
    assert shares_per_unit(128, 64, cus) == 0
    for name, w, _, ns in CASES:
        units = w.batch * w.kv_heads * -(-w.group // 8)
        assert shares_per_unit(units, ns, cus) > 0, name
    if cus == 256:
        assert shares_per_unit(128, 8, cus) == 2
        assert shares_per_unit(8, 128, cus) == 32
        assert shares_per_unit(32, 128, cus) == 8     # 15 steal slots per share


def test_schedule_is_per_thread():
    """Two threads calling at the same time, one under the static schedule
    and one under the steal schedule, each with its own stream and
    workspace: the static thread's outputs equal a static call bitwise and
    its share words stay zero; the steal thread's words show its shares'
    published chunk counts and its outputs match the oracle."""
    import threading
    fd = H.fd()
    w = W.Workload("thr", 3, 32, 4, 128, "bf16", kv_len=None)
    inp = W.make_inputs(w, H.DEV, seed=33, lengths=[5000, 3000, 4100])
    ns = 8
    n = fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim)
    prev = fd.fd_set_schedule(fd.FD_SCHED_STATIC)
    ref = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns)
    fd.fd_set_schedule(prev)
    torch.cuda.synchronize()
    got, errors = {}, []
    gate = threading.Barrier(2)

    def worker(name, sched):
        try:
            fd.fd_set_schedule(sched)
            s = torch.cuda.Stream()
            ws = torch.zeros(n, dtype=torch.uint8, device=H.DEV)
            outs = []
            gate.wait()
            for _ in range(10):
                outs.append(fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                                   workspace=ws, stream=s))
            s.synchronize()
            got[name] = (outs, ws)
        except Exception as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=worker, args=("static", fd.FD_SCHED_STATIC)),
          threading.Thread(target=worker, args=("steal", fd.FD_SCHED_STEAL))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    _, _, steal_off = _offsets(w, ns)
    outs, ws = got["static"]
    assert all(torch.equal(o, ref) for o in outs)
    assert not ws[steal_off:].any()
    outs, ws = got["steal"]
    check_workspace(inp, ns, ws)
    assert ws[steal_off:].any()
    for o in outs:
        check_vs_oracle(inp, o)


def test_noalloc_entry_point_under_the_steal_schedule():
    """fd_decode_attention_noalloc runs the steal schedule on the static
    scratch's control block: two calls in a row (the second smaller) match
    the oracle."""
    fd = H.fd()
    prev = fd.fd_set_schedule(fd.FD_SCHED_STEAL)
    try:
        for lengths, seed in (([20000, 9000, 15000], 51), ([6000, 3000], 52)):
            w = W.Workload("noalloc_steal", len(lengths), 16, 4, 128, "f16", kv_len=None)
            inp = W.make_inputs(w, H.DEV, seed=seed, lengths=lengths)
            out = torch.empty_like(inp.q)
            H.announce("noalloc steal", lengths)
            fd.fd_decode_attention_noalloc(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8, out)
            torch.cuda.synchronize()
            check_vs_oracle(inp, out)
    finally:
        fd.fd_set_schedule(prev)


def test_garbage_in_the_control_block():
    """The reset kernel zeroes the share words before each steal launch:
    a workspace whose partials, arrival counters and share words all hold
    0x7f bytes gives the oracle's output and clean word invariants."""
    fd = H.fd()
    w = W.llama(16, 8192)
    inp = W.make_inputs(w, H.DEV, seed=12)
    ns = 8
    ws = torch.full((fd.fd_workspace_bytes(w.batch, w.heads, ns, w.dim),), 0x7f,
                    dtype=torch.uint8, device=H.DEV)
    out, ws = steal_call(inp, ns, workspace=ws)
    check_vs_oracle(inp, out)
    check_workspace(inp, ns, ws)
