"""GPU tests with exact answers: split boundaries and varlen indexing made
bit-exactly observable, edge cases, and a grid of head dims x dtypes x group
sizes with ragged tiles against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    H.fd().fd_set_kernel_path(H.fd().FD_PATH_AUTO)


@pytest.fixture(params=["valu", "mfma", "unpacked"])
def kernel_path(request):
    """Run the test on each split kernel (MFMA falls back to VALU where the
    matrix-core kernel does not exist; "unpacked" is the VALU kernel with one
    query head per workgroup)."""
    fd = H.fd()
    prev = fd.fd_set_kernel_path({"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA,
                                  "unpacked": fd.FD_PATH_UNPACKED}[request.param])
    H.announce("kernel path", request.param)
    yield request.param
    fd.fd_set_kernel_path(prev)


def _bounds(L, ns):
    """Proportional bounds, including the empty splits that ns > L gives
    (the oracle raises there; the library documents LSE=-inf, o=0)."""
    if L >= ns >= 1:
        return oracle.split_bounds(L, ns)
    return [(L * s // ns, L * (s + 1) // ns) for s in range(ns)]


def structured_inputs(lengths, heads, kv_heads, dim, dtype, ns, layout, pad=3):
    """K = 0 so every score is 0 and every key weighs exactly 1. V carries
    integers: channel 0 is 1 at each split's first key, channel 1 is 1 at its
    last key, channel 2 is the sequence index, channel 3 the KV head index,
    channel 4 the key position mod 16. Rows outside every sequence are NaN."""
    B = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((B, heads, dim)).astype(np.float32)).to(DT[dtype])
    if layout == "packed":
        k = torch.full((T + pad, kv_heads, dim), float("nan"))
        v = torch.full((T + pad, kv_heads, dim), float("nan"))
        k[:T] = 0
        v[:T] = 0
    else:
        S = max(lengths)
        k = torch.full((B, kv_heads, S + pad, dim), float("nan"))
        v = torch.full((B, kv_heads, S + pad, dim), float("nan"))
    for b, L in enumerate(lengths):
        for j in range(kv_heads):
            if layout == "packed":
                rows = v[int(cu[b]):int(cu[b]) + L, j]
            else:
                k[b, j, :L] = 0
                v[b, j, :L] = 0
                rows = v[b, j, :L]
            rows[:, 2] = b
            rows[:, 3] = j
            rows[:, 4] = torch.arange(L) % 16
            for a, e in _bounds(L, ns):
                if e > a:
                    rows[a, 0] = 1
                    rows[e - 1, 1] = 1
    w = W.Workload("structured", B, heads, kv_heads, dim, dtype, kv_len=None, layout=layout,
                   num_splits=ns)
    cu_t = torch.tensor(cu, dtype=torch.int32)
    return W.Inputs(w, q.to(H.DEV), k.to(DT[dtype]).to(H.DEV), v.to(DT[dtype]).to(H.DEV),
                    cu_t.to(H.DEV), list(lengths))


CASES = [
    # lengths, heads, kv_heads, dim, dtype, ns, layout
    ([10000], 8, 1, 128, "f32", 7, "packed"),
    ([10000], 8, 1, 128, "f32", 1000, "packed"),
    ([1, 2, 3, 17, 64, 65, 300], 28, 4, 128, "f16", 1, "packed"),
    ([8, 9, 31, 257, 1000, 4097], 28, 4, 128, "f16", 8, "packed"),
    ([256, 300, 511], 16, 2, 64, "bf16", 16, "bhsd"),
    ([4096] * 2, 4, 4, 16, "f16", 16, "bhsd"),
    ([129, 4, 77], 32, 8, 32, "bf16", 4, "packed"),
    ([5, 33, 1], 6, 2, 16, "f32", 1, "bhsd"),
    ([100, 37, 64], 32, 2, 128, "f16", 37, "packed"),   # group 16: two row chunks
    ([3, 10, 5], 8, 1, 64, "f16", 7, "packed"),         # ns > some lengths: empty splits
    ([0, 12, 40], 8, 2, 128, "bf16", 4, "packed"),      # an empty sequence
    ([1, 15, 16, 17, 33, 4099], 16, 2, 128, "bf16", 3, "packed"),
    ([2000, 7, 64], 24, 4, 128, "f16", 5, "bhsd"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-d{c[3]}-g{c[1]//c[2]}-ns{c[5]}-{c[6]}")
def test_split_bounds_and_varlen_indexing_are_exact(case, kernel_path):
    lengths, heads, kv_heads, dim, dtype, ns, layout = case
    inp = structured_inputs(lengths, heads, kv_heads, dim, dtype, ns, layout)
    G = heads // kv_heads
    ws, opart, lse2 = H.gpu_split(inp, ns, scale=0.37)
    for b, L in enumerate(lengths):
        for h in range(heads):
            j = h // G
            for s, (a, e) in enumerate(_bounds(L, ns)):
                n = e - a
                o = opart[b, h, s]
                if n == 0:
                    assert lse2[b, s, h] == -np.inf and not o.any(), (b, h, s)
                    continue
                assert round(2.0 ** float(lse2[b, s, h])) == n, (b, h, s, lse2[b, s, h], n)
                assert round(float(o[0]) * n) == 1 and round(float(o[1]) * n) == 1, (b, h, s)
                # sequence and KV-head indices come back as exact integers
                assert round(float(o[2])) == b and round(float(o[3])) == j, (b, h, s, o[2], o[3])
                assert abs(float(o[2]) - b) <= 1e-6 * max(1, b) and abs(float(o[3]) - j) <= 1e-6 * max(1, j)
                assert round(float(o[4]) * n) == sum(t % 16 for t in range(a, e)), (b, h, s)
    out = H.host(H.gpu_attention(inp, ns, scale=0.37))
    for b, L in enumerate(lengths):
        for h in range(heads):
            if L == 0:
                assert not out[b, h].any()
                continue
            assert round(float(out[b, h, 2])) == b and round(float(out[b, h, 3])) == h // G
            n_nonempty = sum(1 for a, e in _bounds(L, ns) if e > a)
            assert abs(float(out[b, h, 0]) - n_nonempty / L) <= 1e-2 * max(1.0, n_nonempty / L)


# ------------------------------------------------------------ edge cases --
def _rand_inputs(lengths, heads, kv_heads, dim, dtype, layout="packed", seed=0, pad=0):
    w = W.Workload("edge", len(lengths), heads, kv_heads, dim, dtype, kv_len=None, layout=layout)
    return W.make_inputs(w, H.DEV, seed=seed, lengths=lengths, pad_rows=pad)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_key_returns_its_value_exactly(dtype, kernel_path):
    inp = _rand_inputs([1, 1, 1], 8, 2, 128, dtype)
    out = H.gpu_attention(inp, 1)
    G = 4
    for b in range(3):
        for h in range(8):
            assert torch.equal(out[b, h], inp.v[b, h // G]), (b, h)


def test_empty_sequence_gives_zero_rows():
    inp = _rand_inputs([0, 50, 0], 8, 2, 64, "f16", pad=4)
    for ns in (1, 3):
        out = H.host(H.gpu_attention(inp, ns))
        assert not out[0].any() and not out[2].any()
        ref = oracle.attention_rows(H.host(inp.q[1, 0:4]), H.host(inp.k[0:50, 0]),
                                    H.host(inp.v[0:50, 0]), 1.0 / math.sqrt(64))
        assert H.max_err(out[1, 0:4], ref) <= H.TOL["f16"]


@pytest.mark.parametrize("layout", ["packed", "bhsd"])
def test_nan_outside_sequences_is_never_read(layout, kernel_path):
    inp = _rand_inputs([1, 77, 200, 5], 16, 2, 128, "f16", layout=layout, pad=64)
    for ns in (1, 5):
        out = H.host(H.gpu_attention(inp, ns))
        assert np.isfinite(out).all()
        ref = H.oracle_full(inp, None)
        assert H.max_err(out, ref) <= H.TOL["f16"]


def test_bshd_layout_matches_bhsd_bitwise(kernel_path):
    """[batch, max_len, kv_heads, dim] K/V (kv_layout "bshd") reads the same
    values in the same order as [batch, kv_heads, max_len, dim], so the
    outputs are bitwise equal; the latter is checked against the oracle."""
    inp = _rand_inputs([300, 77, 1000], 16, 2, 128, "f16", layout="bhsd", seed=9)
    k_s = inp.k.transpose(1, 2).contiguous()
    v_s = inp.v.transpose(1, 2).contiguous()
    fdm = H.fd()
    for ns in (1, 4):
        a = fdm.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, layout="bhsd")
        b = fdm.fd_decode_attention(inp.q, k_s, v_s, inp.cu_seqlens_k, ns, layout="bshd")
        torch.cuda.synchronize()
        assert torch.equal(a, b), ns
        assert H.max_err(H.host(a), H.oracle_full(inp, ns)) <= H.TOL["f16"]


def test_planned_split_count_when_none_is_given():
    """num_splits=None plans on the device lengths (empty sequences left
    out) and gives the same output as passing that count explicitly."""
    fdm = H.fd()
    inp = _rand_inputs([5000, 0, 1200, 64], 32, 8, 128, "bf16", seed=13)
    live = [L for L in inp.lengths if L > 0]
    ns = fdm.fd_plan_splits(len(live), 32, 8, 128, fdm.FD_BF16, live)
    a = fdm.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, None)
    b = fdm.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    u = fdm.fd_decode_attention_unnorm(inp.q, inp.k, inp.v, inp.cu_seqlens_k, None)
    torch.cuda.synchronize()
    assert H.max_err(H.host(u), H.host(b)) <= H.TOL["bf16"]
    assert not H.host(a)[1].any()


def test_offsets_need_not_start_at_zero(kernel_path):
    """cu_seqlens_k is any non-decreasing offset array: here it starts at 37
    and holds an empty sequence, and every K/V row outside the sequences is
    NaN, so a read of one would show in the output."""
    lengths = [300, 0, 1000, 17]
    base = _rand_inputs(lengths, 16, 2, 128, "f16", seed=5)
    off, pad, T = 37, 16, sum(lengths)
    k = torch.full((off + T + pad, 2, 128), float("nan"), dtype=base.k.dtype, device=H.DEV)
    v = torch.full_like(k, float("nan"))
    k[off:off + T] = base.k[:T]
    v[off:off + T] = base.v[:T]
    cu = (base.cu_seqlens_k + off).contiguous()
    inp = W.Inputs(base.workload, base.q, k, v, cu, lengths)
    cu_h = cu.cpu().tolist()
    assert cu_h[0] == off
    for ns in (1, 3):
        out = H.host(H.gpu_attention(inp, ns))
        assert np.isfinite(out).all()
        assert not out[1].any()
        for b in (0, 2, 3):
            for j in range(2):
                ref = oracle.attention_rows(H.host(base.q[b, 8 * j:8 * (j + 1)]),
                                            H.host(k[cu_h[b]:cu_h[b + 1], j]),
                                            H.host(v[cu_h[b]:cu_h[b + 1], j]), 1.0 / math.sqrt(128))
                err = H.max_err(out[b, 8 * j:8 * (j + 1)], ref)
                assert err <= H.TOL["f16"], (ns, b, j, err)


@pytest.mark.parametrize("group,kv_heads", [(16, 2), (64, 1), (9, 3), (12, 1)])
@pytest.mark.parametrize("dim", [64, 128])
def test_groups_larger_than_one_pass(group, kv_heads, dim, kernel_path):
    inp = _rand_inputs([300, 1025], group * kv_heads, kv_heads, dim, "bf16")
    for ns in (1, 4):
        out = H.host(H.gpu_attention(inp, ns))
        assert H.max_err(out, H.oracle_full(inp, ns)) <= H.TOL["bf16"]


@pytest.mark.parametrize("scale", [-0.3, 2.0, 1e-3])
def test_non_default_scales(scale):
    """fp32 at scales away from 1/sqrt(dim) (negative, 23x and 0.01x of it).
    At 23x the scores reach |s| ~ 60 and their own fp32 forward error moves
    the output by about the fp32 tolerance whatever the kernel (the VALU
    kernel reaches 0.97 of 1e-5 over 12 seeds, the matrix-core kernel 1.08):
    every element is held to the tolerance plus that named bound
    (H.scaled_bound), as in the random sweep's non-default scales."""
    for lens, ns in (([700, 64, 1], 1), ([700, 64, 3], 3)):
        inp = _rand_inputs(lens, 8, 1, 128, "f32")
        out = H.host(H.gpu_attention(inp, ns, scale=scale))
        q, k, v = H.host(inp.q), H.host(inp.k), H.host(inp.v)
        cu = inp.cu_seqlens_k.cpu().tolist()
        for b in range(len(lens)):
            kr = oracle.kv_rows(k, cu, b, 0, "packed")
            vr = oracle.kv_rows(v, cu, b, 0, "packed")
            qr = q[b].astype(np.float64)
            ref = oracle.attention_rows(qr, kr, vr, scale)
            bound = H.scaled_bound(qr, kr, vr, scale, "f32", ref)
            assert (np.abs(out[b] - ref) - bound).max() <= 0.0, (lens, b, H.max_err(out[b], ref))


def test_repeat_calls_are_bitwise_identical(kernel_path):
    inp = _rand_inputs([5000, 3000], 28, 4, 128, "f16")
    a = H.gpu_attention(inp, 8).clone()
    b = H.gpu_attention(inp, 8).clone()
    assert torch.equal(a, b)
    ws1, o1, l1 = H.gpu_split(inp, 8)
    ws2, o2, l2 = H.gpu_split(inp, 8)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_runs_on_a_side_stream():
    inp = _rand_inputs([3000, 17], 16, 2, 128, "bf16")
    ref = H.gpu_attention(inp, 4).clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = H.fd().fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 4, layout="packed",
                                         stream=s)
    s.synchronize()
    assert torch.equal(out, ref)


def test_concurrent_calls_on_two_streams():
    """The library keeps no per-call state: calls issued alternately on two
    streams (each with its own workspace and output, different inputs and
    kernel configurations, running concurrently) give exactly what each
    call gives alone."""
    fdm = H.fd()
    a = _rand_inputs([3000, 17, 800], 28, 4, 128, "f16", seed=21)      # matrix-core kernel
    b = _rand_inputs([4096, 4096], 8, 8, 64, "bf16", layout="bhsd", seed=22)  # VALU kernel
    ref_a = H.gpu_attention(a, 8).clone()
    ref_b = H.gpu_attention(b, 16).clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = torch.empty(fdm.fd_workspace_bytes(3, 28, 8, 128), dtype=torch.uint8, device=H.DEV)
    ws2 = torch.empty(fdm.fd_workspace_bytes(2, 8, 16, 64), dtype=torch.uint8, device=H.DEV)
    outs_a = [torch.empty_like(a.q) for _ in range(6)]
    outs_b = [torch.empty_like(b.q) for _ in range(6)]
    torch.cuda.synchronize()
    for i in range(6):
        fdm.fd_decode_attention(a.q, a.k, a.v, a.cu_seqlens_k, 8, out=outs_a[i], workspace=ws1,
                                stream=s1)
        fdm.fd_decode_attention(b.q, b.k, b.v, b.cu_seqlens_k, 16, out=outs_b[i], workspace=ws2,
                                layout="bhsd", stream=s2)
    torch.cuda.synchronize()
    for i in range(6):
        assert torch.equal(outs_a[i], ref_a), i
        assert torch.equal(outs_b[i], ref_b), i


def test_default_buffers_belong_to_the_call_stream():
    """With stream=s given outside any stream context and no workspace or
    out, the binding's own buffers are allocated on s. Memory that torch
    then hands out on the default stream while s still runs cannot be the
    workspace: scribbling over such blocks leaves the result exact."""
    fdm = H.fd()
    inp = _rand_inputs([16384] * 8, 32, 8, 128, "bf16", seed=31)
    ns = 16
    ref = H.gpu_attention(inp, ns).clone()
    need = fdm.fd_workspace_bytes(8, 32, ns, 128)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(fdm.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, stream=s))
        # the call's temporaries are freed on return; grab blocks of the same
        # size on the default stream and overwrite them at once
        junk = [torch.empty(need, dtype=torch.uint8, device=H.DEV) for _ in range(4)]
        for j in junk:
            j.fill_(0xFF)
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_kernel_path_per_thread_calls():
    """Two threads, each with its own kernel path and stream, calling at the
    same time: each gets its own path's result, bitwise (the VALU and the
    matrix-core kernels round differently, so a crossed setting shows)."""
    import threading
    fdm = H.fd()
    inp = _rand_inputs([5000, 3000, 4100], 32, 4, 128, "bf16", seed=33)
    refs = {}
    for name, path in (("valu", fdm.FD_PATH_VALU), ("mfma", fdm.FD_PATH_MFMA)):
        prev = fdm.fd_set_kernel_path(path)
        refs[name] = H.gpu_attention(inp, 8).clone()
        fdm.fd_set_kernel_path(prev)
    assert not torch.equal(refs["valu"], refs["mfma"])
    got, errors = {}, []
    gate = threading.Barrier(2)

    def worker(name, path):
        try:
            fdm.fd_set_kernel_path(path)
            s = torch.cuda.Stream()
            outs = []
            gate.wait()
            for _ in range(20):
                outs.append(fdm.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8,
                                                    stream=s))
            s.synchronize()
            got[name] = outs
        except Exception as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=worker, args=("valu", fdm.FD_PATH_VALU)),
          threading.Thread(target=worker, args=("mfma", fdm.FD_PATH_MFMA))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for name in ("valu", "mfma"):
        assert len(got[name]) == 20
        for o in got[name]:
            assert torch.equal(o, refs[name]), name


@pytest.mark.parametrize("batch", [64, 65, 130])
@pytest.mark.parametrize("dtype,dim,heads,kvh", [("bf16", 128, 16, 4), ("f16", 64, 8, 8)])
def test_large_varlen_batches(batch, dtype, dim, heads, kvh, kernel_path):
    """Unequal lengths (empty sequences included) at and past the batch size
    up to which workgroups take sequences longest first (64): above it each
    workgroup reads its sequence's offsets itself."""
    rng = np.random.default_rng(batch + dim)
    lengths = [int(x) for x in rng.integers(0, 600, size=batch)]
    lengths[batch // 2] = 0
    inp = _rand_inputs(lengths, heads, kvh, dim, dtype, seed=batch, pad=8)
    q, k, v = H.host(inp.q), H.host(inp.k), H.host(inp.v)
    cu = inp.cu_seqlens_k.cpu().tolist()
    G = heads // kvh
    for ns in (1, 3):
        out = H.host(H.gpu_attention(inp, ns))
        assert np.isfinite(out).all()
        for b, L in enumerate(lengths):
            for j in range(kvh):
                rows = out[b, j * G:(j + 1) * G]
                if L == 0:
                    assert not rows.any(), (ns, b, j)
                    continue
                ref = oracle.attention_rows(q[b, j * G:(j + 1) * G], k[cu[b]:cu[b + 1], j],
                                            v[cu[b]:cu[b + 1], j], 1.0 / math.sqrt(dim))
                assert H.max_err(rows, ref) <= H.TOL[dtype], (ns, b, j, L)


def test_split_then_combine_equals_the_whole_call():
    inp = _rand_inputs([4000, 900], 32, 8, 128, "bf16")
    fd = H.fd()
    whole = H.gpu_attention(inp, 6)
    ws = fd.fd_decode_split(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 6)
    out = torch.empty_like(inp.q)
    fd.fd_decode_combine(ws, 2, 32, 128, 6, out)
    torch.cuda.synchronize()
    assert torch.equal(out, whole)


def test_bad_arguments_raise_without_launching():
    inp = _rand_inputs([10], 8, 2, 128, "f16")
    fd = H.fd()
    with pytest.raises(fd.FdError):
        fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 0)
    with pytest.raises(fd.FdError):
        fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 2, scale=float("nan"))


# ---------------------------------------------------------- generic grid --
GRID_LENS = [1, 37, 64, 65, 300, 1029]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("dim", [16, 32, 64, 128])
@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6, 7, 8])
def test_grid_dims_dtypes_groups(dtype, dim, group, kernel_path):
    """Ragged lengths spanning one to many tiles, two KV heads, ns=1 and a
    split count that cuts tiles mid-way."""
    inp = _rand_inputs(GRID_LENS, 2 * group, 2, dim, dtype, seed=group * 7 + dim)
    ref = H.oracle_full(inp, None)
    for ns in (1, 3):
        out = H.host(H.gpu_attention(inp, ns))
        err = H.max_err(out, ref)
        assert err <= H.TOL[dtype], (dtype, dim, group, ns, err)


@pytest.mark.parametrize("lens,heads,kvh,dim,dt,ns", [
    ([4096] * 4, 32, 32, 128, "f16", 16),           # MHA, 2048 workgroups
    ([65536], 16, 2, 128, "f16", 128),              # 256 workgroups on 2 groups
    ([777, 30000, 64, 5000], 28, 4, 128, "bf16", 8),
    ([3000, 100], 8, 1, 64, "f32", 37),
])
def test_whole_call_matches_split_then_combine_over_many_calls(lens, heads, kvh, dim, dt, ns,
                                                              kernel_path):
    """Fifty whole calls on one workspace are bitwise equal to the split and
    combine launches made separately."""
    fd = H.fd()
    inp = _rand_inputs(lens, heads, kvh, dim, dt)
    ws2 = fd.fd_decode_split(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns)
    ref = torch.empty_like(inp.q)
    fd.fd_decode_combine(ws2, len(lens), heads, dim, ns, ref)
    ws = torch.empty(fd.fd_workspace_bytes(len(lens), heads, ns, dim), dtype=torch.uint8,
                     device=H.DEV)
    outs = [fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, workspace=ws)
            for _ in range(50)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


@pytest.mark.parametrize("lens", [[16384], [20000, 16390]])
def test_maximum_split_count(lens):
    """FD_MAX_SPLITS splits: one key per split at L = 16384, ragged sizes
    above it; the combine walks 16384 partial rows per head."""
    fd = H.fd()
    ns = fd.FD_MAX_SPLITS
    inp = _rand_inputs(lens, 8, 1, 128, "f16", seed=21)
    out = H.host(H.gpu_attention(inp, ns))
    assert H.max_err(out, H.oracle_full(inp, None)) <= H.TOL["f16"]
    ws, opart, lse2 = H.gpu_split(inp, ns)
    q, k, v = H.host(inp.q), H.host(inp.k), H.host(inp.v)
    op_ref, lse_ref = oracle.attention_partials(q, k, v, inp.cu_seqlens_k.cpu().tolist(), 8, 1,
                                                ns, inp.workload.sm_scale)
    assert H.max_err(opart, op_ref) <= H.TOL["f16"]
    assert H.max_err(lse2, lse_ref * H.LOG2E) <= 1e-4
