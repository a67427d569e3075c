"""GPU parity of the second workspace format (flash_decode_splitk.py,
MiniInfer): ceil-equal split bounds and unnormalised per-split state
(m_s, l_s, acc_s), merged by rescaling to the largest m_s.

Bounds and varlen indexing are checked bit-exactly on structured inputs (all
scores 0, so m_s = 0, l_s = key count and acc_s = sums of integers, exact in
fp32). On random inputs the state is compared with the fp64 oracle through
the quantities it defines: m_s and m_s + log2 l_s (the split's base-2 LSE)
within 1e-4 -- the fp32 rounding of base-2 scores of magnitude <= ~10 summed
over <= 128 products -- and acc_s / l_s and the merged output within the
dtype tolerances (fp32 1e-5, fp16 2e-3, bf16 1e-2)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
LOG_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    H.fd().fd_set_kernel_path(H.fd().FD_PATH_AUTO)
    torch.cuda.empty_cache()


@pytest.fixture(params=["valu", "mfma", "unpacked"])
def kernel_path(request):
    fd = H.fd()
    prev = fd.fd_set_kernel_path({"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA,
                                  "unpacked": fd.FD_PATH_UNPACKED}[request.param])
    H.announce("kernel path", request.param)
    yield request.param
    fd.fd_set_kernel_path(prev)


def gpu_states(inp, ns, scale=None):
    w = inp.workload
    fd = H.fd()
    H.announce("fd_decode_split_unnorm", w.name, f"ns={ns}", f"lens[:4]={inp.lengths[:4]}")
    ws = fd.fd_decode_split_unnorm(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                   scale=w.sm_scale if scale is None else scale, layout=w.layout)
    torch.cuda.synchronize()
    acc, m, l = fd.workspace_views_unnorm(ws, w.batch, w.heads, w.dim, ns)
    return ws, H.host(acc), H.host(m), H.host(l)


def gpu_attention_unnorm(inp, ns, scale=None):
    w = inp.workload
    H.announce("fd_decode_attention_unnorm", w.name, f"ns={ns}")
    out = H.fd().fd_decode_attention_unnorm(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                            scale=w.sm_scale if scale is None else scale,
                                            layout=w.layout)
    torch.cuda.synchronize()
    return out


def oracle_states(inp, ns, scale=None):
    w = inp.workload
    cu = inp.cu_seqlens_k.cpu().tolist()
    sc = w.sm_scale if scale is None else scale
    q, k, v = H.host(inp.q), H.host(inp.k), H.host(inp.v)
    m, l, acc = oracle.attention_states(q, k, v, cu, w.heads, w.kv_heads, ns, sc, layout=w.layout)
    o = oracle.attention_split_merge_states(q, k, v, cu, w.heads, w.kv_heads, ns, sc,
                                            layout=w.layout)
    return m, l, acc, o


def compare_states(inp, ns, scale=None):
    dtype = inp.workload.dtype
    _, acc, m, l = gpu_states(inp, ns, scale)
    om, ol, oacc, oo = oracle_states(inp, ns, scale)
    empty = np.isneginf(om)
    assert np.array_equal(np.isneginf(m), empty), "empty splits differ"
    assert not l[empty].any() and not acc[empty].any()
    full = ~empty
    assert np.abs(m[full] - om[full]).max(initial=0) <= LOG_TOL * max(1.0, np.abs(om[full]).max(initial=0))
    lse_gpu = m[full] + np.log2(l[full])
    lse_ref = om[full] + np.log2(ol[full])
    assert np.abs(lse_gpu - lse_ref).max(initial=0) <= LOG_TOL * max(1.0, np.abs(lse_ref).max(initial=0))
    part = acc[full] / l[full][:, None]
    part_ref = oacc[full] / ol[full][:, None]
    assert H.max_err(part, part_ref) <= H.TOL[dtype]
    out = H.host(gpu_attention_unnorm(inp, ns, scale))
    err = H.max_err(out, oo)
    print(f"  {inp.workload.name} ns={ns} out err={err:.3e}", flush=True)
    assert err <= H.TOL[dtype], (inp.workload.name, ns, err)


# ---------------------------------------------------- structured, exact --
def structured_inputs(lengths, heads, kv_heads, dim, dtype, ns, layout, pad=3):
    """K = 0: every score is 0, so m_s = 0 and l_s is the key count. V
    carries integers: channel 0 is 1 at each ceil-equal split's first key,
    channel 1 at its last, channel 2 the sequence index, channel 3 the KV
    head, channel 4 the key position mod 16. Memory outside every sequence
    is NaN."""
    B = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    rng = np.random.default_rng(11)
    q = torch.from_numpy(rng.standard_normal((B, heads, dim)).astype(np.float32)).to(DT[dtype])
    if layout == "packed":
        k = torch.full((T + pad, kv_heads, dim), float("nan"))
        v = torch.full((T + pad, kv_heads, dim), float("nan"))
        k[:T] = 0
        v[:T] = 0
    else:
        S = max(max(lengths), 1)
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
            for a, e in oracle.split_bounds_ceil(L, ns):
                if e > a:
                    rows[a, 0] = 1
                    rows[e - 1, 1] = 1
    w = W.Workload("structured_ceil", B, heads, kv_heads, dim, dtype, kv_len=None, layout=layout,
                   num_splits=ns)
    cu_t = torch.tensor(cu, dtype=torch.int32)
    return W.Inputs(w, q.to(H.DEV), k.to(DT[dtype]).to(H.DEV), v.to(DT[dtype]).to(H.DEV),
                    cu_t.to(H.DEV), list(lengths))


CASES = [
    # lengths, heads, kv_heads, dim, dtype, ns, layout
    ([10], 8, 1, 128, "f32", 6, "packed"),             # the page's example: empty 6th split
    ([10000], 8, 1, 128, "f32", 7, "packed"),
    ([10000], 8, 1, 128, "f32", 1000, "packed"),
    ([1, 2, 3, 17, 64, 65, 300], 28, 4, 128, "f16", 8, "packed"),   # ns > L for short ones
    ([8, 9, 31, 257, 1000, 4097], 28, 4, 128, "f16", 16, "packed"),
    ([256, 300, 511], 16, 2, 64, "bf16", 16, "bhsd"),
    ([129, 4, 77], 32, 8, 32, "bf16", 40, "packed"),
    ([100, 37, 64], 32, 2, 128, "f16", 37, "packed"),  # group 16: two row chunks
    ([0, 12, 40], 8, 2, 128, "bf16", 5, "packed"),     # an empty sequence
    ([5, 33, 1], 6, 2, 16, "f32", 4, "bhsd"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-d{c[3]}-g{c[1]//c[2]}-ns{c[5]}-{c[6]}")
def test_ceil_bounds_and_states_are_exact(case, kernel_path):
    lengths, heads, kv_heads, dim, dtype, ns, layout = case
    inp = structured_inputs(lengths, heads, kv_heads, dim, dtype, ns, layout)
    G = heads // kv_heads
    _, acc, m, l = gpu_states(inp, ns, scale=0.37)
    for b, L in enumerate(lengths):
        for h in range(heads):
            j = h // G
            for s, (a, e) in enumerate(oracle.split_bounds_ceil(L, ns)):
                n = e - a
                x = acc[b, h, s]
                if n == 0:
                    assert m[b, h, s] == -np.inf and l[b, h, s] == 0 and not x.any(), (b, h, s)
                    continue
                assert m[b, h, s] == 0.0 and l[b, h, s] == n, (b, h, s, m[b, h, s], l[b, h, s], n)
                assert x[0] == 1 and x[1] == 1, (b, h, s, x[:2])
                assert x[2] == b * n and x[3] == j * n, (b, h, s, x[2:4])
                assert x[4] == sum(t % 16 for t in range(a, e)), (b, h, s)
    out = H.host(gpu_attention_unnorm(inp, ns, scale=0.37))
    for b, L in enumerate(lengths):
        for h in range(heads):
            if L == 0:
                assert not out[b, h].any()
                continue
            assert round(float(out[b, h, 2])) == b and round(float(out[b, h, 3])) == h // G
            nonempty = sum(1 for a, e in oracle.split_bounds_ceil(L, ns) if e > a)
            assert abs(float(out[b, h, 0]) - nonempty / L) <= 1e-2 * max(1.0, nonempty / L)


# -------------------------------------------------- random inputs, oracle --
def _rand(lengths, heads, kv_heads, dim, dtype, layout="packed", seed=0, pad=0):
    w = W.Workload("unnorm", len(lengths), heads, kv_heads, dim, dtype, kv_len=None, layout=layout)
    return W.make_inputs(w, H.DEV, seed=seed, lengths=lengths, pad_rows=pad)


@pytest.mark.parametrize("ns", [7, 1000, 1])
def test_tiny_exactness_case(ns, kernel_path):
    """fp32, 8 query heads on 1 KV head, d=128, 10,000 keys."""
    compare_states(W.make_inputs(W.tiny(), H.DEV), ns)


@pytest.mark.parametrize("dim", [16, 64, 128])
def test_mha_head_dims(dim, kernel_path):
    """MHA at batch 4, 32 heads, fp16, [B,H,S,D]; 1024 keys (the 4096-key
    benchmark shape at a size the oracle walks in seconds), 16 splits."""
    w = W.with_(W.mha(dim), kv_len=1024)
    compare_states(W.make_inputs(w, H.DEV), 16)


@pytest.mark.parametrize("ns", [3, 32, 128])
def test_llama_bf16(ns, kernel_path):
    """32/8 heads, bf16, one 8192-key sequence and a ragged second one."""
    compare_states(_rand([8192, 1111], 32, 8, 128, "bf16", seed=3), ns)


def test_varlen_ragged_with_empty_tails(kernel_path):
    """28/4 heads (group 7), fp16, lengths down to 1 key with 12 splits:
    many empty tail splits."""
    compare_states(_rand([1, 5, 11, 12, 13, 700, 3001], 28, 4, 128, "f16", seed=5, pad=16), 12)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("group", [1, 3, 8, 16])
def test_grid(dtype, group, kernel_path):
    compare_states(_rand([1, 37, 300, 1029], 2 * group, 2, 64, dtype, seed=group), 5)


def test_page_selftest_shape():
    """flash_decode_splitk.py's self-test shape: B2 H4 D64 L256, 4 splits."""
    w = W.Workload("page_selftest", 2, 4, 4, 64, "f16", kv_len=256, layout="bhsd", num_splits=4)
    compare_states(W.make_inputs(w, H.DEV, seed=0), 4)


# ----------------------------------------------------------- consistency --
def test_whole_call_matches_split_then_combine():
    fd = H.fd()
    inp = _rand([4000, 900, 3], 32, 8, 128, "bf16", seed=9)
    whole = gpu_attention_unnorm(inp, 6).clone()
    ws = fd.fd_decode_split_unnorm(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 6)
    out = torch.empty_like(inp.q)
    fd.fd_decode_combine_unnorm(ws, 3, 32, 128, 6, out)
    torch.cuda.synchronize()
    assert torch.equal(out, whole)


def test_single_split_equals_the_other_format():
    """With one split both formats run the same single launch."""
    inp = _rand([700, 65], 16, 2, 128, "f16", seed=4)
    a = gpu_attention_unnorm(inp, 1).clone()
    b = H.gpu_attention(inp, 1)
    assert torch.equal(a, b)


def test_formats_agree_within_tolerance():
    inp = _rand([3000, 2222], 28, 4, 128, "f16", seed=6)
    a = H.host(gpu_attention_unnorm(inp, 8))
    b = H.host(H.gpu_attention(inp, 8))
    assert H.max_err(a, b) <= H.TOL["f16"]


def test_all_empty_sequences_give_zero_rows():
    inp = _rand([0, 0], 8, 2, 64, "f16", pad=4)
    for ns in (1, 3):
        out = H.host(gpu_attention_unnorm(inp, ns))
        assert not out.any()


def test_maximum_split_count_unnorm():
    """FD_MAX_SPLITS ceil-equal splits over 20,000 and 9,000 keys: size 2,
    so the shorter sequence leaves thousands of empty tail splits."""
    ns = H.fd().FD_MAX_SPLITS
    compare_states(_rand([20000, 9000], 8, 1, 128, "f16", seed=22), ns)
