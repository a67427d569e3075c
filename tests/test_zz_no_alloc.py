"""fd_decode_attention_noalloc (no workspace argument; the partials go to the
library's static per-GPU scratch) through the C ABI: its output equals
fd_decode_attention's on the same inputs, over two calls in a row -- the
second smaller than the first, so stale partials of the first call in the
scratch would show -- and the oracle's within the dtype tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _inputs(lengths, heads, kv_heads, dim, dtype, seed):
    w = W.Workload("noalloc", len(lengths), heads, kv_heads, dim, dtype, kv_len=None)
    return W.make_inputs(w, H.DEV, seed=seed, lengths=lengths, pad_rows=4)


CASES = [  # (lengths, heads, kv_heads, dim, dtype, num_splits): larger call first
    ([9000, 4097, 12000, 700, 5000], 28, 4, 128, "f16", 16),
    ([300, 1000], 8, 2, 64, "bf16", 4),
]


def test_noalloc_equals_the_workspace_call_twice_in_a_row():
    H.require_gpu()
    fd = H.fd()
    for i, (lens, heads, kvh, dim, dtype, ns) in enumerate(CASES):
        inp = _inputs(lens, heads, kvh, dim, dtype, seed=40 + i)
        H.announce("fd_decode_attention_noalloc", lens, heads, kvh, dim, dtype, f"ns={ns}")
        ref = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns)
        out = torch.full_like(inp.q, float("nan"))
        fd.fd_decode_attention_noalloc(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        err = H.max_err(H.host(out), H.oracle_full(inp, ns))
        assert err <= H.TOL[dtype], (i, err)


def test_noalloc_single_split_and_repeat():
    """One split writes out directly (no scratch); repeated calls are
    bitwise identical."""
    H.require_gpu()
    fd = H.fd()
    inp = _inputs([2000, 31, 4100], 16, 2, 128, "bf16", seed=50)
    ref1 = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 1)
    out = torch.empty_like(inp.q)
    fd.fd_decode_attention_noalloc(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 1, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref1)
    ref8 = fd.fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8)
    for _ in range(3):
        fd.fd_decode_attention_noalloc(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 8, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref8)


def test_noalloc_refuses_calls_beyond_the_scratch():
    H.require_gpu()
    fd = H.fd()
    # 64 heads x 1100 splits x (128 + 1) floats > 16 MiB
    inp = _inputs([1200], 64, 64, 128, "f16", seed=51)
    out = torch.zeros_like(inp.q)
    with pytest.raises(fd.FdError) as e:
        fd.fd_decode_attention_noalloc(inp.q, inp.k, inp.v, inp.cu_seqlens_k, 1100, out)
    assert e.value.status == 5 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not out.any()
