"""The whole call under HIP graph capture: libfd allocates nothing, records
no memset and never synchronises inside a call, so a decode step can be
captured once and replayed. Each replay is checked bitwise against an eager
call on the same inputs, with eager work (new q values, other calls) between
the replays."""
import pytest
import torch

import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.empty_cache()


CASES = [
    # (lengths, heads, kv_heads, dim, dtype, layout, ns, unnormalised format)
    ([4096] * 2, 8, 8, 128, "f16", "bhsd", 16, False),     # VALU kernel, split + combine
    ([3000, 17, 900], 28, 4, 128, "bf16", "packed", 8, False),  # matrix-core kernel
    ([500, 64], 16, 2, 64, "f16", "packed", 1, False),      # one launch, written directly
    ([1000, 3, 250], 32, 8, 128, "f16", "packed", 5, True),  # (m, l, acc) format
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-d{c[3]}-ns{c[6]}-{'mi' if c[7] else 'lse'}")
def test_graph_replays_match_eager(case):
    lengths, heads, kvh, dim, dtype, layout, ns, unnorm = case
    fdm = H.fd()
    w = W.Workload("graph", len(lengths), heads, kvh, dim, dtype, kv_len=None, layout=layout)
    inp = W.make_inputs(w, H.DEV, seed=3, lengths=lengths, pad_rows=8)
    q_alt = W.make_inputs(w, H.DEV, seed=4, lengths=lengths).q
    q_buf = inp.q.clone()
    call = fdm.fd_decode_attention_unnorm if unnorm else fdm.fd_decode_attention
    wsize = (fdm.fd_workspace_bytes_unnorm if unnorm else fdm.fd_workspace_bytes)(
        len(lengths), heads, ns, dim)
    ws = torch.empty(max(1, wsize), dtype=torch.uint8, device=H.DEV)
    out_g = torch.empty_like(inp.q)

    def run(q, out, stream):
        call(q, inp.k, inp.v, inp.cu_seqlens_k, ns, out=out, workspace=ws, layout=layout,
             stream=stream)

    # warm up on a side stream, as capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(q_buf, out_g, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(q_buf, out_g, torch.cuda.current_stream())
    torch.cuda.synchronize()

    def eager(q):
        out = torch.empty_like(q)
        run(q, out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return out

    ref_a, ref_b = eager(inp.q), eager(q_alt)
    for rep, (src, ref) in enumerate([(inp.q, ref_a), (q_alt, ref_b), (inp.q, ref_a)]):
        q_buf.copy_(src)            # eager work between replays
        eager(q_alt)                # another call on the same workspace
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), (case, rep)
    del g
