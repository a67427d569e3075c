"""Seeded random sweep over the whole call: each case draws dtype, head dim,
group size, KV heads, batch, ragged lengths (empty sequences and lengths
below the split count included), split count, K/V layout (packed,
[B, Hkv, S, D], [B, S, Hkv, D]), split format, kernel path and sometimes a
non-default scale, and checks every output element against the fp64
oracle's direct attention (empty sequences: zero rows). K/V rows outside
the sequences are NaN, so an over-read shows.

Bound: the dtype's max-abs tolerance, plus one unit in the last place of
the output dtype at the reference's magnitude, plus the forward error of
fp32 scores, 4 * 2^-24 * max|s| * max|v| (s = scale * q.k). The output is
written in the input dtype, as the pages' reference casts it; with scales
up to 16x the default the softmax collapses onto a few keys and |o|
approaches the largest |v| (about 4), where one bf16 ulp is 0.016 -- so the
final cast of even the exact result can miss a fixed 1e-2 -- and scores
reach |s| ~ 70, whose fp32 rounding alone moves an fp32 output by ~1e-5.
At the default scale (all the workload tests) outputs stay far below 1,
|s| stays near 5, and the fixed tolerances apply unchanged."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

N_CASES = 120
PATHS = {"auto": 0, "valu": 1, "mfma": 2, "unpacked": 3}
MANTISSA_BITS = {"f32": 23, "f16": 10, "bf16": 7}


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output dtype at |x| (normal range; the smallest normal
    exponent is a floor for tiny values)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(ax)) - MANTISSA_BITS[dtype])


def _draw(i: int):
    rng = np.random.default_rng(20261202 + i)
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    dim = int(rng.choice([16, 32, 64, 128]))
    group = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16]))
    kv_heads = int(rng.integers(1, 5))
    batch = int(rng.integers(1, 7))
    lengths = []
    for _ in range(batch):
        kind = rng.random()
        if kind < 0.1:
            lengths.append(0)
        elif kind < 0.35:
            lengths.append(int(rng.integers(1, 17)))
        elif kind < 0.75:
            lengths.append(int(rng.integers(17, 301)))
        else:
            lengths.append(int(rng.integers(301, 3001)))
    if max(lengths) == 0:
        lengths[0] = 5
    ns = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64]))
    layout = str(rng.choice(["packed", "bhsd", "bshd"]))
    fmt = str(rng.choice(["lse", "unnorm"]))
    path = str(rng.choice(list(PATHS)))
    scale = None if rng.random() < 0.6 else float(rng.uniform(-1.0, 2.0))
    return dict(dtype=dtype, dim=dim, group=group, kv_heads=kv_heads, lengths=lengths, ns=ns,
                layout=layout, fmt=fmt, path=path, scale=scale, seed=i)


CASES = [_draw(i) for i in range(N_CASES)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("c", CASES, ids=lambda c: (
    f"s{c['seed']}-{c['dtype']}-d{c['dim']}-g{c['group']}x{c['kv_heads']}-ns{c['ns']}-"
    f"{c['layout']}-{c['fmt']}-{c['path']}"))
def test_random_case_matches_oracle(c):
    fd = H.fd()
    heads = c["group"] * c["kv_heads"]
    base_layout = "packed" if c["layout"] == "packed" else "bhsd"
    w = W.Workload(f"random{c['seed']}", len(c["lengths"]), heads, c["kv_heads"], c["dim"],
                   c["dtype"], kv_len=None, layout=base_layout)
    inp = W.make_inputs(w, H.DEV, seed=c["seed"], lengths=c["lengths"], pad_rows=8)
    k, v = inp.k, inp.v
    if c["layout"] == "bshd":
        k = k.transpose(1, 2).contiguous()
        v = v.transpose(1, 2).contiguous()
    scale = w.sm_scale if c["scale"] is None else c["scale"]
    call = fd.fd_decode_attention_unnorm if c["fmt"] == "unnorm" else fd.fd_decode_attention
    H.announce("random", c)
    prev = fd.fd_set_kernel_path(PATHS[c["path"]])
    try:
        out = call(inp.q, k, v, inp.cu_seqlens_k, c["ns"], scale=scale, layout=c["layout"])
        torch.cuda.synchronize()
    finally:
        fd.fd_set_kernel_path(prev)
    out = H.host(out)
    assert np.isfinite(out).all()
    q = H.host(inp.q)
    cu = inp.cu_seqlens_k.cpu().tolist()
    G = c["group"]
    kh, vh = H.host(inp.k), H.host(inp.v)
    for b, L in enumerate(c["lengths"]):
        for j in range(c["kv_heads"]):
            rows = out[b, j * G:(j + 1) * G]
            if L == 0:
                assert not rows.any(), (b, j)
                continue
            kr = oracle.kv_rows(kh, cu, b, j, base_layout)
            vr = oracle.kv_rows(vh, cu, b, j, base_layout)
            qr = q[b, j * G:(j + 1) * G].astype(np.float64)
            ref = oracle.attention_rows(qr, kr, vr, scale)
            score_err = 4.0 * 2.0 ** -24 * np.abs(scale * (qr @ kr.T)).max() * np.abs(vr).max()
            excess = np.abs(rows - ref) - (H.TOL[c["dtype"]] + ulp(ref, c["dtype"]) + score_err)
            assert excess.max() <= 0.0, (b, j, L, H.max_err(rows, ref), excess.max())
