"""Seeded random sweep over the whole call: each case draws dtype, head dim,
group size, KV heads, batch, ragged lengths (empty sequences and lengths
below the split count included), split count, K/V layout (packed,
[B, Hkv, S, D], [B, S, Hkv, D]), split format, kernel path, sometimes a
non-default scale, the single-launch (fused) combine and the queue or
steal schedule, and checks every output element against the fp64
oracle's direct attention (empty sequences: zero rows). K/V rows outside
the sequences are NaN, so an over-read shows.

Bound. Draws at the default scale 1/sqrt(dim) are held to the dtype's
max-abs tolerance (fp32 1e-5, fp16 2e-3, bf16 1e-2), unchanged. Draws with
another scale (up to 23x the default) concentrate the softmax on a few
keys, so the output approaches single V entries (|o| up to ~4) and three
rounding steps that average out at the default scale no longer do. For
those draws each element o_d is allowed, on top of the tolerance:

  * half a unit in the last place of the output dtype at |o_d|: the result
    is rounded to nearest in the input dtype, as the pages' reference casts
    it (flash_decode_splitk.py returns out.to(q.dtype));
  * the effect of the fp32 scores' forward error. Per key, the computed
    score is s_t + delta_t with |delta_t| <= |scale| gamma_D sum_i |q_i k_ti|
    + 3u|s_t| + 2^-22: the dot-product bound |fl(x.y) - x.y| <=
    gamma_n sum |x_i y_i|, gamma_n = nu / (1 - nu), u = 2^-24, for any
    summation order (Higham, Accuracy and Stability of Numerical
    Algorithms, 2nd ed., eq. (3.5)), the fp32 roundings of scale*log2(e), of
    the product and of the max subtraction, and the exp2 instruction's
    error. Perturbing the scores by delta moves the softmax-weighted mean
    by at most sum_t w_t |v_td - o_d| expm1(|delta_t| + D_w),
    D_w = ln sum_t w_t e^|delta_t| (the weights' ratio to the exact ones is
    e^delta_t / sum_u w_u e^delta_u);
  * for fp16/bf16 inputs, the rounding of the probabilities to the input
    type before the P.V products (the TileLang page's cast of P):
    u_dtype sum_t w_t |v_td|, u_dtype = 2^-11 (fp16), 2^-8 (bf16).

w_t are the exact softmax weights, from the fp64 oracle's scores."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

N_CASES = 200
PATHS = {"auto": 0, "valu": 1, "mfma": 2, "unpacked": 3}
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
    # drawn last, so the draws above are those of the sweep without them
    combine = "fused" if rng.random() < 0.35 else "separate"
    u = rng.random()
    sched = "queue" if u < 0.35 else "steal" if u < 0.6 else "auto"
    return dict(dtype=dtype, dim=dim, group=group, kv_heads=kv_heads, lengths=lengths, ns=ns,
                layout=layout, fmt=fmt, path=path, scale=scale, combine=combine, sched=sched,
                seed=i)


CASES = [_draw(i) for i in range(N_CASES)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    H.require_gpu()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("c", CASES, ids=lambda c: (
    f"s{c['seed']}-{c['dtype']}-d{c['dim']}-g{c['group']}x{c['kv_heads']}-ns{c['ns']}-"
    f"{c['layout']}-{c['fmt']}-{c['path']}-{c['combine']}-{c['sched']}"))
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
    prev_c = fd.fd_set_combine(fd.FD_COMBINE_FUSED if c["combine"] == "fused"
                               else fd.FD_COMBINE_SEPARATE)
    prev_s = fd.fd_set_schedule({"queue": fd.FD_SCHED_QUEUE, "steal": fd.FD_SCHED_STEAL,
                                 "auto": fd.FD_SCHED_AUTO}[c["sched"]])
    try:
        out = call(inp.q, k, v, inp.cu_seqlens_k, c["ns"], scale=scale, layout=c["layout"])
        torch.cuda.synchronize()
    finally:
        fd.fd_set_kernel_path(prev)
        fd.fd_set_combine(prev_c)
        fd.fd_set_schedule(prev_s)
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
            if c["scale"] is None:
                bound = H.TOL[c["dtype"]]
            else:
                bound = H.scaled_bound(qr, kr, vr, scale, c["dtype"], ref)
            excess = np.abs(rows - ref) - bound
            assert excess.max() <= 0.0, (b, j, L, H.max_err(rows, ref), excess.max())
