"""Shared helpers of the GPU parity tests: run libfd on seeded inputs and
compare with the fp64 oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import workloads as W

# Max-abs error allowed against the fp64 oracle, per input dtype.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
LOG2E = 1.0 / math.log(2.0)
DEV = "cuda:0"


def fd():
    import decode_attention_09_amd as m
    return m


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (run with -m 'not gpu' on CPU)"
    fd().load_library()


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float32 host copy (fp16/bf16 values are exactly representable)."""
    return t.detach().to(torch.float32).cpu().numpy()


def gpu_attention(inp: W.Inputs, ns: int, scale=None, stream=None):
    w = inp.workload
    announce("fd_decode_attention", w.name, f"ns={ns}", f"lens[:4]={inp.lengths[:4]}")
    out = fd().fd_decode_attention(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                                   scale=w.sm_scale if scale is None else scale,
                                   layout=w.layout, stream=stream)
    torch.cuda.synchronize()
    return out


def gpu_split(inp: W.Inputs, ns: int, scale=None):
    w = inp.workload
    announce("fd_decode_split", w.name, f"ns={ns}")
    ws = fd().fd_decode_split(inp.q, inp.k, inp.v, inp.cu_seqlens_k, ns,
                              scale=w.sm_scale if scale is None else scale, layout=w.layout)
    torch.cuda.synchronize()
    opart, lse = fd().workspace_views(ws, w.batch, w.heads, w.dim, ns)
    return ws, host(opart), host(lse)


def oracle_full(inp: W.Inputs, ns: int | None = None, scale=None):
    """Oracle output for the whole batch (split+merge when ns is valid for
    every sequence, direct otherwise)."""
    w = inp.workload
    q, k, v = host(inp.q), host(inp.k), host(inp.v)
    cu = inp.cu_seqlens_k.cpu().tolist()
    sc = w.sm_scale if scale is None else scale
    if ns is not None and min(inp.lengths) >= ns:
        return oracle.attention_split_merge(q, k, v, cu, w.heads, w.kv_heads, ns, sc,
                                            layout=w.layout)
    return oracle.attention_direct(q, k, v, cu, w.heads, w.kv_heads, sc, layout=w.layout)


def oracle_pairs(inp: W.Inputs, pairs, scale=None, workers: int = 1):
    """Oracle rows for (b, kv_head) pairs, copying only their K/V rows to the
    host, one pair at a time. With workers > 1 the oracle evaluations run in
    a thread pool (numpy releases the GIL) while the next pair is copied.
    Returns {(b, kvh): o [G, D]}."""
    from concurrent.futures import ThreadPoolExecutor
    w = inp.workload
    G = w.group
    sc = w.sm_scale if scale is None else scale
    cu = inp.cu_seqlens_k.cpu().tolist()

    def rows(b, j):
        L = cu[b + 1] - cu[b]
        if w.layout == "packed":
            return host(inp.k[cu[b]:cu[b + 1], j, :]), host(inp.v[cu[b]:cu[b + 1], j, :])
        return host(inp.k[b, j, :L, :]), host(inp.v[b, j, :L, :])

    res = {}
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        futs, pending = {}, []
        for n, (b, j) in enumerate(pairs):
            kr, vr = rows(b, j)
            qr = host(inp.q[b, j * G:(j + 1) * G, :])
            f = ex.submit(oracle.attention_rows, qr, kr, vr, sc)
            futs[(b, j)] = f
            pending.append(f)
            del kr, vr
            if len(pending) >= 2 * max(1, workers):   # bound the host copies held
                pending.pop(0).result()
            if (n + 1) % 16 == 0:
                announce(f"  oracle pairs copied: {n + 1}/{len(pairs)}")
        for key, f in futs.items():
            res[key] = f.result()
    return res


MANTISSA_BITS = {"f32": 23, "f16": 10, "bf16": 7}
U32 = 2.0 ** -24                                   # fp32 unit roundoff
U_P = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}  # rounding of P


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output dtype at |x| (normal range; the smallest normal
    exponent is a floor for tiny values)."""
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(ax)) - MANTISSA_BITS[dtype])


def scaled_bound(qr, kr, vr, scale, dtype, ref):
    """Per-element bound [G, D] on |computed - exact| for one (sequence, KV
    head) at a non-default scale (the full derivation is in the docstring of
    tests/test_gpu_random.py). On top of the dtype tolerance: the effect on
    the softmax-weighted mean of the fp32 scores' forward error (per key
    |scale| gamma_D sum_i |q_i k_ti| -- the dot-product bound of Higham,
    Accuracy and Stability of Numerical Algorithms, eq. (3.5), for any
    summation order -- plus the roundings of the scale, the product, the max
    subtraction and exp2), the rounding of P to a 16-bit input type, and
    half an ulp of the output dtype at |o| (the cast of the result)."""
    s = scale * (qr @ kr.T)                                     # [G, L]
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)                           # exact weights
    n = qr.shape[1]
    gamma = n * U32 / (1.0 - n * U32)
    delta = abs(scale) * gamma * (np.abs(qr) @ np.abs(kr).T) + 3 * U32 * np.abs(s) + 2.0 ** -22
    d_w = np.log((w * np.exp(delta)).sum(axis=1, keepdims=True))
    f = w * np.expm1(delta + d_w)
    e_s = np.stack([f[g] @ np.abs(vr - ref[g]) for g in range(ref.shape[0])])
    e_p = U_P[dtype] * (w @ np.abs(vr))
    rest = TOL[dtype] + e_s + e_p
    return rest + 0.5 * ulp(np.abs(ref) + rest, dtype)


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    assert np.isfinite(d).all(), "non-finite values in the comparison"
    return float(d.max())
