"""Plain fp64 CPU oracle for single-query split-KV decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library and imports
nothing from it.

Every input is converted exactly to float64 and every step below is the
plain definition, one (batch, KV head) at a time, with no blocking or fusion.
Numpy's matmul is the only library primitive used (for q.K^T and p.V).

Sources (web pages this follows):
  * "decode_attention_splitkv.py", TileLang tutorial chapter 18
    (split-KV / flash decoding skeleton), function ``gqa_decode_splitkv``:
    GQA head packing (query head h reads KV head h // (heads // kv_heads)),
    varlen KV addressed by ``cu_seqlens_k``, proportional split bounds, the
    split epilogue (normalised partial output plus its log-sum-exp) and the
    combine segment (log-sum-exp weighted merge). Its docstring states the
    constraint that every split covers at least one key.
  * "flash_decode_splitk.py" (MiniInfer), ``flash_decode_reference``: direct
    softmax(q K^T * scale) V with the default scale 1/sqrt(dim), and the
    [batch, heads, seqlen, dim] layout.
  * "04_flash_decoding.py", CS349E lecture 11, demo 1: per-split o_s and
    lse_s = log sum exp(scores), merged as lse = log sum exp(lse_s) and
    o = sum exp(lse_s - lse) o_s, which equals direct attention exactly.

Readings where the pages leave a step open (each one is also listed in the
design notes):
  * LSE is kept in natural-log units here; the GPU workspace stores base-2
    units and tests convert with ln 2.
  * ``scale`` multiplies q.k before the softmax (natural-exp units).
  * A split with no keys is an error (the page says the scheduler must
    prevent it), so ``split_bounds`` raises when num_splits > seqlen.

The second split format, that of ``_splitk_stage1_kernel`` /
``_splitk_reduce_kernel`` in "flash_decode_splitk.py" (MiniInfer), is here
too: ceil-equal split bounds (``split_bounds_ceil``, empty tail splits
allowed) and the unnormalised per-split state (running max m, sum l and
accumulator acc in base-2 units of the scaled scores, ``split_states_rows``)
merged by rescaling to the largest m (``merge_states``). Readings: a split
with no keys has state (-inf, 0, 0) (the stage-1 kernel's initial values,
written unchanged when its key loop is empty); a row whose splits are all
empty merges to zeros (the page's host check keeps KV_LEN >= 1, so it
never reaches that case).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "split_bounds",
    "kv_rows",
    "attention_rows",
    "split_partials_rows",
    "merge_partials",
    "attention_direct",
    "attention_partials",
    "attention_split_merge",
    "head_pairs",
    "split_bounds_ceil",
    "split_states_rows",
    "merge_states",
    "attention_states",
    "attention_split_merge_states",
]


def split_bounds(seqlen: int, num_splits: int) -> list[tuple[int, int]]:
    """Proportional split bounds of one sequence.

    decode_attention_splitkv.py, split segment: split ``sid`` covers keys
    ``[seqlen*sid // num_splits, seqlen*(sid+1) // num_splits)``. The
    docstring's constraint (every split covers at least one key, i.e.
    ``num_splits <= seqlen``) is enforced by raising ValueError.
    Python integers, so the product never overflows.
    """
    seqlen = int(seqlen)
    num_splits = int(num_splits)
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    if seqlen < num_splits:
        raise ValueError(
            f"num_splits={num_splits} > seqlen={seqlen}: some split would be empty")
    return [(seqlen * s // num_splits, seqlen * (s + 1) // num_splits)
            for s in range(num_splits)]


def kv_rows(kv: np.ndarray, cu_seqlens_k, b: int, kvh: int, layout: str) -> np.ndarray:
    """Rows of sequence ``b``, KV head ``kvh`` as a float64 [L_b, dim] array.

    layout "packed": kv is [total_kv, kv_heads, dim] and sequence b owns rows
    [cu[b], cu[b+1]) (decode_attention_splitkv.py, varlen comment and
    shape_kv). layout "bhsd": kv is [batch, kv_heads, max_len, dim] and
    sequence b owns rows [0, cu[b+1]-cu[b]) of kv[b, kvh]
    (flash_decode_splitk.py uses [batch, heads, seqlen, dim]).
    """
    start = int(cu_seqlens_k[b])
    end = int(cu_seqlens_k[b + 1])
    if end < start:
        raise ValueError("cu_seqlens_k must be non-decreasing")
    if layout == "packed":
        rows = kv[start:end, kvh, :]
    elif layout == "bhsd":
        rows = kv[b, kvh, 0:end - start, :]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return np.asarray(rows, dtype=np.float64)


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Direct attention for R query rows over one KV sequence.

    q [R, D], k [L, D], v [L, D] -> o [R, D] = softmax(scale * q k^T) v,
    the definition used by flash_decode_reference (here in float64 with no
    cast of the probabilities). The max is subtracted before exp only to
    keep exp finite; it cancels in the ratio.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("attention over an empty KV sequence is undefined")
    s = scale * (q @ k.T)                       # [R, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def split_partials_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                        num_splits: int, scale: float):
    """Per-split normalised outputs and log-sum-exps for one KV sequence.

    For each proportional split [a, e): o_s = softmax(scale q k_[a,e)^T) v_[a,e)
    and lse_s = ln sum_{t in [a,e)} exp(scale q.k_t)  (natural log), the
    pair the split epilogue of decode_attention_splitkv.py writes out
    (there in base 2) and 04_flash_decoding.py demo 1 describes.
    Returns (o_parts [R, ns, D], lse [ns, R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bounds = split_bounds(k.shape[0], num_splits)
    R, D = q.shape
    o_parts = np.empty((R, num_splits, D), dtype=np.float64)
    lse = np.empty((num_splits, R), dtype=np.float64)
    for s_idx, (a, e) in enumerate(bounds):
        sc = scale * (q @ k[a:e].T)             # [R, e-a]
        m = sc.max(axis=1, keepdims=True)
        p = np.exp(sc - m)
        l = p.sum(axis=1, keepdims=True)
        o_parts[:, s_idx, :] = (p @ v[a:e]) / l
        lse[s_idx, :] = (m + np.log(l))[:, 0]
    return o_parts, lse


def merge_partials(o_parts: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """Exact log-sum-exp merge of split results for one set of rows.

    o_parts [R, ns, D], lse [ns, R] (natural log) -> o [R, D] with
    L = max_s lse_s + ln sum_s exp(lse_s - max), w_s = exp(lse_s - L),
    o = sum_s w_s o_s: the combine segment of decode_attention_splitkv.py
    (weight of split s for head row i applied to that row), and
    04_flash_decoding.py demo 1.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    mx = lse.max(axis=0)                        # [R]
    total = mx + np.log(np.exp(lse - mx).sum(axis=0))
    w = np.exp(lse - total)                     # [ns, R]
    return np.einsum("sr,rsd->rd", w, o_parts)


def head_pairs(heads: int, kv_heads: int):
    """Query heads of each KV head: KV head j serves heads [j*G, (j+1)*G),
    G = heads // kv_heads (decode_attention_splitkv.py: ``cur_kv_head``)."""
    if heads % kv_heads != 0:
        raise ValueError("heads must be a multiple of kv_heads")
    g = heads // kv_heads
    return [(j, list(range(j * g, (j + 1) * g))) for j in range(kv_heads)]


def _check(q, cu_seqlens_k, heads, kv_heads):
    q = np.asarray(q)
    if q.ndim != 3 or q.shape[1] != heads:
        raise ValueError("q must be [batch, heads, dim]")
    if len(cu_seqlens_k) != q.shape[0] + 1:
        raise ValueError("cu_seqlens_k must have batch + 1 entries")
    if heads % kv_heads != 0:
        raise ValueError("heads must be a multiple of kv_heads")


def attention_direct(q, k, v, cu_seqlens_k, heads: int, kv_heads: int, scale: float,
                     layout: str = "packed", pairs=None) -> np.ndarray:
    """Direct decode attention for a whole batch: o [batch, heads, dim] fp64.

    ``pairs`` optionally restricts the work to a list of (b, kv_head); the
    rows not computed are left as NaN (used to sample large workloads).
    """
    _check(q, cu_seqlens_k, heads, kv_heads)
    B, H, D = q.shape
    out = np.full((B, H, D), np.nan, dtype=np.float64)
    groups = dict(head_pairs(heads, kv_heads))
    todo = pairs if pairs is not None else [(b, j) for b in range(B) for j in range(kv_heads)]
    for b, j in todo:
        hs = groups[j]
        kr = kv_rows(k, cu_seqlens_k, b, j, layout)
        vr = kv_rows(v, cu_seqlens_k, b, j, layout)
        out[b, hs, :] = attention_rows(np.asarray(q[b, hs, :], dtype=np.float64), kr, vr, scale)
    return out


def attention_partials(q, k, v, cu_seqlens_k, heads: int, kv_heads: int,
                       num_splits: int, scale: float, layout: str = "packed", pairs=None):
    """Split phase for a whole batch.

    Returns (o_parts [batch, heads, ns, dim], lse [batch, ns, heads]) in the
    shapes of ``part_shape`` and ``lse_shape`` of decode_attention_splitkv.py
    (lse in natural log here). Entries of (b, kv_head) pairs not in ``pairs``
    are NaN.
    """
    _check(q, cu_seqlens_k, heads, kv_heads)
    B, H, D = q.shape
    o_parts = np.full((B, H, num_splits, D), np.nan, dtype=np.float64)
    lse = np.full((B, num_splits, H), np.nan, dtype=np.float64)
    groups = dict(head_pairs(heads, kv_heads))
    todo = pairs if pairs is not None else [(b, j) for b in range(B) for j in range(kv_heads)]
    for b, j in todo:
        hs = groups[j]
        kr = kv_rows(k, cu_seqlens_k, b, j, layout)
        vr = kv_rows(v, cu_seqlens_k, b, j, layout)
        op, ls = split_partials_rows(np.asarray(q[b, hs, :], dtype=np.float64), kr, vr,
                                     num_splits, scale)
        o_parts[b, hs, :, :] = op
        lse[b, :, hs] = ls.T
    return o_parts, lse


def attention_split_merge(q, k, v, cu_seqlens_k, heads: int, kv_heads: int,
                          num_splits: int, scale: float, layout: str = "packed",
                          pairs=None) -> np.ndarray:
    """Split phase followed by the exact merge: o [batch, heads, dim] fp64."""
    o_parts, lse = attention_partials(q, k, v, cu_seqlens_k, heads, kv_heads,
                                      num_splits, scale, layout, pairs)
    B, H, ns, D = o_parts.shape
    out = np.full((B, H, D), np.nan, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            if np.isnan(lse[b, 0, h]):
                continue
            out[b, h:h + 1, :] = merge_partials(o_parts[b, h:h + 1], lse[b, :, h:h + 1])
    return out


# --------------------------------------------------------------------------
# MiniInfer's format: ceil-equal bounds, unnormalised (m, l, acc) state
# --------------------------------------------------------------------------
LOG2E = 1.0 / math.log(2.0)


def split_bounds_ceil(seqlen: int, num_splits: int) -> list[tuple[int, int]]:
    """Ceil-equal split bounds of one sequence.

    flash_decode_splitk.py, ``_splitk_stage1_kernel``: every split spans
    ``size = ceil(seqlen / num_splits)`` keys from ``sid * size``, cut at
    ``seqlen``. Splits that start at or past the end are empty; they are
    returned as ``(seqlen, seqlen)``. num_splits < 1 raises.
    """
    seqlen = int(seqlen)
    num_splits = int(num_splits)
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    if seqlen < 0:
        raise ValueError("seqlen must be >= 0")
    size = -(-seqlen // num_splits)
    return [(min(s * size, seqlen), min(s * size + size, seqlen)) for s in range(num_splits)]


def split_states_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      num_splits: int, scale: float):
    """Unnormalised state of every ceil-equal split of one KV sequence.

    With base-2 scaled scores s2_t = scale * log2(e) * q.k_t
    (``q * (sm_scale * 1.44269504)`` in _splitk_stage1_kernel), over the keys
    t of split s:  m_s = max_t s2_t,  l_s = sum_t 2^(s2_t - m_s),
    acc_s = sum_t 2^(s2_t - m_s) v_t  -- the values the stage-1 kernel's
    running update ends with. An empty split has (-inf, 0, 0).
    Returns (m [ns, R], l [ns, R], acc [R, ns, D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, D = q.shape
    m = np.full((num_splits, R), -np.inf, dtype=np.float64)
    l = np.zeros((num_splits, R), dtype=np.float64)
    acc = np.zeros((R, num_splits, D), dtype=np.float64)
    for s_idx, (a, e) in enumerate(split_bounds_ceil(k.shape[0], num_splits)):
        if e <= a:
            continue
        s2 = (scale * LOG2E) * (q @ k[a:e].T)   # [R, e-a]
        ms = s2.max(axis=1)
        p = np.exp2(s2 - ms[:, None])
        m[s_idx] = ms
        l[s_idx] = p.sum(axis=1)
        acc[:, s_idx, :] = p @ v[a:e]
    return m, l, acc


def merge_states(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """_splitk_reduce_kernel for one set of rows: m, l [ns, R], acc [R, ns, D]
    -> o [R, D] with M = max_s m_s, alpha_s = 2^(m_s - M),
    o = sum_s alpha_s acc_s / sum_s alpha_s l_s. Rows whose splits are all
    empty (M = -inf) give zeros."""
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    acc = np.asarray(acc, dtype=np.float64)
    R = m.shape[1]
    out = np.zeros((R, acc.shape[2]), dtype=np.float64)
    for r in range(R):
        M = m[:, r].max()
        if M == -np.inf:
            continue
        alpha = np.exp2(m[:, r] - M)            # 0 for empty splits
        out[r] = (alpha @ acc[r]) / (alpha @ l[:, r])
    return out


def attention_states(q, k, v, cu_seqlens_k, heads: int, kv_heads: int,
                     num_splits: int, scale: float, layout: str = "packed", pairs=None):
    """Stage 1 for a whole batch: (m [batch, heads, ns], l [batch, heads, ns],
    acc [batch, heads, ns, dim]), the shapes of M_BUF / L_BUF ([bh, ns]) and
    ACC_BUF ([bh, ns, dim]) in flash_decode_splitk.py. Pairs not in ``pairs``
    are NaN."""
    _check(q, cu_seqlens_k, heads, kv_heads)
    B, H, D = q.shape
    m = np.full((B, H, num_splits), np.nan, dtype=np.float64)
    l = np.full((B, H, num_splits), np.nan, dtype=np.float64)
    acc = np.full((B, H, num_splits, D), np.nan, dtype=np.float64)
    groups = dict(head_pairs(heads, kv_heads))
    todo = pairs if pairs is not None else [(b, j) for b in range(B) for j in range(kv_heads)]
    for b, j in todo:
        hs = groups[j]
        kr = kv_rows(k, cu_seqlens_k, b, j, layout)
        vr = kv_rows(v, cu_seqlens_k, b, j, layout)
        ms, ls, accs = split_states_rows(np.asarray(q[b, hs, :], dtype=np.float64), kr, vr,
                                         num_splits, scale)
        m[b, hs, :] = ms.T
        l[b, hs, :] = ls.T
        acc[b, hs, :, :] = accs
    return m, l, acc


def attention_split_merge_states(q, k, v, cu_seqlens_k, heads: int, kv_heads: int,
                                 num_splits: int, scale: float, layout: str = "packed",
                                 pairs=None) -> np.ndarray:
    """Stage 1 then the reduce, for a whole batch: o [batch, heads, dim]."""
    m, l, acc = attention_states(q, k, v, cu_seqlens_k, heads, kv_heads, num_splits, scale,
                                 layout, pairs)
    B, H, ns, D = acc.shape
    out = np.full((B, H, D), np.nan, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            if np.isnan(m[b, h, 0]):
                continue
            out[b, h:h + 1, :] = merge_states(m[b, h][:, None], l[b, h][:, None], acc[b, h:h + 1])
    return out
