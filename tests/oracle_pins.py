"""Independent checks that pin the fp64 oracle to the mathematics.

Each ``pin_*`` function takes the oracle module (or a stand-in with the same
functions) and raises AssertionError when the oracle disagrees with something
other than itself: closed forms, exhaustive integer properties, a 50-digit
Decimal brute force, torch's float64 scaled_dot_product_attention, or a
metamorphic relation. ``test_oracle.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on oracles with planted mistakes, which
every mutant must fail.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import torch


def _rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# split bounds: exhaustive integer properties
# --------------------------------------------------------------------------
def pin_split_bounds(orc, max_len: int = 120):
    """Proportional bounds (decode_attention_splitkv.py, split segment): for
    every 1 <= ns <= L the splits tile [0, L) in order, each has floor(L/ns)
    or ceil(L/ns) keys, exactly L mod ns of them have the larger size, and
    split s starts at floor(L*s/ns). ns > L and ns < 1 raise."""
    for L in range(1, max_len + 1):
        for ns in range(1, L + 1):
            b = orc.split_bounds(L, ns)
            assert len(b) == ns
            assert b[0][0] == 0 and b[-1][1] == L
            sizes = [e - a for a, e in b]
            for (a0, e0), (a1, _) in zip(b, b[1:]):
                assert e0 == a1
            lo, hi = L // ns, -(-L // ns)
            assert all(s in (lo, hi) for s in sizes), (L, ns, sizes)
            assert sum(1 for s in sizes if s == hi and hi != lo) == (L % ns)
            assert min(sizes) >= 1
            for s, (a, _) in enumerate(b):
                assert a == math.floor(L * s / ns) if L * s < 2 ** 52 else True
        for bad in (L + 1, L + 7):
            try:
                orc.split_bounds(L, bad)
            except ValueError:
                pass
            else:
                raise AssertionError(f"split_bounds({L},{bad}) must raise")
    for bad in (0, -1):
        try:
            orc.split_bounds(10, bad)
        except ValueError:
            pass
        else:
            raise AssertionError("num_splits < 1 must raise")
    # 64-bit-sized products stay exact (Python ints).
    big = orc.split_bounds(2 ** 40 + 3, 7)
    assert big[3][0] == (2 ** 40 + 3) * 3 // 7


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def pin_closed_forms(orc):
    rng = _rng(1)
    D = 16
    # One key: softmax is 1, the output is that key's value exactly.
    q = rng.standard_normal((3, D))
    k = rng.standard_normal((1, D))
    v = rng.standard_normal((1, D))
    o = orc.attention_rows(q, k, v, 0.7)
    assert np.array_equal(o, np.broadcast_to(v, (3, D))), "L=1 must return v0"
    # Zero query: uniform weights, output = mean of V, lse_s = ln(count_s).
    L = 37
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    q0 = np.zeros((2, D))
    o = orc.attention_rows(q0, k, v, 0.3)
    assert np.abs(o - v.mean(axis=0)).max() < 1e-14
    op, lse = orc.split_partials_rows(q0, k, v, 5, 0.3)
    for s, (a, e) in enumerate(orc.split_bounds(L, 5)):
        assert np.abs(lse[s] - math.log(e - a)).max() < 1e-14
        assert np.abs(op[:, s, :] - v[a:e].mean(axis=0)).max() < 1e-14
    # Zero keys: same as zero query.
    o = orc.attention_rows(rng.standard_normal((2, D)), np.zeros((L, D)), v, 0.3)
    assert np.abs(o - v.mean(axis=0)).max() < 1e-14
    # Two keys: o = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1.
    q = rng.standard_normal((4, D))
    k = rng.standard_normal((2, D))
    v = rng.standard_normal((2, D))
    sc = 0.25
    o = orc.attention_rows(q, k, v, sc)
    for r in range(4):
        s0, s1 = sc * float(q[r] @ k[0]), sc * float(q[r] @ k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.abs(o[r] - (w0 * v[0] + w1 * v[1])).max() < 1e-14
    # A dominant key (score larger by >= 60 than all others) gives its value.
    k = rng.standard_normal((50, D)) * 0.01
    q = np.zeros((1, D)); q[0, 0] = 1.0
    k[17, 0] = 6000.0
    v = rng.standard_normal((50, D))
    o = orc.attention_rows(q, k, v, 0.01)
    # every other key has weight < exp(-59), so only rounding of v[17] remains
    assert np.abs(o[0] - v[17]).max() < 1e-15
    # Scale enters as exp(scale * q.k): scores scaled by 1/2 equal keys halved.
    q = rng.standard_normal((2, D)); k = rng.standard_normal((9, D)); v = rng.standard_normal((9, D))
    assert np.abs(orc.attention_rows(q, k, v, 0.5) - orc.attention_rows(q, 0.5 * k, v, 1.0)).max() < 1e-14


# --------------------------------------------------------------------------
# Decimal brute force
# --------------------------------------------------------------------------
def _decimal_attention(q, k, v, scale):
    """Sum_t exp(s_t) v_t / Sum_t exp(s_t) and ln Sum_t exp(s_t) at 50 digits,
    with no max subtraction (exact arithmetic needs none)."""
    getcontext().prec = 50
    R, D = q.shape
    L = k.shape[0]
    sc = Decimal(repr(float(scale)))
    outs, lses = [], []
    for r in range(R):
        ws = []
        for t in range(L):
            dot = sum(Decimal(repr(float(q[r, d]))) * Decimal(repr(float(k[t, d]))) for d in range(D))
            ws.append((sc * dot).exp())
        tot = sum(ws)
        outs.append([float(sum(ws[t] * Decimal(repr(float(v[t, d]))) for t in range(L)) / tot)
                     for d in range(D)])
        lses.append(float(tot.ln()))
    return np.array(outs), np.array(lses)


def pin_decimal_bruteforce(orc):
    rng = _rng(2)
    for trial in range(6):
        R = int(rng.integers(1, 4))
        L = int(rng.integers(1, 13))
        D = int(rng.integers(1, 5))
        q = rng.standard_normal((R, D)) * 2
        k = rng.standard_normal((L, D)) * 2
        v = rng.standard_normal((L, D))
        scale = float(rng.uniform(0.2, 1.5))
        ref_o, ref_lse = _decimal_attention(q, k, v, scale)
        o = orc.attention_rows(q, k, v, scale)
        assert np.abs(o - ref_o).max() < 1e-13, ("direct", trial)
        for ns in range(1, L + 1):
            op, lse = orc.split_partials_rows(q, k, v, ns, scale)
            for s, (a, e) in enumerate(orc.split_bounds(L, ns)):
                so, sl = _decimal_attention(q, k[a:e], v[a:e], scale)
                assert np.abs(op[:, s, :] - so).max() < 1e-13, ("part", trial, ns, s)
                assert np.abs(lse[s] - sl).max() < 1e-13, ("lse", trial, ns, s)
            om = orc.merge_partials(op, lse)
            assert np.abs(om - ref_o).max() < 1e-13, ("merge", trial, ns)


# --------------------------------------------------------------------------
# library cross-check: torch float64 scaled_dot_product_attention
# --------------------------------------------------------------------------
def _sdpa(q, k, v, scale, group):
    """q [B,H,D], k/v [B,Hkv,L,D] -> [B,H,D] via torch SDPA in float64, with
    K/V head j repeated for query heads j*G..j*G+G-1."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[:, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).repeat_interleave(group, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).repeat_interleave(group, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o[:, :, 0, :].numpy()


def pin_torch_sdpa(orc):
    rng = _rng(3)
    for (B, H, Hkv, D, L, ns) in [(2, 4, 4, 64, 256, 4), (1, 8, 1, 128, 300, 7),
                                  (3, 28, 4, 32, 97, 8), (2, 32, 8, 16, 64, 64)]:
        q = rng.standard_normal((B, H, D))
        kb = rng.standard_normal((B, Hkv, L, D))
        vb = rng.standard_normal((B, Hkv, L, D))
        cu = [b * L for b in range(B + 1)]
        scale = 1.0 / math.sqrt(D)
        ref = _sdpa(q, kb, vb, scale, H // Hkv)
        o_d = orc.attention_direct(q, kb, vb, cu, H, Hkv, scale, layout="bhsd")
        o_s = orc.attention_split_merge(q, kb, vb, cu, H, Hkv, ns, scale, layout="bhsd")
        assert np.abs(o_d - ref).max() < 1e-12, ("direct vs sdpa", B, H, Hkv, D)
        assert np.abs(o_s - ref).max() < 1e-12, ("split vs sdpa", B, H, Hkv, D)
        # Same data in the packed varlen layout [total, Hkv, D].
        kp = kb.transpose(0, 2, 1, 3).reshape(B * L, Hkv, D)
        vp = vb.transpose(0, 2, 1, 3).reshape(B * L, Hkv, D)
        o_p = orc.attention_split_merge(q, kp, vp, cu, H, Hkv, ns, scale, layout="packed")
        assert np.abs(o_p - ref).max() < 1e-12, ("packed vs sdpa", B, H, Hkv, D)
    # Varlen: each packed sequence equals SDPA on that sequence alone.
    lens = [5, 64, 1, 33]
    H, Hkv, D = 6, 2, 16
    q = rng.standard_normal((len(lens), H, D))
    tot = sum(lens)
    kp = rng.standard_normal((tot, Hkv, D)); vp = rng.standard_normal((tot, Hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    o = orc.attention_split_merge(q, kp, vp, cu, H, Hkv, 1, 0.4, layout="packed")
    for b, L in enumerate(lens):
        a = cu[b]
        ks = kp[a:a + L].transpose(1, 0, 2)[None]
        vs = vp[a:a + L].transpose(1, 0, 2)[None]
        ref = _sdpa(q[b:b + 1], ks, vs, 0.4, H // Hkv)
        assert np.abs(o[b:b + 1] - ref).max() < 1e-12, ("varlen seq", b)


# --------------------------------------------------------------------------
# invariant: split + merge equals direct (04_flash_decoding.py, demo 1)
# --------------------------------------------------------------------------
def pin_split_invariant(orc, splits=(1, 7, 64, 1000)):
    """S = 10,000 keys, d = 128, R in {1, 8} packed query rows,
    ns in {1, 7, 64, 1000}: the merged result equals direct attention to
    1e-12 (demo 1 asserts exactness down to 10 keys per split)."""
    rng = np.random.default_rng(0)
    S, d = 10000, 128
    for R in (1, 8):
        q = rng.standard_normal((R, d))
        K, V = rng.standard_normal((S, d)), rng.standard_normal((S, d))
        scale = 1.0 / math.sqrt(d)
        ref = orc.attention_rows(q, K, V, scale)
        for ns in splits:
            op, lse = orc.split_partials_rows(q, K, V, ns, scale)
            o = orc.merge_partials(op, lse)
            assert np.abs(o - ref).max() <= 1e-12, (R, ns, np.abs(o - ref).max())
            # the per-split LSEs must also merge to the direct LSE
            s = scale * (q @ K.T)
            m = s.max(axis=1)
            direct_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            mx = lse.max(axis=0)
            merged = mx + np.log(np.exp(lse - mx).sum(axis=0))
            assert np.abs(merged - direct_lse).max() <= 1e-12


# --------------------------------------------------------------------------
# metamorphic relations
# --------------------------------------------------------------------------
def pin_metamorphic(orc):
    rng = _rng(4)
    # GQA equals MHA with each KV head repeated G times (query head h reads
    # KV head h // G).
    B, H, Hkv, D, L = 2, 12, 3, 8, 40
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B * L, Hkv, D)); v = rng.standard_normal((B * L, Hkv, D))
    cu = [0, L, 2 * L]
    G = H // Hkv
    o_gqa = orc.attention_split_merge(q, k, v, cu, H, Hkv, 3, 0.35)
    o_mha = orc.attention_split_merge(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                      cu, H, H, 3, 0.35)
    assert np.abs(o_gqa - o_mha).max() < 1e-14
    # The KV head for query head h is h // G: moving head h's query to a head
    # of another group changes its result unless the groups' K/V are equal.
    o_alt = orc.attention_direct(q, k, v, cu, H, Hkv, 0.35)
    for h in range(H):
        j = h // G
        ref = orc.attention_rows(q[:, h, :][0:1], k[0:L, j, :], v[0:L, j, :], 0.35)
        assert np.abs(o_alt[0, h] - ref[0]).max() < 1e-14
    # Permuting (k, v) pairs within a sequence leaves the output unchanged.
    perm = rng.permutation(L)
    kp = k.copy(); vp = v.copy()
    kp[0:L] = k[0:L][perm]; vp[0:L] = v[0:L][perm]
    o1 = orc.attention_direct(q, k, v, cu, H, Hkv, 0.35)
    o2 = orc.attention_direct(q, kp, vp, cu, H, Hkv, 0.35)
    assert np.abs(o1 - o2).max() < 1e-14
    # A sequence inside a varlen batch equals the same sequence run alone.
    lens = [3, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    q = rng.standard_normal((3, H, D))
    k = rng.standard_normal((sum(lens), Hkv, D)); v = rng.standard_normal((sum(lens), Hkv, D))
    o = orc.attention_split_merge(q, k, v, cu, H, Hkv, 3, 0.5)
    for b in range(3):
        a, e = cu[b], cu[b + 1]
        ob = orc.attention_split_merge(q[b:b + 1], k[a:e], v[a:e], [0, e - a], H, Hkv, 3, 0.5)
        assert np.abs(o[b] - ob[0]).max() < 1e-14
    # Shifting all scores of a split by a constant (adding c to every key
    # along q) leaves o_s unchanged and shifts lse_s by scale * c * |q|^2-like
    # term: here q = e0 and keys get +c in channel 0.
    qq = np.zeros((1, D)); qq[0, 0] = 1.0
    kk = rng.standard_normal((20, D)); vv = rng.standard_normal((20, D))
    op1, l1 = orc.split_partials_rows(qq, kk, vv, 4, 0.5)
    kk2 = kk.copy(); kk2[:, 0] += 3.0
    op2, l2 = orc.split_partials_rows(qq, kk2, vv, 4, 0.5)
    assert np.abs(op1 - op2).max() < 1e-13
    assert np.abs((l2 - l1) - 1.5).max() < 1e-13


# --------------------------------------------------------------------------
# MiniInfer's format: ceil-equal bounds and unnormalised (m, l, acc) states
# --------------------------------------------------------------------------
def pin_split_bounds_ceil(orc, max_len: int = 120):
    """Ceil-equal bounds (flash_decode_splitk.py, stage-1 kernel), for every
    0 <= L <= max_len and 1 <= ns <= 2L + 2: the non-empty splits come first
    and tile [0, L) in order; all of them but the last have the same size,
    the last at most that size and at least 1 key; that common size is the
    smallest with which ns splits reach L; every later split is (L, L).
    Worked example: L = 10, ns = 6 gives five splits of 2 keys and an empty
    sixth. ns < 1 raises."""
    for L in range(0, max_len + 1):
        for ns in range(1, 2 * L + 3):
            b = orc.split_bounds_ceil(L, ns)
            assert len(b) == ns, (L, ns)
            nonempty = [x for x in b if x[1] > x[0]]
            n = len(nonempty)
            assert b[:n] == nonempty, (L, ns, b)
            assert all(x == (L, L) for x in b[n:]), (L, ns, b)
            pos = 0
            for a, e in nonempty:
                assert a == pos, (L, ns, b)
                pos = e
            assert pos == L, (L, ns, b)
            if n:
                size = nonempty[0][1] - nonempty[0][0]
                assert all(e - a == size for a, e in nonempty[:-1]), (L, ns, b)
                assert 1 <= nonempty[-1][1] - nonempty[-1][0] <= size
                # the smallest size with which ns equal splits cover L
                assert size * ns >= L and (size - 1) * ns < L, (L, ns, size)
    assert orc.split_bounds_ceil(10, 6) == [(0, 2), (2, 4), (4, 6), (6, 8), (8, 10), (10, 10)]
    for bad in (0, -3):
        try:
            orc.split_bounds_ceil(10, bad)
        except ValueError:
            pass
        else:
            raise AssertionError("num_splits < 1 must raise")


def _decimal_states(q, k, v, scale):
    """m = max_t s2_t, l = sum_t 2^(s2_t - m), acc = sum_t 2^(s2_t - m) v_t at
    50 digits, s2_t = scale * q.k_t / ln 2."""
    getcontext().prec = 50
    ln2 = Decimal(2).ln()
    R, D = q.shape
    L = k.shape[0]
    sc = Decimal(repr(float(scale)))
    ms, ls, accs = [], [], []
    for r in range(R):
        s2 = [sc * sum(Decimal(repr(float(q[r, d]))) * Decimal(repr(float(k[t, d])))
                       for d in range(D)) / ln2 for t in range(L)]
        m = max(s2)
        w = [((x - m) * ln2).exp() for x in s2]
        ms.append(float(m))
        ls.append(float(sum(w)))
        accs.append([float(sum(w[t] * Decimal(repr(float(v[t, d]))) for t in range(L)))
                     for d in range(D)])
    return np.array(ms), np.array(ls), np.array(accs)


def pin_states_decimal(orc):
    """Per-split states against a 50-digit brute force on tiny inputs, for
    every split count up to L + 3 (empty tail splits included), and their
    merge against the brute-force direct attention."""
    rng = _rng(5)
    for trial in range(5):
        R = int(rng.integers(1, 4))
        L = int(rng.integers(1, 11))
        D = int(rng.integers(1, 5))
        q = rng.standard_normal((R, D)) * 2
        k = rng.standard_normal((L, D)) * 2
        v = rng.standard_normal((L, D))
        scale = float(rng.uniform(0.2, 1.5))
        ref_o, _ = _decimal_attention(q, k, v, scale)
        for ns in range(1, L + 4):
            m, l, acc = orc.split_states_rows(q, k, v, ns, scale)
            assert m.shape == (ns, R) and l.shape == (ns, R) and acc.shape == (R, ns, D)
            for s, (a, e) in enumerate(orc.split_bounds_ceil(L, ns)):
                if e == a:
                    assert np.all(m[s] == -np.inf) and not l[s].any() and not acc[:, s].any()
                    continue
                dm, dl, dacc = _decimal_states(q, k[a:e], v[a:e], scale)
                assert np.abs(m[s] - dm).max() < 1e-13, ("m", trial, ns, s)
                assert np.abs(l[s] - dl).max() < 1e-13 * max(1.0, dl.max()), ("l", trial, ns, s)
                assert np.abs(acc[:, s] - dacc).max() < 1e-13 * max(1.0, np.abs(dacc).max())
            o = orc.merge_states(m, l, acc)
            assert np.abs(o - ref_o).max() < 1e-13, ("merge", trial, ns)


def pin_states_closed_forms(orc):
    rng = _rng(6)
    D, L = 16, 37
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    # zero query: every s2 is 0, so m_s = 0, l_s = key count, acc_s = sum of V
    m, l, acc = orc.split_states_rows(np.zeros((2, D)), k, v, 5, 0.3)
    for s, (a, e) in enumerate(orc.split_bounds_ceil(L, 5)):
        assert np.all(m[s] == 0.0) and np.all(l[s] == e - a)
        assert np.abs(acc[:, s] - v[a:e].sum(axis=0)).max() < 1e-13
    # one key per split: l = 1, acc = v, m = scale * q.k / ln 2
    q = rng.standard_normal((3, D))
    m, l, acc = orc.split_states_rows(q, k[:4], v[:4], 4, 0.7)
    assert np.all(l == 1.0) and np.array_equal(acc, np.broadcast_to(v[:4], (3, 4, D)))
    assert np.abs(m - 0.7 * (q @ k[:4].T).T / math.log(2.0)).max() < 1e-13
    # the merge does not depend on each split's reference max: (m + c,
    # l * 2^-c, acc * 2^-c) merges to the same output
    m, l, acc = orc.split_states_rows(q, k, v, 6, 0.4)
    c = rng.uniform(-3, 3, size=(6, 1))
    o1 = orc.merge_states(m, l, acc)
    o2 = orc.merge_states(m + c, l * np.exp2(-c), acc * np.exp2(-c).T[:, :, None])
    assert np.abs(o1 - o2).max() < 1e-13
    # a row whose splits are all empty merges to zeros
    z = orc.merge_states(np.full((3, 2), -np.inf), np.zeros((3, 2)), np.zeros((2, 3, D)))
    assert not z.any()


def pin_states_sdpa(orc):
    """Stage 1 + reduce for whole batches against torch float64 SDPA, both
    layouts, GQA, split counts beyond the sequence length (empty splits)."""
    rng = _rng(7)
    for (B, H, Hkv, D, L, ns) in [(2, 4, 4, 64, 256, 4), (1, 8, 1, 128, 300, 7),
                                  (3, 28, 4, 32, 10, 6), (2, 32, 8, 16, 5, 16)]:
        q = rng.standard_normal((B, H, D))
        kb = rng.standard_normal((B, Hkv, L, D))
        vb = rng.standard_normal((B, Hkv, L, D))
        cu = [b * L for b in range(B + 1)]
        scale = 1.0 / math.sqrt(D)
        ref = _sdpa(q, kb, vb, scale, H // Hkv)
        o = orc.attention_split_merge_states(q, kb, vb, cu, H, Hkv, ns, scale, layout="bhsd")
        assert np.abs(o - ref).max() < 1e-12, ("bhsd", B, H, Hkv, D, ns)
        kp = kb.transpose(0, 2, 1, 3).reshape(B * L, Hkv, D)
        vp = vb.transpose(0, 2, 1, 3).reshape(B * L, Hkv, D)
        o = orc.attention_split_merge_states(q, kp, vp, cu, H, Hkv, ns, scale, layout="packed")
        assert np.abs(o - ref).max() < 1e-12, ("packed", B, H, Hkv, D, ns)
        m, l, acc = orc.attention_states(q, kp, vp, cu, H, Hkv, ns, scale)
        assert m.shape == (B, H, ns) and l.shape == (B, H, ns) and acc.shape == (B, H, ns, D)


# --------------------------------------------------------------------------
# whole-batch split partials (the workspace's layout), against the library
# --------------------------------------------------------------------------
def pin_batch_partials(orc):
    """attention_partials on varlen batches whose offsets do not start at 0,
    in both layouts: partial s of head h of sequence b is torch float64 SDPA
    over that sequence's keys [L*s/ns, L*(s+1)/ns) (the bounds of
    decode_attention_splitkv.py), and its LSE, stored at [b, s, h], is
    scipy's logsumexp of the scaled scores over the same keys."""
    from scipy.special import logsumexp
    rng = _rng(11)
    for layout in ("packed", "bhsd"):
        for (H, Hkv, D, lens, ns, off) in [(4, 2, 8, [9, 13, 7], 3, 3), (6, 3, 16, [20, 11], 5, 0),
                                           (8, 1, 4, [6], 6, 2)]:
            B, G = len(lens), H // Hkv
            q = rng.standard_normal((B, H, D))
            scale = 0.3
            cu = [off]
            for L in lens:
                cu.append(cu[-1] + L)
            if layout == "packed":
                kv_k = rng.standard_normal((cu[-1] + 2, Hkv, D))
                kv_v = rng.standard_normal((cu[-1] + 2, Hkv, D))
                cu_arg = cu
                rows = lambda kv, b, j: kv[cu[b]:cu[b + 1], j]
            else:
                S = max(lens) + 1
                kv_k = rng.standard_normal((B, Hkv, S, D))
                kv_v = rng.standard_normal((B, Hkv, S, D))
                cu_arg = [0]
                for L in lens:
                    cu_arg.append(cu_arg[-1] + L)
                rows = lambda kv, b, j: kv[b, j, :lens[b]]
            op, lse = orc.attention_partials(q, kv_k, kv_v, cu_arg, H, Hkv, ns, scale,
                                             layout=layout)
            assert op.shape == (B, H, ns, D) and lse.shape == (B, ns, H)
            for b, L in enumerate(lens):
                for h in range(H):
                    kr, vr = rows(kv_k, b, h // G), rows(kv_v, b, h // G)
                    for s in range(ns):
                        a, e = L * s // ns, L * (s + 1) // ns
                        ref = _sdpa(q[b:b + 1, h:h + 1], kr[None, None, a:e], vr[None, None, a:e],
                                    scale, 1)[0, 0]
                        assert np.abs(op[b, h, s] - ref).max() < 1e-12, (layout, b, h, s)
                        ref_lse = logsumexp(scale * (kr[a:e] @ q[b, h]))
                        assert abs(lse[b, s, h] - ref_lse) < 1e-12, (layout, b, h, s)


def pin_batch_states(orc):
    """attention_states (MiniInfer's format) on varlen batches whose offsets do
    not start at 0, both layouts, split counts past some lengths: over split
    s of flash_decode_splitk.py's ceil-equal bounds (size = ceil(L/ns) keys
    from s*size, cut at L), acc_s / l_s is torch float64 SDPA over the
    split's keys, m_s + log2(l_s) is scipy's logsumexp of the natural scaled
    scores times log2(e), and m_s the largest base-2 scaled score; an empty
    split holds (-inf, 0, 0)."""
    from scipy.special import logsumexp
    rng = _rng(12)
    log2e = 1.0 / math.log(2.0)
    for layout in ("packed", "bhsd"):
        for (H, Hkv, D, lens, ns, off) in [(4, 2, 8, [9, 13, 3], 5, 3), (6, 3, 16, [20, 11], 4, 0),
                                           (8, 1, 4, [6], 8, 2)]:
            B, G = len(lens), H // Hkv
            q = rng.standard_normal((B, H, D))
            scale = 0.3
            cu = [off]
            for L in lens:
                cu.append(cu[-1] + L)
            if layout == "packed":
                kv_k = rng.standard_normal((cu[-1] + 2, Hkv, D))
                kv_v = rng.standard_normal((cu[-1] + 2, Hkv, D))
                cu_arg = cu
                rows = lambda kv, b, j: kv[cu[b]:cu[b + 1], j]
            else:
                S = max(lens) + 1
                kv_k = rng.standard_normal((B, Hkv, S, D))
                kv_v = rng.standard_normal((B, Hkv, S, D))
                cu_arg = [0]
                for L in lens:
                    cu_arg.append(cu_arg[-1] + L)
                rows = lambda kv, b, j: kv[b, j, :lens[b]]
            m, l, acc = orc.attention_states(q, kv_k, kv_v, cu_arg, H, Hkv, ns, scale,
                                             layout=layout)
            assert m.shape == (B, H, ns) and l.shape == (B, H, ns) and acc.shape == (B, H, ns, D)
            for b, L in enumerate(lens):
                size = -(-L // ns)
                for h in range(H):
                    kr, vr = rows(kv_k, b, h // G), rows(kv_v, b, h // G)
                    for s in range(ns):
                        a, e = min(s * size, L), min(s * size + size, L)
                        if e <= a:
                            assert m[b, h, s] == -np.inf and l[b, h, s] == 0, (layout, b, h, s)
                            assert not acc[b, h, s].any(), (layout, b, h, s)
                            continue
                        ref = _sdpa(q[b:b + 1, h:h + 1], kr[None, None, a:e], vr[None, None, a:e],
                                    scale, 1)[0, 0]
                        assert np.abs(acc[b, h, s] / l[b, h, s] - ref).max() < 1e-12, \
                            (layout, b, h, s)
                        x = scale * (kr[a:e] @ q[b, h])
                        assert abs(m[b, h, s] + math.log2(l[b, h, s]) - logsumexp(x) * log2e) \
                            < 1e-12, (layout, b, h, s)
                        assert abs(m[b, h, s] - x.max() * log2e) < 1e-12, (layout, b, h, s)


ALL_PINS = [pin_split_bounds, pin_closed_forms, pin_decimal_bruteforce, pin_torch_sdpa,
            pin_split_invariant, pin_metamorphic, pin_split_bounds_ceil, pin_states_decimal,
            pin_states_closed_forms, pin_states_sdpa, pin_batch_partials, pin_batch_states]
