"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant replaces one function of the oracle module for the duration of
the test (the module's own internal calls see the replacement too) with a
plausible slip: a wrong index, a dropped term, a transposed operand, the
other split rule. The pins in ``oracle_pins`` must reject every one of them;
a mutant that survives would mean the pins cannot tell that slip from the
definition.
"""
import numpy as np
import pytest

import oracle.attention as A
from tests import oracle_pins as pins

_orig = {n: getattr(A, n) for n in ("split_bounds", "kv_rows", "attention_rows",
                                     "split_partials_rows", "merge_partials", "head_pairs",
                                     "split_bounds_ceil", "split_states_rows",
                                     "merge_states", "attention_partials",
                                     "attention_states")}


def _bounds_ceil_equal(seqlen, num_splits):
    # the other split rule (size = ceil(L/ns), start = s*size): can be empty
    size = -(-seqlen // num_splits)
    if num_splits < 1:
        raise ValueError
    return [(min(s * size, seqlen), min(s * size + size, seqlen)) for s in range(num_splits)]


def _bounds_off_by_one(seqlen, num_splits):
    b = _orig["split_bounds"](seqlen, num_splits)
    return [(a, min(e + 1, seqlen)) for a, e in b]


def _heads_modulo(heads, kv_heads):
    # query head h -> KV head h % kv_heads instead of h // G
    g = heads // kv_heads
    return [(j, [h for h in range(heads) if h % kv_heads == j]) for j in range(kv_heads)] if g else []


def _kv_rows_drop_last(kv, cu, b, kvh, layout):
    return _orig["kv_rows"](kv, cu, b, kvh, layout)[:-1] if int(cu[b + 1]) - int(cu[b]) > 1 \
        else _orig["kv_rows"](kv, cu, b, kvh, layout)


def _kv_rows_next_seq(kv, cu, b, kvh, layout):
    # reads the rows one position late (off-by-one varlen base)
    start, end = int(cu[b]) + 1, int(cu[b + 1]) + 1
    if layout == "packed":
        r = kv[start:end, kvh, :]
        if r.shape[0] < end - start:
            r = kv[start - 1:end - 1, kvh, :]
        return np.asarray(r, dtype=np.float64)
    return np.asarray(kv[b, kvh, 1:end - start + 1, :], dtype=np.float64)


def _rows_scale_squared(q, k, v, scale):
    return _orig["attention_rows"](q, k, v, scale * scale)


def _rows_kv_swapped(q, k, v, scale):
    return _orig["attention_rows"](q, v, k, scale)


def _partials_lse_no_max(q, k, v, ns, scale):
    op, lse = _orig["split_partials_rows"](q, k, v, ns, scale)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    for s, (a, e) in enumerate(A.split_bounds(k.shape[0], ns)):
        sc = scale * (q @ k[a:e].T)
        m = sc.max(axis=1)
        lse[s] = lse[s] - m            # forgot to add the max back
    return op, lse


def _partials_unnormalised(q, k, v, ns, scale):
    op, lse = _orig["split_partials_rows"](q, k, v, ns, scale)
    k = np.asarray(k, dtype=np.float64)
    for s, (a, e) in enumerate(A.split_bounds(k.shape[0], ns)):
        op[:, s, :] *= (e - a)         # sum instead of mean-like normalisation
    return op, lse


def _merge_no_normaliser(o_parts, lse):
    lse = np.asarray(lse, dtype=np.float64)
    w = np.exp(lse - lse.max(axis=0))  # weights not divided by their sum
    return np.einsum("sr,rsd->rd", w, np.asarray(o_parts, dtype=np.float64))


def _merge_uniform(o_parts, lse):
    return np.asarray(o_parts, dtype=np.float64).mean(axis=1)


def _merge_weight_by_dim(o_parts, lse):
    # weight indexed by the wrong axis: every row gets row 0's weights
    lse = np.asarray(lse, dtype=np.float64)
    mx = lse.max(axis=0)
    total = mx + np.log(np.exp(lse - mx).sum(axis=0))
    w = np.exp(lse - total)
    w = np.repeat(w[:, :1], w.shape[1], axis=1)
    return np.einsum("sr,rsd->rd", w, np.asarray(o_parts, dtype=np.float64))


def _ceil_bounds_floor_size(seqlen, num_splits):
    # size = floor(L/ns) with the remainder dropped
    if num_splits < 1:
        raise ValueError
    size = seqlen // num_splits
    return [(min(s * size, seqlen), min(s * size + size, seqlen)) for s in range(num_splits)]


def _ceil_bounds_proportional(seqlen, num_splits):
    # the proportional rule where the ceil-equal one is meant
    if num_splits < 1:
        raise ValueError
    return [(seqlen * s // num_splits, seqlen * (s + 1) // num_splits) for s in range(num_splits)]


def _states_natural_exp(q, k, v, ns, scale):
    # weights e^(s2 - m) instead of 2^(s2 - m)
    m, l, acc = _orig["split_states_rows"](q, k, v, ns, scale)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    for s, (a, e) in enumerate(A.split_bounds_ceil(k.shape[0], ns)):
        if e > a:
            s2 = scale / np.log(2.0) * (q @ k[a:e].T)
            p = np.exp(s2 - s2.max(axis=1, keepdims=True))
            l[s] = p.sum(axis=1)
            acc[:, s, :] = p @ v[a:e]
    return m, l, acc


def _states_normalised(q, k, v, ns, scale):
    # acc divided by l already (the other format's o_s)
    m, l, acc = _orig["split_states_rows"](q, k, v, ns, scale)
    with np.errstate(invalid="ignore", divide="ignore"):
        acc = np.where(l.T[:, :, None] > 0, acc / l.T[:, :, None], 0.0)
    return m, l, acc


def _states_natural_max(q, k, v, ns, scale):
    # m kept in natural-log units while the weights use base 2
    m, l, acc = _orig["split_states_rows"](q, k, v, ns, scale)
    return m * np.log(2.0), l, acc


def _merge_states_no_alpha_on_l(m, l, acc):
    m = np.asarray(m); l = np.asarray(l); acc = np.asarray(acc)
    out = np.zeros((m.shape[1], acc.shape[2]))
    for r in range(m.shape[1]):
        M = m[:, r].max()
        if M == -np.inf:
            continue
        alpha = np.exp2(m[:, r] - M)
        out[r] = (alpha @ acc[r]) / l[:, r].sum()
    return out


def _merge_states_sum_acc(m, l, acc):
    m = np.asarray(m); l = np.asarray(l); acc = np.asarray(acc)
    out = np.zeros((m.shape[1], acc.shape[2]))
    for r in range(m.shape[1]):
        if m[:, r].max() == -np.inf:
            continue
        out[r] = acc[r].sum(axis=0) / l[:, r].sum()
    return out


def _batch_partials_splits_reversed(q, k, v, cu, heads, kv_heads, ns, scale, layout="packed",
                                    pairs=None):
    # partials and LSEs stored in reverse split order: every merge stays exact,
    # only the per-split layout the workspace is compared against is wrong
    op, lse = _orig["attention_partials"](q, k, v, cu, heads, kv_heads, ns, scale, layout, pairs)
    return op[:, :, ::-1, :], lse[:, ::-1, :]


def _batch_states_splits_reversed(q, k, v, cu, heads, kv_heads, ns, scale, layout="packed",
                                  pairs=None):
    # (m, l, acc) stored in reverse split order: every merge stays exact
    m, l, acc = _orig["attention_states"](q, k, v, cu, heads, kv_heads, ns, scale, layout, pairs)
    return m[:, :, ::-1], l[:, :, ::-1], acc[:, :, ::-1, :]


MUTANTS = {
    "batch_partials_splits_reversed": ("attention_partials", _batch_partials_splits_reversed),
    "batch_states_splits_reversed": ("attention_states", _batch_states_splits_reversed),
    "ceil_bounds_floor_size": ("split_bounds_ceil", _ceil_bounds_floor_size),
    "ceil_bounds_proportional": ("split_bounds_ceil", _ceil_bounds_proportional),
    "states_natural_exp": ("split_states_rows", _states_natural_exp),
    "states_normalised": ("split_states_rows", _states_normalised),
    "states_natural_max": ("split_states_rows", _states_natural_max),
    "merge_states_no_alpha_on_l": ("merge_states", _merge_states_no_alpha_on_l),
    "merge_states_sum_acc": ("merge_states", _merge_states_sum_acc),
    "bounds_ceil_equal": ("split_bounds", _bounds_ceil_equal),
    "bounds_off_by_one": ("split_bounds", _bounds_off_by_one),
    "heads_modulo": ("head_pairs", _heads_modulo),
    "kv_rows_drop_last": ("kv_rows", _kv_rows_drop_last),
    "kv_rows_shifted": ("kv_rows", _kv_rows_next_seq),
    "scale_squared": ("attention_rows", _rows_scale_squared),
    "kv_swapped": ("attention_rows", _rows_kv_swapped),
    "lse_no_max": ("split_partials_rows", _partials_lse_no_max),
    "partials_unnormalised": ("split_partials_rows", _partials_unnormalised),
    "merge_no_normaliser": ("merge_partials", _merge_no_normaliser),
    "merge_uniform": ("merge_partials", _merge_uniform),
    "merge_weight_wrong_row": ("merge_partials", _merge_weight_by_dim),
}

# cheapest pins first; the test stops at the first one that rejects the mutant
_ORDER = [pins.pin_closed_forms, pins.pin_metamorphic, pins.pin_split_bounds,
          pins.pin_split_bounds_ceil, pins.pin_states_closed_forms, pins.pin_torch_sdpa,
          pins.pin_states_sdpa, pins.pin_decimal_bruteforce, pins.pin_states_decimal,
          pins.pin_split_invariant, pins.pin_batch_partials, pins.pin_batch_states]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    for pin in _ORDER:
        try:
            pin(A)
        except Exception:
            return
    pytest.fail(f"mutant {name} passed every pin")
