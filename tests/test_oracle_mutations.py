"""Planted mistakes: each test breaks the oracle in one plausible way (on the
CPU, through monkeypatch) and asserts that the pins of tests/oracle_checks.py
notice. A mutant that survived would mean the pins could not tell a correct
oracle from that broken one."""
from __future__ import annotations

import numpy as np
import pytest

import oracle_checks as C
from oracle import moe_oracle as O

F64 = np.float64


def _silu_wrong_sign(a):
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(a))


def _swiglu_swapped(X, w1, w3, w2):
    return _orig_swiglu(X, w3, w1, w2)


def _swiglu_w2_transposed(X, w1, w3, w2):
    X = np.asarray(X, F64)
    a = X @ np.asarray(O.weight_f32(w1), F64)
    b = X @ np.asarray(O.weight_f32(w3), F64)
    W2 = np.asarray(O.weight_f32(w2), F64)
    W2 = W2.T if W2.shape[0] == W2.shape[1] else W2[::-1]
    return (O.silu(a) * b) @ W2


def _logits_without_bias(x, w_router, bias):
    return np.asarray(x, F64) @ np.asarray(w_router, F64)


def _weights_without_renorm(scores, idx, cfg):
    return np.take_along_axis(scores, idx.astype(np.int64), axis=1) * float(cfg.route_scale)


def _weights_without_scale(scores, idx, cfg):
    w = np.take_along_axis(scores, idx.astype(np.int64), axis=1)
    return w / w.sum(axis=1, keepdims=True) if cfg.renorm else w


def _by_score_high_index_first(ids, score):
    return sorted(ids, key=lambda e: (-score[e], -e))


def _group_score_max(scores_of_group):
    return float(max(scores_of_group))


def _select_ignoring_groups(score, cfg):
    return sorted(range(cfg.E), key=lambda e: (-score[e], e))[: cfg.k]


def _no_shared(inp, cfg, X32):
    return np.zeros((X32.shape[0], cfg.d))


def _identity_as_absent(cfg, e):
    k = _orig_kind(cfg, e)
    return "absent" if k == "identity" else k


def _tables_unstable(idx, E):
    counts, offsets, ss, sp = _orig_tables(idx, E)
    ss = ss.copy()
    for e in range(E):
        ss[offsets[e]:offsets[e + 1]] = ss[offsets[e]:offsets[e + 1]][::-1]
    sp = np.empty_like(ss)
    sp[ss] = np.arange(ss.size, dtype=np.int32)
    return counts, offsets, ss, sp


def _quantise_half_away(v32):
    v32 = np.asarray(v32, np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = v32 / safe[..., None]
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127)
    return np.where(s[..., None] > 0, q, 0).astype(np.int8), s


def _quantise_scale_128(v32):
    v32 = np.asarray(v32, np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    s = (amax / np.float32(128.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(v32 / safe[..., None]), -127, 127)
    return np.where(s[..., None] > 0, q, 0).astype(np.int8), s


def _softmax_without_max_shift_but_wrong_axis(z, gate):
    if gate == "softmax":
        e = np.exp(z)
        return e / e.sum(axis=0, keepdims=True)
    return _orig_scores(z, gate)


def _margins_group_gap_wrong_index(z, scores, cfg):
    """Group gap taken one place too late (between the first and second
    dropped groups instead of the last kept and the first dropped)."""
    mz, mg = _orig_margins(z, scores, cfg)
    if cfg.topk_group and cfg.topk_group + 1 < cfg.n_group:
        gsize = cfg.E // cfg.n_group
        for t in range(z.shape[0]):
            gs = sorted((sum(sorted(scores[t, g * gsize:(g + 1) * gsize], reverse=True)[:2])
                         for g in range(cfg.n_group)), reverse=True)
            mg[t] = gs[cfg.topk_group] - gs[cfg.topk_group + 1]
    return mz, mg


def _margins_moge_ignoring_groups(z, scores, cfg):
    """Per-group quota margin taken over the global k + 1 largest logits, as
    if there were no group boundaries."""
    mz, mg = _orig_margins(z, scores, cfg)
    if cfg.per_group_k:
        for t in range(z.shape[0]):
            v = sorted(z[t], reverse=True)[: cfg.k + 1]
            mz[t] = min(v[i] - v[i + 1] for i in range(len(v) - 1))
    return mz, mg


_orig_swiglu = O.swiglu
_orig_kind = O.expert_kind
_orig_tables = O.routing_tables
_orig_scores = O.gate_scores
_orig_margins = O.selection_margins

MUTANTS = {
    "silu sign flipped": ("silu", _silu_wrong_sign),
    "gate/up projections swapped": ("swiglu", _swiglu_swapped),
    "down projection transposed/reversed": ("swiglu", _swiglu_w2_transposed),
    "router bias dropped": ("router_logits", _logits_without_bias),
    "renormalisation dropped": ("gate_weights", _weights_without_renorm),
    "route_scale ignored": ("gate_weights", _weights_without_scale),
    "ties go to the higher index": ("_by_score", _by_score_high_index_first),
    "group score = group max": ("group_score", _group_score_max),
    "groups and quotas ignored": ("select_token", _select_ignoring_groups),
    "shared expert dropped": ("shared_ffn", _no_shared),
    "identity experts dropped": ("expert_kind", _identity_as_absent),
    "permutation not stable": ("routing_tables", _tables_unstable),
    "int8 rounding half away from zero": ("quantise_rows", _quantise_half_away),
    "int8 scale amax/128": ("quantise_rows", _quantise_scale_128),
    "softmax over the wrong axis": ("gate_scores", _softmax_without_max_shift_but_wrong_axis),
    "group gap taken at the wrong index": ("selection_margins", _margins_group_gap_wrong_index),
    "per-group margin ignores the group boundaries": ("selection_margins", _margins_moge_ignoring_groups),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    try:
        failures = C.all_checks(O)
    except Exception as exc:            # a crash also counts as caught
        failures = [repr(exc)]
    assert failures, f"planted mistake '{mutant}' went unnoticed by every pin"


def test_unmutated_oracle_passes_every_check():
    assert C.all_checks(O) == []
