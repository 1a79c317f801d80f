"""Independent checks that pin the CPU oracle (used by the oracle pin tests and
by the planted-mistake tests, which rerun them against a deliberately broken
oracle and expect at least one to fail).

Nothing here calls into the oracle's helpers: the brute force below is its own
pure-Python implementation, written as a dense mixture (every expert evaluated
for every token, a gate vector that is zero off the selection) with selection
by rank counting instead of sorting.
"""
from __future__ import annotations

import math

import numpy as np

from moe_inputs.configs import MoEConfig
from moe_inputs.gen import quantise_weight_int8

import golden_cases as G


# ----------------------------------------------------------------------------
# pure-Python dense-mixture brute force (float cases only)
# ----------------------------------------------------------------------------
def _lt_rank(vals, i, ids):
    """Rank of i among ids under (descending value, ascending id)."""
    return sum(1 for j in ids if vals[j] > vals[i] or (vals[j] == vals[i] and j < i))


def _gate_vector(score, cfg):
    E, k = cfg.E, cfg.k
    gs = E // cfg.n_group
    g_of = [e // gs for e in range(E)]
    chosen = []
    if cfg.per_group_k:
        for e in range(E):
            members = [m for m in range(E) if g_of[m] == g_of[e]]
            if _lt_rank(score, e, members) < cfg.per_group_k:
                chosen.append(e)
    else:
        allowed = list(range(E))
        if cfg.topk_group:
            gscore = []
            for g in range(cfg.n_group):
                first = second = -math.inf
                for e in range(g * gs, (g + 1) * gs):
                    v = score[e]
                    if v > first:
                        first, second = v, first
                    elif v > second:
                        second = v
                gscore.append(first + second)
            keep = [g for g in range(cfg.n_group)
                    if _lt_rank(gscore, g, range(cfg.n_group)) < cfg.topk_group]
            allowed = [e for e in range(E) if g_of[e] in keep]
        chosen = [e for e in allowed if _lt_rank(score, e, allowed) < k]
    total = sum(score[e] for e in chosen)
    gate = [0.0] * E
    for e in chosen:
        gate[e] = (score[e] / total if cfg.renorm else score[e]) * cfg.route_scale
    order = sorted(chosen, key=lambda e: _lt_rank(score, e, chosen))
    return gate, order


def _ffn(xrow, W1, W3, W2):
    d, I = len(W1), len(W1[0])
    h = []
    for i in range(I):
        a = sum(xrow[r] * W1[r][i] for r in range(d))
        b = sum(xrow[r] * W3[r][i] for r in range(d))
        h.append(a / (1.0 + math.exp(-a)) * b if a > -700 else 0.0)
    return [sum(h[i] * W2[i][c] for i in range(I)) for c in range(len(W2[0]))]


def brute_force(inp, cfg):
    """Returns (idx list per token, gate vectors, y) by explicit loops."""
    as_list = lambda a: np.asarray(a, dtype=np.float64).tolist()
    X = as_list(G_x(inp))
    Wr = as_list(inp["w_router"])
    b = as_list(inp["bias"]) if inp.get("bias") is not None else [0.0] * cfg.E
    ys, idxs, gates = [], [], []
    for x in X:
        z = [sum(x[i] * Wr[i][e] for i in range(cfg.d)) + b[e] for e in range(cfg.E)]
        if cfg.gate == "softmax":
            m = max(z)
            ex = [math.exp(v - m) for v in z]
            s = [v / sum(ex) for v in ex]
        else:
            s = [1.0 / (1.0 + math.exp(-v)) for v in z]
        gate, order = _gate_vector(s, cfg)
        y = [0.0] * cfg.d
        if cfg.shared_inter:
            y = _ffn(x, as_list(inp["sw1"]), as_list(inp["sw3"]), as_list(inp["sw2"]))
        for e in range(cfg.E):
            if cfg.ffn_begin <= e < cfg.ffn_begin + cfg.n_ffn:
                el = e - cfg.ffn_begin
                u = _ffn(x, as_list(inp["w1"][el]), as_list(inp["w3"][el]), as_list(inp["w2"][el]))
            elif cfg.zero_begin <= e < cfg.zero_begin + cfg.n_zero:
                u = list(x)
            else:
                u = [0.0] * cfg.d
            y = [y[c] + gate[e] * u[c] for c in range(cfg.d)]
        ys.append(y)
        idxs.append(order)
        gates.append(gate)
    return idxs, gates, np.asarray(ys)


def G_x(inp):
    from moe_inputs.gen import x_f32
    return x_f32(inp)


def random_tiny_case(seed: int):
    """A random tiny float layer covering every routing mode in turn."""
    rng = np.random.default_rng(seed)
    mode = seed % 4
    d = int(rng.integers(2, 7))
    I = int(rng.integers(1, 5))
    if mode == 0:       # plain softmax
        E = int(rng.integers(2, 9)); k = int(rng.integers(1, E + 1))
        kw = dict(gate="softmax")
    elif mode == 1:     # plain sigmoid
        E = int(rng.integers(2, 9)); k = int(rng.integers(1, E + 1))
        kw = dict(gate="sigmoid")
    elif mode == 2:     # group-limited sigmoid
        G = int(rng.integers(2, 5)); gs = int(rng.integers(2, 4)); E = G * gs
        tg = int(rng.integers(1, G + 1)); k = int(rng.integers(1, tg * gs + 1))
        kw = dict(gate="sigmoid", n_group=G, topk_group=tg)
    else:               # per-group quota
        G = int(rng.integers(2, 5)); gs = int(rng.integers(1, 4)); E = G * gs
        pg = int(rng.integers(1, gs + 1)); k = G * pg
        kw = dict(gate=str(rng.choice(["softmax", "sigmoid"])), n_group=G, per_group_k=pg)
    n_ffn = int(rng.integers(0, E + 1))
    n_zero = int(rng.integers(0, E - n_ffn + 1))
    shared = int(rng.integers(0, 2)) * int(rng.integers(1, 4))
    cfg = MoEConfig(name=f"tiny{seed}", T=int(rng.integers(1, 5)), d=d, E=E, k=k,
                    renorm=bool(rng.integers(0, 2)), route_scale=float(rng.choice([1.0, 2.5])),
                    ffn_begin=0, n_ffn=n_ffn, zero_begin=n_ffn, n_zero=n_zero, inter=I,
                    shared_inter=shared, dtype="f32", **kw)
    cfg.check()
    inp = {"cfg": cfg, "x": rng.standard_normal((cfg.T, d)),
           "w_router": rng.standard_normal((d, E)),
           "bias": rng.standard_normal(E) if rng.integers(0, 2) else None}
    if rng.integers(0, 3) == 0:          # force exact score ties through duplicated router columns
        j = int(rng.integers(0, E)); jj = int(rng.integers(0, E))
        inp["w_router"][:, jj] = inp["w_router"][:, j]
        if inp["bias"] is not None:
            inp["bias"][jj] = inp["bias"][j]
    if n_ffn:
        inp["w1"] = rng.standard_normal((n_ffn, d, I))
        inp["w3"] = rng.standard_normal((n_ffn, d, I))
        inp["w2"] = rng.standard_normal((n_ffn, I, d))
    if shared:
        inp["sw1"] = rng.standard_normal((d, shared))
        inp["sw3"] = rng.standard_normal((d, shared))
        inp["sw2"] = rng.standard_normal((shared, d))
    return cfg, inp


# ----------------------------------------------------------------------------
# checks, each returning a list of failure messages (empty = pass)
# ----------------------------------------------------------------------------
def check_golden_layer(O, name):
    cfg, inp, exp = G.layer_case(name)
    r = O.moe_layer(inp, cfg)
    bad = []
    if r["idx"].tolist() != exp["idx"]:
        bad.append(f"{name}: idx {r['idx'].tolist()} != {exp['idx']}")
    for key in ("w", "scores", "y"):
        want = G.array(exp[key])
        got = np.asarray(r[key], np.float64)
        if got.shape != want.shape or not np.allclose(got, want, rtol=1e-9, atol=1e-12):
            bad.append(f"{name}: {key} {got.tolist()} != {want.tolist()}")
    return bad


def check_golden_int8(O):
    raw = G.load("int8_rows.json")
    q, s = O.quantise_rows(np.asarray(raw["rows"], np.float32))
    bad = []
    if q.tolist() != raw["expected"]["q"]:
        bad.append(f"int8 q {q.tolist()}")
    if s.tolist() != [float(v) for v in raw["expected"]["s"]]:
        bad.append(f"int8 s {s.tolist()}")
    return bad


def check_golden_w8a8_parts(O):
    cfg, inp, exp = G.layer_case("w8a8_ffn.json")
    u, parts = O.swiglu_w8a8(O.x_f32(inp).astype(np.float32), inp["w1"][0], inp["s1"][0],
                             inp["w3"][0], inp["s3"][0], inp["w2"][0], inp["s2"][0],
                             return_parts=True)
    bad = []
    for key in ("qx", "sx", "A", "B", "qh", "sh", "Y"):
        want = G.array(exp[key])
        got = np.asarray(parts[key], np.float64)
        if got.shape != want.shape or not np.array_equal(got, want):
            bad.append(f"w8a8 {key}: {got.tolist()} != {want.tolist()}")
    if not np.allclose(u, G.array(exp["y"]), rtol=1e-12):
        bad.append(f"w8a8 u {u.tolist()}")
    return bad


def check_brute_force(O, seeds=range(40)):
    bad = []
    for seed in seeds:
        cfg, inp = random_tiny_case(seed)
        idx_bf, gate_bf, y_bf = brute_force(inp, cfg)
        r = O.moe_layer(inp, cfg)
        if r["idx"].tolist() != idx_bf:
            bad.append(f"seed {seed}: idx {r['idx'].tolist()} != {idx_bf}")
            continue
        g = np.zeros((cfg.T, cfg.E))
        np.put_along_axis(g, r["idx"].astype(np.int64), r["w"], axis=1)
        if not np.allclose(g, np.asarray(gate_bf), rtol=1e-12, atol=1e-15):
            bad.append(f"seed {seed}: gate weights differ")
        if not np.allclose(r["y"], y_bf, rtol=1e-10, atol=1e-12):
            bad.append(f"seed {seed}: y max err {np.abs(r['y'] - y_bf).max()}")
    return bad


def check_routing_tables(O, seeds=range(20)):
    bad = []
    for seed in seeds:
        rng = np.random.default_rng(seed)
        T, E = int(rng.integers(1, 50)), int(rng.integers(1, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, ss, sp = O.routing_tables(idx, E)
        flat = idx.reshape(-1)
        if counts.tolist() != np.bincount(flat, minlength=E).tolist():
            bad.append(f"seed {seed}: counts")
        if offsets.tolist() != [0] + np.cumsum(np.bincount(flat, minlength=E)).tolist():
            bad.append(f"seed {seed}: offsets")
        if ss.tolist() != np.argsort(flat, kind="stable").tolist():
            bad.append(f"seed {seed}: sorted_slot")
        if not np.array_equal(sp[ss], np.arange(flat.size)):
            bad.append(f"seed {seed}: slot_pos is not the inverse")
    return bad


def all_checks(O):
    bad = []
    for name in G.LAYER_CASES:
        bad += check_golden_layer(O, name)
    bad += check_golden_int8(O)
    bad += check_golden_w8a8_parts(O)
    bad += check_brute_force(O)
    bad += check_routing_tables(O)
    bad += check_selection_margins(O)
    return bad


def quantised_weight(rng, K, N):
    """int8 weight + per-column scale of a random [K, N] fp32 matrix."""
    return quantise_weight_int8(rng.standard_normal((K, N)).astype(np.float32) * np.float32(0.02))


def check_selection_margins(O):
    """Hand-worked margins (tests/golden/selection_margins.json) of the plain,
    group-limited and per-group-quota rules; scores are taken from the
    library's softmax / logistic functions (scipy), not from the oracle."""
    import scipy.special as sps
    raw = G.load("selection_margins.json")
    bad = []
    for case in raw["cases"]:
        cfg = MoEConfig(**case["cfg"])
        cfg.check()
        z = np.asarray(case["z"], np.float64)
        s = sps.softmax(z, axis=1) if cfg.gate == "softmax" else sps.expit(z)
        mz, mg = O.selection_margins(z, s, cfg)
        want_z = np.asarray(G.value(case["expected"]["mz"]), np.float64)
        want_g = np.asarray([np.inf if v is None else G.value(v) for v in case["expected"]["mg"]], np.float64)
        if mz.shape != want_z.shape or not np.allclose(mz, want_z, rtol=1e-12, atol=1e-15):
            bad.append(f"margins {cfg.name}: mz {mz.tolist()} != {want_z.tolist()}")
        if mg.shape != want_g.shape or not np.allclose(mg, want_g, rtol=1e-12, atol=1e-15):
            bad.append(f"margins {cfg.name}: mg {mg.tolist()} != {want_g.tolist()}")
    return bad
