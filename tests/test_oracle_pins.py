"""Pins of the CPU oracle: hand-worked cases, pure-Python brute force, library
routines, closed forms and invariants. CPU only."""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special as sps
import torch

import golden_cases as G
import oracle_checks as C
from moe_inputs.configs import MoEConfig
from oracle import moe_oracle as O


@pytest.mark.parametrize("name", G.LAYER_CASES)
def test_golden_layer(name):
    assert C.check_golden_layer(O, name) == []


def test_golden_int8_rows():
    assert C.check_golden_int8(O) == []


def test_golden_w8a8_parts():
    assert C.check_golden_w8a8_parts(O) == []


def test_brute_force_dense_mixture():
    assert C.check_brute_force(O, seeds=range(120)) == []


def test_selection_margins_hand_worked():
    """Group-limited, per-group-quota and plain margins against hand-worked values."""
    assert C.check_selection_margins(O) == []


def test_routing_tables_vs_stable_argsort():
    assert C.check_routing_tables(O, seeds=range(60)) == []


def test_topk_vs_stable_argsort():
    rng = np.random.default_rng(3)
    for trial in range(50):
        E = int(rng.integers(2, 300)); k = int(rng.integers(1, min(E, 16) + 1))
        cfg = MoEConfig(name="t", T=4, d=1, E=E, k=k, gate="softmax")
        s = np.round(rng.random((4, E)), 2)          # coarse values -> many exact ties
        got = O.select_experts(s, cfg)
        want = np.argsort(-s, axis=1, kind="stable")[:, :k]
        assert np.array_equal(got, want)


def test_gate_scores_vs_scipy():
    z = np.random.default_rng(0).standard_normal((7, 33)) * 5
    assert np.allclose(O.gate_scores(z, "softmax"), sps.softmax(z, axis=1), rtol=1e-14)
    assert np.allclose(O.gate_scores(z, "sigmoid"), sps.expit(z), rtol=1e-14)


def _torch_swiglu(x, w1, w3, w2):
    x, w1, w3, w2 = (torch.as_tensor(np.asarray(a, np.float64)) for a in (x, w1, w3, w2))
    return (torch.nn.functional.silu(x @ w1) * (x @ w3) @ w2).numpy()


def test_single_expert_is_swiglu():
    """E = 1, k = 1: the layer reduces to one SwiGLU FFN (torch CPU fp64)."""
    rng = np.random.default_rng(1)
    cfg = MoEConfig(name="e1", T=9, d=16, E=1, k=1, gate="softmax", n_ffn=1, inter=24, dtype="f32")
    inp = {"x": rng.standard_normal((9, 16)), "w_router": rng.standard_normal((16, 1)), "bias": None,
           "w1": rng.standard_normal((1, 16, 24)), "w3": rng.standard_normal((1, 16, 24)),
           "w2": rng.standard_normal((1, 24, 16))}
    y = O.moe_layer(inp, cfg)["y"]
    assert np.allclose(y, _torch_swiglu(inp["x"], inp["w1"][0], inp["w3"][0], inp["w2"][0]),
                       rtol=1e-12, atol=1e-12)


def test_full_softmax_mixture():
    """k = E with softmax and renorm: the dense softmax mixture of all experts."""
    rng = np.random.default_rng(2)
    E, d, I = 5, 8, 6
    cfg = MoEConfig(name="kE", T=6, d=d, E=E, k=E, gate="softmax", n_ffn=E, inter=I, dtype="f32")
    inp = {"x": rng.standard_normal((6, d)), "w_router": rng.standard_normal((d, E)),
           "bias": rng.standard_normal(E), "w1": rng.standard_normal((E, d, I)),
           "w3": rng.standard_normal((E, d, I)), "w2": rng.standard_normal((E, I, d))}
    p = sps.softmax(inp["x"] @ inp["w_router"] + inp["bias"], axis=1)
    want = sum(p[:, [e]] * _torch_swiglu(inp["x"], inp["w1"][e], inp["w3"][e], inp["w2"][e])
               for e in range(E))
    assert np.allclose(O.moe_layer(inp, cfg)["y"], want, rtol=1e-12, atol=1e-12)


def test_all_identity_returns_scaled_input():
    rng = np.random.default_rng(4)
    for gate in ("softmax", "sigmoid"):
        cfg = MoEConfig(name="id", T=11, d=12, E=10, k=4, gate=gate, zero_begin=0, n_zero=10,
                        route_scale=1.75, dtype="f32")
        inp = {"x": rng.standard_normal((11, 12)), "w_router": rng.standard_normal((12, 10)),
               "bias": None}
        assert np.allclose(O.moe_layer(inp, cfg)["y"], 1.75 * inp["x"], rtol=1e-13)


def test_no_resident_expert_gives_shared_only():
    rng = np.random.default_rng(5)
    cfg = MoEConfig(name="ns", T=7, d=10, E=16, k=3, gate="sigmoid", ffn_begin=0, n_ffn=0,
                    shared_inter=8, dtype="f32")
    inp = {"x": rng.standard_normal((7, 10)), "w_router": rng.standard_normal((10, 16)),
           "bias": None, "sw1": rng.standard_normal((10, 8)), "sw3": rng.standard_normal((10, 8)),
           "sw2": rng.standard_normal((8, 10))}
    want = _torch_swiglu(inp["x"], inp["sw1"], inp["sw3"], inp["sw2"])
    assert np.allclose(O.moe_layer(inp, cfg)["y"], want, rtol=1e-12, atol=1e-12)


def test_selection_invariants_on_workload_routers():
    """Distinct in-range ids, weights summing to 1, one expert per group (MoGE),
    at most topk_group groups touched (group-limited), on each workload's router."""
    from moe_inputs import CONFIGS, make_inputs
    for cfg in CONFIGS.values():
        small = cfg.replace(T=min(cfg.T, 96), n_ffn=0, zero_begin=0, n_zero=0, shared_inter=0)
        inp = make_inputs(small)
        z, s, idx, w = O.route(inp, small)
        assert idx.min() >= 0 and idx.max() < cfg.E
        assert all(len(set(row)) == cfg.k for row in idx.tolist())
        assert np.allclose(w.sum(axis=1), cfg.route_scale, rtol=0, atol=4e-16)
        assert np.all(w > 0)
        gsz = cfg.E // cfg.n_group
        if cfg.per_group_k:
            assert all(sorted(set(e // gsz for e in row)) == list(range(cfg.n_group))
                       for row in idx.tolist())
        if cfg.topk_group:
            assert all(len(set(e // gsz for e in row)) <= cfg.topk_group for row in idx.tolist())
        # slots ordered by descending score
        sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
        assert np.all(np.diff(sel, axis=1) <= 0)


def test_quantise_rows_properties():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((50, 300)) * rng.random((50, 1)) * 10).astype(np.float32)
    v[3] = 0
    q, s = O.quantise_rows(v)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    assert np.all(q[3] == 0) and s[3] == 0
    err = np.abs(v.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    amax_pos = np.argmax(np.abs(v), axis=1)
    rows = np.arange(50) != 3
    assert np.all(np.abs(q[rows, amax_pos[rows]]) == 127)


def test_int_matmul_exact_vs_python_ints():
    rng = np.random.default_rng(7)
    a = rng.integers(-127, 128, (5, 300)).astype(np.int8)
    b = rng.integers(-127, 128, (300, 4)).astype(np.int8)
    got = O.int_matmul(a, b)
    want = [[sum(int(a[i, r]) * int(b[r, j]) for r in range(300)) for j in range(4)] for i in range(5)]
    assert got.tolist() == want


def test_w8a8_close_to_float_ffn_on_dequantised_weights():
    """The W8A8 FFN approximates the float FFN with the dequantised weights to
    within int8 activation-rounding error (a consistency check, not parity)."""
    rng = np.random.default_rng(8)
    d, I = 256, 128
    q1, s1 = C.quantised_weight(rng, d, I)
    q3, s3 = C.quantised_weight(rng, d, I)
    q2, s2 = C.quantised_weight(rng, I, d)
    x = rng.standard_normal((6, d)).astype(np.float32)
    u = O.swiglu_w8a8(x, q1, s1, q3, s3, q2, s2)
    deq = lambda q, s: q.astype(np.float64) * s[None, :].astype(np.float64)
    ref = O.swiglu(x, deq(q1, s1), deq(q3, s3), deq(q2, s2))
    rms = np.sqrt((ref ** 2).mean())
    assert np.sqrt(((u - ref) ** 2).mean()) / rms < 0.03      # int8 rounding noise, about 1%
    assert np.abs(u - ref).max() / rms < 0.15


def test_selection_margin_is_zero_on_exact_ties():
    cfg = MoEConfig(name="m", T=1, d=1, E=4, k=2, gate="softmax")
    z = np.array([[0.5, 0.2, 0.2, 0.1]])
    mz, _ = O.selection_margins(z, O.gate_scores(z, "softmax"), cfg)
    assert mz[0] == 0.0
    z = np.array([[0.5, 0.3, 0.2, 0.1]])
    mz, _ = O.selection_margins(z, O.gate_scores(z, "softmax"), cfg)
    assert np.isclose(mz[0], 0.1)


def test_selection_margin_of_a_lone_candidate_is_infinite():
    """One expert (E = 1), or groups of one expert with a quota of one: no
    other candidate, so no order or swap can be decided by rounding."""
    z = np.array([[0.7], [-2.0]])
    mz, mg = O.selection_margins(z, O.gate_scores(z, "softmax"), MoEConfig(name="m", T=2, d=1, E=1, k=1,
                                                                           gate="softmax"))
    assert np.all(np.isinf(mz)) and np.all(np.isinf(mg))
    z = np.array([[0.3, 0.9, 0.1]])
    cfg = MoEConfig(name="m", T=1, d=1, E=3, k=3, gate="sigmoid", n_group=3, per_group_k=1)
    mz, _ = O.selection_margins(z, O.gate_scores(z, "sigmoid"), cfg)
    # only the final order of the three chosen remains: 0.9 - 0.3 and 0.3 - 0.1
    assert np.isclose(mz[0], 0.2)


def test_group_margin_when_every_group_is_kept():
    """topk_group == n_group keeps every group: no group is dropped, so the
    group gap is +inf, and selection reduces to plain top-k (same ids as with
    one group)."""
    z = np.array([[0.9, -0.2, 0.4, 0.1, 0.3, -0.5]])
    s = O.gate_scores(z, "sigmoid")
    cfg = MoEConfig(name="m", T=1, d=1, E=6, k=3, gate="sigmoid", n_group=3, topk_group=3)
    mz, mg = O.selection_margins(z, s, cfg)
    assert np.isinf(mg[0]) and np.isclose(mz[0], 0.1)   # 0.9, 0.4, 0.3 | 0.1: smallest gap 0.4 - 0.3
    plain = MoEConfig(name="m", T=1, d=1, E=6, k=3, gate="sigmoid")
    assert O.select_experts(s, cfg).tolist() == O.select_experts(s, plain).tolist() == [[0, 2, 4]]


def test_round_output_bf16_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0 - 2 ** -7, 1e-3])
    got = O.round_output(vals, "bf16")
    assert got.tolist()[:4] == [1.0, 1.0, 1.0 + 2 ** -6, -3.0]
    assert abs(got[4] - 1e-3) <= 2 ** -9 * 1e-3
