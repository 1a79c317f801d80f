"""Host logic of the launch-limit table (tuning.py), on the CPU: the choice
of the fastest candidate from timed runs, the table's JSON round trip, the
load bucket and the key. No call reaches a GPU."""
from __future__ import annotations

import numpy as np
import pytest


@pytest.fixture(scope="module")
def TU():
    from moe_expert_layer_fp32_amd import tuning
    return tuning


def test_fastest_candidate_is_kept(TU, tmp_path):
    # each candidate's calls cost a known time on a simulated clock; (128, 128)
    # is the cheapest
    cost = {(0, 0): 3e-4, (96, 0): 2e-4, (128, 0): 2e-4, (192, 0): 4e-4, (128, 128): 5e-5, (192, 192): 1e-4}
    calls = []
    now = [0.0]

    def run(t, i):
        key = (0, 0) if t is None else (t.shared_ffn1_wgs, t.shared_ffn2_wgs)
        calls.append(key)
        now[0] += cost[key]

    cache = TU.TilingCache()
    best = cache.tune("k", run, lambda: None, calls=4, reps=2, clock=lambda: now[0])
    assert best == TU.limits(128, 128)
    assert cache.lookup("k") == best
    # every candidate ran (3 warm-up + 4 timed calls per round, 2 rounds)
    assert {c: calls.count(c) for c in cost} == {c: 14 for c in cost}
    assert cache.table["k"]["us"] == {TU.label(TU.limits(*c)): round(v * 1e6, 2) for c, v in cost.items()}
    p = tmp_path / "limits.json"
    cache.save(str(p))
    again = TU.TilingCache.load(str(p))
    assert again.lookup("k") == best and again.lookup("other") is None


def test_library_choice_is_no_struct(TU):
    assert TU.to_struct(None) is None
    assert TU.to_struct(TU.limits()) is None
    t = TU.to_struct(TU.limits(96, 0, 8, 0))
    assert (t.shared_ffn1_wgs, t.shared_ffn2_wgs, t.routed_ffn1_wgs, t.routed_ffn2_wgs) == (96, 0, 8, 0)
    assert TU.label(TU.limits(96, 0, 8, 0)) == "96/0/8/0/0/0/0/0"


def test_load_bucket_and_key(TU):
    from moe_expert_layer_fp32_amd import lib as L
    counts = np.array([0, 5, 64, 3, 200, 1])
    # resident experts 1..3: largest count 64 -> ceil(log2(65)) = 7
    assert TU.load_bucket(counts, 1, 3) == 7
    assert TU.load_bucket(counts, 0, 1) == 0
    assert TU.load_bucket(counts, 4, 1) == 8
    d = L.MoeDesc(T=512, d=7168, E=256, k=8)
    k1, k2 = TU.shape_key(d, 2, 5), TU.shape_key(d, 2, 6)
    assert k1 != k2 and "T=512" in k1 and "streams=2" in k1
    assert TU.shape_key(L.MoeDesc(T=256, d=7168, E=256, k=8), 2, 5) != k1
