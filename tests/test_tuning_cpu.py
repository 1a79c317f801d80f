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
    assert TU.label(TU.limits(96, 0, 8, 0)) == "96/0/8/0/0/0/0/0/0"
    t = TU.to_struct(TU.limits(decode_tile_rows=32))
    assert t.decode_tile_rows == 32 and TU.label(TU.limits(decode_tile_rows=32)) == "0/0/0/0/0/0/0/0/32"


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


def test_candidates_by_regime(TU):
    """Decode shapes: the shared caps and the per-expert tile classes applied
    early; prefill shapes: caps of the shared and routed products crossed
    with 256-row routed tiles on and off. The library's own choice is always
    a candidate, and every candidate is a valid moe_tuning."""
    from moe_expert_layer_fp32_amd import lib as L
    from moe_inputs import get
    dec = L.desc_from_config(get("dsv3_decode_share_bf16"))
    pre = L.desc_from_config(get("prefill_zipf_bf16"))
    for d, streams in ((dec, 2), (dec, 1), (pre, 2), (pre, 1)):
        cands = TU.candidates_for(d, streams)
        assert TU.limits() in cands
        assert len({TU.label(c) for c in cands}) == len(cands)
        for c in cands:
            assert set(c) == set(TU.FIELDS) and all(v >= 0 for v in c.values())
            TU.to_struct(c)
    assert any(c["prefill_tokens"] == dec.T for c in TU.candidates_for(dec, 2))
    assert any(c["decode_tile_rows"] == 32 for c in TU.candidates_for(dec, 2))
    assert not any(c["decode_tile_rows"] for c in TU.candidates_for(pre, 2))
    pre2 = TU.candidates_for(pre, 2)
    assert any(c["big_min_rows"] == TU.NO_BIG for c in pre2)
    assert any(c["routed_ffn1_wgs"] > 0 for c in pre2) and any(c["shared_ffn1_wgs"] > 0 for c in pre2)
    assert not any(c["shared_ffn1_wgs"] or c["routed_ffn1_wgs"] for c in TU.candidates_for(pre, 1))


def test_merge_into_and_shipped_table(TU, tmp_path):
    """Entries merged into a JSON table keep the others; the shipped table
    loads and every entry in it is a complete, valid set of limits."""
    p = tmp_path / "table.json"
    TU.TilingCache({"a": {"limits": TU.limits(1), "us": {}}}).merge_into(str(p))
    TU.TilingCache({"b": {"limits": TU.limits(2), "us": {}}}).merge_into(str(p))
    t = TU.TilingCache.load(str(p))
    assert t.lookup("a") == TU.limits(1) and t.lookup("b") == TU.limits(2)
    shipped = TU.TilingCache.shipped()
    for key, entry in shipped.table.items():
        assert set(entry["limits"]) == set(TU.FIELDS), key
        assert all(int(v) >= 0 for v in entry["limits"].values()), key
        # the kept limits are the fastest of the candidates timed for the entry
        us = entry["us"]
        assert TU.label(entry["limits"]) in us, key
        assert us[TU.label(entry["limits"])] == min(us.values()), key
