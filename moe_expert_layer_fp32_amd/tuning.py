"""Launch limits and tile choices for moe_layer chosen from measured runs.

This is the history-based tiling cache of SwiftGMM (page "华为技术披露集
VOL.12：昇腾×盘古", section SwiftGMM：专家计算突击队，闪电速度抵达推理算力战场):
tile parameters are predicted from past loads instead of being fixed. Here
the parameters are the members of moe_tuning: the tile choice by per-expert
row count (the prefill threshold, theta of the weight-streaming class, the
256-row classes of experts and of dense products, the decode tile height)
and the workgroup caps of
each product. For one layer shape, stream count and bucket of its
per-expert token counts, a few candidates are timed on the caller's own
layer calls and the fastest is kept in a host-side table. The table is keyed
by plain values and saved to JSON; the package ships one measured on an
MI355X for the workloads of this repository (tuning_table.json), which
callers load instead of tuning from empty. A serving loop takes the bucket
from the counts of its previous call (moe_aux.counts), so choosing an entry
never waits for the device.

The caps matter where the shared expert runs on a second stream: persistent
GEMMs can occupy every compute unit while the other stream's products wait
for room, and a product whose tiles do not fill the last round of compute
units leaves room the other stream can use. Whether that pays depends on the
shape, so it is measured rather than modelled.
"""
from __future__ import annotations

import json
import math
import os
import time
from typing import Callable

import numpy as np

from . import lib as L

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuning_table.json")

FIELDS = ("shared_ffn1_wgs", "shared_ffn2_wgs", "routed_ffn1_wgs", "routed_ffn2_wgs",
          "prefill_tokens", "stream_max_rows", "big_min_rows", "dense_big_rows", "decode_tile_rows")

# Candidate caps (shared gate/up, shared down); (0, 0) is the library's own
# choice and always a candidate.
SHARED_CANDIDATES = ((0, 0), (96, 0), (128, 0), (192, 0), (128, 128), (192, 192))
NO_BIG = 1 << 30          # a big_min_rows / dense_big_rows no layer reaches: 256-row tiles off


def candidates_for(desc: L.MoeDesc, streams: int) -> list[dict]:
    """Candidate limits for one layer shape. Decode sizes (below the default
    prefill threshold of 1024 tokens): the shared expert's caps, the
    per-expert tile classes of the prefill regime applied early, and 32-row
    tiles for the routed experts (with and without the widest caps). Prefill
    sizes: caps of the shared products and of the routed gate/up, with and
    without 256-row tiles for routed experts."""
    out = []
    has_shared = desc.shared_inter > 0
    if desc.T < 1024:
        shared = SHARED_CANDIDATES if (has_shared and streams == 2) else ((0, 0),)
        for c in shared:
            out.append(limits(*c))
        out.append(limits(prefill_tokens=max(1, desc.T)))
        best_caps = shared[-1] if len(shared) > 1 else (0, 0)
        for theta in (32, 64):   # experts up to theta rows on the 32-row streaming kernel
            out.append(limits(stream_max_rows=theta))
            if best_caps != (0, 0):
                out.append(limits(best_caps[0], best_caps[1], stream_max_rows=theta))
        for c in shared:            # 32-row tiles for the routed experts
            out.append(limits(c[0], c[1], decode_tile_rows=32))
        return out
    shared = ((0, 0), (128, 128), (128, 0), (192, 192)) if (has_shared and streams == 2) else ((0, 0),)
    routed = ((0, 0), (160, 0)) if streams == 2 else ((0, 0),)
    for big in (0, NO_BIG):
        for sc in shared:
            for rc in routed:
                out.append(limits(sc[0], sc[1], rc[0], rc[1], big_min_rows=big))
    return out


def limits(shared_ffn1_wgs=0, shared_ffn2_wgs=0, routed_ffn1_wgs=0, routed_ffn2_wgs=0, prefill_tokens=0,
           stream_max_rows=0, big_min_rows=0, dense_big_rows=0, decode_tile_rows=0) -> dict:
    return dict(zip(FIELDS, (shared_ffn1_wgs, shared_ffn2_wgs, routed_ffn1_wgs, routed_ffn2_wgs, prefill_tokens,
                             stream_max_rows, big_min_rows, dense_big_rows, decode_tile_rows)))


def label(lim: dict) -> str:
    """Short name of a limits dict: its members in FIELDS order."""
    return "/".join(str(int(lim.get(f, 0))) for f in FIELDS)


def to_struct(lim: dict | None) -> L.MoeTuning | None:
    """moe_tuning for a limits dict (None: no limits)."""
    if lim is None or not any(lim.values()):
        return None
    return L.MoeTuning(**{f: int(lim.get(f, 0)) for f in FIELDS})


def load_bucket(counts, ffn_begin: int, n_ffn: int) -> int:
    """Bucket of the per-expert token counts of the resident FFN experts:
    ceil(log2(1 + largest count)), which fixes how many row tiles the
    largest expert needs."""
    c = np.asarray(counts)[ffn_begin:ffn_begin + n_ffn]
    return int(math.ceil(math.log2(1 + int(c.max())))) if c.size else 0


def shape_key(desc: L.MoeDesc, streams: int, bucket: int) -> str:
    """Table key: the layer shape, the number of streams and the load bucket."""
    parts = [f"{f}={getattr(desc, f)}" for f in ("T", "d", "E", "k", "n_ffn", "n_zero", "inter", "shared_inter",
                                                 "dtype", "gate", "n_group", "topk_group", "per_group_k")]
    return ",".join(parts + [f"streams={streams}", f"bucket={bucket}"])


class TilingCache:
    """Host-side table: key -> {"limits": {...}, "us": {label(candidate): time}}."""

    def __init__(self, table: dict | None = None):
        self.table = dict(table or {})

    def lookup(self, key: str) -> dict | None:
        e = self.table.get(key)
        return None if e is None else dict(e["limits"])

    def tune(self, key: str, run: Callable[[L.MoeTuning | None, int], None], sync: Callable[[], None],
             candidates=SHARED_CANDIDATES, calls: int = 20, reps: int = 3,
             clock: Callable[[], float] = time.perf_counter) -> dict:
        """Time every candidate and keep the fastest for `key`. Candidates are
        limits dicts or tuples of the leading fields. run(tuning, i)
        enqueues the i-th layer call with that moe_tuning; sync() waits for the
        device. Each candidate's time is the best over `reps` rounds of
        `calls` calls (the calls are device-bound, so wall time between two
        synchronisations is device time). clock: seconds, monotonic."""
        as_dict = [c if isinstance(c, dict) else limits(*c) for c in candidates]
        cands = {label(lim): lim for lim in as_dict}
        times: dict[str, float] = {}
        for _ in range(reps):
            for name, lim in cands.items():
                t = to_struct(lim)
                for i in range(3):
                    run(t, i)
                sync()
                t0 = clock()
                for i in range(calls):
                    run(t, i)
                sync()
                us = (clock() - t0) / calls * 1e6
                times[name] = min(us, times.get(name, math.inf))
        best = min(times, key=times.get)
        self.table[key] = {"limits": dict(cands[best]), "us": {k: round(v, 2) for k, v in times.items()}}
        return dict(cands[best])

    def save(self, path: str) -> None:
        with open(path, "w") as f:
            json.dump(self.table, f, indent=1, sort_keys=True)

    @classmethod
    def load(cls, path: str) -> "TilingCache":
        with open(path) as f:
            return cls(json.load(f))

    @classmethod
    def shipped(cls) -> "TilingCache":
        """The table measured for this repository's workloads (empty if absent)."""
        return cls.load(TABLE_PATH) if os.path.exists(TABLE_PATH) else cls()

    def merge_into(self, path: str) -> None:
        """Add this table's entries to the JSON table at `path` (created if absent)."""
        old = TilingCache.load(path).table if os.path.exists(path) else {}
        old.update(self.table)
        TilingCache(old).save(path)
