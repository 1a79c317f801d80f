"""Host-side checks of bench.py's algorithmic work counts (no GPU).

The whole-layer byte count is pinned to the sizes worked out by hand from
the workload shapes (every resident expert active): weights of the resident
experts and of the shared expert, the fp32 router, x read and y written."""
from __future__ import annotations

import importlib.util
import os

import numpy as np
import pytest

from moe_inputs import get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _all_active(cfg, rows_each=3):
    c = np.zeros(cfg.E, np.int64)
    c[cfg.ffn_begin:cfg.ffn_begin + cfg.n_ffn] = rows_each
    return c


# (workload, bytes per call with every resident expert active), written out
# from the shapes: n_ffn * 3 d I * w (+ int8 scales 4 (2I + d) per expert),
# shared 3 d I_s * w (+ scales), router 4 d E, x and y 2 * T d * xb.
HAND = {
    "longcat_zero_bf16": 64 * 3 * 1024 * 512 * 2 + 4 * 1024 * 96 + 2 * 256 * 1024 * 2,
    "dsv3_decode_share_bf16": 8 * 3 * 7168 * 2048 * 2 + 3 * 7168 * 2048 * 2 + 4 * 7168 * 256 + 2 * 512 * 7168 * 2,
    "pangu_moge_w8a8": (64 * (3 * 5120 * 1536 + 4 * (2 * 1536 + 5120)) + 3 * 5120 * 4096 + 4 * (2 * 4096 + 5120)
                        + 4 * 5120 * 64 + 2 * 456 * 5120 * 2),
    "prefill_zipf_bf16": 32 * 3 * 7168 * 2048 * 2 + 3 * 7168 * 2048 * 2 + 4 * 7168 * 256 + 2 * 8192 * 7168 * 2,
}


@pytest.mark.parametrize("name", sorted(HAND))
def test_layer_bytes_match_hand_count(name):
    B = _bench()
    cfg = get(name)
    (byts, flops), = B.layer_algorithmic(cfg, [_all_active(cfg)])
    assert byts == HAND[name]
    R = 3 * cfg.n_ffn
    assert flops == 2.0 * R * 3 * cfg.d * cfg.inter + 2.0 * cfg.T * 3 * cfg.d * cfg.shared_inter


def test_layer_bytes_count_only_experts_with_tokens():
    B = _bench()
    cfg = get("dsv3_decode_share_bf16")
    c = _all_active(cfg)
    c[cfg.ffn_begin + 2] = 0
    (full, _), (fewer, _) = B.layer_algorithmic(cfg, [_all_active(cfg), c])
    assert full - fewer == 3 * cfg.d * cfg.inter * 2


def test_gate_up_bytes_and_flops():
    B = _bench()
    cfg = get("longcat_zero_bf16")
    c = _all_active(cfg, rows_each=5)
    (byts, flops, R, active), = B.ffn1_algorithmic(cfg, [c])
    assert (R, active) == (5 * 64, 64)
    # W1 and W3 of the 64 experts with tokens, x read once (256 rows); no
    # gathered rows, no h
    assert byts == 64 * 2 * 1024 * 512 * 2 + 256 * 1024 * 2
    assert flops == 2.0 * R * 1024 * 2 * 512
    cfg = get("prefill_zipf_bf16")
    sb, sf = B.shared_ffn1_algorithmic(cfg)
    assert sb == 2 * 7168 * 2048 * 2 + 8192 * 7168 * 2
    assert sf == 2.0 * 8192 * 7168 * 2 * 2048


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus 2 exits with status 2 and says why, before any
    device work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_lines_summarise_each_child(monkeypatch):
    """decode_workloads: one child run of bench.py per decode workload, with
    the parent's steps and warm-up and no nested decode lines; each child's
    last JSON line is summarised, and a child that fails leaves its exit
    status instead of failing the parent (no GPU: the child runs are faked)."""
    import json
    import subprocess
    import types
    bench = _bench()
    calls = []

    def fake_run(cmd, capture_output, text, timeout):
        calls.append(cmd)
        name = cmd[cmd.index("--config") + 1]
        if name == "pangu_moge_w8a8":
            return types.SimpleNamespace(returncode=1, stdout="", stderr="boom")
        line = {"value": 1.0, "unit": "tokens/s", "ms_per_step": 0.5, "dtype": "bf16", "config": {"workload": name},
                "roofline": {"bound": "hbm", "achieved": 4000.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.5,
                             "kernel": "k", "mean_us": 10.0, "traffic": None, "extra": 1},
                "layer_roofline": {"bound": "hbm", "achieved": 3000.0, "peak": 8000.0, "unit": "GB/s",
                                   "frac": 0.375},
                "tuning": {"limits": {"decode_tile_rows": 32}}}
        return types.SimpleNamespace(returncode=0, stdout="progress\n" + json.dumps(line) + "\n", stderr="")

    monkeypatch.setattr(subprocess, "run", fake_run)
    args = types.SimpleNamespace(steps=7, warmup=3, no_tune=False)
    out = bench.decode_lines(args)
    assert list(out) == list(bench.DECODE_CONFIGS)
    for cmd in calls:
        assert cmd[cmd.index("--steps") + 1] == "7" and cmd[cmd.index("--warmup") + 1] == "3"
        assert "--no-decode" in cmd and "--no-cpu-baseline" in cmd
    assert out["pangu_moge_w8a8"] == {"error": "exit status 1"}
    ok = out["longcat_zero_bf16"]
    assert ok["ms_per_step"] == 0.5 and ok["roofline"]["frac"] == 0.5 and "extra" not in ok["roofline"]
    assert ok["layer_roofline"]["frac"] == 0.375 and ok["tuning"] == {"decode_tile_rows": 32}
