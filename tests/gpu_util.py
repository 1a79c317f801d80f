"""Helpers of the GPU parity tests: cached device layers, the routing
comparison with near-tie exclusion, and the output error measures."""
from __future__ import annotations

import functools
import json
import math
import os
import sys

import numpy as np
import torch

from moe_inputs import get, make_inputs
from moe_inputs.gen import weight_f32, x_f32
from oracle import moe_oracle as O

U32 = 2.0 ** -24


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def record(**fields):
    """Append measured figures to $MOE_PARITY_REPORT (JSON lines) when set."""
    path = os.environ.get("MOE_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(fields) + "\n")


@functools.lru_cache(maxsize=2)
def inputs(name: str, T: int | None = None, seed: int = 0):
    cfg = get(name)
    if T is not None:
        cfg = cfg.replace(T=T)
    return cfg, make_inputs(cfg, seed=seed)


@functools.lru_cache(maxsize=1)
def device_layer(name: str, T: int | None = None, seed: int = 0):
    from moe_expert_layer_fp32_amd.layer import DeviceLayer
    cfg, inp = inputs(name, T, seed)
    say(f"[gpu] packing {cfg.name} T={cfg.T} seed={seed}")
    return DeviceLayer(cfg, inp)


def np_of(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def logit_error_bound(x64: np.ndarray, wr64: np.ndarray, z: np.ndarray, dtype: str) -> np.ndarray:
    """Per-token bound on |z_gpu - z| used to call a decision a near-tie.

    The GPU sums K = d products (three exact bf16 planes per weight for bf16
    and W8A8 layers, 3d terms) in fp32. A rounding-error random walk gives
    about sqrt(K) * 2^-24 * sqrt(sum_i (x_i W_ie)^2); the bound takes 16 times
    that plus a few ulp of |z| for the final additions.
    """
    K = x64.shape[1] * (1 if dtype == "f32" else 3)
    s2 = (x64 ** 2) @ (wr64 ** 2)
    b = 16.0 * math.sqrt(K) * U32 * np.sqrt(s2) + 8.0 * U32 * np.abs(z)
    return b.max(axis=1)


def compare_routing(cfg, ref: dict, idx_gpu: np.ndarray, w_gpu: np.ndarray, x64, wr64,
                    w_tol: float = 1e-5):
    """Exact ids and weights within w_tol for every token whose decision is
    clear of a tie; for near-tie tokens, that the GPU's choice is a valid one
    within rounding of the oracle's. Returns the near-tie mask.

    Near-tie tokens must still satisfy every rule of the selection: distinct
    ids in range; at most topk_group groups (group-limited) or exactly
    per_group_k ids in every group (per-group quota); positive weights that
    sum to route_scale (renormalised). And every id the GPU picked that the
    oracle did not must lie within twice the logit error bound of the
    oracle's boundary value: the k-th largest logit among the oracle's
    candidates (plain and group-limited), the per_group_k-th largest logit of
    its group (quota), or, for an id of a group the oracle dropped, a group
    score within twice its bound of the last group the oracle kept."""
    bz = logit_error_bound(x64, wr64, ref["z"], cfg.dtype)
    bg = 2 * (0.5 * bz + 1e-6)                 # group scores: sigmoid slope <= 1/4, two scores summed
    mz, mg = O.selection_margins(ref["z"], ref["scores"], cfg)
    amb = (mz <= 2 * bz) | (mg <= bg)
    clear = ~amb
    bad = np.argwhere(idx_gpu[clear] != ref["idx"][clear])
    assert bad.size == 0, (f"{bad.shape[0]} id mismatches on clear tokens; first token "
                           f"{np.flatnonzero(clear)[bad[0][0]]}")
    werr = np.abs(w_gpu[clear] - ref["w"][clear]).max() if clear.any() else 0.0
    assert werr <= w_tol, f"gate weight error {werr}"
    gsize = cfg.E // cfg.n_group
    for t in np.flatnonzero(amb):
        row = idx_gpu[t]
        zt, st = ref["z"][t], ref["scores"][t]
        assert len(set(row.tolist())) == cfg.k and row.min() >= 0 and row.max() < cfg.E, f"token {t}: ids {row}"
        assert np.all(w_gpu[t] > 0), f"token {t}: weights {w_gpu[t]}"
        if cfg.renorm:
            assert abs(float(w_gpu[t].sum()) - cfg.route_scale) <= 1e-6 * max(1.0, cfg.route_scale), \
                f"token {t}: weights sum {w_gpu[t].sum()}"
        groups = row // gsize
        oracle_row = set(ref["idx"][t].tolist())
        swapped = [int(e) for e in row if int(e) not in oracle_row]
        if cfg.per_group_k:
            assert np.array_equal(np.bincount(groups, minlength=cfg.n_group),
                                  np.full(cfg.n_group, cfg.per_group_k)), f"token {t}: quota {row}"
            for e in swapped:
                g = e // gsize
                bound = np.sort(zt[g * gsize:(g + 1) * gsize])[::-1][cfg.per_group_k - 1]
                assert zt[e] >= bound - 2 * bz[t], f"token {t}: id {e} far from its group's boundary"
            continue
        if cfg.topk_group:
            assert len(set(groups.tolist())) <= cfg.topk_group, f"token {t}: groups {groups}"
            gscore = np.array([O.group_score(st[g * gsize:(g + 1) * gsize]) for g in range(cfg.n_group)])
            kept = set(sorted(range(cfg.n_group), key=lambda g: (-gscore[g], g))[: cfg.topk_group])
            last_kept = min(gscore[g] for g in kept)
            cand = np.concatenate([zt[g * gsize:(g + 1) * gsize] for g in sorted(kept)])
            kth = np.sort(cand)[::-1][cfg.k - 1]
            for e in swapped:
                g = e // gsize
                if g in kept:
                    assert zt[e] >= kth - 2 * bz[t], f"token {t}: id {e} far from the k boundary"
                else:
                    assert gscore[g] >= last_kept - bg[t], f"token {t}: group {g} far from the kept groups"
            continue
        kth = np.sort(zt)[::-1][cfg.k - 1]
        for e in swapped:
            assert zt[e] >= kth - 2 * bz[t], f"token {t}: id {e} far from the k boundary"
    return amb


# ----------------------------------------------------------------------------
# outputs
# ----------------------------------------------------------------------------
def half_ulp(v: np.ndarray, out_dtype: str) -> np.ndarray:
    """Half a unit in the last place of |v| in the output type."""
    bits = 8 if out_dtype != "f32" else 24
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - bits)


def output_errors(y_gpu: np.ndarray, y_ref: np.ndarray, out_dtype: str):
    """(literal, beyond_rounding): max|y_gpu - y_ref| / rms(y_ref), and the same
    after allowing each element the half-ulp of rounding once to the output
    type (the single rounding the definition itself ends with)."""
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    diff = np.abs(y_gpu - y_ref)
    allow = half_ulp(np.maximum(np.abs(y_ref), np.abs(y_gpu)), out_dtype)
    return float(diff.max() / rms), float(np.maximum(diff - allow, 0).max() / rms)


TOL = {"f32": 1e-5, "bf16": 2e-2, "w8a8": 1e-2}


def _ffn_allowance(cfg, inp, X32: np.ndarray, e_local=None) -> np.ndarray:
    """Elementwise bound on how far one FFN's output rows (resident expert
    e_local, or the shared expert when None) may move under the layer's own
    intermediate precision, beyond the exact result:
    - bf16: h stored in bf16 (half an ulp of each h, through |W2|) and the
      output row rounded once to bf16 (half an ulp of it);
    - W8A8: int8 codes of h within rounding of a half-integer boundary may
      take the neighbouring code (h_code_flip_allowance);
    - fp32: fp32 accumulation of the three products, bounded by n * 2^-24 *
      sum |terms| (first order), through SwiGLU (|silu'| <= 1.1)."""
    # the shared expert's arrays are the experts' names with an "s" in front
    pick = (lambda n: inp["s" + n]) if e_local is None else (lambda n: inp[n][e_local])
    if cfg.dtype == "w8a8":
        args = [pick(n) for n in ("w1", "s1", "w3", "s3", "w2", "s2")]
        _, parts = O.swiglu_w8a8(X32, *args, return_parts=True)
        return h_code_flip_allowance(parts["h"].astype(np.float32), parts["sh"], args[4], args[5])
    W1, W3, W2 = (np.asarray(weight_f32(pick(n)), np.float64) for n in ("w1", "w3", "w2"))
    X = np.asarray(X32, np.float64)
    a, b = X @ W1, X @ W3
    sa = O.silu(a)
    h = sa * b
    aW2 = np.abs(W2)
    if cfg.dtype == "bf16":
        return half_ulp(h, "bf16") @ aW2 + half_ulp(h @ W2, "bf16")
    u = 2.0 ** -24
    da = X.shape[1] * u * (np.abs(X) @ np.abs(W1))
    db = X.shape[1] * u * (np.abs(X) @ np.abs(W3))
    dh = 1.1 * np.abs(b) * da + np.abs(sa) * db + 4 * u * np.abs(h)
    return dh @ aW2 + W2.shape[0] * u * (np.abs(h) @ aW2)


def layer_allowance(cfg, inp, idx: np.ndarray, w: np.ndarray, tokens=None) -> np.ndarray:
    """Per output element: sum_j |w_tj| * (the allowance of expert e_tj's row,
    _ffn_allowance) + the shared expert's, for the ids given. Identity experts
    contribute x, which is exact; non-resident ones nothing."""
    X32 = np.asarray(O.x_f32(inp))
    if tokens is not None:
        X32 = X32[np.asarray(tokens)]
    n, k = idx.shape
    allow = np.zeros((n, cfg.d))
    for e in np.unique(idx):
        e = int(e)
        if O.expert_kind(cfg, e) != "ffn":
            continue
        tj = np.argwhere(idx == e)
        r = _ffn_allowance(cfg, inp, X32[tj[:, 0]], e - cfg.ffn_begin)
        np.add.at(allow, tj[:, 0], np.abs(w[tj[:, 0], tj[:, 1]])[:, None] * r)
    if cfg.shared_inter:
        allow += _ffn_allowance(cfg, inp, X32)
    return allow


def h_code_flip_allowance(h32: np.ndarray, sh: np.ndarray, q2: np.ndarray, s2: np.ndarray,
                          eps: float = 1e-4) -> np.ndarray:
    """Per-element allowance for int8 codes of h that sit within eps of a
    half-integer boundary of h/s_h. The GPU computes h in fp32 (relative error
    a few 1e-7, so at most ~1e-4 in code units); where the oracle's h lies that
    close to a boundary the GPU may take the neighbouring code, which moves
    output column n by exactly s_h * |q2[i, n]| * s2[n]. Returns that sum over
    the near-tie codes of each row, shape [rows, d]."""
    r = np.abs(h32.astype(np.float64) / np.where(sh > 0, sh, 1)[:, None])
    near = np.abs(r - np.floor(r) - 0.5) < eps
    q2abs = np.abs(q2.astype(np.float64))
    return (near.astype(np.float64) @ q2abs) * sh[:, None].astype(np.float64) * s2[None, :]


def x64_of(inp) -> np.ndarray:
    return np.asarray(x_f32(inp), np.float64)
