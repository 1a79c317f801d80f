"""Seeded synthetic inputs for the MoE expert layer.

Both the CPU oracle and the GPU tests/bench take their inputs from here. This
module only draws random numbers and stores them in the element types a layer
call consumes; it computes no step of the layer.

Recipe (every workload):
* numpy PCG64 seeded with ``SeedSequence(cfg.seed)``; child streams are spawned
  in a fixed order: x, router, bias permutation, one per resident FFN expert
  (drawing W1, W3, W2 in that order), shared expert (W1, W3, W2).
* x ~ N(0, 1); every weight, the router's included, ~ N(0, 0.02) (0.02 is the
  standard deviation). Values are drawn in fp32 and rounded to nearest-even
  into the workload's element type; the router weight stays fp32.
* int8 weights (w8a8): per output channel n, s[n] = max_k |W[k, n]| / 127 in
  fp32 and q = clamp(rint(W / s[n]), -127, 127); a weight arrives as (q, s).
* Router bias: ``("const", v, b, e)`` puts v on ids [b, e); ``("zipf", s)`` gives
  expert e the log-popularity ln p_r(e), p_r proportional to r^-s over ranks
  r = 1..E, with the rank of each expert taken from a seeded permutation.

bf16 values are carried as uint16 bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from .configs import MoEConfig

WEIGHT_STD = 0.02


# ----------------------------------------------------------------------------
# element-type helpers
# ----------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantise_weight_int8(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-output-channel int8 for a [..., K, N] fp32 weight."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=-2)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint(w / safe[..., None, :])
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _store(a32: np.ndarray, dtype: str):
    if dtype == "f32":
        return a32
    if dtype == "bf16":
        return bf16_bits(a32)
    raise ValueError(dtype)


def _expert_weights(ss, d, inter, dtype):
    """(W1 [d, I], W3 [d, I], W2 [I, d]) of one expert, plus int8 scales."""
    g = _rng(ss)
    w1 = _normal(g, (d, inter), WEIGHT_STD)
    w3 = _normal(g, (d, inter), WEIGHT_STD)
    w2 = _normal(g, (inter, d), WEIGHT_STD)
    if dtype == "w8a8":
        q1, s1 = quantise_weight_int8(w1)
        q3, s3 = quantise_weight_int8(w3)
        q2, s2 = quantise_weight_int8(w2)
        return (q1, q3, q2), (s1, s3, s2)
    return (_store(w1, dtype), _store(w3, dtype), _store(w2, dtype)), None


def router_bias(cfg: MoEConfig, ss: np.random.SeedSequence):
    kind = cfg.bias[0]
    if kind == "none":
        return None
    b = np.zeros(cfg.E, dtype=np.float32)
    if kind == "const":
        _, value, lo, hi = cfg.bias
        b[lo:hi] = np.float32(value)
        return b
    if kind == "zipf":
        s = float(cfg.bias[1])
        ranks = _rng(ss).permutation(cfg.E) + 1          # rank r(e) in 1..E
        p = np.arange(1, cfg.E + 1, dtype=np.float64) ** (-s)
        p /= p.sum()
        b[:] = np.log(p[ranks - 1]).astype(np.float32)
        return b
    raise ValueError(cfg.bias)


def make_inputs(cfg: MoEConfig, seed: int | None = None, threads: int | None = None) -> dict:
    """All tensors of one layer call, in the logical layouts of the C ABI.

    Keys: x [T, d]; w_router [d, E] fp32; bias [E] fp32 or None;
    w1, w3 [n_ffn, d, I] and w2 [n_ffn, I, d]; sw1, sw3 [d, Is] and sw2 [Is, d]
    when a shared expert exists; for w8a8 also s1, s3 [n_ffn, I], s2 [n_ffn, d],
    ss1, ss3 [Is], ss2 [d]. x is fp32 (f32) or bf16 bits (bf16, w8a8); expert
    weights are fp32, bf16 bits or int8 by workload.
    """
    cfg.check()
    seed = cfg.seed if seed is None else seed
    root = np.random.SeedSequence(seed)
    ss_x, ss_r, ss_b, ss_experts, ss_shared = root.spawn(5)
    xdtype = "f32" if cfg.dtype == "f32" else "bf16"
    out: dict = {"cfg": cfg, "seed": seed}
    out["x"] = _store(_normal(_rng(ss_x), (cfg.T, cfg.d), 1.0), xdtype)
    out["w_router"] = _normal(_rng(ss_r), (cfg.d, cfg.E), WEIGHT_STD)
    out["bias"] = router_bias(cfg, ss_b)

    n = cfg.n_ffn
    if n:
        wdt = {"f32": np.float32, "bf16": np.uint16, "w8a8": np.int8}[cfg.dtype]
        w1 = np.empty((n, cfg.d, cfg.inter), dtype=wdt)
        w3 = np.empty((n, cfg.d, cfg.inter), dtype=wdt)
        w2 = np.empty((n, cfg.inter, cfg.d), dtype=wdt)
        if cfg.dtype == "w8a8":
            s1 = np.empty((n, cfg.inter), np.float32)
            s3 = np.empty((n, cfg.inter), np.float32)
            s2 = np.empty((n, cfg.d), np.float32)
        children = ss_experts.spawn(n)

        def fill(e):
            (a, b, c), sc = _expert_weights(children[e], cfg.d, cfg.inter, cfg.dtype)
            w1[e], w3[e], w2[e] = a, b, c
            if sc is not None:
                s1[e], s3[e], s2[e] = sc

        nthreads = threads or min(8, os.cpu_count() or 1)
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(n)))
        out.update(w1=w1, w3=w3, w2=w2)
        if cfg.dtype == "w8a8":
            out.update(s1=s1, s3=s3, s2=s2)

    if cfg.shared_inter:
        (a, b, c), sc = _expert_weights(ss_shared, cfg.d, cfg.shared_inter, cfg.dtype)
        out.update(sw1=a, sw3=b, sw2=c)
        if sc is not None:
            out.update(ss1=sc[0], ss3=sc[1], ss2=sc[2])
    return out


def x_f32(inp: dict) -> np.ndarray:
    """The exact values of x (bf16 bits decoded; float arrays as given)."""
    return weight_f32(inp["x"])


def weight_f32(a: np.ndarray) -> np.ndarray:
    """Exact values of a stored array: bf16 bits decoded to fp32, int8 widened
    to fp32, float arrays (fp32, or fp64 in hand-built cases) returned as given."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f32(a)
    if a.dtype == np.int8:
        return a.astype(np.float32)
    return a


def make_routing(cfg: MoEConfig, seed: int = 1, skew: float = 0.0) -> tuple[np.ndarray, np.ndarray]:
    """A random routing decision for exercising the downstream steps alone.

    Returns topk_idx [T, k] int32 (k distinct ids per token in [0, E)) and
    topk_w [T, k] fp32 (positive, each row summing to about 1). With skew > 0
    ids are drawn with probability proportional to (rank)^-skew, so some
    experts receive many tokens and some none.
    """
    g = _rng(np.random.SeedSequence([seed, 0x5EED]))
    if skew > 0:
        p = np.arange(1, cfg.E + 1, dtype=np.float64) ** (-skew)
        p = p[g.permutation(cfg.E)]
        p /= p.sum()
    else:
        p = None
    idx = np.empty((cfg.T, cfg.k), dtype=np.int32)
    for t in range(cfg.T):
        idx[t] = g.choice(cfg.E, size=cfg.k, replace=False, p=p)
    w = g.random((cfg.T, cfg.k), dtype=np.float32) + np.float32(0.05)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w
