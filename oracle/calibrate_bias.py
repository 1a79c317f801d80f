"""Find the identity-expert logit offset of the zero-computation workload.

The LongCat-style workload puts a constant offset on the logits of its 32
identity experts so that about 30% of the T*k selections land on them (the
pages give LongCat-Flash's zero-computation experts a varying share of each
token's activated parameters). This script bisects that offset with the
oracle's own routing of the seeded input and prints the value, rounded to a
multiple of 2^-10, that is written as a literal into moe_inputs/configs.py.

Run: python -m oracle.calibrate_bias
"""
from __future__ import annotations

import numpy as np

from moe_inputs import get, make_inputs
from oracle import moe_oracle as O

TARGET = 0.30


def identity_share(cfg, inp, beta: float) -> float:
    lo, hi = cfg.zero_begin, cfg.zero_begin + cfg.n_zero
    bias = np.zeros(cfg.E)
    bias[lo:hi] = beta
    z = O.router_logits(O.x_f32(inp), inp["w_router"], bias)
    idx = O.select_experts(O.gate_scores(z, cfg.gate), cfg)
    return float(np.mean((idx >= lo) & (idx < hi)))


def main() -> None:
    cfg = get("longcat_zero_bf16").replace(n_ffn=0)      # routing only needs x and W_r
    inp = make_inputs(cfg)
    a, b = -1.0, 1.0                                       # share(a) < target < share(b)
    for _ in range(40):
        m = 0.5 * (a + b)
        if identity_share(cfg, inp, m) < TARGET:
            a = m
        else:
            b = m
    beta = round(0.5 * (a + b) * 1024) / 1024
    print(f"beta = {beta!r}  share = {identity_share(cfg, inp, beta):.4f}")


if __name__ == "__main__":
    main()
