"""Workload descriptors for the MoE expert layer.

A descriptor fixes the shape of one layer call: T tokens of hidden size d, a
router over E experts choosing k per token, which expert ids are resident
SwiGLU FFN experts and which are zero-computation (identity) experts, the
expert and shared-expert inner sizes, and the arithmetic type.

The five workloads below are the deployments the pages describe, reduced to
what one device computes:

* ``tiny_fp32``: a small fp32 layer (T 64, d 128, 8 experts, top-2) that the
  oracle finishes instantly; parity only.
* ``longcat_zero_bf16``: LongCat-Flash's mix of routed FFN experts and
  zero-computation experts (page "LongCat-Flash与GLM-4.6V ... 拆解MoE困局": 512
  routed + 256 zero-computation experts; page "基于Atlas 900 A3 SuperPoD的
  LongCat-Flash ... 背景介绍": activated parameters vary per token). Scaled to
  64 FFN + 32 identity experts, a bias on the identity ids makes about 30% of
  selections land on them.
* ``dsv3_decode_share_bf16``: the one-device share of a DeepSeek-V3 decode
  instance (page "DeepSeek ... Atlas 800I A2": 8 routed + 1 shared expert per
  card), sigmoid router with group-limited selection.
* ``pangu_moge_w8a8``: Pangu Pro MoE's grouped experts (page "昇腾×盘古":
  MoGE, grouped experts for balanced load) with int8 weights and activations
  (quantised activations travel with their scales, page "DeepSeek ...
  通信通信并发"; QuantBatchMatmul, page "LongCat-Flash ... 优化措施三").
* ``prefill_zipf_bf16``: a prefill batch of 4 x 2048 tokens whose expert
  popularity follows a Zipf law, so per-expert token counts range from a
  handful to thousands (the load jitter of page "LongCat-Flash与GLM-4.6V ...
  拆解MoE困局").

Nothing in this module computes any step of the layer.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

GATES = ("softmax", "sigmoid")
DTYPES = ("f32", "bf16", "w8a8")


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens
    d: int                      # hidden size
    E: int                      # experts scored by the router
    k: int                      # experts selected per token
    gate: str                   # "softmax" | "sigmoid"
    n_group: int = 1            # contiguous expert groups (1 = no grouping)
    topk_group: int = 0         # group-limited routing: groups kept (0 = off)
    per_group_k: int = 0        # MoGE: experts taken from every group (0 = off)
    renorm: bool = True         # divide selected weights by their sum
    route_scale: float = 1.0
    ffn_begin: int = 0          # resident FFN experts: ids [ffn_begin, ffn_begin + n_ffn)
    n_ffn: int = 0
    zero_begin: int = 0         # identity experts: ids [zero_begin, zero_begin + n_zero)
    n_zero: int = 0
    inter: int = 0              # expert FFN inner size I
    shared_inter: int = 0       # shared expert inner size (0 = no shared expert)
    dtype: str = "bf16"         # "f32" | "bf16" | "w8a8"
    bias: tuple = ("none",)     # ("none",) | ("const", value, begin, end) | ("zipf", s)
    seed: int = 0
    description: str = ""

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def slots(self) -> int:
        return self.T * self.k

    def check(self) -> None:
        assert self.gate in GATES, self.gate
        assert self.dtype in DTYPES, self.dtype
        assert 1 <= self.k <= self.E
        assert self.E % self.n_group == 0
        assert 0 <= self.ffn_begin and self.ffn_begin + self.n_ffn <= self.E
        assert 0 <= self.zero_begin and self.zero_begin + self.n_zero <= self.E
        ffn = set(range(self.ffn_begin, self.ffn_begin + self.n_ffn))
        assert not ffn & set(range(self.zero_begin, self.zero_begin + self.n_zero))
        if self.per_group_k:
            assert self.k == self.n_group * self.per_group_k
            assert self.per_group_k <= self.E // self.n_group
        if self.topk_group:
            assert self.n_group > 1 and self.topk_group <= self.n_group
            assert self.E // self.n_group >= 2
            assert self.k <= self.topk_group * (self.E // self.n_group)


# The identity-expert logit offset of ``longcat_zero_bf16`` is a literal found by
# oracle/calibrate_bias.py (bisection on the oracle's routing of this exact
# seeded input) so that the identity share of the T*k selections is 0.30.
LONGCAT_IDENTITY_BIAS = -0.0556640625

CONFIGS: dict[str, MoEConfig] = {
    c.name: c
    for c in [
        MoEConfig(
            name="tiny_fp32", T=64, d=128, E=8, k=2, gate="softmax",
            ffn_begin=0, n_ffn=8, inter=256, dtype="f32",
            description="T64 d128, softmax over 8 experts, top-2, fp32",
        ),
        MoEConfig(
            name="longcat_zero_bf16", T=256, d=1024, E=96, k=8, gate="softmax",
            ffn_begin=0, n_ffn=64, zero_begin=64, n_zero=32, inter=512, dtype="bf16",
            bias=("const", LONGCAT_IDENTITY_BIAS, 64, 96),
            description="T256 d1024, softmax over 96 = 64 FFN + 32 identity experts, top-8, bf16",
        ),
        MoEConfig(
            name="dsv3_decode_share_bf16", T=512, d=7168, E=256, k=8, gate="sigmoid",
            n_group=8, topk_group=4, ffn_begin=0, n_ffn=8, inter=2048, shared_inter=2048,
            dtype="bf16",
            description="T512 d7168, sigmoid over 256, 8 groups top-4 groups, top-8; "
                        "8 resident experts + shared, bf16",
        ),
        MoEConfig(
            name="pangu_moge_w8a8", T=456, d=5120, E=64, k=8, gate="softmax",
            n_group=8, per_group_k=1, ffn_begin=0, n_ffn=64, inter=1536, shared_inter=4096,
            dtype="w8a8",
            description="T456 d5120, softmax over 64 in 8 groups, top-1 per group; "
                        "int8 weights + per-token int8 activations, bf16 out",
        ),
        MoEConfig(
            name="prefill_zipf_bf16", T=8192, d=7168, E=256, k=8, gate="sigmoid",
            ffn_begin=0, n_ffn=32, inter=2048, shared_inter=2048, dtype="bf16",
            bias=("zipf", 1.1),
            description="T8192 (4 x 2048) d7168, sigmoid over 256, top-8, Zipf(1.1) expert "
                        "popularity; 32 resident experts + shared, bf16",
        ),
    ]
}

# Short aliases in the order the workloads are listed above.
ALIASES = {f"C{i + 1}": name for i, name in enumerate(CONFIGS)}


def get(name: str) -> MoEConfig:
    name = ALIASES.get(name, name)
    cfg = CONFIGS[name]
    cfg.check()
    return cfg
