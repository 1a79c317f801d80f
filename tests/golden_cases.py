"""Loader for the hand-worked cases under tests/golden/.

Entries are numbers or closed-form expressions over ln, exp, sqrt, e and
f32() (round to fp32), evaluated here with math; nothing is taken from the
oracle.
"""
from __future__ import annotations

import ast
import json
import math
import os

import numpy as np

from moe_inputs.configs import MoEConfig

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_FUNCS = {"ln": math.log, "exp": math.exp, "sqrt": math.sqrt,
          "f32": lambda v: float(np.float32(v))}
_NAMES = {"e": math.e}


def _ev(node):
    if isinstance(node, ast.Expression):
        return _ev(node.body)
    if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
        return float(node.value)
    if isinstance(node, ast.Name) and node.id in _NAMES:
        return _NAMES[node.id]
    if isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.UAdd)):
        v = _ev(node.operand)
        return -v if isinstance(node.op, ast.USub) else v
    if isinstance(node, ast.BinOp):
        a, b = _ev(node.left), _ev(node.right)
        ops = {ast.Add: lambda: a + b, ast.Sub: lambda: a - b, ast.Mult: lambda: a * b,
               ast.Div: lambda: a / b, ast.Pow: lambda: a ** b}
        return ops[type(node.op)]()
    if isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id in _FUNCS:
        return _FUNCS[node.func.id](*[_ev(a) for a in node.args])
    raise ValueError(f"unsupported expression node {ast.dump(node)}")


def value(v):
    if isinstance(v, str):
        return _ev(ast.parse(v, mode="eval"))
    if isinstance(v, list):
        return [value(u) for u in v]
    return float(v)


def array(v, dtype=np.float64):
    return np.asarray(value(v), dtype=dtype)


def load(name: str) -> dict:
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        return json.load(f)


def layer_case(name: str):
    """(cfg, inp, expected) of a layer-level fixture."""
    raw = load(name)
    cfg = MoEConfig(**raw["cfg"])
    cfg.check()
    inp = {"cfg": cfg}
    for key, v in raw["inputs"].items():
        if cfg.dtype == "w8a8" and key in ("w1", "w3", "w2", "sw1", "sw3", "sw2"):
            inp[key] = array(v).astype(np.int8)
        elif key in ("s1", "s3", "s2", "ss1", "ss3", "ss2"):
            inp[key] = array(v).astype(np.float32)
        else:
            inp[key] = array(v)
    inp.setdefault("bias", None)
    return cfg, inp, raw["expected"]


LAYER_CASES = ["softmax_top2_bias.json", "sigmoid_group_limited.json", "moge_route_scale.json",
               "w8a8_ffn.json"]
