"""Device-resident weights and buffers for one MoE layer, driving libmoe.so.

Memory and marshalling only: host arrays are copied to the GPU once, packed
there by the library's pack kernels, and every layer step runs in the HIP
kernels behind the C ABI.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import lib as L
from .hip_events import Event


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float64:
        a = a.astype(np.float32)
    return torch.from_numpy(a).to(device)


def empty_bytes(n: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


class SecondStream:
    """A second stream of default priority with the fork/join events that
    moe_aux takes for running the shared expert concurrently."""

    def __init__(self, device="cuda"):
        self.stream = torch.cuda.Stream(device=device)
        self.fork = Event(timing=False)
        self.join = Event(timing=False)

    def fill(self, aux: L.MoeAux) -> L.MoeAux:
        aux.stream2 = self.stream.cuda_stream
        aux.ev_fork = self.fork.handle
        aux.ev_join = self.join.handle
        return aux


class DeviceLayer:
    """Packed weights of one layer plus convenience wrappers of the C ABI."""

    def __init__(self, cfg, inp: dict, device="cuda", keep_logical: bool = False):
        self.cfg = cfg
        self.device = device
        self.desc = L.desc_from_config(cfg)
        self.xdtype = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        self.x = to_device(inp["x"], device)
        self._keep = []
        d = self.desc

        def packed(part, a, b=None):
            buf = empty_bytes(L.moe_packed_bytes(d, part), device)
            L.moe_pack_weights(d, part, a, b, buf)
            return buf

        wr = to_device(np.asarray(inp["w_router"], np.float32), device)
        self.router = packed(L.PACK_ROUTER, wr)
        self.bias = None if inp.get("bias") is None else to_device(np.asarray(inp["bias"], np.float32), device)
        self.logical = {"w_router": wr} if keep_logical else None
        self.w13 = self.w2 = self.sw13 = self.sw2 = None
        self.scales = {}
        if cfg.n_ffn:
            w1, w3, w2 = (to_device(inp[n], device) for n in ("w1", "w3", "w2"))
            self.w13 = packed(L.PACK_W13, w1, w3)
            self.w2 = packed(L.PACK_W2, w2)
            if keep_logical:
                self.logical.update(w1=w1, w3=w3, w2=w2)
            if cfg.dtype == "w8a8":
                for n in ("s1", "s3", "s2"):
                    self.scales[n] = to_device(np.asarray(inp[n], np.float32), device)
        if cfg.shared_inter:
            a, b, c = (to_device(inp[n], device) for n in ("sw1", "sw3", "sw2"))
            self.sw13 = packed(L.PACK_SW13, a, b)
            self.sw2 = packed(L.PACK_SW2, c)
            if cfg.dtype == "w8a8":
                for n in ("ss1", "ss3", "ss2"):
                    self.scales[n] = to_device(np.asarray(inp[n], np.float32), device)
        torch.cuda.synchronize()
        p = L.ptr
        s = self.scales
        self.weights = L.MoeWeights(
            router=p(self.router), logit_bias=p(self.bias), w13=p(self.w13), w2=p(self.w2),
            s1=p(s.get("s1")), s3=p(s.get("s3")), s2=p(s.get("s2")), sw13=p(self.sw13), sw2=p(self.sw2),
            ss1=p(s.get("ss1")), ss3=p(s.get("ss3")), ss2=p(s.get("ss2")))

    # ------------------------------------------------------------------
    def desc_for(self, T: int | None) -> L.MoeDesc:
        return self.desc if T is None else L.desc_from_config(self.cfg, T=T)

    def workspace(self, op: int, T: int | None = None) -> torch.Tensor:
        return empty_bytes(L.moe_workspace_bytes(self.desc_for(T), op), self.device)

    def r_max(self, T: int | None = None) -> int:
        T = self.cfg.T if T is None else T
        return T * self.cfg.k if self.cfg.n_ffn else 0

    # ------------------------------------------------------------------
    def route_topk(self, x=None, ws=None):
        x = self.x if x is None else x
        T = x.shape[0]
        d = self.desc_for(T)
        idx = torch.empty((T, self.cfg.k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.cfg.k), dtype=torch.float32, device=self.device)
        ws = self.workspace(L.OP_ROUTE_TOPK, T) if ws is None else ws
        L.moe_route_topk(d, self.weights, x, idx, w, ws)
        return idx, w

    def permute(self, topk_idx):
        T = topk_idx.shape[0]
        d = self.desc_for(T)
        dev = self.device
        counts = torch.empty(self.cfg.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(self.cfg.E + 1, dtype=torch.int32, device=dev)
        ss = torch.empty(max(T * self.cfg.k, 1), dtype=torch.int32, device=dev)
        sp = torch.empty(max(T * self.cfg.k, 1), dtype=torch.int32, device=dev)
        L.moe_permute(d, topk_idx, counts, offsets, ss, sp, self.workspace(L.OP_PERMUTE, T))
        return counts, offsets, ss, sp

    def grouped_ffn(self, which: int, offsets=None, sorted_slot=None, x=None):
        x = self.x if x is None else x
        T = x.shape[0]
        d = self.desc_for(T)
        nrows = self.r_max(T) if which == L.FFN_ROUTED else T
        rows = torch.empty((max(nrows, 1), self.cfg.d), dtype=torch.float32, device=self.device)
        ws = self.workspace(L.OP_FFN_ROUTED if which == L.FFN_ROUTED else L.OP_FFN_SHARED, T)
        L.moe_grouped_ffn(d, self.weights, which, x, offsets, sorted_slot, rows, ws)
        return rows

    def combine(self, rows, shared_rows, topk_idx, topk_w, offsets, slot_pos, x=None):
        x = self.x if x is None else x
        T = x.shape[0]
        y = torch.empty((T, self.cfg.d), dtype=self.xdtype, device=self.device)
        L.moe_combine(self.desc_for(T), x, rows, shared_rows, topk_idx, topk_w, offsets, slot_pos, y)
        return y

    def layer(self, x=None, y=None, aux: L.MoeAux | None = None, ws=None, second: SecondStream | None = None,
              tuning: L.MoeTuning | None = None):
        """moe_layer; with `second`, the shared expert runs on its stream;
        `tuning`: launch limits (moe_tuning)."""
        x = self.x if x is None else x
        T = x.shape[0]
        y = torch.empty((T, self.cfg.d), dtype=self.xdtype, device=self.device) if y is None else y
        ws = self.workspace(L.OP_LAYER, T) if ws is None else ws
        if second is not None:
            aux = second.fill(L.MoeAux() if aux is None else aux)
        if tuning is not None:
            aux = L.MoeAux() if aux is None else aux
            aux.tuning = ctypes.pointer(tuning)
        L.moe_layer(self.desc_for(T), self.weights, x, y, aux, ws)
        return y

    def layer_with_tables(self, x=None, ws=None, second: SecondStream | None = None,
                          tuning: L.MoeTuning | None = None, intermediates: bool = False):
        """moe_layer plus its routing tables (and W8A8 activation codes) via
        moe_aux; with `intermediates`, also the routed SwiGLU rows h, the expert
        output rows and (W8A8) the int8 codes and scales of h, T*k rows of
        capacity each."""
        x = self.x if x is None else x
        T, k, E, dev = x.shape[0], self.cfg.k, self.cfg.E, self.device
        t = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                 topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
                 counts=torch.empty(E, dtype=torch.int32, device=dev),
                 offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                 sorted_slot=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
                 slot_pos=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev))
        if self.cfg.dtype == "w8a8":
            t["q_x"] = torch.empty((T, self.cfg.d), dtype=torch.int8, device=dev)
            t["s_x"] = torch.empty(T, dtype=torch.float32, device=dev)
        if intermediates and self.cfg.n_ffn > 0:
            cap = max(T * k, 1)
            fdt = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
            t["h"] = torch.empty((cap, self.cfg.inter), dtype=fdt, device=dev)
            t["rows"] = torch.empty((cap, self.cfg.d), dtype=fdt, device=dev)
            if self.cfg.dtype == "w8a8":
                t["q_h"] = torch.empty((cap, self.cfg.inter), dtype=torch.int8, device=dev)
                t["s_h"] = torch.empty(cap, dtype=torch.float32, device=dev)
        aux = L.MoeAux(**{n: L.ptr(v) for n, v in t.items()})
        y = self.layer(x, aux=aux, ws=ws, second=second, tuning=tuning)
        return y, t
