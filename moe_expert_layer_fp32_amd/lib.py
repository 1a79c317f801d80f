"""ctypes binding of libmoe.so (include/moe.h), one Python function per entry
point, same names.

This layer only marshals arguments: torch tensors on the GPU supply device
pointers, torch's current stream supplies the HIP stream. Every step of the
layer runs in the library's HIP kernels; there is no CPU fallback. If the
library has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
          -4: "MOE_ERR_HIP"}
GATE = {"softmax": 0, "sigmoid": 1}
DTYPE = {"f32": 0, "bf16": 1, "w8a8": 2}
FFN_ROUTED, FFN_SHARED = 0, 1
PACK_ROUTER, PACK_W13, PACK_W2, PACK_SW13, PACK_SW2 = range(5)
OP_ROUTE_TOPK, OP_PERMUTE, OP_FFN_ROUTED, OP_FFN_SHARED, OP_COMBINE, OP_LAYER = range(6)

# Every symbol include/moe.h declares.
EXPORTS = ("moe_workspace_bytes", "moe_status_str", "moe_packed_bytes", "moe_pack_weights",
           "moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer", "moe_layer_static",
           "moe_stream_read")
STATIC_WORKSPACE_BYTES = 64 << 20   # MOE_STATIC_WORKSPACE_BYTES
STREAM_READ_WGS = 2048              # MOE_STREAM_READ_WGS


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("per_group_k", ctypes.c_int32), ("renorm", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("ffn_begin", ctypes.c_int32), ("n_ffn", ctypes.c_int32), ("zero_begin", ctypes.c_int32),
                ("n_zero", ctypes.c_int32), ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_vp = ctypes.c_void_p


class MoeWeights(ctypes.Structure):
    _fields_ = [("router", _vp), ("logit_bias", _vp), ("w13", _vp), ("w2", _vp), ("s1", _vp), ("s3", _vp),
                ("s2", _vp), ("sw13", _vp), ("sw2", _vp), ("ss1", _vp), ("ss3", _vp), ("ss2", _vp)]


class MoeTuning(ctypes.Structure):
    _fields_ = [("shared_ffn1_wgs", ctypes.c_int32), ("shared_ffn2_wgs", ctypes.c_int32),
                ("routed_ffn1_wgs", ctypes.c_int32), ("routed_ffn2_wgs", ctypes.c_int32),
                ("prefill_tokens", ctypes.c_int32), ("stream_max_rows", ctypes.c_int32),
                ("big_min_rows", ctypes.c_int32), ("dense_big_rows", ctypes.c_int32),
                ("decode_tile_rows", ctypes.c_int32)]


class MoeAux(ctypes.Structure):
    _fields_ = [("topk_idx", _vp), ("topk_w", _vp), ("counts", _vp), ("offsets", _vp), ("sorted_slot", _vp),
                ("slot_pos", _vp), ("q_x", _vp), ("s_x", _vp), ("ev_ffn1_begin", _vp), ("ev_ffn1_end", _vp),
                ("ev_ffn2_begin", _vp), ("ev_ffn2_end", _vp), ("stream2", _vp), ("ev_fork", _vp),
                ("ev_join", _vp), ("tuning", ctypes.POINTER(MoeTuning)), ("h", _vp), ("q_h", _vp), ("s_h", _vp),
                ("rows", _vp), ("ev_sffn1_begin", _vp), ("ev_sffn1_end", _vp), ("ev_sffn2_begin", _vp),
                ("ev_sffn2_end", _vp)]


_lib_handle = None


def load_library() -> ctypes.CDLL:
    """Load libmoe.so (raises when it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_expert_layer_fp32_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        D = ctypes.POINTER(MoeDesc)
        W = ctypes.POINTER(MoeWeights)
        lib.moe_workspace_bytes.argtypes = [D, ctypes.c_int]
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_status_str.argtypes = [ctypes.c_int32]
        lib.moe_status_str.restype = ctypes.c_char_p
        lib.moe_packed_bytes.argtypes = [D, ctypes.c_int]
        lib.moe_packed_bytes.restype = ctypes.c_size_t
        lib.moe_pack_weights.argtypes = [D, ctypes.c_int, P, P, P, ctypes.c_size_t, P]
        lib.moe_route_topk.argtypes = [D, W, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_permute.argtypes = [D, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_grouped_ffn.argtypes = [D, W, ctypes.c_int, P, P, P, P, P, ctypes.c_size_t, P]
        lib.moe_combine.argtypes = [D, P, P, P, P, P, P, P, P, P]
        lib.moe_layer.argtypes = [D, W, P, P, ctypes.POINTER(MoeAux), P, ctypes.c_size_t, P]
        lib.moe_layer_static.argtypes = [D, W, P, P, ctypes.POINTER(MoeAux), P]
        lib.moe_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
        for fn in ("moe_pack_weights", "moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine",
                   "moe_layer", "moe_layer_static", "moe_stream_read"):
            getattr(lib, fn).restype = ctypes.c_int32
        _lib_handle = lib
    return _lib_handle


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def desc_from_config(cfg, T: int | None = None) -> MoeDesc:
    """The C descriptor of a workload (optionally with another token count)."""
    return MoeDesc(T=cfg.T if T is None else T, d=cfg.d, E=cfg.E, k=cfg.k, gate=GATE[cfg.gate],
                   n_group=cfg.n_group, topk_group=cfg.topk_group, per_group_k=cfg.per_group_k,
                   renorm=int(cfg.renorm), route_scale=float(cfg.route_scale), ffn_begin=cfg.ffn_begin,
                   n_ffn=cfg.n_ffn, zero_begin=cfg.zero_begin, n_zero=cfg.n_zero, inter=cfg.inter,
                   shared_inter=cfg.shared_inter, dtype=DTYPE[cfg.dtype])


def ptr(t) -> int | None:
    """Device address of a CUDA tensor (None for None / raw ints passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def stream_handle(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _byref(desc):
    return ctypes.byref(desc)


# ----------------------------------------------------------------------------
# entry points (names as in include/moe.h)
# ----------------------------------------------------------------------------
def moe_workspace_bytes(desc: MoeDesc, op: int) -> int:
    return int(load_library().moe_workspace_bytes(_byref(desc), op))


def moe_status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def moe_packed_bytes(desc: MoeDesc, part: int) -> int:
    return int(load_library().moe_packed_bytes(_byref(desc), part))


def moe_pack_weights(desc, part, src_a, src_b, dst, stream=None) -> None:
    _check("moe_pack_weights", load_library().moe_pack_weights(
        _byref(desc), part, ptr(src_a), ptr(src_b), ptr(dst), dst.numel() * dst.element_size(),
        stream_handle(stream)))


def moe_route_topk(desc, weights: MoeWeights, x, topk_idx, topk_w, ws, stream=None) -> None:
    _check("moe_route_topk", load_library().moe_route_topk(
        _byref(desc), ctypes.byref(weights), ptr(x), ptr(topk_idx), ptr(topk_w), ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_permute(desc, topk_idx, counts, offsets, sorted_slot, slot_pos, ws=None, stream=None) -> None:
    _check("moe_permute", load_library().moe_permute(
        _byref(desc), ptr(topk_idx), ptr(counts), ptr(offsets), ptr(sorted_slot), ptr(slot_pos), ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_grouped_ffn(desc, weights: MoeWeights, which: int, x, offsets, sorted_slot, rows, ws,
                    stream=None) -> None:
    _check("moe_grouped_ffn", load_library().moe_grouped_ffn(
        _byref(desc), ctypes.byref(weights), which, ptr(x), ptr(offsets), ptr(sorted_slot), ptr(rows),
        ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_combine(desc, x, rows, shared_rows, topk_idx, topk_w, offsets, slot_pos, y, stream=None) -> None:
    _check("moe_combine", load_library().moe_combine(
        _byref(desc), ptr(x), ptr(rows), ptr(shared_rows), ptr(topk_idx), ptr(topk_w), ptr(offsets),
        ptr(slot_pos), ptr(y), stream_handle(stream)))


def moe_layer(desc, weights: MoeWeights, x, y, aux: MoeAux | None, ws, stream=None) -> None:
    _check("moe_layer", load_library().moe_layer(
        _byref(desc), ctypes.byref(weights), ptr(x), ptr(y), ctypes.byref(aux) if aux is not None else None,
        ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    _check("moe_stream_read", load_library().moe_stream_read(ptr(buf), nbytes, ptr(sink), stream_handle(stream)))


def moe_layer_static(desc, weights: MoeWeights, x, y, aux: MoeAux | None, stream=None) -> None:
    _check("moe_layer_static", load_library().moe_layer_static(
        _byref(desc), ctypes.byref(weights), ptr(x), ptr(y), ctypes.byref(aux) if aux is not None else None,
        stream_handle(stream)))
