"""The C ABI on the CPU: libmoe.so loads, exports every symbol moe.h declares,
and rejects bad arguments on the host before anything is launched (no call
here reaches a GPU)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from moe_inputs import CONFIGS, get

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000   # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    from moe_expert_layer_fp32_amd import lib
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m moe_expert_layer_fp32_amd.build)")
    lib.load_library()
    return lib


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function(L):
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS), declared
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layouts_match_header(L, tmp_path):
    """Size and member offsets of every ctypes struct of the binding equal
    what a C compiler makes of moe.h."""
    structs = {"moe_desc": L.MoeDesc, "moe_weights": L.MoeWeights, "moe_aux": L.MoeAux,
               "moe_tuning": L.MoeTuning}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        lines += [f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));' for f, _ in py._fields_]
    lines.append("return 0; }")
    src, exe = tmp_path / "layout.c", tmp_path / "layout"
    src.write_text("\n".join(lines))
    subprocess.run(["gcc", "-std=c11", "-Wall", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    checked = 0
    for line in filter(None, out):
        cname, field, val = line.split()
        py = structs[cname]
        want = ctypes.sizeof(py) if field == "sizeof" else getattr(py, field).offset
        assert int(val) == want, line
        checked += 1
    assert checked == sum(len(py._fields_) + 1 for py in structs.values())


def test_status_strings(L):
    assert L.moe_status_str(0) == "MOE_OK"
    assert L.moe_status_str(-3) == "MOE_ERR_WORKSPACE"
    assert L.moe_status_str(-99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workspace_and_packed_sizes(L, name):
    cfg = get(name)
    d = L.desc_from_config(cfg)
    assert L.moe_workspace_bytes(d, L.OP_LAYER) > 0
    slots = cfg.T * cfg.k
    assert L.moe_workspace_bytes(d, L.OP_PERMUTE) == (0 if slots <= 8192 else -(-slots // 2048) * cfg.E * 4)
    wb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    assert L.moe_packed_bytes(d, L.PACK_W13) == cfg.n_ffn * cfg.d * cfg.inter * 2 * wb
    assert L.moe_packed_bytes(d, L.PACK_W2) == cfg.n_ffn * cfg.d * cfg.inter * wb
    assert L.moe_packed_bytes(d, L.PACK_SW13) == cfg.d * cfg.shared_inter * 2 * wb
    ep = (cfg.E + 15) // 16 * 16
    assert L.moe_packed_bytes(d, L.PACK_ROUTER) == ep * cfg.d * (4 if cfg.dtype == "f32" else 6)


def _layer(L, d, ws_bytes=1 << 40, x=FAKE, y=FAKE, router=FAKE):
    lib = L.load_library()
    w = L.MoeWeights(router=router, w13=FAKE, w2=FAKE, s1=FAKE, s3=FAKE, s2=FAKE, sw13=FAKE, sw2=FAKE,
                     ss1=FAKE, ss3=FAKE, ss2=FAKE)
    return lib.moe_layer(ctypes.byref(d), ctypes.byref(w), x, y, None, FAKE, ws_bytes, None)


def _desc(L, **kw):
    cfg = get("dsv3_decode_share_bf16").replace(**kw)
    return L.desc_from_config(cfg)


BAD = [
    (dict(k=300), -1),                             # k > E
    (dict(gate="softmax"), 0),                     # control (valid; fails later on workspace only if too small)
]


@pytest.mark.parametrize("field,value,status", [
    ("k", 257, -1), ("E", 0, -1), ("T", -1, -1), ("gate", 7, -1), ("dtype", 9, -1), ("n_group", 3, -1),
    ("topk_group", 9, -1), ("per_group_k", 2, -1), ("ffn_begin", 250, -1), ("zero_begin", 4, None),
    ("d", 7100, -2), ("inter", 2000, -2), ("shared_inter", 100, -2), ("E", 512, -2), ("k", 17, -2),
    ("T", 1 << 18, -2),
])
def test_descriptor_validation(L, field, value, status):
    d = _desc(L)
    setattr(d, field, value)
    if field == "zero_begin":        # identity ids overlapping the resident FFN ids
        d.n_zero = 8
        status = -1
    if field == "E" and value == 512:
        d.n_group = 8
    assert _layer(L, d) == status
    assert L.moe_workspace_bytes(d, L.OP_LAYER) == 0


def test_group_limits(L):
    d = _desc(L)
    d.n_group, d.topk_group, d.E = 128, 4, 256      # > 64 groups with group-limited routing
    assert _layer(L, d) == -2
    d = L.desc_from_config(get("pangu_moge_w8a8"))
    d.k = 6                                         # MoGE: k must be n_group * per_group_k
    assert _layer(L, d) == -1


def test_workspace_too_small_and_null_pointers(L):
    d = _desc(L)
    need = L.moe_workspace_bytes(d, L.OP_LAYER)
    assert _layer(L, d, ws_bytes=need - 1) == -3
    assert _layer(L, d, x=None) == -1
    assert _layer(L, d, router=None) == -1
    lib = L.load_library()
    assert lib.moe_permute(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert lib.moe_combine(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    w = L.MoeWeights()
    assert lib.moe_grouped_ffn(ctypes.byref(d), ctypes.byref(w), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               None) == -1
    assert lib.moe_grouped_ffn(ctypes.byref(d), ctypes.byref(w), 5, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               None) == -1
    assert lib.moe_route_topk(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -1


def test_second_stream_needs_both_events(L):
    d = _desc(L)
    lib = L.load_library()
    w = L.MoeWeights(router=FAKE, w13=FAKE, w2=FAKE, sw13=FAKE, sw2=FAKE)
    for given in (dict(stream2=FAKE), dict(stream2=FAKE, ev_fork=FAKE), dict(ev_join=FAKE),
                  dict(stream2=FAKE, ev_fork=FAKE, ev_join=FAKE, stream=FAKE)):
        stream = given.pop("stream", None)
        aux = L.MoeAux(**given)
        assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, ctypes.byref(aux), FAKE, 1 << 40,
                             stream) == -1, given
    # all three given: validation passes and only the workspace check fails
    aux = L.MoeAux(stream2=FAKE, ev_fork=FAKE, ev_join=FAKE)
    assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, ctypes.byref(aux), FAKE, 0, None) == -3


def test_negative_launch_limit_rejected(L):
    d = _desc(L)
    lib = L.load_library()
    w = L.MoeWeights(router=FAKE, w13=FAKE, w2=FAKE, sw13=FAKE, sw2=FAKE)
    for field in ("shared_ffn1_wgs", "shared_ffn2_wgs", "routed_ffn1_wgs", "routed_ffn2_wgs"):
        t = L.MoeTuning(**{field: -1})
        aux = L.MoeAux(tuning=ctypes.pointer(t))
        assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, ctypes.byref(aux), FAKE, 1 << 40,
                             None) == -1, field
    # a decode tile height other than 32 or 64
    for rows in (-1, 16, 48, 128):
        t = L.MoeTuning(decode_tile_rows=rows)
        aux = L.MoeAux(tuning=ctypes.pointer(t))
        assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, ctypes.byref(aux), FAKE, 1 << 40,
                             None) == -1, rows
    # zero and positive limits pass validation; only the workspace check fails
    for t in (L.MoeTuning(shared_ffn1_wgs=128, routed_ffn2_wgs=0), L.MoeTuning(decode_tile_rows=32),
              L.MoeTuning(decode_tile_rows=64)):
        aux = L.MoeAux(tuning=ctypes.pointer(t))
        assert lib.moe_layer(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, ctypes.byref(aux), FAKE, 0, None) == -3


def test_pack_rejects_small_destination(L):
    d = _desc(L)
    lib = L.load_library()
    need = L.moe_packed_bytes(d, L.PACK_W13)
    assert lib.moe_pack_weights(ctypes.byref(d), L.PACK_W13, FAKE, FAKE, FAKE, need - 1, None) == -3
    assert lib.moe_pack_weights(ctypes.byref(d), L.PACK_W13, FAKE, None, FAKE, need, None) == -1
    assert lib.moe_pack_weights(ctypes.byref(d), 99, FAKE, FAKE, FAKE, need, None) == -1


@pytest.mark.parametrize("n_ffn", [0, 8])
def test_combine_requires_routing_tables_for_every_n_ffn(L, n_ffn):
    """moe_combine reads offsets[ffn_begin] and each selection's slot_pos even
    when no FFN expert is resident, so NULL tables are rejected on the host
    (MOE_ERR_INVALID_ARG) before anything is launched, whatever n_ffn is."""
    lib = L.load_library()
    d = _desc(L, n_ffn=n_ffn, shared_inter=0)
    rows = FAKE if n_ffn else None
    for offsets, slot_pos in ((None, FAKE), (FAKE, None), (None, None)):
        assert lib.moe_combine(ctypes.byref(d), FAKE, rows, None, FAKE, FAKE, offsets, slot_pos, FAKE,
                               None) == -1, (offsets, slot_pos)
    if n_ffn:   # the expert rows stay required with resident experts
        assert lib.moe_combine(ctypes.byref(d), FAKE, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    # with T == 0 every call is a no-op that reads nothing
    d.T = 0
    assert lib.moe_combine(ctypes.byref(d), None, None, None, None, None, None, None, None, None) == 0


def test_layer_static_refuses_before_any_hip_call(L):
    """moe_layer_static: a workspace need above MOE_STATIC_WORKSPACE_BYTES is
    MOE_ERR_WORKSPACE and an invalid descriptor keeps moe_layer's status, both
    returned on the host before any HIP call (none is possible here)."""
    lib = L.load_library()
    w = L.MoeWeights(router=FAKE, w13=FAKE, w2=FAKE, sw13=FAKE, sw2=FAKE)
    big = _desc(L)                                    # the DeepSeek-style share needs ~360 MiB
    assert L.moe_workspace_bytes(big, L.OP_LAYER) > L.STATIC_WORKSPACE_BYTES
    assert lib.moe_layer_static(ctypes.byref(big), ctypes.byref(w), FAKE, FAKE, None, None) == -3
    bad = _desc(L)
    bad.k = 300
    assert lib.moe_layer_static(ctypes.byref(bad), ctypes.byref(w), FAKE, FAKE, None, None) == -1
    small = L.desc_from_config(get("longcat_zero_bf16"))
    assert 0 < L.moe_workspace_bytes(small, L.OP_LAYER) <= L.STATIC_WORKSPACE_BYTES


def test_static_workspace_size_matches_header(L):
    text = open(os.path.join(ROOT, "include", "moe.h"), encoding="utf-8").read()
    m = re.search(r"#define MOE_STATIC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.STATIC_WORKSPACE_BYTES


def test_stream_read_validates_before_any_launch(L):
    """moe_stream_read: null pointers, a size not a multiple of 16 and a
    misaligned buffer are MOE_ERR_INVALID_ARG before any launch; zero bytes
    launch nothing."""
    lib = L.load_library()
    assert lib.moe_stream_read(None, 1 << 20, FAKE, None) == -1
    assert lib.moe_stream_read(FAKE, 1 << 20, None, None) == -1
    assert lib.moe_stream_read(FAKE, (1 << 20) + 8, FAKE, None) == -1
    assert lib.moe_stream_read(FAKE + 4, 1 << 20, FAKE, None) == -1
    assert lib.moe_stream_read(None, 0, None, None) == 0


def test_stream_read_slices_match_header(L):
    text = open(os.path.join(ROOT, "include", "moe.h"), encoding="utf-8").read()
    m = re.search(r"#define MOE_STREAM_READ_WGS (\d+)", text)
    assert m and int(m.group(1)) == L.STREAM_READ_WGS
