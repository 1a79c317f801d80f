"""moe_layer_static (the entry point that allocates nothing: its workspace is
the library's own device array) against moe_layer with a caller workspace,
through the C ABI: two calls in a row, the second with fewer tokens, each
bit-identical to moe_layer on the same inputs. Runs alone in a fresh process
and after the other GPU tests."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from moe_expert_layer_fp32_amd import load_library
    load_library()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name,T_first,T_second,tile_rows",
                         [("longcat_zero_bf16", None, 77, 0), ("tiny_fp32", None, 13, 0),
                          ("dsv3_decode_share_bf16", 64, 40, 32)])
def test_layer_static_matches_layer(name, T_first, T_second, tile_rows):
    """tile_rows 32: the DeepSeek-style share (shared expert, group-limited
    selection) on 32-row decode tiles, whose gate/up reduction runs on the
    wavefronts of one workgroup, through moe_tuning in both calls."""
    import ctypes
    import gpu_util as U
    from moe_expert_layer_fp32_amd import lib as L
    from moe_expert_layer_fp32_amd import tuning as TU
    lay = U.device_layer(name)
    t = TU.to_struct(TU.limits(decode_tile_rows=tile_rows)) if tile_rows else None
    for T in (T_first or lay.cfg.T, T_second):
        x = lay.x[:T].contiguous()
        d = lay.desc_for(T)
        assert L.moe_workspace_bytes(d, L.OP_LAYER) <= L.STATIC_WORKSPACE_BYTES
        U.say(f"[gpu] moe_layer_static {name} T={T} tile_rows={tile_rows}")
        want = lay.layer(x, tuning=t)             # moe_layer with its own workspace
        got = torch.empty_like(want)
        aux = L.MoeAux(tuning=ctypes.pointer(t)) if t is not None else None
        L.moe_layer_static(d, lay.weights, x, got, aux)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want)), f"{name} T={T}"
