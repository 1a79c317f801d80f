"""GPU parity: every step of the HIP path (through the C ABI) against the CPU
oracle on the same seeded inputs.

Bars: routing tables bit-exact given the same ids; int8 activation codes
bit-exact; gate weights within 1e-5; outputs within max|err|/rms of 1e-5
(fp32), 2e-2 (bf16), 1e-2 (W8A8) beyond the single rounding to the output
type (the literal measure is asserted too where rounding allows it). Tokens
whose expert choice sits within rounding of a tie are checked for validity
only.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as U
from moe_inputs import get, make_inputs, make_routing
from moe_inputs.configs import MoEConfig
from moe_inputs.gen import bf16_to_f32
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

DECODE = ["tiny_fp32", "longcat_zero_bf16", "dsv3_decode_share_bf16", "pangu_moge_w8a8"]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from moe_expert_layer_fp32_amd import load_library
    load_library()


def _L():
    from moe_expert_layer_fp32_amd import lib as L
    from moe_expert_layer_fp32_amd.layer import DeviceLayer, to_device
    return L, DeviceLayer, to_device


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------
def _unpack_experts(buf: np.ndarray, G, K, N, S, elem_bytes, KF):
    """Inverse of the packed layout, written from its definition: per matrix,
    blocks of up to 8 fragment columns (16 columns each); inside a block the
    order is step kt, plane s, fragment j; a fragment holds lane q*16 + r
    (column r, reduction elements q*KF/4 + i)."""
    per = KF // 4
    dt = {4: np.float32, 2: np.uint16, 1: np.int8}[elem_bytes]
    NT, KT = N // 16, K // KF
    flat = buf.view(dt).reshape(G, -1)
    out = np.empty((G, S, K, N), dtype=dt)
    pos = 0
    for cb in range(0, NT, 8):
        w = min(8, NT - cb)
        n = KT * S * w * 64 * per
        blk = flat[:, pos:pos + n].reshape(G, KT, S, w, 4, 16, per)   # g kt s j q r i
        blk = blk.transpose(0, 2, 1, 4, 6, 3, 5)                       # g s kt q i j r
        out[:, :, :, cb * 16:(cb + w) * 16] = blk.reshape(G, S, K, w * 16)
        pos += n
    assert pos == flat.shape[1]
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16", "w8a8"])
def test_pack_expert_fragments_roundtrip(dtype):
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="pack", T=4, d=128, E=4, k=1, gate="softmax", n_ffn=3, inter=192,
                    shared_inter=64, dtype=dtype)
    inp = make_inputs(cfg)
    U.say(f"[gpu] pack roundtrip {dtype}")
    lay = DeviceLayer(cfg, inp)
    KF = {"f32": 4, "bf16": 32, "w8a8": 64}[dtype]
    eb = {"f32": 4, "bf16": 2, "w8a8": 1}[dtype]
    w13 = _unpack_experts(lay.w13.cpu().numpy(), 3, 128, 192, 2, eb, KF)
    assert np.array_equal(w13[:, 0], inp["w1"]) and np.array_equal(w13[:, 1], inp["w3"])
    w2 = _unpack_experts(lay.w2.cpu().numpy(), 3, 192, 128, 1, eb, KF)
    assert np.array_equal(w2[:, 0], inp["w2"])
    sw13 = _unpack_experts(lay.sw13.cpu().numpy(), 1, 128, 64, 2, eb, KF)
    assert np.array_equal(sw13[0, 0], inp["sw1"]) and np.array_equal(sw13[0, 1], inp["sw3"])


@pytest.mark.parametrize("name", ["tiny_fp32", "longcat_zero_bf16", "dsv3_decode_share_bf16"])
def test_router_planes_sum_exactly_to_router(name):
    L, DeviceLayer, to_device = _L()
    cfg = get(name).replace(n_ffn=0, n_zero=0, zero_begin=0, shared_inter=0, T=4)
    inp = make_inputs(cfg)
    U.say(f"[gpu] router planes {name}")
    lay = DeviceLayer(cfg, inp)
    buf = lay.router.cpu().numpy()
    Ep = (cfg.E + 15) // 16 * 16
    if cfg.dtype == "f32":
        w = _unpack_experts(buf, 1, cfg.d, Ep, 1, 4, 4)[0, 0]
        assert np.array_equal(w[:, :cfg.E], inp["w_router"]) and not w[:, cfg.E:].any()
        return
    planes = _unpack_experts(buf, 1, cfg.d, Ep, 3, 2, 32)[0]          # 3 x d x Ep bf16 bits
    vals = bf16_to_f32(planes).astype(np.float64)
    total = vals.sum(axis=0)
    assert np.array_equal(total[:, :cfg.E], inp["w_router"].astype(np.float64))
    # hi carries the leading bits: |mid| <= ulp(hi)/2, |lo| <= ulp(mid)/2
    assert np.all(np.abs(vals[1]) <= np.abs(vals[0]) * 2.0 ** -8 + 1e-45)


# ----------------------------------------------------------------------------
# router + top-k
# ----------------------------------------------------------------------------
ROUTE_CASES = [("tiny_fp32", None), ("tiny_fp32", 333), ("longcat_zero_bf16", None),
               ("dsv3_decode_share_bf16", None), ("pangu_moge_w8a8", None), ("prefill_zipf_bf16", 1024)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_topk(name, T):
    L, DeviceLayer, to_device = _L()
    cfg = get(name).replace(n_ffn=0, n_zero=0, zero_begin=0, shared_inter=0)
    if T:
        cfg = cfg.replace(T=T)
    inp = make_inputs(cfg)
    U.say(f"[gpu] route_topk {name} T={cfg.T}")
    lay = DeviceLayer(cfg, inp)
    idx, w = lay.route_topk()
    torch.cuda.synchronize()
    ref = dict(zip(("z", "scores", "idx", "w"), O.route(inp, cfg)))
    amb = U.compare_routing(cfg, ref, U.np_of(idx), U.np_of(w), U.x64_of(inp),
                            inp["w_router"].astype(np.float64))
    assert amb.mean() < 0.05


@pytest.mark.parametrize("E,k,gate", [(1, 1, "softmax"), (2, 2, "sigmoid"), (3, 2, "softmax"), (5, 4, "sigmoid"),
                                      (255, 16, "softmax")])
def test_route_expert_counts(E, k, gate):
    """Plain top-k over expert counts that leave lanes and slots of the
    gate's wavefront empty (4 experts per lane: E 1, 2, 3, 5) or one slot
    short of all 256 (E 255, the largest k)."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="expert_counts", T=70, d=128, E=E, k=k, gate=gate, n_ffn=min(E, 4), inter=64, dtype="bf16")
    inp = make_inputs(cfg)
    U.say(f"[gpu] route E={E} k={k} {gate}")
    lay = DeviceLayer(cfg, inp)
    idx, w = lay.route_topk()
    torch.cuda.synchronize()
    ref = dict(zip(("z", "scores", "idx", "w"), O.route(inp, cfg)))
    amb = U.compare_routing(cfg, ref, U.np_of(idx), U.np_of(w), U.x64_of(inp),
                            inp["w_router"].astype(np.float64))
    assert amb.mean() < 0.05


@pytest.mark.parametrize("E,n_group,topk_group,k,gate", [
    (96, 12, 3, 6, "sigmoid"),    # groups of 8 experts: 2 lanes each
    (64, 4, 2, 4, "softmax"),     # groups of 16: 4 lanes each
    (160, 5, 2, 8, "sigmoid"),    # groups of 32: 8 lanes each, 24 lanes past E
    (96, 8, 3, 6, "sigmoid"),     # groups of 12: 3 lanes, not a power of two
    (90, 15, 4, 8, "softmax"),    # groups of 6: not whole lanes
    (256, 2, 1, 8, "sigmoid"),    # groups of 128: 32 lanes, across rows of 16
    (64, 32, 6, 8, "sigmoid"),    # groups of 2: half a lane, 32 groups
])
def test_route_group_limited_shapes(E, n_group, topk_group, k, gate):
    """Group-limited selection over group sizes that are and are not whole
    blocks of at most 16 lanes (4 experts per lane): the gate scores groups
    inside their own lanes in the first case, one group at a time over the
    wavefront otherwise."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="groups", T=200, d=256, E=E, k=k, gate=gate, n_group=n_group, topk_group=topk_group,
                    dtype="bf16")
    inp = make_inputs(cfg)
    U.say(f"[gpu] route group-limited E={E} groups={n_group} keep={topk_group} k={k} {gate}")
    lay = DeviceLayer(cfg, inp)
    idx, w = lay.route_topk()
    torch.cuda.synchronize()
    ref = dict(zip(("z", "scores", "idx", "w"), O.route(inp, cfg)))
    amb = U.compare_routing(cfg, ref, U.np_of(idx), U.np_of(w), U.x64_of(inp),
                            inp["w_router"].astype(np.float64))
    assert amb.mean() < 0.05


@pytest.mark.parametrize("E,n_group,per_group_k,gate", [
    (64, 8, 2, "softmax"),     # groups of 8 (2 lanes): two quota rounds side by side
    (128, 16, 1, "sigmoid"),   # groups of 8, 16 groups
    (96, 4, 3, "sigmoid"),     # groups of 24: 6 lanes, not a power of two
    (60, 10, 1, "softmax"),    # groups of 6: not whole lanes
    (256, 2, 4, "sigmoid"),    # groups of 128: 32 lanes
])
def test_route_per_group_quota_shapes(E, n_group, per_group_k, gate):
    """Per-group quota selection (per_group_k from every group) over group
    sizes that are and are not whole blocks of at most 16 lanes: the groups'
    rounds run side by side in the first case, one group at a time
    otherwise."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="quota", T=200, d=256, E=E, k=n_group * per_group_k, gate=gate, n_group=n_group,
                    per_group_k=per_group_k, dtype="bf16")
    inp = make_inputs(cfg)
    U.say(f"[gpu] route quota E={E} groups={n_group} per_group_k={per_group_k} {gate}")
    lay = DeviceLayer(cfg, inp)
    idx, w = lay.route_topk()
    torch.cuda.synchronize()
    ref = dict(zip(("z", "scores", "idx", "w"), O.route(inp, cfg)))
    amb = U.compare_routing(cfg, ref, U.np_of(idx), U.np_of(w), U.x64_of(inp),
                            inp["w_router"].astype(np.float64))
    assert amb.mean() < 0.05


TIE_CASES = [
    # plain top-k: twins in different lanes and (21, 23) in one lane
    (dict(E=32, k=6), ((3, 17), (9, 30), (5, 12), (21, 23))),
    # per-group quota, groups of 8: twins in one lane (17, 19), in the two
    # lanes of one group (40, 45) and (3, 6)
    (dict(E=64, k=16, n_group=8, per_group_k=2), ((17, 19), (40, 45), (3, 6))),
]


@pytest.mark.parametrize("case", range(len(TIE_CASES)))
def test_route_exact_ties_go_to_lower_id(case):
    """Duplicated router columns give bit-identical logits on both sides; the
    lower expert id must win every such tie."""
    L, DeviceLayer, to_device = _L()
    shape, twins = TIE_CASES[case]
    for gate in ("softmax", "sigmoid"):
        cfg = MoEConfig(name="ties", T=96, d=256, gate=gate, dtype="bf16", **shape)
        inp = make_inputs(cfg)
        wr = inp["w_router"]
        for a, b in twins:
            wr[:, b] = wr[:, a]
        U.say(f"[gpu] exact ties {shape} {gate}")
        lay = DeviceLayer(cfg, inp)
        idx, w = lay.route_topk()
        ref = dict(zip(("z", "scores", "idx", "w"), O.route(inp, cfg)))
        got = U.np_of(idx)
        for a, b in twins:
            # whenever both twins are chosen the lower id comes first; when only
            # one is chosen it is the lower id
            for t in range(cfg.T):
                row = got[t].tolist()
                if b in row:
                    assert a in row and row.index(a) < row.index(b)
        U.compare_routing(cfg, ref, got, U.np_of(w), U.x64_of(inp), wr.astype(np.float64))


# ----------------------------------------------------------------------------
# permute
# ----------------------------------------------------------------------------
def _permute_case(T, k, E, seed, skew=0.0):
    cfg = MoEConfig(name="perm", T=T, d=64, E=E, k=k, gate="softmax", dtype="bf16")
    idx, _ = make_routing(cfg, seed=seed, skew=skew)
    return cfg, idx


PERMUTE_CASES = [(256, 8, 96, 1, 0.0), (512, 8, 256, 2, 0.0), (456, 8, 64, 3, 0.0), (8192, 8, 256, 4, 1.1),
                 (1, 1, 1, 5, 0.0), (1, 16, 16, 6, 0.0), (333, 3, 7, 7, 2.0), (65536, 16, 256, 8, 1.1),
                 (3000, 4, 32, 10, 0.0), (4096, 3, 3, 11, 1.5)]


@pytest.mark.parametrize("T,k,E,seed,skew", PERMUTE_CASES)
def test_permute_bit_exact(T, k, E, seed, skew):
    L, DeviceLayer, to_device = _L()
    cfg, idx = _permute_case(T, k, E, seed, skew)
    U.say(f"[gpu] permute T={T} k={k} E={E}")
    d = L.desc_from_config(cfg)
    ti = torch.from_numpy(idx).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * k, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.moe_permute(d, ti, counts, offsets, ss, sp, _permute_ws(L, d))
    want = O.routing_tables(idx, E)
    for got, ref, name in zip((counts, offsets, ss, sp), want, ("counts", "offsets", "sorted_slot", "slot_pos")):
        assert np.array_equal(U.np_of(got), ref), name


@pytest.mark.parametrize("T", [1000, 6000])   # one workgroup; three chunks
def test_permute_all_tokens_on_one_expert_and_empty_experts(T):
    L, DeviceLayer, to_device = _L()
    k, E = 3, 40
    idx = np.stack([np.array([7, 0, 39])] * T).astype(np.int32)
    cfg = MoEConfig(name="perm", T=T, d=64, E=E, k=k, gate="softmax", dtype="bf16")
    U.say("[gpu] permute skewed")
    counts, offsets, ss, sp = _run_permute(L, cfg, idx)
    want = O.routing_tables(idx, E)
    assert all(np.array_equal(a, b) for a, b in zip((counts, offsets, ss, sp), want))


def _permute_ws(L, d):
    n = L.moe_workspace_bytes(d, L.OP_PERMUTE)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


def _run_permute(L, cfg, idx):
    T, k, E = cfg.T, cfg.k, cfg.E
    ti = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    out = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    d = L.desc_from_config(cfg)
    L.moe_permute(d, ti, *out, _permute_ws(L, d))
    return [U.np_of(t) for t in out]


@pytest.mark.parametrize("T,k", [(300, 4), (2500, 4)])   # one workgroup; several chunks (10000 slots)
def test_permute_drops_out_of_range_ids(T, k):
    """Ids outside [0, E) are not counted and get slot_pos -1; the rest is the
    stable sort of the valid slots (library routine: numpy stable argsort)."""
    L, DeviceLayer, to_device = _L()
    cfg, idx = _permute_case(T, k, 32, 9)
    idx = idx.copy()
    idx[5, 1] = -1
    idx[17, 3] = 32
    idx[200, 0] = 1 << 20
    idx[T - 1, k - 1] = -7
    U.say("[gpu] permute out-of-range ids")
    counts, offsets, ss, sp = _run_permute(L, cfg, idx)
    flat = idx.reshape(-1)
    ok = (flat >= 0) & (flat < cfg.E)
    valid_slots = np.flatnonzero(ok)
    order = valid_slots[np.argsort(flat[ok], kind="stable")]
    assert np.array_equal(counts, np.bincount(flat[ok], minlength=cfg.E))
    assert offsets[-1] == ok.sum()
    assert np.array_equal(ss[: ok.sum()], order)
    assert np.all(sp[~ok] == -1)
    assert np.array_equal(sp[order], np.arange(ok.sum()))


# ----------------------------------------------------------------------------
# grouped FFN (routed and shared) on a given routing
# ----------------------------------------------------------------------------
FFN_CASES = [("tiny_fp32", None, 0.0), ("longcat_zero_bf16", None, 0.0), ("dsv3_decode_share_bf16", None, 0.0),
             ("pangu_moge_w8a8", None, 0.0), ("dsv3_decode_share_bf16", 300, 1.5)]


def _expected_rows(cfg, inp, idx, tables):
    """Oracle rows in sorted order, and (W8A8) the per-element allowance for
    int8 codes of h that are near-ties."""
    counts, offsets, ss, sp = tables
    base = offsets[cfg.ffn_begin]
    R = offsets[cfg.ffn_begin + cfg.n_ffn] - base
    x = np.asarray(O.x_f32(inp), np.float32)
    rows = np.zeros((R, cfg.d))
    allow = np.zeros((R, cfg.d))
    for el in range(cfg.n_ffn):
        e = cfg.ffn_begin + el
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        X = x[ss[r0:r1] // cfg.k]
        if cfg.dtype == "w8a8":
            u, parts = O.swiglu_w8a8(X, inp["w1"][el], inp["s1"][el], inp["w3"][el], inp["s3"][el],
                                     inp["w2"][el], inp["s2"][el], return_parts=True)
            allow[r0 - base:r1 - base] = U.h_code_flip_allowance(
                parts["h"].astype(np.float32), parts["sh"], inp["w2"][el], inp["s2"][el])
        else:
            u = O.expert_ffn(inp, cfg, el, X)
        rows[r0 - base:r1 - base] = u
    return rows, allow


@pytest.mark.parametrize("name,T,skew", FFN_CASES)
def test_grouped_ffn_routed(name, T, skew):
    L, DeviceLayer, to_device = _L()
    cfg, inp = U.inputs(name, T)
    lay = U.device_layer(name, T)
    idx, _ = make_routing(cfg, seed=11, skew=skew)
    U.say(f"[gpu] grouped_ffn routed {name} T={cfg.T} skew={skew}")
    counts, offsets, ss, sp = lay.permute(torch.from_numpy(idx).cuda())
    rows = lay.grouped_ffn(L.FFN_ROUTED, offsets, ss)
    torch.cuda.synchronize()
    tables = O.routing_tables(idx, cfg.E)
    want, allow = _expected_rows(cfg, inp, idx, tables)
    got = U.np_of(rows)[: want.shape[0]]
    lit, _ = U.output_errors(got, want, "f32")
    rms = float(np.sqrt(np.mean(want ** 2)))
    beyond_flips = float(np.maximum(np.abs(got - want) - allow, 0).max() / rms)
    U.record(test="grouped_ffn_routed", cfg=cfg.name, T=cfg.T, skew=skew, rows=int(want.shape[0]),
             err_rows_literal=lit, err_rows_beyond_code_flips=beyond_flips,
             rows_with_near_tie_codes=int((allow > 0).any(axis=1).sum()))
    assert beyond_flips <= U.TOL[cfg.dtype], f"rows error {beyond_flips} (literal {lit})"


# rows per resident expert at the tile boundaries: none, one, 63/64/65
# (one 64-row tile, or the switch from the 64-row to the 128-row launch at
# prefill sizes), 127/128/129 (one or two 128-row tiles, two or three 64-row)
BOUNDARY_COUNTS = (0, 1, 63, 64, 65, 127, 128, 129)


@pytest.mark.parametrize("T", [600, 1100])
@pytest.mark.parametrize("dtype", ["bf16", "w8a8"])
def test_grouped_ffn_tile_boundaries(T, dtype):
    """Resident experts with exactly 0, 1, 63, 64, 65, 127, 128 and 129 rows,
    in the decode regime (600 tokens: 64-row tiles) and the prefill regime
    (1100 tokens: 64-row launch up to 64 rows, 128-row launch above); the
    other tokens go to non-resident experts. Every row against the oracle."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="bounds", T=T, d=256, E=16, k=1, gate="softmax", n_ffn=8, inter=128, dtype=dtype)
    inp = make_inputs(cfg, seed=7)
    lay = DeviceLayer(cfg, inp)
    g = np.random.default_rng(19)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(BOUNDARY_COUNTS)])
    rest = g.integers(8, 16, size=T - ids.size).astype(np.int32)
    idx = g.permutation(np.concatenate([ids, rest])).reshape(T, 1).astype(np.int32)
    U.say(f"[gpu] tile boundaries T={T} {dtype} counts={BOUNDARY_COUNTS}")
    counts, offsets, ss, sp = lay.permute(torch.from_numpy(idx).cuda())
    rows = lay.grouped_ffn(L.FFN_ROUTED, offsets, ss)
    torch.cuda.synchronize()
    assert U.np_of(counts)[:8].tolist() == list(BOUNDARY_COUNTS)
    want, allow = _expected_rows(cfg, inp, idx, O.routing_tables(idx, cfg.E))
    got = U.np_of(rows)[: want.shape[0]]
    rms = float(np.sqrt(np.mean(want ** 2)))
    beyond_flips = float(np.maximum(np.abs(got - want) - allow, 0).max() / rms)
    U.record(test="grouped_ffn_tile_boundaries", T=T, dtype=dtype, err_rows_beyond_code_flips=beyond_flips)
    assert beyond_flips <= U.TOL[dtype], f"rows error {beyond_flips}"


# rows per resident expert around the 256-row tiles of the prefill regime:
# empty, streaming (<= 64), 128-row tiles (65 .. 255), one 256-row tile
# (256), a ragged second one (257), and two or three 256-row tiles
BIG_COUNTS = (0, 1, 64, 65, 255, 256, 257, 511, 512, 513)


@pytest.mark.parametrize("inter", [128, 256])
def test_grouped_ffn_big_tile_boundaries(inter):
    """Prefill regime (2900 tokens, bf16): resident experts with 0, 1, 64,
    65, 255, 256, 257, 511, 512 and 513 rows, so every row-count class runs
    (64-row streaming tiles, 128-row tiles, 256-row tiles with full and
    ragged last tiles); every row against the oracle, plus the shared expert
    over all 2900 tokens in 256-row tiles (a ragged last m-tile)."""
    L, DeviceLayer, to_device = _L()
    T = 2900
    cfg = MoEConfig(name="bigtiles", T=T, d=256, E=16, k=1, gate="softmax", n_ffn=10, inter=inter,
                    shared_inter=256, dtype="bf16")
    inp = make_inputs(cfg, seed=8)
    lay = DeviceLayer(cfg, inp)
    g = np.random.default_rng(23)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(BIG_COUNTS)])
    rest = g.integers(10, 16, size=T - ids.size).astype(np.int32)
    idx = g.permutation(np.concatenate([ids, rest])).reshape(T, 1).astype(np.int32)
    U.say(f"[gpu] big tile boundaries T={T} inter={inter} counts={BIG_COUNTS}")
    counts, offsets, ss, sp = lay.permute(torch.from_numpy(idx).cuda())
    rows = lay.grouped_ffn(L.FFN_ROUTED, offsets, ss)
    shared = lay.grouped_ffn(L.FFN_SHARED)
    torch.cuda.synchronize()
    assert U.np_of(counts)[:10].tolist() == list(BIG_COUNTS)
    want, _ = _expected_rows(cfg, inp, idx, O.routing_tables(idx, cfg.E))
    got = U.np_of(rows)[: want.shape[0]]
    lit, _ = U.output_errors(got, want, "f32")
    U.record(test="grouped_ffn_big_tile_boundaries", inter=inter, err_rows_literal=lit)
    assert lit <= U.TOL["bf16"], f"routed rows error {lit}"
    want_s = O.shared_ffn(inp, cfg, np.asarray(O.x_f32(inp), np.float32))
    lit_s, _ = U.output_errors(U.np_of(shared), want_s, "f32")
    U.record(test="grouped_ffn_big_tile_boundaries_shared", inter=inter, err_rows_literal=lit_s)
    assert lit_s <= U.TOL["bf16"], f"shared rows error {lit_s}"


@pytest.mark.parametrize("policy", [
    dict(prefill_tokens=256, stream_max_rows=100, big_min_rows=300, dense_big_rows=512),
    dict(prefill_tokens=256, stream_max_rows=16, big_min_rows=64, dense_big_rows=256),
    dict(prefill_tokens=4096),                       # the decode regime at 1500 tokens
])
def test_layer_tile_policy(policy):
    """moe_layer under non-default tile choices (moe_tuning: the prefill
    threshold, theta of the weight-streaming class, the 256-row class of
    experts and of dense products), one and two streams, against the
    oracle; the routing tables are those of the default call."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    cfg = MoEConfig(name="policy", T=1500, d=512, E=32, k=4, gate="sigmoid", n_ffn=20, inter=256,
                    shared_inter=256, dtype="bf16", bias=("zipf", 1.1))
    inp = make_inputs(cfg, seed=4)
    lay = DeviceLayer(cfg, inp)
    t = L.MoeTuning(**policy)
    U.say(f"[gpu] layer tile policy {policy}")
    y = _check_layer(cfg, inp, lay, tuning=t)
    y2 = _check_layer(cfg, inp, lay, second=SecondStream(), tuning=t)
    y0 = lay.layer()
    torch.cuda.synchronize()
    _, dev = U.output_errors(U.np_of(y), U.np_of(y0).astype(np.float64), cfg.dtype)
    U.record(test="layer_tile_policy", policy=policy, err_vs_default=dev)
    assert torch.equal(_bits(y), _bits(y2))


@pytest.mark.parametrize("name", ["longcat_zero_bf16", "pangu_moge_w8a8"])
def test_layer_writes_nothing_outside_its_buffers(name):
    """Guard bands around y and every moe_aux output buffer (filled with a
    fixed byte pattern) are untouched after a layer call, and the routed rows
    and h buffers are not written past the R rows the routing produced."""
    L, DeviceLayer, to_device = _L()
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    U.say(f"[gpu] guard bands {name}")
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    G = 4096                      # guard bytes on each side
    PAT = 0x5A

    def guarded(nbytes):
        buf = torch.full((nbytes + 2 * G,), PAT, dtype=torch.uint8, device="cuda")
        return buf, buf[G:G + nbytes]

    shapes = dict(topk_idx=T * k * 4, topk_w=T * k * 4, counts=E * 4, offsets=(E + 1) * 4, sorted_slot=T * k * 4,
                  slot_pos=T * k * 4, h=T * k * cfg.inter * (2 if cfg.dtype == "bf16" else 4),
                  rows=T * k * d * (2 if cfg.dtype == "bf16" else 4))
    if cfg.dtype == "w8a8":
        shapes.update(q_x=T * d, s_x=T * 4, q_h=T * k * cfg.inter, s_h=T * k * 4)
    bufs = {n: guarded(b) for n, b in shapes.items()}
    ybuf, yv = guarded(T * d * 2)
    aux = L.MoeAux(**{n: L.ptr(v) for n, (_, v) in bufs.items()})
    lay.layer(y=yv.view(torch.bfloat16).view(T, d), aux=aux)
    torch.cuda.synchronize()
    for n, (buf, _) in list(bufs.items()) + [("y", (ybuf, yv))]:
        b = U.np_of(buf)
        assert (b[:G] == PAT).all() and (b[-G:] == PAT).all(), f"{n} written outside its buffer"
    offs = U.np_of(bufs["offsets"][1].view(torch.int32))
    R = int(offs[cfg.ffn_begin + cfg.n_ffn] - offs[cfg.ffn_begin])
    for n, width in (("rows", d * (2 if cfg.dtype == "bf16" else 4)), ("h", cfg.inter * (2 if cfg.dtype == "bf16" else 4))):
        tail = U.np_of(bufs[n][1])[R * width:]
        assert (tail == PAT).all(), f"{n} written past row {R}"


@pytest.mark.parametrize("name", ["dsv3_decode_share_bf16", "pangu_moge_w8a8"])
def test_grouped_ffn_shared(name):
    L, DeviceLayer, to_device = _L()
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    U.say(f"[gpu] grouped_ffn shared {name}")
    rows = lay.grouped_ffn(L.FFN_SHARED)
    X = np.asarray(O.x_f32(inp), np.float32)
    allow = 0.0
    if cfg.dtype == "w8a8":
        want, parts = O.swiglu_w8a8(X, inp["sw1"], inp["ss1"], inp["sw3"], inp["ss3"], inp["sw2"], inp["ss2"],
                                    return_parts=True)
        allow = U.h_code_flip_allowance(parts["h"].astype(np.float32), parts["sh"], inp["sw2"], inp["ss2"])
    else:
        want = O.shared_ffn(inp, cfg, X)
    got = U.np_of(rows)
    lit, _ = U.output_errors(got, want, "f32")
    beyond = float(np.maximum(np.abs(got - want) - allow, 0).max() / np.sqrt(np.mean(want ** 2)))
    U.record(test="grouped_ffn_shared", cfg=cfg.name, T=cfg.T, err_rows_literal=lit,
             err_rows_beyond_code_flips=beyond)
    assert beyond <= U.TOL[cfg.dtype], f"shared rows error {beyond} (literal {lit})"


# ----------------------------------------------------------------------------
# combine on given rows
# ----------------------------------------------------------------------------
# 1088 columns over 37 tokens: a thread's second 1024-column pass holds
# only a 64-column tail
COMBINE_RAGGED = MoEConfig(name="combine_cols", T=37, d=1088, E=16, k=4, gate="softmax", ffn_begin=0, n_ffn=8,
                           zero_begin=8, n_zero=4, inter=64, dtype="bf16")


@pytest.mark.parametrize("name", ["tiny_fp32", "longcat_zero_bf16", "combine_cols"])
@pytest.mark.parametrize("with_shared", [False, True])
def test_combine(name, with_shared):
    """moe_combine on given expert rows (random), its own routing tables, and
    (with_shared) a given shared-expert row per token: y = shared + the
    weighted rows of resident experts + the weighted x of identity experts,
    against the same sum written out in fp64."""
    L, DeviceLayer, to_device = _L()
    if name == COMBINE_RAGGED.name:
        cfg = COMBINE_RAGGED
        inp = make_inputs(cfg)
        lay = DeviceLayer(cfg, inp)
    else:
        cfg, inp = U.inputs(name)
        lay = U.device_layer(name)
    idx, w = make_routing(cfg, seed=21)
    rng = np.random.default_rng(22)
    R = cfg.T * cfg.k
    rows = rng.standard_normal((R, cfg.d)).astype(np.float32)
    shared = rng.standard_normal((cfg.T, cfg.d)).astype(np.float32) if with_shared else None
    U.say(f"[gpu] combine {name} shared={with_shared}")
    counts, offsets, ss, sp = lay.permute(torch.from_numpy(idx).cuda())
    # the shared rows are read only when the descriptor has a shared expert
    desc = L.desc_from_config(cfg.replace(shared_inter=64) if with_shared else cfg)
    xdev = lay.x
    y = torch.empty((cfg.T, cfg.d), dtype=lay.xdtype, device="cuda")
    L.moe_combine(desc, xdev, torch.from_numpy(rows).cuda(),
                  torch.from_numpy(shared).cuda() if with_shared else None, torch.from_numpy(idx).cuda(),
                  torch.from_numpy(w).cuda(), offsets, sp, y)
    torch.cuda.synchronize()
    _, off_ref, _, sp_ref = O.routing_tables(idx, cfg.E)
    x = np.asarray(O.x_f32(inp), np.float64)
    Uu = np.zeros((cfg.T, cfg.k, cfg.d))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = idx[t, j]
            kind = O.expert_kind(cfg, e)
            if kind == "ffn":
                Uu[t, j] = rows[sp_ref[t * cfg.k + j] - off_ref[cfg.ffn_begin]]
            elif kind == "identity":
                Uu[t, j] = x[t]
    want = O.weighted_sum(Uu, w, None if shared is None else shared.astype(np.float64))
    _, beyond = U.output_errors(U.np_of(y), want, cfg.dtype)
    assert beyond <= 1e-6
    if with_shared:   # the shared rows really entered the sum
        _, without = U.output_errors(U.np_of(y), O.weighted_sum(Uu, w, None), cfg.dtype)
        assert without > 0.1


@pytest.mark.parametrize("T,skew", [(2048, 0.0), (2100, 1.5)])
def test_grouped_ffn_large_tiles(T, skew):
    """Many rows per weight: prefill-sized experts (hundreds of rows, 128-row
    tiles, the skewed case mixing in 64-row tiles) and a dense shared expert
    of 2048+ tokens with a split reduction (ragged token count)."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="bigtile", T=T, d=512, E=8, k=2, gate="softmax", n_ffn=8, inter=256, shared_inter=512,
                    dtype="bf16")
    inp = make_inputs(cfg)
    lay = DeviceLayer(cfg, inp)
    idx, _ = make_routing(cfg, seed=5, skew=skew)
    U.say(f"[gpu] large tiles T={T} skew={skew} counts={np.bincount(idx.ravel(), minlength=8).tolist()}")
    counts, offsets, ss, sp = lay.permute(torch.from_numpy(idx).cuda())
    rows = lay.grouped_ffn(L.FFN_ROUTED, offsets, ss)
    shared = lay.grouped_ffn(L.FFN_SHARED)
    torch.cuda.synchronize()
    want, _ = _expected_rows(cfg, inp, idx, O.routing_tables(idx, cfg.E))
    got = U.np_of(rows)[: want.shape[0]]
    lit, beyond = U.output_errors(got, want, "f32")
    U.record(test="grouped_ffn_large_tiles", T=T, skew=skew, err_rows_literal=lit)
    assert lit <= U.TOL["bf16"], f"routed rows error {lit}"
    X = np.asarray(O.x_f32(inp), np.float32)
    want_s = O.shared_ffn(inp, cfg, X)
    lit_s, _ = U.output_errors(U.np_of(shared), want_s, "f32")
    U.record(test="grouped_ffn_large_tiles_shared", T=T, err_rows_literal=lit_s)
    assert lit_s <= U.TOL["bf16"], f"shared rows error {lit_s}"


@pytest.mark.parametrize("T", [4200, 4096])
def test_grouped_ffn_shared_panel_order(T):
    """A dense expert with many 128-row tiles and no split reduction, walked
    in panels of 8 m-tiles: 4200 rows give 33 m-tiles (a ragged last tile
    and a last panel of one m-tile), 4096 rows 32; gate/up and down both 8
    column blocks. Checked on every row."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="panels", T=T, d=1024, E=8, k=2, gate="softmax", n_ffn=2, inter=64, shared_inter=1024,
                    dtype="bf16")
    inp = make_inputs(cfg)
    lay = DeviceLayer(cfg, inp)
    U.say(f"[gpu] shared expert panel order T={T} d={cfg.d} I_s={cfg.shared_inter}")
    shared = lay.grouped_ffn(L.FFN_SHARED)
    torch.cuda.synchronize()
    X = np.asarray(O.x_f32(inp), np.float32)
    want = O.shared_ffn(inp, cfg, X)
    lit, _ = U.output_errors(U.np_of(shared), want, "f32")
    U.record(test="grouped_ffn_shared_panel_order", T=T, err_rows_literal=lit)
    assert lit <= U.TOL["bf16"], f"shared rows error {lit}"


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
LAYER_CASES = [("tiny_fp32", None), ("tiny_fp32", 333), ("longcat_zero_bf16", None), ("longcat_zero_bf16", 77),
               ("dsv3_decode_share_bf16", None), ("dsv3_decode_share_bf16", 129), ("pangu_moge_w8a8", None)]


ANY_SHAPE_TOL = 1e-4


def _check_layer(cfg, inp, lay, tokens=None, ws=None, second=None, tuning=None, any_shape=False):
    """moe_layer against the oracle. any_shape (shapes drawn at random, where
    one token can be a large share of the batch and a few expert rows can
    make up the output): near-tie tokens may be up to a quarter of the batch
    (or one token), a batch whose exact output is all zero must come out all
    zero, and the allowance also covers what the layer's intermediate
    precision may move each expert row (gpu_util.layer_allowance: bf16 h and
    rows, W8A8 h codes at a rounding boundary, fp32 accumulation)."""
    y, t = lay.layer_with_tables(ws=ws, second=second, tuning=tuning)
    torch.cuda.synchronize()
    idx_gpu, w_gpu = U.np_of(t["topk_idx"]), U.np_of(t["topk_w"])
    ref = O.moe_layer(inp, cfg, tokens=tokens)
    sel = slice(None) if tokens is None else np.asarray(tokens)
    x64 = U.x64_of(inp)[sel]
    amb = U.compare_routing(cfg, ref, idx_gpu[sel], w_gpu[sel], x64, inp["w_router"].astype(np.float64))
    if any_shape:
        assert amb.sum() <= max(1, amb.size // 4), f"{int(amb.sum())} near-tie tokens of {amb.size}"
    else:
        assert amb.mean() < 0.05
    clear = ~amb
    y_all = U.np_of(y)[sel]
    y_gpu = y_all[clear]
    if any_shape and clear.any() and not np.any(ref["y"][clear]):
        assert not np.any(y_gpu), "exact output is zero"
        lit = beyond = 0.0
    elif any_shape and clear.any():
        tok = np.arange(cfg.T)[sel][clear]
        rows = U.layer_allowance(cfg, inp, ref["idx"][clear], ref["w"][clear], tokens=tok)
        ref_c = ref["y"][clear]
        rms = float(np.sqrt(np.mean(ref_c ** 2)))
        diff = np.abs(y_gpu - ref_c)
        allow = U.half_ulp(np.maximum(np.abs(ref_c), np.abs(y_gpu)), cfg.dtype) + rows
        lit, beyond = float(diff.max() / rms), float(np.maximum(diff - allow, 0).max() / rms)
    else:
        lit, beyond = U.output_errors(y_gpu, ref["y"][clear], cfg.dtype)
    # Near-tie tokens: the oracle rerun on the GPU's own ids (downstream on
    # identical top-k indices), weights and outputs compared on every one.
    beyond_amb = 0.0
    if amb.any():
        tok_all = np.arange(cfg.T)[sel]
        amb_tok = tok_all[amb]
        ref_amb = O.moe_layer(inp, cfg, tokens=amb_tok, topk_idx=idx_gpu[sel][amb])
        werr = float(np.abs(w_gpu[sel][amb] - ref_amb["w"]).max())
        assert werr <= 1e-5, f"near-tie gate weights under identical ids: {werr}"
        # rms of the whole compared batch, so a handful of tokens is measured
        # on the same scale as the rest
        rms_all = float(np.sqrt(np.mean(ref["y"][clear] ** 2))) if clear.any() else 1.0
        if any_shape and rms_all == 0.0:
            rms_all = max(float(np.sqrt(np.mean(ref_amb["y"] ** 2))), 1e-30)
        diff = np.abs(y_all[amb] - ref_amb["y"])
        allow = U.half_ulp(np.maximum(np.abs(ref_amb["y"]), np.abs(y_all[amb])), cfg.dtype)
        if any_shape:
            allow = allow + U.layer_allowance(cfg, inp, idx_gpu[sel][amb], ref_amb["w"], tokens=amb_tok)
        beyond_amb = float(np.maximum(diff - allow, 0).max() / rms_all)
    U.say(f"    {cfg.name} T={cfg.T}: max|err|/rms literal {lit:.3e} beyond-rounding {beyond:.3e} "
          f"near-tie tokens {int(amb.sum())} (their error under identical ids {beyond_amb:.3e})")
    U.record(test="layer", cfg=cfg.name, T=cfg.T, sampled=None if tokens is None else len(tokens),
             err_literal=lit, err_beyond_rounding=beyond, near_tie_tokens=int(amb.sum()),
             near_tie_err_beyond_rounding=beyond_amb)
    # any_shape: beyond the allowance the residual is fp32 arithmetic (measured
    # <= 1.1e-6 of rms over 568 shapes), so the bar is 1e-4 for every dtype
    tol = min(U.TOL[cfg.dtype], ANY_SHAPE_TOL) if any_shape else U.TOL[cfg.dtype]
    assert beyond <= tol, f"error beyond rounding {beyond} > {tol}"
    assert beyond_amb <= tol, f"near-tie error beyond rounding {beyond_amb} > {tol}"
    # routing tables of the layer are the stable sort of its own ids
    counts, offsets, ss, sp = (U.np_of(t[n]) for n in ("counts", "offsets", "sorted_slot", "slot_pos"))
    flat = idx_gpu.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=cfg.E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(ss, np.argsort(flat, kind="stable"))
    assert np.array_equal(sp[ss], np.arange(flat.size))
    if tokens is None and not amb.any():
        assert all(np.array_equal(a, b) for a, b in zip((counts, offsets, ss, sp),
                                                          O.routing_tables(ref["idx"], cfg.E)))
    if cfg.dtype == "w8a8":
        q, s = O.quantise_rows(np.asarray(O.x_f32(inp), np.float32))
        assert np.array_equal(U.np_of(t["q_x"]), q)
        assert np.array_equal(U.np_of(t["s_x"]).view(np.uint32), s.view(np.uint32))
    return y


@pytest.mark.parametrize("name,T", LAYER_CASES)
def test_layer(name, T):
    cfg, inp = U.inputs(name, T)
    lay = U.device_layer(name, T)
    U.say(f"[gpu] layer {name} T={cfg.T}")
    _check_layer(cfg, inp, lay)


PREFILL_SAMPLED_TOKENS = 512


def test_layer_prefill_full_size():
    """The full prefill workload (T 8192, d 7168, 32 of 256 experts resident,
    Zipf popularity) in the launch configuration bench.py times (shared
    expert on a second stream), against the oracle:
    - the ids of all 8192 tokens (exact where clear of a tie, valid within
      rounding where not) and their gate weights;
    - the layer output on 512 sampled tokens (near-tie tokens under the
      GPU's own ids);
    - every expert output row (moe_aux.rows) of the largest resident expert,
      the smallest non-empty one, and the experts either side of the 64-row
      split (64-row weight-streaming tiles below, 128-row tiles above), at
      K = 7168, against the oracle's FFN of the same tokens."""
    from moe_expert_layer_fp32_amd.layer import SecondStream
    cfg, inp = U.inputs("prefill_zipf_bf16")
    lay = U.device_layer("prefill_zipf_bf16")
    U.say("[gpu] layer prefill_zipf_bf16 T=8192 (full size, two streams, intermediates)")
    y, t = lay.layer_with_tables(second=SecondStream(), intermediates=True)
    torch.cuda.synchronize()
    idx_gpu, w_gpu = U.np_of(t["topk_idx"]), U.np_of(t["topk_w"])
    x64, wr64 = U.x64_of(inp), inp["w_router"].astype(np.float64)
    U.say("    oracle routing of all 8192 tokens")
    z, sc, idx, w = O.route(inp, cfg)
    amb = U.compare_routing(cfg, dict(z=z, scores=sc, idx=idx, w=w), idx_gpu, w_gpu, x64, wr64)
    assert amb.mean() < 0.05
    U.record(test="prefill_full_size_routing", tokens=cfg.T, near_tie_tokens=int(amb.sum()))

    # layer output on sampled tokens, downstream on the GPU's own ids
    toks = np.sort(np.random.default_rng(5).choice(cfg.T, PREFILL_SAMPLED_TOKENS, replace=False))
    U.say(f"    oracle layer on {toks.size} sampled tokens")
    ref = O.moe_layer(inp, cfg, tokens=toks, topk_idx=idx_gpu[toks])
    y_s = U.np_of(y)[toks]
    lit, beyond = U.output_errors(y_s, ref["y"], cfg.dtype)
    U.say(f"    sampled output: literal {lit:.3e} beyond rounding {beyond:.3e}")
    U.record(test="prefill_full_size_output", sampled=int(toks.size), err_literal=lit, err_beyond_rounding=beyond)
    assert beyond <= U.TOL[cfg.dtype]

    # expert output rows of chosen experts, every row
    counts, offsets, ss = (U.np_of(t[n]) for n in ("counts", "offsets", "sorted_slot"))
    res = counts[cfg.ffn_begin:cfg.ffn_begin + cfg.n_ffn]
    nz = np.flatnonzero(res > 0)
    small = nz[res[nz] <= 64]
    large = nz[res[nz] > 64]
    pick = {"largest": int(nz[np.argmax(res[nz])]), "smallest": int(nz[np.argmin(res[nz])])}
    if small.size:
        pick["largest <= 64 rows"] = int(small[np.argmax(res[small])])
    if large.size:
        pick["smallest > 64 rows"] = int(large[np.argmin(res[large])])
    base = offsets[cfg.ffn_begin]
    X32 = np.asarray(O.x_f32(inp), np.float32)
    for what, el in pick.items():
        e = cfg.ffn_begin + el
        r0, r1 = offsets[e], offsets[e + 1]
        tokens = ss[r0:r1] // cfg.k
        U.say(f"    rows of expert {e} ({what}, {r1 - r0} rows)")
        got = U.np_of(t["rows"][r0 - base:r1 - base])
        want = O.expert_ffn(inp, cfg, el, X32[tokens])
        lit_r, beyond_r = U.output_errors(got, want, "bf16")
        U.record(test="prefill_full_size_rows", expert=e, which=what, rows=int(r1 - r0), err_literal=lit_r,
                 err_beyond_rounding=beyond_r)
        assert beyond_r <= U.TOL["bf16"], f"expert {e} ({what}): {beyond_r}"


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def _check_w8a8_integer_products(cfg, inp, t, silu_exact):
    """The W8A8 layer's integer products through its own intermediates:
    - h codes and scales: bit-exact against quantising the GPU's own h;
    - down projection: every expert output row bit-exact against the exact
      integer product of the GPU's own h codes with the int8 weights, scaled
      as the kernel scales its int32 accumulator (float(acc) * s_h * s_w2,
      each product rounded to fp32);
    - gate/up (silu_exact): h bit-exact against the exact integer products of
      the int8 x codes, scaled the same way, when every gate value is large
      enough (>= 20) that the kernel's SiLU returns its argument exactly;
      else within a few fp32 ulps of SiLU of those scaled products.
    A one-step error in an int32 accumulator below 2^24 changes the fp32
    value it is converted to, and with it these results."""
    offsets, ss = U.np_of(t["offsets"]), U.np_of(t["sorted_slot"])
    qx, sx = U.np_of(t["q_x"]), U.np_of(t["s_x"])
    q_ref, s_ref = O.quantise_rows(np.asarray(O.x_f32(inp), np.float32))
    assert np.array_equal(qx, q_ref) and np.array_equal(sx.view(np.uint32), s_ref.view(np.uint32))
    h, qh, sh, rows = (U.np_of(t[n]) for n in ("h", "q_h", "s_h", "rows"))
    base = offsets[cfg.ffn_begin]
    max_acc = 0
    for el in range(cfg.n_ffn):
        e = cfg.ffn_begin + el
        r0, r1 = offsets[e] - base, offsets[e + 1] - base
        if r1 == r0:
            continue
        tok = ss[offsets[e]:offsets[e + 1]] // cfg.k
        A = O.int_matmul(qx[tok], inp["w1"][el])
        B = O.int_matmul(qx[tok], inp["w3"][el])
        ga = _f32(_f32(_f32(A) * sx[tok][:, None]) * _f32(inp["s1"][el])[None, :])
        up = _f32(_f32(_f32(B) * sx[tok][:, None]) * _f32(inp["s3"][el])[None, :])
        hg = h[r0:r1]
        if silu_exact:
            assert ga.min() >= 20.0, "precondition of the exact SiLU"
            assert np.array_equal(hg.view(np.uint32), _f32(ga * up).view(np.uint32)), f"h of expert {e}"
        else:
            want = O.silu(ga.astype(np.float64)) * up.astype(np.float64)
            tol = 8 * 2.0 ** -23 * np.abs(want) + 1e-6 * np.abs(want).max()
            assert np.all(np.abs(hg - want) <= tol), f"h of expert {e}"
        q_own, s_own = O.quantise_rows(hg)
        assert np.array_equal(qh[r0:r1], q_own) and np.array_equal(sh[r0:r1].view(np.uint32), s_own.view(np.uint32))
        Y = O.int_matmul(qh[r0:r1], inp["w2"][el])
        max_acc = max(max_acc, float(np.abs(Y).max()), float(np.abs(A).max()), float(np.abs(B).max()))
        want_rows = _f32(_f32(_f32(Y) * sh[r0:r1][:, None]) * _f32(inp["s2"][el])[None, :])
        assert np.array_equal(rows[r0:r1].view(np.uint32), want_rows.view(np.uint32)), f"rows of expert {e}"
    return max_acc


def test_w8a8_integer_products_full_layer():
    """The W8A8 workload (T 456, d 5120, 64 experts) through moe_layer's own
    intermediates: down projection and h codes bit-exact, gate/up within the
    SiLU's few ulps of the exact integer products."""
    cfg, inp = U.inputs("pangu_moge_w8a8")
    lay = U.device_layer("pangu_moge_w8a8")
    U.say("[gpu] W8A8 integer products pangu_moge_w8a8 (full layer)")
    _, t = lay.layer_with_tables(intermediates=True)
    torch.cuda.synchronize()
    max_acc = _check_w8a8_integer_products(cfg, inp, t, silu_exact=False)
    U.record(test="w8a8_integer_products_full_layer", max_abs_accumulator=max_acc)


@pytest.mark.parametrize("T,E,k,inter", [(64, 8, 2, 256), (300, 64, 4, 512)])
def test_w8a8_integer_products_exact(T, E, k, inter):
    """Bit-exact int32 accumulators of both W8A8 products: non-negative x and
    gate weights, gate scales raised so every gate value is >= 20, where the
    kernel's SiLU is exactly its argument. 8 experts of inter 256 split the
    gate/up reduction over two workgroups per tile (partial sums added by the
    reduce pass); 64 experts of inter 512 run unsplit."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="w8exact", T=T, d=1024, E=E, k=k, gate="softmax", n_ffn=E, inter=inter, dtype="w8a8")
    inp = make_inputs(cfg, seed=3)
    inp["x"] = inp["x"] & np.uint16(0x7FFF)                 # bf16 bits: clear the sign
    inp["w1"] = np.abs(inp["w1"]).astype(np.int8)
    qx, sx = O.quantise_rows(np.asarray(O.x_f32(inp), np.float32))
    for el in range(cfg.n_ffn):
        A = O.int_matmul(qx, inp["w1"][el])
        a_min = (A * sx[:, None].astype(np.float64) * inp["s1"][el][None, :].astype(np.float64)).min()
        if a_min < 24.0:
            inp["s1"][el] = (inp["s1"][el] * np.float32(24.0 / max(a_min, 1e-3))).astype(np.float32)
    lay = DeviceLayer(cfg, inp)
    U.say(f"[gpu] W8A8 integer products exact T={T} E={E} inter={inter}")
    _, t = lay.layer_with_tables(intermediates=True)
    torch.cuda.synchronize()
    max_acc = _check_w8a8_integer_products(cfg, inp, t, silu_exact=True)
    assert max_acc < 2 ** 24
    U.record(test="w8a8_integer_products_exact", T=T, max_abs_accumulator=max_acc)


@pytest.mark.parametrize("T,d,inter", [(33, 8256, 64), (17, 1088, 320), (5, 64, 6208)])
def test_w8a8_code_shapes(T, d, inter):
    """Row quantisation over row lengths that leave part of a wavefront's
    columns empty (64: a quarter of one load; 1088, 320: a partial second
    load), that need several 8192-column passes (8256) or a wide register
    set (6208), and a zero row (token 0: x = 0, so its h row is 0 too): codes
    and scales of x and h bit-exact, the products as in the full-layer test."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="w8codes", T=T, d=d, E=4, k=2, gate="softmax", n_ffn=4, inter=inter, dtype="w8a8")
    inp = make_inputs(cfg, seed=4)
    inp["x"][0] = 0
    lay = DeviceLayer(cfg, inp)
    U.say(f"[gpu] W8A8 code shapes T={T} d={d} inter={inter}")
    _, t = lay.layer_with_tables(intermediates=True)
    torch.cuda.synchronize()
    assert float(U.np_of(t["s_x"])[0]) == 0.0 and not U.np_of(t["q_x"])[0].any()
    _check_w8a8_integer_products(cfg, inp, t, silu_exact=False)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("name,T", [("prefill_zipf_bf16", None), ("dsv3_decode_share_bf16", None),
                                    ("dsv3_decode_share_bf16", 129), ("pangu_moge_w8a8", None)])
def test_layer_shared_expert_on_second_stream(name, T):
    """The shared expert forked onto a second stream gives the single-stream
    result bit for bit, and the caller's stream sees it joined."""
    from moe_expert_layer_fp32_amd.layer import SecondStream
    lay = U.device_layer(name, T)
    U.say(f"[gpu] second stream {name} T={lay.cfg.T}")
    one = lay.layer().clone()
    second = SecondStream()
    for _ in range(3):
        two = lay.layer(second=second).clone()     # consumed on the caller's stream, no host sync between
        torch.cuda.synchronize()
        assert torch.equal(_bits(one), _bits(two))


@pytest.mark.parametrize("name", ["longcat_zero_bf16", "dsv3_decode_share_bf16", "pangu_moge_w8a8"])
def test_layer_is_deterministic(name):
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    U.say(f"[gpu] determinism {name}")
    a = lay.layer().clone()
    b = lay.layer()
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_layer_zero_tokens_is_a_noop():
    L, DeviceLayer, to_device = _L()
    lay = U.device_layer("longcat_zero_bf16")
    x = lay.x[:0]
    U.say("[gpu] layer T=0")
    y = lay.layer(x)
    torch.cuda.synchronize()
    assert y.shape == (0, lay.cfg.d)


def test_layer_single_token():
    cfg, inp = U.inputs("dsv3_decode_share_bf16")
    lay = U.device_layer("dsv3_decode_share_bf16")
    U.say("[gpu] layer T=1")
    for t in (0, 37):
        y = lay.layer(lay.x[t:t + 1].contiguous())
        ref = O.moe_layer(inp, cfg, tokens=[t])
        _, beyond = U.output_errors(U.np_of(y), ref["y"], cfg.dtype)
        assert beyond <= U.TOL[cfg.dtype]


@pytest.mark.parametrize("dtype,gate", [("f32", "softmax"), ("bf16", "sigmoid"), ("w8a8", "softmax")])
def test_layer_odd_shapes(dtype, gate):
    """Shapes off the tile grid (d 192, I 320, I_s 192: no 128-element
    chunk, untiled column counts), 97 tokens, k 5 of 40 experts with
    resident FFN ids 3..22, identity ids 30..35 and the rest held elsewhere."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="odd", T=97, d=192, E=40, k=5, gate=gate, ffn_begin=3, n_ffn=20, zero_begin=30, n_zero=6,
                    inter=320, shared_inter=192, dtype=dtype, route_scale=1.25)
    inp = make_inputs(cfg)
    U.say(f"[gpu] layer odd shapes {dtype} {gate}")
    _check_layer(cfg, inp, DeviceLayer(cfg, inp))


@pytest.mark.parametrize("T", [1024, 1025])
def test_layer_sort_boundary(T):
    """T*k = 8192 slots, the most one permutation workgroup sorts, and one
    token past it (the chunked permutation). Two calls on one workspace that
    starts filled with 0xFF bytes give identical results."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="sortb", T=T, d=256, E=64, k=8, gate="softmax", n_ffn=64, inter=128, dtype="bf16")
    inp = make_inputs(cfg)
    lay = DeviceLayer(cfg, inp)
    ws = lay.workspace(L.OP_LAYER)
    ws.fill_(255)
    U.say(f"[gpu] layer sort boundary T={T} slots={T * cfg.k}")
    y = _check_layer(cfg, inp, lay, ws=ws)
    y2, t2 = lay.layer_with_tables(ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y2))
    flat = U.np_of(t2["topk_idx"]).reshape(-1)
    assert np.array_equal(U.np_of(t2["sorted_slot"]), np.argsort(flat, kind="stable"))


@pytest.mark.parametrize("name,T,limits", [("longcat_zero_bf16", None, None), ("dsv3_decode_share_bf16", None, None),
                                           ("pangu_moge_w8a8", None, None), ("prefill_zipf_bf16", 2048, None),
                                           ("dsv3_decode_share_bf16", None, {"shared_ffn1_wgs": 128,
                                                                             "decode_tile_rows": 32})])
def test_layer_graph_replay(name, T, limits):
    """moe_layer captured into a HIP graph (with the shared expert forked onto
    a second stream inside the capture where there is one) replays to the
    eager result bit for bit; new inputs are copied into the captured input
    buffer between replays, with eager work and synchronisations between.
    W8A8 records ev_join twice on the second stream, prefill sizes ev_fork
    twice (the small experts' down product on the second stream); the
    DeepSeek-style call also under its table's limits (capped shared
    gate/up, 32-row routed tiles)."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    from moe_expert_layer_fp32_amd import tuning as TU
    cfg, inp = U.inputs(name, T)
    lay = U.device_layer(name, T)
    second = SecondStream() if cfg.shared_inter else None
    t = TU.to_struct(TU.limits(**limits)) if limits else None
    xs = [lay.x.clone(), lay.x.flip(0).contiguous()]
    eager = [lay.layer(x=xi, second=second, tuning=t) for xi in xs]
    torch.cuda.synchronize()
    x_buf, y_buf = xs[0].clone(), torch.empty_like(eager[0])
    ws = lay.workspace(L.OP_LAYER)
    U.say(f"[gpu] graph capture {name} streams={2 if second else 1} limits={limits}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.layer(x=x_buf, y=y_buf, ws=ws, second=second, tuning=t)
    torch.cuda.synchronize()
    for rep in range(3):
        for xi, ye in zip(xs, eager):
            x_buf.copy_(xi)
            lay.layer(x=xs[1 - rep % 2])   # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(_bits(y_buf), _bits(ye)), f"replay {rep}"
    del g


@pytest.mark.parametrize("name,caps", [("dsv3_decode_share_bf16", (128, 128, 0, 0)),
                                       ("pangu_moge_w8a8", (96, 192, 64, 40)),
                                       ("longcat_zero_bf16", (0, 0, 1, 8))])
def test_layer_launch_limits(name, caps):
    """moe_layer under workgroup caps (moe_tuning), with the shared expert on
    a second stream: narrower persistent grids and splits of the reduction,
    down to the smallest grid (a cap of 1), still match the oracle and give
    the same routing tables."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    from moe_expert_layer_fp32_amd import tuning as TU
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    t = TU.to_struct(TU.limits(*caps))
    U.say(f"[gpu] layer {name} launch limits {caps}")
    second = SecondStream() if cfg.shared_inter else None
    y = _check_layer(cfg, inp, lay, second=second, tuning=t)
    y0 = lay.layer(second=second)
    torch.cuda.synchronize()
    _, dev = U.output_errors(U.np_of(y), U.np_of(y0).astype(np.float64), cfg.dtype)
    U.record(test="layer_launch_limits", cfg=name, caps=list(caps), err_vs_uncapped=dev)


@pytest.mark.parametrize("name,theta", [("dsv3_decode_share_bf16", 32), ("pangu_moge_w8a8", 56),
                                        ("longcat_zero_bf16", 20), ("tiny_fp32", 16)])
def test_layer_decode_stream_theta(name, theta):
    """Decode workloads with a caller's theta: experts with at most theta rows
    go to the 32-row weight-streaming kernel, the others to the 64-row tiles
    (split reduction where the layer uses one), chosen per expert on the
    device; against the oracle, one and two streams."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    t = L.MoeTuning(stream_max_rows=theta)
    U.say(f"[gpu] layer {name} decode theta {theta}")
    y = _check_layer(cfg, inp, lay, tuning=t)
    if cfg.shared_inter:
        y2 = lay.layer(second=SecondStream(), tuning=t)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y2))


@pytest.mark.parametrize("name,extra", [("dsv3_decode_share_bf16", {}), ("longcat_zero_bf16", {}),
                                        ("pangu_moge_w8a8", {}), ("tiny_fp32", {}),
                                        ("longcat_zero_bf16", {"stream_max_rows": 20}),
                                        ("dsv3_decode_share_bf16", {"shared_ffn1_wgs": 128})])
def test_layer_decode_tile_rows_32(name, extra):
    """Decode workloads on 32-row routed tiles (moe_tuning.decode_tile_rows):
    experts of at most 32 rows (DeepSeek-style share, reduction split over
    the wavefronts of one workgroup) take one tile, larger ones several (LongCat-style, W8A8 with its int8 path,
    fp32); also beside a caller's theta and under a shared cap. Against the
    oracle, and equal to the 64-row call up to fp32 summation order."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    from moe_expert_layer_fp32_amd import tuning as TU
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    t = TU.to_struct(TU.limits(decode_tile_rows=32, **extra))
    U.say(f"[gpu] layer {name} 32-row decode tiles {extra}")
    second = SecondStream() if cfg.shared_inter else None
    y = _check_layer(cfg, inp, lay, second=second, tuning=t)
    y0 = lay.layer(second=second)
    torch.cuda.synchronize()
    _, dev = U.output_errors(U.np_of(y), U.np_of(y0).astype(np.float64), cfg.dtype)
    U.record(test="layer_decode_tile_rows_32", cfg=name, extra=extra, err_vs_64_rows=dev)


def test_layer_wave_split_equals_slices():
    """DeepSeek-style decode share: the routed gate/up reduction of 7168 is cut
    into four 1792-element ranges either way. On 64-row tiles the ranges run
    on four workgroups and the reduce pass adds their partial sums in order;
    on 32-row tiles (bf16) they run on the four wavefronts of one workgroup
    and are added in LDS in the same order. The SwiGLU rows h and the layer
    output must therefore be equal, value for value, and the 32-row call must
    still match the oracle."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd import tuning as TU
    name = "dsv3_decode_share_bf16"
    cfg, inp = U.inputs(name)
    lay = U.device_layer(name)
    U.say(f"[gpu] layer {name} wave-split gate/up against four split workgroups")
    y32, t32 = lay.layer_with_tables(tuning=TU.to_struct(TU.limits(decode_tile_rows=32)), intermediates=True)
    y64, t64 = lay.layer_with_tables(tuning=TU.to_struct(TU.limits(decode_tile_rows=64)), intermediates=True)
    torch.cuda.synchronize()
    assert torch.equal(t32["offsets"], t64["offsets"])
    off = U.np_of(t32["offsets"])
    rows = int(off[cfg.ffn_begin + cfg.n_ffn] - off[cfg.ffn_begin])
    assert rows > 0
    assert torch.equal(t32["h"][:rows].float(), t64["h"][:rows].float())
    assert torch.equal(t32["rows"][:rows].float(), t64["rows"][:rows].float())
    assert torch.equal(y32.float(), y64.float())
    _check_layer(cfg, inp, lay, tuning=TU.to_struct(TU.limits(decode_tile_rows=32)))


@pytest.mark.parametrize("T,lift", [(96, 2.0), (160, 3.0)])
def test_layer_wave_split_multi_tile_experts(T, lift):
    """A decode shape whose gate/up reduction is split four ways (8 resident
    experts x 16 column blocks, d 1024: four 256-element ranges), with a logit
    lift on the resident experts so that most of them get more than 32 rows:
    on 32-row tiles they take two or more m-tiles (a ragged last one), each
    reduced on the four wavefronts of one workgroup. Equal, value for value,
    to the 64-row call (four split workgroups and the reduce pass) and
    against the oracle."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd import tuning as TU
    cfg = MoEConfig(name=f"wave_split_{T}", T=T, d=1024, E=32, k=4, gate="softmax", n_ffn=8, inter=2048,
                    dtype="bf16", bias=("const", lift, 0, 8))
    cfg.check()
    inp = make_inputs(cfg, seed=23)
    lay = DeviceLayer(cfg, inp)
    U.say(f"[gpu] wave-split multi-tile experts T={T} lift={lift}")
    y32, t32 = lay.layer_with_tables(tuning=TU.to_struct(TU.limits(decode_tile_rows=32)), intermediates=True)
    y64, t64 = lay.layer_with_tables(tuning=TU.to_struct(TU.limits(decode_tile_rows=64)), intermediates=True)
    torch.cuda.synchronize()
    counts = U.np_of(t32["counts"])[:cfg.n_ffn]
    assert (counts > 32).sum() >= 4, f"too few experts above one 32-row tile: {counts.tolist()}"
    rows = int(counts.sum())
    assert torch.equal(t32["offsets"], t64["offsets"])
    assert torch.equal(t32["h"][:rows].float(), t64["h"][:rows].float())
    assert torch.equal(y32.float(), y64.float())
    _check_layer(cfg, inp, lay, tuning=TU.to_struct(TU.limits(decode_tile_rows=32)))
    U.record(test="layer_wave_split_multi_tile_experts", T=T, counts=counts.tolist())


def _random_config(seed: int, prefill: bool = False) -> MoEConfig:
    """A seeded layer shape drawn across the descriptor's ranges: the three
    compute types, both gates, plain / group-limited / per-group-quota
    selection, identity experts before or after the resident range, with and
    without a shared expert, token counts from 1 to 513 (prefill: 1024 to
    2048, the regime of the per-expert tile classes and, for bf16, 256-row
    tiles and the two-stream order)."""
    r = np.random.default_rng(1000 + seed + (100000 if prefill else 0))
    dtype = ("f32", "bf16", "w8a8")[seed % 3]
    gate = ("softmax", "sigmoid")[int(r.integers(2))]
    E = int(r.choice([4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 160, 256]))
    mode = int(r.integers(3))     # 0 plain, 1 group-limited, 2 per-group quota
    divs = [g for g in range(2, min(E, 64) + 1) if E % g == 0]
    n_group, topk_group, per_group_k = 1, 0, 0
    if mode == 1:
        groups = [g for g in divs if E // g >= 2]
        if groups:
            n_group = int(r.choice(groups))
            topk_group = int(r.integers(1, n_group + 1))
    elif mode == 2:
        groups = [g for g in divs if g <= 16]
        if groups:
            n_group = int(r.choice(groups))
            per_group_k = int(r.integers(1, min(E // n_group, 16 // n_group) + 1))
    if per_group_k:
        k = n_group * per_group_k
    else:
        k = int(r.integers(1, min(E, 16, topk_group * (E // n_group) if topk_group else 16) + 1))
    n_zero = int(r.integers(1, E // 4 + 1)) if E >= 4 and r.random() < 0.4 else 0
    n_ffn = int(r.integers(1, E - n_zero + 1))
    if n_zero and r.random() < 0.5:      # identity experts ahead of the resident ones
        zero_begin = int(r.integers(0, E - n_zero - n_ffn + 1))
        ffn_begin = zero_begin + n_zero
    else:
        ffn_begin = int(r.integers(0, E - n_zero - n_ffn + 1))
        zero_begin = ffn_begin + n_ffn if n_zero else 0
    T = int(r.choice([1024, 1100, 1536, 2048])) if prefill else int(r.choice([1, 3, 17, 64, 100, 255, 513]))
    d = int(r.choice([64, 128, 256, 512])) if prefill else int(r.choice([64, 128, 192, 256, 512, 1024]))
    return MoEConfig(name=f"random{'_prefill' if prefill else ''}{seed}", T=T, d=d, E=E, k=k, gate=gate,
                     n_group=n_group,
                     topk_group=topk_group, per_group_k=per_group_k, ffn_begin=ffn_begin, n_ffn=n_ffn,
                     zero_begin=zero_begin, n_zero=n_zero, inter=int(r.choice([64, 128, 256, 320, 512])),
                     shared_inter=int(r.choice([0, 0, 64, 256])), dtype=dtype, seed=seed)


@pytest.mark.parametrize("seed", range(100))
def test_layer_random_shapes(seed):
    """Seeded random layer shapes against the oracle (any_shape checks, see
    _check_layer): one stream; two streams where there is a shared expert;
    every even seed also on 32-row decode tiles (moe_tuning; among them
    bf16 shapes whose gate/up reduction is split four ways, which then runs on
    the four wavefronts of one workgroup)."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    from moe_expert_layer_fp32_amd import tuning as TU
    cfg = _random_config(seed)
    cfg.check()
    inp = make_inputs(cfg, seed=seed)
    U.say(f"[gpu] random layer {seed}: {cfg}")
    lay = DeviceLayer(cfg, inp)
    y1 = _check_layer(cfg, inp, lay, any_shape=True)
    if cfg.shared_inter:
        y2 = _check_layer(cfg, inp, lay, second=SecondStream(), any_shape=True)
        assert torch.equal(_bits(y1), _bits(y2)), "two streams differ from one"
    if seed % 2 == 0:
        _check_layer(cfg, inp, lay, tuning=TU.to_struct(TU.limits(decode_tile_rows=32)), any_shape=True)


@pytest.mark.parametrize("seed", range(32))
def test_layer_random_prefill_shapes(seed):
    """Seeded random shapes at prefill sizes (1024 to 2048 tokens) against
    the oracle, one stream and, with a shared expert, two."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    cfg = _random_config(seed, prefill=True)
    cfg.check()
    inp = make_inputs(cfg, seed=seed)
    U.say(f"[gpu] random prefill layer {seed}: {cfg}")
    lay = DeviceLayer(cfg, inp)
    y1 = _check_layer(cfg, inp, lay, any_shape=True)
    if cfg.shared_inter:
        y2 = _check_layer(cfg, inp, lay, second=SecondStream(), any_shape=True)
        assert torch.equal(_bits(y1), _bits(y2)), "two streams differ from one"


def test_layer_largest_k_group_limited():
    """k = 16 (the largest built), group-limited selection of 4 of 8 groups
    over 256 experts, 16 resident, two streams."""
    L, DeviceLayer, to_device = _L()
    from moe_expert_layer_fp32_amd.layer import SecondStream
    cfg = MoEConfig(name="k16", T=64, d=256, E=256, k=16, gate="sigmoid", n_group=8, topk_group=4, n_ffn=16,
                    inter=128, shared_inter=128, dtype="bf16")
    inp = make_inputs(cfg)
    U.say("[gpu] layer k=16 group-limited")
    lay = DeviceLayer(cfg, inp)
    y = _check_layer(cfg, inp, lay)
    two = lay.layer(second=SecondStream())
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(two))


def test_layer_all_identity_experts():
    """Every expert a zero-computation expert: y = route_scale * x, rounded once."""
    L, DeviceLayer, to_device = _L()
    cfg = MoEConfig(name="ident", T=100, d=256, E=16, k=4, gate="sigmoid", zero_begin=0, n_zero=16,
                    route_scale=1.5, dtype="bf16")
    inp = make_inputs(cfg)
    U.say("[gpu] layer all identity")
    lay = DeviceLayer(cfg, inp)
    y = U.np_of(lay.layer())
    want = 1.5 * np.asarray(O.x_f32(inp), np.float64)
    _, beyond = U.output_errors(y, want, "bf16")
    assert beyond <= 1e-5
