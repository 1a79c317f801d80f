"""Throughput of the MoE expert layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--layers L]

A step is one moe_layer call (router + top-k, permute, grouped SwiGLU FFN,
shared expert, combine) over one batch of T tokens. Steps cycle through L
independently generated layers (as consecutive MoE layers of a model would),
so the weights of the step being timed are not still sitting in the 256 MB
last-level cache from the step before; L is chosen so the L layers' weights
exceed 1 GB. Inputs are resident in HBM before the timed region.

Prints one JSON line: value = tokens/s over the K timed steps, plus the
roofline of the dominant kernel and the CPU oracle's throughput on a bounded
sample of the same workload. The dominant kernel is the largest launch of the
call: for the prefill workload (the default, 8192 tokens) the shared expert's
gate/up projection with SwiGLU (matrix-core bound: algorithmic flops per
launch / its mean duration), for the decode workloads the routed experts'
gate/up projection with SwiGLU (HBM bound: algorithmic bytes per launch / its
mean duration). Durations come from HIP events stamped by the launch's own
dispatch on the stream it runs on. `layer_roofline` applies the same roofline
to the whole call. With the default workload the line also carries
`decode_workloads`: the three decode workloads, each timed the same way by
this script in a child process (`--no-decode` skips them).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores
INT8_PEAK_TOPS = 5000.0        # dense int8 matrix cores
FP32_PEAK_TFLOPS = 157.3
DEFAULT_CONFIG = "prefill_zipf_bf16"
COMPUTE_UNITS = 256
METRIC = "MoE-layer tokens/s at 1 GPU; decode HBM GB/s %peak; prefill MFMA %peak"
def traffic_file(workload: str) -> str:
    """Where the HBM traffic record of a workload's dominant launch lives."""
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
CSRC = os.path.join(ROOT, "moe_expert_layer_fp32_amd", "csrc")
COPY_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default=DEFAULT_CONFIG)
    p.add_argument("--layers", type=int, default=0, help="layers cycled (0: enough for > 1 GB of weights)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the HBM read-ceiling measurement (moe_stream_read over 2 GiB)")
    p.add_argument("--no-tune", action="store_true",
                   help="skip choosing the launch limits from measured runs (tuning.py)")
    p.add_argument("--limits", default="",
                   help="JSON object of moe_tuning fields to use for every call instead of tuning")
    p.add_argument("--tune", action="store_true",
                   help="time the candidate limits even when the shipped table has an entry for this shape")
    p.add_argument("--save-tuning", default="",
                   help="merge the entry tuned by this run into the JSON table at this path")
    p.add_argument("--graph", action="store_true",
                   help="also time the same calls replayed from one captured HIP graph (graph_replay)")
    p.add_argument("--streams", type=int, default=2, choices=(1, 2),
                   help="2: the shared expert runs on a second stream (when the workload has one)")
    p.add_argument("--no-decode", action="store_true",
                   help="with the default workload: skip the decode workloads' lines (decode_workloads)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run 5 device copies of 1 GiB (the known-size kernel for counter calibration)")
    p.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                   help="turn rocprofv3 --pmc counter_collection.csv files into the traffic record")
    p.add_argument("--traffic-kernel", default="",
                   help="with --traffic: the kernel name the dominant launch has in the counter files")
    p.add_argument("--traffic-occurrence", type=int, default=0,
                   help="with --traffic: which dispatch of that kernel within each layer call (0 = first)")
    p.add_argument("--traffic-per-call", type=int, default=1,
                   help="with --traffic: dispatches of that kernel per layer call")
    p.add_argument("--traffic-launch", default="",
                   help="with --traffic: which launch the record describes (shared_ffn1 or routed_ffn1)")
    return p.parse_args()


# Sources that define the launches the traffic counters describe: their
# kernels, the headers they include, and the host code that sizes them.
TRAFFIC_SOURCES = ("gemm_lds.hip", "gemm_big.hip", "tiles.h", "common.h", "kernels.h", "api.cpp")


def kernel_hash() -> str:
    """Hash of the sources of the counted kernel and its launch: counters
    taken on one version do not describe another."""
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_values(path: str) -> dict:
    import csv
    out: dict = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic_record(paths, cfg_name: str, kernel: str, occurrence: int, per_call: int, launch: str) -> dict:
    """HBM bytes per launch of the dominant kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for a
    device copy of COPY_BYTES bytes (read COPY_BYTES, write COPY_BYTES). The
    launch is the `occurrence`-th of `per_call` dispatches of `kernel` in each
    layer call (the same kernel can serve several products of a call)."""
    import statistics
    fetch, write, cal_f, cal_w = (counter_values(p) for p in paths)
    copy = [k for k in cal_f if "copyBuffer" in k]
    cf = statistics.median(cal_f[copy[0]]) * 1024.0
    cw = statistics.median(cal_w[copy[0]]) * 1024.0
    f_scale, w_scale = COPY_BYTES / cf, COPY_BYTES / cw
    names = [k for k in fetch if kernel and kernel in k]
    if len(names) != 1:
        raise SystemExit(f"--traffic-kernel {kernel!r} matches {len(names)} kernels: {names}")
    name = names[0]
    f_all, w_all = fetch[name], write[name]
    f_sel = f_all[occurrence::per_call]
    w_sel = w_all[occurrence::per_call]
    fb = statistics.median(f_sel) * 1024.0 * f_scale
    wb = statistics.median(w_sel) * 1024.0 * w_scale
    return {"workload": cfg_name, "launch": launch, "kernel": name, "occurrence": occurrence, "per_call": per_call,
            "dispatches": len(f_sel), "kernel_sha": kernel_hash(),
            "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
            "bytes_per_launch": fb + wb, "fetch_scale": f_scale, "write_scale": w_scale,
            "copy_bytes": COPY_BYTES}


# Launch-level algorithmic bytes follow the layer's rule (layer_algorithmic):
# weights that must be read and the launch's input read once; the gathered
# (permuted) rows and the h rows the launch writes are intermediates of this
# implementation and are not counted.
def ffn1_algorithmic(cfg, counts_per_layer, tokens_per_layer=None):
    """Algorithmic work of one launch of the routed gate/up projection:
    bytes = W1 and W3 (and int8 column scales) of every resident expert that
    received tokens, plus the activation row of every token routed to one of
    them read once (d elements: x, or its int8 codes in the W8A8 layer;
    tokens_per_layer gives that token count, else all T); flops = 2 * R * d
    * 2I."""
    wb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    xb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    out = []
    for li, counts in enumerate(counts_per_layer):
        n_tok = cfg.T if tokens_per_layer is None else int(tokens_per_layer[li])
        res = counts[cfg.ffn_begin:cfg.ffn_begin + cfg.n_ffn]
        active = int((res > 0).sum())
        R = int(res.sum())
        wbytes = active * 2 * cfg.d * cfg.inter * wb
        if cfg.dtype == "w8a8":
            wbytes += active * 2 * cfg.inter * 4        # fp32 column scales
        byts = wbytes + n_tok * cfg.d * xb
        flops = 2.0 * R * cfg.d * 2 * cfg.inter
        out.append((byts, flops, R, active))
    return out


def shared_ffn1_algorithmic(cfg):
    """Algorithmic work of one launch of the shared expert's gate/up
    projection (dense over all T tokens): bytes = its W1 and W3 (and int8
    column scales) and the activations read once; flops = 2 * T * d * 2 I_s."""
    wb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    xb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    byts = 2 * cfg.d * cfg.shared_inter * wb + cfg.T * cfg.d * xb
    if cfg.dtype == "w8a8":
        byts += 2 * cfg.shared_inter * 4
    return byts, 2.0 * cfg.T * cfg.d * 2 * cfg.shared_inter


def layer_algorithmic(cfg, counts_per_layer):
    """Algorithmic work of one whole layer call (the layer's own count):
    bytes = W1, W3 and W2 (and int8 scales) of every resident FFN expert that
    received tokens, the shared expert's weights, the fp32 router (4 d E) and
    x read plus y written (T d each, in the layer's element type); flops =
    the expert and shared-expert products, 2 n_e 3 d I per expert and
    2 T 3 d I_s (the router's 2 T d E is counted apart)."""
    wb = {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype]
    xb = {"f32": 4, "bf16": 2, "w8a8": 2}[cfg.dtype]
    scale_b = 4 if cfg.dtype == "w8a8" else 0
    shared_b = 3 * cfg.d * cfg.shared_inter * wb + (2 * cfg.shared_inter + cfg.d) * scale_b if cfg.shared_inter else 0
    out = []
    for counts in counts_per_layer:
        res = counts[cfg.ffn_begin:cfg.ffn_begin + cfg.n_ffn]
        active = int((res > 0).sum())
        R = int(res.sum())
        byts = (active * (3 * cfg.d * cfg.inter * wb + (2 * cfg.inter + cfg.d) * scale_b) + shared_b
                + 4 * cfg.d * cfg.E + 2 * cfg.T * cfg.d * xb)
        flops = 2.0 * R * 3 * cfg.d * cfg.inter + 2.0 * cfg.T * 3 * cfg.d * cfg.shared_inter
        out.append((byts, flops))
    return out


def hbm_read_ceiling(L, nbytes: int = 2 << 30, reps: int = 10) -> dict:
    """The practical HBM read ceiling on this device: moe_stream_read (one
    contiguous slice per workgroup, 16-byte loads) over a buffer well above
    the 256 MB last-level cache, mean of `reps` back-to-back reads between two
    events, after three untimed ones."""
    import torch
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(L.STREAM_READ_WGS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        L.moe_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        L.moe_stream_read(buf, nbytes, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": nbytes, "us": round(ms * 1e3, 1),
            "kernel": f"moe_stream_read, {L.STREAM_READ_WGS} workgroups, one contiguous slice each"}


def cpu_info() -> dict:
    """Model name and core counts of this host: physical cores (distinct
    (physical id, core id) pairs of /proc/cpuinfo), logical CPUs, and the
    CPUs this process may run on."""
    model, pairs, logical = "unknown", set(), 0
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model == "unknown":
                    model = val
                elif key == "processor":
                    logical += 1
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None:
                    pairs.add((phys, core))
                    phys = core = None
        if phys is not None:
            pairs.add((phys, core))
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"cpu_model": model, "physical_cores": len(pairs) or None, "logical_cpus": logical or os.cpu_count(),
            "cpus_available": avail}


def cpu_baseline(cfg, inp, seconds: float):
    """The oracle as it stands, timed on this host on a bounded sample: once
    with every BLAS thread numpy has, once with one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe_oracle as O

    sample = cfg.T
    if cfg.T * cfg.d * max(cfg.inter, cfg.shared_inter, 1) > 256 * 1024 * 2048:
        sample = 64
    toks = np.arange(sample)

    def timed(budget):
        t0 = time.perf_counter()
        n = 0
        while True:
            O.moe_layer(inp, cfg, tokens=toks)
            n += sample
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    n, el = timed(seconds)
    with threadpool_limits(limits=1):
        n1, el1 = timed(seconds / 2)
    info = cpu_info()
    return {"value": n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} tokens: {n // sample} oracle calls on the first {sample} tokens of the "
                      f"{cfg.name} batch, {el:.1f} s wall, numpy fp64 with {threads} BLAS threads",
            "one_thread": {"value": n1 / el1, "unit": "tokens/s", "cores": 1,
                           "sample": f"{n1} tokens in {n1 // sample} calls, {el1:.1f} s wall"},
            **info}


def graph_replay(L, layers, desc, y, ws, second, K, tuning=None):
    """The same layer calls (one per cycled layer, no timing events, the same
    launch limits) captured into one HIP graph and replayed: wall time per call."""
    import torch
    aux = second.fill(L.MoeAux()) if second is not None else None
    if aux is not None and tuning is not None:
        aux.tuning = ctypes.pointer(tuning)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for lay in layers:
            L.moe_layer(desc, lay.weights, lay.x, y, aux, ws)
    reps = max(1, K // len(layers))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / (reps * len(layers))
    del g
    return {"ms_per_step": round(per_call * 1e3, 4), "value": round(layers[0].cfg.T / per_call, 1),
            "calls": reps * len(layers)}


def main() -> int:
    args = parse()
    if args.traffic:
        rec = traffic_record(args.traffic, args.config, args.traffic_kernel, args.traffic_occurrence,
                             args.traffic_per_call, args.traffic_launch)
        with open(traffic_file(args.config), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if args.copy_calibration:
        import torch
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MoE layer here is one device's share and this "
              "build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from moe_expert_layer_fp32_amd import lib as L
    from moe_expert_layer_fp32_amd.hip_events import Event
    from moe_expert_layer_fp32_amd.layer import DeviceLayer, SecondStream
    from moe_inputs import get, make_inputs

    cfg = get(args.config)
    per_layer_bytes = max(1, (cfg.n_ffn * 3 * cfg.d * cfg.inter + 3 * cfg.d * cfg.shared_inter)
                          * {"f32": 4, "bf16": 2, "w8a8": 1}[cfg.dtype])
    n_layers = args.layers or max(1, min(8, -(-(1 << 30) // per_layer_bytes)))
    torch.cuda.set_device(0)
    layers, inputs0 = [], None
    for s in range(n_layers):
        inp = make_inputs(cfg, seed=cfg.seed + s)
        if s == 0:
            inputs0 = inp
        layers.append(DeviceLayer(cfg, inp))
        if s:
            del inp
    desc = layers[0].desc
    ws = layers[0].workspace(L.OP_LAYER)
    y = torch.empty((cfg.T, cfg.d), dtype=layers[0].xdtype, device="cuda")

    # Routing tables of each layer (outside the timed region) for the
    # algorithmic byte count of the dominant kernel.
    counts_per_layer, routed_tokens = [], []
    for lay in layers:
        _, t = lay.layer_with_tables()
        counts_per_layer.append(t["counts"].cpu().numpy())
        ids = t["topk_idx"].cpu().numpy()
        resident = (ids >= cfg.ffn_begin) & (ids < cfg.ffn_begin + cfg.n_ffn)
        routed_tokens.append(int(resident.any(axis=1).sum()))   # tokens with a resident selection
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    prefill = cfg.T >= 4096
    # The dominant launch: the shared expert's gate/up for the prefill
    # workload (when it has a shared expert), else the routed gate/up.
    dom_shared = prefill and cfg.shared_inter > 0
    # Timing events with a device-scope release (see hip_events): stamped by
    # the launches' own dispatch, they add no L2 write-back between kernels,
    # so the timed steps run as untimed ones do.
    ev = [(Event(), Event()) for _ in range(K)]
    ev_s = [(Event(), Event()) for _ in range(K)] if cfg.shared_inter else None
    auxes = []
    for i, (a, b) in enumerate(ev):
        aux = L.MoeAux(ev_ffn1_begin=a.handle, ev_ffn1_end=b.handle)
        if ev_s is not None:
            aux.ev_sffn1_begin, aux.ev_sffn1_end = ev_s[i][0].handle, ev_s[i][1].handle
        auxes.append(aux)
    second = SecondStream() if args.streams == 2 and cfg.shared_inter else None
    if second is not None:
        for a in auxes:
            second.fill(a)
    warm_aux = second.fill(L.MoeAux()) if second is not None else None

    # Launch limits from measured runs (untimed): only the shared expert on
    # the second stream has candidates.
    tuned, t_struct = None, None
    if args.limits:
        from moe_expert_layer_fp32_amd import tuning as TU
        lim = TU.limits(**json.loads(args.limits))
        t_struct = TU.to_struct(lim)     # None: every field 0, the library's own choice
        tp = ctypes.pointer(t_struct) if t_struct is not None else None
        for a in auxes + ([warm_aux] if warm_aux is not None else []):
            a.tuning = tp
        if warm_aux is None:
            warm_aux = L.MoeAux(tuning=tp)
        tuned = {"limits": lim, "source": "--limits"}
    elif not args.no_tune:
        # The tiling table: the shipped entry for this shape, stream count and
        # load bucket, else limits timed now on these calls (untimed region).
        from moe_expert_layer_fp32_amd import tuning as TU
        streams = 2 if second is not None else 1
        bucket = max(TU.load_bucket(c, cfg.ffn_begin, cfg.n_ffn) for c in counts_per_layer)
        key = TU.shape_key(desc, streams, bucket)
        cache = TU.TilingCache.shipped()
        lim = None if args.tune else cache.lookup(key)
        source = "shipped table"
        if lim is None:
            source = "tuned in this run"
            tune_aux = second.fill(L.MoeAux()) if second is not None else L.MoeAux()

            def run(t, i):
                tune_aux.tuning = ctypes.pointer(t) if t is not None else None
                lay = layers[i % n_layers]
                L.moe_layer(desc, lay.weights, lay.x, y, tune_aux, ws)

            fresh = TU.TilingCache()
            lim = fresh.tune(key, run, torch.cuda.synchronize, candidates=TU.candidates_for(desc, streams),
                             calls=max(5, min(20, 4000 // max(1, cfg.T))))
            cache.table[key] = fresh.table[key]
            if args.save_tuning:
                fresh.merge_into(args.save_tuning)
        t_struct = TU.to_struct(lim)
        if t_struct is not None:
            for a in auxes:
                a.tuning = ctypes.pointer(t_struct)
            if warm_aux is None:
                warm_aux = L.MoeAux()
            warm_aux.tuning = ctypes.pointer(t_struct)
        tuned = {"limits": lim, "source": source, "key": key, "candidates_us": cache.table[key].get("us"),
                 "candidate_order": "/".join(TU.FIELDS), "load_bucket": bucket}

    for i in range(W):
        lay = layers[i % n_layers]
        L.moe_layer(desc, lay.weights, lay.x, y, warm_aux, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        lay = layers[i % n_layers]
        L.moe_layer(desc, lay.weights, lay.x, y, auxes[i], ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    peak = INT8_PEAK_TOPS if cfg.dtype == "w8a8" else (FP32_PEAK_TFLOPS if cfg.dtype == "f32" else BF16_PEAK_TFLOPS)

    def launch_roofline(ms, byts, flops, bound, what):
        """Roofline object of one launch: algorithmic work per launch over
        its mean duration from the stamped events."""
        mean_s = float(ms.mean()) / 1e3
        if bound == "mfma":
            r = {"bound": "mfma", "achieved": round(float(flops.mean()) / mean_s / 1e12, 2), "peak": peak,
                 "unit": "TFLOP/s"}
        else:
            r = {"bound": "hbm", "achieved": round(float(byts.mean()) / mean_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s"}
        r["frac"] = round(r["achieved"] / r["peak"], 4)
        r["kernel"] = what
        r["mean_us"] = round(mean_s * 1e6, 2)
        r["p10_p50_p90_us"] = [round(float(v) * 1e3, 2) for v in np.percentile(ms, [10, 50, 90])]
        r["alg_bytes_per_launch"] = int(byts.mean())
        r["alg_flops_per_launch"] = float(flops.mean())
        return r

    bound = "mfma" if prefill else "hbm"
    ffn1_ms = np.array([a.elapsed_ms(b) for a, b in ev])
    alg = ffn1_algorithmic(cfg, counts_per_layer, routed_tokens)
    alg_bytes = np.array([alg[i % n_layers][0] for i in range(K)])
    alg_flops = np.array([alg[i % n_layers][1] for i in range(K)])
    routed_what = ("routed-expert gate/up projection + SwiGLU (" +
                   ("two launches on the layer's stream: experts with at most 64 rows, then larger experts"
                    if prefill else "one launch") + ")")
    routed_roof = launch_roofline(ffn1_ms, alg_bytes, alg_flops, bound, routed_what)
    if dom_shared:
        sb, sf = shared_ffn1_algorithmic(cfg)
        s_ms = np.array([a.elapsed_ms(b) for a, b in ev_s])
        roof = launch_roofline(s_ms, np.full(K, float(sb)), np.full(K, sf), "mfma",
                               "shared-expert gate/up projection + SwiGLU (one launch per step" +
                               (", on the second stream beside the routed experts)" if second is not None
                                else ")"))
        roof_name = "shared_ffn1"
        # A cap on the shared gate/up's grid confines the launch to that many
        # compute units (its 256-row tiles take one per workgroup); the
        # fraction on those units says how well the tiles run there.
        cap = int((tuned or {}).get("limits", {}).get("shared_ffn1_wgs", 0) or 0)
        if second is not None and 0 < cap < COMPUTE_UNITS:
            roof["compute_units"] = cap
            roof["frac_on_its_compute_units"] = round(roof["frac"] * COMPUTE_UNITS / cap, 4)
    else:
        roof = routed_roof
        roof_name = "routed_ffn1"
    roof["traffic"] = None
    if os.path.exists(traffic_file(cfg.name)):
        tr = json.load(open(traffic_file(cfg.name)))
        if tr.get("kernel_sha") == kernel_hash() and tr.get("workload") == cfg.name and \
                tr.get("launch") == roof_name:
            roof["traffic"] = tr.get("bytes_per_launch")

    # The whole layer call against the same roofline: algorithmic bytes (or
    # flops) per call over the measured time per call.
    lay_alg = layer_algorithmic(cfg, counts_per_layer)
    step_s = wall / K
    if prefill:
        la = float(np.mean([lay_alg[i % n_layers][1] for i in range(K)])) / step_s / 1e12
        layer_roof = {"bound": "mfma", "achieved": round(la, 2), "peak": roof["peak"], "unit": "TFLOP/s"}
    else:
        la = float(np.mean([lay_alg[i % n_layers][0] for i in range(K)])) / step_s / 1e9
        layer_roof = {"bound": "hbm", "achieved": round(la, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    layer_roof["frac"] = round(layer_roof["achieved"] / layer_roof["peak"], 4)
    layer_roof["alg_per_call"] = (float(np.mean([a[1] for a in lay_alg])) if prefill
                                  else int(np.mean([a[0] for a in lay_alg])))

    ceiling = None
    if not args.no_ceiling:
        ceiling = hbm_read_ceiling(L)
        if roof["bound"] == "hbm":
            roof["frac_of_read_ceiling"] = round(roof["achieved"] / ceiling["achieved"], 4)
        if layer_roof["bound"] == "hbm":
            layer_roof["frac_of_read_ceiling"] = round(layer_roof["achieved"] / ceiling["achieved"], 4)

    graph = None
    if args.graph:
        graph = graph_replay(L, layers, desc, y, ws, second, K, t_struct if tuned else None)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inputs0, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(cfg.T * K / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "w8a8": "int8"}[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "gate": cfg.gate,
                   "n_ffn": cfg.n_ffn, "n_zero": cfg.n_zero, "inter": cfg.inter,
                   "shared_inter": cfg.shared_inter, "layers_cycled": n_layers,
                   "streams": 2 if second is not None else 1,
                   "global_batch": cfg.T, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer_roofline": layer_roof,
        **({"routed_ffn1_roofline": routed_roof} if dom_shared else {}),
        "cpu_baseline": cpu,
        **({"hbm_read_ceiling": ceiling} if ceiling is not None else {}),
    }
    if tuned is not None:
        rec["tuning"] = tuned
    if graph is not None:
        rec["graph_replay"] = graph
    if args.config == DEFAULT_CONFIG and not args.no_decode and not args.limits:
        rec["decode_workloads"] = decode_lines(args)
    print(json.dumps(rec), flush=True)
    return 0


DECODE_CONFIGS = ("longcat_zero_bf16", "dsv3_decode_share_bf16", "pangu_moge_w8a8")


def decode_lines(args) -> dict:
    """The decode workloads, each timed by this script in a child process
    (same steps and warm-up, tuned table, no CPU baseline): calls per second
    as tokens/s, the call time, the dominant launch's and the whole call's HBM
    roofline. A child that fails leaves its exit status instead."""
    out = {}
    for name in DECODE_CONFIGS:
        cmd = [sys.executable, os.path.abspath(__file__), "--config", name, "--steps", str(args.steps),
               "--warmup", str(args.warmup), "--no-cpu-baseline", "--no-ceiling", "--no-decode"]
        if args.no_tune:
            cmd.append("--no-tune")
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        except subprocess.TimeoutExpired:
            out[name] = {"error": "timed out"}
            continue
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            out[name] = {"error": f"exit status {r.returncode}"}
            continue
        b = json.loads(lines[-1])
        roof, lay = b["roofline"], b["layer_roofline"]
        out[name] = {"value": b["value"], "unit": b["unit"], "ms_per_step": b["ms_per_step"],
                     "dtype": b["dtype"], "config": b["config"],
                     "roofline": {k: roof.get(k) for k in ("bound", "achieved", "peak", "unit", "frac", "kernel",
                                                           "mean_us", "traffic")},
                     "layer_roofline": {k: lay.get(k) for k in ("bound", "achieved", "peak", "unit", "frac")},
                     "tuning": (b.get("tuning") or {}).get("limits")}
    return out


if __name__ == "__main__":
    sys.exit(main())
