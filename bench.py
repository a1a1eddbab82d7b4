#!/usr/bin/env python3
"""Throughput of the fused MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload cfg2_M64] [--act A] [--quant Q]
                    [--gpus 1] [--no-prefill] [--prefill-steps P]

One step is one whole pass of the layer -- route + (fp8 quantise) + align,
GEMM1 + activation, GEMM2 + combine -- over one batch of synthetic tokens
already resident in HBM, issued as one moe_forward call through the C ABI on
the current HIP stream.  The default workload is the decode-sized bf16 gated
MoE (hidden 2048, 128 experts, top-8, intermediate 768) at M = 64 tokens.  K
steps are timed back to back between two device synchronisations (wall
clock; HIP events on the stream at both ends give the GPU's own time).

The dominant kernel (GEMM1, which streams two thirds of the weight bytes) is
then timed in a second loop of K passes issued as the separate entry points,
with HIP events recorded on the same stream around GEMM1 only (an event
record costs the stream about 3 us at decode sizes, so the pass is not cut at
every kernel boundary); a short loop with events at every call gives the
other calls' share (``layer``).

Printed: one JSON line.  ``roofline`` relates GEMM1's algorithmic bytes
(W13 of the experts the batch routes to, the tokens' hidden rows and the
half-width intermediate it writes) to its event-timed duration and the 8 TB/s
HBM peak -- or, where its MFMA time at the nominal peaks exceeds its weight
streaming time (prefill sizes), its algorithmic FLOPs to the dense MFMA peak
of its dtype; ``roofline.layer`` does the same for the whole pass and the
step time.  ``prefill`` times, with the default arguments, one moe_forward
pass per step (after untimed warm-up passes) of the three prefill-sized
workloads (fp8 block-scaled with
the shared expert at M = 4096 -- HBM-bound by its arithmetic intensity --,
fp8 per-tensor relu^2 and W4A8 at M = 8192) and relates each pass and its
GEMM1 to the fp8 MFMA peak (or HBM).  ``measured_peaks`` are the same
device's achievable read-stream bandwidth and MFMA throughput, measured after
the timed regions with the library's measurement kernels; ``cpu_baseline`` is
the CPU oracle timed on a bounded sample of the headline workload on the host
cores; ``sweep`` gives every token count of the headline configuration, each
pass timed alone after evicting the caches (one moe_forward call, and the
separate entry points).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
METRIC = "MoE layer tokens/s + % HBM roofline (M≤64) / % MFMA peak (M≥4096)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="cfg2_M64")
    ap.add_argument("--act", choices=("silu", "relu2", "gelu_tanh"), default=None,
                    help="replace the workload's activation (same shapes otherwise)")
    ap.add_argument("--quant", default=None,
                    choices=("bf16", "fp8_tensor", "fp8_block", "w4a8", "mxfp8", "mxfp4"),
                    help="replace the workload's weight format (same shapes otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured read-stream and MFMA-loop peaks")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill-sized workloads' block")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=10,
                    help="untimed passes of each prefill workload before its timed steps "
                         "(2 left those passes 5-6%% short of their steady state)")
    ap.add_argument("--prefill-workloads", default="cfg3_M4096,cfg4_M8192,cfg5_M8192")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for counter scaling)")
    return ap.parse_args()


def workload(name):
    import synth
    cid, m = name.split("_M")
    return synth.CONFIGS[int(cid.replace("cfg", ""))], int(m)


def to_dev(a):
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 \
        else torch.from_numpy(a)
    return t.to("cuda")


def make_layer(cfg, W, a1, a2):
    import torch
    from mixture_experts_layer_09_amd.layer import MoELayer
    sc = lambda v: None if v is None else torch.tensor(float(v), dtype=torch.float32,
                                                       device="cuda")
    return MoELayer(cfg.H, cfg.I, cfg.E_routed, cfg.top_k, cfg.act, cfg.quant,
                    to_dev(W["w13"]), to_dev(W["w2"]), to_dev(W["w13_scale"]),
                    to_dev(W["w2_scale"]), sc(a1), sc(a2), n_shared=cfg.n_shared,
                    shared_gate=cfg.shared_gate, renormalize=cfg.renormalize)


def weight_bytes_per_expert(cfg):
    el = {"bf16": 2.0, "fp8_tensor": 1.0, "fp8_block": 1.0, "w4a8": 0.5, "mxfp8": 1.0,
          "mxfp4": 0.5}[cfg.quant]
    w13 = cfg.N1 * cfg.H * el
    w2 = cfg.H * cfg.I * el
    if cfg.quant == "fp8_block":
        w13 += (cfg.N1 // 128) * (cfg.H // 128) * 4
        w2 += (cfg.H // 128) * (cfg.I // 128) * 4
    elif cfg.quant == "w4a8":
        w13 += cfg.N1 * (cfg.H // 128) * 2
        w2 += cfg.H * (cfg.I // 128) * 2
    elif cfg.quant == "fp8_tensor":
        w13 += 4
        w2 += 4
    elif cfg.quant in ("mxfp8", "mxfp4"):
        w13 += cfg.N1 * cfg.H // 32        # one E8M0 byte per 32 weights
        w2 += cfg.H * cfg.I // 32
    return w13, w2


def algorithmic(cfg, M, ids):
    """Bytes and FLOPs the pass must move / do, from the realised routing."""
    import numpy as np
    valid = ids[(ids >= 0) & (ids < cfg.E)]
    touched = int(np.unique(valid).size)
    A_v = int(valid.size)
    w13, w2 = weight_bytes_per_expert(cfg)
    a_el = 2 if cfg.quant == "bf16" else 1
    x_b = M * cfg.H * 2
    gemm1_bytes = touched * w13 + x_b + A_v * cfg.I * a_el
    layer_bytes = (touched * (w13 + w2) + x_b + M * cfg.E_routed * 4
                   + 2 * A_v * cfg.I * a_el + M * cfg.H * 2)
    flops = 2.0 * A_v * cfg.H * cfg.N1 + 2.0 * A_v * cfg.I * cfg.H
    gemm1_flops = 2.0 * A_v * cfg.H * cfg.N1
    return dict(touched=touched, assignments=A_v, gemm1_bytes=gemm1_bytes,
                layer_bytes=layer_bytes, flops=flops, gemm1_flops=gemm1_flops)


class Pass:
    """One layer pass through the component entry points on the current stream,
    with events around each."""

    def __init__(self, layer, x, logits, T):
        self.layer, self.x, self.logits, self.T = layer, x, logits, T
        self.b = layer.buffers(T)

    def run(self, ev=None, g1_ev=None):
        """ev: 4 events around every call; g1_ev: 2 events around GEMM1 only."""
        L, T, b = self.layer, self.T, self.b
        if ev is not None:
            ev[0].record()
        L.prepare(T, self.logits, self.x, b)
        if ev is not None:
            ev[1].record()
        if g1_ev is not None:
            g1_ev[0].record()
        L.gemm1(T, self.x, b)
        if ev is not None:
            ev[2].record()
        if g1_ev is not None:
            g1_ev[1].record()
        L.gemm2(T, b)
        if ev is not None:
            ev[3].record()


KERNEL_SOURCES = ("moe_gemm.hip", "moe_gemm_common.hpp", "moe_device.hpp", "moe_plan.cpp",
                  "moe_plan.hpp")


def kernel_sources_digest():
    """First 16 hex digits of the SHA-256 over the sources that decide the
    GEMM kernels and their launch shapes; a stored counter record is only
    valid while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_09_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(workload_key):
    """HBM bytes per GEMM1 launch from the committed counter summaries
    (profiles/traffic_*.md: FETCH_SIZE and WRITE_SIZE per dispatch, each
    scaled by what the counter reads for a copy of known size), or None when
    no record covers this workload or the kernel sources changed since."""
    import glob
    import re
    digest = kernel_sources_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        with open(path) as fh:
            m = re.search(r"```json\s*(\{.*?\})\s*```", fh.read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("bench_workload") == workload_key and rec.get("sources_sha256_16") == digest:
            return int(rec["traffic_bytes_per_launch"])
    return None


def copy_calibration(mib):
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))


def cpu_baseline(cfg, W, tok, sc, min_seconds):
    """The oracle as it stands, on the same workload's batch, repeated until at
    least `min_seconds` of host time are spent."""
    import numpy as np
    import oracle
    from synth.inputs import bf16_bits_to_f32
    x = bf16_bits_to_f32(tok["x_bits"]).astype(np.float64)
    M = x.shape[0]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_forward(x, W["w13"], W["w2"], quant=cfg.quant, act=cfg.act,
                           E_routed=cfg.E_routed, top_k=cfg.top_k,
                           renormalize=cfg.renormalize, n_shared=cfg.n_shared,
                           shared_gate=cfg.shared_gate, logits=tok["logits"],
                           w13_scale=W["w13_scale"], w2_scale=W["w2_scale"],
                           a1=sc["a1"], a2=sc["a2"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 0) for i in threadpool_info()) or None
    except Exception:
        pass
    return {"value": round(reps * M / el, 3), "unit": "tokens/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{reps} full pass(es) of the {M}-token batch ({cfg.name}), "
                      f"fp64 NumPy, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    cfg, M = workload(args.workload)
    key = args.workload
    if args.act is not None and args.act != cfg.act:
        import dataclasses
        cfg = dataclasses.replace(cfg, act=args.act)
        key = f"{key}_{args.act}"
    if args.quant is not None and args.quant != cfg.quant:
        import dataclasses
        cfg = dataclasses.replace(cfg, quant=args.quant)
        key = f"{key}_{args.quant}"
    W = synth.make_weights(cfg)
    tok = synth.make_tokens(cfg, M)
    sc = synth.make_act_scales(cfg, tok["x_bits"])
    layer = make_layer(cfg, W, sc["a1"], sc["a2"])
    x, lg = to_dev(tok["x_bits"]), to_dev(tok["logits"])
    out_buf = torch.empty((M, cfg.H), dtype=torch.bfloat16, device="cuda")
    ids_buf = torch.empty((M, cfg.K_slots), dtype=torch.int32, device="cuda")

    def step():
        layer.forward(x, lg, topk_ids=ids_buf, out=out_buf)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K passes, one moe_forward call each, between two
    # synchronisations; events on the stream at both ends only.
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record()
    for _ in range(args.steps):
        step()
    r1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    gpu_ms = r0.elapsed_time(r1) / args.steps

    # The dominant kernel: K passes as the separate entry points, events
    # around GEMM1 only; then the other calls' share from a short loop with
    # events at every call.
    ps = Pass(layer, x, lg, M)
    g1 = gemm1_us(ps, args.steps)
    pre, g2 = breakdown(ps, min(args.steps, 20))

    ids = ids_buf.cpu().numpy()
    alg = algorithmic(cfg, M, ids)
    roof, mfma_bound, achieved, mdt = roofline(cfg, alg, g1, key)
    roof["layer"] = layer_roofline(cfg, alg, ms)
    out = {
        "metric": METRIC,
        "value": round(M / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE.get(cfg.quant, "fp8"),
        "data": "synthetic",
        "config": {"workload": workload_text(cfg, M), "tokens": M, "global_batch": M,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"gpu_ms_per_step": round(gpu_ms, 4), "us_route_align_quant": round(float(pre), 2),
                  "us_gemm1": round(float(g1), 2), "us_gemm2_combine": round(float(g2), 2),
                  "algorithmic_bytes": int(alg["layer_bytes"]),
                  "hbm_frac": round(alg["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "tflops": round(alg["flops"] / (ms * 1e-3) / 1e12, 3),
                  "touched_experts": alg["touched"], "assignments": alg["assignments"]},
    }
    del ps
    if not args.no_prefill and args.workload == "cfg2_M64" and args.act is None \
            and args.quant is None:
        out["prefill"] = prefill_block(args)
    if not args.no_peaks:
        pk = measured_peaks()
        out["measured_peaks"] = pk
        mp = pk[f"{mdt}_mfma_tflops"] if mfma_bound else pk["hbm_read_gbs"]
        out["roofline"]["measured_peak"] = mp
        out["roofline"]["frac_of_measured"] = round(achieved / mp, 4)
    if not args.no_sweep:
        out["sweep"] = sweep(cfg, W, layer)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, W, tok, sc, args.cpu_seconds)
    print(json.dumps(out), flush=True)


DTYPE = {"bf16": "bf16", "w4a8": "int4xfp8", "mxfp8": "mxfp8", "mxfp4": "mxfp4xmxfp8"}


def workload_text(cfg, M):
    return (f"{cfg.name} M={M}: hidden {cfg.H}, {cfg.E_routed} routed + {cfg.n_shared} shared "
            f"experts, top-{cfg.top_k}, intermediate {cfg.I}, {cfg.act}, {cfg.quant}")


def gemm1_us(ps, n):
    """Average GEMM1 duration (us) over n passes of the separate entry points,
    from HIP events recorded on the launching stream around GEMM1 only."""
    import numpy as np
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        ps.run(g1_ev=evs[k])
    torch.cuda.synchronize()
    return float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)


def breakdown(ps, n):
    """Average (route + align + quantise, GEMM2 + combine) durations in us."""
    import numpy as np
    import torch
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    for k in range(n):
        ps.run(evb[k])
    torch.cuda.synchronize()
    pre = np.mean([e[0].elapsed_time(e[1]) for e in evb]) * 1e3
    g2 = np.mean([e[2].elapsed_time(e[3]) for e in evb]) * 1e3
    return float(pre), float(g2)


def roofline(cfg, alg, g1, key):
    """GEMM1's roofline: the larger of its weight-streaming and its MFMA time at
    the nominal peaks decides the bound."""
    mdt = "bf16" if cfg.quant == "bf16" else "fp8"
    mpeak = MFMA_PEAK_TFLOPS[mdt]
    mfma_bound = alg["gemm1_flops"] / (mpeak * 1e12) > alg["gemm1_bytes"] / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        achieved = alg["gemm1_flops"] / (g1 * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": "gemm1_act", "achieved": round(achieved, 1),
                "peak": mpeak, "unit": "TFLOP/s", "frac": round(achieved / mpeak, 4),
                "traffic": traffic_record(key),
                "algorithmic_flops_per_launch": int(alg["gemm1_flops"]),
                "avg_launch_us": round(float(g1), 2)}
    else:
        achieved = alg["gemm1_bytes"] / (g1 * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": "gemm1_act", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_record(key),
                "algorithmic_bytes_per_launch": int(alg["gemm1_bytes"]),
                "avg_launch_us": round(float(g1), 2)}
    return roof, mfma_bound, achieved, mdt


def layer_roofline(cfg, alg, ms):
    """The whole pass against its binding roofline (by arithmetic intensity)."""
    mdt = "bf16" if cfg.quant == "bf16" else "fp8"
    mpeak = MFMA_PEAK_TFLOPS[mdt]
    t = ms * 1e-3
    if alg["flops"] / (mpeak * 1e12) > alg["layer_bytes"] / (HBM_PEAK_GBS * 1e9):
        a = alg["flops"] / t / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": mpeak, "unit": "TFLOP/s",
                "frac": round(a / mpeak, 4), "algorithmic_flops": int(alg["flops"]),
                "ms_per_pass": round(ms, 4)}
    a = alg["layer_bytes"] / t / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(alg["layer_bytes"]),
            "ms_per_pass": round(ms, 4)}


def prefill_block(args):
    """One moe_forward pass per step of each prefill-sized workload: tokens/s,
    TFLOP/s and the pass's and GEMM1's fractions of their roofline."""
    import torch
    import synth
    res = []
    for name in args.prefill_workloads.split(","):
        cfg, M = workload(name)
        t_gen = time.perf_counter()
        W = synth.make_weights(cfg)
        tok = synth.make_tokens(cfg, M)
        sc = synth.make_act_scales(cfg, tok["x_bits"])
        layer = make_layer(cfg, W, sc["a1"], sc["a2"])
        del W
        x, lg = to_dev(tok["x_bits"]), to_dev(tok["logits"])
        out = torch.empty((M, cfg.H), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((M, cfg.K_slots), dtype=torch.int32, device="cuda")
        gen_s = time.perf_counter() - t_gen
        for _ in range(args.prefill_warmup):
            layer.forward(x, lg, topk_ids=ids, out=out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.prefill_steps):
            layer.forward(x, lg, topk_ids=ids, out=out)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.prefill_steps
        ps = Pass(layer, x, lg, M)
        g1 = gemm1_us(ps, 5)
        pre, g2 = breakdown(ps, 5)
        alg = algorithmic(cfg, M, ids.cpu().numpy())
        roof, _, _, _ = roofline(cfg, alg, g1, name)
        lay = layer_roofline(cfg, alg, ms)
        res.append({"workload": workload_text(cfg, M), "key": name, "tokens": M,
                    "steps": args.prefill_steps, "warmup": args.prefill_warmup,
                    "ms_per_step": round(ms, 4), "tokens_per_s": round(M / (ms * 1e-3), 1),
                    "tflops": round(alg["flops"] / (ms * 1e-3) / 1e12, 1),
                    "dtype": DTYPE.get(cfg.quant, "fp8"), "layer": lay,
                    "gemm1": {"us": round(g1, 1), "bound": roof["bound"], "frac": roof["frac"],
                              "achieved": roof["achieved"], "unit": roof["unit"]},
                    "us_route_align_quant": round(pre, 1), "us_gemm2_combine": round(g2, 1),
                    "setup_s": round(gen_s, 1)})
        print(f"prefill {name}: {ms:.3f} ms/pass", file=sys.stderr, flush=True)
        del layer, ps, x, lg, out, ids
        torch.cuda.empty_cache()
    return res


def measured_peaks():
    """The achievable peaks on this device, measured after the timed region
    with the library's measurement kernels (include/moe_probe.h): a 2 GiB
    non-temporal read stream, and dense bf16 / fp8 MFMA loops on all SIMDs."""
    import torch
    import mixture_experts_layer_09_amd as moe

    def timed(fn, n):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n

    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.empty(moe.lib.moe_probe_read_blocks(), dtype=torch.int32, device="cuda")
    t = timed(lambda: moe.probe_read(buf, sink), 10)
    out = {"hbm_read_gbs": round(buf.numel() / t / 1e9, 1)}
    del buf
    msink = torch.empty(moe.lib.moe_probe_mfma_blocks() * 256, dtype=torch.float32, device="cuda")
    for dt in ("bf16", "fp8"):
        flops = [0]
        t = timed(lambda: flops.__setitem__(0, moe.probe_mfma(dt, 2000, msink)), 5)
        out[f"{dt}_mfma_tflops"] = round(flops[0] / t / 1e12, 1)
    out["method"] = ("moe_probe_read over 2 GiB (16-byte non-temporal lane loads); "
                     "moe_probe_mfma: 8 independent MFMA chains per wave, 4 waves per SIMD")
    return out


def sweep(cfg, W, layer):
    """Each token count of the configuration, timed one pass at a time with
    the caches evicted (a 512 MiB write) before each, outside the events:
    `us_median` is one moe_forward call (the library issues its kernels
    back to back from one host call), `us_components_median` the separate
    entry points the timed steps above issue from Python."""
    import numpy as np
    import torch
    import synth
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    res = []

    def timed(run, n=10):
        times = []
        for _ in range(n):
            flush.fill_(1.0)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            run()
            e.record()
            e.synchronize()
            times.append(s.elapsed_time(e) * 1e3)
        return times

    for M in cfg.Ms:
        tok = synth.make_tokens(cfg, M)
        x, lg = to_dev(tok["x_bits"]), to_dev(tok["logits"])
        ps = Pass(layer, x, lg, M)
        out = torch.empty((M, cfg.H), dtype=torch.bfloat16, device="cuda")
        fwd = lambda: layer.forward(x, lg, out=out)
        for _ in range(3):
            ps.run()
            fwd()
        comp = timed(ps.run)
        times = timed(fwd)
        us = float(np.median(times))
        alg = algorithmic(cfg, M, ps.b["topk_ids"].cpu().numpy())
        res.append({"M": M, "us_median": round(us, 2), "us_min": round(float(min(times)), 2),
                    "tokens_per_s": round(M / (us * 1e-6), 1),
                    "hbm_frac": round(alg["layer_bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "us_components_median": round(float(np.median(comp)), 2),
                    "touched_experts": alg["touched"]})
    del flush
    return res


if __name__ == "__main__":
    main()
