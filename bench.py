"""Benchmark of the KDA operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one kda_chunk_fwd call (gate, intra-chunk tiles, UT/WY transform and
inter-chunk scan) over the 64K-token training-shaped prefill: B=1, H=16,
T=65536, d_k=d_v=128, bf16 q/k/v, fp32 theta ~ N(0, 2), beta, S0 = 0, seeded
synthetic data already resident in HBM.  The timed region is exactly K steps
between two device synchronisations, measured with HIP events on the stream the
kernels run on (one event between consecutive calls, so the mean, median and
minimum per call are all reported).  Before it come W untimed warm-up calls and
then further untimed calls until --min-warm-s seconds of sustained work have
passed: the GPU's clocks rise over the first tens of milliseconds of load, and a
serving or training loop runs at the settled clocks.  Every leg below is timed
the same way.

Legs, each an object of the JSON line: the same prefill with the output gate
("output_gate"); the 1M-token prefill B=1, H=16, T=2^20 ("prefill_1m"); the
backward pass at B=32, T=4096 and at the 64K prefill ("backward"); the ablation
of the bounded gate at B=32, H=16, T=4096, one segment ("ablation"); the decode
step over 1,024 consecutive in-place steps at B=256 (the workload), and at B=512
and 1024 beside a device copy of the same bytes, where the fp32 state (512 MiB,
1 GiB) is well beyond the 256 MB last-level cache ("decode"); the device's own
description and what a streaming copy and a dense bf16 matrix-core loop reach on
it ("device", "measured_peaks"); and the fp64 oracle timed on the host cores on
a bounded sample of the same prefill ("cpu_baseline").  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix-core peak
METRIC = "KDA chunk_fwd tokens/s @H16 d128 T64K; % bf16 MFMA peak; decode GB/s"


def prefill_work(B, T, H, dk, dv, es=2, s0=False, chunk=16):
    """Algorithmic flops and HBM bytes of one chunked prefill.
    flops per token*head: 6*dk*dv (state products) + 6*C*dk (A_kk, A_qk, W) + 4*C*dv (Ut, A_qk U);
    bytes per token*head: q, k, v, o in the storage type, theta fp32, beta fp32; plus S_T (and S0)."""
    th = B * T * H
    flops = th * (6 * dk * dv + 6 * chunk * dk + 4 * chunk * dv)
    nbytes = th * (es * (2 * dk + dv) + es * dv + 4 * dk + 4) + B * H * dk * dv * 4 * (2 if s0 else 1)
    return flops, nbytes


def decode_work(B, H, dk, dv, es=2):
    """Per step: fp32 state read + write, token inputs and output."""
    nbytes = B * H * (8 * dk * dv + es * (2 * dk + dv) + 4 * dk + 4 + es * dv)
    flops = B * H * 7 * dk * dv
    return flops, nbytes


MIN_WARM_S = 0.3   # sustained untimed work before every timed leg (clock ramp)


def time_calls(fn, steps, warmup, stream, min_warm_s=None):
    """W warm-up calls, then more until min_warm_s of sustained work, then `steps`
    timed calls with an event between consecutive calls.  Returns a dict of the
    mean (total / steps), median and minimum milliseconds per call, the host wall
    time per call, and how many untimed calls ran."""
    import torch
    min_warm_s = MIN_WARM_S if min_warm_s is None else min_warm_s
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    extra, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(4):
            fn()
        extra += 4
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return {"mean": ev[0].elapsed_time(ev[-1]) / steps, "median": med, "min": per[0],
            "wall": wall / steps * 1e3, "warmup_calls": warmup, "clock_warmup_calls": extra}


def timing_fields(t):
    return {"ms_mean": t["mean"], "ms_median": t["median"], "ms_min": t["min"],
            "untimed_calls": t["warmup_calls"] + t["clock_warmup_calls"]}


CHUNK_SOURCES = ("kda_chunk.hip", "kda_map.hip", "kda_out.hip", "kda_device.hpp", "kda_launch.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def chunk_source_digest():
    """sha256 over the sources of the chunked-prefill kernels: stored counter readings
    are only reported while the kernels they were taken on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_gated_delta_12_amd", "csrc")
    for name in CHUNK_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(workload, segments):
    """HBM bytes per kda_chunk_fwd call measured with FETCH_SIZE / WRITE_SIZE (rocprofv3
    --pmc, scaled by the counters of a copy of known size), or None when no reading exists
    for these kernel sources, workload and segment count."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("segments") != segments or rec.get("source_sha256") != chunk_source_digest():
        return None
    return rec.get("bytes_per_call")


def copy_calibration(mib, dev):
    """One elementwise copy (negation) of `mib` MiB of fp32: reads and writes exactly
    mib MiB each, so its FETCH_SIZE / WRITE_SIZE readings convert counter units to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(x, T_sample, threads):
    """The oracle as it stands, on the first T_sample tokens of every head."""
    import oracle
    sl = {k: (v[:, :T_sample].contiguous().cpu() if v is not None and v.dim() >= 3 else v)
          for k, v in x.items() if k != "S0"}
    t0 = time.perf_counter()
    oracle.chunk_fwd(sl["q"], sl["k"], sl["v"], sl["theta"], sl["beta"], None, nthreads=threads)
    dt = time.perf_counter() - t0
    B = x["q"].shape[0]
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"value": B * T_sample / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_nproc": os.cpu_count(), "host_cpus_usable": usable,
            "sample": f"first {T_sample} tokens of all {x['q'].shape[2]} heads of the same prefill "
                      f"(fp64 token-by-token recurrence on {threads} threads, one per head, {dt:.1f} s)"}


def measured_peaks(dev, stream, steps):
    """What the device delivers to kernels that do nothing else: a streaming copy of
    1 GiB (read + write) and a dense bf16 matrix-core loop (2 workgroups of 4
    wavefronts per compute unit, 8 independent 16x16x32 chains per wavefront)."""
    import torch
    from chunked_gated_delta_12_amd import peaks
    info = peaks.device_info(torch.cuda.current_device())
    n = 1 << 30
    src = torch.ones(n // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    t = time_calls(lambda: peaks.copy(src, dst, stream), steps, 3, stream)
    copy = {"bytes_moved": 2 * n, "GB_s": 2 * n / (t["mean"] * 1e-3) / 1e9,
            "GB_s_best": 2 * n / (t["min"] * 1e-3) / 1e9, **timing_fields(t)}
    del src, dst
    wg = 2 * info["compute_units"]
    sink = torch.empty(wg * 256, device=dev, dtype=torch.float32)
    iters = 40000
    flop = wg * 4 * iters * 8 * peaks.MFMA_FLOP
    t = time_calls(lambda: peaks.mfma_bf16(sink, wg, iters, stream), 10, 2, stream)
    clock_peak = info["compute_units"] * info["clock_mhz"] * 1e6 * 4096 / 1e12
    mfma = {"workgroups": wg, "iters": iters, "flop": flop,
            "TFLOP_s": flop / (t["mean"] * 1e-3) / 1e12, "TFLOP_s_best": flop / (t["min"] * 1e-3) / 1e12,
            "clock_derived_peak_TFLOP_s": clock_peak, **timing_fields(t)}
    return info, {"copy_1gib": copy, "mfma_bf16_loop": mfma}


def main():
    global MIN_WARM_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--min-warm-s", type=float, default=MIN_WARM_S,
                    help="untimed sustained work before each timed leg, after the warm-up calls")
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=1024,
                    help="decode steps timed as one interval (the workload is 1,024 consecutive steps)")
    ap.add_argument("--decode-batches", default="256,512,1024",
                    help="decode batch sizes to time (256 is the workload; larger ones put the state "
                         "beyond the last-level cache)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the timing of the calls with the output gate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-1m", action="store_true",
                    help="skip the timing of the 1M-token prefill (B=1, H=16, T=2^20)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the backward pass (kda_chunk_bwd)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the timing of the unbounded-gate ablation (kda_chunk_fwd_unbounded)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the copy and matrix-core reference measurements")
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one elementwise copy of MIB MiB (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the KDA operator "
              "shards over batch and heads without communication", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_gated_delta_12_amd as kda
    from chunked_gated_delta_12_amd import inputs as kin

    MIN_WARM_S = args.min_warm_s
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load_library()
    stream = torch.cuda.current_stream(dev)

    w = kin.WORKLOADS[args.workload]
    x = kin.chunk_inputs(w, device=dev)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    seg = args.segments or kda.kda_chunk_fwd_auto_segments(B, T, H, dk, dv)
    o = torch.empty((B, T, H, dv), device=dev, dtype=x["q"].dtype)
    S_T = torch.empty((B, H, dk, dv), device=dev, dtype=torch.float32)
    nws = kda.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, seg)
    ws = torch.empty(max(nws, 16), device=dev, dtype=torch.uint8)

    def step():
        kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["theta"], x["beta"], x["S0"], segments=seg,
                          o=o, S_T=S_T, workspace=ws, stream=stream)

    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    tm = time_calls(step, args.steps, args.warmup, stream)
    ms = tm["mean"]
    es = 2 if w.dtype == "bf16" else 4
    flops, nbytes = prefill_work(B, T, H, dk, dv, es=es, s0=x["S0"] is not None)
    achieved_gbs = nbytes / (ms * 1e-3) / 1e9
    achieved_tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": B * T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "wall_ms_per_step": tm["wall"],
        "timing": {**timing_fields(tm), "clock_warmup_s": MIN_WARM_S,
                   "tokens_per_s_at_median": B * T / (tm["median"] * 1e-3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "dk": dk, "dv": dv,
                   "theta": f"N({w.theta_mu},{w.theta_sigma})", "segments": seg,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": stored_traffic(w.name, seg),
                     "kernel": "kda_chunk_fwd (map + combine + out kernels, one call)",
                     "algorithmic_bytes": nbytes},
        "mfma": {"achieved": achieved_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": achieved_tflops / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": flops},
    }

    if not args.no_gated:
        # the same prefill with the output gate o * sigmoid(z): z is read once more
        z = kin.output_gate_preact((B, T, H, dv), w.dtype, w.seed, device=dev)
        og = torch.empty_like(o)

        def gstep():
            kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["theta"], x["beta"], z, x["S0"],
                                    segments=seg, o=og, S_T=S_T, workspace=ws, stream=stream)

        gt = time_calls(gstep, args.steps, args.warmup, stream)
        gms = gt["mean"]
        gbytes = nbytes + B * T * H * dv * es
        ggbs = gbytes / (gms * 1e-3) / 1e9
        out["output_gate"] = {"workload": w.name, "call": "kda_chunk_fwd_gated", "ms_per_step": gms,
                              **timing_fields(gt),
                              "tokens_per_s": B * T / (gms * 1e-3), "achieved": ggbs,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ggbs / HBM_PEAK_GBS,
                              "algorithmic_bytes": gbytes, "time_vs_ungated": gms / ms}
        del z, og

    if not args.no_decode:
        from chunked_gated_delta_12_amd import peaks
        base = kin.DECODE_WORKLOADS["decode_b256"]
        legs = {}
        for bsz in [int(b) for b in args.decode_batches.split(",") if b]:
            dw = kin.scaled(base, B=bsz) if bsz != base.B else base
            S, gen = kin.decode_state(dw, device=dev)
            nt = 16
            tok = kin.decode_token(dw, gen, device=dev, steps=nt)
            od = torch.empty((dw.B, dw.H, dw.dv), device=dev, dtype=torch.bfloat16)
            it = [0]

            def dstep():
                i = it[0] % nt
                it[0] += 1
                kda.kda_decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["theta"][i], tok["beta"][i],
                                    S, o=od, stream=stream)

            dt_ = time_calls(dstep, args.decode_steps, args.warmup, stream)
            dms = dt_["mean"]
            dfl, dby = decode_work(dw.B, dw.H, dw.dk, dw.dv)
            gbs = dby / (dms * 1e-3) / 1e9
            leg = {"workload": dw.name if bsz == base.B else f"decode_b{bsz}", "B": dw.B, "H": dw.H,
                   "d": dw.dk, "state_bytes": S.numel() * 4, "ms_per_step": dms, **timing_fields(dt_),
                   "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                   "tokens_per_s": dw.B / (dms * 1e-3), "algorithmic_bytes": dby,
                   "steps_timed": args.decode_steps}
            if not args.no_peaks:
                # a device copy of the state's bytes (read once, written once) in the same run
                dst = torch.empty_like(S)
                ct = time_calls(lambda: peaks.copy(S, dst, stream), 50, 3, stream)
                cgbs = 2 * S.numel() * 4 / (ct["mean"] * 1e-3) / 1e9
                leg["copy_same_state_bytes"] = {"GB_s": cgbs, **timing_fields(ct)}
                leg["achieved_vs_copy"] = gbs / cgbs
                del dst
            if bsz == base.B and not args.no_gated:
                zd = kin.output_gate_preact((nt, dw.B, dw.H, dw.dv), dw.dtype, dw.seed, device=dev)

                def gdstep():
                    i = it[0] % nt
                    it[0] += 1
                    kda.kda_decode_step_gated(tok["q"][i], tok["k"][i], tok["v"][i], tok["theta"][i],
                                              tok["beta"][i], S, zd[i], o=od, stream=stream)

                gdt = time_calls(gdstep, args.decode_steps, args.warmup, stream)
                gdms = gdt["mean"]
                gdby = dby + dw.B * dw.H * dw.dv * 2
                leg["output_gate"] = {"ms_per_step": gdms, **timing_fields(gdt),
                                      "achieved": gdby / (gdms * 1e-3) / 1e9,
                                      "frac": gdby / (gdms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "algorithmic_bytes": gdby}
                del zd
            legs[bsz] = leg
            del S, tok, od
        first = legs.get(base.B) or next(iter(legs.values()))
        out["decode"] = dict(first)
        out["decode"]["by_batch"] = {str(b): {k: v for k, v in l.items() if k != "output_gate"}
                                     for b, l in legs.items()}

    if not args.no_1m and w.name == "prefill_64k":
        # The 1M-context shape: B=1, H=16, T=2^20, d=128, same distributions (16 GiB of inputs).
        mw = kin.WORKLOADS["prefill_1m"]
        mx = kin.chunk_inputs(mw, device=dev)
        mseg = kda.kda_chunk_fwd_auto_segments(mw.B, mw.T, mw.H, mw.dk, mw.dv)
        mo = torch.empty((mw.B, mw.T, mw.H, mw.dv), device=dev, dtype=mx["q"].dtype)
        mS = torch.empty((mw.B, mw.H, mw.dk, mw.dv), device=dev, dtype=torch.float32)
        mws = torch.empty(max(16, kda.kda_chunk_fwd_workspace_size(mw.B, mw.T, mw.H, mw.dk, mw.dv, mseg)),
                          device=dev, dtype=torch.uint8)

        def mstep():
            kda.kda_chunk_fwd(mx["q"], mx["k"], mx["v"], mx["theta"], mx["beta"], mx["S0"], segments=mseg,
                              o=mo, S_T=mS, workspace=mws, stream=stream)

        mt = time_calls(mstep, 5, 2, stream)
        mms = mt["mean"]
        mfl, mby = prefill_work(mw.B, mw.T, mw.H, mw.dk, mw.dv, es=2, s0=mx["S0"] is not None)
        out["prefill_1m"] = {"workload": mw.name, "B": mw.B, "H": mw.H, "T": mw.T, "d": mw.dk,
                             "segments": mseg, "ms_per_call": mms, **timing_fields(mt),
                             "tokens_per_s": mw.B * mw.T / (mms * 1e-3),
                             "achieved": mby / (mms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": mby / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": mby,
                             "calls_timed": 5}
        del mx, mo, mS, mws

    if not args.no_backward and w.name == "prefill_64k":
        # The backward pass (segmented at this 64K prefill, one segment at the batch
        # shape): at the batch shape of the ablation and at this 64K prefill.
        bw = {}
        for label, bwk, reps in (("B32_T4096", kin.scaled(w, B=32, T=4096), 10), ("prefill_64k", w, 10)):
            bx = kin.chunk_inputs(bwk, device=dev) if bwk is not w else x
            gdo = torch.Generator(device=dev).manual_seed(bwk.seed + 2000)
            bdo = torch.randn((bwk.B, bwk.T, bwk.H, bwk.dv), generator=gdo, device=dev).to(bx["q"].dtype)
            bws = torch.empty(kda.kda_chunk_bwd_workspace_size(bwk.B, bwk.T, bwk.H, bwk.dk, bwk.dv),
                              dtype=torch.uint8, device=dev)

            def bwstep():
                kda.kda_chunk_bwd(bx["q"], bx["k"], bx["v"], bx["theta"], bx["beta"], bdo, bx["S0"],
                                  workspace=bws, stream=stream)

            bt = time_calls(bwstep, reps, 2, stream)
            bms = bt["mean"]
            th = bwk.B * bwk.T * bwk.H
            bby = th * (es * (2 * bwk.dk + 2 * bwk.dv) + 4 * bwk.dk + 4 + 4 * (3 * bwk.dk + bwk.dv) + 4)
            bw[label] = {"B": bwk.B, "H": bwk.H, "T": bwk.T, "d": bwk.dk, "ms_per_call": bms,
                         **timing_fields(bt),
                         "tokens_per_s": bwk.B * bwk.T / (bms * 1e-3), "algorithmic_bytes": bby,
                         "achieved": bby / (bms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bby / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, "calls_timed": reps}
            del bdo, bws
            if bwk is not w:
                del bx
        out["backward"] = {"call": "kda_chunk_bwd", **bw}

    if not args.no_ablation:
        # What the bound buys: the same batch-parallel prefill (one segment, 512 sequences
        # filling the chip) with the bounded gate (dense matrix-core diagonal tiles) and with
        # the unbounded -softplus gate (position-wise fp32 diagonal tiles).
        aw = kin.scaled(w, B=32, T=4096)
        ax = kin.chunk_inputs(aw, device=dev)
        ao = torch.empty((aw.B, aw.T, aw.H, aw.dv), device=dev, dtype=ax["q"].dtype)
        aS = torch.empty((aw.B, aw.H, aw.dk, aw.dv), device=dev, dtype=torch.float32)
        aseg = kda.kda_chunk_fwd_auto_segments(aw.B, aw.T, aw.H, aw.dk, aw.dv)

        def bstep():
            kda.kda_chunk_fwd(ax["q"], ax["k"], ax["v"], ax["theta"], ax["beta"], ax["S0"], segments=aseg,
                              o=ao, S_T=aS, stream=stream)

        def ustep():
            kda.kda_chunk_fwd_unbounded(ax["q"], ax["k"], ax["v"], ax["theta"], ax["beta"], ax["S0"],
                                        o=ao, S_T=aS, stream=stream)

        bt = time_calls(bstep, 20, 5, stream)
        ut = time_calls(ustep, 20, 5, stream)
        bms, ums = bt["mean"], ut["mean"]
        ntok = aw.B * aw.T
        out["ablation"] = {"workload": f"B={aw.B} H={aw.H} T={aw.T} d={aw.dk} {aw.dtype}, "
                                       f"theta N({aw.theta_mu},{aw.theta_sigma}), {aseg} segment(s)",
                           "bounded_call": "kda_chunk_fwd", "unbounded_call": "kda_chunk_fwd_unbounded",
                           "bounded_ms": bms, "unbounded_ms": ums, "unbounded_vs_bounded": ums / bms,
                           "bounded_ms_median": bt["median"], "unbounded_ms_median": ut["median"],
                           "bounded_tokens_per_s": ntok / (bms * 1e-3),
                           "unbounded_tokens_per_s": ntok / (ums * 1e-3)}
        del ax, ao, aS

    if not args.no_peaks:
        info, pk = measured_peaks(dev, stream, 20)
        out["device"] = info
        out["measured_peaks"] = pk
        out["roofline"]["frac_of_measured_copy"] = achieved_gbs / pk["copy_1gib"]["GB_s"]
        out["mfma"]["frac_of_measured_loop"] = achieved_tflops / pk["mfma_bf16_loop"]["TFLOP_s"]

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, dev)

    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1, B * H))
        Ts = min(args.cpu_tokens, T)
        out["cpu_baseline"] = cpu_baseline(x, Ts, threads)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
