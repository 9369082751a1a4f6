"""Benchmark of the KDA operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one kda_chunk_fwd call (gate, intra-chunk tiles, UT/WY transform and
inter-chunk scan) over the 64K-token training-shaped prefill: B=1, H=16,
T=65536, d_k=d_v=128, bf16 q/k/v, fp32 theta ~ N(0, 2), beta, S0 = 0, seeded
synthetic data already resident in HBM.  The timed region is exactly K steps
between two device synchronisations, measured with HIP events on the stream the
kernels run on, after W untimed warm-up calls (the clocks settle after about
60 calls).  The same prefill with the output gate (kda_chunk_fwd_gated) is
timed the same way and reported in the "output_gate" object.  The 1M-token
prefill (B=1, H=16, T=2^20) is reported in "prefill_1m", and the ablation of the
bounded gate (kda_chunk_fwd against kda_chunk_fwd_unbounded at B=32, H=16,
T=4096, one segment) in "ablation".  The backward pass (kda_chunk_bwd) is timed
at that batch shape and at the 64K prefill ("backward").  The decode step (B=256,
H=16 fp32 state, in place) is timed over 1,024 consecutive steps as one interval
and reported in the "decode" object.  The fp64 oracle is timed on the host cores on a bounded
sample of the same prefill ("cpu_baseline").  Prints one JSON line.
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


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall / steps * 1e3


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
    return {"value": B * T_sample / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {T_sample} tokens of all {x['q'].shape[2]} heads of the same prefill "
                      f"(fp64 token-by-token recurrence, {dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU's clocks rise over the first ~50 ms of sustained work (a prefill call
    # takes ~1.2 ms cold and ~0.77 ms after about 60 calls), so the default warm-up
    # runs 100 calls before the timed ones.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=1024,
                    help="decode steps timed as one interval (the workload is 1,024 consecutive steps)")
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
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run one elementwise copy of MIB MiB (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the KDA operator "
              "shards over batch and heads without communication, see DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_gated_delta_12_amd as kda
    from chunked_gated_delta_12_amd import inputs as kin

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
    ms, wall_ms = time_calls(step, args.steps, args.warmup, stream)
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
        "wall_ms_per_step": wall_ms,
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

        gms, _ = time_calls(gstep, args.steps, args.warmup, stream)
        gbytes = nbytes + B * T * H * dv * es
        ggbs = gbytes / (gms * 1e-3) / 1e9
        out["output_gate"] = {"workload": w.name, "call": "kda_chunk_fwd_gated", "ms_per_step": gms,
                              "tokens_per_s": B * T / (gms * 1e-3), "achieved": ggbs,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ggbs / HBM_PEAK_GBS,
                              "algorithmic_bytes": gbytes, "time_vs_ungated": gms / ms}
        del z, og

    if not args.no_decode:
        dw = kin.DECODE_WORKLOADS["decode_b256"]
        S, gen = kin.decode_state(dw, device=dev)
        nt = 16
        tok = kin.decode_token(dw, gen, device=dev, steps=nt)
        od = torch.empty((dw.B, dw.H, dw.dv), device=dev, dtype=torch.bfloat16)
        it = [0]

        def dstep():
            i = it[0] % nt
            it[0] += 1
            kda.kda_decode_step(tok["q"][i], tok["k"][i], tok["v"][i], tok["theta"][i], tok["beta"][i], S,
                                o=od, stream=stream)

        dms, _ = time_calls(dstep, args.decode_steps, args.warmup, stream)
        dfl, dby = decode_work(dw.B, dw.H, dw.dk, dw.dv)
        gbs = dby / (dms * 1e-3) / 1e9
        out["decode"] = {"workload": dw.name, "B": dw.B, "H": dw.H, "d": dw.dk, "ms_per_step": dms,
                         "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "tokens_per_s": dw.B / (dms * 1e-3), "algorithmic_bytes": dby,
                         "steps_timed": args.decode_steps}
        if not args.no_gated:
            zd = kin.output_gate_preact((nt, dw.B, dw.H, dw.dv), dw.dtype, dw.seed, device=dev)

            def gdstep():
                i = it[0] % nt
                it[0] += 1
                kda.kda_decode_step_gated(tok["q"][i], tok["k"][i], tok["v"][i], tok["theta"][i],
                                          tok["beta"][i], S, zd[i], o=od, stream=stream)

            gdms, _ = time_calls(gdstep, args.decode_steps, args.warmup, stream)
            gdby = dby + dw.B * dw.H * dw.dv * 2
            out["decode"]["output_gate"] = {"ms_per_step": gdms, "achieved": gdby / (gdms * 1e-3) / 1e9,
                                            "frac": gdby / (gdms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                            "algorithmic_bytes": gdby}
            del zd
        del S, tok

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

        mms, _ = time_calls(mstep, 5, 3, stream)
        mfl, mby = prefill_work(mw.B, mw.T, mw.H, mw.dk, mw.dv, es=2, s0=mx["S0"] is not None)
        out["prefill_1m"] = {"workload": mw.name, "B": mw.B, "H": mw.H, "T": mw.T, "d": mw.dk,
                             "segments": mseg, "ms_per_call": mms, "tokens_per_s": mw.B * mw.T / (mms * 1e-3),
                             "achieved": mby / (mms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": mby / (mms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": mby,
                             "calls_timed": 5}
        del mx, mo, mS, mws

    if not args.no_backward and w.name == "prefill_64k":
        # The backward pass (fp32 matrix cores; segmented at this 64K prefill, one segment at
        # the batch shape): at the batch shape of the ablation and at this 64K prefill.
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

            bms, _ = time_calls(bwstep, reps, 3, stream)
            th = bwk.B * bwk.T * bwk.H
            bby = th * (es * (2 * bwk.dk + 2 * bwk.dv) + 4 * bwk.dk + 4 + 4 * (3 * bwk.dk + bwk.dv) + 4)
            bw[label] = {"B": bwk.B, "H": bwk.H, "T": bwk.T, "d": bwk.dk, "ms_per_call": bms,
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

        bms, _ = time_calls(bstep, 20, 20, stream)
        ums, _ = time_calls(ustep, 20, 20, stream)
        ntok = aw.B * aw.T
        out["ablation"] = {"workload": f"B={aw.B} H={aw.H} T={aw.T} d={aw.dk} {aw.dtype}, "
                                       f"theta N({aw.theta_mu},{aw.theta_sigma}), {aseg} segment(s)",
                           "bounded_call": "kda_chunk_fwd", "unbounded_call": "kda_chunk_fwd_unbounded",
                           "bounded_ms": bms, "unbounded_ms": ums, "unbounded_vs_bounded": ums / bms,
                           "bounded_tokens_per_s": ntok / (bms * 1e-3),
                           "unbounded_tokens_per_s": ntok / (ums * 1e-3)}
        del ax, ao, aS

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, dev)

    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1))
        Ts = min(args.cpu_tokens, T)
        out["cpu_baseline"] = cpu_baseline(x, Ts, threads)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
