#!/usr/bin/env python3
"""Bench: batch-1 cachedStep tokens/s of GPT-2 124M (fp32, int8 group-64 and binary16
weight storage) on one MI355X, as absolute numbers and as a fraction of the HBM
roofline, with the CPU oracle timed on the host beside it.

A step is one cachedStep call: one token through the 12 blocks and the tied head.
The workload is the 128-position session (uniform-random token ids, seed 101) of
the seed-0 N(0, 0.02) checkpoint: the timed steps walk positions 0..127 and start
over from an empty cache.  Inputs are resident in HBM before timing starts.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
FP32_MFMA_PEAK_TF = 157.3  # MI355X dense fp32 matrix

# Algorithmic bytes of one batch-1 step at position p (shapes only):
#   fp32: 48 block matrices 339,738,624 B + tied head 154,389,504 B + LayerNorm/bias
#         485,376 B + two embedding rows 6,144 B = 494,619,648 B;
#   int8: codes 123,532,032 B + group scales 7,720,752 B + LayerNorm/bias 485,376 B
#         + embedding rows 6,144 B = 131,744,304 B;
#   binary16 storage: block matrices 169,869,312 B + head 77,194,752 B + LayerNorm/bias
#         485,376 B + embedding rows (binary32) 6,144 B = 247,555,584 B;
#   both: key/value rows read for positions 0..p (73,728 B each, the new one
#         included) and 201,028 B of logits written.
F32_FIXED = 494_619_648
Q8_FIXED = 123_532_032 + 7_720_752 + 485_376 + 6_144
F16_FIXED = 169_869_312 + 77_194_752 + 485_376 + 6_144
KV_PER_POS = 73_728
LOGITS = 201_028
PREFILL_FLOP = 21_743_271_936 + 304_349_184  # block GEMMs + causal attention at T = 128
# Batched step, 64 sessions: 2 FLOP per weight and session over the 48 block matrices and
# the head (123,532,032 weights), i.e. 15,812,100,096 FLOP per step; fp32 vector FMA peak.
BATCH = 64
BATCH_FLOP = 2 * BATCH * 123_532_032
FP32_VECTOR_PEAK_TF = 157.3


def step_bytes(fixed: int, p: int) -> int:
    return fixed + KV_PER_POS * (p + 1) + LOGITS


# Measured memory traffic of the fp32 step kernel: a text summary under profiles/
# (two rocprofv3 --pmc runs of `bench.py --pmc-probe`, FETCH_SIZE then WRITE_SIZE,
# scaled by a plain copy of known size).  Its figures hold for the kernel sources
# they name by SHA-256; after any change to those sources the traffic is unknown
# (null) until the counters are taken again.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_fused_f32_b1_traffic.md")
KERNEL_SOURCES = ["fused.hip", "device.hpp", "internal.hpp", "layout.hpp"]
PMC_COPY_BYTES = 256 << 20


def kernel_sources_sha256() -> str:
    import hashlib
    hsh = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "stream_gpt_transformer_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def measured_traffic(key: str = "traffic_bytes_per_launch"):
    """Bytes per step launch (fp32 kernel; key ..._f16 for the binary16-weight kernel)
    from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(vals[key])
    except (KeyError, ValueError):
        return None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter runs: 128 fp32, 128 int8, then 128 binary16 steps (positions 0..127) and one "
                         "device copy of 256 MiB, nothing timed or printed")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the decode step is a single-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import stream_gpt_transformer_amd as g
    import synth

    dev = torch.device("cuda", int(os.environ.get("LOCAL_RANK", 0)))
    torch.cuda.set_device(dev)
    w = synth.make_checkpoint(0, synth.GPT2)
    toks = synth.make_tokens(synth.SEED_SESSION, 128)
    ck = torch.from_numpy(w).to(dev)
    m = g.Model(ck, g.GPT2_PACK_F32 | g.GPT2_PACK_Q8 | g.GPT2_PACK_F16)
    torch.cuda.synchronize()
    del ck
    stream = torch.cuda.current_stream()
    cache = m.new_cache(128)
    logits = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device=dev)
    h, ws, c, lp, s = m.handle, m.ws.data_ptr(), cache.data_ptr(), logits.data_ptr(), stream.cuda_stream
    PER = g.GPT2_CACHE_WORDS_PER_POS

    def run(fn, n, start=0):
        for i in range(start, start + n):
            p = i % 128
            rc = fn(h, c, p * PER, int(toks[p]), p, ws, lp, s)
            if rc:
                raise g.Gpt2Error(rc, fn.__name__)

    def timed(fn, steps, warmup):
        run(fn, warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(fn, steps)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        fixed = {g.gpt2_cached_step: F32_FIXED, g.gpt2_q8_cached_step: Q8_FIXED, g.gpt2_f16_cached_step: F16_FIXED}[fn]
        nbytes = sum(step_bytes(fixed, i % 128) for i in range(steps))
        return ms, nbytes

    if args.pmc_probe:
        run(g.gpt2_cached_step, 128)
        run(g.gpt2_q8_cached_step, 128)
        run(g.gpt2_f16_cached_step, 128)
        src = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        m.close()
        return 0

    ms32, b32 = timed(g.gpt2_cached_step, args.steps, args.warmup)
    ms8, b8 = timed(g.gpt2_q8_cached_step, args.steps, args.warmup)
    ms16, b16 = timed(g.gpt2_f16_cached_step, args.steps, args.warmup)
    tok32 = args.steps / (ms32 * 1e-3)
    tok8 = args.steps / (ms8 * 1e-3)
    tok16 = args.steps / (ms16 * 1e-3)
    gbs32 = b32 / (ms32 * 1e-3) / 1e9
    gbs8 = b8 / (ms8 * 1e-3) / 1e9
    gbs16 = b16 / (ms16 * 1e-3) / 1e9

    # int8 quantizer granularity variants (weight-scale group, input-scale group; 0 =
    # the whole row): ms/step over the 128-position session and the logits' deviation
    # from the fp32 step's on the same tokens (synthetic weights: a size of the
    # quantization error, not an accuracy claim)
    ref = torch.empty((128, g.GPT2_VOCAB), dtype=torch.float32, device=dev)
    vcache = m.new_cache(128)
    for p in range(128):
        g.gpt2_cached_step(h, vcache.data_ptr(), p * PER, int(toks[p]), p, ws, ref[p].data_ptr(), s)
    vout = torch.empty_like(ref)
    variants = []
    for gw, gx in ((64, 64), (0, 64), (64, 0), (0, 0), (128, 128), (256, 256)):
        if gw == 64:
            mv = m
        else:
            ckv = torch.from_numpy(w).to(dev)
            mv = g.Model(ckv, g.GPT2_PACK_Q8, q8_weight_group=gw)
            del ckv
        vts = []
        for rep in range(2):
            vcache.zero_()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for p in range(128):
                rc = g.gpt2_q8_cached_step_grouped(mv.handle, gx, vcache.data_ptr(), p * PER, int(toks[p]), p,
                                                   mv.ws.data_ptr(), vout[p].data_ptr(), s)
                if rc:
                    raise g.Gpt2Error(rc, "gpt2_q8_cached_step_grouped")
            e1.record(stream)
            torch.cuda.synchronize()
            vts.append(e0.elapsed_time(e1) / 128)
        dl = (vout - ref).abs()
        variants.append({"weight_group": gw or "row", "input_group": gx or "row",
                         "ms_per_step": round(min(vts), 4),
                         "kernel": "single launch" if gx == 64 else "per phase",
                         "max_abs_dlogit_vs_fp32": round(float(dl.max()), 5),
                         "mean_abs_dlogit_vs_fp32": round(float(dl.mean()), 6)})
        if mv is not m:
            mv.close()
            del mv

    # greedy generation on the device: an 8-token prompt and 120 chosen tokens
    # (127 steps and 120 on-device choices per call), median of 5 calls
    gprompt = toks[:8].tolist()
    gcache = torch.zeros(128 * PER, dtype=torch.float32, device=dev)
    gout = torch.empty(120, dtype=torch.int32, device=dev)
    gst = torch.empty(1, dtype=torch.int32, device=dev)
    gts = []
    for i in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        m.generate(gcache, gprompt, 120, logits, gout, gst)
        e1.record(stream)
        torch.cuda.synchronize()
        if i:
            gts.append(e0.elapsed_time(e1))
    assert int(gst.item()) == 0
    gms = statistics.median(gts)

    # batched step: 64 sessions (seeded token streams 1000..1063) advanced together over
    # positions 0..127, after a warm-up pass over positions 0..15; per batched step, the
    # median of three passes over the 128 positions (each pass rewrites the cache rows
    # it reads, so every pass does the same work)
    btoks = np.stack([synth.make_tokens(synth.SEED_BATCH_BASE + b, 128) for b in range(BATCH)])
    bcaches = torch.zeros((BATCH, 128 * PER), dtype=torch.float32, device=dev)
    blog = torch.empty((BATCH, g.GPT2_VOCAB), dtype=torch.float32, device=dev)

    def bstep(p):
        rc = g.gpt2_batched_cached_step(h, bcaches.data_ptr(), 128 * PER, [p * PER] * BATCH,
                                        btoks[:, p].tolist(), [p] * BATCH, ws, blog.data_ptr(), s)
        if rc:
            raise g.Gpt2Error(rc, "gpt2_batched_cached_step")

    for p in range(16):
        bstep(p)
    torch.cuda.synchronize()
    bts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for p in range(128):
            bstep(p)
        e1.record(stream)
        torch.cuda.synchronize()
        bts.append(e0.elapsed_time(e1) / 128)
    bms = statistics.median(bts)
    del bcaches, blog

    # prefill: median of 20 infer(128) calls after warm-up
    ptoks = synth.make_tokens(synth.SEED_PREFILL, 128).tolist()
    for _ in range(3):
        g.gpt2_infer(h, ptoks, ws, lp, s)
    pts = []
    for _ in range(20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.gpt2_infer(h, ptoks, ws, lp, s)
        e1.record(stream)
        torch.cuda.synchronize()
        pts.append(e0.elapsed_time(e1))
    pms = statistics.median(pts)

    cpu = None
    if not args.skip_cpu:
        import oracle
        oracle.build() if not os.path.exists(oracle.LIB) else None
        nthreads = min(os.cpu_count() or 1, 16)
        oracle.set_threads(nthreads)
        ocache = np.zeros(128 * PER, np.float32)
        t0 = time.perf_counter()
        n = 0
        # the session's positions in order, starting over from an empty cache after 127,
        # until the time budget is spent (at least one step)
        while n == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            p = n % 128
            rc, _ = oracle.cached_step(synth.GPT2, w, ocache, p * PER, int(toks[p]), p)
            assert rc == 0
            n += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(n / el, 3), "unit": "tok/s", "cores": oracle.max_threads(), "kind": "oracle",
               "sample": f"{n} fp32 cachedStep calls cycling positions 0..127 of the same 128-token session "
                         f"({el:.1f} s, OpenMP over independent outputs)"}

    out = {
        "metric": "batch-1 cachedStep tok/s (fp32 & int8-g64) + % of HBM roofline",
        "value": round(tok32, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms32 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seed-0 N(0,0.02) weights, seeded uniform token ids)",
        "config": {"workload": "GPT-2 124M batch-1 cachedStep, 128-position session, fp32",
                   "positions": "0..127 cycled", "batch": 1},
        "roofline": {"bound": "hbm", "achieved": round(gbs32, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs32 / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
        "int8_g64": {"value": round(tok8, 1), "unit": "tok/s", "ms_per_step": round(ms8 / args.steps, 5),
                     "roofline": {"bound": "hbm", "achieved": round(gbs8, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs8 / HBM_PEAK_GBS, 4)}},
        "f16_weights": {"value": round(tok16, 1), "unit": "tok/s", "ms_per_step": round(ms16 / args.steps, 5),
                        "roofline": {"bound": "hbm", "achieved": round(gbs16, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs16 / HBM_PEAK_GBS, 4),
                                     "traffic": measured_traffic("traffic_bytes_per_launch_f16")}},
        "q8_variants": {"session": "128 positions, seed-101 tokens, seed-0 checkpoint", "rows": variants},
        "batched": {"value": round(BATCH / (bms * 1e-3), 1), "unit": "tok/s", "ms_per_step": round(bms, 4),
                    "sample": "64 sessions advanced together, positions 0..127 (fp32), median of 3 passes",
                    "roofline": {"bound": "alu", "achieved": round(BATCH_FLOP / (bms * 1e-3) / 1e12, 2),
                                 "peak": FP32_VECTOR_PEAK_TF, "unit": "TFLOP/s",
                                 "frac": round(BATCH_FLOP / (bms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TF, 4)}},
        "generate": {"value": round(120 / (gms * 1e-3), 1), "unit": "tok/s", "ms_per_call": round(gms, 3),
                     "sample": "fp32 greedy, 8-token prompt + 120 tokens chosen on the GPU (127 steps)"},
        "prefill": {"value": round(128 / (pms * 1e-3), 1), "unit": "tok/s", "ms_median": round(pms, 4),
                    "roofline": {"bound": "mfma", "achieved": round(PREFILL_FLOP / (pms * 1e-3) / 1e12, 2),
                                 "peak": FP32_MFMA_PEAK_TF, "unit": "TFLOP/s",
                                 "frac": round(PREFILL_FLOP / (pms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TF, 4)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    m.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
