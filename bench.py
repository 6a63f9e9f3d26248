#!/usr/bin/env python3
"""Bench: batch-1 cachedStep tokens/s of GPT-2 124M (fp32, int8 group-64 and binary16
weight storage) on one MI355X, as absolute numbers and as a fraction of the HBM
roofline, with the CPU oracle timed on the host beside it.

A step is one cachedStep call: one token through the 12 blocks and the tied head.
The workload is the 128-position session (uniform-random token ids, seed 101) of
the seed-0 N(0, 0.02) checkpoint.  Each weight form first runs the whole session in
order, which fills a 128-position cache; the timed steps then take positions
p = 37*i mod 128 (i = 0, 1, ...), so any number of steps samples the whole range
0..127 (128 steps visit every position once), each step reading the session's
rows 0..p-1 and rewriting row p with the same values.  Inputs are resident in HBM
before timing starts.  After every timed leg the workspace error word is read: a
nonzero word (a bounded wait inside the step gave up, so that step's outputs are
invalid) is printed in the line and the bench exits with status 1.
Prints one JSON line.

--timeline: per-block phase times of the single-launch step from its timestamp
hook (fp32 and int8 at chosen positions) and per-position step times over the
session, as a markdown summary (no JSON line).
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
# the head (123,532,032 weights), i.e. 15,812,100,096 FLOP per step, against the fp32
# vector FMA rate: 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz = 78.6 TFLOP/s with
# the unpacked instructions this library is built for (packed fp32 is turned off); the
# packed-instruction figure, 157.3 TFLOP/s, is reported beside it.
BATCH = 64
BATCH_FLOP = 2 * BATCH * 123_532_032
FP32_VECTOR_PEAK_TF = 78.6
FP32_VECTOR_PACKED_PEAK_TF = 157.3

STRIDE = 37  # odd, so p = 37 i mod 128 visits all 128 positions in any 128 consecutive steps
NPOS = 128


def step_bytes(fixed: int, p: int) -> int:
    return fixed + KV_PER_POS * (p + 1) + LOGITS


def spread_positions(n: int, start: int = 0):
    return [(STRIDE * i) % NPOS for i in range(start, start + n)]


# Measured memory traffic of the step kernels: a text summary under profiles/ (two
# rocprofv3 --pmc runs of `bench.py --pmc-probe`, FETCH_SIZE then WRITE_SIZE, scaled by
# a plain copy of known size).  Its figures hold for the kernel sources they name by
# SHA-256; after any change to those sources the traffic is unknown (null) until the
# counters are taken again.
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
    """Bytes per step launch (fp32 kernel; key ..._f16 / ..._q8 for the other forms)
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, toks, cycle_seconds: float) -> dict:
    """The oracle as it stands, on the host: single-thread medians of the fp32 and
    int8 steps at positions 0..7 and one infer(128); then all threads (OpenMP over
    independent outputs, bit-identical to one thread) cycling the fp32 and int8 steps
    over the session for a time budget, and one infer(128)."""
    import numpy as np

    import oracle
    import synth
    if not os.path.exists(oracle.LIB):
        oracle.build()
    d = synth.GPT2
    per = oracle.cache_words_per_pos(d)
    q8 = oracle.q8_quantize_weights(d, w)  # the packing, not timed

    def step(kind, cache, p):
        if kind == "int8":
            rc, _ = oracle.q8_cached_step(d, w, q8[0], q8[1], cache, p * per, int(toks[p]), p)
        else:
            rc, _ = oracle.cached_step(d, w, cache, p * per, int(toks[p]), p)
        assert rc == 0, rc

    def first8(kind):
        cache = np.zeros(8 * per, np.float32)
        ts = []
        for p in range(8):
            t0 = time.perf_counter()
            step(kind, cache, p)
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    def cycle(kind, seconds):
        cache = np.zeros(NPOS * per, np.float32)
        n, t0 = 0, time.perf_counter()
        while n == 0 or time.perf_counter() - t0 < seconds:
            step(kind, cache, n % NPOS)
            n += 1
        el = time.perf_counter() - t0
        return n, el

    def infer128():
        t0 = time.perf_counter()
        rc, _ = oracle.infer(d, w, toks[:NPOS])
        assert rc == 0, rc
        return time.perf_counter() - t0

    oracle.set_threads(1)
    st = {"fp32_step_ms_median_pos0_7": round(first8("fp32") * 1e3, 2),
          "int8_step_ms_median_pos0_7": round(first8("int8") * 1e3, 2),
          "infer128_s": round(infer128(), 2)}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    nthreads = max(1, min(avail, 16))
    oracle.set_threads(nthreads)
    used = oracle.max_threads()
    n32, el32 = cycle("fp32", cycle_seconds)
    n8, el8 = cycle("int8", cycle_seconds / 2)
    inf_all = infer128()
    return {"value": round(n32 / el32, 3), "unit": "tok/s", "cores": used, "kind": "oracle",
            "sample": f"fp32 cachedStep on {used} threads: {n32} calls cycling positions 0..127 of the 128-token "
                      f"session ({el32:.1f} s); int8 {n8} calls ({el8:.1f} s); infer(128) once; single-thread: "
                      f"steps at positions 0..7 and one infer(128)",
            "host_cpus": os.cpu_count(), "affinity_cpus": avail, "cpu_model": cpu_model(),
            "single_thread": st,
            "all_threads": {"threads": used, "fp32_tok_s": round(n32 / el32, 3), "int8_tok_s": round(n8 / el8, 3),
                            "infer128_s": round(inf_all, 2)}}


# ---- --timeline ---------------------------------------------------------------
# The single-launch step's timestamp hook (gpt2_test_fused_trace) writes a 100 MHz
# wall-clock stamp per workgroup: slot 0 at its start; for block l, computed by the
# set l % 2, slot 1+4l when the block input x is in LDS (head units: after their
# share of the reduce-scatter), 2+4l when a regular unit's QKV rows are published
# (head units: attention output ready), 3+4l when x1 is in LDS, 4+4l when the
# XCD's GELU slice is in LDS; 49 head input, 50 head rows done, 51 end.  Workgroup
# b runs on XCD b % 8 with rank b // 8 (the kernel checks this placement): set =
# rank % 2, q = rank // 2, and it is a head unit when q < (2 if XCD < 4 else 1).
TICK_US = 0.01
NGRID = 256


def _roles():
    reg = {0: [], 1: []}
    head = {0: [], 1: []}
    for b in range(NGRID):
        X, rank = b % 8, b // 8
        st, q = rank % 2, rank // 2
        (head if q < (2 if X < 4 else 1) else reg)[st].append(b)
    return reg, head


def _block_phases(tr):
    """tr: [256][64] int ticks of one launch -> per-block phase times (us)."""
    import numpy as np
    reg, head = _roles()
    t0 = tr[:, 0].min()
    t = (tr.astype(np.int64) - t0) * TICK_US

    def med(slot, units):
        return float(np.median(t[units, slot]))

    rows = []
    for l in range(12):
        st = l % 2
        rows.append({"in": med(1 + 4 * l, reg[st]), "qkv": med(2 + 4 * l, reg[st]), "att": med(2 + 4 * l, head[st]),
                     "x1": med(3 + 4 * l, reg[st]), "g": med(4 + 4 * l, reg[st])})
    allu = list(range(NGRID))
    head_in, head_done, end = med(49, allu), float(t[:, 50].max()), float(t[:, 51].max())
    head_rows_start, head_preloaded = med(55, allu), med(57, allu)
    for l in range(12):
        rows[l]["next"] = rows[l + 1]["in"] if l < 11 else head_in
    # inside block 6 (set 0): regular units' wave 0 (52 the MLP terms' reduce-scatter
    # begins, 53 after the workgroup barrier, 54 x published, 56 x1 published) and wave 1
    # (59 after the QKV barrier, 60 LayerNorm output loaded, 62 MLP phase start, 63 MLP
    # partials published); head units' wave 0 (52 its reduce-scatter begins, 54 q/k/v
    # received, 56 output-projection terms published)
    det = {f"r{k}": med(k, reg[0]) for k in (52, 53, 54, 56, 59, 60, 62, 63)}
    det.update({f"h{k}": med(k, head[0]) for k in (52, 54, 56)})
    det.update({"head_rows_start": head_rows_start, "head_preloaded": head_preloaded})
    rows.append(det)
    return rows, head_in, head_done, end


def timeline_report(g, m, call, filled_cache, stream, positions, reps) -> int:
    import numpy as np
    import torch
    dev = m.packed.device
    trace = torch.zeros(NGRID * 64, dtype=torch.int64, device=dev)
    forms = (("fp32", g.gpt2_cached_step), ("int8-g64", g.gpt2_q8_cached_step))
    print("# Timeline of the single-launch step (medians over workgroups of a role, then over "
          f"{reps} launches; us from the first workgroup's start)\n")
    for name, fn in forms:
        cache = filled_cache(fn)
        for pos in positions:
            runs = []
            for _ in range(reps):
                trace.zero_()
                torch.cuda.synchronize()
                g.gpt2_test_fused_trace(trace.data_ptr())
                call(fn, cache, pos)
                torch.cuda.synchronize()
                g.gpt2_test_fused_trace(None)
                runs.append(_block_phases(trace.view(NGRID, 64).cpu().numpy()))
            keys = ("in", "qkv", "att", "x1", "g", "next")
            rows = [{k: float(np.median([r[0][l][k] for r in runs])) for k in keys} for l in range(12)]
            det = {k: float(np.median([r[0][12][k] for r in runs])) for k in runs[0][0][12]}
            head_in = float(np.median([r[1] for r in runs]))
            head_done = float(np.median([r[2] for r in runs]))
            end = float(np.median([r[3] for r in runs]))
            print(f"## {name}, position {pos}\n")
            print("| block | x in | x -> QKV published | QKV -> attention out | attention -> x1 | "
                  "x1 -> GELU slice | GELU -> next x | block |")
            print("|---|---|---|---|---|---|---|---|")
            for l, r in enumerate(rows):
                print(f"| {l} | {r['in']:.2f} | {r['qkv'] - r['in']:.2f} | {r['att'] - r['qkv']:.2f} | "
                      f"{r['x1'] - r['att']:.2f} | {r['g'] - r['x1']:.2f} | {r['next'] - r['g']:.2f} | "
                      f"{r['next'] - r['in']:.2f} |")
            blk = [r["next"] - r["in"] for r in rows]
            seg = {k: float(np.mean([r[b] - r[a] for r in rows]))
                   for a, b, k in (("in", "qkv", "qkv"), ("qkv", "att", "att"), ("att", "x1", "x1"),
                                   ("x1", "g", "g"), ("g", "next", "next"))}
            print(f"| mean | | {seg['qkv']:.2f} | {seg['att']:.2f} | {seg['x1']:.2f} | {seg['g']:.2f} | "
                  f"{seg['next']:.2f} | {float(np.mean(blk)):.2f} |\n")
            print(f"- start -> block 0 input: {rows[0]['in']:.2f} us; head input at {head_in:.2f} us; "
                  f"head rows done {head_done:.2f} us (head {head_done - head_in:.2f} us); last workgroup ends "
                  f"{end:.2f} us; head rows start {det['head_rows_start']:.2f} us (after the final LayerNorm), "
                  f"preloaded rows used by {det['head_preloaded']:.2f} us")
            b6 = rows[6]["in"]
            print("- inside block 6, us after its x is in LDS (previous block's MLP terms polled -> next input): "
                  f"regular wave 0: reduce-scatter begins {det['r52'] - b6:.2f}, after the barrier "
                  f"{det['r53'] - b6:.2f}, x published {det['r54'] - b6:.2f}, x1 published {det['r56'] - b6:.2f}; "
                  f"regular wave 1: after QKV barrier {det['r59'] - b6:.2f}, LayerNorm output loaded "
                  f"{det['r60'] - b6:.2f}, MLP phase start {det['r62'] - b6:.2f}, MLP partials published "
                  f"{det['r63'] - b6:.2f}; head wave 0: reduce-scatter begins {det['h52'] - b6:.2f}, "
                  f"q/k/v received {det['h54'] - b6:.2f}, output-projection terms published "
                  f"{det['h56'] - b6:.2f}\n")
        # per-position step time over the session (events around each launch), median of 3 passes
        per = np.zeros((3, NPOS))
        for rep in range(3):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(NPOS + 1)]
            ev[0].record(stream)
            for p in range(NPOS):
                call(fn, cache, p)
                ev[p + 1].record(stream)
            torch.cuda.synchronize()
            per[rep] = [ev[p].elapsed_time(ev[p + 1]) * 1e3 for p in range(NPOS)]
        med = np.median(per, axis=0)
        print(f"## {name}: step time by position (us, median of 3 passes over the session)\n")
        print("| positions | " + " | ".join(f"{a}..{a + 15}" for a in range(0, NPOS, 16)) + " |")
        print("|---|" + "---|" * (NPOS // 16))
        print("| mean | " + " | ".join(f"{med[a:a + 16].mean():.1f}" for a in range(0, NPOS, 16)) + " |\n")
        print(f"- session mean {med.mean():.2f} us, min {med.min():.2f}, max {med.max():.2f}\n")
    st = m.status()
    print(f"- workspace error word after the runs: {st}")
    return 1 if st else 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="time budget of the all-thread fp32 cycling leg (int8 takes half)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter runs: 128 fp32, 128 int8, then 128 binary16 steps (positions 0..127) and one "
                         "device copy of 256 MiB, nothing timed or printed")
    ap.add_argument("--prefill-probe", action="store_true",
                    help="for counter runs: 10 infer(128) calls and 10 batched steps (64 sessions, positions 0..9), "
                         "nothing timed or printed")
    ap.add_argument("--cache-probe", action="store_true",
                    help="fp32 and int8 step times with and without a 1 GiB device write between steps (which "
                         "evicts the L2 and the 256 MB Infinity Cache), markdown, no JSON line")
    ap.add_argument("--timeline", action="store_true",
                    help="per-block phase times and per-position step times (markdown), no JSON line")
    ap.add_argument("--timeline-positions", default="1,64,127")
    ap.add_argument("--timeline-reps", type=int, default=7)
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
    toks = synth.make_tokens(synth.SEED_SESSION, NPOS)
    ck = torch.from_numpy(w).to(dev)
    m = g.Model(ck, g.GPT2_PACK_F32 | g.GPT2_PACK_Q8 | g.GPT2_PACK_F16)
    torch.cuda.synchronize()
    del ck
    stream = torch.cuda.current_stream()
    logits = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device=dev)
    h, ws, lp, s = m.handle, m.ws.data_ptr(), logits.data_ptr(), stream.cuda_stream
    PER = g.GPT2_CACHE_WORDS_PER_POS
    FIXED = {g.gpt2_cached_step: F32_FIXED, g.gpt2_q8_cached_step: Q8_FIXED, g.gpt2_f16_cached_step: F16_FIXED}

    def call(fn, cache, p):
        rc = fn(h, cache.data_ptr(), p * PER, int(toks[p]), p, ws, lp, s)
        if rc:
            raise g.Gpt2Error(rc, fn.__name__)

    def filled_cache(fn):
        """A 128-position cache holding the session's rows (the session run in order)."""
        cache = m.new_cache(NPOS)
        for p in range(NPOS):
            call(fn, cache, p)
        return cache

    def timed(fn, steps, warmup):
        cache = filled_cache(fn)
        for p in spread_positions(warmup):
            call(fn, cache, p)
        pos = spread_positions(steps, warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for p in pos:
            call(fn, cache, p)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), sum(step_bytes(FIXED[fn], p) for p in pos), m.status()

    if args.pmc_probe:
        for fn in (g.gpt2_cached_step, g.gpt2_q8_cached_step, g.gpt2_f16_cached_step):
            filled_cache(fn)
        src = torch.ones(PMC_COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        st = m.status()
        m.close()
        return 1 if st else 0

    if args.cache_probe:
        # Each step timed alone (events on the step), positions spread over the filled
        # session; "evicted": a 1 GiB fill runs between steps, so no weight byte a step
        # reads can still be in the L2 or the Infinity Cache from the step before.
        big = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        print("# Step time with the caches warm and with them evicted between steps\n")
        print("| step | warm: median us | evicted: median us | evicted / warm |")
        print("|---|---|---|---|")
        for name, fn in (("fp32", g.gpt2_cached_step), ("int8-g64", g.gpt2_q8_cached_step)):
            cache = filled_cache(fn)
            res = {}
            for mode in ("warm", "evicted"):
                ts = []
                for p in spread_positions(128):
                    if mode == "evicted":
                        big.fill_(1.0)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    call(fn, cache, p)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1000)
                res[mode] = statistics.median(ts)
            print(f"| {name} | {res['warm']:.1f} | {res['evicted']:.1f} | {res['evicted'] / res['warm']:.3f} |")
        st = m.status()
        print(f"\n- workspace error word after the runs: {st}")
        m.close()
        return 1 if st else 0

    if args.prefill_probe:
        ptoks = synth.make_tokens(synth.SEED_PREFILL, NPOS).tolist()
        for _ in range(10):
            g.gpt2_infer(h, ptoks, ws, lp, s)
        btoks = np.stack([synth.make_tokens(synth.SEED_BATCH_BASE + b, NPOS) for b in range(BATCH)])
        bcaches = torch.zeros((BATCH, NPOS * PER), dtype=torch.float32, device=dev)
        blog = torch.empty((BATCH, g.GPT2_VOCAB), dtype=torch.float32, device=dev)
        for p in range(10):
            rc = g.gpt2_batched_cached_step(h, bcaches.data_ptr(), NPOS * PER, [p * PER] * BATCH,
                                            btoks[:, p].tolist(), [p] * BATCH, ws, blog.data_ptr(), s)
            if rc:
                raise g.Gpt2Error(rc, "gpt2_batched_cached_step")
        torch.cuda.synchronize()
        st = m.status()
        m.close()
        return 1 if st else 0

    if args.timeline:
        rc = timeline_report(g, m, call, filled_cache, stream,
                             [int(x) for x in args.timeline_positions.split(",") if x != ""], args.timeline_reps)
        m.close()
        return rc

    status = {}
    ms32, b32, status["fp32"] = timed(g.gpt2_cached_step, args.steps, args.warmup)
    ms8, b8, status["int8"] = timed(g.gpt2_q8_cached_step, args.steps, args.warmup)
    ms16, b16, status["binary16"] = timed(g.gpt2_f16_cached_step, args.steps, args.warmup)
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
    ref = torch.empty((NPOS, g.GPT2_VOCAB), dtype=torch.float32, device=dev)
    vcache = m.new_cache(NPOS)
    for p in range(NPOS):
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
            for p in range(NPOS):
                rc = g.gpt2_q8_cached_step_grouped(mv.handle, gx, vcache.data_ptr(), p * PER, int(toks[p]), p,
                                                   mv.ws.data_ptr(), vout[p].data_ptr(), s)
                if rc:
                    raise g.Gpt2Error(rc, "gpt2_q8_cached_step_grouped")
            e1.record(stream)
            torch.cuda.synchronize()
            vts.append(e0.elapsed_time(e1) / NPOS)
        status[f"q8_variant_{gw or 'row'}_{gx or 'row'}"] = mv.status()
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
    gcache = torch.zeros(NPOS * PER, dtype=torch.float32, device=dev)
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
    status["generate"] = m.status()
    status["generate_logits"] = int(gst.item())
    gms = statistics.median(gts)

    # batched step: 64 sessions (seeded token streams 1000..1063) advanced together over
    # positions 0..127, after a warm-up pass over positions 0..15; per batched step, the
    # median of three passes over the 128 positions (each pass rewrites the cache rows
    # it reads, so every pass does the same work)
    btoks = np.stack([synth.make_tokens(synth.SEED_BATCH_BASE + b, NPOS) for b in range(BATCH)])
    bcaches = torch.zeros((BATCH, NPOS * PER), dtype=torch.float32, device=dev)
    blog = torch.empty((BATCH, g.GPT2_VOCAB), dtype=torch.float32, device=dev)

    def bstep(p):
        rc = g.gpt2_batched_cached_step(h, bcaches.data_ptr(), NPOS * PER, [p * PER] * BATCH,
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
        for p in range(NPOS):
            bstep(p)
        e1.record(stream)
        torch.cuda.synchronize()
        bts.append(e0.elapsed_time(e1) / NPOS)
    bms = statistics.median(bts)
    status["batched"] = m.status()
    del bcaches, blog

    # prefill: median of 20 infer(128) calls after warm-up
    ptoks = synth.make_tokens(synth.SEED_PREFILL, NPOS).tolist()
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
    status["prefill"] = m.status()

    cpu = None if args.skip_cpu else cpu_baseline(w, toks, args.cpu_seconds)

    bflops = BATCH_FLOP / (bms * 1e-3) / 1e12
    pos_note = (f"positions 37*i mod 128 over a filled 128-position cache "
                f"({'all 128' if args.steps >= NPOS else str(len(set(spread_positions(args.steps, args.warmup))))} "
                f"distinct positions timed)")
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
                   "positions": pos_note, "batch": 1},
        "roofline": {"bound": "hbm", "achieved": round(gbs32, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs32 / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
        "status": status,
        "int8_g64": {"value": round(tok8, 1), "unit": "tok/s", "ms_per_step": round(ms8 / args.steps, 5),
                     "roofline": {"bound": "hbm", "achieved": round(gbs8, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(gbs8 / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic("traffic_bytes_per_launch_q8")}},
        "f16_weights": {"value": round(tok16, 1), "unit": "tok/s", "ms_per_step": round(ms16 / args.steps, 5),
                        "roofline": {"bound": "hbm", "achieved": round(gbs16, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs16 / HBM_PEAK_GBS, 4),
                                     "traffic": measured_traffic("traffic_bytes_per_launch_f16")}},
        "q8_variants": {"session": "128 positions, seed-101 tokens, seed-0 checkpoint", "rows": variants},
        "batched": {"value": round(BATCH / (bms * 1e-3), 1), "unit": "tok/s", "ms_per_step": round(bms, 4),
                    "sample": "64 sessions advanced together, positions 0..127 (fp32), median of 3 passes",
                    "roofline": {"bound": "alu", "achieved": round(bflops, 2), "peak": FP32_VECTOR_PEAK_TF,
                                 "unit": "TFLOP/s", "frac": round(bflops / FP32_VECTOR_PEAK_TF, 4),
                                 "peak_packed_fp32": FP32_VECTOR_PACKED_PEAK_TF,
                                 "frac_of_packed_peak": round(bflops / FP32_VECTOR_PACKED_PEAK_TF, 4)}},
        "generate": {"value": round(120 / (gms * 1e-3), 1), "unit": "tok/s", "ms_per_call": round(gms, 3),
                     "sample": "fp32 greedy, 8-token prompt + 120 tokens chosen on the GPU (127 steps)"},
        "prefill": {"value": round(NPOS / (pms * 1e-3), 1), "unit": "tok/s", "ms_median": round(pms, 4),
                    "roofline": {"bound": "mfma", "achieved": round(PREFILL_FLOP / (pms * 1e-3) / 1e12, 2),
                                 "peak": FP32_MFMA_PEAK_TF, "unit": "TFLOP/s",
                                 "frac": round(PREFILL_FLOP / (pms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TF, 4)}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    m.close()
    bad = {k: v for k, v in status.items() if v}
    if bad:
        print(f"workspace error words set: {bad}; the timed outputs are invalid", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
