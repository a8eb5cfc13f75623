#!/usr/bin/env python3
"""Benchmark of the block-quantized integer GEMM/GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only-headline]

One step = the decode hot path on the decode workload (M=1, K=4096, N=12288):
quantize the fp32 activation row to Q8_0, then the thin-M Q8_0 GEMV against
Q8_0 weights, both in one launch (quantize_qgemm_q8_0).  The same step as two
calls (quantize_q8_0, qgemm_q8_0) and the GEMV alone are reported beside it.  The weights are rotated over 8 resident copies (428 MB, more
than the 256 MB Infinity Cache) so every step streams its weights from HBM.
`value` is algorithmic bytes per step / time per step (GB/s); inputs are
resident in HBM before timing starts.

Also reported (key "also"): the small Q8_0 GEMM (M=16, K=256, N=512; time
per call, launch-bound), the M=4 and M=16 decode steps, the prefill GEMM
(M=2048, K=5120, N=17408) and a short-prompt prefill against the same weights
(M=128), the long-prefill GEMM (M=18432, K=5120, N=5120, Student-t
activations with outlier channels), the grouped W4A8 MoE GEMM (947 tokens,
top-8 of 128 experts, K=2048, N=768) and its decode form (1, 4 and 16
tokens), the activation quantizer, the MoE combine, the GGUF import and the
host-CPU W4A8 decode kernel, each with its own roofline or baseline.

"roofline" describes the step's kernel (the fused quantize + GEMV): achieved =
algorithmic bytes per launch / mean launch duration, from HIP events recorded
on the launch stream around a timed region of back-to-back launches.  Timed
loops are captured once in a HIP graph and replayed (so Python launch
overhead is not counted); each graph's output is first checked bit for bit
against an eager run.  "eager_ms_per_step" is the same step launched from
Python one call at a time.

"cpu_baseline" times the CPU oracle (plain C; it splits its work over output
rows, so the single-row step runs on one thread) on the same step for ~5 s,
and names the host CPU.  Each "also" line carries "cpu_oracle": the oracle
timed on that configuration (the large GEMMs and the MoE GEMM on a stated
sample of their rows), ~25 s in all.  Both are reported baselines, not
targets.  "distribution" gives the median and 10th / 90th percentiles over
the timed replays of the headline step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8-equiv TOPS (% MFMA peak) prefill GEMM; GB/s (% HBM peak) M=1 GEMV"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0      # dense int8 MFMA, MI355X
# fp32 vector FMA lane-ops per second: MI355X's published 157.3 TFLOP/s fp32
# vector rate counts each FMA as two flops (256 CU x 128 lanes x 2.4 GHz);
# that rate needs packed fp32 instructions, which this library does not use.
# Unpacked, a SIMD retires 16 fp32 FMA lanes per cycle (the published fp64
# vector rate, 78.6 TFLOP/s): 256 CU x 64 lanes x 2.4 GHz.
VALU_LANE_OPS_PEAK = 157.3e12 / 2
VALU_LANE_OPS_UNPACKED = 78.6e12 / 2


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--only-headline", action="store_true", help="skip the secondary workloads")
    p.add_argument("--cpu-seconds", type=float, default=5.0,
                   help="seconds of oracle work for the headline step's CPU baseline")
    p.add_argument("--reps", type=int, default=15,
                   help="timed graph replays of the headline step (each of --steps launches)")
    p.add_argument("--workloads", default="decode,small,decode_m,prefill,prefill_short,long,moe,moe_decode,combine,gguf,host",
                   help="comma list of workloads to run (profiling); the JSON line "
                        "is printed only when decode is among them.  'copy' (never a "
                        "default) runs a plain device copy of known size, the "
                        "reference that HBM byte counters are scaled by")
    return p.parse_args()


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


WARM_S = 0.025  # untimed graph replays before each timed one


class Timer:
    """Mean duration per launch from HIP events recorded on the launch stream
    around a timed region of back-to-back launches.  Launch-bound loops are
    captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed, so the
    figure is GPU time, not Python launch overhead; every graph is first
    replayed against an eager run and its output compared bit for bit, then
    replayed untimed for WARM_S seconds before the one timed replay."""

    def __init__(self, torch):
        self.torch = torch

    def loop(self, fn, iters, graph=True, check=None, reps=1):
        """Mean ms per launch.  With reps > 1 the graph is replayed `reps`
        times, each replay timed on its own; the median is returned and the
        per-replay figures are kept in self.samples."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if not graph:
            torch.cuda.synchronize()
            a.record()
            for i in range(iters):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            self.samples = [a.elapsed_time(b) / iters]
            return self.samples[0]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(3):
                fn(i)              # warm up on the capture stream
            fn(iters - 1)          # eager run of the graph's last launch
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        if check is not None:
            ref = check().clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                fn(i)
        torch.cuda.synchronize()
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            if check is not None and not torch.equal(check(), ref):
                raise RuntimeError("graph replay %d differs from the eager result" % rep)
        # untimed replays until the GPU has been busy for WARM_S (its clocks
        # ramp over the first ~15 ms of load in a fresh process)
        t0 = time.time()
        while time.time() - t0 < WARM_S:
            g.replay()
            torch.cuda.synchronize()
        self.samples = []
        for _ in range(reps):
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            self.samples.append(a.elapsed_time(b) / iters)
        del g
        return float(np.median(self.samples))


def distribution(samples_ms):
    """Median and 10th / 90th percentiles of per-replay means, in µs."""
    q = np.percentile(np.asarray(samples_ms) * 1e3, [10, 50, 90])
    return {"replays": len(samples_ms), "p10_us": round(float(q[0]), 3),
            "median_us": round(float(q[1]), 3), "p90_us": round(float(q[2]), 3)}


# Workload names of the secondary lines; the CPU-oracle lines attach to the
# GPU lines by these names.
def name_small(s):
    return "small Q8_0 GEMM M=%d K=%d N=%d" % (s.m, s.k, s.n)


def name_decode(s):
    return "decode M=%d K=%d N=%d" % (s.m, s.k, s.n)


def name_gemm(name, s):
    return "%s GEMM M=%d K=%d N=%d" % (name, s.m, s.k, s.n)


def name_moe(m):
    return "grouped W4A8 T=%d top-%d E=%d K=%d N=%d" % (m.tokens, m.top_k, m.experts, m.k, m.n)


def name_moe_decode(m, T, active):
    return ("grouped W4A8 decode T=%d top-%d E=%d K=%d N=%d (%d active experts)"
            % (T, m.top_k, m.experts, m.k, m.n, active))


CSRC = os.path.join(ROOT, "block_quantized_integer_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TRAFFIC_SOURCE = ("stored figure, not measured in this run: HBM bytes per launch from the "
                  "rocprofv3 FETCH_SIZE and WRITE_SIZE passes recorded in profiles/traffic.json "
                  "(each scaled by a plain copy's reading); null when the kernel's sources have "
                  "changed since the counters were taken")


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic(key):
    """Measured HBM bytes per launch of one kernel on one workload, from the
    rocprofv3 FETCH_SIZE and WRITE_SIZE passes recorded in profiles/traffic.json
    (each scaled by the factor that a plain copy of known size gives the same
    counter).  None when no record exists or when the kernel's sources have
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_sha256(rec["sources"]):
        return None
    return rec["hbm_bytes_per_launch"]


def bench_copy(torch):
    """A plain device copy of known size (512 MiB read + 512 MiB written per
    launch): the calibration that FETCH_SIZE / WRITE_SIZE are scaled by."""
    n = 128 << 20
    x = torch.randn(n, device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log("copy calibration: 5 launches of neg over %d fp32 (%d bytes read, %d written each)"
        % (n, 4 * n, 4 * n))


def device_q8(bqi, torch, rows, k, std, gen, t_dist=False, outlier_cols=None):
    """Synthetic fp32 matrix on the device (seeded torch generator), quantized
    with the library's own quantize_q8_0."""
    if t_dist:
        # Student-t(3) = N / sqrt(chi2_3 / 3)
        z = torch.randn((rows, k), generator=gen, device="cuda", dtype=torch.float32)
        c = torch.randn((rows, k, 3), generator=gen, device="cuda", dtype=torch.float32)
        x = z / torch.sqrt((c * c).sum(-1) / 3.0)
        del c
        if outlier_cols is not None:
            x[:, torch.as_tensor(outlier_cols, device="cuda")] *= 20.0
    else:
        x = torch.randn((rows, k), generator=gen, device="cuda", dtype=torch.float32) * std
    q, d = bqi.quantize_q8_0(x)
    return x, q, d


def bench_headline(bqi, torch, W, args):
    s = W.DECODE[0]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    copies = 8
    log("decode workload M=%d K=%d N=%d, %d weight copies" % (s.m, s.k, s.n, copies))
    wq, wd = [], []
    for c in range(copies):
        _, q, d = device_q8(bqi, torch, s.n, s.k, 0.02, gen)
        wq.append(q)
        wd.append(d)
    x = torch.randn((s.m, s.k), generator=gen, device="cuda", dtype=torch.float32)
    aq = torch.empty((s.m, s.k), dtype=torch.int8, device="cuda")
    ad = torch.empty((s.m, s.k // 32), dtype=torch.int16, device="cuda")
    y = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        # the whole decode hot path in one launch: quantize x, multiply by W
        bqi.quantize_qgemm_q8_0(x, wq[i % copies], wd[i % copies], y, aq, ad)

    def step_two_calls(i):
        bqi.quantize_q8_0(x, aq, ad)
        bqi.qgemm_q8_0(aq, ad, wq[i % copies], wd[i % copies], y)

    def gemv(i):
        bqi.qgemm_q8_0(aq, ad, wq[i % copies], wd[i % copies], y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    T = Timer(torch)
    ms_step = T.loop(step, args.steps, check=lambda: y, reps=args.reps)
    dist = distribution(T.samples)
    ms_step_eager = T.loop(step, args.steps, graph=False)
    ms_two = T.loop(step_two_calls, args.steps, check=lambda: y)
    gemv_mean = T.loop(gemv, args.steps, check=lambda: y)

    w_bytes = s.n * s.k + s.n * (s.k // 32) * 2
    a_bytes = s.m * s.k + s.m * (s.k // 32) * 2
    y_bytes = s.m * s.n * 4
    gemv_bytes = w_bytes + a_bytes + y_bytes
    quant_bytes = s.m * s.k * 4 + a_bytes
    step_bytes = gemv_bytes + quant_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode GEMV M=1 K=4096 N=12288 (quantize_qgemm_q8_0: "
                               "quantize + Q8_0 GEMV in one launch)",
                   "m": s.m, "k": s.k, "n": s.n, "weights": "Q8_0 of N(0,0.02)",
                   "activations": "N(0,1) fp32, quantized to Q8_0 in the step",
                   "weight_copies_rotated": copies, "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "k_gemv_reg<1,4,ACT_F32> (quantize + GEMV)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic("k_gemv_reg<1,4,ACT_F32> decode M=1 fused"),
                     "traffic_source": TRAFFIC_SOURCE,
                     "bytes_per_launch": step_bytes,
                     "mean_launch_us": round(ms_step * 1e3, 3),
                     "timing": "median over %d timed replays of a HIP graph of %d back-to-back "
                               "launches (HIP events on the launch stream around each replay), "
                               "after %d eager warm-up steps and %.0f ms of untimed replays"
                               % (args.reps, args.steps, args.warmup, WARM_S * 1e3),
                     "distribution": dist},
        "eager_ms_per_step": round(ms_step_eager, 6),
        "two_call_step": {"calls": "quantize_q8_0 + qgemm_q8_0", "ms_per_step": round(ms_two, 6),
                          "GB/s": round(step_bytes / (ms_two * 1e-3) / 1e9, 2)},
        "gemv_only": {"kernel": "k_gemv_reg<1,4,ACT_Q8>", "mean_launch_us": round(gemv_mean * 1e3, 3),
                      "bytes_per_launch": gemv_bytes,
                      "GB/s": round(gemv_bytes / (gemv_mean * 1e-3) / 1e9, 2),
                      "frac_hbm_peak": round(gemv_bytes / (gemv_mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "traffic": traffic("k_gemv_reg<1,4> decode M=1")}
    }
    ctx = dict(s=s, wq=wq, wd=wd, x=x, step_bytes=step_bytes)
    return res, ctx


def bench_small(bqi, torch, W, iters):
    """The small Q8_0 GEMM configuration (M=16, K=256, N=512, seed 0): the
    whole call (quantize the fp32 activations and the GEMM, one launch of the
    MFMA thin-M kernel with the quantizer inside) is a few microseconds of
    latency, so it is reported as time per call."""
    s = W.SMALL
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    _, wq, wd = device_q8(bqi, torch, s.n, s.k, 0.02, gen)
    x = torch.randn((s.m, s.k), generator=gen, device="cuda", dtype=torch.float32)
    aq = torch.empty((s.m, s.k), dtype=torch.int8, device="cuda")
    ad = torch.empty((s.m, s.k // 32), dtype=torch.int16, device="cuda")
    y = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    log("small Q8_0 GEMM M=%d K=%d N=%d" % (s.m, s.k, s.n))
    T = Timer(torch)
    call = lambda i: bqi.quantize_qgemm_q8_0(x, wq, wd, y, aq, ad)
    ms = T.loop(call, iters, check=lambda: y, reps=9)
    dist = distribution(T.samples)
    ms_gemm = T.loop(lambda i: bqi.qgemm_q8_0(aq, ad, wq, wd, y), iters, check=lambda: y)
    ms_eager = T.loop(call, iters, graph=False)
    return {"workload": name_small(s),
            "kernel": "k_gemv_mfma16<1, ACT_F32> (quantize + GEMM in one launch)",
            "value": round(ms * 1e3, 3), "unit": "us per call (quantize + GEMM)",
            "higher_is_better": False, "bound": "launch",
            "distribution": dist,
            "gemm_only_us": round(ms_gemm * 1e3, 3),
            "eager_us_per_call": round(ms_eager * 1e3, 3),
            "int8_equiv_TOPS": round(2.0 * s.m * s.n * s.k / (ms * 1e-3) / 1e12, 4)}


def bench_decode_variants(bqi, torch, W, iters):
    """The decode GEMV at M = 4 and M = 16 (the other decode sizes of the
    configuration): the whole step through quantize_qgemm_q8_0 (the quantizer
    and the GEMV: one launch only pays off for M = 1) and the GEMV alone, 8
    rotated weight copies."""
    res = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    s1 = W.DECODE[0]
    copies = 8
    wq, wd = [], []
    for c in range(copies):
        _, q, d = device_q8(bqi, torch, s1.n, s1.k, 0.02, gen)
        wq.append(q)
        wd.append(d)
    for s in W.DECODE[1:]:
        log("decode workload M=%d K=%d N=%d" % (s.m, s.k, s.n))
        x = torch.randn((s.m, s.k), generator=gen, device="cuda", dtype=torch.float32)
        aq = torch.empty((s.m, s.k), dtype=torch.int8, device="cuda")
        ad = torch.empty((s.m, s.k // 32), dtype=torch.int16, device="cuda")
        y = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
        bqi.quantize_q8_0(x, aq, ad)
        T = Timer(torch)
        # the API step (one launch for m = 1 only; here quantize + GEMV)
        step = lambda i: bqi.quantize_qgemm_q8_0(x, wq[i % copies], wd[i % copies], y, aq, ad)
        gemv = "k_gemv_mfma16" if s.m > 4 else "k_gemv_reg<%d,4,ACT_Q8>" % s.m
        kernel = "k_quantize_q8_0 + " + gemv
        ms_step = T.loop(step, iters, check=lambda: y)
        ms_gemv = T.loop(lambda i: bqi.qgemm_q8_0(aq, ad, wq[i % copies], wd[i % copies], y), iters,
                         check=lambda: y)
        w_bytes = s.n * s.k + s.n * (s.k // 32) * 2
        a_bytes = s.m * s.k + s.m * (s.k // 32) * 2
        gemv_bytes = w_bytes + a_bytes + s.m * s.n * 4
        step_bytes = gemv_bytes + s.m * s.k * 4 + a_bytes
        res.append({"workload": name_decode(s), "kernel": kernel,
                    "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
                    "ms_per_step": round(ms_step, 6),
                    "frac_hbm_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "bytes_per_step": step_bytes,
                    "gemv_only": {"kernel": gemv, "mean_launch_us": round(ms_gemv * 1e3, 3),
                                  "GB/s": round(gemv_bytes / (ms_gemv * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(gemv_bytes / (ms_gemv * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes": gemv_bytes,
                                  "hbm_bytes_stored_counters": traffic("%s decode M=%d" % (gemv.split("<")[0], s.m))}})
    return res


def bench_gemm(bqi, torch, W, name, iters):
    s = {"prefill": W.PREFILL, "prefill_short": W.PREFILL_SHORT, "long": W.LONG}[name]
    gen = torch.Generator(device="cuda")
    gen.manual_seed({"prefill": 2, "long": 3, "prefill_short": 4}[name])
    # the library runs grids of at most one 128 x 128 tile per CU on its
    # 8-wave kernel, larger grids on the 4-wave one
    tiles = -(-s.m // 128) * -(-s.n // 128)
    kernel = ("k_gemm_mfma_w8" if tiles <= torch.cuda.get_device_properties(0).multi_processor_count
              else "k_gemm_mfma")
    log("%s GEMM M=%d K=%d N=%d" % (name, s.m, s.k, s.n))
    if name == "long":
        xa, aq, ad = device_q8(bqi, torch, s.m, s.k, 1.0, gen, t_dist=True,
                               outlier_cols=W.outlier_columns(s.k))
    else:
        xa, aq, ad = device_q8(bqi, torch, s.m, s.k, 1.0, gen)
    _, wq, wd = device_q8(bqi, torch, s.n, s.k, 0.02, gen)
    y = torch.empty((s.m, s.n), dtype=torch.float32, device="cuda")
    T = Timer(torch)
    mean = T.loop(lambda i: bqi.qgemm_q8_0(aq, ad, wq, wd, y), iters, check=lambda: y)
    # 100 launches per graph: with a handful, the graph's own launch cost
    # would be spread over too few of these short kernels
    qmean = T.loop(lambda i: bqi.quantize_q8_0(xa, aq, ad), 100, check=lambda: aq)
    ops = 2.0 * s.m * s.n * s.k
    tops = ops / (mean * 1e-3) / 1e12
    out_blocks = s.m * s.n * (s.k // 32)
    valu_ops = 2.0 * out_blocks  # the scale epilogue's two fp32 ops per output-block
    byt = (s.m + s.n) * (s.k + s.k // 32 * 2) + s.m * s.n * 4
    qbytes = s.m * s.k * 4 + s.m * (s.k + s.k // 32 * 2)
    del xa
    return {
        "workload": name_gemm(name, s),
        "kernel": kernel, "value": round(tops, 2), "unit": "int8-equiv TOPS",
        "mean_launch_us": round(mean * 1e3, 2),
        "frac_int8_mfma_peak": round(tops / INT8_PEAK_TOPS, 4),
        "epilogue_valu_frac": round(valu_ops / (mean * 1e-3) / VALU_LANE_OPS_PEAK, 4),
        "epilogue_valu_frac_unpacked": round(valu_ops / (mean * 1e-3) / VALU_LANE_OPS_UNPACKED, 4),
        "hbm_bytes_algorithmic": byt,
        "hbm_bytes_stored_counters": traffic("%s %s" % (kernel, name)),
        "quantize": {"kernel": "k_quantize_q8_0", "mean_launch_us": round(qmean * 1e3, 2),
                     "GB/s": round(qbytes / (qmean * 1e-3) / 1e9, 1),
                     "frac_hbm_peak": round(qbytes / (qmean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def bench_moe(bqi, torch, W, iters):
    m = W.MOE
    log("moe grouped W4A8: %d tokens top-%d of %d experts K=%d N=%d"
        % (m.tokens, m.top_k, m.experts, m.k, m.n))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    _, aq, ad = device_q8(bqi, torch, m.tokens, m.k, 1.0, gen)
    ids = torch.from_numpy(W.topk_ids(m.tokens, m.top_k, m.experts)).cuda()
    copies = 5
    wq, wd = [], []
    for _ in range(copies):
        wq.append(torch.randint(0, 256, (m.experts, m.n, m.k // 2), generator=gen,
                                device="cuda", dtype=torch.uint8))
        e = torch.randint(-12, -5, (m.experts, m.n, m.k // 32), generator=gen, device="cuda")
        mant = torch.rand((m.experts, m.n, m.k // 32), generator=gen, device="cuda") + 1.0
        wd.append(torch.ldexp(mant, e.float()).half().view(torch.int16))
    y = torch.empty((m.tokens, m.top_k, m.n), dtype=torch.float32, device="cuda")
    ws = torch.empty(bqi.workspace_size(m.tokens, m.top_k, m.experts, m.k), dtype=torch.uint8,
                     device="cuda")
    fn = lambda i: bqi.qgemm_w4a8_grouped(aq, ad, ids, wq[i % copies], wd[i % copies], y, ws)
    T = Timer(torch)
    mean = T.loop(fn, iters, check=lambda: y)
    R = m.tokens * m.top_k
    byt = (m.experts * m.n * (m.k // 2 + m.k // 32 * 2) + m.tokens * (m.k + m.k // 32 * 2)
           + R * 4 + R * m.n * 4)
    ops = 2.0 * R * m.n * m.k
    gbs = byt / (mean * 1e-3) / 1e9
    return {"workload": name_moe(m),
            "kernel": "k_route + k_grouped_w4a8", "value": round(gbs, 1), "unit": "GB/s",
            "mean_call_us": round(mean * 1e3, 2),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "int8_equiv_TOPS": round(ops / (mean * 1e-3) / 1e12, 2),
            "epilogue_valu_frac_unpacked": round(2.0 * R * m.n * (m.k // 32) / (mean * 1e-3)
                                                 / VALU_LANE_OPS_UNPACKED, 4),
            "weight_copies_rotated": copies, "hbm_bytes_algorithmic": byt,
            "hbm_bytes_stored_counters": traffic("k_grouped_w4a8 moe")}


def bench_moe_decode(bqi, torch, W, iters):
    """Grouped W4A8 decode on the MoE expert shapes: T in {1, 4, 16} tokens,
    top-8 of 128 experts, K=2048, N=768 (the v_dot4 GEMV path).  Bytes count
    the weights of the experts that receive rows, read once; 3 rotated weight
    copies (340 MB) defeat the Infinity Cache."""
    m = W.MOE
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    copies = 3
    wq, wd = [], []
    for _ in range(copies):
        wq.append(torch.randint(0, 256, (m.experts, m.n, m.k // 2), generator=gen,
                                device="cuda", dtype=torch.uint8))
        e = torch.randint(-12, -5, (m.experts, m.n, m.k // 32), generator=gen, device="cuda")
        mant = torch.rand((m.experts, m.n, m.k // 32), generator=gen, device="cuda") + 1.0
        wd.append(torch.ldexp(mant, e.float()).half().view(torch.int16))
    res = []
    for T in (1, 4, 16):
        _, aq, ad = device_q8(bqi, torch, T, m.k, 1.0, gen)
        ids_np = W.topk_ids(T, m.top_k, m.experts, seed=T)
        ids = torch.from_numpy(ids_np).cuda()
        y = torch.empty((T, m.top_k, m.n), dtype=torch.float32, device="cuda")
        ws = torch.empty(bqi.workspace_size(T, m.top_k, m.experts, m.k), dtype=torch.uint8,
                         device="cuda")
        fn = lambda i: bqi.qgemm_w4a8_grouped(aq, ad, ids, wq[i % copies], wd[i % copies], y, ws)
        mean = Timer(torch).loop(fn, iters, check=lambda: y)
        active = len(np.unique(ids_np))
        R = T * m.top_k
        byt = (active * m.n * (m.k // 2 + m.k // 32 * 2) + T * (m.k + m.k // 32 * 2)
               + R * 4 + R * m.n * 4)
        gbs = byt / (mean * 1e-3) / 1e9
        res.append({"workload": name_moe_decode(m, T, active),
                    "kernel": "k_grouped_gemv (no routing pass)", "value": round(gbs, 1), "unit": "GB/s",
                    "mean_call_us": round(mean * 1e3, 2),
                    "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "hbm_bytes_algorithmic": byt, "weight_copies_rotated": copies,
                    "hbm_bytes_stored_counters": traffic("k_grouped_gemv moe decode T=%d" % T)})
    return res


def bench_host_w4a8(bqi, W):
    """The host-CPU integer-SIMD W4A8 path (AVX2 vpmaddubsw) on the grouped
    decode workload (T tokens, top-8 of 128 experts, K=2048, N=768, weights in
    host RAM), against the plain CPU oracle on the same cores.  Synchronous
    host work: no GPU involved."""
    import oracle
    m = W.MOE
    g = np.random.default_rng(9)
    wq4 = g.integers(0, 256, (m.experts, m.n, m.k // 2), dtype=np.uint8)
    wd = W.random_scales("moe", 730, (m.experts, m.n, m.k // 32))
    threads = oracle.default_threads()
    res = []
    for T in (1, 4, 16):
        qa = W.random_int8("moe", 731, (T, m.k), seed=T)
        da = W.random_scales("moe", 732, (T, m.k // 32), seed=T)
        ids = W.topk_ids(T, m.top_k, m.experts, seed=T)
        active = len(np.unique(ids))
        wbytes = active * m.n * (m.k // 2 + m.k // 32 * 2)

        def timed(fn, min_s=0.5):
            fn()
            n, t0 = 0, time.perf_counter()
            while True:
                fn()
                n += 1
                el = time.perf_counter() - t0
                if el >= min_s:
                    return el / n
        t_simd = timed(lambda: bqi.qgemm_w4a8_grouped_host(qa, da, ids, wq4, wd, threads))
        t_orc = timed(lambda: oracle.qgemm_w4a8_grouped(qa, da, ids, wq4, wd, nthreads=threads))
        res.append({"workload": "host W4A8 decode T=%d top-%d E=%d K=%d N=%d (%d active experts)"
                                % (T, m.top_k, m.experts, m.k, m.n, active),
                    "kernel": "qgemm_w4a8_grouped_host (AVX2 vpmaddubsw)",
                    "value": round(T / t_simd, 1), "unit": "tokens/s",
                    "ms_per_call": round(t_simd * 1e3, 3),
                    "weight_GB/s": round(wbytes / t_simd / 1e9, 2),
                    "cores": threads,
                    "oracle_ms_per_call": round(t_orc * 1e3, 3),
                    "speedup_vs_oracle": round(t_orc / t_simd, 2)})
    return res


def bench_combine(bqi, torch, W, iters):
    """MoE combine on the MoE workload's output shape (947 tokens x top-8 x
    768): an HBM stream; 12 rotated copies of y (280 MB) defeat the 256 MB
    Infinity Cache."""
    m = W.MOE
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    copies = 12
    ys = [torch.randn((m.tokens, m.top_k, m.n), generator=gen, device="cuda") for _ in range(copies)]
    p = torch.softmax(torch.randn((m.tokens, m.top_k), generator=gen, device="cuda"), dim=1)
    out = torch.empty((m.tokens, m.n), device="cuda")
    T = Timer(torch)
    mean = T.loop(lambda i: bqi.moe_combine_f32(ys[i % copies], p, out), iters, check=lambda: out)
    byt = 4 * (m.tokens * m.top_k * m.n + m.tokens * m.top_k + m.tokens * m.n)
    gbs = byt / (mean * 1e-3) / 1e9
    return {"workload": "MoE combine T=%d top-%d N=%d" % (m.tokens, m.top_k, m.n),
            "kernel": "k_moe_combine", "value": round(gbs, 1), "unit": "GB/s",
            "mean_launch_us": round(mean * 1e3, 2), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "hbm_bytes_algorithmic": byt, "y_copies_rotated": copies,
            "hbm_bytes_stored_counters": traffic("k_moe_combine moe")}


def bench_gguf(bqi, torch, W, iters):
    """GGUF import of the prefill weight matrix as Q8_0 (17408 x 5120) and of
    the MoE expert weights as Q4_0 (128 x 768 x 2048): byte shuffles at HBM
    rate; two rotated source copies each."""
    res = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for fmt, rows, k in (("q8_0", W.PREFILL.n, W.PREFILL.k),
                         ("q4_0", W.MOE.experts * W.MOE.n, W.MOE.k)):
        per = 34 if fmt == "q8_0" else 18
        nbytes = rows * (k // 32) * per
        srcs = [torch.randint(0, 256, (nbytes,), generator=gen, device="cuda", dtype=torch.uint8)
                for _ in range(2)]
        codes, scales = (bqi.gguf_q8_0_to_planar if fmt == "q8_0" else bqi.gguf_q4_0_to_planar)(
            srcs[0], rows, k)
        f = bqi.gguf_q8_0_to_planar if fmt == "q8_0" else bqi.gguf_q4_0_to_planar
        T = Timer(torch)
        mean = T.loop(lambda i: f(srcs[i % 2], rows, k, codes, scales), iters, check=lambda: codes)
        byt = 2 * nbytes
        gbs = byt / (mean * 1e-3) / 1e9
        res.append({"workload": "GGUF %s import %dx%d" % (fmt.upper(), rows, k),
                    "kernel": "k_gguf_split", "value": round(gbs, 1), "unit": "GB/s",
                    "mean_launch_us": round(mean * 1e3, 2),
                    "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "hbm_bytes_algorithmic": byt,
                    "hbm_bytes_stored_counters": traffic("k_gguf_split %s %dx%d" % (fmt, rows, k))})
        del srcs, codes, scales
        torch.cuda.empty_cache()
    return res


def cpu_info():
    """The host CPU model (first /proc/cpuinfo entry) and its thread counts."""
    model, logical = None, 0
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name") and model is None:
                    model = line.split(":", 1)[1].strip()
                elif line.startswith("processor"):
                    logical += 1
    except OSError:
        pass
    return {"model": model, "logical_cpus": logical, "usable_cpus": len(os.sched_getaffinity(0))}


def _timed(fn, seconds, min_runs=1):
    """(seconds per call, calls): fn repeated until `seconds` have passed."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if n >= min_runs and el >= seconds:
            return el / n, n


def cpu_baseline(W, step_bytes, seconds):
    """The CPU oracle (test infrastructure, plain C) on the same decode step:
    quantize the activation row, then the full GEMV."""
    import oracle
    s = W.DECODE[0]
    threads = oracle.default_threads()
    w = W.weights("decode", s.n, s.k)
    qw, dw = oracle.quantize_q8_0(w)
    x = W.activations("decode", s.m, s.k)

    def step(nt):
        qa, da = oracle.quantize_q8_0(x)
        oracle.qgemm_q8_0(qa, da, qw, dw, nthreads=nt)
    per, n = _timed(lambda: step(threads), seconds)
    used = min(threads, s.m)  # the oracle splits its work by output row
    cpu = cpu_info()
    return {"value": round(step_bytes / per / 1e9, 3), "unit": "GB/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu["model"], "host_logical_cpus": cpu["logical_cpus"],
            "sample": "%d full decode steps (quantize 1x4096 + GEMV 12288x4096), %.4f s each; "
                      "the oracle splits the GEMV over output rows, so a single-row step runs on "
                      "one thread" % (n, per)}


def cpu_oracle_lines(W, time_scale=1.0):
    """The CPU oracle (plain C, threads over output rows) timed on each secondary
    configuration, in the unit of that configuration's GPU line where the
    sample allows it.  Large GEMMs are timed on a sample of their activation
    rows against all weight rows (the oracle's cost is linear in the rows);
    about 2 s of oracle work each.  Keyed by the GPU line's workload name."""
    import oracle
    threads = oracle.default_threads()
    out = {}

    def rec(value, unit, sample, rows, **kw):
        # the oracle splits its work by output row: min(threads, rows) threads
        d = {"value": value, "unit": unit, "cores": min(threads, rows), "kind": "oracle",
             "sample": sample}
        d.update(kw)
        return d

    # small GEMM, whole call (quantize + GEMM), all threads and one thread
    s = W.SMALL
    x = W.activations("small", s.m, s.k)
    qw, dw = oracle.quantize_q8_0(W.weights("small", s.n, s.k))

    def small(nt):
        qa, da = oracle.quantize_q8_0(x)
        oracle.qgemm_q8_0(qa, da, qw, dw, nthreads=nt)
    per, n = _timed(lambda: small(threads), 1.0 * time_scale)
    per1, n1 = _timed(lambda: small(1), 1.0 * time_scale)
    out[name_small(s)] = rec(
        round(per * 1e6, 2), "us per call (quantize + GEMM)", "%d whole calls" % n, s.m,
        single_thread={"value": round(per1 * 1e6, 2), "unit": "us per call",
                       "sample": "%d whole calls on 1 thread" % n1})

    # decode M = 4, 16 (whole steps; bytes as in the GPU lines)
    s1 = W.DECODE[0]
    qw, dw = oracle.quantize_q8_0(W.weights("decode", s1.n, s1.k))
    for sd in W.DECODE[1:]:
        x = W.activations("decode", sd.m, sd.k)

        def dstep():
            qa, da = oracle.quantize_q8_0(x)
            oracle.qgemm_q8_0(qa, da, qw, dw, nthreads=threads)
        per, n = _timed(dstep, 2.0 * time_scale)
        a_bytes = sd.m * sd.k + sd.m * (sd.k // 32) * 2
        byt = sd.n * sd.k + sd.n * (sd.k // 32) * 2 + a_bytes + sd.m * sd.n * 4 + sd.m * sd.k * 4 + a_bytes
        out[name_decode(sd)] = rec(
            round(byt / per / 1e9, 3), "GB/s", "%d whole steps, %.4f s each" % (n, per), sd.m)
    del qw, dw

    # prefill, short prefill and long prefill: sampled activation rows
    for name, shape, rows in (("prefill", W.PREFILL, 32), ("prefill_short", W.PREFILL_SHORT, 32),
                              ("long", W.LONG, 96)):
        wl = "prefill" if name == "prefill_short" else name
        if name != "prefill_short":
            qw, dw = oracle.quantize_q8_0(W.weights(wl, shape.n, shape.k))
        x = W.activations(wl, rows, shape.k)

        def gstep():
            qa, da = oracle.quantize_q8_0(x)
            oracle.qgemm_q8_0(qa, da, qw, dw, nthreads=threads)
        per, n = _timed(gstep, 1.5 * time_scale)
        tops = 2.0 * rows * shape.n * shape.k / per / 1e12
        out[name_gemm(name, shape)] = rec(
            round(tops, 5), "int8-equiv TOPS",
            "%d of %d activation rows against all %d weight rows (quantize + GEMM), %d runs of "
            "%.3f s; the whole GEMM would take about %.1f s" % (rows, shape.m, shape.n, n, per,
                                                              per * shape.m / rows), rows)
    del qw, dw

    # grouped W4A8: a sample of tokens with their top-8 routes
    m = W.MOE
    wq4, wd = W.random_w4_codes(m.experts, m.n, m.k)
    ids = W.topk_ids(m.tokens, m.top_k, m.experts)
    tok = 96
    qa, da = oracle.quantize_q8_0(W.activations("moe", tok, m.k))
    per, n = _timed(lambda: oracle.qgemm_w4a8_grouped(qa, da, ids[:tok], wq4, wd, nthreads=threads),
                    1.5 * time_scale)
    out[name_moe(m)] = rec(
        round(2.0 * tok * m.top_k * m.n * m.k / per / 1e12, 5), "int8-equiv TOPS",
        "%d of %d tokens (%d routed rows), %d runs of %.3f s; the whole call would take about "
        "%.1f s" % (tok, m.tokens, tok * m.top_k, n, per, per * m.tokens / tok), tok * m.top_k)

    # grouped W4A8 decode, whole calls; bytes as in the GPU lines
    for T in (1, 4, 16):
        ids_t = W.topk_ids(T, m.top_k, m.experts, seed=T)
        qa, da = oracle.quantize_q8_0(W.activations("moe", T, m.k, seed=T))
        per, n = _timed(lambda: oracle.qgemm_w4a8_grouped(qa, da, ids_t, wq4, wd, nthreads=threads),
                        0.5 * time_scale)
        active = len(np.unique(ids_t))
        R = T * m.top_k
        byt = (active * m.n * (m.k // 2 + m.k // 32 * 2) + T * (m.k + m.k // 32 * 2)
               + R * 4 + R * m.n * 4)
        out[name_moe_decode(m, T, active)] = rec(
            round(byt / per / 1e9, 3), "GB/s", "%d whole calls, %.4f s each" % (n, per), R)
    del wq4, wd
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    import block_quantized_integer_amd as bqi
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bqi.lib()
    wl = set(args.workloads.split(","))
    res, ctx = None, None
    if "copy" in wl:
        bench_copy(torch)
    if "decode" in wl:
        res, ctx = bench_headline(bqi, torch, W, args)
        log("headline: %.1f GB/s per step (%.2f us, %.1f%% of HBM peak); two calls %.2f us; "
            "GEMV alone %.2f us (%.1f%%)" % (
                res["value"], res["roofline"]["mean_launch_us"], 100 * res["roofline"]["frac"],
                res["two_call_step"]["ms_per_step"] * 1e3, res["gemv_only"]["mean_launch_us"],
                100 * res["gemv_only"]["frac_hbm_peak"]))
        del ctx["wq"], ctx["wd"]
        torch.cuda.empty_cache()
    also = []
    if not args.only_headline:
        if "small" in wl:
            also.append(bench_small(bqi, torch, W, 200))
            log(json.dumps(also[-1]))
        if "decode_m" in wl:
            for r in bench_decode_variants(bqi, torch, W, 200):
                also.append(r)
                log(json.dumps(r))
            torch.cuda.empty_cache()
        for name in ("prefill", "prefill_short", "long"):
            if name in wl:
                also.append(bench_gemm(bqi, torch, W, name, 20))
                log(json.dumps(also[-1]))
                torch.cuda.empty_cache()
        if "moe" in wl:
            also.append(bench_moe(bqi, torch, W, 50))
            log(json.dumps(also[-1]))
            torch.cuda.empty_cache()
        if "moe_decode" in wl:
            for r in bench_moe_decode(bqi, torch, W, 400):
                also.append(r)
                log(json.dumps(r))
            torch.cuda.empty_cache()
        if "combine" in wl:
            also.append(bench_combine(bqi, torch, W, 400))
            log(json.dumps(also[-1]))
            torch.cuda.empty_cache()
        if "gguf" in wl:
            for r in bench_gguf(bqi, torch, W, 60):
                also.append(r)
                log(json.dumps(r))
        if "host" in wl:
            for r in bench_host_w4a8(bqi, W):
                also.append(r)
                log(json.dumps(r))
    if res is None:
        return
    if not args.no_cpu:
        log("cpu baseline (~%.0f s)" % args.cpu_seconds)
        res["cpu_baseline"] = cpu_baseline(W, ctx["step_bytes"], args.cpu_seconds)
        if also:
            log("cpu oracle on the other configurations")
            legs = cpu_oracle_lines(W)
            for r in also:
                if r.get("workload") in legs:
                    r["cpu_oracle"] = legs[r["workload"]]
    if also:
        res["also"] = also
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
