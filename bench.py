"""Benchmark: one NVFP4 training step of a Llama-3-8B-shaped MLP on one MI355X.

A step is one pass of the whole hot path over 32768 tokens (seq 8192 x
batch 4, the benchmark shape of the readjensen.com NVFP4 training-recipe page,
benchmark paragraph), with the recipe of that page's recipe paragraph:

  fprop   quantize X (1x16 RNE), W_gu and W_down (16x16 RNE)
          H = X W_gu^T                     32768 x 28672 x 4096
          Act = silu(gate) * up  (BF16), fused with both amaxes of Act
          quantize Act (1x16 RNE)
          Y = Act W_down^T                 32768 x 4096 x 14336
  bwd     dY, dH synthetic (Student-t(3) x 1e-3)
          down:    dAct = dY W_down        32768 x 14336 x 4096   (dY 1x16 SR)
                   dW_down = dY^T Act      4096 x 14336 x 32768   (RHT16 + SR / RHT16)
          gate/up: dX = dH W_gu            32768 x 4096 x 28672   (dH 1x16 SR)
                   dW_gu = dH^T X          28672 x 4096 x 32768   (RHT16 + SR / RHT16)

Every GEMM runs K-major x K-major (the NT kernel): the operands that are
contracted over their rows (the weights in dgrad, both wgrad inputs) are
quantized with transposed output, i.e. stored as the K-major tensors W^T,
dY^T, Act^T, dH^T, X^T.  The transposed weights reuse the amax of the
untransposed call; X, Act, dY and dH get both of their tensor amaxes (plain,
and of the column RHT) from one read (nvfp4_amax).

Inputs are resident in HBM before timing starts.  The JSON line reports the
step's NVFP4 GEMM throughput (GEMM FLOPs / step time), per-kernel HIP-event
timings, the roofline of the dominant GEMM kernel and the CPU oracle's
throughput on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense FP16/BF16 MFMA
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=64)
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a plain 1 GiB copy kernel (for HBM counter calibration)")
    ap.add_argument("--step-only", action="store_true",
                    help="the training-step line without the decode and mxfp4 objects "
                         "(for profiling the step's kernels alone)")
    ap.add_argument("--mx-only", action="store_true",
                    help="time only the MXFP4 comparison path and print its JSON object")
    ap.add_argument("--kv-only", action="store_true",
                    help="print only the NVFP4 KV-cache write/read object")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode-shape GEMMs and print their JSON object "
                         "(for profiling the skinny kernel; not the bench line)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_llama8b.json")
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_bit_microscaled_amd", "csrc", "gemm.hip")


def gemm_traffic():
    """Average HBM bytes per launch of the GEMM kernel over the step's six
    launches, from the committed rocprofv3 counter summary, or None when it is
    missing or was taken on a different GEMM source."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(GEMM_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    """HIP events around each library call on the current stream, grouped by kind."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.enabled = False

    def run(self, kind, fn, *a, name=None, **kw):
        if not self.enabled:
            return fn(*a, **kw)
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*a, **kw)
        e1.record()
        self.pending.append((kind, name, e0, e1))
        return r

    def totals(self, by_name=False):
        out = {}
        for kind, name, e0, e1 in self.pending:
            key = name if by_name else kind
            if key is None:
                continue
            t, n = out.get(key, (0.0, 0))
            out[key] = (t + e0.elapsed_time(e1), n + 1)
        return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import torch.nn.functional as F

    import nvfp4_bit_microscaled_amd as nv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode_only:
        print(json.dumps({"decode": decode_bench(torch, nv, workloads)}), flush=True)
        return
    if args.kv_only:
        print(json.dumps({"kv_cache": kv_bench(torch, nv, workloads)}), flush=True)
        return
    if args.mx_only:
        cfg = workloads.LLAMA8B
        X = workloads.activations(cfg["tokens"], cfg["hidden"], cfg["x_seed"], device="cuda")
        W_gu = workloads.weights(2 * cfg["ffn"], cfg["hidden"], cfg["wgu_seed"], device="cuda")
        print(json.dumps({"mxfp4": mxfp4_bench(torch, nv, X, W_gu)}), flush=True)
        return
    cfg = workloads.LLAMA8B
    T, D, Fh = cfg["tokens"], cfg["hidden"], cfg["ffn"]
    mask = workloads.sign_mask(cfg["mask_seed"])
    sr_seed = cfg["sr_seed"]

    print("generating inputs on the GPU", file=sys.stderr, flush=True)
    X = workloads.activations(T, D, cfg["x_seed"], device="cuda")
    W_gu = workloads.weights(2 * Fh, D, cfg["wgu_seed"], device="cuda")
    W_down = workloads.weights(D, Fh, cfg["wdown_seed"], device="cuda")
    dY = workloads.gradients(T, D, cfg["dy_seed"], device="cuda")
    dH = workloads.gradients(T, 2 * Fh, cfg["dh_seed"], device="cuda")
    torch.cuda.synchronize()

    timer = Timer(torch)
    gemm_flops = {}   # (name) -> flops per call
    qbytes = {}       # (name) -> algorithmic HBM bytes per call
    swbytes = {}      # the fused SwiGLU + amax pass

    def qb(rows, cols, in_bytes=2, amax_pass=True):
        # read input (twice when the amax pass runs) + codes + scales
        return rows * cols * (in_bytes * (2 if amax_pass else 1) + 0.5 + 1 / 16)

    def Q(name, x, **kw):
        qbytes[name] = qb(*x.shape, amax_pass=kw.get("amax_in") is None)
        return timer.run("quantize", nv.quantize, x, name=name, **kw)

    def AMX(name, x):
        # max |x| and max |RHT16 down the columns of x| in one read
        qbytes[name] = x.shape[0] * x.shape[1] * 2
        return timer.run("quantize", nv.amax, x, rht_mask=mask, name=name)

    def SWIGLU(name, h):
        # act = silu(gate) * up with both amaxes of act: reads H, writes act
        swbytes[name] = h.shape[0] * h.shape[1] * 2 + h.shape[0] * (h.shape[1] // 2) * 2
        return timer.run("swiglu", nv.swiglu_amax, h, mask, out=buf("Act", (h.shape[0], h.shape[1] // 2)))

    def G(name, role, a, b, M, N, K, out=None):
        gemm_flops[name] = 2.0 * M * N * K
        return timer.run("gemm_" + role, nv.gemm, "NT", a, b, out_dtype=torch.bfloat16,
                         out=out)

    bufs = {}

    def buf(name, shape):
        t = bufs.get(name)
        if t is None:
            t = bufs[name] = torch.empty(*shape, dtype=torch.bfloat16, device=dev)
        return t

    # A second stream (default priority) takes the HBM-bound quantizations of
    # each phase while the main stream runs the VALU-bound ones; the streams
    # meet before every GEMM, so GEMMs always run alone.  side waits for the
    # main stream at each fork, so memory the caching allocator hands out
    # again is never reused while the other stream may still read it.
    side = torch.cuda.Stream(device=dev)

    def fork():
        e = torch.cuda.Event()
        e.record(torch.cuda.current_stream())
        side.wait_event(e)

    def join():
        e = torch.cuda.Event()
        e.record(side)
        torch.cuda.current_stream().wait_event(e)

    def step():
        # ---- fprop: weights on the side stream, X on the main one
        fork()
        with torch.cuda.stream(side):
            wgu = Q("Wgu_2d", W_gu, block2d=True)
            wdn = Q("Wdown_2d", W_down, block2d=True)
        ax, axt = AMX("X_amax2", X)
        xq = Q("X_rows", X, amax_in=ax)
        join()
        H = G("fprop_gu", "fprop", xq, wgu, T, 2 * Fh, D, out=buf("H", (T, 2 * Fh)))
        act, aa, aat = SWIGLU("Act_swiglu_amax2", H)
        aq = Q("Act_rows", act, amax_in=aa)
        G("fprop_down", "fprop", aq, wdn, T, D, Fh, out=buf("Y", (T, D)))
        # ---- backward, down projection: both dY quantizations (stochastic
        # rounding, VALU-bound) beside W_down^T and Act^T (HBM-bound)
        ady, adyt = AMX("dY_amax2", dY)
        fork()
        with torch.cuda.stream(side):
            wdn_t = Q("Wdown_2d_T", W_down, block2d=True, transpose=True, amax_in=wdn.amax)
            at = Q("Act_cols_rht_T", act, axis=0, rht=True, mask=mask, transpose=True, amax_in=aat)
        dyq = Q("dY_rows_sr", dY, sr=True, seed=sr_seed, stream_id=0, amax_in=ady)
        dyt = Q("dY_cols_rht_sr_T", dY, axis=0, rht=True, mask=mask, sr=True, seed=sr_seed,
                stream_id=1, transpose=True, amax_in=adyt)
        join()
        G("dgrad_down", "dgrad", dyq, wdn_t, T, Fh, D, out=buf("dAct", (T, Fh)))
        G("wgrad_down", "wgrad", dyt, at, D, Fh, T, out=buf("dWdown", (D, Fh)))
        # ---- backward, gate/up projection: the same split
        adh, adht = AMX("dH_amax2", dH)
        fork()
        with torch.cuda.stream(side):
            wgu_t = Q("Wgu_2d_T", W_gu, block2d=True, transpose=True, amax_in=wgu.amax)
            xt = Q("X_cols_rht_T", X, axis=0, rht=True, mask=mask, transpose=True, amax_in=axt)
        dhq = Q("dH_rows_sr", dH, sr=True, seed=sr_seed, stream_id=0, amax_in=adh)
        dht = Q("dH_cols_rht_sr_T", dH, axis=0, rht=True, mask=mask, sr=True, seed=sr_seed,
                stream_id=1, transpose=True, amax_in=adht)
        join()
        G("dgrad_gu", "dgrad", dhq, wgu_t, T, D, 2 * Fh, out=buf("dX", (T, D)))
        G("wgrad_gu", "wgrad", dht, xt, 2 * Fh, D, T, out=buf("dWgu", (2 * Fh, D)))

    if args.calibration_copy:
        # a plain elementwise copy of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    print("warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, bracketed by synchronizations
    timer.enabled = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    totals = timer.totals()
    print("timed %d steps: %.3f ms/step (host wall %.3f s)" % (args.steps, ms_step, wall),
          file=sys.stderr, flush=True)

    flops_step = sum(gemm_flops.values())
    value = flops_step / (ms_step * 1e-3) / 1e12
    per_kind = {k: {"ms_per_step": t / args.steps, "calls_per_step": n / args.steps}
                for k, (t, n) in totals.items()}
    # the six GEMMs by role (all the NT kernel): flops and average launch time
    role_flops = {"fprop": gemm_flops["fprop_gu"] + gemm_flops["fprop_down"],
                  "dgrad": gemm_flops["dgrad_down"] + gemm_flops["dgrad_gu"],
                  "wgrad": gemm_flops["wgrad_down"] + gemm_flops["wgrad_gu"]}
    gemm_roles = {}
    for role, fl in role_flops.items():
        t, n = totals["gemm_" + role]
        gemm_roles[role] = {"tflops": fl * args.steps / (t * 1e-3) / 1e12,
                            "avg_launch_ms": t / n, "launches": n}
    # each quantize / amax call: time, algorithmic GB/s, and what bounds it
    # (the stochastic-rounding calls are bound by VALU work: Philox and the
    # exact SR selection; the others stream HBM)
    q_calls = {}
    for name, (t, n) in timer.totals(by_name=True).items():
        if name not in qbytes:
            continue
        q_calls[name] = {"us": round(t / n * 1e3, 1),
                         "GBps": round(qbytes[name] / (t / n * 1e-3) / 1e9, 1),
                         "bound": "valu" if "_sr" in name else "hbm"}
    q_bytes = sum(qbytes.values()) * args.steps
    gemm_t = sum(totals["gemm_" + k][0] for k in role_flops)
    # the quantize phases' wall time: the step outside the GEMMs and the
    # SwiGLU pass, which run alone on the main stream (the per-call times
    # overlap across the two streams, so their sum is not a duration)
    q_wall = ms_step * args.steps - gemm_t - totals["swiglu"][0]
    gemm_n = sum(totals["gemm_" + k][1] for k in role_flops)
    achieved = flops_step * args.steps / (gemm_t * 1e-3) / 1e12
    line = {
        "metric": "NVFP4 GEMM TFLOPS (8B MLP shapes) + quantize GB/s, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, f16 mfma, f32 accumulate",
        "data": "synthetic (seeded activations/weights/Student-t gradients, HBM-resident)",
        "config": {"workload": "llama3-8b-mlp-fwd+bwd-step", "tokens": T, "hidden": D,
                   "ffn": Fh, "gemm_tflop_per_step": round(flops_step / 1e12, 4),
                   "parallelism": "none (1 GPU)"},
        "gemm_only_tflops": round(achieved, 2),
        "gemm_by_role": {k: {kk: round(vv, 4) for kk, vv in v.items()}
                         for k, v in gemm_roles.items()},
        "quantize_GBps": round(q_bytes / (q_wall * 1e-3) / 1e9, 1),
        "quantize_frac_of_hbm": round(q_bytes / (q_wall * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "quantize_wall_ms_per_step": round(q_wall / args.steps, 4),
        "quantize_by_call": q_calls,
        "swiglu_GBps": round(sum(swbytes.values()) * args.steps / (totals["swiglu"][0] * 1e-3) / 1e9, 1),
        "time_breakdown_ms_per_step": {("quantize_calls_sum" if k == "quantize" else k):
                                       round(v["ms_per_step"], 4) for k, v in per_kind.items()},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_kk (K-major x K-major, all six MLP GEMMs)",
                     "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "avg_launch_ms": round(gemm_t / gemm_n, 4),
                     "traffic": gemm_traffic()},
    }
    del bufs
    torch.cuda.empty_cache()
    if not args.step_only:
        line["decode"] = decode_bench(torch, nv, workloads)
        line["mxfp4"] = mxfp4_bench(torch, nv, X, W_gu)
        line["kv_cache"] = kv_bench(torch, nv, workloads)
        line["dequantize_rht16"] = dequant_rht_bench(torch, nv, X, mask)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, torch, nv, workloads, X, W_gu)
    print(json.dumps(line), flush=True)


def dequant_rht_bench(torch, nv, X, mask, reps=20):
    """The two HBM streams outside the step: dequantize X's NVFP4 copy
    (32768 x 4096, 1x16) to BF16 and FP32, and the standalone RHT16 down X's
    columns (BF16 in, FP32 out). Mean of back-to-back calls, HIP events."""
    xq = nv.quantize(X)
    n = X.numel()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    out = {"shape": "%d x %d" % tuple(X.shape), "timing": "mean of %d back-to-back calls" % reps}
    for name, dt, ob in (("dequant_bf16", torch.bfloat16, 2), ("dequant_f32", torch.float32, 4)):
        us = timed(lambda: nv.dequantize(xq, dt))
        b = n * (0.5 + 1 / 16 + ob)
        out[name] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                     "frac_of_hbm": round(b / us / 1e3 / HBM_PEAK_GBPS, 4), "bytes": int(b)}
    us = timed(lambda: nv.rht16(X, axis=0, mask=mask))
    b = n * (2 + 4)
    out["rht16_cols"] = {"us": round(us, 2), "GBps": round(b / us / 1e3, 1),
                         "frac_of_hbm": round(b / us / 1e3 / HBM_PEAK_GBPS, 4), "bytes": int(b)}
    return out


def decode_bench(torch, nv, workloads):
    """Decode-style skinny NT GEMM: activations [M, 8192] x weights [28672, 8192],
    both 1x16 RNE.  HBM-bound on the packed weights (codes + scales).  Four
    copies of the quantized weights (4 x 132 MB, twice the 256 MB Infinity
    Cache) are cycled through 40 back-to-back launches, so every launch reads
    weights evicted by the three before it; `us` is the mean per launch.
    `us_isolated` is the median of 10 single launches, each after a 1 GiB read
    that evicts the cache (HIP events around one launch also count its
    dispatch)."""
    import dataclasses
    cfg = workloads.DECODE
    K, N = cfg["k"], cfg["n"]
    w0 = nv.quantize(workloads.weights(N, K, cfg["w_seed"], device="cuda"))
    ws = [w0] + [dataclasses.replace(w0, codes=w0.codes.clone(), scales=w0.scales.clone())
                 for _ in range(3)]
    x = workloads.activations(64, K, cfg["act_seed"], device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    wbytes = N * K * (0.5 + 1 / 16)
    out = {}
    for M in cfg["ms"]:
        a = nv.quantize(x[:M].contiguous())
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        for i in range(4):
            nv.gemm("NT", a, ws[i], out=y)
        reps = 40
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            nv.gemm("NT", a, ws[i % 4], out=y)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        iso = []
        for it in range(12):
            flush.sum()
            f0 = torch.cuda.Event(enable_timing=True)
            f1 = torch.cuda.Event(enable_timing=True)
            f0.record()
            nv.gemm("NT", a, w0, out=y)
            f1.record()
            torch.cuda.synchronize()
            if it >= 2:
                iso.append(f0.elapsed_time(f1))
        # the same weights with BF16 activations (weight-only GEMM)
        ab = x[:M].contiguous()
        for i in range(4):
            nv.gemm_w4a16(ab, ws[i], out=y)
        e0.record()
        for i in range(reps):
            nv.gemm_w4a16(ab, ws[i % 4], out=y)
        e1.record()
        torch.cuda.synchronize()
        t16 = e0.elapsed_time(e1) * 1e-3 / reps
        out["M%d" % M] = {"us": round(t * 1e6, 2),
                          "w4a16_us": round(t16 * 1e6, 2),
                          "weights_GBps": round(wbytes / t / 1e9, 1),
                          "frac_of_hbm": round(wbytes / t / 1e9 / HBM_PEAK_GBPS, 4),
                          "tflops": round(2.0 * M * N * K / t / 1e12, 2),
                          "us_isolated": round(sorted(iso)[len(iso) // 2] * 1e3, 2)}
    del flush
    return {"shape": "M x 28672 x 8192, weights 1x16 along K (w4a16_us: BF16 activations)",
            "weight_bytes": int(wbytes),
            "timing": "mean of 40 back-to-back launches over 4 weight copies (528 MB, "
                      "cache-cold each launch); us_isolated: median of 10 single launches "
                      "after a cache-evicting read", **out}


def mxfp4_bench(torch, nv, X, W):
    """The power-of-two-scaled MXFP4 format the pages compare NVFP4 with, on
    the step's first GEMM (X [32768, 4096] x W_gu [28672, 4096]^T): GEMM time
    on the native scaled FP4 MFMA against the same GEMM in NVFP4 (f16 MFMA),
    quantize bandwidth, and each format's mean squared error on X."""
    T, D = X.shape
    N = W.shape[0]
    reps = 5
    y = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        fn()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    xm, wm = nv.mx_quantize(X), nv.mx_quantize(W)
    t_q = timed(lambda: nv.mx_quantize(X, out=xm))
    t_mx = timed(lambda: nv.mx_gemm(xm, wm, out=y))
    xn, wn = nv.quantize(X), nv.quantize(W, block2d=True)
    t_nv = timed(lambda: nv.gemm("NT", xn, wn, out=y))
    del y
    fl = 2.0 * T * N * D
    xf = X.float()
    mse_mx = ((nv.mx_dequantize(xm, torch.float32) - xf) ** 2).mean().item()
    mse_nv = ((nv.dequantize(xn, torch.float32) - xf) ** 2).mean().item()
    qb = T * D * (2 + 0.5 + 1 / 32)
    return {"gemm": "%d x %d x %d NT, BF16 out" % (T, N, D),
            "kernel": "k_gemm_mx (v_mfma_scale_f32_32x32x64_f8f6f4, FP4 x FP4)",
            "mx_gemm_ms": round(t_mx, 4), "mx_gemm_tflops": round(fl / t_mx / 1e9, 1),
            "mx_frac_of_fp4_peak": round(fl / t_mx / 1e9 / MFMA_FP4_PEAK_TFLOPS, 4),
            "nvfp4_gemm_ms": round(t_nv, 4), "nvfp4_gemm_tflops": round(fl / t_nv / 1e9, 1),
            "mx_quantize_GBps": round(qb / (t_q * 1e-3) / 1e9, 1),
            "mse_on_X": {"mxfp4": mse_mx, "nvfp4": mse_nv,
                         "nvfp4_less_error": round(1 - mse_nv / mse_mx, 4)}}


def kv_bench(torch, nv, workloads):
    """NVFP4 KV cache of a Llama-3-8B-shaped model (8 KV heads x 128 = 1024
    features): 262144 BF16 token rows written in pages of 16 over a cache of
    262144 slots, and every slot gathered back (another page order) to BF16.
    Both are HBM streams; bytes per call are the algorithmic ones: the write
    reads 2 B per feature and the slot index and writes 0.5 + 1/16 B per
    feature, the read the reverse.  Mean of 10 back-to-back calls (537 MB of
    BF16 per call, twice the Infinity Cache)."""
    cfg = workloads.KVCACHE
    T, C, S = cfg["tokens"], cfg["cols"], cfg["num_slots"]
    x = workloads.activations(T, C, cfg["x_seed"], device="cuda")
    amax = x.float().abs().max().reshape(1)
    slots = workloads.paged_slots(T, S, cfg["slot_seed"]).cuda()
    rslots = workloads.paged_slots(S, S, cfg["read_seed"]).cuda()
    cache = nv.kv_cache_create(S, C, amax)
    out = torch.empty(S, C, dtype=torch.bfloat16, device="cuda")
    reps = 10
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        fn()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_w = timed(lambda: nv.kv_cache_write(cache, x, slots))
    t_r = timed(lambda: nv.kv_cache_read(cache, rslots, torch.bfloat16, out=out))
    wb = T * C * (2 + 0.5 + 1 / 16) + 8 * T
    rb = S * C * (0.5 + 1 / 16 + 2) + 8 * S
    del x, out, cache
    return {"shape": "%d tokens x %d features, cache of %d slots, pages of 16" % (T, C, S),
            "kernels": "k_kv_write<bf16>, k_kv_read<bf16 out>",
            "write_us": round(t_w * 1e6, 2), "write_GBps": round(wb / t_w / 1e9, 1),
            "write_frac_of_hbm": round(wb / t_w / 1e9 / HBM_PEAK_GBPS, 4),
            "read_us": round(t_r * 1e6, 2), "read_GBps": round(rb / t_r / 1e9, 1),
            "read_frac_of_hbm": round(rb / t_r / 1e9 / HBM_PEAK_GBPS, 4),
            "bytes_per_call": {"write": int(wb), "read": int(rb)}}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, torch, nv, workloads, X, W_gu):
    """The oracle, as it stands, on a bounded sample of the step: fprop GEMM 1
    for the first `rows` tokens (all 28672 outputs, full K = 4096)."""
    import numpy as np

    import oracle
    rows = args.cpu_sample_rows
    cores = len(os.sched_getaffinity(0))
    oracle.set_num_threads(cores)
    x = X[:rows].cpu()
    w = W_gu.cpu()
    t0 = time.perf_counter()
    xc, xs, xts, _ = oracle.quantize(workloads.bf16_bits(x),
                                     amax_in=float(X.abs().max().item()))
    wc, wsc, wts, _ = oracle.quantize(workloads.bf16_bits(w), block2d=True)
    tq = time.perf_counter() - t0
    N, K = w.shape
    ms, ns = np.meshgrid(np.arange(rows), np.arange(N), indexing="ij")
    t1 = time.perf_counter()
    oracle.gemm_pairs("NT", rows, N, K, (xc, xs, xts, False), (wc, wsc, wts, True), ms.ravel(),
                      ns.ravel())
    tg = time.perf_counter() - t1
    # the same on one thread, over rows / cores tokens (about the same wall time)
    rows1 = max(1, rows // cores)
    ms1, ns1 = np.meshgrid(np.arange(rows1), np.arange(N), indexing="ij")
    oracle.set_num_threads(1)
    t2 = time.perf_counter()
    oracle.gemm_pairs("NT", rows1, N, K, (xc, xs, xts, False), (wc, wsc, wts, True), ms1.ravel(),
                      ns1.ravel())
    t1s = time.perf_counter() - t2
    oracle.set_num_threads(cores)
    flops = 2.0 * rows * N * K
    flops1 = 2.0 * rows1 * N * K
    qbytes = (x.numel() + w.numel()) * (2 + 0.5 + 1 / 16) + w.numel() * 2
    return {"value": round(flops / tg / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "fprop GEMM 1 (NT, 2D-quantized W_gu) on the first %d tokens: "
                      "%d x %d x %d FP64 dot products (%.2f GFLOP) in %.1f s"
                      % (rows, rows, N, K, flops / 1e9, tg),
            "single_thread_value": round(flops1 / t1s / 1e12, 6),
            "single_thread_sample": "the same GEMM on the first %d tokens, one thread, %.1f s"
                                    % (rows1, t1s),
            "quantize_GBps": round(qbytes / tq / 1e9, 4),
            "quantize_sample": "X rows 0-%d (1x16 RNE) and W_gu (16x16 RNE, amax pass), %.1f s"
                               % (rows - 1, tq)}


if __name__ == "__main__":
    main()
