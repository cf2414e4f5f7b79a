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
contracted over their rows are stored as the K-major tensors W^T, dY^T,
Act^T, dH^T, X^T.  The wgrad inputs are quantized with transposed output; the
16x16-block weights are transpose-consistent, so W^T is W's own quantization
with its codes and scales transposed (nvfp4_transpose), not a second
quantization.  X, Act, dY and dH get both of their tensor amaxes (plain, and
of the column RHT) from one read (nvfp4_amax).

Inputs are resident in HBM before timing starts.  The JSON line reports the
step's NVFP4 GEMM throughput (GEMM FLOPs / step time), per-kernel HIP-event
timings (inside the step and alone), the roofline of the dominant GEMM kernel
and the CPU oracle's throughput on bounded samples of the same work.  Beside
it (unless --step-only): the decode GEMMs, the MXFP4 comparison, the KV cache,
dequantize/RHT16, and the same step at one GPU's token share of a
Llama-3.1-405B MLP (8192 tokens, hidden 16384, intermediate 53248).
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
    ap.add_argument("--quant-only", action="store_true",
                    help="one untimed step, then only the isolated replay of its quantize, "
                         "amax, transpose and SwiGLU calls (for per-kernel counters); prints "
                         "the calls in replay order with their times")
    ap.add_argument("--c5-only", action="store_true",
                    help="print only the Llama-3.1-405B token-share step object (for "
                         "profiling its kernels)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode-shape GEMMs and print their JSON object "
                         "(for profiling the decode kernels; not the bench line)")
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
        self.recorded = None   # list: named calls of one step, kept for the isolated replay

    def run(self, kind, fn, *a, name=None, **kw):
        if self.recorded is not None and name is not None:
            self.recorded.append((kind, name, fn, a, kw))
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
    if args.c5_only:
        print(json.dumps({"llama405b_share": c5_bench(torch, nv, workloads, dev)}), flush=True)
        return

    print("generating inputs on the GPU", file=sys.stderr, flush=True)
    ms = MlpStep(torch, nv, workloads, workloads.LLAMA8B, dev)
    if args.calibration_copy:
        # a plain elementwise copy of known size: reads 1 GiB, writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.quant_only:
        ms.step()
        torch.cuda.synchronize()
        calls = ms.record_calls()
        iso = isolated_times(torch, calls, dev, reps=3)
        print(json.dumps({"quant_only": {
            "replay": "each call once untimed, then a 1 GiB cache-evicting read, then 3 "
                      "times back to back (timed), in this order",
            "order": [name for _, name, _, _, _ in calls],
            "isolated_us": {k: round(v, 2) for k, v in iso.items()},
            "bytes": {k: int(v) for k, v in ms.qbytes.items()}}}), flush=True)
        return

    print("warmup", file=sys.stderr, flush=True)
    r = run_step_bench(torch, ms, args.steps, args.warmup, dev, isolated=True)
    print("timed %d steps: %.3f ms/step (host wall %.3f s)" % (args.steps, r["ms_per_step"],
                                                             r["host_wall_s"]),
          file=sys.stderr, flush=True)
    cfg = workloads.LLAMA8B
    line = {
        "metric": "NVFP4 GEMM TFLOPS (8B MLP shapes) + quantize GB/s, % of MI355X roofline",
        "value": round(r["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, f16 mfma, f32 accumulate",
        "data": "synthetic (seeded activations/weights/Student-t gradients, HBM-resident)",
        "config": {"workload": "llama3-8b-mlp-fwd+bwd-step", "tokens": cfg["tokens"],
                   "hidden": cfg["hidden"], "ffn": cfg["ffn"],
                   "gemm_tflop_per_step": round(r["flops_step"] / 1e12, 4),
                   "parallelism": "none (1 GPU)"},
    }
    line.update(r["report"])
    line["roofline"] = {"bound": "mfma",
                        "kernel": "k_gemm_kk (K-major x K-major, all six MLP GEMMs)",
                        "achieved": round(r["gemm_tflops"], 2), "peak": MFMA_F16_PEAK_TFLOPS,
                        "unit": "TFLOP/s",
                        "frac": round(r["gemm_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                        "avg_launch_ms": round(r["gemm_avg_launch_ms"], 4),
                        "traffic": gemm_traffic()}
    X, W_gu, mask = ms.X, ms.W_gu, ms.mask
    ms.free_buffers()
    torch.cuda.empty_cache()
    if not args.step_only:
        # the decode shapes are a workload of their own: measured after the
        # GPU has idled out of the training step's power transient (right
        # after a 20 s GEMM load they ran 1-2 us slower, 3 s later as cold)
        time.sleep(3.0)
        line["decode"] = decode_bench(torch, nv, workloads)
        line["mxfp4"] = mxfp4_bench(torch, nv, X, W_gu)
        line["kv_cache"] = kv_bench(torch, nv, workloads)
        line["dequantize_rht16"] = dequant_rht_bench(torch, nv, X, mask)
        del ms
        torch.cuda.empty_cache()
        line["llama405b_share"] = c5_bench(torch, nv, workloads, dev)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, torch, nv, workloads, X, W_gu)
    print(json.dumps(line), flush=True)


class MlpStep:
    """One NVFP4 MLP training step (fprop, dgrad, wgrad of both projections)
    over seeded synthetic inputs resident in HBM, with every library call
    named and timed through a Timer.  cfg: tokens, hidden, ffn and seeds
    (workloads.LLAMA8B or workloads.LLAMA405B)."""

    def __init__(self, torch, nv, workloads, cfg, dev):
        self.torch, self.nv, self.cfg, self.dev = torch, nv, cfg, dev
        T, D, Fh = cfg["tokens"], cfg["hidden"], cfg["ffn"]
        self.T, self.D, self.Fh = T, D, Fh
        self.mask = workloads.sign_mask(cfg["mask_seed"])
        self.sr_seed = cfg["sr_seed"]
        self.X = workloads.activations(T, D, cfg["x_seed"], device="cuda")
        self.W_gu = workloads.weights(2 * Fh, D, cfg["wgu_seed"], device="cuda")
        self.W_down = workloads.weights(D, Fh, cfg["wdown_seed"], device="cuda")
        self.dY = workloads.gradients(T, D, cfg["dy_seed"], device="cuda")
        self.dH = workloads.gradients(T, 2 * Fh, cfg["dh_seed"], device="cuda")
        torch.cuda.synchronize()
        self.timer = Timer(torch)
        self.gemm_flops = {}   # name -> flops per call
        self.qbytes = {}       # name -> algorithmic HBM bytes per call
        self.swbytes = {}      # the fused SwiGLU + amax pass
        self.bufs = {}
        # A second stream (default priority) takes the HBM-bound quantizations
        # of each phase while the main stream runs the VALU-bound ones; the
        # streams meet before every GEMM, so GEMMs always run alone.  side
        # waits for the main stream at each fork, so memory the caching
        # allocator hands out again is never reused while the other stream
        # may still read it.
        self.side = torch.cuda.Stream(device=dev)

    # ---- named library calls (bytes / flops recorded per call)
    @staticmethod
    def qb(rows, cols, in_bytes=2, amax_pass=True, block2d=False):
        # read input (twice when the amax pass runs) + codes + scales (one
        # byte per 16 elements in 1x16 blocks, per 256 in 16x16 blocks)
        return rows * cols * (in_bytes * (2 if amax_pass else 1) + 0.5
                              + (1 / 256 if block2d else 1 / 16))

    def Q(self, name, x, **kw):
        self.qbytes[name] = self.qb(*x.shape, amax_pass=kw.get("amax_in") is None,
                                    block2d=kw.get("block2d", False))
        return self.timer.run("quantize", self.nv.quantize, x, name=name, **kw)

    def TR(self, name, q):
        # storage transpose of a 16x16-block operand: codes and scales read
        # and written once
        self.qbytes[name] = q.rows * q.cols * 2 * (0.5 + 1 / 256)
        return self.timer.run("quantize", self.nv.transpose, q, name=name)

    def AMX(self, name, x):
        # max |x| and max |RHT16 down the columns of x| in one read
        self.qbytes[name] = x.shape[0] * x.shape[1] * 2
        return self.timer.run("quantize", self.nv.amax, x, rht_mask=self.mask, name=name)

    def SWIGLU(self, name, h):
        # act = silu(gate) * up with both amaxes of act: reads H, writes act
        self.swbytes[name] = h.shape[0] * h.shape[1] * 2 + h.shape[0] * (h.shape[1] // 2) * 2
        return self.timer.run("swiglu", self.nv.swiglu_amax, h, self.mask, name=name,
                              out=self.buf("Act", (h.shape[0], h.shape[1] // 2)))

    def G(self, name, role, a, b, M, N, K, out=None):
        self.gemm_flops[name] = 2.0 * M * N * K
        return self.timer.run("gemm_" + role, self.nv.gemm, "NT", a, b,
                              out_dtype=self.torch.bfloat16, out=out)

    def buf(self, name, shape):
        t = self.bufs.get(name)
        if t is None:
            t = self.bufs[name] = self.torch.empty(*shape, dtype=self.torch.bfloat16,
                                                   device=self.dev)
        return t

    def free_buffers(self):
        self.bufs = {}

    def fork(self):
        e = self.torch.cuda.Event()
        e.record(self.torch.cuda.current_stream())
        self.side.wait_event(e)

    def join(self):
        e = self.torch.cuda.Event()
        e.record(self.side)
        self.torch.cuda.current_stream().wait_event(e)

    def step(self):
        torch, T, D, Fh, mask, sr_seed = self.torch, self.T, self.D, self.Fh, self.mask, self.sr_seed
        Q, TR, AMX, G, buf = self.Q, self.TR, self.AMX, self.G, self.buf
        X, W_gu, W_down, dY, dH = self.X, self.W_gu, self.W_down, self.dY, self.dH
        # ---- fprop: weights on the side stream, X on the main one
        self.fork()
        with torch.cuda.stream(self.side):
            wgu = Q("Wgu_2d", W_gu, block2d=True)
            wdn = Q("Wdown_2d", W_down, block2d=True)
        ax, axt = AMX("X_amax2", X)
        xq = Q("X_rows", X, amax_in=ax)
        self.join()
        H = G("fprop_gu", "fprop", xq, wgu, T, 2 * Fh, D, out=buf("H", (T, 2 * Fh)))
        act, aa, aat = self.SWIGLU("Act_swiglu_amax2", H)
        aq = Q("Act_rows", act, amax_in=aa)
        G("fprop_down", "fprop", aq, wdn, T, D, Fh, out=buf("Y", (T, D)))
        # ---- backward, down projection: both dY quantizations (stochastic
        # rounding, VALU-bound) beside W_down^T and Act^T
        ady, adyt = AMX("dY_amax2", dY)
        self.fork()
        with torch.cuda.stream(self.side):
            wdn_t = TR("Wdown_2d_T", wdn)
            at = Q("Act_cols_rht_T", act, axis=0, rht=True, mask=mask, transpose=True,
                   amax_in=aat)
        dyq = Q("dY_rows_sr", dY, sr=True, seed=sr_seed, stream_id=0, amax_in=ady)
        dyt = Q("dY_cols_rht_sr_T", dY, axis=0, rht=True, mask=mask, sr=True, seed=sr_seed,
                stream_id=1, transpose=True, amax_in=adyt)
        self.join()
        G("dgrad_down", "dgrad", dyq, wdn_t, T, Fh, D, out=buf("dAct", (T, Fh)))
        G("wgrad_down", "wgrad", dyt, at, D, Fh, T, out=buf("dWdown", (D, Fh)))
        # ---- backward, gate/up projection: the same split
        adh, adht = AMX("dH_amax2", dH)
        self.fork()
        with torch.cuda.stream(self.side):
            wgu_t = TR("Wgu_2d_T", wgu)
            xt = Q("X_cols_rht_T", X, axis=0, rht=True, mask=mask, transpose=True, amax_in=axt)
        dhq = Q("dH_rows_sr", dH, sr=True, seed=sr_seed, stream_id=0, amax_in=adh)
        dht = Q("dH_cols_rht_sr_T", dH, axis=0, rht=True, mask=mask, sr=True, seed=sr_seed,
                stream_id=1, transpose=True, amax_in=adht)
        self.join()
        G("dgrad_gu", "dgrad", dhq, wgu_t, T, D, 2 * Fh, out=buf("dX", (T, D)))
        G("wgrad_gu", "wgrad", dht, xt, 2 * Fh, D, T, out=buf("dWgu", (2 * Fh, D)))

    def record_calls(self):
        """Run one step untimed and return its named non-GEMM calls."""
        self.timer.enabled = False
        self.timer.recorded = []
        self.step()
        self.torch.cuda.synchronize()
        calls = self.timer.recorded
        self.timer.recorded = None
        return calls


def run_step_bench(torch, ms, steps, warmup, dev, isolated=True):
    """Warm up, time `steps` steps between two synchronizations, then (when
    `isolated`) replay every quantize, amax, transpose and SwiGLU call of one
    more step alone: the per-kernel times the two-stream step cannot give."""
    for _ in range(warmup):
        ms.step()
    torch.cuda.synchronize()
    timer = ms.timer
    timer.pending = []
    timer.enabled = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        ms.step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / steps
    timer.enabled = False
    totals = timer.totals()
    by_name = timer.totals(by_name=True)
    iso = isolated_times(torch, ms.record_calls(), dev) if isolated else None

    gemm_flops, qbytes, swbytes = ms.gemm_flops, ms.qbytes, ms.swbytes
    flops_step = sum(gemm_flops.values())
    role_flops = {"fprop": gemm_flops["fprop_gu"] + gemm_flops["fprop_down"],
                  "dgrad": gemm_flops["dgrad_down"] + gemm_flops["dgrad_gu"],
                  "wgrad": gemm_flops["wgrad_down"] + gemm_flops["wgrad_gu"]}
    gemm_roles = {}
    for role, fl in role_flops.items():
        t, n = totals["gemm_" + role]
        gemm_roles[role] = {"tflops": round(fl * steps / (t * 1e-3) / 1e12, 2),
                            "avg_launch_ms": round(t / n, 4), "launches": n}
    # each quantize / amax / transpose call: its time inside the step, its
    # time alone, its algorithmic bytes and (from the committed counter
    # summary, while it matches the source) what bounds it
    q_calls = {}
    counters = quantize_counters()
    for name, (t, n) in by_name.items():
        if name not in qbytes:
            continue
        c = {"us_in_step": round(t / n * 1e3, 1), "bytes": int(qbytes[name])}
        if iso is not None:
            it = iso[name]
            c.update({"isolated_us": round(it, 1),
                      "isolated_GBps": round(qbytes[name] / (it * 1e-6) / 1e9, 1),
                      "isolated_frac_of_hbm": round(qbytes[name] / (it * 1e-6) / 1e9
                                                    / HBM_PEAK_GBPS, 4)})
        if counters is not None and name in counters:
            c["bound"] = counters[name].get("bound")
            c["counters"] = counters[name]
        q_calls[name] = c
    q_bytes = sum(qbytes.values()) * steps
    gemm_t = sum(totals["gemm_" + k][0] for k in role_flops)
    gemm_n = sum(totals["gemm_" + k][1] for k in role_flops)
    # the quantize phases' wall time: the step outside the GEMMs and the
    # SwiGLU pass, which run alone on the main stream (the per-call times
    # overlap across the two streams, so their sum is not a duration)
    q_wall = ms_step * steps - gemm_t - totals["swiglu"][0]
    achieved = flops_step * steps / (gemm_t * 1e-3) / 1e12
    report = {
        "gemm_only_tflops": round(achieved, 2),
        "gemm_by_role": gemm_roles,
        "quantize_GBps": round(q_bytes / (q_wall * 1e-3) / 1e9, 1),
        "quantize_frac_of_hbm": round(q_bytes / (q_wall * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "quantize_wall_ms_per_step": round(q_wall / steps, 4),
    }
    if iso is not None:
        q_iso = sum(iso[k] for k in qbytes)
        report.update({
            "quantize_isolated_GBps": round(sum(qbytes.values()) / (q_iso * 1e-6) / 1e9, 1),
            "quantize_isolated_frac_of_hbm": round(sum(qbytes.values()) / (q_iso * 1e-6) / 1e9
                                                   / HBM_PEAK_GBPS, 4),
            "quantize_isolated_ms_per_step": round(q_iso / 1e3, 4),
            "swiglu_isolated_us": round(iso["Act_swiglu_amax2"], 1)})
    report.update({
        "quantize_by_call": q_calls,
        "swiglu_GBps": round(sum(swbytes.values()) * steps / (totals["swiglu"][0] * 1e-3)
                             / 1e9, 1),
        "time_breakdown_ms_per_step": {("quantize_calls_sum" if k == "quantize" else k):
                                       round(t / steps, 4) for k, (t, n) in totals.items()},
    })
    return {"ms_per_step": ms_step, "host_wall_s": wall, "flops_step": flops_step,
            "tflops_step": flops_step / (ms_step * 1e-3) / 1e12, "gemm_tflops": achieved,
            "gemm_avg_launch_ms": gemm_t / gemm_n, "report": report}


def c5_bench(torch, nv, workloads, dev, steps=3, warmup=1):
    """The same fwd+bwd step at one GPU's token share of a Llama-3.1-405B MLP
    (8192 tokens, hidden 16384, intermediate 53248): the benchmark paragraph
    of the readjensen.com NVFP4 training-recipe page, where the pages report
    the largest gain.  Two of its GEMMs have K above one FP32 accumulation
    chain (dgrad gate+up 106496, fprop down 53248) and run as K slices."""
    cfg = workloads.LLAMA405B
    ms = MlpStep(torch, nv, workloads, cfg, dev)
    r = run_step_bench(torch, ms, steps, warmup, dev, isolated=False)
    out = {"workload": "llama3.1-405b-mlp-fwd+bwd-step, one GPU's token share",
           "tokens": cfg["tokens"], "hidden": cfg["hidden"], "ffn": cfg["ffn"],
           "steps": steps, "warmup": warmup,
           "ms_per_step": round(r["ms_per_step"], 3),
           "tflops_step": round(r["tflops_step"], 2),
           "gemm_tflop_per_step": round(r["flops_step"] / 1e12, 3),
           "gemm_frac_of_mfma_peak": round(r["gemm_tflops"] / MFMA_F16_PEAK_TFLOPS, 4)}
    out.update({k: v for k, v in r["report"].items() if k != "quantize_by_call"})
    out["quantize_us_in_step"] = {k: v["us_in_step"] for k, v in
                                  r["report"]["quantize_by_call"].items()}
    del ms
    torch.cuda.empty_cache()
    return out


def isolated_times(torch, calls, dev, reps=10):
    """Kernel time (us) of each recorded call run alone on one stream: the
    mean of `reps` back-to-back repetitions between two events, after one
    untimed call and a 1 GiB read that evicts the L2 and the 256 MB Infinity
    Cache.  Back-to-back calls re-read their input; every input here but the
    two 16x16 weights' codes is at least as large as the Infinity Cache, so
    little of it is still cached when the next call starts."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    out = {}
    for kind, name, fn, a, kw in calls:
        fn(*a, **kw)
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(*a, **kw)
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / reps
    del flush
    return out


QCOUNTER_FILE = os.path.join(ROOT, "profiles", "quantize_counters_llama8b.json")
QUANT_SOURCE = os.path.join(ROOT, "nvfp4_bit_microscaled_amd", "csrc", "quantize.hip")


def quantize_counters():
    """Per-call counter summary of the step's quantize kernels (HBM bytes, VALU
    busy, the bound they imply) from the committed rocprofv3 run, or None when
    it is missing or was taken on a different quantize source."""
    import hashlib
    try:
        with open(QCOUNTER_FILE) as f:
            rec = json.load(f)
        with open(QUANT_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("quantize_source_sha256") != sha:
        return None
    return rec.get("calls")


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
    """Decode-shape NT GEMM: activations [M, 8192] x weights [28672, 8192],
    both 1x16 RNE.  HBM-bound on the packed weights (codes + scales).  Four
    copies of the quantized weights (4 x 132 MB, twice the 256 MB Infinity
    Cache) are cycled through 40 back-to-back launches, so every launch reads
    weights evicted by the three before it; `us` is the mean per launch
    (HIP events around the 40), `us_graph` the same 40 launches captured in
    one HIP graph and replayed (a decode loop's way to launch; w4a16_us is
    timed that way too).
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
    reps = 40
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def graph_time(launch):
        """Mean seconds per launch of `reps` launches captured in one HIP graph
        and replayed (twice untimed, then three timed replays)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(4):
                launch(i)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                launch(i)
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e-3 / (3 * reps)

    for M in cfg["ms"]:
        a = nv.quantize(x[:M].contiguous())
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        for i in range(4):
            nv.gemm("NT", a, ws[i], out=y)
        e0.record()
        for i in range(reps):
            nv.gemm("NT", a, ws[i % 4], out=y)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        t_graph = graph_time(lambda i: nv.gemm("NT", a, ws[i % 4], out=y))
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
        t16 = graph_time(lambda i: nv.gemm_w4a16(ab, ws[i % 4], out=y))
        out["M%d" % M] = {"us": round(t * 1e6, 2),
                          "us_graph": round(t_graph * 1e6, 2),
                          "w4a16_us": round(t16 * 1e6, 2),
                          "weights_GBps": round(wbytes / t / 1e9, 1),
                          "frac_of_hbm": round(wbytes / t / 1e9 / HBM_PEAK_GBPS, 4),
                          "tflops": round(2.0 * M * N * K / t / 1e12, 2),
                          "us_isolated": round(sorted(iso)[len(iso) // 2] * 1e3, 2)}
    del flush
    return {"shape": "M x 28672 x 8192, weights 1x16 along K (w4a16_us: BF16 activations)",
            "weight_bytes": int(wbytes),
            "timing": "mean of 40 back-to-back launches over 4 weight copies (528 MB, "
                      "cache-cold each launch; us_graph, w4a16_us: the 40 captured in one HIP "
                      "graph); us_isolated: median of 10 single launches after a "
                      "cache-evicting read", **out}


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
    # NVFP4 operands whose block scales are powers of two, equal across each
    # 32-K pair (random codes; A 1x16, W 16x16): nvfp4_gemm_native takes the
    # native scaled FP4 MFMA for them (check, E8M0 planes and GEMM timed
    # together), against nvfp4_gemm's FP16 path on the same operands
    g = torch.Generator(device="cuda").manual_seed(12)
    pow2 = torch.tensor([e << 3 for e in range(5, 12)], dtype=torch.uint8, device="cuda")

    def pow2_operand(rows, block2d):
        codes = torch.randint(0, 256, (rows, D // 2), dtype=torch.uint8, device="cuda",
                              generator=g)
        srows = rows // 16 if block2d else rows
        idx = torch.randint(0, len(pow2), (srows, D // 32), device="cuda", generator=g)
        scales = pow2[idx].repeat_interleave(2, dim=1).contiguous()
        return nv.NVFP4Tensor(codes, scales, torch.ones(1, device="cuda"),
                              torch.zeros(1, device="cuda"), rows, D, block2d, 1)

    xp, wp = pow2_operand(T, False), pow2_operand(N, True)
    used = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_native = timed(lambda: nv.gemm_native(xp, wp, out=y, used_native=used))
    native_used = int(used.item())
    t_fp16 = timed(lambda: nv.gemm("NT", xp, wp, out=y))
    del y, xp, wp
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
            "nvfp4_native_pow2_scales": {
                "call": "nvfp4_gemm_native on NVFP4 operands with power-of-two block scales "
                        "(check + E8M0 planes + k_gemm_mx)",
                "used_native": native_used, "ms": round(t_native, 4),
                "tflops": round(fl / t_native / 1e9, 1),
                "fp16_path_ms": round(t_fp16, 4),
                "fp16_path_tflops": round(fl / t_fp16 / 1e9, 1)},
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
    """The oracle, as it stands, on bounded samples of the same work (all host
    cores unless stated):
      - value: fprop GEMM 1 for the first `rows` tokens (all 28672 outputs,
        full K = 4096), FP64 dot products of the quantized operands;
      - single_thread_value: the same on rows / cores tokens, one thread;
      - quantize: the whole of X (32768 x 4096, 1x16 RNE with its amax pass)
        and W_gu (16x16 with its amax pass);
      - tiny: the 256 x 256 quantize / dequantize and the 128 x 128 x 256 GEMM
        in full;
      - decode_m1: the decode weight (28672 x 8192, 1x16) quantized and the
        M = 1 GEMM in full."""
    import numpy as np

    import oracle
    rows = args.cpu_sample_rows
    cores = len(os.sched_getaffinity(0))
    oracle.set_num_threads(cores)
    out = {"unit": "TFLOP/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model()}
    # quantize: all of X and W_gu (2.56 B/elem with the amax pass read: 4.56)
    xc_all = X.cpu()
    w = W_gu.cpu()
    t0 = time.perf_counter()
    oracle.quantize(workloads.bf16_bits(xc_all))
    wc, wsc, wts, _ = oracle.quantize(workloads.bf16_bits(w), block2d=True)
    tq = time.perf_counter() - t0
    qbytes = (xc_all.numel() + w.numel()) * (2 * 2 + 0.5) + xc_all.numel() / 16 + w.numel() / 256
    out["quantize_GBps"] = round(qbytes / tq / 1e9, 4)
    out["quantize_sample"] = ("all of X (32768 x 4096, 1x16 RNE) and W_gu (28672 x 4096, "
                              "16x16 RNE), each with its amax pass, %.1f s" % tq)
    # GEMM: fprop GEMM 1 on the first `rows` tokens
    x = X[:rows].cpu()
    xc, xs, xts, _ = oracle.quantize(workloads.bf16_bits(x), amax_in=float(X.abs().max().item()))
    N, K = w.shape
    m_, n_ = np.meshgrid(np.arange(rows), np.arange(N), indexing="ij")
    t1 = time.perf_counter()
    oracle.gemm_pairs("NT", rows, N, K, (xc, xs, xts, False), (wc, wsc, wts, True), m_.ravel(),
                      n_.ravel())
    tg = time.perf_counter() - t1
    flops = 2.0 * rows * N * K
    out["value"] = round(flops / tg / 1e12, 6)
    out["sample"] = ("fprop GEMM 1 (NT, 2D-quantized W_gu) on the first %d tokens: "
                     "%d x %d x %d FP64 dot products (%.2f GFLOP) in %.1f s"
                     % (rows, rows, N, K, flops / 1e9, tg))
    # the same on one thread, over rows / cores tokens (about the same wall time)
    rows1 = max(1, rows // cores)
    m1, n1 = np.meshgrid(np.arange(rows1), np.arange(N), indexing="ij")
    oracle.set_num_threads(1)
    t2 = time.perf_counter()
    oracle.gemm_pairs("NT", rows1, N, K, (xc, xs, xts, False), (wc, wsc, wts, True), m1.ravel(),
                      n1.ravel())
    t1s = time.perf_counter() - t2
    oracle.set_num_threads(cores)
    out["single_thread_value"] = round(2.0 * rows1 * N * K / t1s / 1e12, 6)
    out["single_thread_sample"] = "the same GEMM on the first %d tokens, one thread, %.1f s" % (
        rows1, t1s)
    # the tiny workload in full
    cfg = workloads.TINY
    t3 = time.perf_counter()
    a_c, a_s, a_t, _ = oracle.quantize(workloads.bf16_bits(
        workloads.activations(*cfg["act"], seed=cfg["act_seed"])))
    oracle.dequantize(a_c, a_s, a_t, *cfg["act"])
    b_c, b_s, b_t, _ = oracle.quantize(workloads.bf16_bits(
        workloads.weights(*cfg["w"], seed=cfg["w_seed"])), block2d=True)
    M_, N_, K_ = cfg["gemm"]
    oracle.gemm_full("NT", M_, N_, K_, (a_c[:M_], a_s[:M_], a_t, False), (b_c, b_s, b_t, True))
    out["tiny_full_s"] = round(time.perf_counter() - t3, 4)
    # decode M = 1 in full: quantize the weight, then the 1 x 28672 x 8192 GEMM
    dc = workloads.DECODE
    wd = workloads.weights(dc["n"], dc["k"], seed=dc["w_seed"])
    ad = workloads.activations(64, dc["k"], seed=dc["act_seed"])[:1]
    t4 = time.perf_counter()
    dw = oracle.quantize(workloads.bf16_bits(wd))
    tqd = time.perf_counter() - t4
    da = oracle.quantize(workloads.bf16_bits(ad))
    t5 = time.perf_counter()
    oracle.gemm_full("NT", 1, dc["n"], dc["k"], (da[0], da[1], da[2], False),
                     (dw[0], dw[1], dw[2], False))
    tgd = time.perf_counter() - t5
    out["decode_m1"] = {"weight_quantize_s": round(tqd, 3), "gemm_s": round(tgd, 3),
                        "gemm_GFLOPs": round(2.0 * dc["n"] * dc["k"] / tgd / 1e9, 3),
                        "sample": "28672 x 8192 weight (1x16 RNE with amax pass), then the "
                                  "M = 1 GEMM over all 28672 outputs"}
    return out


if __name__ == "__main__":
    main()
