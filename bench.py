"""Benchmark: SageBwd INT8 attention forward + backward on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the
forward (preparation + fused attention kernel) and the backward (preparation,
dK/dV kernel, dQ kernel), all through the library's C ABI on torch's current
stream, with inputs already resident in HBM.  As in training, the backward
reads the quantized Q and K from the forward's workspace (--no-reuse makes it
re-quantize them; the results are bit-identical).  Throughput is reported as
fwd+bwd TOPS = sum over (batch, head) of 14 N^2 d (4 forward + 10 backward,
halved when causal) per step time.

    python bench.py [--steps K] [--warmup W] [--workload llama16k] [--no-cpu-baseline]

Prints one JSON line.  HIP events bracket every stage of every timed step, so
the per-kernel averages (and the roofline of the dominant kernel) come from the
same timed region.  The CPU baseline times the oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd attention TOPS, causal H=32 d=64 N=8K/16K; % of MFMA peak"
METRIC_FP4 = "fwd attention TOPS (FP4 inference forward), causal H=32 d=64 N=16K; % of MFMA peak"
INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, published (dense FP8 is the same 5.0 PFLOP/s)
FP4_PEAK_TOPS = 10100.0          # MI355X dense FP4 MFMA, published
KERNEL_SOURCES = {
    "FWD_ATTN": ["fwd.hip", "attn.h", "common.h"],
    "BWD_DKDV": ["bwd.hip", "attn.h", "common.h"],
    "BWD_DQ": ["bwd.hip", "attn.h", "common.h"],
}
# algorithmic matmul work of each attention kernel, in units of 2*N^2*d per
# head (times 1/2 when causal), as the metric counts it: forward QK^T + P~V;
# dK/dV kernel QK^T, P^T dO, dO V^T, dS^T Q; dQ kernel dS K (it also
# recomputes QK^T and dO V^T, which the metric does not count again)
KERNEL_UNITS = {"FWD_ATTN": 2, "BWD_DKDV": 4, "BWD_DQ": 1}
# vector-ALU issue ceiling: 256 CUs x 4 SIMDs, one wave64 instruction per SIMD
# every 4 cycles at the 2.4 GHz rating
VALU_PEAK_INSTR_PER_S = 1024 * 2.4e9 / 4


def source_sha(stage: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "bit_trainable_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_profile(stage: str, workload: str):
    """The committed rocprofv3 summary of one kernel on one workload (HBM
    bytes per launch, the profiled average duration, the shader clock measured
    under load), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{stage.lower()}_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        c = json.load(fh)
    if c.get("source_sha") != source_sha(stage):
        return None
    return c


def cpu_baseline(w, seconds: float, mode: str = "int8"):
    """Time the oracle (faithful forward + backward, its MXFP8 mode, or the
    FP4 forward alone) on whole heads of a causal-prefix sub-problem of the
    workload: the first n tokens of head (0, h), h = 0, 1, ... until about
    ``seconds`` have elapsed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as W
    from oracle import faithful, fp4, mxfp8

    F = {"int8": faithful, "mxfp8": mxfp8, "fp4": fp4}[mode]

    n = min(w.N, 2048)
    done_heads = 0
    t0 = time.perf_counter()
    while True:
        x = W.make_head(w, 0, done_heads % w.H)
        f = {k: W.bf16_bits_to_f32(v)[:n] for k, v in x.items()}
        pp = F.prepare(f["q"], f["k"], f["v"], w.smooth_q, w.smooth_k)
        o, lse = F.fwd_head(pp, w.causal)
        if mode != "fp4":
            o_b = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o[:n].astype(np.float32)))
            bp = F.prepare_bwd(pp, f["v"], o_b, lse[:n].astype(np.float32), f["do"])
            F.bwd_head(bp, w.causal)
        done_heads += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    ops = done_heads * (4.0 if mode == "fp4" else 14.0) * n * n * 64 * (0.5 if w.causal else 1.0)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": cores, "blas_threads": int(threads), "kind": "oracle",
            "sample": f"{'faithful' if mode == 'int8' else mode} {'fwd' if mode == 'fp4' else 'fwd+bwd'} of {done_heads} whole head(s) of the first {n} tokens of {w.name} "
                      f"(causal={w.causal}) in {el:.1f} s; {cores} host cores available to the process "
                      f"({os.cpu_count()} in the machine), BLAS threads {threads}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--int8-dp", action="store_true",
                    help="time the all-INT8 ablation (dO V^T from INT8 codes) instead of the method's FP16 dO V^T")
    ap.add_argument("--qk-norm", action="store_true", help="fuse QK-norm into the path (normalizes the inputs' rows)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="time the MXFP8 mode (E4M3 codes, E8M0 exponents per 32x32 block) instead of INT8")
    ap.add_argument("--fp4", action="store_true",
                    help="time the FP4 inference forward (MXFP4: E2M1 codes, E8M0 exponents per 32 values) alone")
    ap.add_argument("--no-reuse", action="store_true",
                    help="let the backward re-quantize Q and K instead of reading the forward's workspace")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size before timing (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "heads shard across GPUs without communication, but no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_trainable_attention_amd as sb
    import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = W.make_inputs(w)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    del x
    p = sb.make_params(w.B, w.H, w.N, w.causal, w.smooth_q, w.smooth_k, int8_dp=args.int8_dp, qk_norm=args.qk_norm,
                       mxfp8=args.mxfp8, fp4=args.fp4)
    lib = sb.load_library()
    import ctypes
    ws_f = torch.empty(lib.sagebwd_fwd_workspace_size(ctypes.byref(p)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(0 if args.fp4 else lib.sagebwd_bwd_workspace_size(ctypes.byref(p)), dtype=torch.uint8,
                       device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    stages = ["FWD_PREPARE", "FWD_ATTN", "BWD_PREPARE", "BWD_DKDV", "BWD_DQ"]
    if args.fp4:
        stages = ["FWD_PREPARE", "FWD_ATTN"]                 # an inference forward: no backward

    def step(events=None):
        for i, s in enumerate(stages):
            if events is not None:
                events[i].record()
            if s.startswith("FWD"):
                sb.fwd_stage(s, q, k, v, o, lse, ws_f, p)
            else:
                sb.bwd_stage(s, q, k, v, o, lse, do, dq, dk, dv, ws_b, p, fwd_ws=None if args.no_reuse else ws_f)
        if events is not None:
            events[len(stages)].record()

    if args.calib_copy_mib > 0:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    stage_ms = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, s in enumerate(stages)}

    causal_f = 0.5 if w.causal else 1.0
    unit = 2.0 * w.N * w.N * w.d * w.bh * causal_f          # one 2*N^2*d matmul over all heads
    ops_step = (2 if args.fp4 else 7) * unit                 # fwd+bwd: 4 + 10 = 14 N^2 d; fwd alone 4 N^2 d
    tops = ops_step / (ms_step * 1e-3) / 1e12

    mode_suffix = "_mxfp8" if args.mxfp8 else "_fp4" if args.fp4 else ""
    dom = max((s for s in KERNEL_UNITS if s in stage_ms), key=lambda s: stage_ms[s])
    ach = KERNEL_UNITS[dom] * unit / (stage_ms[dom] * 1e-3) / 1e12
    peak = FP4_PEAK_TOPS if args.fp4 else INT8_PEAK_TOPS
    prof = None if (args.int8_dp or args.qk_norm or args.no_reuse) else load_profile(dom, w.name + mode_suffix)
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4),
            "traffic": prof.get("hbm_bytes_per_launch") if prof else None,
            "avg_launch_ms": round(stage_ms[dom], 4)}
    if prof:
        # the same kernel's average duration in the committed rocprofv3 kernel
        # statistics, and the fraction it gives; the shader clock measured under
        # load (GRBM_GUI_ACTIVE cycles of one XCD over the kernel's duration)
        # and the fraction of the peak at that clock (the peak scales with it)
        ach_p = KERNEL_UNITS[dom] * unit / (prof["avg_ms_profile"] * 1e-3) / 1e12
        roof["avg_launch_ms_profile"] = round(prof["avg_ms_profile"], 4)
        roof["frac_profile"] = round(ach_p / peak, 4)
        roof["sclk_mhz_measured"] = round(prof["sclk_mhz"], 0)
        roof["frac_at_measured_sclk"] = round(ach / (peak * prof["sclk_mhz"] / 2400.0), 4)
        if prof.get("valu_instr_per_launch"):
            # the bound these kernels actually meet: vector-ALU issue.  A wave64
            # VALU instruction occupies a 16-lane SIMD for 4 cycles, so the chip
            # issues at most 1024 SIMDs x 2.4 GHz / 4 of them per second; the
            # kernel's count per launch is the committed SQ_INSTS_VALU (MFMA
            # instructions included), its time this run's launch average
            n_valu = prof["valu_instr_per_launch"]
            valu_ach = n_valu / (stage_ms[dom] * 1e-3)
            roof["valu"] = {"instr_per_launch": n_valu, "achieved": round(valu_ach / 1e9, 1),
                            "peak": round(VALU_PEAK_INSTR_PER_S / 1e9, 1), "unit": "G wave64 instr/s",
                            "frac": round(valu_ach / VALU_PEAK_INSTR_PER_S, 4),
                            "frac_at_measured_sclk": round(valu_ach / (VALU_PEAK_INSTR_PER_S * prof["sclk_mhz"] / 2400.0), 4),
                            "busy_profile": prof.get("valu_busy_profile")}
    out = {
        "metric": METRIC_FP4 if args.fp4 else METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if args.int8_dp else "e4m3 (dO.V^T f16)" if args.mxfp8 else "e2m1" if args.fp4 else "i8 (dO.V^T f16)",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "smooth_q": w.smooth_q, "smooth_k": w.smooth_k, "ops_per_step": ops_step,
                   "bwd_reuses_fwd_quantization": not args.no_reuse, "int8_dp": bool(args.int8_dp),
                   "qk_norm": bool(args.qk_norm), "mxfp8": bool(args.mxfp8), "fp4": bool(args.fp4)},
        "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
        # 12 of the 14 N^2 d units are INT8 and 2 (dO V^T, fwd-side none) FP16 at half the INT8 rate,
        # so the MFMA floor of the mix is 14/16 of the INT8 peak (FP4 forward: the FP4 peak)
        "frac_blended_mfma_peak": round(tops / (FP4_PEAK_TOPS if args.fp4 else INT8_PEAK_TOPS * 14.0 / 16.0), 4),
        "stage_ms": {s: round(t, 4) for s, t in stage_ms.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, "fp4" if args.fp4 else "mxfp8" if args.mxfp8 else "int8")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
