#!/usr/bin/env python3
"""Benchmark of the VDN hybrid video-to-video attention layer on one MI355X.

One step = one whole layer (fp8 quantiser where used, v re-layout + frame Grams,
per-frame Cholesky maps, state scan, readout weights, windowed + anchored softmax
attention with the linear readout + gated merge in its epilogue, anchor merge)
over one batch of seeded synthetic inputs already resident in HBM.

Workloads (`--config`):
  0  F=20  N=16   H=2  d=32  fp32          tiny
  1  F=30  N=256  H=8  d=64  bf16          small
  2  F=45  N=1024 H=16 d=128 bf16          mid
  3  F=90  N=4032 H=24 d=128 bf16          768p / 14.4 s shaped layer (default)
  4  F=180 N=4032 H=24 d=128 bf16, q.k in fp8 E4M3   long stream
`--extra-tokens T` appends T text / audio tokens to the sequence (plain softmax
for every interaction involving them); `--out-proj D` follows the layer with the
two branches' output projections.

Prints ONE JSON line.  Every timed step is bracketed by its own pair of HIP events
on the launch stream, and so is every stage of it; ms_per_step and stages_ms are
medians over the timed steps.  Besides the contract fields the line carries
  roofline      the dominant kernel (softmax attention + fused readout):
                algorithmic FLOP per launch (4 d H N^2 P(F), P = visited frame
                pairs, plus the readout's 2 d^2 N H (F-2)) / its median duration;
                `traffic` is the HBM bytes per launch from the committed rocprofv3
                counter summary of this workload (FETCH_SIZE + WRITE_SIZE, each
                scaled by its reading on a copy of known size), null when there is
                none or the kernel source changed after it was taken;
  readout       the readout inside the layer: the attention stage's median with
                the readout fused minus without it (the softmax branch alone,
                interleaved with layer runs), and the standalone readout kernel
                (the O_lin = W q entry point) against 8 TB/s;
  cpu_baseline  the fp64 oracle on the host (rank 0, N=1): in full for the three
                small workloads, else on a bounded sample extrapolated to a layer.
With `--vendor-attention` the line also carries `vendor_attention`: torch's fused
attention (its flash / memory-efficient kernels only, never the math fallback) on
the dense sub-problem of one interior chunk (all heads; the chunk's 5 query frames
against its 17 key frames, no mask), timed on the same device beside the layer as
a same-box library reference for the attention kernel's TFLOP/s.
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

METRIC = "hybrid-attn layer ms + TFLOP/s & %roofline at 90 frames×4032 tok, H=24,d=128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

CONFIGS = {
    0: dict(F=20, N=16, H=2, d=32, precision="fp32", workload="vdn_hybrid_attn_tiny_fp32"),
    1: dict(F=30, N=256, H=8, d=64, precision="bf16", workload="vdn_hybrid_attn_small"),
    2: dict(F=45, N=1024, H=16, d=128, precision="bf16", workload="vdn_hybrid_attn_mid"),
    3: dict(F=90, N=4032, H=24, d=128, precision="bf16", workload="vdn_hybrid_attn_768p_14s"),
    4: dict(F=180, N=4032, H=24, d=128, precision="bf16_fp8qk", workload="vdn_hybrid_attn_long_stream_fp8qk"),
}
# workloads small enough for the oracle to run in full on the host
FULL_ORACLE = (0, 1, 2)
# committed counter summaries (HBM bytes of the attention kernel) per workload
PROFILE = {
    2: os.path.join(ROOT, "profiles", "layer_kernels_mid_45f_1024tok.txt"),
    3: os.path.join(ROOT, "profiles", "layer_kernels_768p_14s.txt"),
    4: os.path.join(ROOT, "profiles", "layer_kernels_long_stream_180f_fp8qk.txt"),
}


def frame_pairs(F):
    import hybrid_sparse_linear_chunked_amd as vdn
    P = 0
    for row in vdn.schedule(F):
        nq = int(row[1]) - int(row[0]) + 1
        nk = sum(int(row[4 + 2 * x]) - int(row[3 + 2 * x]) + 1 for x in range(int(row[2])))
        P += nq * nk
    return P


def algorithmic_work(F, N, H, d, T=0, eb=2):
    """FLOP of each part of the method (not of dense attention) and readout bytes;
    T extra tokens add video x extra and extra x all softmax pairs."""
    P = frame_pairs(F)
    C = (F + 4) // 5
    soft = 4.0 * d * H * N * N * P                  # Q.K^T and P.V over visited pairs
    soft += 4.0 * d * H * T * (2.0 * F * N + T)     # with extra tokens
    grams = 4.0 * d * d * N * max(F - 2, 0) * H     # K K^T and V K^T per non-anchor frame
    scan = 2.0 * H * max(F - 11, 0) * (7.0 / 3.0) * d ** 3
    readout = 2.0 * d * d * max(F - 2, 0) * N * H
    # standalone readout kernel: q in, O_lin out (non-anchor frames), W in (bf16)
    ro_bytes = 2.0 * max(F - 2, 0) * N * H * d * eb + C * H * d * d * eb
    return dict(P=P, soft=soft, grams=grams, scan=scan, readout=readout, total=soft + grams + scan + readout,
                readout_bytes=ro_bytes)


def measured_traffic(config):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter summary, or None when there is none for this workload or the kernel
    source changed after the counters were taken."""
    import hashlib
    path = PROFILE.get(config)
    if not path or not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(os.path.join(ROOT, "hybrid_sparse_linear_chunked_amd", "csrc", "attn.hip"),
                              "rb").read()).hexdigest()[:16]
    recorded, traffic = None, None
    for line in open(path):
        if line.startswith("attn.hip sha256[:16] when measured:"):
            recorded = line.rsplit(":", 1)[1].strip()
        if line.startswith("attn_lds_kernel traffic_bytes_per_launch:"):
            traffic = float(line.rsplit(":", 1)[1])
    return traffic if recorded == sha else None


def _blas_info():
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    cores = max([x.get("num_threads", 1) for x in info if x.get("user_api") == "blas"] or [1])
    blas = ",".join(sorted({f"{x.get('internal_api')} {x.get('version')}" for x in info if x.get("user_api") == "blas"}))
    return cores, blas


def _host_inputs(F, N, H, d, heads, fp32, seed=0):
    """q, k, v of the listed heads as the device sees them (bf16-rounded unless
    fp32), in float64 for the oracle; beta, gate of those heads."""
    import numpy as np
    import torch
    import vdn_synth
    dt = torch.float32 if fp32 else torch.bfloat16

    def gen(name):
        out = torch.empty((F, N, len(heads), d), dtype=dt)
        vdn_synth.tensor(name, F, N, H, d, seed=seed, heads=heads, out=out,
                         convert=lambda b: torch.from_numpy(b).to(dt))
        return out.to(torch.float64).numpy()

    q, k, v = gen("q"), gen("k"), gen("v")
    beta = vdn_synth.beta(F, H, seed=seed).astype(np.float64)[:, heads]
    gate = vdn_synth.gate(H, d, seed=seed).astype(np.float64)[heads]
    return q, k, v, beta, gate


def cpu_baseline_full(F, N, H, d, fp32):
    """The whole fp64 oracle on every head, frame and token: softmax branch (one
    query frame at a time over its gathered key frames), forward and backward
    states, readout, merge; timed end to end (ms)."""
    from oracle import vdn_oracle as orc
    heads = list(range(H))
    q, k, v, beta, gate = _host_inputs(F, N, H, d, heads, fp32)
    import numpy as np
    # one head at a time (as the oracle itself loops), with a progress line per head
    sec = 0.0
    O_soft = np.zeros_like(q)
    for h in heads:
        t0 = time.perf_counter()
        O_soft[:, :, h:h + 1] = orc.softmax_branch(q, k, v, heads=[h])
        sec += time.perf_counter() - t0
        print(f"[bench] oracle softmax branch, head {h + 1}/{H}: {sec:.1f} s so far", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    Sf, Sb = orc.vda_states(k, v, beta)
    O_lin = orc.linear_branch(q, Sf, Sb)
    orc.merge(O_soft, O_lin, gate)
    sec += time.perf_counter() - t0
    cores, blas = _blas_info()
    return {
        "value": 1000.0 * sec, "unit": "ms", "cores": cores, "kind": "oracle",
        "sample": f"the whole layer, fp64 NumPy oracle, all {H} heads, {F} frames, {N} tokens per frame "
                  f"(measured, not extrapolated); {sec:.1f} s of CPU work",
        "sample_seconds": round(sec, 2), "measured": True,
        "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "blas": blas,
    }


def cpu_baseline_sampled(F, N, H, d, fp32, tokens=2560):
    """The fp64 oracle on a bounded sample of the workload, extrapolated to one
    layer (ms).  Sample: heads 0 and H-1; the softmax of `tokens` query tokens of
    one query frame of every work class (anchor / edge chunk / next-to-edge /
    interior), scaled by the class's token count; both heads' whole forward +
    backward state computation; one frame's readout per head scaled to F-2 frames;
    the sum scaled from 2 heads to H."""
    from oracle import vdn_oracle as orc
    heads = sorted({0, H - 1})
    q, k, v, beta, _ = _host_inputs(F, N, H, d, heads, fp32)
    hs = list(range(len(heads)))
    tokens = min(tokens, N)
    classes = {}
    for i in range(F):
        classes.setdefault(len(orc.softmax_frames(i, F)), []).append(i)
    t0 = time.perf_counter()
    soft_s = 0.0
    for nk, frames in sorted(classes.items()):
        i = frames[len(frames) // 2]
        a = time.perf_counter()
        orc.softmax_branch(q, k, v, frames=[i], heads=hs, tokens=range(tokens))
        soft_s += (time.perf_counter() - a) / tokens * N * len(frames)
    a = time.perf_counter()
    Sf, Sb = orc.vda_states(k, v, beta)
    states_s = time.perf_counter() - a
    a = time.perf_counter()
    orc.linear_branch(q, Sf, Sb, frames=[F // 2])
    readout_s = (time.perf_counter() - a) * max(F - 2, 0)
    sample_s = time.perf_counter() - t0
    layer_ms = 1000.0 * H * (soft_s + states_s + readout_s) / len(heads)
    cores, blas = _blas_info()
    return {
        "value": layer_ms, "unit": "ms", "cores": cores, "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, heads {heads} of {H}: softmax of {tokens} query tokens of one frame "
                   f"per work class ({len(classes)} classes), full forward+backward VDA states, one "
                   f"frame's readout; extrapolated by token/frame counts and to {H} heads; "
                   f"{sample_s:.1f} s of CPU work"),
        "sample_seconds": round(sample_s, 2), "measured": False,
        "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "blas": blas,
    }


def vendor_attention(F, N, H, d, dev, reps):
    """torch's fused scaled-dot-product attention (flash, else memory-efficient
    kernel; the math fallback is excluded) on one interior chunk's dense problem:
    5 query frames against 17 key frames (15 window frames + 2 anchors), all heads,
    bf16, no mask.  FLOP = 4 d H Nq Nk; median of `reps` timed calls after 2."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    nq_f, nk_f = 5, 17
    if F < 20:
        return {"skipped": "fewer than 4 chunks"}
    g = torch.Generator(device=dev).manual_seed(0)
    Lq, Lk = nq_f * N, nk_f * N
    qd = torch.randn((1, H, Lq, d), device=dev, dtype=torch.bfloat16, generator=g)
    kd = torch.randn((1, H, Lk, d), device=dev, dtype=torch.bfloat16, generator=g)
    vd = torch.randn((1, H, Lk, d), device=dev, dtype=torch.bfloat16, generator=g)
    flop = 4.0 * d * H * Lq * Lk
    out = {"shape": {"H": H, "Lq": Lq, "Lk": Lk, "d": d, "dtype": "bf16"}, "flop_per_call": flop}
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([backend]):
                for _ in range(2):
                    torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)
                torch.cuda.synchronize()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(reps)]
                for a, b in ev:
                    a.record()
                    torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)
                    b.record()
                torch.cuda.synchronize()
        except RuntimeError as e:                      # no such kernel for this device / shape
            print(f"[bench] vendor attention ({name}): {str(e).splitlines()[0]}", file=sys.stderr, flush=True)
            continue
        t = statistics.median([a.elapsed_time(b) for a, b in ev])
        tf = flop / (t * 1e-3) / 1e12
        out.update({"backend": f"torch scaled_dot_product_attention ({name})", "ms": round(t, 4),
                    "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        print(f"[bench] vendor attention ({name}): {t:.3f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
        break
    else:
        out["backend"] = None
    del qd, kd, vd
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 20; 5 for the two largest)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default 3; 2 for the two largest)")
    ap.add_argument("--config", type=int, default=3, choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--precision", default=None, choices=["fp32", "bf16", "bf16_fp8qk", "fp8"],
                    help="run the workload's shape in another precision (fp8: the full-fp8 softmax branch, "
                         "P.V on E4M3 codes too); the line names the precision in its workload")
    ap.add_argument("--extra-tokens", type=int, default=0, metavar="T",
                    help="append T text / audio tokens to the layer's sequence (no CPU baseline)")
    ap.add_argument("--out-proj", type=int, default=0, metavar="D",
                    help="follow the layer with the two branches' output projections to D channels "
                         "(no CPU baseline)")
    ap.add_argument("--vendor-attention", action="store_true",
                    help="also time torch's fused attention on one interior chunk's dense sub-problem "
                         "(a same-box library reference for the attention kernel's TFLOP/s)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (a known-size kernel "
                         "that calibrates the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}); "
              "the layer shards by head across GPUs but no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    big = args.config >= 3
    steps = args.steps if args.steps is not None else (5 if big else 20)
    warmup = args.warmup if args.warmup is not None else (2 if big else 3)

    import torch
    import hybrid_sparse_linear_chunked_amd as vdn
    import vdn_synth

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return

    cfg = dict(CONFIGS[args.config])
    if args.precision and args.precision != cfg["precision"]:
        if (args.precision == "fp32") != (cfg["precision"] == "fp32"):
            print("bench.py: --precision switches between the bf16-I/O precisions only", file=sys.stderr)
            sys.exit(2)
        cfg["precision"] = args.precision
        cfg["workload"] = cfg["workload"] + "_as_" + args.precision
    F, N, H, d, prec = cfg["F"], cfg["N"], cfg["H"], cfg["d"], cfg["precision"]
    p = vdn.PRECISIONS[prec]
    fp32 = prec == "fp32"
    dt = torch.float32 if fp32 else torch.bfloat16
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()

    T = args.extra_tokens
    Dp = args.out_proj
    if T and Dp:
        print("bench.py: --extra-tokens and --out-proj are separate workloads", file=sys.stderr)
        sys.exit(2)
    if (T or Dp) and fp32:
        print("bench.py: extra tokens and output projections need a bf16 workload", file=sys.stderr)
        sys.exit(2)

    def gen(name):
        out = torch.empty((F, N, H, d), dtype=dt)
        vdn_synth.tensor(name, F, N, H, d, out=out, convert=lambda b: torch.from_numpy(b).to(dt))
        if T > 0:
            ext = torch.from_numpy(vdn_synth.extra(name, T, H, d)).to(dt)
            out = torch.cat([out.reshape(F * N, H, d), ext], dim=0)
        return out.to(dev)

    q, k, v = gen("q"), gen("k"), gen("v")
    beta = torch.from_numpy(vdn_synth.beta(F, H)).to(dev)
    gate = torch.from_numpy(vdn_synth.gate(H, d)).to(dev)
    O = torch.empty_like(q)
    if T > 0:
        ws = vdn.new_workspace_mixed(F, N, T, H, d, p, device=dev)
    elif Dp > 0:
        ws = vdn.new_workspace_proj(F, N, H, d, Dp, p, device=dev)
        Wp = torch.from_numpy(vdn_synth.proj_weights(Dp, H * d)).to(torch.bfloat16).to(dev)
        Y = torch.empty((F * N, Dp), dtype=torch.bfloat16, device=dev)
    else:
        ws = vdn.new_workspace(F, N, H, d, p, device=dev)
    # the video tokens as [F, N, H, d] (the first F*N tokens when there are extras)
    qv, kv, vv = (x[:F * N].view(F, N, H, d) for x in (q, k, v)) if T > 0 else (q, k, v)
    torch.cuda.synchronize()
    print(f"[bench] config {args.config}: inputs ready in {time.perf_counter() - t0:.1f} s; workspace "
          f"{ws.numel() / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    def step():
        if Dp > 0:
            vdn.hybrid_attn_proj(q, k, v, beta, gate, Wp, precision=p, out=Y, workspace=ws)
        elif T > 0:
            vdn.hybrid_attn_mixed(q, k, v, beta, gate, F, N, precision=p, out=O, workspace=ws)
        else:
            vdn.hybrid_attn(q, k, v, beta, gate, precision=p, out=O, workspace=ws)

    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{warmup} done", file=sys.stderr, flush=True)

    # stages the layer runs in this precision: the quantiser only with fp8 q.k; the
    # bf16 and fp8 layers run the readout and merge in the attention kernel, the
    # fp32 layer in its own pass
    run = [st for st, name in enumerate(vdn.STAGES)
           if (name != "quant" or prec in ("bf16_fp8qk", "fp8")) and (name != "readout" or fp32)
           and (name != "proj" or Dp > 0)]

    def new_pair():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()              # torch creates the HIP event on its first record
        b.record()
        return a, b

    ev = {(s, st): new_pair() for s in range(steps) for st in run}
    step_ev = [new_pair() for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s in range(steps):
        for st in run:
            vdn.set_stage_events(st, *ev[(s, st)])
        step_ev[s][0].record()
        step()
        step_ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for st in run:
        vdn.set_stage_events(st, None, None)
    per_step = [a.elapsed_time(b) for a, b in step_ev]
    ms = statistics.median(per_step)
    stages = {vdn.STAGES[st]: statistics.median([ev[(s, st)][0].elapsed_time(ev[(s, st)][1]) for s in range(steps)])
              for st in run}
    print(f"[bench] {steps} steps: median {ms:.3f} ms/step, mean {statistics.fmean(per_step):.3f} "
          f"(wall {1000 * wall / steps:.2f})", file=sys.stderr, flush=True)

    work = algorithmic_work(F, N, H, d, T, eb=4 if fp32 else 2)
    proj_flop = 2.0 * F * N * Dp * 2 * H * d       # [O_soft | g O_lin] [W_s | W_l]^T
    work["total"] += proj_flop
    attn_ms = stages["attn"]
    # the dominant kernel: softmax branch, plus the fused W q in the bf16 / fp8 layers
    kflop = work["soft"] + (0.0 if fp32 else work["readout"])
    if prec == "bf16_fp8qk":
        # q.k at the fp8 peak, p.v and W q at the bf16 peak: their time-weighted peak
        half = work["soft"] / 2
        peak = kflop / (half / PEAK_FP8_TFLOPS + (half + work["readout"]) / PEAK_BF16_TFLOPS)
    elif prec == "fp8":
        # q.k and p.v at the fp8 peak, W q at the bf16 peak
        peak = kflop / (work["soft"] / PEAK_FP8_TFLOPS + work["readout"] / PEAK_BF16_TFLOPS)
    elif fp32:
        peak = PEAK_FP32_TFLOPS
    else:
        peak = PEAK_BF16_TFLOPS
    achieved = kflop / (attn_ms * 1e-3) / 1e12
    traffic = measured_traffic(args.config) if (T == 0 and Dp == 0 and not args.precision) else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, calibrated on a copy, from "
                                   "the committed summary of this workload (kernel source unchanged)")
                if traffic is not None else None,
                "kernel": "attn_kernel (fp32)" if fp32 else "attn_lds_kernel", "flop_per_launch": kflop,
                "kernel_ms": round(attn_ms, 4)}

    readout = None
    if T == 0 and Dp == 0:
        ro_st = vdn.STAGES.index("readout")
        att_st = vdn.STAGES.index("attn")
        Sf, Sb = vdn.vda_states(kv, vv, beta, precision=p, workspace=ws)
        reps = 3 if big else 10
        ro_ev = [new_pair() for _ in range(reps)]
        lay_ev = [new_pair() for _ in range(reps)]
        soft_ev = [new_pair() for _ in range(reps)]
        Os = torch.empty_like(q)
        torch.cuda.synchronize()
        for r in range(reps):
            vdn.set_stage_events(ro_st, *ro_ev[r])
            O_lin = vdn.vda_linear(qv, Sf, Sb, precision=p, workspace=ws)
            vdn.set_stage_events(ro_st, None, None)
            del O_lin
            if not fp32:
                # the attention stage with the readout fused (the layer) and without
                # it (the softmax branch alone), interleaved
                vdn.set_stage_events(att_st, *lay_ev[r])
                step()
                vdn.set_stage_events(att_st, *soft_ev[r])
                vdn.softmax_branch(q, k, v, precision=p, out=Os, workspace=ws)
                vdn.set_stage_events(att_st, None, None)
        torch.cuda.synchronize()
        ro_ms = statistics.median([a.elapsed_time(b) for a, b in ro_ev])
        gbs = work["readout_bytes"] / (ro_ms * 1e-3) / 1e9
        readout = {"standalone": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": work["readout_bytes"],
                                  "kernel_ms": round(ro_ms, 4),
                                  "kernel": "readout_kernel (the O_lin = W q entry point)" if not fp32
                                  else "readout_f32_kernel (the fp32 layer's readout pass)"}}
        if not fp32:
            lay = statistics.median([a.elapsed_time(b) for a, b in lay_ev])
            sof = statistics.median([a.elapsed_time(b) for a, b in soft_ev])
            readout["fused_in_layer"] = {
                "attn_with_readout_ms": round(lay, 4), "attn_softmax_only_ms": round(sof, 4),
                "marginal_ms": round(lay - sof, 4),
                "standalone_roofline_ms": round(work["readout_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
                "note": "the layer's readout runs in the attention kernel's epilogue (q and O are not re-read); "
                        "its cost is the attention stage with it minus without it, medians of interleaved runs"}
        del Sf, Sb, Os

    dtype = {"fp32": "fp32", "bf16": "bf16", "bf16_fp8qk": "bf16+fp8e4m3(q.k)", "fp8": "bf16+fp8e4m3(q.k,p.v)"}[prec]
    result = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": cfg["workload"] + (f"_with_{T}_text_tokens" if T else "")
                   + (f"_with_out_proj_{Dp}" if Dp else ""), "F": F, "N": N, "H": H, "d": d,
                   "precision": prec, "frame_pairs": work["P"], "extra_tokens": T, "out_proj": Dp},
        "ms_statistic": "median of per-step HIP-event times",
        "ms_per_step_mean": round(statistics.fmean(per_step), 3),
        "tflops": round(work["total"] / (ms * 1e-3) / 1e12, 2),
        "layer_flop": work["total"],
        "roofline": roofline,
        "readout": readout,
        "stages_ms": {k2: round(v2, 4) for k2, v2 in stages.items()},
    }
    if Dp > 0:
        pj_ms = stages["proj"]
        pj = proj_flop / (pj_ms * 1e-3) / 1e12
        result["proj"] = {"bound": "mfma", "achieved": round(pj, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(pj / PEAK_BF16_TFLOPS, 4), "kernel": "proj_kernel",
                          "flop_per_launch": proj_flop, "kernel_ms": round(pj_ms, 3)}
    del q, k, v, O, ws
    if args.vendor_attention and not fp32 and T == 0 and Dp == 0:
        result["vendor_attention"] = vendor_attention(F, N, H, d, dev, reps=5 if big else 10)
        result["vendor_attention"]["ours_tflops"] = round(achieved, 2)
    if not args.no_cpu_baseline and T == 0 and Dp == 0:
        full = args.config in FULL_ORACLE
        print(f"[bench] timing the oracle ({'whole layer' if full else 'bounded sample'})", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline_full(F, N, H, d, fp32) if full else cpu_baseline_sampled(F, N, H, d, fp32)
        print("[bench] oracle done", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
