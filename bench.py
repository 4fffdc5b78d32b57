#!/usr/bin/env python3
"""Benchmark of the VDN hybrid video-to-video attention layer on one MI355X.

One step = one whole layer (fp8 quantiser where used, v re-layout + frame Grams,
per-frame Cholesky maps, state scan, readout weights, windowed + anchored softmax
attention with the linear readout + gated merge in its epilogue, anchor merge)
over one batch of seeded synthetic inputs already resident in HBM.

Default workload: F=90 latent frames x N=4032 tokens (48 x 84 patches), H=24,
d=128, bf16 -- the 768p / 14.4 s shaped layer.  `--config 4` runs the F=180
fp8-q.k variant instead; `--extra-tokens T` appends T text / audio tokens to the
sequence (plain softmax for every interaction involving them).

Prints ONE JSON line.  Besides the contract fields it carries
  roofline      dominant kernel (softmax attention + fused readout): algorithmic
                FLOP per launch (4 d H N^2 P(F), P = visited frame pairs, plus the
                readout's 2 d^2 N H (F-2)) / its mean duration from HIP events
                recorded on the launch stream around every timed launch;
  stages_ms     mean duration of every stage over the timed steps;
  readout       the readout kernel on its own (the O_lin = W q entry point, timed
                after the layer): algorithmic bytes and fraction of 8 TB/s;
  cpu_baseline  the fp64 oracle timed on a bounded sample (rank 0, N=1 only) and
                extrapolated to one layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn layer ms + TFLOP/s & %roofline at 90 frames×4032 tok, H=24,d=128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

CONFIGS = {
    3: dict(F=90, N=4032, H=24, d=128, precision="bf16", workload="vdn_hybrid_attn_768p_14s"),
    4: dict(F=180, N=4032, H=24, d=128, precision="bf16_fp8qk", workload="vdn_hybrid_attn_long_stream_fp8qk"),
    2: dict(F=45, N=1024, H=16, d=128, precision="bf16", workload="vdn_hybrid_attn_mid"),
}


def frame_pairs(F):
    import hybrid_sparse_linear_chunked_amd as vdn
    P = 0
    for row in vdn.schedule(F):
        nq = int(row[1]) - int(row[0]) + 1
        nk = sum(int(row[4 + 2 * x]) - int(row[3 + 2 * x]) + 1 for x in range(int(row[2])))
        P += nq * nk
    return P


def algorithmic_work(F, N, H, d, T=0):
    """FLOP of each part of the method (not of dense attention) and readout bytes;
    T extra tokens add video x extra and extra x all softmax pairs."""
    P = frame_pairs(F)
    C = (F + 4) // 5
    soft = 4.0 * d * H * N * N * P                  # Q.K^T and P.V over visited pairs
    soft += 4.0 * d * H * T * (2.0 * F * N + T)     # with extra tokens
    grams = 4.0 * d * d * N * max(F - 2, 0) * H     # K K^T and V K^T per non-anchor frame
    scan = 2.0 * H * max(F - 11, 0) * (7.0 / 3.0) * d ** 3
    readout = 2.0 * d * d * max(F - 2, 0) * N * H
    # standalone readout kernel: q in, O_lin out (non-anchor frames), bf16 W in
    ro_bytes = 2.0 * max(F - 2, 0) * N * H * d * 2 + C * H * d * d * 2
    return dict(P=P, soft=soft, grams=grams, scan=scan, readout=readout, total=soft + grams + scan + readout,
                readout_bytes=ro_bytes)


PROFILE = {3: os.path.join(ROOT, "profiles", "layer_kernels_768p_14s.txt")}


def measured_traffic(config):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by its reading on a
    copy kernel of known size), or None when there is no summary for this
    workload or the kernel source changed after the counters were taken."""
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


def cpu_baseline(F, N, H, d, seed=0, tokens=2560):
    """Time the fp64 oracle on a bounded sample of the workload and extrapolate to
    one layer (ms).  Sample: heads 0 and H-1; the softmax of `tokens` query tokens
    of one query frame of every work class (anchor / edge chunk / next-to-edge /
    interior); both heads' whole forward + backward state computation; one frame's
    readout per head."""
    import numpy as np
    import torch
    import threadpoolctl
    import vdn_synth
    from oracle import vdn_oracle as orc

    heads = sorted({0, H - 1})

    def gen(name):
        out = torch.empty((F, N, len(heads), d), dtype=torch.bfloat16)
        vdn_synth.tensor(name, F, N, H, d, seed=seed, heads=heads, out=out,
                         convert=lambda b: torch.from_numpy(b).to(torch.bfloat16))
        return out.to(torch.float64).numpy()

    q, k, v = gen("q"), gen("k"), gen("v")
    beta = vdn_synth.beta(F, H, seed=seed).astype(np.float64)[:, heads]
    hs = list(range(len(heads)))
    classes = {}
    for i in range(F):
        classes.setdefault(len(orc.softmax_frames(i, F)), []).append(i)
    t0 = time.perf_counter()
    soft_s = 0.0
    for nk, frames in sorted(classes.items()):
        i = frames[len(frames) // 2]
        a = time.perf_counter()
        orc.softmax_branch(q, k, v, frames=[i], heads=hs, tokens=range(tokens))
        per_token = (time.perf_counter() - a) / tokens
        soft_s += per_token * N * len(frames)
    a = time.perf_counter()
    Sf, Sb = orc.vda_states(k, v, beta)
    states_s = time.perf_counter() - a
    a = time.perf_counter()
    orc.linear_branch(q, Sf, Sb, frames=[F // 2])
    readout_s = (time.perf_counter() - a) * max(F - 2, 0)
    sample_s = time.perf_counter() - t0
    per_head = (soft_s + states_s + readout_s) / len(heads)
    layer_ms = 1000.0 * H * per_head
    info = threadpoolctl.threadpool_info()
    cores = max([x.get("num_threads", 1) for x in info] or [1])
    blas = ",".join(sorted({f"{x.get('internal_api')} {x.get('version')}" for x in info if x.get("user_api") == "blas"}))
    return {
        "value": layer_ms, "unit": "ms", "cores": cores, "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, heads {heads} of {H}: softmax of {tokens} query tokens of one frame "
                   f"per work class ({len(classes)} classes), full forward+backward VDA states, one "
                   f"frame's readout; extrapolated by token/frame counts and to {H} heads; "
                   f"{sample_s:.1f} s of CPU work"),
        "sample_seconds": round(sample_s, 2),
        "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "blas": blas,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3, choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-tokens", type=int, default=0, metavar="T",
                    help="append T text / audio tokens to the layer's sequence (no CPU baseline)")
    ap.add_argument("--out-proj", type=int, default=0, metavar="D",
                    help="follow the layer with the two branches' output projections to D channels "
                         "(no CPU baseline)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (a known-size kernel "
                         "that calibrates the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}); "
              "the layer shards by head across GPUs but no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

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

    cfg = CONFIGS[args.config]
    F, N, H, d, prec = cfg["F"], cfg["N"], cfg["H"], cfg["d"], cfg["precision"]
    p = vdn.PRECISIONS[prec]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()

    T = args.extra_tokens
    Dp = args.out_proj
    if T and Dp:
        print("bench.py: --extra-tokens and --out-proj are separate workloads", file=sys.stderr)
        sys.exit(2)

    def gen(name):
        out = torch.empty((F, N, H, d), dtype=torch.bfloat16)
        vdn_synth.tensor(name, F, N, H, d, out=out,
                         convert=lambda b: torch.from_numpy(b).to(torch.bfloat16))
        if T > 0:
            ext = torch.from_numpy(vdn_synth.extra(name, T, H, d)).to(torch.bfloat16)
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
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; workspace "
          f"{ws.numel() / 2**30:.2f} GiB", file=sys.stderr, flush=True)

    def step():
        if Dp > 0:
            vdn.hybrid_attn_proj(q, k, v, beta, gate, Wp, precision=p, out=Y, workspace=ws)
        elif T > 0:
            vdn.hybrid_attn_mixed(q, k, v, beta, gate, F, N, precision=p, out=O, workspace=ws)
        else:
            vdn.hybrid_attn(q, k, v, beta, gate, precision=p, out=O, workspace=ws)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] warmup {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    # stages the layer runs in this precision: the quantiser only with fp8 q.k; the
    # bf16 and fp8 layers run the readout and merge in the attention kernel
    run = [st for st, name in enumerate(vdn.STAGES)
           if (name != "quant" or prec == "bf16_fp8qk") and name != "readout" and (name != "proj" or Dp > 0)]
    ev = {(s, st): (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for s in range(args.steps) for st in run}
    for pair in ev.values():       # torch creates the HIP event on its first record
        pair[0].record()
        pair[1].record()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(args.steps):
        for st in run:
            vdn.set_stage_events(st, *ev[(s, st)])
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for st in run:
        vdn.set_stage_events(st, None, None)
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    stages = {}
    for st in run:
        vals = [ev[(s, st)][0].elapsed_time(ev[(s, st)][1]) for s in range(args.steps)]
        stages[vdn.STAGES[st]] = sum(vals) / len(vals)
    print(f"[bench] {args.steps} steps: {ms:.2f} ms/step (wall {1000 * wall / args.steps:.2f})",
          file=sys.stderr, flush=True)

    work = algorithmic_work(F, N, H, d, T)
    proj_flop = 2.0 * F * N * Dp * 2 * H * d       # [O_soft | g O_lin] [W_s | W_l]^T
    work["total"] += proj_flop
    attn_ms = stages["attn"]
    kflop = work["soft"] + work["readout"]      # softmax branch + the fused W q
    if prec == "bf16_fp8qk":
        # q.k at the fp8 peak, p.v and W q at the bf16 peak: their time-weighted peak
        half = work["soft"] / 2
        peak = kflop / (half / PEAK_FP8_TFLOPS + (half + work["readout"]) / PEAK_BF16_TFLOPS)
    else:
        peak = PEAK_BF16_TFLOPS
    achieved = kflop / (attn_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": measured_traffic(args.config) if T == 0 else None,
                "kernel": "attn_lds_kernel", "flop_per_launch": kflop, "kernel_ms": round(attn_ms, 3)}

    # the readout kernel on its own, for its HBM roofline (outside the timed layer)
    ro_st = vdn.STAGES.index("readout")
    Sf, Sb = vdn.vda_states(kv, vv, beta, precision=p, workspace=ws)
    ro_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(6)]
    for e0, e1 in ro_ev:           # torch creates the HIP event on its first record
        e0.record()
        e1.record()
    for e0, e1 in ro_ev:
        vdn.set_stage_events(ro_st, e0, e1)
        O_lin = vdn.vda_linear(qv, Sf, Sb, precision=p, workspace=ws)
        del O_lin
    vdn.set_stage_events(ro_st, None, None)
    torch.cuda.synchronize()
    ro_vals = [e0.elapsed_time(e1) for e0, e1 in ro_ev[1:]]
    ro_ms = sum(ro_vals) / len(ro_vals)
    del Sf, Sb
    readout = None
    if ro_ms:
        gbs = work["readout_bytes"] / (ro_ms * 1e-3) / 1e9
        readout = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": work["readout_bytes"],
                   "kernel_ms": round(ro_ms, 4), "kernel": "readout_kernel (O_lin = W q, standalone)"}
    result = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["workload"] + (f"_with_{T}_text_tokens" if T else "")
                   + (f"_with_out_proj_{Dp}" if Dp else ""), "F": F, "N": N, "H": H, "d": d,
                   "precision": prec, "frame_pairs": work["P"], "extra_tokens": T, "out_proj": Dp},
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
    if not args.no_cpu_baseline and T == 0 and Dp == 0:
        print("[bench] timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(F, N, H, d)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
