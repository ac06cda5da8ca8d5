"""Benchmark: MoE expert block forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]
                    [--no-cpu-baseline] [--profile-steps N]

A step is one full pass of the hot path over one batch of synthetic tokens:
router logits -> top-k/softmax -> permute -> grouped gate/up GEMM + SwiGLU ->
grouped down GEMM + row scale -> combine, then combine backward -> grouped FFN
backward (dGU with dSwiGLU, dX, dW_down, dW_gate_up) -> route backward ->
router backward -> permute backward.  By default (--rows gathered) the
gate/up and dGU GEMMs read their token rows straight from X and dY (the
permute gather and the combine-backward copy folded into their operand
loads; X_perm is still stored for the dW_gate_up GEMM); --rows stored runs
every step through stored X_perm / dY_perm.  Both are bit-identical; the
JSON line also times the other arrangements.  Inputs are resident in HBM
before the timed region starts.

The JSON line also carries, apart from the headline step: the other routed
workloads' whole steps (--other-workloads, default the Zipf-skewed T=16384
and the Qwen3-30B-A3B-like T=32768 layers), one expert-parallel rank's share
(the grouped FFN alone over 8192 pre-routed rows), and the step with frozen
experts and rank-16 LoRA.

Prints one JSON line.  Besides throughput it reports the dominant kernel's
roofline (its algorithmic FLOPs or HBM bytes per launch, whichever bounds it
at peak, over its average launch time measured with HIP events on the stream
the kernel runs on) and the CPU oracle's throughput on a bounded sample of the
same workload.
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

METRIC = "MoE layer fwd+bwd tokens/s + grouped-GEMM % bf16 MFMA peak (gpt-oss-20b-like)"


def gemm_flops(R, d, f):
    """Algorithmic FLOPs of each grouped GEMM launch (routed rows only)."""
    return {
        "gg_fwd_gate_up_swiglu": 4.0 * R * d * f,
        "gg_fwd_down_scale": 2.0 * R * d * f,
        "gg_bwd_dh_dswiglu": 2.0 * R * d * f,
        "gg_bwd_dx": 4.0 * R * d * f,
        "gg_bwd_dw_down": 2.0 * R * d * f,
        "gg_bwd_dw_gate_up": 4.0 * R * d * f,
    }


def gemm_bytes(R, d, f, E, T=None):
    """Algorithmic HBM bytes of each grouped GEMM launch: every operand read
    once and every output written once (bf16 activations and weights, fp32
    weight gradients and combine weights).  With T, the gathered forms: the
    gate/up and dW_gate_up GEMMs read the token rows of X, the dH GEMM those
    of dY, from the unpermuted [T, d] tensor, whose bytes count once."""
    b = 2.0
    t = R if T is None else T
    return {
        "gg_fwd_gate_up_swiglu": b * (t * d + E * 2 * f * d + R * 2 * f + R * f),
        "gg_fwd_down_scale": b * (R * f + E * d * f + R * d) + 4.0 * R,
        # dY rows, W_down, the saved GU (H is recomputed from it), dGU, w
        "gg_bwd_dh_dswiglu": b * (t * d + E * d * f + R * 2 * f + R * 2 * f) + 4.0 * R,
        "gg_bwd_dx": b * (R * 2 * f + E * 2 * f * d + R * d),
        "gg_bwd_dw_down": b * (R * f + R * d) + 4.0 * E * d * f,
        "gg_bwd_dw_gate_up": b * (t * d + R * 2 * f) + 4.0 * E * 2 * f * d,
    }


def row_bytes(T, d, E, k):
    """Algorithmic HBM bytes of the row kernels (bf16 rows, int32 maps, fp32
    weights): each token row and each routed row read or written once."""
    R = T * k
    tok, rows = 2.0 * T * d, 2.0 * R * d
    return {
        "permute_rows": tok + rows + 4.0 * R + 4.0 * R + 4.0 * R,  # + slot_to_row, topk_w, w_perm
        "combine": rows + tok + 4.0 * R,
        "combine_bwd": tok + rows + 4.0 * R,
        "row_scale": tok + rows + 4.0 * R + 4.0 * R,                # dY once (token order) + w
        "permute_bwd": rows + tok + 4.0 * R + 4.0 * T * E + 2.0 * E * d,  # + d_logits, W_r
    }


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/hbm_traffic.json), or None if the summary is for another
    workload or the GEMM source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            j = json.load(fh)
        with open(os.path.join(ROOT, j["source"]), "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
    except (OSError, ValueError, KeyError):
        return None
    if sha != j.get("source_sha256") or j.get("workload") != workload:
        return None
    b = j.get("bytes_per_launch", {}).get(kernel)
    return None if b is None else round(b["read"] + b["write"])


def cpu_baseline(w, a, sample_tokens, min_seconds=10.0):
    """Oracle fwd+bwd on the first `sample_tokens` tokens of the same inputs,
    repeated until at least `min_seconds` have passed."""
    import numpy as np
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    sample_tokens = min(sample_tokens, w.T)
    s = slice(0, sample_tokens)
    x, dy = a["x"][s], a["dy"][s]
    noise = None if a["noise"] is None else a["noise"][s]
    # whole fwd+bwd passes until at least min_seconds of CPU work
    passes, t0 = 0, time.perf_counter()
    while True:
        o = O.layer_forward(x, a["w_r"], a["w_gu"], a["w_down"], w.k, a["bias"], noise, bf16=True)
        O.layer_backward(o, x, a["w_r"], a["w_gu"], a["w_down"], dy, w.k, bf16=True)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": passes * sample_tokens / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": "first %d of %d tokens of the same workload, %d fwd+bwd pass(es), %.1f s" %
                      (sample_tokens, w.T, passes, dt)}


def time_ep_share(steps, warmup, dev):
    """One expert-parallel rank's share (4 local experts, 8192 pre-routed rows,
    d = f = 2880): the grouped FFN forward + backward alone, as ExpertShare
    runs it.  Rows per second, the grouped GEMMs' event times and their
    fraction of the bf16 MFMA peak, and the dominant GEMM's roofline."""
    import numpy as np
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd import inputs as I
    from mixture_experts_layer_03_amd.layer import ExpertShare
    w = I.EP8_SHARE
    a = I.make_inputs(w)

    def up(v, bf=True):
        if bf:
            return torch.from_numpy(I.bf16_bits(v).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)

    xp, wgu, wd, dyp = (up(a[n]) for n in ("x_perm", "w_gu", "w_down", "dy_perm"))
    wp = up(a["w_perm"], False)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(a["counts"])]).astype(np.int32)).to(dev)
    sh = ExpertShare(w.T, w.d, w.E, w.f, device=dev)

    def step():
        sh.forward(xp, off, wgu, wd, wp)
        sh.backward(xp, off, wgu, wd, wp, dyp)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    abi.moe_timing_reset()
    abi.moe_timing_enable(True)
    nprof = 5
    for _ in range(nprof):
        step()
    torch.cuda.synchronize()
    abi.moe_timing_enable(False)
    R = w.T
    flops = gemm_flops(R, w.d, w.f)
    nbytes = gemm_bytes(R, w.d, w.f, w.E)
    us = {}
    for n in flops:
        ms, cnt = abi.moe_timing_query(n)
        if cnt:
            us[n] = 1e3 * ms / cnt
    abi.moe_timing_reset()
    out = {"workload": w.name, "counts": [int(c) for c in a["counts"]],
           "ms_per_step": round(el * 1e3 / steps, 4), "rows_per_s": round(R * steps / el, 1),
           "kernels_us": {n: round(v, 1) for n, v in us.items()}}
    if us:
        tot_f = sum(flops[n] for n in us)
        tot_t = sum(us.values()) * 1e-6
        out["grouped_gemm_tflops"] = round(tot_f / tot_t / 1e12, 1)
        out["grouped_gemm_frac_of_bf16_peak"] = round(tot_f / tot_t / 1e12 / PEAK_BF16_TFLOPS, 4)
        dom = max(us, key=us.get)
        t = us[dom] * 1e-6
        t_m, t_h = flops[dom] / (PEAK_BF16_TFLOPS * 1e12), nbytes[dom] / (PEAK_HBM_GBS * 1e9)
        if t_h > t_m:
            ach = nbytes[dom] / t / 1e9
            out["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(ach / PEAK_HBM_GBS, 4)}
        else:
            ach = flops[dom] / t / 1e12
            out["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    del sh
    return out


def time_routed_workload(key, steps, warmup, dev):
    """The whole block fwd+bwd on another routed workload (gathered rows, as
    the headline step): ms per step, tokens/s and the six grouped GEMMs'
    fraction of the bf16 peak from their per-launch event times."""
    import numpy as np
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd import inputs as I
    from mixture_experts_layer_03_amd.layer import MoEBlock
    w = I.BY_KEY[key]
    a = I.make_inputs(w)

    def up(v, bf=True):
        if v is None:
            return None
        if bf:
            return torch.from_numpy(I.bf16_bits(v).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)

    x, wr, wgu, wd, dy = (up(a[n]) for n in ("x", "w_r", "w_gu", "w_down", "dy"))
    bias, noise = up(a["bias"], False), up(a["noise"], False)
    del a
    blk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev, gather=True)

    def step():
        blk.forward(x, wr, wgu, wd, bias, noise)
        blk.backward(x, wr, wgu, wd, dy)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    abi.moe_timing_reset()
    abi.moe_timing_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    abi.moe_timing_enable(False)
    flops = gemm_flops(w.R, w.d, w.f)
    us = {}
    for n in flops:
        for kn in (n, n + "_gather"):
            ms, cnt = abi.moe_timing_query(kn)
            if cnt:
                us[n] = 1e3 * ms / cnt
    abi.moe_timing_reset()
    out = {"workload": w.name, "ms_per_step": round(el * 1e3 / steps, 4),
           "tokens_per_s": round(w.T * steps / el, 1),
           "grouped_gemm_us": {n: round(v, 1) for n, v in us.items()}}
    if us:
        tot = sum(flops[n] for n in us) / (sum(us.values()) * 1e-6) / 1e12
        out["grouped_gemm_tflops"] = round(tot, 1)
        out["grouped_gemm_frac_of_bf16_peak"] = round(tot / PEAK_BF16_TFLOPS, 4)
    del blk
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--profile-steps", type=int, default=5,
                    help="extra steps with per-kernel event timing")
    ap.add_argument("--lora-rank", type=int, default=16,
                    help="also time the step with frozen experts and rank-r LoRA (0: skip)")
    ap.add_argument("--rows", choices=("gathered", "stored"), default="gathered",
                    help="token rows of the timed step: gathered by the GEMMs (X_perm kept "
                         "for dW_gate_up) or stored X_perm / dY_perm")
    ap.add_argument("--no-row-paths", action="store_true",
                    help="skip timing the other row arrangements")
    ap.add_argument("--other-workloads", default="c3,c5",
                    help="routed workloads also timed (whole step, fewer steps), '' for none")
    ap.add_argument("--no-ep-share", action="store_true",
                    help="skip timing the expert-parallel rank's share (grouped FFN alone)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (reference for HBM "
                         "byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mixture_experts_layer_03_amd import abi
    from mixture_experts_layer_03_amd import inputs as I
    from mixture_experts_layer_03_amd.layer import MoEBlock

    w = I.BY_KEY[args.workload]
    if w.routing == "prerouted":
        print("pick a routed workload (c2, c3, c5)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating inputs for %s" % w.name, file=sys.stderr, flush=True)
    a = I.make_inputs(w)

    def up(v, bf=True):
        if v is None:
            return None
        if bf:
            return torch.from_numpy(I.bf16_bits(v).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)

    x, wr, wgu, wd, dy = (up(a[n]) for n in ("x", "w_r", "w_gu", "w_down", "dy"))
    bias, noise = up(a["bias"], False), up(a["noise"], False)
    blk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev,
                   gather=args.rows == "gathered")
    stream = torch.cuda.current_stream()

    def step():
        blk.forward(x, wr, wgu, wd, bias, noise)
        blk.backward(x, wr, wgu, wd, dy)

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T * args.steps / elapsed

    # per-kernel durations: events around each launch, on the launch stream
    kernels = {}
    if args.profile_steps > 0:
        abi.moe_timing_reset()
        abi.moe_timing_enable(True)
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        abi.moe_timing_enable(False)
        names = ["router_logits", "route_topk", "permute_hist", "permute_scan", "permute_place",
                 "permute_rows", "tile_prefix", "gg_fwd_gate_up_swiglu", "gg_fwd_down_scale",
                 "gg_fwd_gate_up_swiglu_gather", "combine", "combine_bwd", "gg_bwd_dh_dswiglu",
                 "gg_bwd_dh_dswiglu_gather", "drs_reduce", "gg_bwd_dx",
                 "row_scale", "gg_bwd_dw_down", "gg_bwd_dw_gate_up", "gg_bwd_dw_gate_up_gather",
                 "route_bwd", "router_dx",
                 "router_dw_partial", "router_dw_reduce", "permute_bwd"]
        for n in names:
            ms, cnt = abi.moe_timing_query(n)
            if cnt:
                kernels[n] = {"ms_total": ms, "launches": cnt}
        for n, v in kernels.items():
            v["avg_us"] = 1e3 * v["ms_total"] / max(1, v["launches"])
        abi.moe_timing_reset()

    # router variants (selection-only bias, load statistics, its balancing
    # step, the auxiliary loss with its gradient) on the last step's logits;
    # timed apart from the block step, which the workload runs without them
    variants = {}
    if args.profile_steps > 0:
        sel_bias = torch.zeros(w.E, dtype=torch.float32, device=dev)
        vb = {"route_topk_biased": w.T * w.E * 4 + w.E * 4 + w.R * 8,
              "expert_load": w.R * 4 + w.E * 4, "bias_update": w.E * 12,
              "aux_loss": w.T * w.E * 12 + w.E * 4}
        def variant_calls():
            abi.moe_route_biased(blk.logits, sel_bias, w.k, blk.topk_idx, blk.topk_w)
            abi.moe_expert_load(blk.topk_idx, w.T, w.E, blk.load, blk.ws)
            abi.moe_aux_loss(blk.logits, blk.load, w.T, w.k, 1e-3, blk.aux, blk.d_logits, blk.ws)
            abi.moe_bias_update(blk.load, w.T, w.k, 1e-3, sel_bias)

        for _ in range(2):              # first launches of these kernels: untimed
            variant_calls()
        torch.cuda.synchronize()
        abi.moe_timing_reset()
        abi.moe_timing_enable(True)
        for _ in range(max(args.profile_steps, 10)):
            variant_calls()
        torch.cuda.synchronize()
        abi.moe_timing_enable(False)
        launches = {"route_topk_biased": ["route_topk_biased"],
                    "expert_load": ["expert_load", "expert_load_reduce"],
                    "bias_update": ["bias_update"],
                    "aux_loss": ["aux_loss", "aux_loss_colsum", "aux_loss_final"]}
        for n in vb:
            us = 0.0
            for ln in launches[n]:
                ms, cnt = abi.moe_timing_query(ln)
                us += 1e3 * ms / max(1, cnt)
            if us > 0:
                variants[n] = {"avg_us_per_call": round(us, 2), "algorithmic_bytes": vb[n],
                               "hbm_frac": round(vb[n] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        abi.moe_timing_reset()

    # the same step with the experts frozen and rank-r LoRA factors on both
    # expert matrices (grouped LoRA): the expert weight gradients are replaced
    # by the LoRA factor gradients
    lora_out = None
    if args.lora_rank > 0:
        lf = I.make_lora_factors(w, args.lora_rank)
        lora = tuple(up(lf[n]) for n in ("a_gu", "b_gu", "a_dn", "b_dn"))
        lblk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev,
                        lora_rank=args.lora_rank, lora_scale=1.0)

        def lstep():
            lblk.forward(x, wr, wgu, wd, bias, noise, lora=lora)
            lblk.backward(x, wr, wgu, wd, dy, lora=lora)

        for _ in range(max(2, args.warmup)):
            lstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            lstep()
        torch.cuda.synchronize()
        lel = time.perf_counter() - t0
        lk = {}
        if args.profile_steps > 0:
            abi.moe_timing_reset()
            abi.moe_timing_enable(True)
            for _ in range(args.profile_steps):
                lstep()
            torch.cuda.synchronize()
            abi.moe_timing_enable(False)
            for n in ("lora_proj", "lora_transpose", "lora_grad", "gg_fwd_gate_up_swiglu",
                      "gg_fwd_down_scale", "gg_bwd_dh_dswiglu", "gg_bwd_dx"):
                ms, cnt = abi.moe_timing_query(n)
                if cnt:
                    lk[n] = round(1e3 * ms / args.profile_steps, 1)
            abi.moe_timing_reset()
        lora_out = {"rank": args.lora_rank, "ms_per_step": round(lel * 1e3 / args.steps, 4),
                    "tokens_per_s": round(w.T * args.steps / lel, 1),
                    "speedup_vs_full_step": round(elapsed / lel, 3),
                    "kernels_us_per_step": lk}
        del lblk

    # the same step with the other arrangements of the token rows: all stored
    # (X_perm, dY_perm), gathered with X_perm kept for dW_gate_up, and
    # gathered everywhere (X_perm never stored)
    row_paths = None
    if not args.no_row_paths:
        row_paths = {("gathered" if args.rows == "gathered" else "stored"):
                     {"ms_per_step": round(ms_per_step, 4)}}
        for name, kw in (("stored", {"gather": False}), ("gathered", {"gather": True}),
                         ("gathered_no_x_perm", {"gather": True, "store_x_perm": False})):
            if name in row_paths:
                continue
            gblk = MoEBlock(w.T, w.d, w.E, w.k, w.f, dtype=torch.bfloat16, device=dev, **kw)

            def gstep():
                gblk.forward(x, wr, wgu, wd, bias, noise)
                gblk.backward(x, wr, wgu, wd, dy)

            for _ in range(max(2, args.warmup)):
                gstep()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                gstep()
            torch.cuda.synchronize()
            gel = time.perf_counter() - t0
            row_paths[name] = {"ms_per_step": round(gel * 1e3 / args.steps, 4)}
            del gblk

    others = {}
    for key in [k for k in args.other_workloads.split(",") if k and k != args.workload]:
        print("bench: workload %s" % key, file=sys.stderr, flush=True)
        others[key] = time_routed_workload(key, max(3, args.steps // 4), 2, dev)

    ep_share = None
    if not args.no_ep_share:
        print("bench: expert-parallel rank share", file=sys.stderr, flush=True)
        ep_share = time_ep_share(args.steps, max(2, args.warmup), dev)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    R = w.R
    flops = gemm_flops(R, w.d, w.f)
    # a gathered GEMM does the algorithmic work of its stored-row counterpart;
    # its gathered operand's bytes are the unpermuted token rows'
    gemm_us, launch_name = {}, {}
    for n in flops:
        for kn in (n, n + "_gather"):
            if kn in kernels:
                gemm_us[n] = kernels[kn]["avg_us"]
                launch_name[n] = kn
    stored_b, gathered_b = gemm_bytes(R, w.d, w.f, w.E), gemm_bytes(R, w.d, w.f, w.E, T=w.T)
    nbytes = {n: (gathered_b if launch_name[n].endswith("_gather") else stored_b)[n]
              for n in gemm_us}
    roofline = None
    gemm_frac = None
    gemm_roof_frac = None
    if gemm_us:
        # a GEMM's roofline time is the larger of its MFMA time and its HBM
        # time at peak; the bound is whichever that is
        t_mfma = {n: flops[n] / (PEAK_BF16_TFLOPS * 1e12) for n in gemm_us}
        t_hbm = {n: nbytes[n] / (PEAK_HBM_GBS * 1e9) for n in gemm_us}
        dom = max(gemm_us, key=gemm_us.get)
        t = gemm_us[dom] * 1e-6
        if t_hbm[dom] > t_mfma[dom]:
            achieved = nbytes[dom] / t / 1e9
            roofline = {"bound": "hbm", "kernel": launch_name[dom], "achieved": round(achieved, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(launch_name[dom], w.name),
                        "avg_launch_us": round(gemm_us[dom], 1),
                        "algorithmic_bytes_per_launch": nbytes[dom],
                        "algorithmic_flop_per_launch": flops[dom]}
        else:
            achieved = flops[dom] / t / 1e12
            roofline = {"bound": "mfma", "kernel": launch_name[dom], "achieved": round(achieved, 1),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                        "traffic": measured_traffic(launch_name[dom], w.name),
                        "avg_launch_us": round(gemm_us[dom], 1),
                        "algorithmic_flop_per_launch": flops[dom],
                        "algorithmic_bytes_per_launch": nbytes[dom]}
        tot_f = sum(flops[n] for n in gemm_us)
        tot_t = sum(gemm_us[n] for n in gemm_us) * 1e-6
        gemm_frac = tot_f / tot_t / 1e12 / PEAK_BF16_TFLOPS
        gemm_roof_frac = sum(max(t_mfma[n], t_hbm[n]) for n in gemm_us) / tot_t

    # row kernels (permute, combine and their adjoints, S) against HBM, and the
    # layer's roofline fraction: the summed roofline times of the GEMMs and
    # row kernels over the measured step
    rows_out, layer_roof_frac = {}, None
    rb = row_bytes(w.T, w.d, w.E, w.k)
    for n, b in rb.items():
        if n in kernels:
            us = kernels[n]["avg_us"]
            gbs = b / (us * 1e-6) / 1e9
            rows_out[n] = {"avg_us": round(us, 1), "algorithmic_bytes": b,
                           "GB_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    # context for the row kernels: a plain device copy (torch's) moving as
    # many bytes as the forward permute (half read, half written), timed per
    # launch with events like the library's kernels
    copy_out = None
    if "permute_rows" in rows_out:
        cb = int(rb["permute_rows"]) // 2 // 16 * 16
        csrc = torch.ones(cb // 4, dtype=torch.float32, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            cdst.copy_(csrc)
            e1.record()
        torch.cuda.synchronize()
        us = sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3 / len(evs)
        gbs = 2 * cb / (us * 1e-6) / 1e9
        copy_out = {"bytes": 2 * cb, "avg_us": round(us, 1), "GB_s": round(gbs, 1),
                    "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        del csrc, cdst
        # and a plain fill (torch's) of the bytes the scatters write (the R
        # routed rows): they write four bytes per byte read, so the write
        # rate bounds them, not the balanced copy's
        fb = 2 * w.R * w.d // 16 * 16
        fdst = torch.empty(fb // 4, dtype=torch.float32, device=dev)
        for _ in range(3):
            fdst.fill_(1.0)
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            fdst.fill_(1.0)
            e1.record()
        torch.cuda.synchronize()
        us = sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3 / len(evs)
        gbs = fb / (us * 1e-6) / 1e9
        copy_out["fill_of_written_bytes"] = {"bytes": fb, "avg_us": round(us, 1),
                                             "GB_s": round(gbs, 1),
                                             "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        del fdst
    if gemm_us:
        roof = sum(max(t_mfma[n], t_hbm[n]) for n in gemm_us)
        roof += sum(rb[n] / (PEAK_HBM_GBS * 1e9) for n in rows_out)
        layer_roof_frac = roof / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, a, min(args.cpu_sample_tokens, w.T))

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "d_model": w.d, "experts": w.E,
                   "top_k": w.k, "d_ff": w.f, "routed_rows": R, "passes": "fwd+bwd",
                   "rows": args.rows},
        "grouped_gemm_frac_of_bf16_peak": None if gemm_frac is None else round(gemm_frac, 4),
        "grouped_gemm_roofline_frac": None if gemm_roof_frac is None else round(gemm_roof_frac, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_us": {n: round(v["avg_us"], 1) for n, v in kernels.items()},
        "row_kernels": rows_out,
        "device_copy_same_bytes": copy_out,
        "layer_roofline_frac": None if layer_roof_frac is None else round(layer_roof_frac, 4),
        "router_variants": variants,
        "lora": lora_out,
        "rows": args.rows,
        "row_paths": row_paths,
        "ep_share": ep_share,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
