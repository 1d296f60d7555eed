#!/usr/bin/env python3
"""Benchmark: GPT-2 124M bf16 forward + next-token cross-entropy on one MI355X.

One step = one gpt_forward call over one [B, T] batch of synthetic token ids
(uniform in [0, V)) with seeded N(0, 0.02) weights, inputs resident in HBM:
embedding, 12 pre-norm blocks, ln_f, tied head (bf16 logits written) and the
fused cross-entropy.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3|4] [--no-cpu-baseline]

The roofline object reports the tied head + cross-entropy kernel (the
largest single launch, 29% of the step's FLOPs) from hipEvents recorded
around its launch inside every timed step.  cpu_baseline times the fp64
oracle on one sequence of the same workload on the host cores.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0


def flops_per_step(cfg, B, T):
    """Algorithmic FLOPs: 2MNK for c_attn, c_proj, c_fc, mlp.c_proj and the tied
    head, plus causal attention 4*D*B*H*T(T+1)/2 (the masked half excluded)."""
    M, C, F, V, L, H = B * T, cfg.n_embd, cfg.n_ff, cfg.vocab, cfg.n_layer, cfg.n_head
    D = C // H
    gemm = 2 * M * C * (3 * C + C + F + F) * L
    head = 2 * M * V * C
    attn = 4 * D * B * H * T * (T + 1) // 2 * L
    return gemm + head + attn, head


def cpu_baseline(cfg, params, ids, n_seq):
    """Time the fp64 oracle on the first n_seq sequences (bounded sample)."""
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        ctx = None
    from decoder_only_transformer_attn_amd import synth
    from oracle import gpt_oracle as O
    P = synth.unpack_f64(cfg, params)
    t0 = time.perf_counter()
    O.forward(P, ids[:n_seq], cfg.n_head, cfg.ln_eps, want_logits=True)
    dt = time.perf_counter() - t0
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    toks = n_seq * ids.shape[1]
    return {"value": round(toks / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {ids.shape[0]} sequences x {ids.shape[1]} tokens, fp64 numpy forward + logits "
                      f"+ loss, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(sequences shard data-parallel across GPUs by design, not implemented here)"}))
        sys.exit(2)

    import torch
    from decoder_only_transformer_attn_amd import lib, synth

    lib.load()
    w = synth.WORKLOADS[args.workload]
    cfg, B, T = w["cfg"], w["B"], w["T"]
    want_logits = args.workload == 3
    params = synth.make_params(cfg, seed=42, cfg_id=args.workload)
    ids = synth.make_ids(cfg, B, T, seed=42, cfg_id=args.workload)
    dev_params = lib.params_to_device(cfg, synth.pack(cfg, params))
    idx = torch.from_numpy(ids).cuda()
    fwd = lib.Forward(cfg, B, T, want_logits=want_logits)
    stream = torch.cuda.current_stream()

    ev = lib.HipEvents(2 * args.steps + 2)
    for _ in range(args.warmup):
        fwd(dev_params, idx)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    hip = ev.hip
    hip.hipEventRecord.argtypes = [lib.ctypes.c_void_p, lib.ctypes.c_void_p]
    hip.hipEventRecord(ev.ev[-2], stream.cuda_stream)
    for s in range(args.steps):
        lib.forward_timed(cfg, dev_params, idx, None, fwd.logits, fwd.token_loss, fwd.mean_loss, fwd.ws,
                          ev.ev[2 * s], ev.ev[2 * s + 1], "head")
    hip.hipEventRecord(ev.ev[-1], stream.cuda_stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = ev.elapsed_ms(len(ev.ev) - 2, len(ev.ev) - 1)
    head_ms = float(np.mean([ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(args.steps)]))
    ev.close()
    loss = float(fwd.mean_loss.item())

    ms = total_ms / args.steps
    tokens = B * T
    flops, head_flops = flops_per_step(cfg, B, T)
    achieved = head_flops / (head_ms * 1e-3) / 1e12
    out = {
        "metric": "tokens/s fwd+loss, GPT-2 124M bf16 B=8 T=1024; % of MFMA peak",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w["name"], "global_batch": B, "seq_len": T, "parallelism": "single-gpu",
                   "logits_written": want_logits},
        "mfma_frac_end_to_end": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "tflops_end_to_end": round(flops / (ms * 1e-3) / 1e12, 1),
        "loss": round(loss, 5),
        "wall_s_timed": round(t_wall, 3),
        "roofline": {"bound": "mfma", "kernel": "head_ce_kernel (tied head GEMM + CE partials)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(head_ms, 4), "flops_per_launch": head_flops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, ids, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
