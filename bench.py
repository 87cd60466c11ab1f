"""Training-step benchmark: GPT-2 124M, bf16 mixed precision, B=16, T=1024,
one MI355X.

A step is the whole hot path on one fresh batch of seeded Zipf(1.1) tokens
already resident in HBM: forward (embedding, 12 blocks, tied classifier,
fused softmax cross-entropy, loss read back to the host), zero_grad,
backward, global-norm clip (1.0) and AdamW (lr 6e-4, betas 0.9/0.999,
eps 1e-8, wd 0.1).  W untimed warmup steps, then K timed steps between
stream synchronisations, timed with HIP events on the library's stream.

Prints one JSON line: tokens/s (value), MFU against the bf16 dense MFMA peak,
the roofline of the dominant kernel class (timed live with HIP events around
each of its launches inside the timed region) and the CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

CONFIGS = {
    "124m": dict(L=12, C=768, NH=12, maxT=1024, V=50257, Vp=50304, B=16, T=1024),
    "350m": dict(L=24, C=1024, NH=16, maxT=1024, V=50257, Vp=50304, B=16, T=1024),
    "1.6b": dict(L=48, C=1600, NH=25, maxT=1024, V=50257, Vp=50304, B=8, T=1024),
}


def flops_per_token(c):
    """Algorithmic FLOPs per token of one training step: linears, causal
    QK^T and PV, classifier over the real vocabulary; backward = 2x forward."""
    L, C, T, V = c["L"], c["C"], c["T"], c["V"]
    return 3 * (L * (24 * C * C + 2 * C * (T + 1)) + 2 * C * V)


def class_work(c, sr=False):
    """Algorithmic work per step of each timed kernel class: (amount, unit)."""
    L, C, T, V, B, NH = c["L"], c["C"], c["T"], c["V"], c["B"], c["NH"]
    BT = B * T
    lin = L * 2 * BT * 12 * C * C
    att = L * 2 * C * (T + 1) * BT  # causal QK^T + PV forward
    N = c["Vp"] * C + c["maxT"] * C + L * (12 * C * C + 13 * C) + 2 * C
    Vp = c["Vp"]
    return {
        "gemm_classifier_fwd": (2 * BT * C * V, "flop", 1),
        "gemm_classifier_dx": (2 * BT * C * V, "flop", 1),
        "gemm_fwd": (lin, "flop", 4 * L),
        "gemm_dx": (lin, "flop", 4 * L),
        # every weight gradient, the classifier's included, in one grouped launch
        "gemm_dw": (lin + 2 * BT * C * V, "flop", 1),
        "attention_fwd": (att, "flop", L),
        "attention_bwd": (2 * att, "flop", L),
        "softmax_ce": (2 * BT * Vp * 2, "byte", 1),
        # fp32 master: read theta, g, m, v, write theta, m, v, bf16 copy; stochastic
        # rounding: read bf16 theta, g, m, v, write bf16 theta, m, v
        "adamw": ((24 if sr else 30) * N, "byte", 1),
        "layernorm_fwd": ((2 * L + 1) * (BT * C * 2 * 2 + 8 * BT), "byte", 2 * L + 1),
        "layernorm_bwd": ((2 * L + 1) * (BT * C * 2 * 4 + 8 * BT), "byte", 2 * L + 1),
    }


def cpu_baseline(c, sample_B, sample_T, seed):
    from oracle import oracle as O
    from transformer_lm_train_amd import synth
    cfg = O.Config(L=c["L"], C=c["C"], NH=c["NH"], maxT=c["maxT"], V=c["V"], Vp=c["Vp"])
    m = O.Model(cfg, sample_B, sample_T)
    m.init(seed)
    x, y = synth.batch(seed, 0, sample_B, sample_T, c["V"], "zipf")
    t0 = time.perf_counter()
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    m.clip_grad_norm(1.0)
    m.adamw(6e-4, 0.9, 0.999, 1e-8, 0.1, 1)
    dt = time.perf_counter() - t0
    return {"value": sample_B * sample_T / dt, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"one fp32 oracle training step (forward, backward, clip, AdamW) of the same model at "
                      f"B={sample_B}, T={sample_T} on Zipf(1.1) tokens: {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="124m", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=1337)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", default="4x512", help="BxT of the oracle sample")
    ap.add_argument("--timing-class", default="auto")
    ap.add_argument("--sr", action="store_true",
                    help="bf16 parameters updated by stochastic rounding (no fp32 master) instead of fp32 masters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_train_amd import gpt2 as G
    from transformer_lm_train_amd import synth

    c = CONFIGS[args.config]
    torch.cuda.set_device(0)
    prec = G.GPT2_BF16_SR if args.sr else G.GPT2_BF16_MIXED
    cfg = G.make_config(c["L"], c["C"], c["NH"], c["maxT"], c["V"], c["Vp"], c["B"], c["T"], prec)
    m = G.Model(cfg, args.seed, device="cuda:0")
    B, T = c["B"], c["T"]
    nb = args.warmup + args.steps + 16
    toks, tgts = [], []
    for s in range(nb):
        x, y = synth.batch(args.seed, s, B, T, c["V"], "zipf")
        toks.append(torch.from_numpy(x.reshape(-1)).cuda())
        tgts.append(torch.from_numpy(y.reshape(-1)).cuda())
    torch.cuda.synchronize()
    hp = dict(lr=6e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    step_no = [0]

    def step(i):
        step_no[0] += 1
        loss = m.forward_device(toks[i], tgts[i], read_loss=True)
        m.zero_grad()
        m.backward()
        m.clip_grad_norm(1.0, read_norm=False)
        m.adamw_step(t=step_no[0], **hp)
        return loss

    print(f"bench: {args.config} bf16 B={B} T={T} warmup {args.warmup} steps {args.steps}", flush=True)
    for i in range(args.warmup):
        loss = step(i)
        print(f"warmup step {i} loss {loss:.4f}", flush=True)

    work = class_work(c, args.sr)
    # choose the dominant kernel class: one untimed-region step per class
    if args.timing_class == "auto":
        per_class = {}
        for k, cls in enumerate(work):
            G.gpt2_kernel_timing_enable(m.h, cls, True)
            step(args.warmup + k % 8)
            n, ms = G.gpt2_kernel_timing_read(m.h)
            per_class[cls] = ms
        G.gpt2_kernel_timing_enable(m.h, "", False)
        dom = max(per_class, key=per_class.get)
        print("per-class ms/step: " + ", ".join(f"{k} {v:.3f}" for k, v in per_class.items()), flush=True)
    else:
        dom = args.timing_class

    stream = torch.cuda.current_stream()
    G.gpt2_kernel_timing_enable(m.h, dom, True)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    losses = []
    for i in range(args.steps):
        losses.append(step(args.warmup + 8 + i))
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    launches, kms = G.gpt2_kernel_timing_read(m.h)
    G.gpt2_kernel_timing_enable(m.h, "", False)
    print(f"timed {args.steps} steps: {total_ms:.1f} ms; losses {losses[0]:.4f} -> {losses[-1]:.4f}", flush=True)

    ms_step = total_ms / args.steps
    tok_s = B * T * args.steps / (total_ms / 1e3)
    fpt = flops_per_token(c)
    mfu = tok_s * fpt / (PEAK_BF16_TFLOPS * 1e12)
    amount, unit, per_step_launches = work[dom]
    avg_ms = kms / max(launches, 1)
    per_launch = amount / per_step_launches
    if unit == "flop":
        achieved = per_launch / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    from transformer_lm_train_amd import pmc_traffic
    # bytes per launch from the committed counter runs, if still current and of this configuration
    traffic = pmc_traffic.recorded(dom, args.config)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(avg_ms, 4)
    roof["launches"] = launches
    m.close()

    cpu = None
    if not args.no_cpu_baseline:
        sb, st = (int(v) for v in args.cpu_sample.split("x"))
        print(f"cpu baseline: oracle B={sb} T={st}", flush=True)
        cpu = cpu_baseline(c, sb, st, args.seed)

    out = {
        "metric": "train tokens/s + MFU % for GPT-2 124M bf16 B=16 T=1024 on 1 MI355X",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "mfu_pct": round(100 * mfu, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"GPT-2 {args.config} training step, "
                               + ("bf16 parameters with stochastic-rounding AdamW (fp32 m/v), " if args.sr else
                                  "bf16 mixed (fp32 master/AdamW), ")
                               + "Zipf(1.1) synthetic tokens", "batch": B, "seq_len": T,
                   "flop_per_token": fpt, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
