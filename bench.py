"""Training-step benchmark: GPT-2 124M, bf16 mixed precision, B=16, T=1024,
one MI355X.

A step is the whole hot path on one fresh batch of seeded Zipf(1.1) tokens
already resident in HBM: forward (embedding, 12 blocks, tied classifier,
fused softmax cross-entropy, loss read back to the host), zero_grad,
backward, global-norm clip (1.0) and AdamW (lr 6e-4, betas 0.9/0.999,
eps 1e-8, wd 0.1).  W untimed warmup steps, then K timed steps between
stream synchronisations, timed with HIP events on the library's stream.

--host-tokens hands the batch over as host arrays instead (the PCIe copy of
the ids inside the step; its line names that in the metric).

Prints one JSON line: tokens/s (value), MFU against the bf16 dense MFMA peak
(and under the 6N + 12*L*C*T FLOPs-per-token convention),
the roofline of the dominant kernel class (timed live with HIP events around
each of its launches inside the timed region), the roofline of every class
(one step each before the timed region) and the CPU oracle timed on bounded
samples of the same model.
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


def class_work(c, sr=False, fused=False, recompute=False, recompute_ln=False):
    """Algorithmic work per step of each timed kernel class: (amount, unit,
    launches per step).  With the fused classifier the logits are recomputed
    in the backward (a class of its own, counted at the classifier's FLOPs)
    in chunks of up to 4096 rows, each with its dX and dwte products, and the
    loss pass only combines the per-row statistics.  With the GELU recompute
    each layer's GELU output is formed again in the backward (read the bf16
    pre-activation, write the output) and the fcproj weight gradients run as
    one launch per layer beside the grouped launch; with the LayerNorm
    recompute each layer's two LayerNorm forwards run again (their bytes as in
    the forward) and the qkv and fc weight gradients run per layer."""
    L, C, T, V, B, NH = c["L"], c["C"], c["T"], c["V"], c["B"], c["NH"]
    BT = B * T
    lin = L * 2 * BT * 12 * C * C
    att = L * 2 * C * (T + 1) * BT  # causal QK^T + PV forward
    N = c["Vp"] * C + c["maxT"] * C + L * (12 * C * C + 13 * C) + 2 * C
    Vp = c["Vp"]
    cls = 2 * BT * C * V
    if fused:
        chunks = -(-BT // 4096)
        head = {
            "gemm_classifier_fwd": (cls, "flop", 1),
            "gemm_classifier_recompute": (cls, "flop", chunks),
            "gemm_classifier_dx": (cls, "flop", chunks),
            "gemm_classifier_dw": (cls, "flop", chunks),
            "gemm_fwd": (lin, "flop", 4 * L),
            "gemm_dx": (lin, "flop", 4 * L),
            "gemm_dw": (lin, "flop", 1),
            "attention_fwd": (att, "flop", L),
            "attention_bwd": (2 * att, "flop", L),
            # read the (max, sum) pairs and the target logits, write loss and lse
            "softmax_ce": (8 * BT * (Vp // 64) + 4 * BT + 8 * BT, "byte", 1),
        }
    else:
        head = {
            "gemm_classifier_fwd": (cls, "flop", 1),
            "gemm_classifier_dx": (cls, "flop", 1),
            "gemm_fwd": (lin, "flop", 4 * L),
            "gemm_dx": (lin, "flop", 4 * L),
            # every weight gradient, the classifier's included, in one grouped launch
            "gemm_dw": (lin + cls, "flop", 1),
            "attention_fwd": (att, "flop", L),
            "attention_bwd": (2 * att, "flop", L),
            "softmax_ce": (2 * BT * Vp * 2, "byte", 1),
        }
    if recompute:
        amount, unit, n = head["gemm_dw"]
        head["gemm_dw"] = (amount, unit, n + L)
        head["gelu_recompute"] = (L * BT * 4 * C * 2 * 2, "byte", L)
    if recompute_ln:
        amount, unit, n = head["gemm_dw"]
        head["gemm_dw"] = (amount, unit, n + 2 * L)
        head["layernorm_recompute"] = (2 * L * (BT * C * 2 * 2 + 8 * BT), "byte", 2 * L)
    return {
        **head,
        # fp32 master: read theta, g, m, v, write theta, m, v, bf16 copy; stochastic
        # rounding: read bf16 theta, g, m, v, write bf16 theta, m, v
        "adamw": ((24 if sr else 30) * N, "byte", 1),
        "layernorm_fwd": ((2 * L + 1) * (BT * C * 2 * 2 + 8 * BT), "byte", 2 * L + 1),
        "layernorm_bwd": ((2 * L + 1) * (BT * C * 2 * 4 + 8 * BT), "byte", 2 * L + 1),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_s(c, B, T, seed, steps=1):
    """Seconds per fp32 oracle training step (forward, backward, clip 1.0,
    AdamW) of model c at B x T on Zipf(1.1) tokens."""
    from oracle import oracle as O
    from transformer_lm_train_amd import synth
    cfg = O.Config(L=c["L"], C=c["C"], NH=c["NH"], maxT=c["maxT"], V=c["V"], Vp=c["Vp"])
    m = O.Model(cfg, B, T)
    m.init(seed)
    x, y = synth.batch(seed, 0, B, T, c["V"], "zipf")
    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        m.forward(x, y)
        m.zero_grad()
        m.backward()
        m.clip_grad_norm(1.0)
        m.adamw(6e-4, 0.9, 0.999, 1e-8, 0.1, t)
    return (time.perf_counter() - t0) / steps


def cpu_baseline(c, seed):
    """The fp32 oracle on the host's cores, on bounded samples of the same
    model: one step at B=1 and the benchmark's T (the headline value, tokens
    per second), and the 124M-shape step at B=4, T=64 the pages time on a
    laptop CPU, at all cores and at one thread."""
    from oracle import oracle as O
    cores = O.num_threads()
    print(f"cpu baseline: oracle B=1 T={c['T']} on {cores} threads", flush=True)
    s1 = _oracle_step_s(c, 1, c["T"], seed)
    print(f"cpu baseline: oracle B=4 T=64, {cores} threads then 1", flush=True)
    s_all = _oracle_step_s(c, 4, 64, seed, steps=2)
    O.set_num_threads(1)
    try:
        s_one = _oracle_step_s(c, 4, 64, seed)
    finally:
        O.set_num_threads(cores)
    return {"value": round(c["T"] / s1, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one fp32 oracle training step (forward, backward, clip, AdamW) of the same model at B=1, "
                      f"T={c['T']} on Zipf(1.1) tokens: {s1:.2f} s, i.e. per-token throughput of a B=1 step "
                      f"(the B={c['B']} step would need ~{c['B']}x the activation memory)",
            "cpu_model": _cpu_model(),
            "B4_T64": {"s_per_step": round(s_all, 3), "tokens_per_s": round(256 / s_all, 1), "threads": cores},
            "B4_T64_one_thread": {"s_per_step": round(s_one, 3), "tokens_per_s": round(256 / s_one, 1),
                                  "threads": 1}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="124m", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=1337)
    ap.add_argument("--batch", type=int, default=0,
                    help="batch size in place of the configuration's (the line's metric names it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing-class", default="auto")
    ap.add_argument("--fused-classifier", action="store_true",
                    help="classifier product fused with the softmax cross-entropy: no logits stored, the backward "
                         "recomputes them in chunks")
    ap.add_argument("--recompute-gelu", action="store_true",
                    help="keep only the pre-activation of the MLP and form its GELU again in the backward "
                         "(less activation memory, one GELU pass per layer more)")
    ap.add_argument("--recompute-layernorm", action="store_true",
                    help="keep one layer's LayerNorm outputs and run each layer's LayerNorm forwards again in "
                         "the backward (less activation memory)")
    ap.add_argument("--host-tokens", action="store_true",
                    help="tokens and targets handed over as host arrays (gpt2_forward: the PCIe copy inside the "
                         "step) instead of device arrays already in HBM")
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

    c = dict(CONFIGS[args.config])
    if args.batch > 0:
        c["B"] = args.batch
    torch.cuda.set_device(0)
    prec = G.GPT2_BF16_SR if args.sr else G.GPT2_BF16_MIXED
    cfg = G.make_config(c["L"], c["C"], c["NH"], c["maxT"], c["V"], c["Vp"], c["B"], c["T"], prec,
                        args.fused_classifier, args.recompute_gelu, args.recompute_layernorm)
    m = G.Model(cfg, args.seed, device="cuda:0")
    B, T = c["B"], c["T"]
    nb = args.warmup + args.steps + 16
    toks, tgts = [], []
    for s in range(nb):
        x, y = synth.batch(args.seed, s, B, T, c["V"], "zipf")
        if args.host_tokens:
            toks.append(np.ascontiguousarray(x.reshape(-1), dtype=np.int32))
            tgts.append(np.ascontiguousarray(y.reshape(-1), dtype=np.int32))
        else:
            toks.append(torch.from_numpy(x.reshape(-1)).cuda())
            tgts.append(torch.from_numpy(y.reshape(-1)).cuda())
    torch.cuda.synchronize()
    hp = dict(lr=6e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    step_no = [0]

    def step(i):
        step_no[0] += 1
        if args.host_tokens:
            loss = m.forward(toks[i], tgts[i], read_loss=True)
        else:
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

    work = class_work(c, args.sr, args.fused_classifier, args.recompute_gelu, args.recompute_layernorm)
    per_class = {}
    # choose the dominant kernel class: one untimed-region step per class
    if args.timing_class == "auto":
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
    # the common convention: 6 FLOPs per parameter and token plus 12*L*C*T for attention
    n_params = c["Vp"] * c["C"] + c["maxT"] * c["C"] + c["L"] * (12 * c["C"] ** 2 + 13 * c["C"]) + 2 * c["C"]
    mfu_6n = tok_s * (6 * n_params + 12 * c["L"] * c["C"] * c["T"]) / (PEAK_BF16_TFLOPS * 1e12)
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
    import pmc_traffic
    # bytes per launch from the committed counter runs, if still current and of this configuration
    traffic = pmc_traffic.recorded(dom, args.config)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(avg_ms, 4)
    roof["launches"] = launches
    # every class's roofline, from its step of the class selection (HIP events
    # around each of its launches, outside the timed region)
    classes = {}
    for cls, ms in per_class.items():
        amount_c, unit_c, nl = work[cls]
        if ms <= 0:
            continue
        if unit_c == "flop":
            a = amount_c / (ms / 1e3) / 1e12
            classes[cls] = {"bound": "mfma", "ms_per_step": round(ms, 4), "achieved": round(a, 1), "unit": "TFLOP/s",
                            "frac": round(a / PEAK_BF16_TFLOPS, 4)}
        else:
            a = amount_c / (ms / 1e3) / 1e9
            classes[cls] = {"bound": "hbm", "ms_per_step": round(ms, 4), "achieved": round(a, 1), "unit": "GB/s",
                            "frac": round(a / PEAK_HBM_GBS, 4)}
        classes[cls]["launches_per_step"] = nl
        classes[cls]["traffic"] = pmc_traffic.recorded(cls, args.config)
    m.close()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(c, args.seed)

    out = {
        # the headline metric names the 124M workload; the other configurations
        # are named for what they run
        "metric": f"train tokens/s + MFU % for GPT-2 {args.config.upper()} bf16 B={B} T={T} on 1 MI355X"
                  + (", tokens from host memory" if args.host_tokens else ""),
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "mfu_pct": round(100 * mfu, 2),
        "mfu_6n_pct": round(100 * mfu_6n, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"GPT-2 {args.config} training step, "
                               + ("bf16 parameters with stochastic-rounding AdamW (fp32 m/v), " if args.sr else
                                  "bf16 mixed (fp32 master/AdamW), ")
                               + ("classifier fused with the softmax cross-entropy (logits recomputed in the "
                                  "backward), " if args.fused_classifier else "")
                               + ("GELU output recomputed in the backward, " if args.recompute_gelu else "")
                               + ("LayerNorm outputs recomputed in the backward, " if args.recompute_layernorm else "")
                               + "Zipf(1.1) synthetic tokens"
                               + (", tokens copied from host memory inside the step" if args.host_tokens else ""),
                   "batch": B, "seq_len": T,
                   "flop_per_token": fpt, "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_classes": classes,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
