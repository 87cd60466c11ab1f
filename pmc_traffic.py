"""Per-kernel-class reductions of rocprofv3 runs of bench.py (measurement
harness; not part of the library).

Subcommands:

  copy      A plain 1 GiB device-to-device copy: the calibration workload.
            Run it under `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE`;
            the counter values of its copy dispatches against the known
            1 GiB give the factor that turns each counter into bytes.

  summary   RUN_DIR OUT_MD [CONFIG]
            For every kernel class of the training step (the classes bench.py
            times): launches and time per step from a `--kernel-trace` run
            (RUN_DIR/trace), MFMA busy (the MfmaUtil metric), VALU busy and
            the transcendental / all-VALU instruction counts (RUN_DIR/mfma,
            RUN_DIR/valu), and HBM bytes per launch (RUN_DIR/fetch and
            RUN_DIR/write, scaled by the copies in RUN_DIR/cal_FETCH_SIZE and
            RUN_DIR/cal_WRITE_SIZE), next to each class's algorithmic work
            from bench.class_work.  Writes the table to OUT_MD and every
            class's bytes per launch to profiles/traffic.json, keyed by the
            sha256 of the kernel sources, so that bench.py reports a class's
            traffic only while its kernels are the ones the counters saw.

The counter runs are `rocprofv3 --pmc <set> --output-format csv -d RUN_DIR/<name>
-o run -- python3 bench.py --steps 2 --warmup 1 --timing-class gemm_fwd
--no-cpu-baseline`, one counter set per run.
"""
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
CSRC = os.path.join("transformer_lm_train_amd", "csrc")
# the bench configuration the recorded entries are taken on (bench.py's default)
RECORDED_CONFIG = "124m"


def kernel_sources():
    d = os.path.join(ROOT, CSRC)
    return [os.path.join(CSRC, f) for f in sorted(os.listdir(d)) if f.endswith((".hip", ".h"))]


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(p.encode() + b"\0" + f.read())
    return h.hexdigest()


def _rows(d):
    with open(os.path.join(d, "run_counter_collection.csv")) as f:
        return list(csv.DictReader(f))


def _calibration(d):
    vals = [float(r["Counter_Value"]) for r in _rows(d) if "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy dispatch in {d}")
    kib = sum(vals) / len(vals)
    return COPY_BYTES / (kib * 1024.0), kib


def recorded(cls, config=RECORDED_CONFIG):
    """HBM bytes per launch recorded for cls, or None when absent, when the
    kernel sources have changed since the counters were taken, or for another
    model configuration than the one they were taken on."""
    if config != RECORDED_CONFIG:
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            e = json.load(f)[cls]
        if e.get("config") != config or sources_digest(e["sources"]) != e["sources_sha256"]:
            return None
        return e["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def copy():
    import torch
    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes 3 times", flush=True)


# ---- kernel classes -----------------------------------------------------------
def _gemm_class(name):
    """Class of a gemm_big_kernel dispatch from its template arguments (BM, BN,
    waves, waves along M, k-step, stages, prefetch, A k-contiguous,
    B k-contiguous, epilogue, occupancy, valid width, grouped)."""
    args = [a.strip() for a in name.split("gemm_big_kernel<", 1)[1].split(">", 1)[0].split(",")]
    a_k, b_k, epi, grouped = args[7] == "true", args[8] == "true", int(args[9]), args[12] == "true"
    if grouped:
        return "gemm_dw"
    if a_k and b_k:
        return "gemm_classifier_fwd" if epi == 0 else "gemm_fwd"
    if a_k and not b_k:
        return "gemm_dx"
    return "gemm_other"


def classify(names):
    """Kernel class of each dispatch of a run, in dispatch order.  The
    classifier's backward-data product runs the same kernel as the linears'
    (a 192-wide NN store); it is the first such dispatch after the loss."""
    out, after_loss = [], False
    for n in names:
        if "gemm_big_kernel" in n:
            c = _gemm_class(n)
            if c == "gemm_dx" and after_loss and ", 0, 2, 192" in n:
                c = "gemm_classifier_dx"
                after_loss = False
        elif "grouped_fixup" in n:
            c = "gemm_dw"
        elif "flash_fwd" in n:
            c = "attention_fwd"
        elif "flash_bwd" in n:
            c = "attention_bwd"
        elif "softmax_ce" in n:
            c = "softmax_ce"
        elif "loss_mean" in n:
            c, after_loss = "loss_mean", True
        elif "adamw" in n:
            c = "adamw"
        elif "layernorm_fwd" in n:
            c = "layernorm_fwd"
        elif "layernorm_bwd" in n:
            c = "layernorm_bwd"
        elif "sumsq" in n or "norm_final" in n:
            c = "grad_norm"
        elif "sum_partials" in n:
            c = "bias_sums"
        elif "enc_" in n or "encoder_" in n or "fill_i32" in n:
            c = "encoder"
        else:
            c = "other"
        out.append(c)
    return out


def _dispatches(d):
    """Counter rows of a run grouped by dispatch, in dispatch order:
    [(kernel name, {counter: value}, duration ns)]."""
    disp = {}
    for r in _rows(d):
        k = int(r["Dispatch_Id"])
        e = disp.setdefault(k, [r["Kernel_Name"], {}, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        e[1][r["Counter_Name"]] = float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _per_class(disp):
    agg = {}
    for (name, ctr, ns), c in zip(disp, classify([d[0] for d in disp])):
        a = agg.setdefault(c, {"n": 0, "ns": 0, "ctr": {}, "wctr": {}})
        a["n"] += 1
        a["ns"] += ns
        for k, v in ctr.items():
            a["ctr"][k] = a["ctr"].get(k, 0.0) + v
            a["wctr"][k] = a["wctr"].get(k, 0.0) + v * ns  # duration-weighted, for percentages
    return agg


# ---- algorithmic HBM bytes per launch of the compute-bound classes ------------
def _nparams(c):
    C = c["C"]
    return c["Vp"] * C + c["maxT"] * C + c["L"] * (12 * C * C + 13 * C) + 2 * C


def _alg_linears_fwd(c):
    """Mean over the four forward linears: X, W (and the residual) read once,
    the output(s) written once, bf16 (fc writes the pre-activation and GELU)."""
    BT, C = c["B"] * c["T"], c["C"]
    qkv = 2 * (BT * C + 3 * C * C + 3 * BT * C)
    att = 2 * (BT * C + C * C + 2 * BT * C)
    fc = 2 * (BT * C + 4 * C * C + 2 * 4 * BT * C)
    fcp = 2 * (4 * BT * C + 4 * C * C + 2 * BT * C)
    return (qkv + att + fc + fcp) / 4


def _alg_linears_dx(c):
    """Mean over the four backward-data products: dY and W read, dX written
    (the fcproj product also reads the pre-activation for GELU')."""
    BT, C = c["B"] * c["T"], c["C"]
    fcp = 2 * (BT * C + 4 * C * C + 2 * 4 * BT * C)
    fc = 2 * (4 * BT * C + 4 * C * C + BT * C)
    att = 2 * (BT * C + C * C + BT * C)
    qkv = 2 * (3 * BT * C + 3 * C * C + BT * C)
    return (fcp + fc + att + qkv) / 4


def _alg_dw(c):
    """The grouped weight-gradient launch: each product's two bf16 operands read
    once and its fp32 gradient written once."""
    BT, C, L, Vp = c["B"] * c["T"], c["C"], c["L"], c["Vp"]
    per_layer = 2 * BT * (C + 4 * C) * 2 + 2 * BT * (C + C) + 2 * BT * (3 * C + C) + 4 * 12 * C * C
    return L * per_layer + 2 * BT * (Vp + C) + 4 * Vp * C


def _alg_classifier(c):
    BT, C, Vp = c["B"] * c["T"], c["C"], c["Vp"]
    return 2 * (BT * C + Vp * C + BT * Vp)


ALG_BYTES = {
    "gemm_fwd": _alg_linears_fwd,
    "gemm_dx": _alg_linears_dx,
    "gemm_dw": _alg_dw,
    "gemm_classifier_fwd": _alg_classifier,
    "gemm_classifier_dx": _alg_classifier,
    # per launch: q, k, v read and the output written (forward); q, k, v, dO, O
    # read and dq, dk, dv written over the backward's two kernels
    "attention_fwd": lambda c: 2 * c["B"] * c["T"] * c["C"] * 4,
    "attention_bwd": lambda c: 2 * c["B"] * c["T"] * c["C"] * 8 / 2,
    # sumsq reads the fp32 gradient once (the finishing kernel is negligible)
    "grad_norm": lambda c: 4 * _nparams(c) / 2,
}


def summary(run, out_md, config=RECORDED_CONFIG):
    sys.path.insert(0, ROOT)
    import bench
    c = bench.CONFIGS[config]
    work = bench.class_work(c)
    with open(os.path.join(run, "trace", "run_kernel_trace.csv")) as f:
        trace = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    tcls = classify([r["Kernel_Name"] for r in trace])
    steps = sum(1 for x in tcls if x == "adamw")
    tt = {}
    for r, k in zip(trace, tcls):
        e = tt.setdefault(k, [0, 0])
        e[0] += 1
        e[1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    mf = _per_class(_dispatches(os.path.join(run, "mfma")))
    va = _per_class(_dispatches(os.path.join(run, "valu")))
    fe = _per_class(_dispatches(os.path.join(run, "fetch")))
    wr = _per_class(_dispatches(os.path.join(run, "write")))
    ff, fkib = _calibration(os.path.join(run, "cal_FETCH_SIZE"))
    wf, wkib = _calibration(os.path.join(run, "cal_WRITE_SIZE"))
    total_ms = sum(v[1] for v in tt.values()) / 1e6 / steps
    lines = [
        f"Trace run: {steps} steps, {total_ms:.2f} ms of kernel time per step. Counter runs: one counter set "
        f"per run (the profiler serialises kernels). HBM bytes: FETCH_SIZE x {ff:.3f} and WRITE_SIZE x {wf:.3f} "
        f"(a 1 GiB device copy reads FETCH_SIZE {fkib:.0f} KiB and WRITE_SIZE {wkib:.0f} KiB). MFMA and VALU busy "
        "are duration-weighted means over the class's dispatches.",
        "",
        "| class | launches/step | ms/step | µs/launch | algorithmic work/launch | achieved | of peak | MFMA busy | "
        "VALU busy | TRANS f32 insts/launch | VALU insts/launch | HBM bytes/launch (read + write) | "
        "HBM bytes / algorithmic bytes |",
        "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|",
    ]
    # counter runs: steps from their AdamW dispatches
    csteps = {id(a): a.get("adamw", {"n": 1})["n"] for a in (mf, va, fe, wr)}
    traffic = {}
    for k in sorted(tt, key=lambda k: -tt[k][1]):
        n, ns = tt[k]
        # a class's launches per step: its products (bench.class_work; the
        # weight gradients' fix-up kernel counts as part of its launch), else
        # its dispatches
        lps = work[k][2] if k in work else n / steps
        us = ns / steps / lps / 1e3
        row = [k, f"{lps:g}" if k in work else f"{lps:.1f}", f"{ns / 1e6 / steps:.3f}", f"{us:.1f}"]
        per_launch = unit = None
        if k in work:
            amount, unit, launches = work[k]
            per_launch = amount / launches
            if unit == "flop":
                ach = per_launch / (us * 1e-6) / 1e12
                row += [f"{per_launch / 1e9:.2f} GFLOP", f"{ach:.0f} TFLOP/s", f"{ach / bench.PEAK_BF16_TFLOPS:.3f}"]
            else:
                ach = per_launch / (us * 1e-6) / 1e9
                row += [f"{per_launch / 1e6:.1f} MB", f"{ach:.0f} GB/s", f"{ach / bench.PEAK_HBM_GBS:.3f}"]
        else:
            row += ["", "", ""]

        def pct(agg, ctr):
            a = agg.get(k)
            return f"{a['wctr'][ctr] / a['ns']:.1f}%" if a and ctr in a["wctr"] and a["ns"] else ""

        def per(agg, ctr, scale=1.0):
            a = agg.get(k)
            return a["ctr"][ctr] * scale / (csteps[id(agg)] * lps) if a and ctr in a["ctr"] else None

        row += [pct(mf, "MfmaUtil"), pct(va, "VALUBusy")]
        t, v = per(va, "SQ_INSTS_VALU_TRANS_F32"), per(va, "SQ_INSTS_VALU")
        row += [f"{t:.3g}" if t is not None else "", f"{v:.3g}" if v is not None else ""]
        fb, wb = per(fe, "FETCH_SIZE", 1024.0 * ff), per(wr, "WRITE_SIZE", 1024.0 * wf)
        if fb is not None and wb is not None:
            row.append(f"{(fb + wb) / 1e6:.1f} ({fb / 1e6:.1f} + {wb / 1e6:.1f}) MB")
            traffic[k] = (fb, wb, fe[k]["n"])
            alg = per_launch if unit == "byte" else (ALG_BYTES[k](c) if k in ALG_BYTES else None)
            row.append(f"{(fb + wb) / alg:.2f}" if alg else "")
        else:
            row += ["", ""]
        lines.append("| " + " | ".join(row) + " |")
    # the kernels themselves, from the trace run's statistics
    with open(os.path.join(run, "trace", "run_kernel_stats.csv")) as f:
        stats = sorted(csv.DictReader(f), key=lambda r: -float(r["TotalDurationNs"]))
    lines += ["", f"Kernels of the trace run (per step: the run's {steps} steps):", "",
              "| ms/step | calls/step | avg µs | kernel |", "|---:|---:|---:|---|"]
    for r in stats:
        ms = float(r["TotalDurationNs"]) / 1e6 / steps
        if ms < 0.005:
            continue
        name = r["Name"].replace("(anonymous namespace)::", "").split("(GemmArgs")[0]
        lines.append(f"| {ms:.3f} | {int(r['Calls']) / steps:.1f} | {float(r['AverageNs']) / 1e3:.1f} | `{name[:110]}` |")
    # a header written by hand above the generated table (title, commands) is kept
    head = []
    if os.path.exists(out_md):
        with open(out_md) as f:
            for ln in f:
                if ln.startswith("Trace run:"):
                    break
                head.append(ln)
    with open(out_md, "w") as f:
        f.write("".join(head) + "\n".join(lines) + "\n")
    srcs = kernel_sources()
    data = {}
    for k, (fb, wb, n) in traffic.items():
        data[k] = {"bytes_per_launch": round(fb + wb), "fetch_bytes_per_launch": round(fb),
                   "write_bytes_per_launch": round(wb), "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                   "calibration": f"1 GiB device copy: FETCH_SIZE {fkib:.0f} KiB, WRITE_SIZE {wkib:.0f} KiB",
                   "dispatches_profiled": n, "config": config,
                   "sources": srcs, "sources_sha256": sources_digest(srcs)}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 4 and sys.argv[1] == "summary":
        summary(sys.argv[2], sys.argv[3], *sys.argv[4:5])
    elif len(sys.argv) >= 2 and sys.argv[1] == "copy":
        copy()
    else:
        print(__doc__)
        sys.exit(2)
