"""HBM traffic of a kernel class from rocprofv3 counter dumps.

Two subcommands:

  copy      a plain 1 GiB device-to-device copy: the calibration workload.
            Run it under `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE`;
            the counter values of its copy dispatches against the known
            1 GiB give the factor that turns each counter into bytes.

  reduce    CLASS LAUNCHES FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR
            SOURCES PATTERN [PATTERN ...]
            Sums FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over the
            dispatches whose kernel name contains one of the patterns, scales
            each by its calibration factor, divides by LAUNCHES (the number
            of launches of the class in the profiled run) and records the
            bytes per launch in profiles/traffic.json under CLASS, with the
            sha256 of the comma-separated SOURCES files (paths relative to
            the repository root) so that a reader can tell whether the
            kernels have changed since.
"""
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


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


def _class_kib(d, patterns):
    tot, n = 0.0, 0
    for r in _rows(d):
        if any(p in r["Kernel_Name"] for p in patterns):
            tot += float(r["Counter_Value"])
            n += 1
    return tot, n


def reduce(cls, launches, fetch_dir, write_dir, cal_fetch, cal_write, sources, patterns):
    ff, fkib = _calibration(cal_fetch)
    wf, wkib = _calibration(cal_write)
    fsum, fn = _class_kib(fetch_dir, patterns)
    wsum, wn = _class_kib(write_dir, patterns)
    per_launch = (fsum * 1024.0 * ff + wsum * 1024.0 * wf) / launches
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data[cls] = {
        "bytes_per_launch": round(per_launch),
        "fetch_bytes_per_launch": round(fsum * 1024.0 * ff / launches),
        "write_bytes_per_launch": round(wsum * 1024.0 * wf / launches),
        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
        "calibration": f"1 GiB device copy: FETCH_SIZE {fkib:.0f} KiB, WRITE_SIZE {wkib:.0f} KiB",
        "dispatches": {"fetch": fn, "write": wn}, "launches": launches, "kernels": patterns,
        "sources": sources, "sources_sha256": sources_digest(sources),
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[cls]))


# the bench configuration every recorded entry was taken on (the counter runs
# use bench.py's default: GPT-2 124M, B=16, T=1024)
RECORDED_CONFIG = "124m"


def recorded(cls, config=RECORDED_CONFIG):
    """Bytes per launch recorded for cls, or None when absent, when the
    kernel sources have changed since the counters were taken, or for another
    model configuration than the one they were taken on."""
    if config != RECORDED_CONFIG:
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            e = json.load(f)[cls]
        if sources_digest(e["sources"]) != e["sources_sha256"]:
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


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "copy":
        copy()
    elif len(sys.argv) >= 10 and sys.argv[1] == "reduce":
        reduce(sys.argv[2], int(sys.argv[3]), sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7],
               sys.argv[8].split(","), sys.argv[9:])
    else:
        print(__doc__)
        sys.exit(2)
