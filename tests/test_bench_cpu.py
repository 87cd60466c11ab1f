"""The benchmark's host-side contract (no GPU): it refuses more than one GPU
with a message and exit status 2, and its algorithmic work per step is the
step's FLOP count: 3 * [L(24 C^2 + 2 C (T + 1)) + 2 C V] per token (linears,
causal QK^T and PV, the classifier over the real vocabulary; the backward
twice the forward), the figures the pages' GPT-2 shapes give (124M at
T = 1024: 797,870,592 per token, 13.07 TFLOP per B=16 step)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,per_token", [("124m", 797_870_592), ("350m", 2_271_860_736),
                                            ("1.6b", 9_802_147_200)])
def test_flops_per_token(name, per_token):
    c = bench.CONFIGS[name]
    assert bench.flops_per_token(c) == per_token


def test_class_work_adds_up_to_the_step():
    c = bench.CONFIGS["124m"]
    w = bench.class_work(c)
    flops = sum(a for a, unit, _ in w.values() if unit == "flop")
    step = bench.flops_per_token(c) * c["B"] * c["T"]
    assert step == 13_072_311_779_328
    # every FLOP of the step sits in exactly one timed class
    assert flops == step
    # the memory-bound classes: AdamW 30 bytes per parameter, softmax CE reads and writes the bf16 logits
    n = 124_475_904
    assert w["adamw"][0] == 30 * n
    assert w["softmax_ce"][0] == 2 * 2 * c["B"] * c["T"] * c["Vp"]
