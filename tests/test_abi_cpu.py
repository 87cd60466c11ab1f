"""CPU-side checks of the C-ABI library: it loads, exports every entry point
include/gpt2.h declares, and its host-only logic (the planner and config
validation) behaves as documented.  No GPU call is made here."""
import os
import re
import subprocess

import pytest

from transformer_lm_train_amd import gpt2 as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    lib = G.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gpt2_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_binding_covers_the_abi():
    for n in declared_functions():
        if n in ("gpt2_last_error", "gpt2_device_params", "gpt2_device_grads", "gpt2_device_shadow"):
            continue
        assert hasattr(G, n), n


def _cfg(**kw):
    base = dict(L=12, C=768, NH=12, maxT=1024, V=50257, Vp=50304, B=16, T=1024, precision=G.GPT2_BF16_MIXED,
                fused=False, recompute=False, recompute_ln=False)
    base.update(kw)
    return G.make_config(base["L"], base["C"], base["NH"], base["maxT"], base["V"], base["Vp"], base["B"],
                         base["T"], base["precision"], base["fused"], base["recompute"], base["recompute_ln"])


def test_plan_sizes():
    n = 124475904
    size = G.gpt2_plan(_cfg())
    # params + grads + m + v (fp32) + bf16 shadow at least
    assert size >= 18 * n
    # activations of 12 layers at B*T = 16384 in bf16 are a few GB, well under 288 GB
    assert size < 16 * 2**30
    fp32 = G.gpt2_plan(_cfg(B=4, T=64, precision=G.GPT2_FP32))
    assert fp32 >= 16 * n
    tiny = G.gpt2_plan(G.make_config(2, 64, 4, 32, 512, 512, 4, 32, G.GPT2_FP32))
    assert tiny >= 16 * 134912


@pytest.mark.parametrize("kw,msg", [
    (dict(C=770), "num_heads"),
    (dict(T=2048), "seq_len"),
    (dict(V=50305), "vocab_size"),
    (dict(precision=7), "precision"),
    (dict(NH=6), "head size 64"),             # bf16 mode needs hs = 64
    (dict(B=1, T=63), "multiples of 64"),     # bf16 mode needs T % 64 == 0
    (dict(B=64, T=33), "multiples of 64"),    # even when B*T is one
    (dict(L=0), "positive"),
])
def test_plan_rejects_bad_configs(kw, msg):
    with pytest.raises(G.GPT2Error) as e:
        G.gpt2_plan(_cfg(**kw))
    assert e.value.code == G.GPT2_EINVAL
    assert msg in str(e.value)


def test_plan_stochastic_rounding_mode():
    # the bf16-parameter mode drops the fp32 copy of every matrix (wte, wpe,
    # qkvw, attprojw, fcw, fcprojw): 4 bytes per parameter outside the
    # LayerNorm and bias tensors, and checks the same shape rules
    L, C, n = 12, 768, 124475904
    small = 2 * L * C + 3 * L * C + L * C + 2 * L * C + 4 * L * C + L * C + 2 * C
    saved = G.gpt2_plan(_cfg()) - G.gpt2_plan(_cfg(precision=G.GPT2_BF16_SR))
    assert abs(saved - 4 * (n - small)) <= 256
    with pytest.raises(G.GPT2Error) as e:
        G.gpt2_plan(_cfg(NH=6, precision=G.GPT2_BF16_SR))
    assert e.value.code == G.GPT2_EINVAL and "head size 64" in str(e.value)


def test_plan_fused_classifier():
    # no B*T x Vp logits: one 4096-row chunk of dlogits plus 8 bytes per row
    # and 64-column group of softmax statistics and 8 per row of target logit
    # and log-sum-exp; the chunk's backward-data product may split its
    # reduction into at most 4 fp32 partial tiles of 4096 x 768 (the workspace
    # grows by at most that), and the classifier leaves the weight-gradient
    # tile list (a few KB)
    BT, Vp, C = 16 * 1024, 50304, 768
    stats = 8 * BT * (Vp // 64) + 8 * BT
    saved = G.gpt2_plan(_cfg()) - G.gpt2_plan(_cfg(fused=True))
    expect = 2 * BT * Vp - 2 * 4096 * Vp - stats
    assert expect - 4 * 4096 * C * 4 <= saved <= expect + 8192
    with pytest.raises(G.GPT2Error) as e:
        G.gpt2_plan(_cfg(B=4, T=64, precision=G.GPT2_FP32, fused=True))
    assert e.value.code == G.GPT2_EINVAL and "bf16" in str(e.value)


def test_plan_recompute_gelu():
    # one layer's GELU output instead of L: (L - 1) * B*T * 4C bf16 values fewer
    # (the grouped weight-gradient tile list loses the fcproj tiles, a few KB)
    L, C, BT = 12, 768, 16 * 1024
    saved = G.gpt2_plan(_cfg()) - G.gpt2_plan(_cfg(recompute=True))
    expect = (L - 1) * BT * 4 * C * 2
    assert expect <= saved <= expect + 65536
    bad = _cfg()
    bad.recompute_gelu = 2
    for cfg, msg in ((_cfg(B=4, T=64, precision=G.GPT2_FP32, recompute=True), "bf16"), (bad, "recompute_gelu")):
        with pytest.raises(G.GPT2Error) as e:
            G.gpt2_plan(cfg)
        assert e.value.code == G.GPT2_EINVAL and msg in str(e.value)


def test_plan_recompute_layernorm():
    # one layer's LN1 and LN2 outputs instead of L: 2 (L - 1) * B*T * C bf16 values
    # fewer (the grouped tile list loses the qkv and fc tiles, a few KB)
    L, C, BT = 12, 768, 16 * 1024
    saved = G.gpt2_plan(_cfg()) - G.gpt2_plan(_cfg(recompute_ln=True))
    expect = 2 * (L - 1) * BT * C * 2
    assert expect <= saved <= expect + 65536
    both = G.gpt2_plan(_cfg()) - G.gpt2_plan(_cfg(recompute=True, recompute_ln=True))
    assert expect + (L - 1) * BT * 4 * C * 2 <= both <= expect + (L - 1) * BT * 4 * C * 2 + 131072
    bad = _cfg()
    bad.recompute_layernorm = 3
    for cfg, msg in ((_cfg(B=4, T=64, precision=G.GPT2_FP32, recompute_ln=True), "bf16"),
                     (bad, "recompute_layernorm")):
        with pytest.raises(G.GPT2Error) as e:
            G.gpt2_plan(cfg)
        assert e.value.code == G.GPT2_EINVAL and msg in str(e.value)
