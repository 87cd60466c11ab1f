"""The stochastic-rounding mode (GPT2_BF16_SR) through the C ABI against the
oracle ("llm.c's Origin and the Future of LLM Compilers", section "Avengers":
stochastic rounding).

* One AdamW step, then a second, from seeded host state (bf16 parameters,
  gradients written into the model's gradient region): m and v to fp32
  rounding; every new parameter a bf16 value equal to the oracle's rounding
  decision wherever that decision is unique.  The kernel computes the update
  in fp32 with its own operation order (and a hardware reciprocal), so its
  fp32 value x may differ from the oracle's by a few ulps of the larger of
  |theta| and |update| (many ulps of x itself when the two nearly cancel).
  Rounding is monotone in x for a fixed draw, so the admissible outcomes are
  the bf16 values between the roundings of x -+ 16 such ulps; where those
  differ (under 1e-3 of the elements) either is accepted.
* Training steps of a small model: losses within the bf16 tolerance of the
  oracle running the same mode, parameters bf16 values throughout, and
  bitwise reproducible from run to run.
"""
import numpy as np
import pytest

from oracle import oracle as O
from transformer_lm_train_amd import gpt2 as G
from transformer_lm_train_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SR_CFG = dict(L=2, C=128, NH=2, maxT=128, V=1000, Vp=1024)


def _cfg(B, T, prec=G.GPT2_BF16_SR):
    d = SR_CFG
    return G.make_config(d["L"], d["C"], d["NH"], d["maxT"], d["V"], d["Vp"], B, T, prec)


def _ocfg():
    d = SR_CFG
    return O.Config(L=d["L"], C=d["C"], NH=d["NH"], maxT=d["maxT"], V=d["V"], Vp=d["Vp"])


def _write(m, dev_ptr, host):
    """Copy a float32 host array to a device address inside the model's buffer."""
    off = dev_ptr - m.buf.data_ptr()
    assert 0 <= off and off + 4 * host.size <= m.nbytes
    m.buf[off: off + 4 * host.size].view(torch.float32).copy_(torch.from_numpy(host))
    torch.cuda.synchronize()


def _admissible(x64, scale, u, k=16):
    """Lowest and highest rounding, under draws u, of the fp32 values within
    k ulps of scale around the fp64 result x64."""
    d = k * np.spacing(np.abs(scale).astype(np.float32)).astype(np.float64)
    lo = O.sr_bf16((x64 - d).astype(np.float32), u)
    hi = O.sr_bf16((x64 + d).astype(np.float32), u)
    return lo, hi


def test_sr_adamw_steps_vs_oracle():
    seed = 11
    m = G.Model(_cfg(2, 64), seed)
    n = G.gpt2_num_params(m.h)
    rng = np.random.default_rng(5)
    p = O.bf16_rne((rng.standard_normal(n) * 0.02).astype(np.float32))
    p[rng.integers(0, n, 1000)] = 0.0
    m.set_params(p)
    assert np.array_equal(m.params(), p)
    om, ov = np.zeros(n, np.float32), np.zeros(n, np.float32)
    op = p.copy()
    hp = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    skip = np.zeros(n, bool)  # elements whose earlier step took the other admissible outcome
    for t in (1, 2):
        print(f"SR AdamW step t={t} n={n}", flush=True)
        g = (rng.standard_normal(n) * 0.01 * rng.choice([0.01, 1.0, 30.0], n)).astype(np.float32)
        _write(m, G.lib().gpt2_device_grads(m.h), g)
        m.adamw_step(hp["lr"], hp["b1"], hp["b2"], hp["eps"], hp["wd"], t)
        got = m.params()
        gm, gv = m.opt_state()
        # the oracle's update and the fp64 value it rounds
        th = op.astype(np.float64)
        pr, mr, vr = th.copy(), om.astype(np.float64), ov.astype(np.float64)
        # fp32 error bounds of m and v: a few ulps of their two terms (m's
        # terms can cancel, so not of m itself); the ABI takes the betas as
        # fp32, and 1 - 0.95f alone is 2.4e-7 off 0.05
        g64 = g.astype(np.float64)
        tol_m = 1e-6 * (hp["b1"] * np.abs(mr) + (1 - hp["b1"]) * np.abs(g64)) + 1e-30
        tol_v = 1e-6 * (hp["b2"] * vr + (1 - hp["b2"]) * g64 * g64) + 1e-30
        O.adamw_update(pr, g.astype(np.float64), mr, vr, t=t, prec="f64", **hp)
        u = O.sr_draws(seed, t, 0, n)
        O.adamw_sr_update(op, g, om, ov, t=t, seed=seed, **hp)
        assert np.array_equal(op, O.sr_bf16(pr.astype(np.float32), u))
        step = th - pr
        lo, hi = _admissible(pr, np.maximum(np.abs(th), np.abs(step)), u)
        amb = lo != hi
        live = ~skip
        assert amb.mean() < 3e-3, amb.mean()
        assert np.all((got.view(np.uint32) & 0xFFFF) == 0), "parameters must be bf16 values"
        ok = (got >= lo) & (got <= hi)
        assert np.all(ok[live]), [(i, th[i], pr[i], got[i], lo[i], hi[i]) for i in np.flatnonzero(live & ~ok)[:5]]
        same = got == op
        assert np.all(same[live & ~amb]), np.flatnonzero(live & ~amb & ~same)[:10]
        assert np.all(np.abs(gm - mr) <= tol_m), np.max(np.abs(gm - mr) / tol_m)
        assert np.all(np.abs(gv - vr) <= tol_v), np.max(np.abs(gv - vr) / tol_v)
        skip |= ~same
    m.close()


def _train(gpu, steps, seed=3, B=4, T=64):
    hp = (1e-4, 0.9, 0.999, 1e-8, 0.1)
    d = SR_CFG
    x, y = synth.batch(seed, 0, B, T, d["V"], "zipf")
    if gpu:
        m = G.Model(_cfg(B, T), seed)
        losses = []
        for t in range(1, steps + 1):
            losses.append(m.forward(x, y))
            m.zero_grad()
            m.backward()
            m.clip_grad_norm(1.0)
            m.adamw_step(*hp, t)
        out = (losses, m.params())
        m.close()
        return out
    m = O.Model(_ocfg(), B, T)
    m.init(seed)
    m.params[:] = O.bf16_rne(m.params)  # the bf16 parameters the mode starts from
    losses = []
    for t in range(1, steps + 1):
        losses.append(m.forward(x, y))
        m.zero_grad()
        m.backward()
        m.clip_grad_norm(1.0)
        m.adamw_sr(*hp, t, seed)
    return losses, m.params.copy()


def test_sr_training_vs_oracle_and_reproducible():
    steps = 6
    print("SR training: oracle", flush=True)
    ol, op = _train(False, steps)
    print("SR training: GPU twice", flush=True)
    gl, gp = _train(True, steps)
    gl2, gp2 = _train(True, steps)
    assert gl == gl2 and np.array_equal(gp, gp2), "SR mode must be bitwise reproducible"
    for a, b in zip(gl, ol):
        assert abs(a - b) <= 1e-2, (gl, ol)
    assert gl[-1] < gl[0] - 0.05, gl
    assert np.all((gp.view(np.uint32) & 0xFFFF) == 0)
    # the two sides round different fp32 values (bf16 activations against
    # fp32), so individual parameters differ by bf16 steps; the whole
    # parameter vector stays close
    rel = np.linalg.norm(gp.astype(np.float64) - op) / np.linalg.norm(op)
    assert rel < 1e-2, rel


def test_sr_initial_parameters_are_the_rounded_init():
    m = G.Model(_cfg(2, 64), 21)
    p = m.params()
    m.close()
    want = O.bf16_rne(O.init_params(_ocfg(), 21))
    assert np.array_equal(p, want)
