"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  Each one checks the oracle against
something other than itself: numbers the pages print (tests/golden), closed
forms, invariants, special cases that reduce to a textbook or numpy routine,
and central finite differences of the fp64 build for every backward.
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from transformer_lm_train_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = O.Config(L=2, C=64, NH=4, maxT=32, V=512, Vp=512)
GPT2_124M = O.Config(L=12, C=768, NH=12, maxT=1024, V=50257, Vp=50304)


def read_golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            vals[k] = int(v)
    return vals


# ----------------------------------------------------------- printed numbers
def test_printed_counts_124m():
    g = read_golden("gpt2_124m_printed.txt")
    cfg = O.Config(L=g["num_layers"], C=g["channels"], NH=g["num_heads"], maxT=g["max_seq_len"],
                   V=g["vocab_size"], Vp=g["padded_vocab_size"])
    n = O.num_params(cfg)
    assert n == g["num_parameters"]
    assert O.num_acts(cfg, g["batch_size"], g["seq_len"]) == g["num_activations"]
    assert 4 * n + g["header_bytes"] == g["file_bytes_fp32"]
    assert 2 * n + g["header_bytes"] == g["file_bytes_bf16"]


def test_param_layout_alternatives_do_not_match():
    """Untied classifier or unpadded wte would miss the printed N."""
    g = read_golden("gpt2_124m_printed.txt")
    sizes = O.param_sizes(GPT2_124M)
    assert sizes[0] == g["padded_vocab_size"] * g["channels"]
    assert sum(sizes) + g["vocab_size"] * g["channels"] != g["num_parameters"]
    assert sum(sizes) - (g["padded_vocab_size"] - g["vocab_size"]) * g["channels"] != g["num_parameters"]


# ----------------------------------------------------------- SplitMix64
def test_splitmix64_published_vectors():
    # First outputs of SplitMix64 seeded with 0 (Steele, Lea & Flood 2014
    # reference generator; the widely used test vectors).
    w = synth.splitmix64(0, np.arange(1, 4, dtype=np.uint64))
    assert [int(x) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_token_streams():
    u = synth.uniforms(7, 0, 200000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.005
    ids = synth.token_stream(1337, 0, 400000, 50257, "zipf")
    # P(id 0) under Zipf(1.1) over 50257 ids: 1 / H where H = sum (k+1)^-1.1
    H = np.sum(np.arange(1, 50258, dtype=np.float64) ** -1.1)
    p0 = (ids == 0).mean()
    assert abs(p0 - 1 / H) < 0.003
    assert ids.min() >= 0 and ids.max() < 50257
    x, y = synth.batch(3, 5, 4, 16, 512, "uniform")
    assert np.array_equal(x.reshape(-1)[1:], y.reshape(-1)[:-1])


# ----------------------------------------------------------- init
def test_init_distribution():
    cfg = O.Config(L=4, C=128, NH=4, maxT=64, V=1000, Vp=1024)
    P = dict(zip(O.PARAM_NAMES, np.split(O.init_params(cfg, 42), np.cumsum(O.param_sizes(cfg))[:-1])))
    from scipy import stats
    for name, sd in (("wte", 0.02), ("wpe", 0.02), ("qkvw", 0.02), ("fcw", 0.02),
                     ("attprojw", 0.02 / math.sqrt(8)), ("fcprojw", 0.02 / math.sqrt(8))):
        x = P[name].astype(np.float64)
        if name == "wte":
            assert np.all(P["wte"][1000 * 128:] == 0)  # padded rows
            x = x[:1000 * 128]
        n = x.size
        assert abs(x.mean()) < 5 * sd / math.sqrt(n)
        assert abs(x.std() / sd - 1) < 5 / math.sqrt(2 * n)
        assert stats.kstest(x / sd, "norm").pvalue > 1e-4
    for name in ("ln1w", "ln2w", "lnfw"):
        assert np.all(P[name] == 1)
    for name in ("ln1b", "ln2b", "lnfb", "qkvb", "attprojb", "fcb", "fcprojb"):
        assert np.all(P[name] == 0)
    # counter-based: the value at a flat index does not depend on anything else
    a = O.init_params(cfg, 42)
    b = O.init_params(cfg, 43)
    assert np.array_equal(a, O.init_params(cfg, 42)) and not np.array_equal(a, b)


# ----------------------------------------------------------- layer pins
def test_encoder_is_gather_plus_position():
    rng = np.random.default_rng(0)
    wte = rng.standard_normal((50, 8)).astype(np.float32)
    wpe = rng.standard_normal((6, 8)).astype(np.float32)
    tok = rng.integers(0, 50, (3, 6)).astype(np.int32)
    out = O.encoder_forward(tok, wte, wpe)
    np.testing.assert_array_equal(out, wte[tok] + wpe[None, :, :])
    dwte = np.zeros_like(wte)
    dwpe = np.zeros_like(wpe)
    dout = rng.standard_normal((3, 6, 8)).astype(np.float32)
    O.encoder_backward(dwte, dwpe, dout, tok)
    ref = np.zeros((50, 8))
    np.add.at(ref, tok.reshape(-1), dout.reshape(-1, 8).astype(np.float64))
    np.testing.assert_allclose(dwte, ref, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(dwpe, dout.sum(0), rtol=1e-5, atol=1e-6)
    unseen = np.setdiff1d(np.arange(50), tok)
    assert np.all(dwte[unseen] == 0)


def test_layernorm_closed_form():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((37, 96)) * 3 + 1.5).astype(np.float64)
    out, mean, rstd = O.layernorm_forward(x, np.ones(96), np.zeros(96), prec="f64")
    var = x.var(axis=1)
    np.testing.assert_allclose(mean, x.mean(1), rtol=1e-12)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var + 1e-5), rtol=1e-12)
    np.testing.assert_allclose(out.mean(1), 0, atol=1e-12)
    np.testing.assert_allclose(out.var(1), var / (var + 1e-5), rtol=1e-10)
    w = rng.standard_normal(96)
    b = rng.standard_normal(96)
    out2, _, _ = O.layernorm_forward(x, w, b, prec="f64")
    np.testing.assert_allclose(out2, out * w + b, rtol=1e-12, atol=1e-12)


def test_matmul_is_numpy_matmul():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((19, 24))
    w = rng.standard_normal((13, 24))
    b = rng.standard_normal(13)
    np.testing.assert_allclose(O.matmul_forward(x, w, b, prec="f64"), x @ w.T + b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.matmul_forward(x, w, None, prec="f64"), x @ w.T, rtol=1e-12, atol=1e-12)
    dout = rng.standard_normal((19, 13))
    dx, dw, db = O.matmul_backward(dout, x, w, prec="f64")
    np.testing.assert_allclose(dx, dout @ w, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, dout.T @ x, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db, dout.sum(0), rtol=1e-12, atol=1e-12)


def _qkv(rng, B, T, C):
    return rng.standard_normal((B, T, 3 * C))


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    B, T, C, NH = 2, 7, 12, 3
    hs = C // NH
    qkv = _qkv(rng, B, T, C)
    out, pre, att = O.attention_forward(qkv, NH, prec="f64")
    v = qkv[:, :, 2 * C:]
    # position 0 sees only itself
    np.testing.assert_allclose(out[:, 0], v[:, 0], rtol=1e-12)
    # rows are distributions over t2 <= t, zero above the diagonal
    np.testing.assert_allclose(att.sum(-1), 1, rtol=1e-12)
    assert np.all(att[..., np.triu_indices(T, 1)[0], np.triu_indices(T, 1)[1]] == 0)
    # q = 0: uniform weights over the prefix, so out_t = mean of v_0..v_t
    q0 = qkv.copy()
    q0[:, :, :C] = 0
    out0, _, _ = O.attention_forward(q0, NH, prec="f64")
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    np.testing.assert_allclose(out0, prefix_mean, rtol=1e-12, atol=1e-12)
    # two keys: att[1,0] = 1 / (1 + exp((q1.k1 - q1.k0) / sqrt(hs))) for each head
    for h in range(NH):
        q1 = qkv[0, 1, h * hs:(h + 1) * hs]
        k0 = qkv[0, 0, C + h * hs:C + (h + 1) * hs]
        k1 = qkv[0, 1, C + h * hs:C + (h + 1) * hs]
        a10 = 1 / (1 + math.exp((q1 @ k1 - q1 @ k0) / math.sqrt(hs)))
        assert abs(att[0, h, 1, 0] - a10) < 1e-12
    # T = 1: output is v
    o1, _, _ = O.attention_forward(qkv[:, :1], NH, prec="f64")
    np.testing.assert_allclose(o1, v[:, :1], rtol=1e-12)
    # future positions do not influence the past
    qkv2 = qkv.copy()
    qkv2[:, 5:] = rng.standard_normal(qkv2[:, 5:].shape)
    out2, _, _ = O.attention_forward(qkv2, NH, prec="f64")
    np.testing.assert_array_equal(out2[:, :5], out[:, :5])


def test_gelu_special_values():
    u = np.array([0.0, 30.0, -30.0, 1.0, -1.0])
    g = O.gelu_forward(u, prec="f64")
    assert g[0] == 0
    assert abs(g[1] - 30) < 1e-12 and abs(g[2]) < 1e-12
    # the tanh form tracks the exact erf form u*Phi(u) closely
    from scipy.special import erf
    x = np.linspace(-6, 6, 2001)
    exact = 0.5 * x * (1 + erf(x / math.sqrt(2)))
    assert np.max(np.abs(O.gelu_forward(x, prec="f64") - exact)) < 1e-3
    d = O.gelu_backward(np.array([0.0, 30.0, -30.0]), np.ones(3), prec="f64")
    np.testing.assert_allclose(d, [0.5, 1.0, 0.0], atol=1e-12)


def test_softmax_ce_closed_forms():
    V, Vp, N = 500, 512, 6
    rng = np.random.default_rng(4)
    # uniform logits over the real vocabulary: loss = ln V exactly, whatever
    # the padded columns hold
    z = np.zeros((N, Vp))
    z[:, V:] = 100.0
    tgt = rng.integers(0, V, N).astype(np.int32)
    loss, probs = O.softmax_ce_forward(z, tgt, V, prec="f64")
    np.testing.assert_allclose(loss, math.log(V), rtol=1e-14)
    assert np.all(probs[:, V:] == 0)
    z = rng.standard_normal((N, Vp)) * 4
    loss, probs = O.softmax_ce_forward(z, tgt, V, prec="f64")
    np.testing.assert_allclose(probs.sum(1), 1, rtol=1e-13)
    assert np.all(probs >= 0)
    np.testing.assert_allclose(loss, -np.log(probs[np.arange(N), tgt]), rtol=1e-12)
    # scipy's logsumexp over the real columns
    from scipy.special import logsumexp
    np.testing.assert_allclose(loss, logsumexp(z[:, :V], axis=1) - z[np.arange(N), tgt], rtol=1e-12)
    d = O.softmax_ce_backward(probs, tgt, np.full(N, 0.25), V, prec="f64")
    onehot = np.zeros((N, Vp))
    onehot[np.arange(N), tgt] = 1
    np.testing.assert_allclose(d[:, :V], 0.25 * (probs - onehot)[:, :V], rtol=1e-13, atol=1e-16)
    assert np.all(d[:, V:] == 0)
    np.testing.assert_allclose(d.sum(1), 0, atol=1e-14)


# ----------------------------------------------------------- finite differences
def _fd_check(f, x, grad, idx, h=1e-5, rtol=1e-6, atol_frac=1e-7):
    """Central differences of scalar f at entries idx of array x vs grad."""
    scale = max(np.max(np.abs(grad)), 1e-30)
    for i in idx:
        old = x.flat[i]
        x.flat[i] = old + h
        fp = f()
        x.flat[i] = old - h
        fm = f()
        x.flat[i] = old
        fd = (fp - fm) / (2 * h)
        an = grad.flat[i]
        assert abs(fd - an) <= rtol * abs(an) + atol_frac * scale + 1e-12, (i, fd, an)


def test_layer_backwards_fd():
    rng = np.random.default_rng(5)
    # layernorm
    N, C = 5, 16
    x = rng.standard_normal((N, C))
    w = rng.standard_normal(C)
    b = rng.standard_normal(C)
    r = rng.standard_normal((N, C))
    _, mean, rstd = O.layernorm_forward(x, w, b, prec="f64")
    dx, dw, db = O.layernorm_backward(r, x, w, mean, rstd, prec="f64")
    f = lambda: float(np.sum(O.layernorm_forward(x, w, b, prec="f64")[0] * r))
    _fd_check(f, x, dx, range(x.size))
    _fd_check(f, w, dw, range(w.size))
    _fd_check(f, b, db, range(b.size))
    # attention
    B, T, C, NH = 2, 6, 12, 3
    qkv = rng.standard_normal((B, T, 3 * C))
    r = rng.standard_normal((B, T, C))
    _, _, att = O.attention_forward(qkv, NH, prec="f64")
    dq = O.attention_backward(r, qkv, att, NH, prec="f64")
    f = lambda: float(np.sum(O.attention_forward(qkv, NH, prec="f64")[0] * r))
    _fd_check(f, qkv, dq, range(qkv.size))
    # gelu
    u = rng.standard_normal(40) * 3
    r = rng.standard_normal(40)
    du = O.gelu_backward(u, r, prec="f64")
    f = lambda: float(np.sum(O.gelu_forward(u, prec="f64") * r))
    _fd_check(f, u, du, range(u.size))
    # softmax + cross-entropy (dloss = 1 per row)
    z = rng.standard_normal((3, 24))
    tgt = np.array([1, 5, 19], np.int32)
    _, probs = O.softmax_ce_forward(z, tgt, 20, prec="f64")
    dz = O.softmax_ce_backward(probs, tgt, np.ones(3), 20, prec="f64")
    f = lambda: float(np.sum(O.softmax_ce_forward(z, tgt, 20, prec="f64")[0]))
    _fd_check(f, z, dz, range(z.size))


def _randomized_model(cfg, B, T, seed, prec="f64"):
    m = O.Model(cfg, B, T, prec)
    m.init(seed)
    rng = np.random.default_rng(seed)
    P = m.P()
    # move every tensor off its special init values so each term is exercised
    for name in ("ln1w", "ln2w", "lnfw"):
        P[name][:] = 1 + 0.1 * rng.standard_normal(P[name].size)
    for name in ("ln1b", "ln2b", "lnfb", "qkvb", "attprojb", "fcb", "fcprojb"):
        P[name][:] = 0.05 * rng.standard_normal(P[name].size)
    for name in ("qkvw", "fcw", "attprojw", "fcprojw", "wpe"):
        P[name][:] *= 5
    P["wte"][: cfg.V * cfg.C] *= 5
    return m


@pytest.mark.parametrize("cfg", [
    O.Config(L=2, C=16, NH=4, maxT=8, V=40, Vp=48),   # padded vocab, 4 heads of size 4
    O.Config(L=1, C=12, NH=2, maxT=6, V=30, Vp=30),
])
def test_model_gradients_fd(cfg):
    B, T = 2, cfg.maxT - 1
    m = _randomized_model(cfg, B, T, 11)
    x, y = synth.batch(5, 0, B, T, cfg.V, "uniform")
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    grads = m.grads.copy()
    f = lambda: m.forward(x, y)
    rng = np.random.default_rng(0)
    o = 0
    for name, size in zip(O.PARAM_NAMES, m.psizes):
        view = m.params[o:o + size]
        g = grads[o:o + size]
        idx = range(size) if size <= 64 else rng.choice(size, 64, replace=False)
        _fd_check(f, view, g, idx)
        o += size
    # pad rows of wte and wpe rows >= T receive no gradient
    G = dict(zip(O.PARAM_NAMES, np.split(grads, np.cumsum(m.psizes)[:-1])))
    assert np.all(G["wte"][cfg.V * cfg.C:] == 0)
    assert np.all(G["wpe"][T * cfg.C:] == 0)


def test_key_bias_gradient_vanishes():
    """A bias on the keys adds q.b_k to every score of a query row, which the
    softmax cancels: in the fp64 oracle the key-bias slice of the qkv-bias
    gradient is zero to rounding, while the query- and value-bias slices are
    not (the reading behind the key-bias carve-out of the GPU parameter
    comparisons after AdamW steps)."""
    m = O.Model(TINY, 4, 32, "f64")
    m.init(1337)
    x, y = synth.batch(1337, 0, 4, 32, TINY.V, "uniform")
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    g = m.G()["qkvb"].reshape(TINY.L, 3, TINY.C)
    assert np.abs(g[:, 1]).max() < 1e-15 * np.abs(g[:, 2]).max()
    assert np.abs(g[:, 0]).max() > 1e-8


def test_backward_accumulates_and_zero_grad_clears():
    m = _randomized_model(TINY, 2, 8, 3, "f64")
    x, y = synth.batch(1, 0, 2, 8, TINY.V, "uniform")
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    g1 = m.grads.copy()
    m.backward()
    np.testing.assert_allclose(m.grads, 2 * g1, rtol=1e-6, atol=1e-12)
    m.zero_grad()
    assert not m.grads.any()


# ----------------------------------------------------------- whole-model closed forms
def test_zero_wte_gives_ln_v():
    cfg = O.Config(L=2, C=32, NH=4, maxT=16, V=300, Vp=384)
    m = O.Model(cfg, 3, 16, "f64")
    m.init(9)
    m.P()["wte"][:] = 0
    x, y = synth.batch(2, 0, 3, 16, cfg.V, "uniform")
    assert abs(m.forward(x, y) - math.log(cfg.V)) < 1e-13


def test_identity_blocks_reduce_to_embedding_classifier():
    """With every block weight and bias zero, attention and MLP add nothing, so
    logits = LN_f(wte[x] + wpe[t]) wte^T."""
    cfg = O.Config(L=3, C=32, NH=4, maxT=16, V=200, Vp=256)
    B, T = 2, 16
    m = O.Model(cfg, B, T, "f64")
    m.init(4)
    P = m.P()
    rng = np.random.default_rng(1)
    for name in ("qkvw", "qkvb", "attprojw", "attprojb", "fcw", "fcb", "fcprojw", "fcprojb"):
        P[name][:] = 0
    P["lnfw"][:] = 1 + 0.1 * rng.standard_normal(cfg.C)
    P["lnfb"][:] = 0.1 * rng.standard_normal(cfg.C)
    x, y = synth.batch(8, 0, B, T, cfg.V, "uniform")
    loss = m.forward(x, y)
    wte = P["wte"].reshape(cfg.Vp, cfg.C)
    wpe = P["wpe"].reshape(cfg.maxT, cfg.C)
    e = (wte[x] + wpe[None, :T]).reshape(B * T, cfg.C)
    mu = e.mean(1, keepdims=True)
    hf = (e - mu) / np.sqrt(e.var(1, keepdims=True) + 1e-5) * P["lnfw"] + P["lnfb"]
    z = hf @ wte.T
    np.testing.assert_allclose(m.logits(), z, rtol=1e-10, atol=1e-12)
    from scipy.special import logsumexp
    ref = np.mean(logsumexp(z[:, :cfg.V], axis=1) - z[np.arange(B * T), y.reshape(-1)])
    assert abs(loss - ref) < 1e-12


@pytest.mark.parametrize("cfg,expect", [
    (TINY, math.log(512) + 64 * 0.02 ** 2 / 2),
])
def test_initial_loss_near_ln_v(cfg, expect):
    m = O.Model(cfg, 4, 32)
    m.init(1337)
    x, y = synth.batch(1337, 0, 4, 32, cfg.V, "uniform")
    loss = m.forward(x, y)
    # logits have std ~ 0.02*sqrt(C) at init, so loss ~ ln V + C*0.02^2/2
    assert abs(loss - expect) < 0.05, loss


def test_adamw_closed_forms():
    rng = np.random.default_rng(6)
    n = 1000
    p0 = rng.standard_normal(n)
    g = rng.standard_normal(n)
    g[:100] = 0
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.1
    p = p0.copy()
    mm = np.zeros(n)
    vv = np.zeros(n)
    O.adamw_update(p, g, mm, vv, lr, b1, b2, eps, wd, 1, prec="f64")
    # t = 1: mhat = g, vhat = g^2
    np.testing.assert_allclose(p, p0 - lr * (g / (np.abs(g) + eps) + wd * p0), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(mm, (1 - b1) * g, rtol=1e-15)
    np.testing.assert_allclose(vv, (1 - b2) * g * g, rtol=1e-15)
    # zero-gradient entries only decay: theta_t = (1 - lr wd)^t theta_0
    for t in range(2, 6):
        O.adamw_update(p, np.where(np.arange(n) < 100, 0.0, g), mm, vv, lr, b1, b2, eps, wd, t, prec="f64")
    np.testing.assert_allclose(p[:100], p0[:100] * (1 - lr * wd) ** 5, rtol=1e-13)
    # constant gradient: mhat = g and vhat = g^2 at every t (bias correction exact)
    p = p0.copy()
    mm[:] = 0
    vv[:] = 0
    for t in range(1, 5):
        O.adamw_update(p, g, mm, vv, lr, b1, b2, eps, 0.0, t, prec="f64")
    step = g / (np.abs(g) + eps)
    np.testing.assert_allclose(p, p0 - 4 * lr * step, rtol=1e-12, atol=1e-14)


def test_clip_invariant():
    m = _randomized_model(TINY, 2, 8, 5, "f64")
    x, y = synth.batch(1, 0, 2, 8, TINY.V, "uniform")
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    g = m.grads.copy()
    n = m.clip_grad_norm(0.0)
    assert n == pytest.approx(np.linalg.norm(g), rel=1e-12)
    c = n / 3
    n2 = m.clip_grad_norm(c)
    assert n2 == pytest.approx(n, rel=1e-12)
    assert np.linalg.norm(m.grads) == pytest.approx(min(n, c), rel=1e-12)
    np.testing.assert_allclose(m.grads, g * (c / n), rtol=1e-12)
    n3 = m.clip_grad_norm(10 * n)
    assert np.linalg.norm(m.grads) == pytest.approx(n3, rel=1e-12)


def test_loss_decreases_over_10_adamw_steps():
    m = O.Model(TINY, 4, 32)
    m.init(1337)
    x, y = synth.batch(1337, 0, 4, 32, TINY.V, "uniform")
    losses = []
    for t in range(1, 11):
        losses.append(m.forward(x, y))
        m.zero_grad()
        m.backward()
        m.adamw(1e-4, 0.9, 0.999, 1e-8, 0.0, t)
    losses.append(m.forward(x, y))
    assert all(b < a for a, b in zip(losses, losses[1:])), losses


def test_thread_count_invariance():
    cfg = O.Config(L=2, C=32, NH=4, maxT=16, V=100, Vp=128)
    out = []
    for nt in (1, max(2, os.cpu_count() or 2)):
        O.set_num_threads(nt)
        m = O.Model(cfg, 3, 16)
        m.init(77)
        x, y = synth.batch(77, 0, 3, 16, cfg.V, "uniform")
        loss = m.forward(x, y)
        m.zero_grad()
        m.backward()
        m.adamw(1e-3, 0.9, 0.999, 1e-8, 0.1, 1)
        out.append((loss, m.grads.copy(), m.params.copy()))
    O.set_num_threads(os.cpu_count() or 1)
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])
    assert np.array_equal(out[0][2], out[1][2])
