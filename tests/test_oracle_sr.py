"""Pins of the oracle's stochastic rounding to bf16 and of its AdamW on bf16
parameters ("llm.c's Origin and the Future of LLM Compilers", section
"Avengers": stochastic rounding; the pages give no formula, so the reading is
the plain unbiased one: round to one of the two bf16 neighbours with the
probability that makes the expectation exact).

What fixes these values independently of the oracle's code:
  * bf16 is the top half of the fp32 bit pattern, so the two bf16 neighbours
    of x and x's position between them follow from its bits; summed over all
    65536 draws the rounded values must give exactly 65536 x (unbiasedness is
    an identity, not a statistic), and the number of draws that round away
    from zero must equal the low 16 bits of x;
  * bf16 values and non-finite inputs come back unchanged;
  * the draw stream is the published SplitMix64 generator (pinned by its
    reference vectors in test_oracle_pins.py), composed as documented;
  * the AdamW update with stochastic rounding averages, over independent
    draws, to the fp64 AdamW value (within a binomial bound), and its m and v
    equal the fp64 ones.
"""
import numpy as np

from oracle import oracle as O
from transformer_lm_train_amd import synth


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def _neighbours(x):
    """(toward zero, away from zero) bf16 neighbours of fp32 x, from its bits."""
    b = _bits(x).astype(np.uint64)
    lo = (b & 0xFFFF0000).astype(np.uint32).view(np.float32)
    hi = ((b & 0xFFFF0000) + 0x10000).astype(np.uint32).view(np.float32)
    return lo, hi


def _sample_values(rng, n):
    """fp32 values of both signs over many binades, some at the top of a
    bf16 binade (mantissa bits 1111111 in the kept half)."""
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    top = rng.integers(0, n, n // 8)
    b = _bits(x).copy()
    b[top] |= 0x007F0000  # kept mantissa all ones: hi is in the next binade
    x = b.view(np.float32)
    return x[np.isfinite(x) & (_bits(x) & 0xFFFF != 0)]


def test_sr_exact_expectation_and_neighbours():
    rng = np.random.default_rng(3)
    u = np.arange(65536, dtype=np.uint32)
    for x in _sample_values(rng, 160):
        r = O.sr_bf16(np.full(65536, x, np.float32), u)
        lo, hi = _neighbours(x)
        assert np.all((r == lo) | (r == hi)), x
        assert abs(float(lo)) <= abs(float(x)) <= abs(float(hi))
        # every result is a bf16 value
        assert np.all(_bits(r) & 0xFFFF == 0)
        # the number of draws going away from zero is the discarded fraction
        assert int(np.sum(r == hi)) == int(_bits(x) & 0xFFFF), x
        # and the mean over all draws is x exactly (the fp64 sum is exact:
        # 65536 values of 8 significant bits)
        assert np.sum(r.astype(np.float64)) == 65536.0 * float(x), x


def test_sr_keeps_bf16_values_and_non_finite():
    rng = np.random.default_rng(4)
    b = (rng.integers(0, 2**16, 4000, dtype=np.uint64) << 16).astype(np.uint32)
    x = b.view(np.float32)
    x = x[np.isfinite(x)]
    for u in (0, 1, 32768, 65535):
        assert np.array_equal(O.sr_bf16(x, u).view(np.uint32), x.view(np.uint32))
    special = np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)
    assert np.array_equal(O.sr_bf16(special, 65535).view(np.uint32), special.view(np.uint32))
    assert np.isnan(O.sr_bf16(np.array([np.nan], np.float32), 12345)[0])


def test_sr_draws_are_the_published_generator():
    # draw(seed, t, i) = top 16 bits of SplitMix64 output i+1 of the stream
    # seeded with SplitMix64 output 2^62 + t of the stream seeded with seed
    for seed, t in ((0, 1), (11, 2), (2**63 + 5, 1000)):
        key = int(synth.splitmix64(seed, np.array([2**62 + t], dtype=np.uint64))[0])
        idx = np.array([0, 1, 2, 1000, 123456789], dtype=np.uint64)
        want = (synth.splitmix64(key, idx + np.uint64(1)) >> np.uint64(48)).astype(np.uint32)
        got = np.array([O.sr_draws(seed, t, int(i), 1)[0] for i in idx], dtype=np.uint32)
        assert np.array_equal(got, want)
    d = O.sr_draws(11, 1, 0, 1 << 18)
    assert d.max() < 65536
    hist = np.bincount(d >> 8, minlength=256)
    chi2 = float(np.sum((hist - hist.mean()) ** 2 / hist.mean()))
    assert chi2 < 400  # 255 degrees of freedom
    assert np.mean(O.sr_draws(11, 2, 0, 1 << 12) == d[: 1 << 12]) < 0.01  # steps draw independently


def test_adamw_sr_update_is_unbiased():
    rng = np.random.default_rng(9)
    n = 512
    p0 = O.bf16_rne((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = (rng.standard_normal(n) * 0.01).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = (rng.random(n) * 1e-5).astype(np.float32)
    hp = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1, t=3)
    # fp64 reference of the same update
    pr, mr, vr = p0.astype(np.float64), m0.astype(np.float64), v0.astype(np.float64)
    O.adamw_update(pr, g.astype(np.float64), mr, vr, prec="f64", **hp)
    x32 = pr.astype(np.float32)
    lo, hi = _neighbours(x32)
    f = (_bits(x32) & 0xFFFF).astype(np.float64) / 65536.0
    K = 400
    acc = np.zeros(n)
    for s in range(K):
        p, m, v = p0.copy(), m0.copy(), v0.copy()
        O.adamw_sr_update(p, g, m, v, seed=1000 + s, **hp)
        assert np.all((p == lo) | (p == hi))
        acc += p
        if s == 0:
            np.testing.assert_allclose(m, mr, rtol=1e-6, atol=1e-12)
            np.testing.assert_allclose(v, vr, rtol=1e-6, atol=1e-15)
            # the draws used are orc_sr_draw(seed, t, i)
            assert np.array_equal(p, O.sr_bf16(x32, O.sr_draws(1000, hp["t"], 0, n)))
    mean = acc / K
    gap = (hi.astype(np.float64) - lo.astype(np.float64))
    sd = np.abs(gap) * np.sqrt(f * (1 - f) / K)
    assert np.all(np.abs(mean - pr) <= 6 * sd + 1e-3 * np.abs(gap))


def test_bf16_rne_helper():
    # the rounding of a bf16 conversion: nearest, ties to even
    x = np.array([1.0 + 2**-9, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 3 * 2**-9, -(1.0 + 2**-8 + 2**-12)],
                 dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -(1.0 + 2**-7)], dtype=np.float32)
    assert np.array_equal(O.bf16_rne(x), want)
