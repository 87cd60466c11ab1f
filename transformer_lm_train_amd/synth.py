"""Seeded synthetic token streams (inputs only; no part of the model's arithmetic).

The pages train on tokenised text bins (tinyshakespeare, FineWeb) that are not
available here, so seeded synthetic streams stand in for them:

* ``uniform``: ids = floor(u * V), used by the tiny configuration;
* ``zipf``: P(id = k) proportional to (k+1)^-s over k in [0, V) (s = 1.1 by
  default, rank k+1 mapped to id k), drawn by inverse CDF with a binary
  search over the cumulative weights in double, for the GPT-2 sizes.

u comes from SplitMix64 (Steele, Lea & Flood 2014): draw number
n = step * 2^32 + i + 1 of the stream seeded with ``seed`` gives u_i =
(w >> 11) * 2^-53.  One step needs B*T+1 ids S; inputs[b,t] = S[b*T+t] and
targets[b,t] = S[b*T+t+1] (targets are the inputs shifted by one).

Both the oracle-side tests and the GPU-side tests and benchmark take their
tokens from here.
"""
import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: np.ndarray) -> np.ndarray:
    """Output number n (n >= 1) of the SplitMix64 stream seeded with seed."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + n.astype(np.uint64) * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniforms(seed: int, step: int, count: int) -> np.ndarray:
    n = np.uint64(step) * np.uint64(1 << 32) + np.arange(1, count + 1, dtype=np.uint64)
    w = splitmix64(seed, n)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


_ZIPF_CDF = {}


def _zipf_cdf(V: int, s: float) -> np.ndarray:
    key = (V, s)
    if key not in _ZIPF_CDF:
        w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
        c = np.cumsum(w)
        _ZIPF_CDF[key] = c / c[-1]
    return _ZIPF_CDF[key]


def token_stream(seed: int, step: int, count: int, V: int, dist: str = "zipf",
                 zipf_s: float = 1.1) -> np.ndarray:
    u = uniforms(seed, step, count)
    if dist == "uniform":
        ids = np.floor(u * V).astype(np.int64)
    elif dist == "zipf":
        ids = np.searchsorted(_zipf_cdf(V, zipf_s), u, side="right")
    else:
        raise ValueError(dist)
    return np.minimum(ids, V - 1).astype(np.int32)


def batch(seed: int, step: int, B: int, T: int, V: int, dist: str = "zipf"):
    """(inputs, targets), each int32 [B, T]: a B*T+1 stream, shifted by one."""
    s = token_stream(seed, step, B * T + 1, V, dist)
    return s[:-1].reshape(B, T).copy(), s[1:].reshape(B, T).copy()
