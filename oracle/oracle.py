"""ctypes front end of the CPU oracle (test infrastructure only).

The oracle is the plain CPU definition of one GPT-2 training step (see
``gpt2_oracle.c`` for the sources it follows).  Only the tests, the smoke
check and the benchmark's CPU-baseline leg use it; the product library never
imports, links or calls anything in this directory.

``Model`` wraps the whole step (init, forward, zero_grad, backward, clip,
AdamW) and exposes parameters, gradients, optimizer state and activations as
numpy views.  The free functions wrap single layers for the pin tests.
"""
import ctypes
import os

import numpy as np

from . import build as _build

PARAM_NAMES = ["wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb"]
ACT_NAMES = ["encoded", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "preatt", "att",
             "attproj", "residual2", "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu",
             "fcproj", "residual3", "lnf", "lnf_mean", "lnf_rstd", "logits", "probs", "losses"]


class Config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("C", ctypes.c_int), ("NH", ctypes.c_int),
                ("maxT", ctypes.c_int), ("V", ctypes.c_int), ("Vp", ctypes.c_int)]

    def __repr__(self):
        return (f"Config(L={self.L}, C={self.C}, NH={self.NH}, maxT={self.maxT}, "
                f"V={self.V}, Vp={self.Vp})")


_LIBS = {}
_NP = {"f32": np.float32, "f64": np.float64}
_CT = {"f32": ctypes.c_float, "f64": ctypes.c_double}


def _lib(precision="f32"):
    if precision in _LIBS:
        return _LIBS[precision]
    path = _build.lib_path(precision)
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    R = ctypes.POINTER(_CT[precision])
    I = ctypes.POINTER(ctypes.c_int)
    sz = ctypes.c_size_t
    cfgp = ctypes.POINTER(Config)
    vp = ctypes.c_void_p
    lib.orc_param_sizes.argtypes = [cfgp, ctypes.POINTER(sz)]
    lib.orc_num_params.argtypes = [cfgp]
    lib.orc_num_params.restype = sz
    lib.orc_act_sizes.argtypes = [cfgp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    lib.orc_num_acts.argtypes = [cfgp, ctypes.c_int, ctypes.c_int]
    lib.orc_num_acts.restype = sz
    lib.orc_init_params.argtypes = [cfgp, ctypes.c_uint64, R]
    lib.orc_create.argtypes = [cfgp, ctypes.c_int, ctypes.c_int]
    lib.orc_create.restype = vp
    lib.orc_free.argtypes = [vp]
    for name in ("orc_params", "orc_grads", "orc_mbuf", "orc_vbuf", "orc_acts", "orc_act_grads"):
        getattr(lib, name).argtypes = [vp]
        getattr(lib, name).restype = R
    lib.orc_model_num_params.argtypes = [vp]
    lib.orc_model_num_params.restype = sz
    lib.orc_forward.argtypes = [vp, I, I]
    lib.orc_forward.restype = ctypes.c_double
    lib.orc_zero_grad.argtypes = [vp]
    lib.orc_backward.argtypes = [vp]
    lib.orc_backward.restype = ctypes.c_int
    lib.orc_clip_grad_norm.argtypes = [vp, ctypes.c_double]
    lib.orc_clip_grad_norm.restype = ctypes.c_double
    d = ctypes.c_double
    lib.orc_adamw.argtypes = [vp, d, d, d, d, d, ctypes.c_int]
    lib.orc_adamw.restype = ctypes.c_int
    i32 = ctypes.c_int
    lib.orc_embed_fwd.argtypes = [I, R, R, i32, i32, i32, R]
    lib.orc_embed_bwd.argtypes = [R, I, i32, i32, i32, R, R]
    lib.orc_norm_fwd.argtypes = [R, R, R, i32, i32, R, R, R]
    lib.orc_norm_bwd.argtypes = [R, R, R, R, R, i32, i32, R, R, R]
    lib.orc_linear_fwd.argtypes = [R, R, R, i32, i32, i32, R]
    lib.orc_linear_bwd.argtypes = [R, R, R, i32, i32, i32, R, R, R]
    lib.orc_attn_fwd.argtypes = [R, i32, i32, i32, i32, R, R, R]
    lib.orc_attn_bwd.argtypes = [R, R, R, i32, i32, i32, i32, R]
    lib.orc_gelu_fwd.argtypes = [R, sz, R]
    lib.orc_gelu_bwd.argtypes = [R, R, sz, R]
    lib.orc_xent_fwd.argtypes = [R, I, i32, i32, i32, R, R]
    lib.orc_xent_bwd.argtypes = [R, R, I, i32, i32, i32, R]
    lib.orc_global_norm.argtypes = [R, sz]
    lib.orc_global_norm.restype = ctypes.c_double
    lib.orc_adamw_update.argtypes = [R, R, R, R, sz, d, d, d, d, d, ctypes.c_int, d]
    F = ctypes.POINTER(ctypes.c_float)
    u64 = ctypes.c_uint64
    lib.orc_sr_draw.argtypes = [u64, ctypes.c_int, u64]
    lib.orc_sr_draw.restype = ctypes.c_uint32
    lib.orc_sr_bf16.argtypes = [ctypes.c_float, ctypes.c_uint32]
    lib.orc_sr_bf16.restype = ctypes.c_float
    U = ctypes.POINTER(ctypes.c_uint32)
    lib.orc_sr_draws.argtypes = [u64, ctypes.c_int, u64, sz, U]
    lib.orc_sr_bf16_array.argtypes = [F, U, sz, F]
    lib.orc_adamw_sr_update.argtypes = [F, F, F, F, sz, d, d, d, d, d, ctypes.c_int, d, u64]
    lib.orc_adamw_sr.argtypes = [vp, d, d, d, d, d, ctypes.c_int, u64]
    lib.orc_adamw_sr.restype = ctypes.c_int
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    _LIBS[precision] = lib
    return lib


def num_threads():
    return _lib("f32").orc_num_threads()


def set_num_threads(n):
    for p in ("f32", "f64"):
        _lib(p).orc_set_num_threads(n)


def param_sizes(cfg):
    s = (ctypes.c_size_t * 16)()
    _lib().orc_param_sizes(ctypes.byref(cfg), s)
    return [int(x) for x in s]


def num_params(cfg):
    return int(_lib().orc_num_params(ctypes.byref(cfg)))


def act_sizes(cfg, B, T):
    s = (ctypes.c_size_t * 23)()
    _lib().orc_act_sizes(ctypes.byref(cfg), B, T, s)
    return [int(x) for x in s]


def num_acts(cfg, B, T):
    return int(_lib().orc_num_acts(ctypes.byref(cfg), B, T))


def init_params(cfg, seed, precision="f32"):
    out = np.zeros(num_params(cfg), dtype=_NP[precision])
    _lib(precision).orc_init_params(ctypes.byref(cfg), ctypes.c_uint64(seed), _ptr(out, precision))
    return out


def _ptr(a, precision="f32"):
    assert a.dtype == _NP[precision] and a.flags["C_CONTIGUOUS"], (a.dtype, precision)
    return a.ctypes.data_as(ctypes.POINTER(_CT[precision]))


def _iptr(a):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _split(flat, sizes, names):
    out, o = {}, 0
    for n, s in zip(names, sizes):
        out[n] = flat[o:o + s]
        o += s
    return out


class Model:
    """The whole training step of the oracle on a fixed (B, T)."""

    def __init__(self, cfg, B, T, precision="f32"):
        self.cfg, self.B, self.T, self.prec = cfg, B, T, precision
        self.lib = _lib(precision)
        self.h = self.lib.orc_create(ctypes.byref(cfg), B, T)
        if not self.h:
            raise ValueError(f"oracle rejected config {cfg} B={B} T={T}")
        self.np = num_params(cfg)
        self.na = num_acts(cfg, B, T)
        dt = _NP[precision]

        def view(fn, n):
            p = fn(self.h)
            return np.ctypeslib.as_array(p, shape=(n,)).view(dt)

        self.params = view(self.lib.orc_params, self.np)
        self.grads = view(self.lib.orc_grads, self.np)
        self.m = view(self.lib.orc_mbuf, self.np)
        self.v = view(self.lib.orc_vbuf, self.np)
        self.acts = view(self.lib.orc_acts, self.na)
        self.act_grads = view(self.lib.orc_act_grads, self.na)
        self.psizes = param_sizes(cfg)
        self.asizes = act_sizes(cfg, B, T)

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            self.lib.orc_free(h)
            self.h = None

    def P(self):
        return _split(self.params, self.psizes, PARAM_NAMES)

    def G(self):
        return _split(self.grads, self.psizes, PARAM_NAMES)

    def A(self):
        return _split(self.acts, self.asizes, ACT_NAMES)

    def init(self, seed):
        self.lib.orc_init_params(ctypes.byref(self.cfg), ctypes.c_uint64(seed),
                                 _ptr(self.params, self.prec))

    def forward(self, inputs, targets=None):
        inputs = np.ascontiguousarray(inputs, dtype=np.int32).reshape(-1)
        assert inputs.size == self.B * self.T
        assert inputs.min() >= 0 and inputs.max() < self.cfg.V
        tp = None
        if targets is not None:
            targets = np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
            assert targets.size == self.B * self.T
            assert targets.min() >= 0 and targets.max() < self.cfg.V
            tp = _iptr(targets)
        self._keep = (inputs, targets)
        return float(self.lib.orc_forward(self.h, _iptr(inputs), tp))

    def zero_grad(self):
        self.lib.orc_zero_grad(self.h)

    def backward(self):
        rc = self.lib.orc_backward(self.h)
        if rc != 0:
            raise RuntimeError("oracle backward needs a forward pass with targets")

    def clip_grad_norm(self, max_norm):
        return float(self.lib.orc_clip_grad_norm(self.h, max_norm))

    def adamw(self, lr, beta1, beta2, eps, weight_decay, t):
        rc = self.lib.orc_adamw(self.h, lr, beta1, beta2, eps, weight_decay, t)
        if rc != 0:
            raise ValueError("t must be >= 1")

    def adamw_sr(self, lr, beta1, beta2, eps, weight_decay, t, seed):
        """AdamW on bf16-valued parameters with stochastic rounding (fp32 oracle only)."""
        rc = self.lib.orc_adamw_sr(self.h, lr, beta1, beta2, eps, weight_decay, t, ctypes.c_uint64(seed))
        if rc != 0:
            raise ValueError("t must be >= 1 and the oracle the fp32 one")

    def logits(self):
        return self.A()["logits"].reshape(self.B * self.T, self.cfg.Vp)


# ---------------------------------------------------------------- layer ops
def _arr(x, prec):
    return np.ascontiguousarray(x, dtype=_NP[prec])


def encoder_forward(inp, wte, wpe, prec="f32"):
    inp = np.ascontiguousarray(inp, dtype=np.int32)
    B, T = inp.shape
    C = wte.shape[1]
    wte, wpe = _arr(wte, prec), _arr(wpe, prec)
    out = np.zeros((B, T, C), _NP[prec])
    _lib(prec).orc_embed_fwd(_iptr(inp), _ptr(wte, prec), _ptr(wpe, prec), B, T, C, _ptr(out, prec))
    return out


def encoder_backward(dwte, dwpe, dout, inp, prec="f32"):
    inp = np.ascontiguousarray(inp, dtype=np.int32)
    B, T = inp.shape
    C = dout.shape[-1]
    dout = _arr(dout, prec)
    _lib(prec).orc_embed_bwd(_ptr(dout, prec), _iptr(inp), B, T, C, _ptr(dwte, prec), _ptr(dwpe, prec))


def layernorm_forward(x, w, b, prec="f32"):
    x, w, b = _arr(x, prec), _arr(w, prec), _arr(b, prec)
    N, C = x.shape
    out = np.zeros_like(x)
    mean = np.zeros(N, _NP[prec])
    rstd = np.zeros(N, _NP[prec])
    _lib(prec).orc_norm_fwd(_ptr(x, prec), _ptr(w, prec), _ptr(b, prec), N, C, _ptr(out, prec), _ptr(mean, prec),
                            _ptr(rstd, prec))
    return out, mean, rstd


def layernorm_backward(dout, x, w, mean, rstd, prec="f32"):
    dout, x, w, mean, rstd = (_arr(a, prec) for a in (dout, x, w, mean, rstd))
    N, C = x.shape
    dx = np.zeros_like(x)
    dw = np.zeros(C, _NP[prec])
    db = np.zeros(C, _NP[prec])
    _lib(prec).orc_norm_bwd(_ptr(dout, prec), _ptr(x, prec), _ptr(w, prec), _ptr(mean, prec), _ptr(rstd, prec),
                            N, C, _ptr(dx, prec), _ptr(dw, prec), _ptr(db, prec))
    return dx, dw, db


def matmul_forward(x, w, bias=None, prec="f32"):
    x, w = _arr(x, prec), _arr(w, prec)
    N, C = x.shape
    OC = w.shape[0]
    out = np.zeros((N, OC), _NP[prec])
    bp = None if bias is None else _ptr(_arr(bias, prec), prec)
    if bias is not None:
        bias = _arr(bias, prec)
        bp = _ptr(bias, prec)
    _lib(prec).orc_linear_fwd(_ptr(x, prec), _ptr(w, prec), bp, N, C, OC, _ptr(out, prec))
    return out


def matmul_backward(dout, x, w, prec="f32"):
    dout, x, w = _arr(dout, prec), _arr(x, prec), _arr(w, prec)
    N, C = x.shape
    OC = w.shape[0]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    db = np.zeros(OC, _NP[prec])
    _lib(prec).orc_linear_bwd(_ptr(dout, prec), _ptr(x, prec), _ptr(w, prec), N, C, OC, _ptr(dx, prec),
                              _ptr(dw, prec), _ptr(db, prec))
    return dx, dw, db


def attention_forward(qkv, NH, prec="f32"):
    qkv = _arr(qkv, prec)
    B, T, C3 = qkv.shape
    C = C3 // 3
    out = np.zeros((B, T, C), _NP[prec])
    pre = np.zeros((B, NH, T, T), _NP[prec])
    att = np.zeros((B, NH, T, T), _NP[prec])
    _lib(prec).orc_attn_fwd(_ptr(qkv, prec), B, T, C, NH, _ptr(out, prec), _ptr(pre, prec), _ptr(att, prec))
    return out, pre, att


def attention_backward(dout, qkv, att, NH, prec="f32"):
    dout, qkv, att = _arr(dout, prec), _arr(qkv, prec), _arr(att, prec)
    B, T, C3 = qkv.shape
    dqkv = np.zeros_like(qkv)
    _lib(prec).orc_attn_bwd(_ptr(dout, prec), _ptr(qkv, prec), _ptr(att, prec), B, T, C3 // 3, NH,
                            _ptr(dqkv, prec))
    return dqkv


def gelu_forward(x, prec="f32"):
    x = _arr(x, prec)
    out = np.zeros_like(x)
    _lib(prec).orc_gelu_fwd(_ptr(x, prec), x.size, _ptr(out, prec))
    return out


def gelu_backward(x, dout, prec="f32"):
    x, dout = _arr(x, prec), _arr(dout, prec)
    dx = np.zeros_like(x)
    _lib(prec).orc_gelu_bwd(_ptr(dout, prec), _ptr(x, prec), x.size, _ptr(dx, prec))
    return dx


def softmax_ce_forward(logits, targets, V, prec="f32"):
    logits = _arr(logits, prec)
    N, Vp = logits.shape
    probs = np.zeros_like(logits)
    losses = np.zeros(N, _NP[prec])
    tp = None
    if targets is not None:
        targets = np.ascontiguousarray(targets, dtype=np.int32)
        tp = _iptr(targets)
    _lib(prec).orc_xent_fwd(_ptr(logits, prec), tp, N, V, Vp, _ptr(probs, prec), _ptr(losses, prec))
    return losses, probs


def softmax_ce_backward(probs, targets, dlosses, V, prec="f32"):
    probs, dlosses = _arr(probs, prec), _arr(dlosses, prec)
    targets = np.ascontiguousarray(targets, dtype=np.int32)
    N, Vp = probs.shape
    d = np.zeros_like(probs)
    _lib(prec).orc_xent_bwd(_ptr(dlosses, prec), _ptr(probs, prec), _iptr(targets), N, V, Vp, _ptr(d, prec))
    return d


def global_norm(g, prec="f32"):
    g = _arr(g, prec)
    return float(_lib(prec).orc_global_norm(_ptr(g, prec), g.size))


def sr_draws(seed, t, i0, n):
    """The 16-bit stochastic-rounding draws of flat indices i0 .. i0+n-1 at AdamW step t."""
    out = np.zeros(n, dtype=np.uint32)
    _lib("f32").orc_sr_draws(ctypes.c_uint64(seed), t, ctypes.c_uint64(i0), n,
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
    return out


def sr_bf16(x, u):
    """Stochastic rounding of fp32 values x to bf16 with draws u (elementwise), widened to float32."""
    x = np.ascontiguousarray(np.ravel(x), dtype=np.float32)
    u = np.ascontiguousarray(np.broadcast_to(np.asarray(u, dtype=np.uint32), x.shape))
    out = np.zeros_like(x)
    F = ctypes.POINTER(ctypes.c_float)
    _lib("f32").orc_sr_bf16_array(x.ctypes.data_as(F), u.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), x.size,
                                  out.ctypes.data_as(F))
    return out


def bf16_rne(x):
    """Round fp32 values to the nearest bf16 value (ties to even), widened to float32: the
    rounding a bf16 conversion of an fp32 value makes (finite values only)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = b >> 16
    rest = b & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return ((keep + up) << 16).astype(np.uint32).view(np.float32)


def adamw_sr_update(params, grads, m, v, lr, b1, b2, eps, wd, t, seed, grad_scale=1.0):
    """AdamW on bf16-valued float32 params with stochastic rounding, in place (params, m, v)."""
    for a in (params, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    grads = _arr(grads, "f32")
    F = ctypes.POINTER(ctypes.c_float)
    c = lambda a: a.ctypes.data_as(F)
    _lib("f32").orc_adamw_sr_update(c(params), c(grads), c(m), c(v), params.size, lr, b1, b2, eps, wd, t,
                                    grad_scale, ctypes.c_uint64(seed))


def adamw_update(params, grads, m, v, lr, b1, b2, eps, wd, t, grad_scale=1.0, prec="f32"):
    grads = _arr(grads, prec)
    _lib(prec).orc_adamw_update(_ptr(params, prec), _ptr(grads, prec), _ptr(m, prec), _ptr(v, prec),
                                params.size, lr, b1, b2, eps, wd, t, grad_scale)
