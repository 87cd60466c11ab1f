"""Thin ctypes binding of the GPT-2 step library (include/gpt2.h).

Argument marshalling only: every step of the training step runs in the HIP
kernels of ``_build/libgpt2mi.so``.  PyTorch provides the device buffer and
the stream.  There is no fallback: if the library is missing the import of
``lib()`` raises.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libgpt2mi.so")

GPT2_OK = 0
GPT2_EINVAL = -22
GPT2_ENOMEM = -12
GPT2_EPERM = -1
GPT2_ERANGE = -34
GPT2_EIO = -5
GPT2_FP32 = 0
GPT2_BF16_MIXED = 1
GPT2_BF16_SR = 2  # bf16 parameters updated by stochastic rounding (no fp32 master)

PARAM_NAMES = ["wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
               "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb"]


class gpt2_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("padded_vocab_size", ctypes.c_int32),
                ("batch_size", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("fused_classifier", ctypes.c_int32),
                ("recompute_gelu", ctypes.c_int32), ("recompute_layernorm", ctypes.c_int32)]


class GPT2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_LIB = None


def lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(gpt2_config)
    ip = ctypes.POINTER(ctypes.c_int32)
    fp = ctypes.POINTER(ctypes.c_float)
    sigs = {
        "gpt2_plan": ([cfgp, ctypes.POINTER(sz)], ctypes.c_int),
        "gpt2_build": ([cfgp, ctypes.c_uint64, vp, sz, vp, ctypes.POINTER(vp)], ctypes.c_int),
        "gpt2_forward": ([vp, ip, ip, fp], ctypes.c_int),
        "gpt2_forward_device": ([vp, vp, vp, fp], ctypes.c_int),
        "gpt2_read_loss": ([vp, fp], ctypes.c_int),
        "gpt2_sync": ([vp], ctypes.c_int),
        "gpt2_zero_grad": ([vp], ctypes.c_int),
        "gpt2_backward": ([vp], ctypes.c_int),
        "gpt2_clip_grad_norm": ([vp, f32, fp], ctypes.c_int),
        "gpt2_adamw_step": ([vp, f32, f32, f32, f32, f32, ctypes.c_int], ctypes.c_int),
        "gpt2_destroy": ([vp], ctypes.c_int),
        "gpt2_last_error": ([], ctypes.c_char_p),
        "gpt2_num_params": ([vp], sz),
        "gpt2_param_offsets": ([vp, ctypes.POINTER(sz)], ctypes.c_int),
        "gpt2_copy_params": ([vp, fp], ctypes.c_int),
        "gpt2_copy_grads": ([vp, fp], ctypes.c_int),
        "gpt2_copy_opt_state": ([vp, fp, fp], ctypes.c_int),
        "gpt2_copy_logits": ([vp, fp], ctypes.c_int),
        "gpt2_copy_losses": ([vp, fp], ctypes.c_int),
        "gpt2_set_params": ([vp, fp], ctypes.c_int),
        "gpt2_set_grads": ([vp, fp], ctypes.c_int),
        "gpt2_device_params": ([vp], vp),
        "gpt2_device_grads": ([vp], vp),
        "gpt2_device_shadow": ([vp], vp),
        "gpt2_kernel_timing_enable": ([vp, ctypes.c_char_p, ctypes.c_int], ctypes.c_int),
        "gpt2_kernel_timing_read": ([vp, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)],
                                    ctypes.c_int),
        "gpt2_test_gemm_nt": ([vp, vp, vp, vp, vp, i32, i32, i32], ctypes.c_int),
        "gpt2_test_gemm_nn": ([vp, vp, vp, vp, i32, i32, i32], ctypes.c_int),
        "gpt2_test_gemm_tn": ([vp, vp, vp, vp, i32, i32, i32], ctypes.c_int),
        "gpt2_test_attention_fwd": ([vp, vp, vp, vp, i32, i32, i32, i32], ctypes.c_int),
        "gpt2_test_attention_bwd": ([vp, vp, vp, vp, vp, vp, i32, i32, i32, i32], ctypes.c_int),
        "gpt2_attention_bwd_noalloc": ([vp, vp, vp, vp, vp, vp, i32, i32, i32, i32], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = L
    return L


def _check(rc):
    if rc != GPT2_OK:
        raise GPT2Error(rc, lib().gpt2_last_error().decode())
    return rc


def _fptr(a):
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _iptr(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def make_config(L, C, NH, maxT, V, Vp, B, T, precision, fused_classifier=False, recompute_gelu=False,
                recompute_layernorm=False):
    return gpt2_config(L, C, NH, maxT, V, Vp, B, T, precision, 1 if fused_classifier else 0,
                       1 if recompute_gelu else 0, 1 if recompute_layernorm else 0)


# ---- the C ABI, one Python function per entry point ------------------------
def gpt2_plan(cfg):
    n = ctypes.c_size_t()
    _check(lib().gpt2_plan(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def gpt2_build(cfg, seed, device_ptr, nbytes, stream_ptr):
    h = ctypes.c_void_p()
    _check(lib().gpt2_build(ctypes.byref(cfg), seed, device_ptr, nbytes, stream_ptr, ctypes.byref(h)))
    return h


def gpt2_forward(h, tokens, targets=None, read_loss=True):
    loss = ctypes.c_float()
    _check(lib().gpt2_forward(h, _iptr(tokens), _iptr(targets), ctypes.byref(loss) if read_loss else None))
    return loss.value if read_loss else None


def gpt2_forward_device(h, d_tokens_ptr, d_targets_ptr=None, read_loss=True):
    loss = ctypes.c_float()
    _check(lib().gpt2_forward_device(h, d_tokens_ptr, d_targets_ptr, ctypes.byref(loss) if read_loss else None))
    return loss.value if read_loss else None


def gpt2_read_loss(h):
    loss = ctypes.c_float()
    _check(lib().gpt2_read_loss(h, ctypes.byref(loss)))
    return loss.value


def gpt2_sync(h):
    _check(lib().gpt2_sync(h))


def gpt2_zero_grad(h):
    _check(lib().gpt2_zero_grad(h))


def gpt2_backward(h):
    _check(lib().gpt2_backward(h))


def gpt2_clip_grad_norm(h, max_norm, read_norm=True):
    n = ctypes.c_float()
    _check(lib().gpt2_clip_grad_norm(h, max_norm, ctypes.byref(n) if read_norm else None))
    return n.value if read_norm else None


def gpt2_adamw_step(h, lr, beta1, beta2, eps, weight_decay, t):
    _check(lib().gpt2_adamw_step(h, lr, beta1, beta2, eps, weight_decay, t))


def gpt2_destroy(h):
    _check(lib().gpt2_destroy(h))


def gpt2_num_params(h):
    return int(lib().gpt2_num_params(h))


def gpt2_param_offsets(h):
    o = (ctypes.c_size_t * 16)()
    _check(lib().gpt2_param_offsets(h, o))
    return [int(x) for x in o]


def gpt2_copy_params(h):
    out = np.empty(gpt2_num_params(h), np.float32)
    _check(lib().gpt2_copy_params(h, _fptr(out)))
    return out


def gpt2_copy_grads(h):
    out = np.empty(gpt2_num_params(h), np.float32)
    _check(lib().gpt2_copy_grads(h, _fptr(out)))
    return out


def gpt2_copy_opt_state(h):
    m = np.empty(gpt2_num_params(h), np.float32)
    v = np.empty_like(m)
    _check(lib().gpt2_copy_opt_state(h, _fptr(m), _fptr(v)))
    return m, v


def gpt2_copy_logits(h, rows, Vp):
    out = np.empty((rows, Vp), np.float32)
    _check(lib().gpt2_copy_logits(h, _fptr(out)))
    return out


def gpt2_copy_losses(h, rows):
    out = np.empty(rows, np.float32)
    _check(lib().gpt2_copy_losses(h, _fptr(out)))
    return out


def gpt2_set_params(h, params):
    params = np.ascontiguousarray(params, dtype=np.float32)
    _check(lib().gpt2_set_params(h, _fptr(params)))


def gpt2_set_grads(h, grads):
    grads = np.ascontiguousarray(grads, dtype=np.float32)
    assert grads.size == gpt2_num_params(h)
    _check(lib().gpt2_set_grads(h, _fptr(grads)))


def gpt2_kernel_timing_enable(h, cls, enable=True):
    _check(lib().gpt2_kernel_timing_enable(h, cls.encode(), 1 if enable else 0))


def gpt2_kernel_timing_read(h):
    n = ctypes.c_int()
    ms = ctypes.c_double()
    _check(lib().gpt2_kernel_timing_read(h, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def gpt2_test_gemm_nt(h, out_ptr, a_ptr, w_ptr, bias_ptr, M, N, K):
    _check(lib().gpt2_test_gemm_nt(h, out_ptr, a_ptr, w_ptr, bias_ptr, M, N, K))


def gpt2_test_gemm_nn(h, dx_ptr, dy_ptr, w_ptr, M, N, K):
    _check(lib().gpt2_test_gemm_nn(h, dx_ptr, dy_ptr, w_ptr, M, N, K))


def gpt2_test_gemm_tn(h, dw_ptr, dy_ptr, x_ptr, M, N, K):
    _check(lib().gpt2_test_gemm_tn(h, dw_ptr, dy_ptr, x_ptr, M, N, K))


def gpt2_test_attention_fwd(h, out_ptr, lse_ptr, qkv_ptr, B, T, C, NH):
    _check(lib().gpt2_test_attention_fwd(h, out_ptr, lse_ptr, qkv_ptr, B, T, C, NH))


def gpt2_test_attention_bwd(h, dqkv_ptr, dout_ptr, qkv_ptr, out_ptr, lse_ptr, B, T, C, NH):
    _check(lib().gpt2_test_attention_bwd(h, dqkv_ptr, dout_ptr, qkv_ptr, out_ptr, lse_ptr, B, T, C, NH))


def gpt2_attention_bwd_noalloc(stream_ptr, dqkv_ptr, dout_ptr, qkv_ptr, out_ptr, lse_ptr, B, T, C, NH):
    _check(lib().gpt2_attention_bwd_noalloc(stream_ptr, dqkv_ptr, dout_ptr, qkv_ptr, out_ptr, lse_ptr, B, T, C, NH))


# ---- convenience wrapper: torch owns the device buffer and the stream -------
class Model:
    """One GPT-2 training step engine on one GPU.

    ``cfg`` is a gpt2_config; the device buffer is a torch uint8 tensor of
    gpt2_plan() bytes and the stream is torch's current stream on ``device``.
    """

    def __init__(self, cfg, seed, device="cuda:0"):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.nbytes = gpt2_plan(cfg)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        self.h = gpt2_build(cfg, seed, self.buf.data_ptr(), self.nbytes, self.stream.cuda_stream)
        self.BT = cfg.batch_size * cfg.seq_len

    def close(self):
        if getattr(self, "h", None):
            gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, tokens, targets=None, read_loss=True):
        tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        if targets is not None:
            targets = np.ascontiguousarray(targets, dtype=np.int32).reshape(-1)
        return gpt2_forward(self.h, tokens, targets, read_loss)

    def forward_device(self, d_tokens, d_targets=None, read_loss=True):
        return gpt2_forward_device(self.h, d_tokens.data_ptr(),
                                   None if d_targets is None else d_targets.data_ptr(), read_loss)

    def zero_grad(self):
        gpt2_zero_grad(self.h)

    def backward(self):
        gpt2_backward(self.h)

    def clip_grad_norm(self, max_norm, read_norm=True):
        return gpt2_clip_grad_norm(self.h, max_norm, read_norm)

    def adamw_step(self, lr, beta1, beta2, eps, weight_decay, t):
        gpt2_adamw_step(self.h, lr, beta1, beta2, eps, weight_decay, t)

    def params(self):
        return gpt2_copy_params(self.h)

    def grads(self):
        return gpt2_copy_grads(self.h)

    def opt_state(self):
        return gpt2_copy_opt_state(self.h)

    def logits(self):
        return gpt2_copy_logits(self.h, self.BT, self.cfg.padded_vocab_size)

    def losses(self):
        return gpt2_copy_losses(self.h, self.BT)

    def set_params(self, p):
        gpt2_set_params(self.h, p)

    def set_grads(self, g):
        gpt2_set_grads(self.h, g)

    def sync(self):
        gpt2_sync(self.h)

    def param_offsets(self):
        return gpt2_param_offsets(self.h)
