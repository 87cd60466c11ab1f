"""Kernel-level parity through the C ABI: the three matrix-product kernels
(forward NT, backward-data NN, backward-weight TN) in fp32 and bf16 modes
against the oracle's linear layer (fp64 build), on shapes that span several
tiles and end in ragged tiles."""
import numpy as np
import pytest

from oracle import oracle as O
from transformer_lm_train_amd import gpt2 as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _model(precision):
    if precision == G.GPT2_BF16_MIXED:
        cfg = G.make_config(1, 64, 1, 64, 64, 64, 1, 64, precision)
    else:
        cfg = G.make_config(1, 16, 2, 8, 16, 16, 1, 8, precision)
    return G.Model(cfg, 1)


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def _host64(t):
    return t.float().cpu().numpy().astype(np.float64)


# bf16 needs the reduction dimension of each product to be a multiple of 64
# (K for NT, N for NN, M for TN) and the others multiples of 8.
# The shapes also reach every tile configuration the dispatcher picks:
# forward N < 1536 / >= 1536 / >= 3072, ragged against 128 and 256 tiles.
BF16_CASES = [(256, 384, 128), (136, 72, 64), (192, 320, 128), (128, 1000, 192), (64, 64, 64),
              (392, 264, 320), (448, 192, 576), (136, 1600, 64), (264, 3080, 128), (320, 3072, 192)]
F32_CASES = [(100, 70, 33), (64, 64, 64), (5, 130, 7), (257, 19, 100)]


def _close(got, ref, rel):
    scale = np.max(np.abs(ref)) + 1e-30
    err = np.max(np.abs(got - ref)) / scale
    l2 = np.linalg.norm(got - ref) / (np.linalg.norm(ref) + 1e-30)
    assert err <= rel and l2 <= rel, (err, l2)


@pytest.mark.parametrize("prec,cases,dt,tol", [
    (G.GPT2_BF16_MIXED, BF16_CASES, "bf16", 8e-3),
    (G.GPT2_FP32, F32_CASES, "f32", 1e-5),
])
def test_gemm_kernels_vs_oracle(prec, cases, dt, tol):
    m = _model(prec)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    rng = np.random.default_rng(0)
    for (M, N, K) in cases:
        print(f"gemm {dt} M={M} N={N} K={K}", flush=True)
        x = _dev(rng.standard_normal((M, K)), tdt)
        w = _dev(rng.standard_normal((N, K)) * 0.1, tdt)
        bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda()
        out = torch.zeros((M, N), dtype=tdt, device="cuda")
        G.gpt2_test_gemm_nt(m.h, out.data_ptr(), x.data_ptr(), w.data_ptr(), bias.data_ptr(), M, N, K)
        torch.cuda.synchronize()
        ref = O.matmul_forward(_host64(x), _host64(w), bias.cpu().numpy().astype(np.float64), prec="f64")
        _close(_host64(out), ref, tol)
        if dt == "bf16" and (N % 64 or M % 64):
            continue
        # backward data: dX[M,K] = dY[M,N] W[N,K]
        dy = _dev(rng.standard_normal((M, N)), tdt)
        dx = torch.zeros((M, K), dtype=tdt, device="cuda")
        G.gpt2_test_gemm_nn(m.h, dx.data_ptr(), dy.data_ptr(), w.data_ptr(), M, N, K)
        # backward weight: dW[N,K] += dY^T X, accumulated onto a non-zero start
        dw0 = rng.standard_normal((N, K)).astype(np.float32)
        dw = torch.from_numpy(dw0).cuda()
        G.gpt2_test_gemm_tn(m.h, dw.data_ptr(), dy.data_ptr(), x.data_ptr(), M, N, K)
        torch.cuda.synchronize()
        rdx, rdw, _ = O.matmul_backward(_host64(dy), _host64(x), _host64(w), prec="f64")
        _close(_host64(dx), rdx, tol)
        _close(dw.cpu().numpy().astype(np.float64) - dw0, rdw, 1e-5 if dt == "f32" else 2e-5)
    m.close()


def test_gemm_tile_widths_at_scale():
    """Forward (NT) and backward-data (NN) products with thousands of rows, at
    output widths that select the 256-wide tile (3072) and the 192-wide tile
    (768, 2304), in one round of tiles (768) or over several rounds (3072,
    2304, and a ragged 8200 x 2056: 297 tiles, not a multiple of the 8 XCDs),
    checked on sampled rows (first, last, random) against the oracle run on
    those rows alone (each output row depends only on its input row)."""
    m = _model(G.GPT2_BF16_MIXED)
    rng = np.random.default_rng(2)
    R = 64
    for M, N in ((16384, 3072), (16384, 768), (16384, 2304), (8200, 2056)):
        rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.integers(0, M, 128)]))
        print(f"gemm tile width M={M} N={N}", flush=True)
        # forward: out[M,N] = x[M,R] W[N,R]^T + b
        x = _dev(rng.standard_normal((M, R)), torch.bfloat16)
        w = _dev(rng.standard_normal((N, R)) * 0.1, torch.bfloat16)
        bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32)).cuda()
        out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        G.gpt2_test_gemm_nt(m.h, out.data_ptr(), x.data_ptr(), w.data_ptr(), bias.data_ptr(), M, N, R)
        torch.cuda.synchronize()
        ref = O.matmul_forward(_host64(x)[rows], _host64(w), bias.cpu().numpy().astype(np.float64), prec="f64")
        _close(_host64(out)[rows], ref, 8e-3)
        # backward data: dX[M,N] = dY[M,R] W2[R,N]  (output width N, reduction R)
        dy = _dev(rng.standard_normal((M, R)), torch.bfloat16)
        w2 = _dev(rng.standard_normal((R, N)) * 0.1, torch.bfloat16)
        dx = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        G.gpt2_test_gemm_nn(m.h, dx.data_ptr(), dy.data_ptr(), w2.data_ptr(), M, R, N)
        torch.cuda.synchronize()
        rdx, _, _ = O.matmul_backward(_host64(dy)[rows], np.zeros((rows.size, N)), _host64(w2), prec="f64")
        _close(_host64(dx)[rows], rdx, 8e-3)
    m.close()


def test_gemm_plain_store_persistent():
    """Plain-store forward products (no bias) over at least two rounds of
    256 x 256 tiles, which run the persistent kernel with register-staged
    64-deep k-steps: a ragged output width (32776 = 128 tiles + 8 columns)
    over two k-steps, ragged rows (4104) over an odd five, and the
    classifier's width and depth (50304 x 768) at 1024 rows; sampled rows
    against the oracle on those rows alone."""
    m = _model(G.GPT2_BF16_MIXED)
    rng = np.random.default_rng(5)
    for M, N, K, nr in ((4096, 32776, 128, 128), (4104, 8192, 320, 128), (1024, 50304, 768, 48)):
        rows = np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), rng.integers(0, M, nr)]))
        print(f"plain-store gemm M={M} N={N} K={K}", flush=True)
        x = _dev(rng.standard_normal((M, K)), torch.bfloat16)
        w = _dev(rng.standard_normal((N, K)) * 0.1, torch.bfloat16)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        G.gpt2_test_gemm_nt(m.h, out.data_ptr(), x.data_ptr(), w.data_ptr(), None, M, N, K)
        torch.cuda.synchronize()
        # every element written (the NaN fill would survive an unwritten tile)
        assert not torch.isnan(out).any().item()
        ref = O.matmul_forward(_host64(x)[rows], _host64(w), None, prec="f64")
        _close(_host64(out)[rows], ref, 8e-3)
    m.close()


def test_gemm_split_k_weight_gradient():
    """The weight-gradient product with a long reduction (split over several
    workgroups, partials summed in a second kernel) against the oracle."""
    cfg = G.make_config(1, 64, 1, 64, 64, 64, 64, 64, G.GPT2_BF16_MIXED)  # B*T = 4096 tokens
    m = G.Model(cfg, 1)
    rng = np.random.default_rng(1)
    # the last case has a wide enough output (256 tiles of 256x256) to take the unsplit path
    for (M, N, K) in [(2048, 192, 64), (4096, 64, 64), (1024, 128, 64), (128, 4096, 4096)]:
        print(f"split-k gemm M={M} N={N} K={K}", flush=True)
        dy = _dev(rng.standard_normal((M, N)), torch.bfloat16)
        x = _dev(rng.standard_normal((M, K)), torch.bfloat16)
        dw0 = rng.standard_normal((N, K)).astype(np.float32)
        dw = torch.from_numpy(dw0).cuda()
        G.gpt2_test_gemm_tn(m.h, dw.data_ptr(), dy.data_ptr(), x.data_ptr(), M, N, K)
        torch.cuda.synchronize()
        _, rdw, _ = O.matmul_backward(_host64(dy), _host64(x), np.zeros((N, K)), prec="f64")
        _close(dw.cpu().numpy().astype(np.float64) - dw0, rdw, 2e-5)
    m.close()


@pytest.mark.parametrize("prec,B,T,NH,hs", [
    (G.GPT2_BF16_MIXED, 2, 320, 2, 64),   # ragged against the 128-row blocks
    (G.GPT2_BF16_MIXED, 1, 1024, 1, 64),  # the full sequence length
    (G.GPT2_BF16_MIXED, 2, 1024, 4, 64),  # 64 blocks: whole heads per XCD, blocks issued longest first
    (G.GPT2_BF16_MIXED, 3, 64, 3, 64),
    (G.GPT2_FP32, 2, 37, 3, 16),
    (G.GPT2_FP32, 1, 130, 2, 64),
])
def test_attention_vs_oracle(prec, B, T, NH, hs):
    C = NH * hs
    bf = prec == G.GPT2_BF16_MIXED
    tdt = torch.bfloat16 if bf else torch.float32
    # a model whose B*NH*T covers the case (its buffers hold the row sums D)
    cfg = G.make_config(1, C, NH, 1024, 64, 64, B, ((T + 63) // 64) * 64, prec)
    m = G.Model(cfg, 1)
    print(f"attention prec={prec} B={B} T={T} NH={NH} hs={hs}", flush=True)
    rng = np.random.default_rng(2)
    qkv = _dev(rng.standard_normal((B, T, 3 * C)), tdt)
    out = torch.zeros((B, T, C), dtype=tdt, device="cuda")
    lse = torch.zeros((B, NH, T), dtype=torch.float32, device="cuda")
    G.gpt2_test_attention_fwd(m.h, out.data_ptr(), lse.data_ptr(), qkv.data_ptr(), B, T, C, NH)
    dout = _dev(rng.standard_normal((B, T, C)), tdt)
    dqkv = torch.zeros_like(qkv)
    G.gpt2_test_attention_bwd(m.h, dqkv.data_ptr(), dout.data_ptr(), qkv.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, T, C, NH)
    torch.cuda.synchronize()
    q64 = _host64(qkv)
    ref, pre, att = O.attention_forward(q64, NH, prec="f64")
    tol = 2e-2 if bf else 1e-5
    _close(_host64(out), ref, tol)
    # lse: log of the softmax normaliser of the scaled scores over t2 <= t
    from scipy.special import logsumexp
    mask = np.tril(np.ones((T, T), bool))
    ref_lse = logsumexp(np.where(mask, pre, -np.inf), axis=-1)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=2e-2 if bf else 1e-5)
    # backward against the oracle run on the GPU's own forward output
    rdq = O.attention_backward(_host64(dout), q64, att, NH, prec="f64")
    _close(_host64(dqkv), rdq, 3e-2 if bf else 1e-5)
    m.close()
