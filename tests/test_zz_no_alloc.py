"""The allocation-free attention backward (gpt2_attention_bwd_noalloc), for
callers that cannot allocate, against the model-bound entry point that runs
the same kernels with the model's own scratch (gpt2_test_attention_bwd):
bit-identical gradients on two calls in a row, the second smaller, and the
size limit rejected with GPT2_EINVAL."""
import numpy as np
import pytest

from transformer_lm_train_amd import gpt2 as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _case(rng, B, T, NH, m):
    C = 64 * NH
    qkv = torch.from_numpy(rng.standard_normal((B, T, 3 * C)).astype(np.float32)).cuda().to(torch.bfloat16)
    out = torch.zeros((B, T, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, NH, T), dtype=torch.float32, device="cuda")
    G.gpt2_test_attention_fwd(m.h, out.data_ptr(), lse.data_ptr(), qkv.data_ptr(), B, T, C, NH)
    dout = torch.from_numpy(rng.standard_normal((B, T, C)).astype(np.float32)).cuda().to(torch.bfloat16)
    return qkv, out, lse, dout


def test_noalloc_attention_backward_matches_model_entry_point():
    # a model whose attention row buffer covers the larger case
    B0, T0, NH0 = 4, 1024, 3
    m = G.Model(G.make_config(1, 64 * NH0, NH0, 1024, 64, 64, B0, T0, G.GPT2_BF16_MIXED), 1)
    stream = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(5)
    for (B, T, NH) in [(B0, T0, NH0), (2, 320, 2)]:  # two calls in a row, the second smaller
        print(f"no-alloc attention backward B={B} T={T} NH={NH}", flush=True)
        C = 64 * NH
        qkv, out, lse, dout = _case(rng, B, T, NH, m)
        ref = torch.full_like(qkv, float("nan"))
        G.gpt2_test_attention_bwd(m.h, ref.data_ptr(), dout.data_ptr(), qkv.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, T, C, NH)
        got = torch.full_like(qkv, float("nan"))
        G.gpt2_attention_bwd_noalloc(stream, got.data_ptr(), dout.data_ptr(), qkv.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, T, C, NH)
        torch.cuda.synchronize()
        r, g = ref.float().cpu().numpy(), got.float().cpu().numpy()
        assert np.all(np.isfinite(r)) and np.abs(r).max() > 0
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    # beyond the static scratch: 2^20 + 64 rows
    with pytest.raises(G.GPT2Error) as e:
        G.gpt2_attention_bwd_noalloc(stream, 1, 1, 1, 1, 1, 1, 1024 + 64, 64 * 1024, 1024)
    assert e.value.code == G.GPT2_EINVAL
    m.close()
