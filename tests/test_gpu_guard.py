"""The non-finite gradient guard of the update, through the C ABI.

The pyshine.com tour of llm.c (global-norm header) clips by the global
gradient norm and skips updates on outliers.  Here a NaN or inf gradient
makes the norm non-finite; the update must then leave every parameter, the
AdamW moments and the bf16 weights bit for bit as they were, whether the norm
is read back on the host (the call itself returns GPT2_ERANGE) or stays on
the device (clip with norm == NULL: the AdamW kernel refuses, and the next
gpt2_sync reports GPT2_ERANGE once).  NaN arithmetic does not fault the GPU.
"""
import numpy as np
import pytest

from transformer_lm_train_amd import gpt2 as G
from transformer_lm_train_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

D = dict(L=2, C=128, NH=2, maxT=128, V=1000, Vp=1024)
HP = dict(lr=6e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _state(m):
    """Parameters, m, v and the raw bf16 weights (None in fp32 mode), as host copies."""
    mm, vv = m.opt_state()
    sh = None
    ptr = G.lib().gpt2_device_shadow(m.h)
    if ptr:
        off = ptr - m.buf.data_ptr()
        sh = m.buf[off:off + 2 * G.gpt2_num_params(m.h)].cpu().numpy().copy()
    return m.params(), mm, vv, sh


def _same(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("prec", [G.GPT2_BF16_MIXED, G.GPT2_BF16_SR, G.GPT2_FP32], ids=["bf16", "sr", "fp32"])
@pytest.mark.parametrize("bad", [np.nan, np.inf], ids=["nan", "inf"])
def test_nonfinite_gradient_refused(prec, bad):
    B, T = 2, 64
    print(f"non-finite guard prec={prec} bad={bad}", flush=True)
    m = G.Model(G.make_config(D["L"], D["C"], D["NH"], D["maxT"], D["V"], D["Vp"], B, T, prec), 5)
    x, y = synth.batch(5, 0, B, T, D["V"], "uniform")
    # one ordinary step, so that m and v are not zero
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    m.clip_grad_norm(1.0, read_norm=False)
    m.adamw_step(t=1, **HP)
    m.sync()
    # a second backward, then one gradient element made non-finite
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    g = m.grads()
    g[len(g) // 3] = bad
    m.set_grads(g)
    before = _state(m)
    # norm stays on the device: the kernel refuses, nothing is raised yet
    m.clip_grad_norm(1.0, read_norm=False)
    m.adamw_step(t=2, **HP)
    with pytest.raises(G.GPT2Error) as e:
        m.sync()
    assert e.value.code == G.GPT2_ERANGE
    _same(_state(m), before)
    m.sync()  # reported once, then cleared
    # norm read on the host: the clip call and the update both refuse
    with pytest.raises(G.GPT2Error) as e:
        m.clip_grad_norm(1.0)
    assert e.value.code == G.GPT2_ERANGE
    with pytest.raises(G.GPT2Error) as e:
        m.adamw_step(t=2, **HP)
    assert e.value.code == G.GPT2_ERANGE
    _same(_state(m), before)
    # finite gradients again: the update goes through
    g[len(g) // 3] = 0.0
    m.set_grads(g)
    m.clip_grad_norm(1.0, read_norm=False)
    m.adamw_step(t=2, **HP)
    m.sync()
    after = _state(m)
    assert not np.array_equal(after[0], before[0])
    assert np.all(np.isfinite(after[0])) and np.all(np.isfinite(after[1])) and np.all(np.isfinite(after[2]))
    m.close()


def test_refusal_reported_by_the_next_loss_read():
    """The refusal also surfaces at the next read-back of a loss, with the
    loss itself still delivered (gpt2_read_loss)."""
    B, T = 2, 64
    m = G.Model(G.make_config(D["L"], D["C"], D["NH"], D["maxT"], D["V"], D["Vp"], B, T, G.GPT2_BF16_MIXED), 9)
    x, y = synth.batch(9, 0, B, T, D["V"], "uniform")
    m.forward(x, y)
    m.zero_grad()
    m.backward()
    g = m.grads()
    g[7] = np.nan
    m.set_grads(g)
    m.clip_grad_norm(1.0, read_norm=False)
    m.adamw_step(t=1, **HP)
    m.forward(x, y, read_loss=False)
    loss = G.ctypes.c_float()
    rc = G.lib().gpt2_read_loss(m.h, G.ctypes.byref(loss))
    assert rc == G.GPT2_ERANGE
    assert np.isfinite(loss.value) and abs(loss.value - np.log(D["V"])) < 0.5
    assert G.gpt2_read_loss(m.h) == pytest.approx(loss.value)  # cleared after one report
    m.close()
