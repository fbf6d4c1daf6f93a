"""GPU parity of the distillation-style forward over [x, z1] (one gated forward,
block-causal mask, teacher and student logits, per-row and per-block TV) against
the oracle.

Tiny fp32 decoder: logits <= 1e-4 abs; TV per row within the triangle-inequality
bound below.  One Qwen3-8B-shaped layer in bf16 with the full 151936 vocabulary:
logits with the bf16-noise tolerance derived in test_gpu_layer8b (two bf16
evaluations cannot agree more closely than either agrees with the exact result).

TV bound: |TV(pT, pS) - TV(qT, qS)| <= TV(pT, qT) + TV(pS, qS) (triangle
inequality of the L1 norm), so the GPU's TV may differ from the oracle's by at
most the distance between the two sides' probability rows, plus float32
summation error.  The TV kernel's own arithmetic is checked against TV recomputed
in float64 from the GPU's logits."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import distill, model
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

TINY = configs.TINY
LOGIT_TOL = 1e-4


def _probs64(logits):
    z = np.asarray(logits, np.float64)
    z = z - z.max(-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(-1, keepdims=True)


def _check_tv(tv_g, tvb_g, T_g, S_g, T_o, S_o, tv_o, B, slack):
    pT_g, pS_g = _probs64(T_g), _probs64(S_g)
    own = distill.tv_rows(pT_g, pS_g)
    assert np.abs(tv_g - own).max() <= 1e-5, "TV kernel arithmetic"
    bound = distill.tv_rows(pT_g, _probs64(T_o)) + distill.tv_rows(pS_g, _probs64(S_o)) + slack
    log(f"  tv: max |gpu-oracle| {np.abs(tv_g - tv_o).max():.2e}, max bound {bound.max():.2e}, "
        f"mean tv {tv_o.mean():.3f}")
    assert np.all(np.abs(tv_g - tv_o) <= bound)
    S, L = tv_g.shape
    blocks = tv_g.astype(np.float64).reshape(S, L // B, B).mean(-1)
    assert np.abs(tvb_g - blocks).max() <= 1e-6


@pytest.fixture(scope="module")
def tiny_w():
    return synth.weights_numpy(TINY, 1000, lm_head_std=0.35, lora_b_std=0.6)


@pytest.mark.parametrize("B", [1, 4, 12, 24])
def test_tiny_distill_forward(tiny_w, B):
    """L = 24 (not a multiple of 16: attention tiles mix x and z1 rows), batch 3
    over two scratch slots (groups of 2 and 1)."""
    L, batch = 24, 3
    log(f"tiny distill L={L} B={B}")
    eng = engine(TINY, tiny_w, max_seqs=2, max_seq_len=2 * L + 8, max_rows=4 * L)
    x = synth.prompts(TINY, 7000 + B, batch, L).astype(np.int32)
    T, S, tv, tvb = eng.distill_forward(dev(x), B)
    eng.sync()
    T_o, S_o, tv_o, tvb_o = distill.distill_forward(TINY, tiny_w, x, B)
    T_g, S_g = host(T), host(S)
    for g, o in ((T_g, T_o), (S_g, S_o)):
        fin = np.isfinite(o)
        assert np.array_equal(np.isfinite(g), fin)
        assert np.abs(g[fin] - o[fin]).max() <= LOGIT_TOL
    _check_tv(host(tv), host(tvb), T_g, S_g, T_o, S_o, tv_o, B, 1e-6)
    assert np.abs(host(tvb) - tvb_o).max() <= 1e-4
    assert eng.free_pages() == eng.n_pages


def test_tiny_distill_leaves_live_sequences_alone(tiny_w):
    log("tiny distill beside a live sequence")
    L = 16
    eng = engine(TINY, tiny_w, max_seqs=2, max_seq_len=64, max_rows=2 * L)
    prompt = synth.prompts(TINY, 7100, 1, 20)[0]
    eng.prefill([0], [prompt])
    eng.sync()
    k0, v0 = eng.kv_export(0, 19)
    k0, v0 = host(k0), host(v0)
    st0, free0 = eng.seq_state(0), eng.free_pages()
    x = synth.prompts(TINY, 7101, 2, L).astype(np.int32)
    T, S, tv, tvb = eng.distill_forward(dev(x), 4)
    eng.sync()
    T_o, S_o, tv_o, _ = distill.distill_forward(TINY, tiny_w, x, 4)
    assert np.abs(host(T)[np.isfinite(T_o)] - T_o[np.isfinite(T_o)]).max() <= LOGIT_TOL
    assert np.abs(host(S)[np.isfinite(S_o)] - S_o[np.isfinite(S_o)]).max() <= LOGIT_TOL
    k1, v1 = eng.kv_export(0, 19)
    assert np.array_equal(host(k1), k0) and np.array_equal(host(v1), v0)
    assert eng.seq_state(0) == st0 and eng.free_pages() == free0


def test_tiny_distill_errors(tiny_w):
    eng = engine(TINY, tiny_w, max_seqs=1, max_seq_len=64, max_rows=32)
    x = dev(synth.prompts(TINY, 7200, 1, 16).astype(np.int32))
    with pytest.raises(uno.UnoError, match="INVALID_ARG"):
        eng.distill_forward(x, 5)                     # L % B != 0
    big = dev(synth.prompts(TINY, 7201, 1, 24).astype(np.int32))
    with pytest.raises(uno.UnoError, match="INVALID_ARG"):
        eng.distill_forward(big, 4)                   # 2L > max_rows
    eng.prefill([0], [synth.prompts(TINY, 7202, 1, 8)[0]])
    with pytest.raises(uno.UnoError, match="OUT_OF_PAGES"):
        eng.distill_forward(x, 4)                     # the only slot is live
    eng.release(0)
    eng.distill_forward(x, 4)
    eng.prefill([0], [synth.prompts(TINY, 7203, 1, 8)[0]])
    eng.draft([0])
    with pytest.raises(uno.UnoError, match="STATE"):
        eng.distill_forward(x, 4)                     # a block awaits verification
    eng.verify([0])
    eng.sync()


CFG8 = configs.LAYER8B


@pytest.fixture(scope="module")
def w8():
    log("layer8b distill: generating weights (with embedding and LM head)")
    return synth.weights_numpy(CFG8, 1001, with_embed=True)


@pytest.mark.parametrize("L,B", [(48, 8), (64, 16), (64, 4), (64, 32)])
def test_layer8b_distill_forward(w8, L, B):
    """L = 48: the LM head runs on the skinny kernel (48 rows); L = 64: the large-M
    kernels; B = 4 and 8: one 16-row attention tile spans several blocks; B = 32: a
    block spans two tiles."""
    log(f"layer8b distill L={L} B={B}")
    eng = engine(CFG8, w8, max_seqs=1, max_seq_len=2 * L + 16, max_rows=2 * L)
    x = synth.prompts(CFG8, 7300 + L + B, 1, L).astype(np.int32)
    T, S, tv, tvb = eng.distill_forward(dev(x), B)
    eng.sync()
    T_g, S_g = host(T), host(S)
    T_o, S_o, tv_o, _ = distill.distill_forward(CFG8, w8, x, B)
    T_e, S_e, _, _ = distill.distill_forward(CFG8.with_(dtype="f32"), w8, x, B)
    for name, g, o, e in (("teacher", T_g, T_o, T_e), ("student", S_g, S_o, S_e)):
        fin = np.isfinite(o)
        assert np.array_equal(np.isfinite(g), fin)
        err = np.abs(g[fin] - o[fin])
        noise = np.abs(o[fin] - e[fin])
        tol = max(3e-2, 2.0 * float(noise.max()))
        gex = np.abs(g[fin] - e[fin]).mean()
        log(f"  {name}: max |gpu-oracle| {err.max():.3e} (bound {tol:.3e}); mean "
            f"{err.mean():.2e}, |gpu-exact| {gex:.2e}, |oracle-exact| {noise.mean():.2e}")
        assert err.max() <= tol
        assert err.mean() <= noise.mean()
        assert gex <= 1.25 * noise.mean()
    _check_tv(host(tv), host(tvb), T_g, S_g, T_o, S_o, tv_o, B, 1e-5)
    del eng


def test_layer8b_distill_needs_whole_row_blocks(w8):
    eng = engine(CFG8, w8, max_seqs=1, max_seq_len=96, max_rows=80)
    x = dev(synth.prompts(CFG8, 7399, 1, 40).astype(np.int32))
    with pytest.raises(uno.UnoError, match="INVALID_ARG"):
        eng.distill_forward(x, 8)
