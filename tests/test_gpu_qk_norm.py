"""GPU parity of the QK-norm option (per-head RMSNorm of q and k, with learned gains,
between the q|k|v projection and RoPE, as in the Qwen3 attention of the base model)
against the oracle.

* tiny float32 decoder: raw forwards (logits <= 1e-4, the paged K/V <= 1e-5),
  whole Psi-Spec iterations (tokens and accept lengths identical, probability TV
  <= 1e-3) and the distillation forward over [x, z1] (the KV-slot path);
* the Qwen3-8B layer shape in bf16: the q / K / V stage (and the rest of the layer)
  at batch 1 (the few-row kernels) and over 128 rows (the tile kernels), with the
  bounds of the other stage tests;
* the layer backward refuses QK-norm contexts (UNO_ERR_UNSUPPORTED)."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import distill, model, psispec
from tests import stage_check as sc
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

TINY = configs.TINY.with_(qk_norm=True)
CFG8 = configs.LAYER8B.with_(qk_norm=True)
LOGIT_TOL = 1e-4
TV_TOL = 1e-3


def _tv(a, b):
    return 0.5 * np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).sum(-1)


def test_tiny_qk_norm_forward_and_cache():
    log("tiny qk-norm forward")
    w = synth.weights_numpy(TINY, 1100, qk_gain_std=0.3)
    eng = engine(TINY, w, max_seqs=2, max_rows=40)
    r = np.random.default_rng(11)
    R = 12
    toks = r.integers(0, TINY.vocab, size=(2, R)).astype(np.int32)
    pos = np.tile(np.arange(R, dtype=np.int32), (2, 1))
    gate = (r.random((2, R)) < 0.5).astype(np.uint8)
    _, lg = eng.forward([0, 1], R, dev(pos.ravel()), dev(gate.ravel()), tokens=dev(toks.ravel()),
                        want_logits=True)
    cache = model.new_cache(TINY, 2, 40)
    ref, _ = model.forward(TINY, w, toks, pos, gate, cache)
    g = host(lg).reshape(2, R, -1)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin)
    err = np.abs(g[fin] - ref[fin]).max()
    log(f"  logits max |gpu-oracle| {err:.2e}")
    assert err <= LOGIT_TOL
    for s in range(2):
        k, v = eng.kv_export(s, R)
        assert np.abs(host(k) - cache["k"][:, s, :R]).max() <= 1e-5
        assert np.abs(host(v) - cache["v"][:, s, :R]).max() <= 1e-5
    eng.sync()


def test_tiny_qk_norm_decode_iterations():
    log("tiny qk-norm decode")
    w = synth.weights_numpy(TINY, 1101, lm_head_std=0.35, lora_b_std=0.6, qk_gain_std=0.3)
    S, seed = 3, 3100
    lens = [16, 5, 9]
    prompts = [synth.prompts(TINY, 2100 + i, 1, L)[0] for i, L in enumerate(lens)]
    ids = [2, 0, 1]
    eng = engine(TINY, w, max_seqs=S, max_seq_len=TINY.max_len + 40, seed=seed)
    eng.prefill(ids, prompts)
    dec = psispec.Decoder(TINY, w, ids, seed, TINY.max_len + 40)
    dec.prefill(prompts)
    for step in range(6):
        y_g, pd_g = eng.draft(ids, want_probs=True)
        out_g, n_g, pv_g = eng.verify(ids, want_probs=True)
        r = dec.step()
        assert _tv(host(pd_g), r["P_d"]).max() <= TV_TOL
        assert _tv(host(pv_g), r["P_v"]).max() <= TV_TOL
        assert np.array_equal(host(y_g), r["y"].astype(np.int32)), step
        assert np.array_equal(host(n_g), r["n_out"]), step
        assert np.array_equal(host(out_g), r["out"]), step
    for i, s in enumerate(ids):
        L, _, _ = eng.seq_state(s)
        assert L == int(dec.n[i])
        k, v = eng.kv_export(s, L)
        assert np.abs(host(k) - dec.cache["k"][:, i, :L]).max() <= 1e-5
        assert np.abs(host(v) - dec.cache["v"][:, i, :L]).max() <= 1e-5
    eng.sync()


def test_tiny_qk_norm_distill_forward():
    L, B, batch = 24, 4, 2
    log(f"tiny qk-norm distill L={L} B={B}")
    w = synth.weights_numpy(TINY, 1102, lm_head_std=0.35, lora_b_std=0.6, qk_gain_std=0.3)
    eng = engine(TINY, w, max_seqs=2, max_seq_len=2 * L + 8, max_rows=4 * L)
    x = synth.prompts(TINY, 7100, batch, L).astype(np.int32)
    T, S, _, _ = eng.distill_forward(dev(x), B)
    eng.sync()
    T_o, S_o, _, _ = distill.distill_forward(TINY, w, x, B)
    for g, o in ((host(T), T_o), (host(S), S_o)):
        fin = np.isfinite(o)
        assert np.array_equal(np.isfinite(g), fin)
        assert np.abs(g[fin] - o[fin]).max() <= LOGIT_TOL


@pytest.fixture(scope="module")
def w8():
    return synth.weights_numpy(CFG8, 1103, with_embed=False, qk_gain_std=0.3)


def test_layer8b_qk_norm_stages_batch1(w8):
    """16 draft rows at context 1024 (the few-row kernels)."""
    import torch
    ctx = 1024
    log(f"8B qk-norm stages batch 1, context {ctx}")
    eng = engine(CFG8, w8, max_seqs=1, max_seq_len=ctx + 64, max_rows=16)
    kc = torch.from_numpy(synth.normal(5101, (1, ctx, CFG8.n_kv_heads, CFG8.head_dim)))
    vc = torch.from_numpy(synth.normal(5102, (1, ctx, CFG8.n_kv_heads, CFG8.head_dim)))
    eng.kv_import(0, kc.to(torch.bfloat16).cuda(), vc.to(torch.bfloat16).cuda(), pending=0)
    pos = np.arange(ctx, ctx + 16)
    gate = np.r_[0, np.ones(15)]
    x = synth.normal(6101, (16, CFG8.d_model))
    bufs = eng.set_trace(16, [0])
    eng.forward([0], 16, dev(pos.astype(np.int32)), dev(gate.astype(np.uint8)), hidden_in=dev(x))
    tr = {f: host(t.float()).astype(np.float64) for f, t in bufs[0].items()}
    eng.set_trace(None)
    k, v = eng.kv_export(0, ctx + 16)
    K, V = host(k.float()).astype(np.float64)[0], host(v.float()).astype(np.float64)[0]
    sc.layer_stages(CFG8, w8["layers"][0], tr, np.arange(16), pos, gate, K, V, "qk-norm batch 1")
    eng.sync()


def test_layer8b_qk_norm_stages_128_rows(w8):
    """8 sequences x 16 draft rows (the tile kernels), contexts 40 .. 600."""
    import torch
    ctxs = [600, 40, 333, 97, 512, 64, 250, 175]
    n, rows = len(ctxs), 16
    log("8B qk-norm stages 8 sequences x 16 rows")
    eng = engine(CFG8, w8, max_seqs=n, max_seq_len=700, max_rows=n * rows)
    gen = torch.Generator(device="cuda").manual_seed(7322)
    for s_, c in enumerate(ctxs):
        shape = (1, c, CFG8.n_kv_heads, CFG8.head_dim)
        eng.kv_import(s_, torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16),
                      torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16), pending=0)
    pos = np.stack([np.arange(c, c + rows) for c in ctxs]).astype(np.int32)
    gate = (np.arange(n * rows).reshape(n, rows) % rows != 0).astype(np.uint8)
    x = synth.normal(7422, (n * rows, CFG8.d_model))
    bufs = eng.set_trace(n * rows, [0])
    eng.forward(list(range(n)), rows, dev(pos.ravel()), dev(gate.ravel()), hidden_in=dev(x))
    tr = {f: host(t.float()).astype(np.float64) for f, t in bufs[0].items()}
    eng.set_trace(None)
    for s_ in (0, 1, 5):
        k, v = eng.kv_export(s_, ctxs[s_] + rows)
        K = host(k.float()).astype(np.float64)[0]
        V = host(v.float()).astype(np.float64)[0]
        sc.layer_stages(CFG8, w8["layers"][0], tr, np.arange(s_ * rows, (s_ + 1) * rows), pos[s_],
                        gate[s_], K, V, f"qk-norm seq {s_} ctx {ctxs[s_]}")
    eng.sync()


def test_qk_norm_layer_backward_is_refused():
    import torch
    cfg = configs.TINY.with_(dtype="bf16", n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2,
                             head_dim=64, ffn_dim=512, vocab=512, lora_rank=32, lora_alpha=64.0,
                             block_size=4, qk_norm=True)
    w = synth.weights_numpy(cfg, 1104, with_embed=False, qk_gain_std=0.3)
    eng = engine(cfg, w, max_seqs=1, max_seq_len=64, max_rows=32)
    x = torch.zeros((16, cfg.d_model), device="cuda")
    kc = torch.zeros((1, 16, cfg.n_kv_heads, cfg.head_dim), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(uno.UnoError) as e:
        eng.lora_layer_backward(0, 4, x, kc, kc, x)
    assert e.value.status == 6
    eng.sync()
