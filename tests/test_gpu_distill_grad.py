"""GPU parity of the distillation backward (the gradient of the block-wise TV loss
with respect to the gated LoRA, base frozen) against the oracle
(oracle/distill_grad.py), stage by stage and end to end.

* TV gradient at the logits (uno_tv_backward) on identical float32 logits of the
  full 151936 vocabulary: per element within 1e-4 of the element's natural scale
  p_S(v) / N (float32 softmax over 1.5e5 terms: relative error ~1e-5), except
  where the oracle's p_S and p_T differ by less than 1e-5 relative, where the sign
  of p_S - p_T is not decided by float32 (those entries' whole effect, through the
  row's centring sum, is bounded separately); TV_i within 1e-5.
* LM-head backward (uno_lm_head_backward) on identical inputs: per element within
  a bound propagated from the arithmetic (two-term gradient: relative 2^-18 per
  term; float32 accumulation over K terms: ~sqrt(K) 2^-24 of sum |terms|; the
  norm backward's own float32 rounding).
* One layer (uno_lora_layer_backward) on identical inputs -- the layer input, the
  x rows' K/V, dL/d(output) -- at the Qwen3-8B shape and on a small config over
  block sizes 1..L: the GPU recomputes the gate-on forward with bf16 storage, and
  two bf16-storage evaluations differ by rounding-boundary flips, so the GPU is
  compared with the bf16-storage oracle with a bound tied to how far that oracle
  sits from the exact (unrounded) one: a relative Frobenius error within half of
  that distance (flips touch a small fraction of the values the exact-vs-bf16
  distance perturbs everywhere) plus 1e-4 (float32), and never above 1e-2.
* The whole backward after a checkpointed distillation forward (uno_distill_backward)
  on a two-layer bf16 model: the checkpoint against the oracle's forward, the
  loss, and the gradients with the same kind of bound.
"""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import distill_grad as dg, model
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

PROJ = model.PROJ
SMALL = configs.TINY.with_(name="small-bf16", dtype="bf16", n_layers=2, d_model=256,
                           n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=512, vocab=512,
                           lora_rank=32, lora_alpha=64.0, block_size=4)


def _bf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _weights(cfg, seed, with_embed=True):
    w = synth.weights_numpy(cfg, seed, with_embed=with_embed, lora_b_std=0.05,
                            lm_head_std=0.1 if with_embed else None)
    r = np.random.default_rng(seed)
    for lw in w["layers"]:
        for k in ("attn_norm", "mlp_norm"):
            lw[k] = _bf(1.0 + 0.2 * r.standard_normal(cfg.d_model))
    w["final_norm"] = _bf(1.0 + 0.2 * r.standard_normal(cfg.d_model))
    return w


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- TV gradient

@pytest.mark.parametrize("V,rows", [(151936, 48), (512, 200)])
def test_tv_backward(V, rows):
    import torch
    log(f"tv_backward V={V} rows={rows}")
    r = np.random.default_rng(V + rows)
    T = (r.standard_normal((rows, V)) * 1.5).astype(np.float32)
    S = (T + r.standard_normal((rows, V)) * 0.7).astype(np.float32)
    T[:, -1] = S[:, -1] = -np.inf                     # the MASK column
    n_total = 4 * rows                                # this call is a slice of a larger loss
    dz, tv = uno.tv_backward(dev(T), dev(S), n_total)
    dz, tv = host(dz), host(tv)
    pT, pS = dg.softmax64(T), dg.softmax64(S)
    ref = dg.tv_logit_grad(T, S) * rows / n_total     # the oracle's N is this call's rows
    assert np.abs(tv - 0.5 * np.abs(pT - pS).sum(-1)).max() <= 1e-5
    scale = pS / n_total
    tie = np.abs(pS - pT) <= 1e-5 * np.maximum(pS, pT)
    ok = ~tie
    err = np.abs(dz - ref)
    log(f"  max err / scale {np.max(err[ok] / np.maximum(scale[ok], 1e-300)):.2e}, ties {tie.sum()}")
    assert np.all(err[ok] <= 1e-4 * scale[ok] + 1e-12 / n_total)
    # a near-tie entry may take either sign: its own value stays within 2 p_S / 2N
    # of the oracle's, and it moves the row's centring sum by at most 2 p_S
    shift = (2 * pS * tie).sum(-1, keepdims=True)
    assert np.all(err <= 1e-4 * scale + pS * shift / (2 * n_total) + 2 * pS * tie / (2 * n_total) + 1e-12)
    assert np.all(dz[:, -1] == 0)


# ---------------------------------------------------------------- LM head

def test_lm_head_backward():
    import torch
    cfg = SMALL.with_(vocab=151936, n_layers=1)
    log("lm_head_backward V=151936 d=256")
    w = _weights(cfg, 9100)
    eng = engine(cfg, w, max_seqs=1, max_seq_len=64, max_rows=64)
    rows = 48
    r = np.random.default_rng(9101)
    xf = r.standard_normal((rows, cfg.d_model)).astype(np.float32)
    dz = (r.standard_normal((rows, cfg.vocab)) * 1e-3).astype(np.float32)
    dx = host(eng.lm_head_backward(dev(xf), dev(dz)))
    W = w["lm_head"].astype(np.float64)
    ref = dg.lm_head_backward(cfg, w, xf.astype(np.float64), dz.astype(np.float64))
    # bound propagated from the arithmetic
    K = cfg.vocab
    Sabs = np.abs(dz.astype(np.float64)) @ np.abs(W)
    Bdh = (2.0 ** -18 + 4 * np.sqrt(K) * 2.0 ** -24) * Sabs
    x = xf.astype(np.float64)
    gain = w["final_norm"].astype(np.float64)
    rs = 1 / np.sqrt(np.mean(x * x, -1, keepdims=True) + cfg.rms_eps)
    hg = model.bf16_round(x * gain)
    dh = dz.astype(np.float64) @ W
    bound = (rs * np.abs(gain) * Bdh + np.abs(x) * rs ** 3 * np.mean(np.abs(hg) * Bdh, -1, keepdims=True)
             + 1e-5 * (rs * np.abs(gain * dh) + np.abs(x) * rs ** 3 * np.mean(np.abs(hg * dh), -1, keepdims=True)))
    err = np.abs(dx - ref)
    log(f"  max err / bound {np.max(err / bound):.3f}, rel {_rel(dx, ref):.2e}")
    assert np.all(err <= bound)


# ---------------------------------------------------------------- one layer

def _layer_case(cfg, w, eng, batch, L, B, seed):
    import torch
    r = np.random.default_rng(seed)
    xin = r.standard_normal((batch * L, cfg.d_model)).astype(np.float32)
    kc = _bf(r.standard_normal((batch, L, cfg.n_kv_heads, cfg.head_dim)))
    vc = _bf(r.standard_normal((batch, L, cfg.n_kv_heads, cfg.head_dim)))
    dy = r.standard_normal((batch * L, cfg.d_model)).astype(np.float32)
    log(f"  layer backward batch={batch} L={L} B={B}")
    dx, ga, gb = eng.lora_layer_backward(0, B, dev(xin), dev(kc, torch.bfloat16),
                                         dev(vc, torch.bfloat16), dev(dy))
    eng.sync()
    got = {"dx": host(dx)}
    for p in PROJ:
        got["A_" + p], got["B_" + p] = host(ga[p]), host(gb[p])
    lw = w["layers"][0]
    ref, exact = {}, {}
    for c, out in ((cfg, ref), (cfg.with_(dtype="f32"), exact)):
        lw64 = {"attn_norm": lw["attn_norm"].astype(np.float64), "mlp_norm": lw["mlp_norm"].astype(np.float64),
                "w": lw["w"], "la": lw["la"], "lb": lw["lb"]}
        _, sv = dg.layer_forward_saved(c, lw64, xin.reshape(batch, L, -1).astype(np.float64),
                                       kc.astype(np.float64), vc.astype(np.float64), B)
        dxo, grads = dg.layer_backward(c, lw64, sv, dy.reshape(batch, L, -1).astype(np.float64))
        out["dx"] = dxo.reshape(batch * L, -1)
        for p in PROJ:
            out["A_" + p], out["B_" + p] = grads[p]
    worst = 0.0
    for k in got:
        e_gpu, e_bf = _rel(got[k], ref[k]), _rel(ref[k], exact[k])
        bound = min(1e-2, 0.5 * e_bf + 1e-4)
        log(f"    {k:7s} gpu-vs-bf16 {e_gpu:.2e}  bf16-vs-exact {e_bf:.2e}  bound {bound:.2e}")
        assert e_gpu <= bound, k
        worst = max(worst, e_gpu / bound)
    return worst


@pytest.fixture(scope="module")
def small_eng():
    w = _weights(SMALL.with_(n_layers=1), 9200, with_embed=False)
    eng = engine(SMALL.with_(n_layers=1), w, max_seqs=1, max_seq_len=128, max_rows=64)
    return w, eng


@pytest.mark.parametrize("batch,L,B", [(3, 32, 4), (2, 32, 32), (1, 48, 1), (2, 16, 8)])
def test_layer_backward_small(small_eng, batch, L, B):
    w, eng = small_eng
    log(f"small layer backward batch={batch} L={L} B={B}")
    _layer_case(SMALL.with_(n_layers=1), w, eng, batch, L, B, 9300 + 10 * B + L)


def test_layer_backward_8b():
    cfg = configs.LAYER8B
    log("8B layer backward: generating weights")
    w = _weights(cfg, 9400, with_embed=False)
    eng = engine(cfg, w, max_seqs=1, max_seq_len=256, max_rows=64)
    _layer_case(cfg, w, eng, 2, 64, 16, 9401)


# ---------------------------------------------------------------- whole backward

def test_distill_backward_two_layers():
    import torch
    cfg = SMALL
    batch, L, B = 3, 32, 8
    log(f"distill backward {cfg.n_layers} layers batch={batch} L={L} B={B}")
    w = _weights(cfg, 9500)
    w["lm_head"] = _bf(synth.normal(9501, w["lm_head"].shape) * 0.2)
    eng = engine(cfg, w, max_seqs=2, max_seq_len=2 * L + 16, max_rows=4 * L)
    x = synth.prompts(cfg, 9502, batch, L).astype(np.int32)
    ck = eng.set_distill_checkpoint(batch, L)
    T, S, _, _ = eng.distill_forward(dev(x), B)
    loss, tv, ga, gb = eng.distill_backward(B, T, S)
    eng.sync()
    # deterministic: a second backward gives the same bits (fixed-order reductions only)
    loss2, tv2, ga2, gb2 = eng.distill_backward(B, T, S)
    eng.sync()
    assert np.array_equal(host(loss), host(loss2)) and np.array_equal(host(tv), host(tv2))
    for p in PROJ:
        assert np.array_equal(host(ga[p]), host(ga2[p])) and np.array_equal(host(gb[p]), host(gb2[p]))
    eng.set_distill_checkpoint(None, L)
    # checkpoint against the oracle's forward (bf16 storage): within forward noise
    ock = dg.distill_checkpoint(cfg, w, x, B)
    xs = host(ck["x"]).reshape(cfg.n_layers + 1, batch, L, -1)
    for l in range(cfg.n_layers):
        assert _rel(xs[l], ock["x_in"][l]) <= 1e-2, l
        assert _rel(host(ck["k"].float())[:, l], ock["k"][l]) <= 1e-2
        assert _rel(host(ck["v"].float())[:, l], ock["v"][l]) <= 1e-2
    assert _rel(xs[-1], ock["x_final"]) <= 1e-2
    # the oracle's gradient at the GPU's own forward values (teacher / student logits,
    # checkpoint): stage-isolated, so the bound of the layer tests applies
    Tg, Sg = host(T), host(S)
    ref_loss = dg.tv_loss(Tg, Sg)
    log(f"  loss gpu {host(loss)[0]:.6f} oracle-at-gpu-logits {ref_loss:.6f}")
    assert abs(host(loss)[0] - ref_loss) <= 1e-5
    dz = dg.tv_logit_grad(Tg, Sg)
    dz = np.where(np.isfinite(Sg), dz, 0.0)
    wf = {k: v for k, v in w.items()}
    dy = dg.lm_head_backward(cfg, wf, xs[-1].reshape(batch * L, -1).astype(np.float64),
                             dz.reshape(batch * L, -1)).reshape(batch, L, -1)
    kk, vv = host(ck["k"].float()).astype(np.float64), host(ck["v"].float()).astype(np.float64)
    exact_cfg = cfg.with_(dtype="f32")
    dy_e = dy.copy()
    for l in reversed(range(cfg.n_layers)):
        lw = w["layers"][l]
        xin = xs[l].astype(np.float64)
        _, sv = dg.layer_forward_saved(cfg, lw, xin, kk[:, l], vv[:, l], B)
        dy, grads = dg.layer_backward(cfg, lw, sv, dy)
        _, sve = dg.layer_forward_saved(exact_cfg, lw, xin, kk[:, l], vv[:, l], B)
        dy_e, grads_e = dg.layer_backward(exact_cfg, lw, sve, dy_e)
        for p in PROJ:
            for j, (gpu, name) in enumerate(((ga[p], "A"), (gb[p], "B"))):
                g = host(gpu)[l]
                e_gpu, e_bf = _rel(g, grads[p][j]), _rel(grads[p][j], grads_e[p][j])
                bound = min(1e-2, 0.5 * e_bf + 1e-4)
                log(f"    layer {l} {name}_{p:5s} gpu-vs-bf16 {e_gpu:.2e} bf16-vs-exact {e_bf:.2e}")
                assert e_gpu <= bound, (l, p, name)


def test_backward_rejects_bad_calls(small_eng):
    w, eng = small_eng
    import torch
    with pytest.raises(uno.UnoError):      # checkpoint armed for another shape
        eng.set_distill_checkpoint(2, 16)
        try:
            eng.distill_forward(dev(np.zeros((1, 16), np.int32)), 4)
        finally:
            eng.set_distill_checkpoint(None, 16)
    x = torch.zeros((16, SMALL.d_model), device="cuda")
    kc = torch.zeros((1, 16, SMALL.n_kv_heads, SMALL.head_dim), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(uno.UnoError):      # L not a multiple of B
        eng.lora_layer_backward(0, 5, x, kc, kc, x)
    with pytest.raises(uno.UnoError):      # layer out of range
        eng.lora_layer_backward(1, 4, x, kc, kc, x)
