"""Pins of the oracle's forward: library routines (torch float64 rms_norm, SDPA,
bfloat16 conversion), closed forms (rotations, single-key attention), and
invariants (incremental decoding with the cache equals the full causal forward;
gate 0 is the base path and gate 1 the merged weight)."""
import math

import numpy as np
import pytest
import torch

from diffusion_drafted_lora_amd import configs, synth
from oracle import model

TINY = configs.TINY


@pytest.fixture(scope="module")
def tiny_w():
    return synth.weights_numpy(TINY, 1000)


def test_bf16_round_matches_torch_conversion():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-30).astype(np.float32),
        (r.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties between bf16 neighbours: 1 + 2^-8 (tie, even down), 1 + 3*2^-8 (tie, up)
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0, 2**-130, 3 * 2**-134],
                 dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = model.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_rms_norm_library_and_closed_form():
    r = np.random.default_rng(1)
    x = r.standard_normal((7, 64)) * 3.0
    g = r.standard_normal(64)
    y = model.rms_norm(x, g, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), 1e-6)
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    y1 = model.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt(np.mean(y1 * y1, axis=-1)), 1.0, atol=1e-12)


def test_rope_is_a_rotation_by_position():
    r = np.random.default_rng(2)
    # head_dim 2: a single pair rotated by angle pos * theta^0 = pos (complex multiply)
    x = r.standard_normal((5, 1, 2))
    pos = np.arange(5)
    y = model.rope(x, pos, 1e6)
    z = (x[:, 0, 0] + 1j * x[:, 0, 1]) * np.exp(1j * pos)
    assert np.allclose(y[:, 0, 0], z.real) and np.allclose(y[:, 0, 1], z.imag)
    # norms are preserved and scores depend only on the position difference
    q = r.standard_normal((1, 16))
    k = r.standard_normal((1, 16))
    s = [float(np.sum(model.rope(q[None], np.array([m]), 1e4) *
                      model.rope(k[None], np.array([m - 3]), 1e4))) for m in (3, 10, 40)]
    assert np.allclose(s, s[0], rtol=1e-10)
    assert np.allclose(np.linalg.norm(model.rope(q[None], np.array([17]), 1e4)),
                       np.linalg.norm(q))
    # pair (i, i + hd/2) uses frequency theta^(-2i/hd)
    e = np.zeros((1, 1, 8))
    e[0, 0, 1] = 1.0
    y = model.rope(e, np.array([1]), 100.0)
    ang = 100.0 ** (-2 * 1 / 8)
    assert np.isclose(y[0, 0, 1], math.cos(ang)) and np.isclose(y[0, 0, 5], math.sin(ang))


def test_attention_against_torch_sdpa_and_closed_forms():
    r = np.random.default_rng(3)
    S, R, J, Hq, Hkv, hd = 2, 5, 9, 8, 2, 16
    q = r.standard_normal((S, R, Hq, hd))
    K = r.standard_normal((S, J, Hkv, hd))
    V = r.standard_normal((S, J, Hkv, hd))
    vis = r.random((S, R, J)) < 0.6
    vis[..., 0] = True
    o = model.attention(q, K, V, vis)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                       # S,Hq,R,hd
    tk = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    mask = torch.from_numpy(vis)[:, None]                             # S,1,R,J
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)
    # one visible key returns its value; q = 0 averages the visible values
    vis1 = np.zeros((S, R, J), dtype=bool)
    vis1[:, :, 4] = True
    o1 = model.attention(q, K, V, vis1)
    assert np.allclose(o1, np.repeat(V[:, None, 4], G, axis=2)[:, None].repeat(R, 1)[:, :, :, :]
                       .reshape(S, R, Hq, hd))
    o0 = model.attention(np.zeros_like(q), K, V, vis)
    mean = np.einsum("srj,sjkd->srkd", vis / vis.sum(-1, keepdims=True), V)
    assert np.allclose(o0, np.repeat(mean, G, axis=2))


def test_gated_lora_special_cases():
    """gate 0 is bit-identical to the base GEMM; gate 1 equals the merged weight."""
    r = np.random.default_rng(4)
    h = r.standard_normal((6, 32))
    W = r.standard_normal((24, 32))
    A = r.standard_normal((8, 32))
    Bm = r.standard_normal((24, 8))
    gate = np.array([0, 1, 0, 1, 1, 0], dtype=np.float64)
    y = model.gated_lora_linear(TINY, h, W, A, Bm, gate)
    s = TINY.lora_alpha / TINY.lora_rank
    base = h @ W.T
    assert np.array_equal(y[gate == 0], base[gate == 0])
    merged = h @ (W + s * Bm @ A).T
    assert np.allclose(y[gate == 1], merged[gate == 1], rtol=1e-12, atol=1e-12)


STORE_POINTS = ("norm", "lora", "q", "k", "v", "attn", "act")


def _torch_forward(cfg, w, tokens, gate, store=()):
    """Independent float64 causal forward from torch library routines (linear,
    rms_norm, scaled_dot_product_attention with is_causal, silu).  ``store`` names
    the values rounded to bfloat16 (torch's conversion) as a bf16 configuration
    stores them: "norm" the gain-scaled RMSNorm input x * g (times the exact
    1 / rms), "lora" the scaled LoRA intermediate, "q" / "k" after RoPE, "v", "attn"
    the attention output and "act" the SwiGLU product."""
    F = torch.nn.functional
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    st = {p: (lambda t: t.to(torch.bfloat16).to(torch.float64)) if p in store else (lambda t: t)
          for p in STORE_POINTS}
    x = T(w["embed"])[torch.from_numpy(np.asarray(tokens))]            # [R, d]
    R = x.shape[0]
    g = T(gate)[:, None]
    s = cfg.lora_alpha / cfg.lora_rank
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    half = hd // 2
    inv = cfg.rope_theta ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
    ang = torch.arange(R, dtype=torch.float64)[:, None] * inv[None]
    cos, sin = torch.cos(ang)[:, None], torch.sin(ang)[:, None]

    def rot(t):
        a, b = t[..., :half], t[..., half:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], -1)

    def norm(xx, gain):
        if "norm" not in store:
            return F.rms_norm(xx, (cfg.d_model,), T(gain), cfg.rms_eps)
        rs = torch.rsqrt(xx.pow(2).mean(-1, keepdim=True) + cfg.rms_eps)
        return st["norm"](xx * T(gain)) * rs

    for lw in w["layers"]:
        def lin(p, hh):
            u = st["lora"](s * F.linear(hh, T(lw["la"][p])))
            return F.linear(hh, T(lw["w"][p])) + g * F.linear(u, T(lw["lb"][p]))
        h = norm(x, lw["attn_norm"])
        qr, kr = lin("q", h).view(R, Hq, hd), lin("k", h).view(R, Hkv, hd)
        if cfg.qk_norm:
            qr = F.rms_norm(qr, (hd,), T(lw["q_norm"]), cfg.rms_eps)
            kr = F.rms_norm(kr, (hd,), T(lw["k_norm"]), cfg.rms_eps)
        q = st["q"](rot(qr)).transpose(0, 1)
        k = st["k"](rot(kr)).transpose(0, 1)
        v = st["v"](lin("v", h).view(R, Hkv, hd)).transpose(0, 1)
        k = k.repeat_interleave(Hq // Hkv, 0)
        v = v.repeat_interleave(Hq // Hkv, 0)
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
        x = x + lin("o", st["attn"](o.transpose(0, 1).reshape(R, Hq * hd)))
        h2 = norm(x, lw["mlp_norm"])
        x = x + lin("down", st["act"](F.silu(lin("gate", h2)) * lin("up", h2)))
    hf = norm(x, w["final_norm"])
    logits = F.linear(hf, T(w["lm_head"]))
    logits[:, cfg.mask_id] = -float("inf")
    return logits.numpy()


def test_forward_matches_torch_library_forward(tiny_w):
    r = np.random.default_rng(5)
    R = 12
    toks = r.integers(0, TINY.vocab, size=R)
    gate = (r.random(R) < 0.5).astype(np.float64)
    ref = _torch_forward(TINY, tiny_w, toks, gate)
    cache = model.new_cache(TINY, 1, R)
    logits, _ = model.forward(TINY, tiny_w, toks[None], np.arange(R)[None], gate[None], cache)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(logits[0]))
    assert np.allclose(logits[0][fin], ref[fin], rtol=1e-9, atol=1e-12)


def test_incremental_decode_equals_full_forward(tiny_w):
    """Feeding rows one at a time (or in blocks) through the cache gives the same
    logits as the full causal forward, and leaves the same cache."""
    r = np.random.default_rng(6)
    R = 11
    toks = r.integers(0, TINY.vocab - 1, size=R)
    full_cache = model.new_cache(TINY, 1, R + 4)
    full, _ = model.forward(TINY, tiny_w, toks[None], np.arange(R)[None], np.zeros((1, R)),
                            full_cache)
    for chunk in (1, 3, 4):
        cache = model.new_cache(TINY, 1, R + 4)
        outs = []
        for a in range(0, R, chunk):
            b = min(R, a + chunk)
            lg, _ = model.forward(TINY, tiny_w, toks[None, a:b], np.arange(a, b)[None],
                                  np.zeros((1, b - a)), cache)
            outs.append(lg[0])
        inc = np.concatenate(outs)
        assert np.allclose(inc, full[0], rtol=1e-10, atol=1e-12)
        assert np.allclose(cache["k"], full_cache["k"], rtol=1e-12, atol=1e-14)
        assert np.allclose(cache["v"], full_cache["v"], rtol=1e-12, atol=1e-14)


def test_stale_cache_entries_beyond_a_row_are_invisible(tiny_w):
    """Garbage beyond a row's position in the cache does not change its output."""
    r = np.random.default_rng(7)
    toks = r.integers(0, TINY.vocab - 1, size=6)
    c1 = model.new_cache(TINY, 1, 16)
    c2 = model.new_cache(TINY, 1, 16)
    c2["k"][:, :, 6:] = r.standard_normal(c2["k"][:, :, 6:].shape) * 50
    c2["v"][:, :, 6:] = r.standard_normal(c2["v"][:, :, 6:].shape) * 50
    a, _ = model.forward(TINY, tiny_w, toks[None], np.arange(6)[None], np.zeros((1, 6)), c1)
    b, _ = model.forward(TINY, tiny_w, toks[None], np.arange(6)[None], np.zeros((1, 6)), c2)
    assert np.array_equal(a, b)


def test_mask_logit_and_probs():
    r = np.random.default_rng(8)
    l = r.standard_normal((3, 10))
    l[:, 9] = -np.inf
    p = model.probs(l)
    assert p.dtype == np.float32
    assert np.all(p[:, 9] == 0)
    ref = torch.softmax(torch.from_numpy(l), -1).numpy().astype(np.float32)
    assert np.allclose(p, ref, rtol=1e-6, atol=1e-9)


def test_bf16_storage_points_are_bf16(tiny_w):
    """In a bf16 configuration every cached K/V value is bf16-representable."""
    cfg = TINY.with_(dtype="bf16")
    w = synth.weights_numpy(cfg, 1000)
    cache = model.new_cache(cfg, 1, 8)
    model.forward(cfg, w, np.arange(5)[None], np.arange(5)[None], np.zeros((1, 5)), cache)
    k = cache["k"][:, 0, :5]
    assert np.array_equal(model.bf16_round(k), k)
    assert np.abs(k).max() > 0


def test_norm_input_is_rms_norm():
    """The GEMM-input form of RMSNorm equals the library RMSNorm exactly in fp32
    configs and within bf16 rounding in bf16 configs."""
    r = np.random.default_rng(9)
    x = r.standard_normal((5, 64)) * 2
    g = r.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), 1e-6).numpy()
    assert np.allclose(model.norm_input(TINY, x, g, 1e-6), ref, rtol=1e-12, atol=1e-12)
    cfg = TINY.with_(dtype="bf16")
    y = model.norm_input(cfg, x, g, 1e-6)
    assert np.allclose(y, ref, rtol=2.0 ** -8, atol=1e-12)
    assert not np.allclose(y, ref, rtol=1e-9, atol=0)


def _bf16_case():
    cfg = TINY.with_(dtype="bf16")
    w = synth.weights_numpy(cfg, 1000, lm_head_std=0.35, lora_b_std=0.6)
    r = np.random.default_rng(10)
    R = 12
    toks = r.integers(0, cfg.vocab - 1, size=R)
    gate = (r.random(R) < 0.5).astype(np.float64)
    cache = model.new_cache(cfg, 1, R)
    logits, _ = model.forward(cfg, w, toks[None], np.arange(R)[None], gate[None], cache)
    return cfg, w, toks, gate, logits[0]


def test_bf16_storage_points_match_torch_library_forward():
    """The bf16 oracle rounds exactly at the storage points of the bf16 reading
    (gain-scaled norm input, LoRA intermediate, q, k, v, attention output, SwiGLU
    product): it equals an independent torch forward that rounds there by torch's
    own bfloat16 conversion."""
    cfg, w, toks, gate, got = _bf16_case()
    ref = _torch_forward(cfg, w, toks, gate, store=STORE_POINTS)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.allclose(got[fin], ref[fin], rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("skip", STORE_POINTS)
def test_bf16_storage_pin_has_power(skip):
    """Leaving out any one rounding point moves the logits far beyond the pin's
    tolerance, so an oracle that forgot (or misplaced) one would fail the pin."""
    cfg, w, toks, gate, got = _bf16_case()
    ref = _torch_forward(cfg, w, toks, gate, store=tuple(p for p in STORE_POINTS if p != skip))
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() > 1e-5


def _qk_norm_weights(cfg, seed):
    w = synth.weights_numpy(cfg, seed)
    r = np.random.default_rng(seed)
    for lw in w["layers"]:
        lw["q_norm"] = 1.0 + 0.3 * r.standard_normal(cfg.head_dim)
        lw["k_norm"] = 1.0 + 0.3 * r.standard_normal(cfg.head_dim)
    return w


def test_qk_norm_forward_matches_torch():
    """The Qwen3-style option: q and k RMS-normalised per head before RoPE, against
    the independent torch forward using torch's rms_norm over the head dimension."""
    cfg = TINY.with_(qk_norm=True)
    w = _qk_norm_weights(cfg, 77)
    r = np.random.default_rng(78)
    R = 10
    toks = r.integers(0, cfg.vocab, size=R)
    gate = (r.random(R) < 0.5).astype(np.float64)
    ref = _torch_forward(cfg, w, toks, gate)
    cache = model.new_cache(cfg, 1, R)
    logits, _ = model.forward(cfg, w, toks[None], np.arange(R)[None], gate[None], cache)
    fin = np.isfinite(ref)
    assert np.allclose(logits[0][fin], ref[fin], rtol=1e-9, atol=1e-12)


def test_qk_norm_is_scale_invariant_and_not_a_no_op():
    """With QK-norm (and eps 0), scaling the q / k projections (and their LoRA up
    rows) by any positive factor leaves the logits unchanged; without it, it changes
    them."""
    for qk in (True, False):
        cfg = TINY.with_(qk_norm=qk, rms_eps=0.0)     # eps would break exact scale invariance
        w = _qk_norm_weights(cfg, 79) if qk else synth.weights_numpy(cfg, 79)
        toks = np.random.default_rng(80).integers(0, cfg.vocab - 1, size=8)
        base, _ = model.forward(cfg, w, toks[None], np.arange(8)[None], np.ones((1, 8)),
                                model.new_cache(cfg, 1, 8))
        w2 = {**w, "layers": []}
        for lw in w["layers"]:
            lw2 = {**lw, "w": dict(lw["w"]), "lb": dict(lw["lb"])}
            for p in ("q", "k"):
                lw2["w"][p] = lw["w"][p] * 3.0
                lw2["lb"][p] = lw["lb"][p] * 3.0
            w2["layers"].append(lw2)
        scaled, _ = model.forward(cfg, w2, toks[None], np.arange(8)[None], np.ones((1, 8)),
                                  model.new_cache(cfg, 1, 8))
        fin = np.isfinite(base)
        same = np.allclose(scaled[fin], base[fin], rtol=1e-6, atol=1e-6)
        assert same == qk, qk
