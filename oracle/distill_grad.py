"""Oracle gradient of the block-wise TV distillation loss with respect to the gated
LoRA (the base weights frozen).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix ([blog] "Diffusion Distillation: one-step distillation + block
diffusion"; [summary] method key points): the frozen AR model is the teacher and
the AR + LoRA diffusion path the student; [x, z1] run as one gated block-causal
forward; the loss is a weighted sum of a DCD term and a block-wise total variation
term between the diffusion and the AR distributions, and the TV term alone
trained best; only the LoRA is trained.

Readings where the pages are silent (listed in the design notes):
* L_TV is the mean over sequences and blocks of the block TV, a block's TV being
  the mean over its rows of TV_i = 0.5 * sum_v |p_T,i(v) - p_S,i(v)|; all blocks
  have B rows, so L_TV is the mean of TV_i over all batch * L rows;
* the teacher distribution is a constant (no gradient through the x rows: they
  run with the gate off, so nothing they compute depends on the LoRA);
* d|u|/du at u = 0 is taken as 0;
* the storage rounding of bf16 configurations (``model._store``) is the identity
  in the backward (straight-through): the gradient is that of the same function
  with exact arithmetic at the rounded values.

Numerics: float64 throughout, softmax in float64 (no float32 rounding of the
probabilities).

Layout conventions follow ``oracle/model.py``: y = h W^T + gate * t B^T with
t = store(s * h A^T), s = alpha / r; W [out, in], A [r, in], B [out, r].
"""
import math

import numpy as np

from . import model
from .distill import block_causal_visible

PROJ = model.PROJ


def softmax64(z):
    """Float64 softmax over the last axis (a -inf logit gets probability 0)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# the loss and its gradient at the student logits

def tv_loss(teacher, student):
    """L_TV: mean over all rows of 0.5 * sum_v |p_T - p_S| (float64)."""
    pT, pS = softmax64(teacher), softmax64(student)
    return float(np.mean(0.5 * np.sum(np.abs(pT - pS), axis=-1)))


def tv_logit_grad(teacher, student):
    """dL_TV / d(student logits), same shape as ``student``.

    With N rows, dL/dp_S(v) = sign(p_S(v) - p_T(v)) / (2N) =: g(v); through the
    softmax, dL/dz(v) = p_S(v) * (g(v) - sum_u p_S(u) g(u)).
    """
    pT, pS = softmax64(teacher), softmax64(student)
    n = int(np.prod(pS.shape[:-1]))
    g = np.sign(pS - pT) / (2.0 * n)
    return pS * (g - np.sum(pS * g, axis=-1, keepdims=True))


# ---------------------------------------------------------------------------
# backward pieces

def rms_backward(cfg, x, gain, eps, dh):
    """Gradient at x of h = store(x * gain) * rs, rs = 1 / sqrt(mean(x^2) + eps),
    given dh (rows on the last axis): rs * gain * dh - x * rs^3 * mean(hg * dh),
    where hg = store(x * gain) is the value the forward used (the rounding itself
    passes the gradient straight through)."""
    x = np.asarray(x, dtype=np.float64)
    rs = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    hg = model._store(cfg, x * gain)
    return rs * gain * dh - x * rs ** 3 * np.mean(hg * dh, axis=-1, keepdims=True)


def rope_backward(dy, pos, theta):
    """RoPE is a rotation by the position's angles, so its transpose is the
    rotation by the opposite angles."""
    return model.rope(dy, -np.asarray(pos, dtype=np.float64), theta)


def silu_backward(g, u, da):
    """a = silu(g) * u with silu(g) = g * sigmoid(g): returns (dg, du)."""
    sg = 1.0 / (1.0 + np.exp(-g))
    return da * u * (sg + g * sg * (1.0 - sg)), da * g * sg


def attention_probs(q, K, V, visible):
    """Softmax attention that also returns the probabilities.

    q [S, R, Hq, hd]; K, V [S, J, Hkv, hd]; visible bool [S, R, J].  Query head h
    reads KV head h // (Hq / Hkv).  Returns o [S, R, Hq, hd] and P [S, Hq, R, J].
    """
    S, R, Hq, hd = q.shape
    G = Hq // K.shape[2]
    Kh = np.repeat(K, G, axis=2).transpose(0, 2, 1, 3)          # [S, Hq, J, hd]
    Vh = np.repeat(V, G, axis=2).transpose(0, 2, 1, 3)
    sc = q.transpose(0, 2, 1, 3) @ Kh.transpose(0, 1, 3, 2) / math.sqrt(hd)
    sc = np.where(visible[:, None], sc, -np.inf)
    P = softmax64(sc)
    return (P @ Vh).transpose(0, 2, 1, 3), P


def attention_backward(q, K, V, P, do):
    """Gradients at q, K and V of o = softmax(q K^T / sqrt(hd)) V (masked entries
    have P = 0).  do [S, R, Hq, hd]; returns dq [S, R, Hq, hd], dK, dV
    [S, J, Hkv, hd] (the query heads of a KV head summed)."""
    S, R, Hq, hd = q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    Kh = np.repeat(K, G, axis=2).transpose(0, 2, 1, 3)          # [S, Hq, J, hd]
    Vh = np.repeat(V, G, axis=2).transpose(0, 2, 1, 3)
    doh = do.transpose(0, 2, 1, 3)                                # [S, Hq, R, hd]
    qh = q.transpose(0, 2, 1, 3)
    dP = doh @ Vh.transpose(0, 1, 3, 2)                           # [S, Hq, R, J]
    dS = P * (dP - np.sum(P * dP, axis=-1, keepdims=True))
    dq = (dS @ Kh) / math.sqrt(hd)
    dKh = (dS.transpose(0, 1, 3, 2) @ qh) / math.sqrt(hd)         # [S, Hq, J, hd]
    dVh = P.transpose(0, 1, 3, 2) @ doh
    J = K.shape[1]
    dK = dKh.reshape(S, Hkv, G, J, hd).sum(axis=2).transpose(0, 2, 1, 3)
    dV = dVh.reshape(S, Hkv, G, J, hd).sum(axis=2).transpose(0, 2, 1, 3)
    return dq.transpose(0, 2, 1, 3), dK, dV


def lora_linear_saved(cfg, lw, name, h):
    """Gate-on projection y = h W^T + t B^T, t = store(s * h A^T); returns (y, t)."""
    s = cfg.lora_alpha / cfg.lora_rank
    t = model._store(cfg, s * (h @ lw["la"][name].T))
    return h @ lw["w"][name].T + t @ lw["lb"][name].T, t


def lora_linear_backward(cfg, lw, name, h, t, dy):
    """Backward of ``lora_linear_saved`` over rows (leading axes flattened).

    dB = dy^T t, dt = dy B, dA = s dt^T h, dh = dy W + s dt A.
    Returns (dh, dA, dB)."""
    s = cfg.lora_alpha / cfg.lora_rank
    A, Bm, W = lw["la"][name], lw["lb"][name], lw["w"][name]
    h2 = h.reshape(-1, h.shape[-1])
    t2 = t.reshape(-1, t.shape[-1])
    d2 = dy.reshape(-1, dy.shape[-1])
    dt = d2 @ Bm
    dB = d2.T @ t2
    dA = s * (dt.T @ h2)
    dh = d2 @ W + s * (dt @ A)
    return dh.reshape(h.shape), dA, dB


# ---------------------------------------------------------------------------
# one layer over the z1 rows

def z1_visible(L, B):
    """Visibility [L, 2L] of z1 row i over [x K/V (L entries) | z1 K/V (L entries)]:
    x rows 0 .. bB-1 and z1 rows bB .. i (b = i // B)."""
    return block_causal_visible(L, B)[L:]


def layer_forward_saved(cfg, lw, x, ctx_k, ctx_v, B):
    """Gate-on layer over the z1 rows x [S, L, d] at positions 0..L-1, attending to
    the x rows' K/V ctx_k, ctx_v [S, L, Hkv, hd] (constants) and to their own.
    Returns (x_out, saved)."""
    S, L, d = x.shape
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = np.broadcast_to(np.arange(L), (S, L))
    eps, th = cfg.rms_eps, cfg.rope_theta
    sv = {"x": x, "pos": pos}
    h1 = model.norm_input(cfg, x, lw["attn_norm"], eps)
    sv["h1"] = h1
    y = {}
    for p in ("q", "k", "v"):
        y[p], sv["t_" + p] = lora_linear_saved(cfg, lw, p, h1)
    q = model._store(cfg, model.rope(y["q"].reshape(S, L, Hq, hd), pos, th))
    k = model._store(cfg, model.rope(y["k"].reshape(S, L, Hkv, hd), pos, th))
    v = model._store(cfg, y["v"].reshape(S, L, Hkv, hd))
    K = np.concatenate([ctx_k, k], axis=1)
    V = np.concatenate([ctx_v, v], axis=1)
    vis = np.broadcast_to(z1_visible(L, B), (S, L, 2 * L))
    o, P = attention_probs(q, K, V, vis)
    o = model._store(cfg, o.reshape(S, L, Hq * hd))
    sv.update(q=q, K=K, V=V, P=P, o=o)
    yo, sv["t_o"] = lora_linear_saved(cfg, lw, "o", o)
    x2 = x + yo
    h2 = model.norm_input(cfg, x2, lw["mlp_norm"], eps)
    yg, sv["t_gate"] = lora_linear_saved(cfg, lw, "gate", h2)
    yu, sv["t_up"] = lora_linear_saved(cfg, lw, "up", h2)
    a = model._store(cfg, yg / (1.0 + np.exp(-yg)) * yu)
    yd, sv["t_down"] = lora_linear_saved(cfg, lw, "down", a)
    sv.update(x2=x2, h2=h2, yg=yg, yu=yu, a=a)
    return x2 + yd, sv


def layer_backward(cfg, lw, sv, dy):
    """Backward of ``layer_forward_saved`` given dL/dx_out dy [S, L, d].

    Returns (dx_in [S, L, d], {proj: (dA, dB)}).  Gradients reaching the x rows'
    K/V are dropped: those are constants of the LoRA.
    """
    S, L, d = dy.shape
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    eps, th = cfg.rms_eps, cfg.rope_theta
    grads = {}
    # MLP block: x_out = x2 + down(a), a = silu(gate(h2)) * up(h2)
    da, grads["down"] = _split(lora_linear_backward(cfg, lw, "down", sv["a"], sv["t_down"], dy))
    dyg, dyu = silu_backward(sv["yg"], sv["yu"], da)
    dh2g, grads["gate"] = _split(lora_linear_backward(cfg, lw, "gate", sv["h2"], sv["t_gate"], dyg))
    dh2u, grads["up"] = _split(lora_linear_backward(cfg, lw, "up", sv["h2"], sv["t_up"], dyu))
    dx2 = dy + rms_backward(cfg, sv["x2"], lw["mlp_norm"], eps, dh2g + dh2u)
    # attention block: x2 = x + o_proj(attention(q, K, V))
    do, grads["o"] = _split(lora_linear_backward(cfg, lw, "o", sv["o"], sv["t_o"], dx2))
    dq, dK, dV = attention_backward(sv["q"], sv["K"], sv["V"], sv["P"],
                                    do.reshape(S, L, Hq, hd))
    dk, dv = dK[:, L:], dV[:, L:]                 # the z1 rows' own K/V
    dyq = rope_backward(dq, sv["pos"], th).reshape(S, L, Hq * hd)
    dyk = rope_backward(dk, sv["pos"], th).reshape(S, L, Hkv * hd)
    dyv = dv.reshape(S, L, Hkv * hd)
    dh1 = 0.0
    for p, dyp in (("q", dyq), ("k", dyk), ("v", dyv)):
        dhp, grads[p] = _split(lora_linear_backward(cfg, lw, p, sv["h1"], sv["t_" + p], dyp))
        dh1 = dh1 + dhp
    dx = dx2 + rms_backward(cfg, sv["x"], lw["attn_norm"], eps, dh1)
    return dx, grads


def _split(res):
    dh, dA, dB = res
    return dh, (dA, dB)


def lm_head_backward(cfg, weights, x_final, dz):
    """Gradient at the final residual stream of logits = rms_norm(x) W_lm^T given
    dL/dlogits dz (the MASK column's -inf is a constant)."""
    dh = dz @ weights["lm_head"]
    return rms_backward(cfg, x_final, weights["final_norm"], cfg.rms_eps, dh)


# ---------------------------------------------------------------------------
# the whole distillation step

def distill_checkpoint(cfg, weights, x, B):
    """The [x, z1] forward (as ``oracle/distill.py``) keeping what the backward
    needs: per layer the z1 rows' residual stream entering it and the x rows' K/V,
    plus the final z1 stream and both halves' logits."""
    x = np.asarray(x, dtype=np.int64)
    S, L = x.shape
    toks = np.concatenate([x, np.full((S, L), cfg.mask_id, dtype=np.int64)], axis=1)
    pos = np.tile(np.concatenate([np.arange(L), np.arange(L)]), (S, 1))
    slots = np.tile(np.arange(2 * L), (S, 1))
    gate = np.concatenate([np.zeros((S, L)), np.ones((S, L))], axis=1)
    vis = np.broadcast_to(block_causal_visible(L, B), (S, 2 * L, 2 * L))
    cache = model.new_cache(cfg, S, 2 * L)
    h = np.asarray(weights["embed"], dtype=np.float64)[toks]
    xs, ks, vs = [], [], []
    for l, lw in enumerate(weights["layers"]):
        xs.append(h[:, L:].copy())
        h = model.layer_forward(cfg, lw, h, pos, gate, cache["k"][l], cache["v"][l], vis,
                                slots=slots)
        ks.append(cache["k"][l][:, :L].copy())
        vs.append(cache["v"][l][:, :L].copy())
    logits = model.lm_logits(cfg, weights, h)
    return {"x_in": xs, "k": ks, "v": vs, "x_final": h[:, L:].copy(),
            "teacher": logits[:, :L], "student": logits[:, L:]}


def distill_grad(cfg, weights, x, B):
    """L_TV of the [x, z1] forward and its gradient with respect to every LoRA
    matrix.  Returns (loss, [per layer {proj: (dA [r, in], dB [out, r])}]).
    The per-head QK-norm option is not part of this gradient."""
    if getattr(cfg, "qk_norm", False):
        raise NotImplementedError("distill_grad: QK-norm configurations are not covered")
    ck = distill_checkpoint(cfg, weights, x, B)
    loss = tv_loss(ck["teacher"], ck["student"])
    dz = tv_logit_grad(ck["teacher"], ck["student"])
    dz = np.where(np.isfinite(ck["student"]), dz, 0.0)
    dy = lm_head_backward(cfg, weights, ck["x_final"], dz)
    grads = [None] * len(weights["layers"])
    for l in reversed(range(len(weights["layers"]))):
        lw = weights["layers"][l]
        _, sv = layer_forward_saved(cfg, lw, ck["x_in"][l], ck["k"][l], ck["v"][l], B)
        dy, grads[l] = layer_backward(cfg, lw, sv, dy)
    return loss, grads
