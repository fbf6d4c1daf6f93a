"""Oracle forward of the diffusion-augmented decoder: one causal Transformer whose
projections carry a per-row gated LoRA.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:
* one causal Transformer holds the frozen AR weights; the diffusion weights are a
  rank-r LoRA (r = 128, alpha = 256 for the 8B models) attached to every layer
  ([summary] method key points; [blog] "method core: one model, two weight sets");
* the drafting path uses base + LoRA, the verifying path the base weights only, and
  one forward may mix the two per row through a gate that switches the adapter off
  on clean rows and on on noisy rows ([blog] "one-step, block-wise distillation");
* draft and verify share one KV cache ([blog] "method core").

What the pages leave open and this oracle reads plainly (listed in the design
notes): a Qwen3-8B-shaped pre-norm decoder with RMSNorm, rotate-half RoPE, grouped
query attention, SwiGLU MLP, no biases, untied embedding / LM head; the LoRA term
on every one of the seven projections is gate * (alpha/r) * (h A^T) B^T; the MASK
id is vocab-1 and its logit is -inf.  Optionally (``cfg.qk_norm``) each query and
key head is RMS-normalised over its head_dim with a learned gain before RoPE, as in
the Qwen3 attention of the base model the pages augment (Uno_Qwen: Qwen3-8B plus a
LoRA, [summary] method key points); off by default.

Numerics: float64 throughout.  When ``cfg.dtype == "bf16"`` values are rounded to
bfloat16 (round-to-nearest-even) at the points where the library stores bf16:
the gain-scaled GEMM input x*g of every RMSNorm (the per-row 1/rms factor is
applied after the product, exactly), the scaled LoRA intermediate, q/k/v after
RoPE (the KV cache), the attention output and the SwiGLU product.  The residual
stream, logits and probabilities are never rounded.

Weights are a dict (see ``tests``' generators): W for projection P is [out, in]
(so y = h @ W.T), LoRA down A_P is [r, in] and up B_P is [out, r].
"""
import math

import numpy as np

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range.  The rounding
    is done directly from float64 (no double rounding through float32).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                   # x = m * 2^e, 0.5 <= |m| < 1
    m = np.rint(m * 256.0) / 256.0       # 8 significant bits, ties to even
    out = np.ldexp(m, e)
    # below the normal range bfloat16 has a fixed quantum of 2^-133
    tiny = np.abs(x) < 2.0 ** -126
    if tiny.any():
        out = np.where(tiny, np.rint(x * 2.0 ** 133) * 2.0 ** -133, out)
    big = np.abs(out) > 3.3895313892515355e38
    if big.any():
        out = np.where(big, np.sign(out) * np.inf, out)
    return out


def _store(cfg, x):
    """The library's storage rounding: bf16 for bf16 configs, none otherwise."""
    return bf16_round(x) if cfg.dtype == "bf16" else np.asarray(x, dtype=np.float64)


def norm_input(cfg, x, g, eps):
    """RMSNorm as a GEMM input: the stored gain-scaled x*g times the exact 1/rms.

    Mathematically rms_norm(x, g); in bf16 configs the rounding sits on x*g.
    """
    x = np.asarray(x, dtype=np.float64)
    rs = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return _store(cfg, x * g) * rs


def rms_norm(x, g, eps):
    """RMSNorm: x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotate-half rotary embedding.

    x: [..., n_heads, hd]; pos: integer array broadcastable to x.shape[:-2].
    Pair (i, i + hd/2) is rotated by angle pos * theta^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv  # [..., 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gated_lora_linear(cfg, h, W, A, B, gate):
    """y = h W^T + gate * ((alpha/r) * h A^T) B^T.

    h: [..., in]; W: [out, in]; A: [r, in]; B: [out, r]; gate: [...] in {0, 1}.
    The scaled intermediate (alpha/r) * h A^T is rounded like any stored bf16 value.
    """
    lead = h.shape[:-1]
    h2 = h.reshape(-1, h.shape[-1])          # one 2-D GEMM instead of a batch of small ones
    y = h2 @ W.T
    if A is not None:
        s = cfg.lora_alpha / cfg.lora_rank
        u = _store(cfg, s * (h2 @ A.T))
        g = np.broadcast_to(np.asarray(gate, dtype=np.float64), lead).reshape(-1)
        y = y + g[:, None] * (u @ B.T)
    return y.reshape(lead + (W.shape[0],))


def attention(q, K, V, visible):
    """Softmax attention with grouped query heads.

    q: [S, R, Hq, hd]; K, V: [S, J, Hkv, hd]; visible: bool [S, R, J].
    Query head h reads KV head floor(h * Hkv / Hq).  Scale 1/sqrt(hd).
    Returns [S, R, Hq, hd].
    """
    S, R, Hq, hd = q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    qg = q.reshape(S, R, Hkv, G, hd).transpose(0, 2, 3, 1, 4)        # [S, Hkv, G, R, hd]
    Kt = K.transpose(0, 2, 3, 1)[:, :, None]                           # [S, Hkv, 1, hd, J]
    scores = (qg @ Kt) / math.sqrt(hd)                                 # [S, Hkv, G, R, J]
    scores = np.where(visible[:, None, None, :, :], scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    p = np.exp(scores - m)
    p = p / np.sum(p, axis=-1, keepdims=True)
    o = p @ V.transpose(0, 2, 1, 3)[:, :, None]                        # [S, Hkv, G, R, hd]
    return o.transpose(0, 3, 1, 2, 4).reshape(S, R, Hq, hd)


def new_cache(cfg, n_seqs, max_len):
    """Contiguous KV cache: K and V of shape [layers, seqs, max_len, Hkv, hd]."""
    shape = (cfg.n_layers, n_seqs, max_len, cfg.n_kv_heads, cfg.head_dim)
    return {"k": np.zeros(shape), "v": np.zeros(shape)}


def _proj(cfg, lw, name, h, gate):
    la, lb = lw.get("la", {}), lw.get("lb", {})
    return gated_lora_linear(cfg, h, lw["w"][name], la.get(name), lb.get(name), gate)


# A layer as five stages.  Each stage returns its result before the storage
# rounding of its output (``_store``), so a stage can be evaluated on its own from
# given inputs; ``layer_forward`` chains them with the rounding in place.

def qkv_stage(cfg, lw, x, pos, gate):
    """Attention inputs of rows x [S, R, d]: q [S, R, Hq, hd] and k [S, R, Hkv, hd]
    after RoPE at positions ``pos``, and v, from the pre-attention RMSNorm and the
    gated q / k / v projections (with ``cfg.qk_norm``, q and k are RMS-normalised
    per head with the gains ``q_norm`` / ``k_norm`` before RoPE)."""
    S, R, _ = x.shape
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    h = norm_input(cfg, x, lw["attn_norm"], cfg.rms_eps)
    q = _proj(cfg, lw, "q", h, gate).reshape(S, R, Hq, hd)
    k = _proj(cfg, lw, "k", h, gate).reshape(S, R, Hkv, hd)
    v = _proj(cfg, lw, "v", h, gate).reshape(S, R, Hkv, hd)
    if getattr(cfg, "qk_norm", False):
        q = rms_norm(q, lw["q_norm"], cfg.rms_eps)
        k = rms_norm(k, lw["k_norm"], cfg.rms_eps)
    return rope(q, pos, cfg.rope_theta), rope(k, pos, cfg.rope_theta), v


def o_stage(cfg, lw, x, o, gate):
    """Residual stream after the attention block: x + o_proj(o), o [S, R, Hq * hd]."""
    return x + _proj(cfg, lw, "o", o, gate)


def mlp_act_stage(cfg, lw, x, gate):
    """SwiGLU product silu(gate(h2)) * up(h2) of the pre-MLP RMSNorm h2 of x."""
    h2 = norm_input(cfg, x, lw["mlp_norm"], cfg.rms_eps)
    g = _proj(cfg, lw, "gate", h2, gate)
    u = _proj(cfg, lw, "up", h2, gate)
    return g / (1.0 + np.exp(-g)) * u


def down_stage(cfg, lw, x, a, gate):
    """Residual stream after the MLP: x + down(a)."""
    return x + _proj(cfg, lw, "down", a, gate)


def layer_forward(cfg, lw, x, pos, gate, kcache, vcache, visible, slots=None):
    """One pre-norm decoder layer on rows x [S, R, d] (float64, updated copy returned).

    Writes this layer's K/V for the rows into kcache/vcache [S, J, Hkv, hd] at cache
    index ``slots`` (default: the RoPE position ``pos``) before attending;
    ``visible`` [S, R, J] says which cache entries each row sees.
    """
    if slots is None:
        slots = pos
    S, R, d = x.shape
    Hq, hd = cfg.n_q_heads, cfg.head_dim
    q, k, v = qkv_stage(cfg, lw, x, pos, gate)
    q, k, v = _store(cfg, q), _store(cfg, k), _store(cfg, v)
    sidx = np.arange(S)[:, None]
    kcache[sidx, slots] = k
    vcache[sidx, slots] = v
    o = _store(cfg, attention(q, kcache, vcache, visible).reshape(S, R, Hq * hd))
    x = o_stage(cfg, lw, x, o, gate)
    a = _store(cfg, mlp_act_stage(cfg, lw, x, gate))
    return down_stage(cfg, lw, x, a, gate)


def lm_logits(cfg, weights, x):
    """Final RMSNorm, LM head, and the MASK column forced to -inf."""
    hf = norm_input(cfg, x, weights["final_norm"], cfg.rms_eps)
    logits = hf @ weights["lm_head"].T
    logits[..., cfg.mask_id] = -np.inf
    return logits


def forward(cfg, weights, tokens, pos, gate, cache, hidden_in=None, visible=None,
            want_logits=True, slots=None):
    """Forward of R rows per sequence against a per-sequence KV cache.

    tokens: int [S, R] (ignored when ``hidden_in`` [S, R, d] is given);
    pos: int [S, R] absolute positions; gate: {0,1} [S, R].
    The rows' K/V are written at ``pos`` in every layer.  By default a row at
    position m sees cached positions [0, m] (decode: the committed context plus the
    in-flight block up to itself); ``visible`` [S, R, J] overrides that, and
    ``slots`` [S, R] (cache indices) decouples where K/V are stored from ``pos``.
    Returns (logits [S, R, V] or None, final residual stream [S, R, d]).
    """
    pos = np.asarray(pos, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float64)
    if hidden_in is not None:
        x = np.asarray(hidden_in, dtype=np.float64).copy()
    else:
        x = np.asarray(weights["embed"], dtype=np.float64)[np.asarray(tokens)]
    J = cache["k"].shape[2]
    if visible is None:
        visible = np.arange(J)[None, None, :] <= pos[:, :, None]
    for l, lw in enumerate(weights["layers"]):
        x = layer_forward(cfg, lw, x, pos, gate, cache["k"][l], cache["v"][l], visible,
                          slots=slots)
    logits = lm_logits(cfg, weights, x) if want_logits else None
    return logits, x


def probs(logits):
    """Softmax over the last axis in float64, returned rounded to float32.

    The sampler and the accept test decide in float32 (the library's precision),
    so the oracle hands them float32 probabilities.
    """
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return (e / np.sum(e, axis=-1, keepdims=True)).astype(np.float32)
