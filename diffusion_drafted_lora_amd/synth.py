"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and lays them out; it holds none of the method's
arithmetic.  Weight layout (the library's and the oracle's): projection weight
``w[P]`` is [out, in] row-major, LoRA down ``la[P]`` is [r, in], LoRA up ``lb[P]``
is [out, r]; the embedding is [vocab, d] and the LM head [vocab, d].  Every matrix
is N(0, std^2) with std 0.02 unless overridden; RMSNorm gains are 1.  bf16
configurations round the float32 draws to bfloat16 (round-to-nearest-even, by
torch's conversion) so both sides start from identical values.
"""
import numpy as np

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def proj_shapes(cfg):
    """(out, in) of the seven projections."""
    d, q, kv, f = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    return {"q": (q, d), "k": (kv, d), "v": (kv, d), "o": (d, q),
            "gate": (f, d), "up": (f, d), "down": (d, f)}


def _to_storage(cfg, a):
    a = np.asarray(a, dtype=np.float32)
    if cfg.dtype == "bf16":
        import torch
        a = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    return a


def weights_numpy(cfg, seed, std=0.02, lm_head_std=None, lora_b_std=None,
                  with_embed=True, with_lora=True, qk_gain_std=0.0):
    """All weights as float32 numpy arrays (bf16-representable for bf16 configs).

    Draw order is fixed: embed, lm_head, then per layer and per projection W, A, B.
    ``lm_head_std`` / ``lora_b_std`` override std for those matrices (used for a
    stress variant whose draft and AR distributions differ a lot).  With
    ``cfg.qk_norm`` the per-head q / k gains are 1, or 1 + N(0, qk_gain_std^2) from
    a generator of their own (the other draws do not move).
    """
    g = np.random.Generator(np.random.Philox(seed))
    gq = np.random.Generator(np.random.Philox(seed + 7919))

    def draw(shape, s):
        return _to_storage(cfg, g.standard_normal(shape, dtype=np.float32) * np.float32(s))

    w = {}
    if with_embed:
        w["embed"] = draw((cfg.vocab, cfg.d_model), std)
        w["lm_head"] = draw((cfg.vocab, cfg.d_model), lm_head_std or std)
    w["final_norm"] = np.ones(cfg.d_model, dtype=np.float32)
    layers = []
    for _ in range(cfg.n_layers):
        lw = {"attn_norm": np.ones(cfg.d_model, dtype=np.float32),
              "mlp_norm": np.ones(cfg.d_model, dtype=np.float32),
              "w": {}, "la": {}, "lb": {}}
        if cfg.qk_norm:
            for k in ("q_norm", "k_norm"):
                lw[k] = _to_storage(cfg, 1.0 + gq.standard_normal(cfg.head_dim, dtype=np.float32)
                                    * np.float32(qk_gain_std))
        for p, (o, i) in proj_shapes(cfg).items():
            lw["w"][p] = draw((o, i), std)
            if with_lora:
                lw["la"][p] = draw((cfg.lora_rank, i), std)
                lw["lb"][p] = draw((o, cfg.lora_rank), lora_b_std or std)
        if not with_lora:
            del lw["la"], lw["lb"]
        layers.append(lw)
    w["layers"] = layers
    return w


def weights_torch(cfg, seed, device, std=0.02, with_embed=True, with_lora=True):
    """Weights generated directly in device memory with torch's generator (for the
    large configurations, where a host draw would take minutes).  Same layout and
    distribution as ``weights_numpy`` but different values."""
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    counter = [0]

    def draw(shape, s):
        gen.manual_seed(seed * 1_000_003 + counter[0])
        counter[0] += 1
        t = torch.empty(shape, dtype=torch.float32, device=device)
        t.normal_(0.0, s, generator=gen)
        return t.to(dt)

    w = {}
    if with_embed:
        w["embed"] = draw((cfg.vocab, cfg.d_model), std)
        w["lm_head"] = draw((cfg.vocab, cfg.d_model), std)
    w["final_norm"] = torch.ones(cfg.d_model, dtype=dt, device=device)
    layers = []
    for _ in range(cfg.n_layers):
        lw = {"attn_norm": torch.ones(cfg.d_model, dtype=dt, device=device),
              "mlp_norm": torch.ones(cfg.d_model, dtype=dt, device=device),
              "w": {}, "la": {}, "lb": {}}
        if cfg.qk_norm:
            lw["q_norm"] = torch.ones(cfg.head_dim, dtype=dt, device=device)
            lw["k_norm"] = torch.ones(cfg.head_dim, dtype=dt, device=device)
        for p, (o, i) in proj_shapes(cfg).items():
            lw["w"][p] = draw((o, i), std)
            if with_lora:
                lw["la"][p] = draw((cfg.lora_rank, i), std)
                lw["lb"][p] = draw((o, cfg.lora_rank), std)
        layers.append(lw)
    w["layers"] = layers
    return w


def prompts(cfg, seed, n_seqs, length=None):
    """Uniform prompts over the non-MASK ids [0, vocab-2], int32 [n_seqs, length]."""
    length = cfg.prompt_len if length is None else length
    g = np.random.Generator(np.random.Philox(seed))
    return g.integers(0, cfg.vocab - 1, size=(n_seqs, length), dtype=np.int64).astype(np.int32)


def normal(seed, shape, std=1.0, dtype=np.float32):
    """Seeded N(0, std^2) array (hidden rows, K/V contexts, probability logits)."""
    g = np.random.Generator(np.random.Philox(seed))
    return (g.standard_normal(shape) * std).astype(dtype)


def prob_rows(seed, shape, alpha=0.5, zero_frac=0.0):
    """Seeded float32 probability rows drawn from a symmetric Dirichlet(alpha) over
    the last axis, optionally with a fraction of exact zeros; used to exercise the
    accept kernel on inputs that no forward produced."""
    g = np.random.Generator(np.random.Philox(seed))
    w = g.gamma(alpha, size=shape)
    if zero_frac > 0:
        w = np.where(g.random(shape) < zero_frac, 0.0, w)
        w[..., 0] += 1e-3
    return (w / w.sum(axis=-1, keepdims=True)).astype(np.float32)
