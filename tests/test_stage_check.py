"""CPU checks of the stage-isolated comparison (tests/stage_check.py) that the GPU
parity tests use: a trace produced by the bf16 oracle itself passes, and traces
with a planted mistake fail."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth
from oracle import model
from tests import stage_check as sc

CFG = configs.TINY.with_(dtype="bf16", d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                         ffn_dim=256, lora_rank=32, lora_alpha=64.0)


def _trace(J=40, R=8, seed=0):
    """One layer of the bf16 oracle on R rows at positions J-R..J-1, with the
    intermediates the library captures."""
    w = synth.weights_numpy(CFG, 1000 + seed, with_embed=False)
    lw = w["layers"][0]
    r = np.random.default_rng(seed)
    Hkv, hd = CFG.n_kv_heads, CFG.head_dim
    K = model.bf16_round(r.standard_normal((J, Hkv, hd)))
    V = model.bf16_round(r.standard_normal((J, Hkv, hd)))
    pos = np.arange(J - R, J)
    gate = (np.arange(R) > 0).astype(np.float64)
    x = r.standard_normal((1, R, CFG.d_model))
    q, k, v = model.qkv_stage(CFG, lw, x, pos[None], gate[None])
    q, k, v = (model.bf16_round(t) for t in (q, k, v))
    K[pos], V[pos] = k[0], v[0]
    vis = np.arange(J)[None, None, :] <= pos[None, :, None]
    o = model.bf16_round(model.attention(q, K[None], V[None], vis).reshape(1, R, -1))
    xm = model.o_stage(CFG, lw, x, o, gate[None])
    a = model.bf16_round(model.mlp_act_stage(CFG, lw, xm, gate[None]))
    xo = model.down_stage(CFG, lw, xm, a, gate[None])
    tr = {"x_in": x[0], "q": q[0].reshape(R, -1), "attn": o[0], "x_mid": xm[0].astype(np.float32),
          "act": a[0], "x_out": xo[0].astype(np.float32)}
    return lw, tr, pos, gate, K, V


def test_oracle_made_trace_passes():
    lw, tr, pos, gate, K, V = _trace()
    sc.layer_stages(CFG, lw, tr, np.arange(len(pos)), pos, gate, K, V, "oracle trace")


@pytest.mark.parametrize("plant", ["q_unrotated", "attn_heads_swapped", "act_truncated",
                                   "k_off_by_one_position", "x_mid_lora_dropped"])
def test_planted_mistakes_fail(plant):
    lw, tr, pos, gate, K, V = _trace(seed=1)
    R = len(pos)
    if plant == "q_unrotated":
        h = model.norm_input(CFG, tr["x_in"][None], lw["attn_norm"], CFG.rms_eps)
        tr["q"] = model.bf16_round(model.gated_lora_linear(CFG, h, lw["w"]["q"], lw["la"]["q"],
                                                           lw["lb"]["q"], gate[None]))[0]
    elif plant == "attn_heads_swapped":
        a = tr["attn"].reshape(R, CFG.n_q_heads, -1)
        tr["attn"] = a[:, ::-1].reshape(R, -1).copy()
    elif plant == "act_truncated":
        # round toward zero instead of to nearest: within one bf16 spacing
        ex = model.mlp_act_stage(CFG, lw, tr["x_mid"][None].astype(np.float64), gate[None])[0]
        m, e = np.frexp(ex)
        tr["act"] = np.ldexp(np.trunc(m * 256.0) / 256.0, e)
    elif plant == "k_off_by_one_position":
        K = K.copy()
        K[pos] = K[pos - 1]
    elif plant == "x_mid_lora_dropped":
        base = tr["x_in"] + model.bf16_round(tr["attn"]) @ lw["w"]["o"].T
        tr["x_mid"] = np.where(gate[:, None] > 0, base, tr["x_mid"]).astype(np.float32)
    with pytest.raises(AssertionError):
        sc.layer_stages(CFG, lw, tr, np.arange(R), pos, gate, K, V, plant)
