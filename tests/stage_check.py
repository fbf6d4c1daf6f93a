"""Stage-isolated comparison of one decoder layer of the HIP path with the oracle.

Each stage is evaluated by the oracle from the GPU's own inputs to that stage (the
intermediates captured with uno_set_trace and the K/V read back from the pages),
so the error measured is the stage's own, without the rounding cascade of the
stages before it.  The oracle's stage value is taken before its storage rounding
("exact").  A bf16 output (q, K, V, the attention output, the SwiGLU product) has
to be the correctly rounded exact value up to a small slack for the kernel's
float32 accumulation and for rounding flips of the layer's internal bf16 values
(the LoRA intermediate; in attention the bf16 probabilities of the P.V product):
within half a bf16 spacing plus that slack.  (An absolute bound cannot apply to
these: at |v| >= 8 half a spacing alone is >= 3.1e-2.)  Every float32 output (the
residual stream after o and after down, the logits) has to be within the 3e-2
absolute bound of the bf16 configurations, and within a slack relative to the
size of the product it adds."""
import numpy as np

from oracle import model
from tests.gpu_util import log

TOL = 3e-2            # absolute bound on bf16 configurations
TV_TOL = 1e-3         # per-row total variation of probability rows
# Slack of a bf16 stage output beyond half a bf16 spacing, relative to the rms of
# the stage's output.  Linear stages: float32 accumulation (~1e-6 relative) plus a
# rare flipped LoRA intermediate element (one bf16 spacing of s * t, 2^-8 |s t|,
# times a LoRA-up weight: ~6e-4 of the output's rms at the 8B shape) -> 2e-3.
LIN_REL = 2e-3
# Attention: its probabilities enter the P.V product as bf16 (relative 2^-9 each),
# so |error| <= 2^-8 * sum_j p_j |v_j| (the attention of |V|).
ATT_REL = 2.0 ** -8
# A float32 residual output x + f(...): the same sources relative to the rms of
# the added product f.
F32_REL = 4e-3


def _rms(a):
    return float(np.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))


def bf16_spacing(x):
    """Distance between neighbouring bfloat16 numbers at |x| (normal range)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_bf16(what, gpu, ex, slack, stats=None):
    """A bf16 output against the oracle's unrounded value: within half a bf16
    spacing plus `slack` (a scalar or an array like ex)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ex = np.asarray(ex, dtype=np.float64)
    assert gpu.shape == ex.shape, (what, gpu.shape, ex.shape)
    err = np.abs(gpu - ex)
    half = 0.5 * np.maximum(bf16_spacing(gpu), bf16_spacing(ex))
    sl = np.broadcast_to(np.asarray(slack, dtype=np.float64), ex.shape)
    over = err - (half + sl)
    mism = float(np.mean(gpu != model.bf16_round(ex)))
    i = np.unravel_index(np.argmax(over), over.shape)
    log(f"  {what}: max |gpu-oracle| {err.max():.3e}, worst err-bound {over.max():.2e} "
        f"(gpu {gpu[i]:.6g}, oracle {ex[i]:.6g}, half spacing {half[i]:.2e}, slack {sl[i]:.2e}), "
        f"bf16 values differing from round(oracle) {100 * mism:.2f}%")
    if stats is not None:
        stats.append((what, float(err.max()), mism))
    assert np.all(over <= 0), (what, np.unravel_index(np.argmax(over), over.shape))


def check_f32(what, gpu, ex, base, stats=None):
    """A float32 residual output base + f against the oracle: within F32_REL of the
    rms of f, and within TOL."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ex = np.asarray(ex, dtype=np.float64)
    err = np.abs(gpu - ex)
    slack = F32_REL * _rms(ex - np.asarray(base, dtype=np.float64))
    log(f"  {what}: max |gpu-oracle| {err.max():.3e} (bound {slack:.2e}), mean {err.mean():.2e}")
    if stats is not None:
        stats.append((what, float(err.max()), 0.0))
    assert err.max() <= min(TOL, slack), what


def swiglu_slack(cfg, lw, x, gate):
    """Slack of the SwiGLU product a = silu(g) * u: the linear-stage slack of each
    pre-activation (LIN_REL of its rms) carried through the product to first order,
    |da| <= |silu'(g)| |u| dg + |silu(g)| du with |silu'| <= 1.1.  (An error in g
    reaches a multiplied by |u|, so a slack relative to the rms of a alone does not
    cover rows where |u| or |silu(g)| sits in the tail.)"""
    h2 = model.norm_input(cfg, x, lw["mlp_norm"], cfg.rms_eps)
    g = model._proj(cfg, lw, "gate", h2, gate)
    u = model._proj(cfg, lw, "up", h2, gate)
    dg, du = LIN_REL * _rms(g), LIN_REL * _rms(u)
    return 1.1 * dg * np.abs(u) + np.abs(g / (1.0 + np.exp(-g))) * du


def tv_rows(p, q):
    return 0.5 * np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)).sum(-1)


def layer_stages(cfg, lw, tr, rows, pos, gate, K, V, label, stats=None):
    """Check the five stages of one layer for the rows `rows` of one sequence.

    tr: the trace of the layer as float64 arrays [R_total, ...]; pos, gate [len(rows)];
    K, V: that sequence's cache of this layer as the GPU held it during the forward
    ([J, Hkv, hd], the rows' own K/V included at their positions)."""
    R = len(rows)
    Hq, Hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = np.asarray(pos, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float64)
    x_in = tr["x_in"][rows][None]
    q_ex, k_ex, v_ex = model.qkv_stage(cfg, lw, x_in, pos[None], gate[None])
    q_g = tr["q"][rows].reshape(1, R, Hq, hd)
    check_bf16(f"{label} q (q|k|v + RoPE)", q_g[0], q_ex[0], LIN_REL * _rms(q_ex), stats)
    check_bf16(f"{label} K written to the pages", K[pos], k_ex[0], LIN_REL * _rms(k_ex), stats)
    check_bf16(f"{label} V written to the pages", V[pos], v_ex[0], LIN_REL * _rms(v_ex), stats)
    J = K.shape[0]
    vis = np.arange(J)[None, None, :] <= pos[None, :, None]
    o_ex = model.attention(q_g, K[None], V[None], vis).reshape(R, Hq * hd)
    o_abs = model.attention(q_g, K[None], np.abs(V)[None], vis).reshape(R, Hq * hd)
    attn = tr["attn"][rows][None]
    check_bf16(f"{label} attention", attn[0], o_ex, ATT_REL * o_abs, stats)
    xm_ex = model.o_stage(cfg, lw, x_in, attn, gate[None])
    check_f32(f"{label} o + residual", tr["x_mid"][rows], xm_ex[0], x_in[0], stats)
    x_mid = tr["x_mid"][rows][None]
    a_ex = model.mlp_act_stage(cfg, lw, x_mid, gate[None])
    check_bf16(f"{label} gate/up + SwiGLU", tr["act"][rows], a_ex[0],
               swiglu_slack(cfg, lw, x_mid, gate[None])[0], stats)
    xo_ex = model.down_stage(cfg, lw, x_mid, tr["act"][rows][None], gate[None])
    check_f32(f"{label} down + residual", tr["x_out"][rows], xo_ex[0], x_mid[0], stats)


def lm_head_stage(cfg, head, x_fin, logits_gpu, probs_gpu, label):
    """LM head + softmax from the GPU's final residual rows: logits within the bf16
    bound, every row's probabilities within TV 1e-3 of the oracle's, and the
    softmax kernel alone (oracle softmax of the GPU's own logits) within 1e-6."""
    ex = model.lm_logits(cfg, head, x_fin)
    fin = np.isfinite(ex)
    assert np.array_equal(fin, np.isfinite(logits_gpu)), label
    err = np.abs(logits_gpu[fin] - ex[fin])
    tv = tv_rows(probs_gpu, model.probs(ex))
    tv_sm = tv_rows(probs_gpu, model.probs(logits_gpu))
    log(f"  {label} logits: max |gpu-oracle| {err.max():.3e}; row TV max {tv.max():.2e} "
        f"(softmax alone {tv_sm.max():.2e})")
    assert err.max() <= TOL, label
    assert tv.max() <= TV_TOL, label
    assert tv_sm.max() <= 1e-6, label
    return ex
