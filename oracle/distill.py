"""Oracle of the distillation-style gated block-causal forward over [x, z1].

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix ([blog] "one-step, block-wise distillation"; [summary] method
key points): the clean sequence x and the fully corrupted sequence z1 are
concatenated as [x, z1] and run in ONE forward under a block-causal mask -- x is
causal; each noisy block of z1 is causal inside and sees every preceding clean
block -- while a gated LoRA is off on the clean rows (teacher logits, AR weights
only) and on on the noisy rows (student logits, AR + LoRA).  A block-wise total
variation distance between the diffusion and AR distributions drives acceptance.

Readings (design notes): z1 is all MASK; z1 row i carries RoPE position i like x
row i; student row i and teacher row i both predict token i+1; TV_i is half the L1
distance of their softmaxes (MASK excluded by its -inf logit); a block's TV is the
mean of its rows' TV.
"""
import numpy as np

from . import model


def block_causal_visible(L, B):
    """Visibility [2L, 2L] of the [x, z1] rows.

    x row i sees x rows 0..i.  z1 row i (block b = i // B) sees x rows 0..bB-1 and
    z1 rows bB..i.
    """
    vis = np.zeros((2 * L, 2 * L), dtype=bool)
    i = np.arange(L)
    vis[:L, :L] = i[None, :] <= i[:, None]
    b0 = (i // B) * B
    vis[L:, :L] = i[None, :] < b0[:, None]
    vis[L:, L:] = (i[None, :] >= b0[:, None]) & (i[None, :] <= i[:, None])
    return vis


def tv_rows(p, q):
    """Per-row total variation 0.5 * sum |p - q| (float64)."""
    return 0.5 * np.sum(np.abs(np.asarray(p, np.float64) - np.asarray(q, np.float64)), axis=-1)


def distill_forward(cfg, weights, x, B):
    """One gated forward of [x, MASK^L] per sequence.

    x: int [S, L].  Returns (teacher_logits [S, L, V], student_logits [S, L, V],
    tv_row [S, L], tv_block [S, L // B]).
    """
    x = np.asarray(x, dtype=np.int64)
    S, L = x.shape
    if L % B:
        raise ValueError("L must be a multiple of B")
    toks = np.concatenate([x, np.full((S, L), cfg.mask_id, dtype=np.int64)], axis=1)
    pos = np.tile(np.concatenate([np.arange(L), np.arange(L)]), (S, 1))
    slots = np.tile(np.arange(2 * L), (S, 1))
    gate = np.concatenate([np.zeros((S, L)), np.ones((S, L))], axis=1)
    vis = np.broadcast_to(block_causal_visible(L, B), (S, 2 * L, 2 * L))
    cache = model.new_cache(cfg, S, 2 * L)
    logits, _ = model.forward(cfg, weights, toks, pos, gate, cache, visible=vis, slots=slots)
    teacher, student = logits[:, :L], logits[:, L:]
    tv = tv_rows(model.probs(teacher), model.probs(student))
    tv_block = tv.reshape(S, L // B, B).mean(axis=-1)
    return teacher, student, tv, tv_block
