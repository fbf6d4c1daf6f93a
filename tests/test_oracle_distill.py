"""Pins of the oracle's [x, z1] gated block-causal forward: the teacher rows equal
the AR forward of x alone, each student block equals a draft-style forward on its
clean prefix, a single block (B = L) sees no clean context, and the TV reduction
meets its closed forms."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth
from oracle import distill, model

TINY = configs.TINY


@pytest.fixture(scope="module")
def tiny_w():
    return synth.weights_numpy(TINY, 1000)


def test_visibility_structure():
    vis = distill.block_causal_visible(8, 4)
    L = 8
    # x causal
    assert np.array_equal(vis[:L, :L], np.tril(np.ones((L, L), dtype=bool)))
    assert not vis[:L, L:].any()
    # z1 row 5 (block 1) sees x 0..3 and z1 4..5
    assert vis[L + 5].nonzero()[0].tolist() == [0, 1, 2, 3, L + 4, L + 5]
    # z1 row 2 (block 0) sees no x row
    assert vis[L + 2].nonzero()[0].tolist() == [L + 0, L + 1, L + 2]


@pytest.mark.parametrize("B", [2, 4, 8])
def test_teacher_and_student_rows(tiny_w, B):
    S, L = 2, 8
    x = synth.prompts(TINY, 2100 + B, S, L)
    teacher, student, tv, tvb = distill.distill_forward(TINY, tiny_w, x, B)
    # teacher rows: AR forward of x alone
    cache = model.new_cache(TINY, S, L)
    ar, _ = model.forward(TINY, tiny_w, x, np.tile(np.arange(L), (S, 1)), np.zeros((S, L)), cache)
    assert np.allclose(teacher, ar, rtol=1e-10, atol=1e-12, equal_nan=True)
    # student block b: AR prefill of x[0, bB), then B MASK rows at bB.. with gate 1
    for b in range(L // B):
        cache = model.new_cache(TINY, S, L)
        if b > 0:
            model.forward(TINY, tiny_w, x[:, : b * B], np.tile(np.arange(b * B), (S, 1)),
                          np.zeros((S, b * B)), cache, want_logits=False)
        rows = np.full((S, B), TINY.mask_id)
        pos = np.tile(np.arange(b * B, (b + 1) * B), (S, 1))
        dr, _ = model.forward(TINY, tiny_w, rows, pos, np.ones((S, B)), cache)
        assert np.allclose(student[:, b * B:(b + 1) * B], dr, rtol=1e-10, atol=1e-12)
    # TV reduction
    pt, ps = model.probs(teacher), model.probs(student)
    assert np.allclose(tv, 0.5 * np.abs(pt.astype(np.float64) - ps).sum(-1))
    assert np.allclose(tvb, tv.reshape(S, L // B, B).mean(-1))
    assert np.all((tv >= 0) & (tv <= 1))


def test_single_block_sees_no_clean_context(tiny_w):
    L = 8
    x1 = synth.prompts(TINY, 2200, 1, L)
    x2 = synth.prompts(TINY, 2201, 1, L)
    _, s1, _, _ = distill.distill_forward(TINY, tiny_w, x1, L)
    _, s2, _, _ = distill.distill_forward(TINY, tiny_w, x2, L)
    assert np.allclose(s1, s2, rtol=1e-12, atol=1e-13)


def test_tv_closed_forms():
    p = synth.prob_rows(1, (5, 9))
    assert np.allclose(distill.tv_rows(p, p), 0.0)
    a = np.zeros((1, 4))
    b = np.zeros((1, 4))
    a[0, :2] = [0.5, 0.5]
    b[0, 2:] = [0.25, 0.75]
    assert np.allclose(distill.tv_rows(a, b), 1.0)
