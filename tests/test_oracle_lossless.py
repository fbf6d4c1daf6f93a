"""Losslessness of the oracle's Psi-Spec sampler, pinned by brute force: on the tiny
vocabulary the empirical law of the generated continuation must match the exact AR
law enumerated by teacher-forced forwards (chi^2, p > 0.01).

Because N(0, 0.02) weights make p and q almost uniform, a broken sampler could pass
unseen; a stress variant (sharper LM head, stronger LoRA) makes the draft and AR
laws differ by a large total variation, and deliberately broken samplers
("always accept", "resample from p instead of the residual") must FAIL there."""
import numpy as np
import pytest
from scipy import stats

from diffusion_drafted_lora_amd import configs, synth
from oracle import model, nucleus, psispec

TINY = configs.TINY
STRESS = dict(lm_head_std=0.35, lora_b_std=0.6)


def _exact_joint2(cfg, w, prompt):
    """Exact AR law of (t1, t2) after ``prompt``: p(t1 | prompt) p(t2 | prompt, t1)."""
    V = cfg.vocab
    P = len(prompt)
    cache = model.new_cache(cfg, 1, P + 2)
    lg, _ = model.forward(cfg, w, np.asarray(prompt)[None], np.arange(P)[None],
                          np.zeros((1, P)), cache)
    l1 = lg[0, -1]
    p1 = np.exp(l1 - l1.max())
    p1 /= p1.sum()
    joint = np.zeros((V, V))
    toks = np.tile(np.concatenate([prompt, [0]]), (V, 1))
    toks[:, -1] = np.arange(V)
    cache = model.new_cache(cfg, V, P + 2)
    lg, _ = model.forward(cfg, w, toks, np.tile(np.arange(P + 1), (V, 1)),
                          np.zeros((V, P + 1)), cache)
    l2 = lg[:, -1]
    p2 = np.exp(l2 - l2.max(axis=1, keepdims=True))
    p2 /= p2.sum(axis=1, keepdims=True)
    joint = p1[:, None] * p2
    joint[cfg.mask_id, :] = 0
    return joint


def _sample_first_two(cfg, w, prompt, N, seed, broken=None, top_p=1.0):
    """Run one Psi-Spec iteration for N sequences (seq ids 0..N-1) sharing a prompt."""
    one = psispec.Decoder(cfg, w, [0], seed, len(prompt) + cfg.block_size + 2)
    one.prefill([prompt])
    out_all = []
    chunk = 20_000
    for a in range(0, N, chunk):
        b = min(N, a + chunk)
        dec = psispec.Decoder(cfg, w, np.arange(a, b), seed, len(prompt) + cfg.block_size + 2,
                              top_p=top_p)
        dec.cache["k"][:] = one.cache["k"]
        dec.cache["v"][:] = one.cache["v"]
        dec.n[:], dec.t[:] = one.n[0], one.t[0]
        r = dec.step(broken=broken)
        out_all.append(r["out"][:, :2])
    return np.concatenate(out_all)


def _chi2_pvalue(obs_pairs, joint):
    V = joint.shape[0]
    N = len(obs_pairs)
    counts = np.zeros((V, V))
    np.add.at(counts, (obs_pairs[:, 0], obs_pairs[:, 1]), 1)
    e = (joint * N).ravel()
    o = counts.ravel()
    assert o[e == 0].sum() == 0, "a sample fell on a zero-probability cell"
    # merge the sparse cells into one bin so every expected count is >= 5
    big = e >= 5
    eb = np.append(e[big], e[~big].sum())
    ob = np.append(o[big], o[~big].sum())
    if eb[-1] == 0:
        eb, ob = eb[:-1], ob[:-1]
    return stats.chisquare(ob, eb * ob.sum() / eb.sum()).pvalue


@pytest.fixture(scope="module")
def tiny_w():
    return synth.weights_numpy(TINY, 1000)


@pytest.fixture(scope="module")
def stress_w():
    return synth.weights_numpy(TINY, 1001, **STRESS)


def test_lossless_first_two_tokens_tiny(tiny_w):
    prompt = synth.prompts(TINY, 2000, 1)[0]
    joint = _exact_joint2(TINY, tiny_w, prompt)
    obs = _sample_first_two(TINY, tiny_w, prompt, 60_000, 3000)
    assert _chi2_pvalue(obs, joint) > 0.01


def _filtered_joint2(cfg, w, prompt, top_p):
    """Exact law of (t1, t2) when every AR conditional is truncated to its top-p
    nucleus: filter(p(t1 | prompt)) filter(p(t2 | prompt, t1)), the float32 laws the
    sampler draws from."""
    V = cfg.vocab
    P = len(prompt)
    cache = model.new_cache(cfg, 1, P + 2)
    lg, _ = model.forward(cfg, w, np.asarray(prompt)[None], np.arange(P)[None],
                          np.zeros((1, P)), cache)
    p1 = nucleus.filter_row(model.probs(lg[0, -1]), top_p).astype(np.float64)
    toks = np.tile(np.concatenate([prompt, [0]]), (V, 1))
    toks[:, -1] = np.arange(V)
    cache = model.new_cache(cfg, V, P + 2)
    lg, _ = model.forward(cfg, w, toks, np.tile(np.arange(P + 1), (V, 1)),
                          np.zeros((V, P + 1)), cache)
    p2 = nucleus.filter_rows(model.probs(lg[:, -1]), top_p).astype(np.float64)
    joint = p1[:, None] * p2
    return joint / joint.sum()


def test_lossless_first_two_tokens_top_p_stress(stress_w):
    """With top-p 0.9 the output law is the filtered AR law: no sample outside the
    nuclei, chi^2 against the filtered joint passes, and against the unfiltered
    joint (what a sampler that skipped the filter would follow) it fails."""
    prompt = synth.prompts(TINY, 2003, 1)[0]
    joint_f = _filtered_joint2(TINY, stress_w, prompt, 0.9)
    joint = _exact_joint2(TINY, stress_w, prompt)
    assert (joint_f > 0).sum() < 0.8 * (joint > 0).sum()      # the filter bites
    obs = _sample_first_two(TINY, stress_w, prompt, 30_000, 3005, top_p=0.9)
    assert _chi2_pvalue(obs, joint_f) > 0.01
    N = len(obs)
    counts = np.zeros_like(joint)
    np.add.at(counts, (obs[:, 0], obs[:, 1]), 1)
    e = joint.ravel() * N
    big = e >= 5
    o = counts.ravel()
    eb, ob = np.append(e[big], e[~big].sum()), np.append(o[big], o[~big].sum())
    assert stats.chisquare(ob, eb * ob.sum() / eb.sum()).pvalue < 1e-6


def _tv_draft_vs_ar(cfg, w, prompt):
    dec = psispec.Decoder(cfg, w, [0], 1, len(prompt) + cfg.block_size + 2)
    dec.prefill([prompt])
    r = dec.step()
    # q_2 against p_2 (AR law of the token after y_1)
    return 0.5 * np.abs(r["P_d"][0, 1].astype(np.float64) - r["P_v"][0, 0]).sum()


def test_stress_variant_has_power(stress_w):
    """The stress weights make the draft and AR laws differ substantially, and
    both planted mistakes are detected while the correct sampler passes."""
    prompt = synth.prompts(TINY, 2003, 1)[0]
    assert _tv_draft_vs_ar(TINY, stress_w, prompt) > 0.25
    joint = _exact_joint2(TINY, stress_w, prompt)
    N = 30_000
    good = _sample_first_two(TINY, stress_w, prompt, N, 3003)
    assert _chi2_pvalue(good, joint) > 0.01
    for broken in ("always_accept", "resample_p"):
        bad = _sample_first_two(TINY, stress_w, prompt, N, 3003, broken=broken)
        assert _chi2_pvalue(bad, joint) < 1e-6, broken


def _teacher_forced_laws(cfg, w, prompt, toks):
    """p(. | prompt, toks[:j]) for every generated position j, per sequence."""
    S, n_new = toks.shape
    P = len(prompt)
    full = np.concatenate([np.tile(prompt, (S, 1)), toks], axis=1)
    cache = model.new_cache(cfg, S, P + n_new)
    lg, _ = model.forward(cfg, w, full, np.tile(np.arange(P + n_new), (S, 1)),
                          np.zeros((S, P + n_new)), cache)
    lg = lg[:, P - 1: P - 1 + n_new]
    p = np.exp(lg - lg.max(axis=-1, keepdims=True))
    return p / p.sum(axis=-1, keepdims=True)


def _positionwise_stat(cfg, w, prompt, toks):
    """Pearson statistic over all positions: observed one-hot counts against the sum
    of each sequence's exact teacher-forced conditional.  With heterogeneous
    conditionals this is conservative (stochastically below chi^2)."""
    laws = _teacher_forced_laws(cfg, w, prompt, toks)
    S, n_new, V = laws.shape
    stat, dof = 0.0, 0
    for j in range(n_new):
        E = laws[:, j].sum(axis=0)
        O = np.bincount(toks[:, j], minlength=V).astype(np.float64)
        big = E >= 5
        Eb = np.append(E[big], E[~big].sum())
        Ob = np.append(O[big], O[~big].sum())
        keep = Eb > 0
        stat += float(((Ob[keep] - Eb[keep]) ** 2 / Eb[keep]).sum())
        dof += int(keep.sum()) - 1
    return stats.chi2.sf(stat, dof)


def test_lossless_all_positions_stress(stress_w):
    """All 32 generated tokens, each scored against its exact AR conditional given
    the sequence's own prefix (teacher forcing); power controls must fail."""
    cfg = TINY
    prompt = synth.prompts(TINY, 2004, 1)[0]
    S = 1500

    def gen(broken=None):
        dec = psispec.Decoder(cfg, stress_w, np.arange(S), 3004, cfg.max_len + 2)
        one = psispec.Decoder(cfg, stress_w, [0], 3004, cfg.max_len + 2)
        one.prefill([prompt])
        dec.cache["k"][:] = one.cache["k"]
        dec.cache["v"][:] = one.cache["v"]
        dec.n[:], dec.t[:] = one.n[0], one.t[0]
        toks, _, _ = dec.generate(cfg.new_tokens, broken=broken)
        return toks

    assert _positionwise_stat(cfg, stress_w, prompt, gen()) > 0.01
    for broken in ("always_accept", "resample_p"):
        # detection: far below the 0.01 acceptance threshold
        assert _positionwise_stat(cfg, stress_w, prompt, gen(broken)) < 1e-3, broken
