"""Pins of the oracle's tree sampler (oracle/tree.py) that do not rely on it:

* one chain is the linear sampler of oracle/psispec.py, draw for draw (tokens,
  accept lengths, cache), with and without top-p;
* at one depth, with synthetic float32 laws p and q on a small vocabulary, the
  emitted token follows p (chi^2), and the probability that every candidate is
  rejected equals the product of the successive residual distances
  beta_1 * beta_2 * ... (beta_1 = TV(p, q), beta_{j+1} = TV(r_{j+1}, q) with
  r_{j+1} = max(0, r_j - q) / beta_j) -- the closed form of recursive rejection;
  a sampler that skips the residual update fails the chi^2 test;
* on the tiny model with the stress weights, every generated token against its
  exact teacher-forced AR conditional (the same statistic as the linear sampler's
  losslessness test), with the planted mistake detected."""
import numpy as np
import pytest
from scipy import stats

from diffusion_drafted_lora_amd import configs, synth
from oracle import model, psispec, rng, tree

TINY = configs.TINY
STRESS = dict(lm_head_std=0.35, lora_b_std=0.6)


@pytest.fixture(scope="module")
def stress_w():
    return synth.weights_numpy(TINY, 1001, **STRESS)


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_one_chain_is_the_linear_sampler(stress_w, top_p):
    prompts = [synth.prompts(TINY, 2000 + i, 1, L)[0] for i, L in enumerate([16, 9, 4, 1])]
    ids = [4, 0, 2, 7]
    lin = psispec.Decoder(TINY, stress_w, ids, 3000, TINY.max_len + 40, top_p=top_p)
    tr = tree.TreeDecoder(TINY, stress_w, ids, 3000, TINY.max_len + 40, top_p=top_p)
    lin.prefill(prompts)
    tr.prefill(prompts)
    for step in range(6):
        a, b = lin.step(), tr.step_tree(1)
        assert np.array_equal(a["out"], b["out"]), step
        assert np.array_equal(a["n_out"], b["n_out"]), step
        assert np.array_equal(a["y"], b["chains"][:, 0]), step
        assert (b["kstar"] == 0).all()
    assert np.array_equal(lin.cache["k"], tr.cache["k"])
    assert np.array_equal(lin.cache["v"], tr.cache["v"])


def _laws(V, seed):
    g = np.random.default_rng(seed)
    p = g.dirichlet(np.full(V, 0.7)).astype(np.float32)
    q = g.dirichlet(np.full(V, 0.7)).astype(np.float32)
    return p, q


def _one_depth(p, q, K, S, seed, broken=None):
    """tree_accept with B = 2: depth 2 is the only decision (its law p), y_1 = 0,
    the K depth-2 candidates drawn from q; returns (emitted depth-2 token, n_out)."""
    V = len(p)
    B = 2
    ids = np.arange(S)
    n = np.full(S, 5)
    it = np.zeros(S, dtype=np.int64)
    P_d = np.broadcast_to(np.stack([np.full(V, 1.0 / V, np.float32), q]), (S, B, V))
    chains = tree.draft_chains(P_d, K, seed, ids, n, it)
    chains[:, :, 0] = 0
    bonus = np.full(V, 1.0 / V, np.float32)
    P_v = np.empty((S, 1 + K, V), np.float32)
    P_v[:, 0] = p
    P_v[:, 1:] = bonus
    out, n_out, _ = tree.tree_accept(P_v, P_d, chains, seed, ids, n, it, broken=broken)
    return out[:, 1], n_out


def _residual_chain(p, q, K):
    """beta_1..beta_K of recursive rejection in exact arithmetic (float64)."""
    r = p.astype(np.float64)
    q = q.astype(np.float64)
    betas = []
    for _ in range(K):
        res = np.maximum(r - q, 0.0)
        b = res.sum()
        betas.append(b)
        r = res / b
    return np.array(betas)


def _chi2_p(tok, p):
    V = len(p)
    O = np.bincount(tok, minlength=V).astype(np.float64)
    E = p.astype(np.float64) / p.sum() * len(tok)
    return stats.chisquare(O, E).pvalue


@pytest.mark.parametrize("K", [2, 4])
def test_one_depth_output_law_and_rejection_rate(K):
    p, q = _laws(8, 41)
    S = 10_000
    tok, n_out = _one_depth(p, q, K, S, 501 + K)
    assert _chi2_p(tok, p) > 0.01
    betas = _residual_chain(p, q, K)
    assert betas[0] > 0.3                                  # the laws differ a lot
    all_rejected = float(np.mean(n_out == 2))              # stop at depth 2: resampled
    expect = float(np.prod(betas))
    sd = np.sqrt(expect * (1 - expect) / S)
    assert abs(all_rejected - expect) <= 5 * sd, (all_rejected, expect)
    # more candidates reject less often
    assert expect < betas[0]


def test_one_depth_skipping_the_residual_is_detected():
    p, q = _laws(8, 41)
    tok, _ = _one_depth(p, q, 4, 10_000, 505, broken="no_residual")
    assert _chi2_p(tok, p) < 1e-6


def test_residual_next_is_the_scaled_residual():
    """The 64-bit route of R_{j+1} = R_j - min(R_j, floor(T_j Q / 2^40)) (a 128-bit
    product split in two words) equals exact integer arithmetic."""
    p, q = _laws(16, 43)
    R = tree.residual_first(p, q)
    for _ in range(3):
        T = int(R.sum(dtype=np.uint64))
        nxt = tree.residual_next(R, q)
        Q = rng.int_weights(q).astype(object)
        exact = [max(0, int(r) - (T * int(qq)) // 2**40) for r, qq in zip(R, Q)]
        assert [int(v) for v in nxt] == exact
        R = nxt


def _gen_tree(cfg, w, prompt, S, K, n_new, seed, broken=None):
    B = cfg.block_size
    cap = len(prompt) + (B + 1) * ((n_new + 1) // 2 + 1) + B + 2
    one = psispec.Decoder(cfg, w, [0], seed, cap)
    one.prefill([prompt])
    dec = tree.TreeDecoder(cfg, w, np.arange(S), seed, cap)
    dec.cache["k"][:] = one.cache["k"]
    dec.cache["v"][:] = one.cache["v"]
    dec.n[:], dec.t[:] = one.n[0], one.t[0]
    toks = np.full((S, n_new), -1, dtype=np.int64)
    got = np.zeros(S, dtype=np.int64)
    while (got < n_new).any():
        r = dec.step_tree(K, broken=broken)
        for s in range(S):
            take = min(int(r["n_out"][s]), n_new - int(got[s]))
            if take > 0:
                toks[s, got[s]: got[s] + take] = r["out"][s, :take]
                got[s] += take
    return toks


def _teacher_forced_laws(cfg, w, prompt, toks):
    S, n_new = toks.shape
    P = len(prompt)
    full = np.concatenate([np.tile(prompt, (S, 1)), toks], axis=1)
    cache = model.new_cache(cfg, S, P + n_new)
    lg, _ = model.forward(cfg, w, full, np.tile(np.arange(P + n_new), (S, 1)),
                          np.zeros((S, P + n_new)), cache)
    lg = lg[:, P - 1: P - 1 + n_new]
    pr = np.exp(lg - lg.max(axis=-1, keepdims=True))
    return pr / pr.sum(axis=-1, keepdims=True)


def _positionwise_p(cfg, w, prompt, toks):
    laws = _teacher_forced_laws(cfg, w, prompt, toks)
    S, n_new, V = laws.shape
    stat, dof = 0.0, 0
    for j in range(n_new):
        E = laws[:, j].sum(axis=0)
        O = np.bincount(toks[:, j], minlength=V).astype(np.float64)
        big = E >= 5
        Eb, Ob = np.append(E[big], E[~big].sum()), np.append(O[big], O[~big].sum())
        keep = Eb > 0
        stat += float(((Ob[keep] - Eb[keep]) ** 2 / Eb[keep]).sum())
        dof += int(keep.sum()) - 1
    return stats.chi2.sf(stat, dof)


def test_tree_lossless_all_positions_stress(stress_w):
    """Three chains, 16 generated tokens per sequence, each scored against its
    exact AR conditional given the sequence's own prefix; the planted mistake is
    detected."""
    prompt = synth.prompts(TINY, 2004, 1)[0]
    S, n_new = 800, 16
    toks = _gen_tree(TINY, stress_w, prompt, S, 3, n_new, 3104)
    assert _positionwise_p(TINY, stress_w, prompt, toks) > 0.01
    bad = _gen_tree(TINY, stress_w, prompt, S, 3, n_new, 3104, broken="no_residual")
    assert _positionwise_p(TINY, stress_w, prompt, bad) < 1e-3
