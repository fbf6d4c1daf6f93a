"""Pins of the oracle's Psi-Spec sampler against closed forms and invariants:
speculative rejection's acceptance rate sum(min(p, q)) and output law p
(Leviathan et al., Cor. 3.6), the geometric accept-length law, the first drafted
token being AR-exact and always kept, tokens-per-forward bounds, commit/rollback
leaving exactly the AR cache, and keyed determinism / resume."""
import numpy as np
import pytest
from scipy import stats

from diffusion_drafted_lora_amd import configs, synth
from oracle import model, psispec, rng

TINY = configs.TINY


@pytest.fixture(scope="module")
def tiny_w():
    return synth.weights_numpy(TINY, 1000)


def _drafts_from(q_rows, seed, seq_ids, n, it):
    """y_2..y_B drawn from q_i with the draft stream (as the draft would)."""
    S, Bm1, V = q_rows.shape
    y = np.zeros((S, Bm1 + 1), dtype=np.int64)
    for i in range(2, Bm1 + 2):
        w = rng.draw_word(seed, seq_ids, n + i, rng.STREAM_DRAFT, it)
        y[:, i - 1], _ = rng.sample_icdf(q_rows[:, i - 2], w)
    return y


def test_accept_rate_and_output_law_single_slot():
    """B = 2: one tested slot.  P(accept) = sum min(p, q); the emitted second token
    is distributed as p."""
    p = np.array([0.30, 0.05, 0.25, 0.0, 0.10, 0.30], dtype=np.float32)
    q = np.array([0.10, 0.40, 0.20, 0.15, 0.15, 0.00], dtype=np.float32)
    N = 60_000
    seq_ids = np.arange(N)
    n = np.full(N, 7)
    it = np.full(N, 2)
    p_rows = np.broadcast_to(np.stack([p, p]), (N, 2, 6))
    q_rows = np.broadcast_to(q[None, None], (N, 1, 6))
    y = _drafts_from(q_rows, 42, seq_ids, n, it)
    out, n_out = psispec.accept_block(p_rows, q_rows, y, 42, seq_ids, n, it)
    beta = float(np.minimum(p, q).sum())
    acc = np.mean(n_out == 3)
    sd = np.sqrt(beta * (1 - beta) / N)
    assert abs(acc - beta) < 5 * sd
    tok2 = out[:, 1]
    counts = np.bincount(tok2, minlength=6)
    assert counts[3] == 0                       # p = 0 is never emitted
    nz = p > 0
    pe = p[nz].astype(np.float64)
    assert stats.chisquare(counts[nz], N * pe / pe.sum()).pvalue > 1e-3
    # the residual alone is max(0, p - q) renormalised: rejected slots follow it
    rej = n_out == 2
    r = np.maximum(p - q, 0).astype(np.float64)
    rc = np.bincount(tok2[rej], minlength=6)
    nzr = r > 0
    assert rc[~nzr].sum() == 0
    assert stats.chisquare(rc[nzr], rej.sum() * r[nzr] / r[nzr].sum()).pvalue > 1e-3


def test_accept_length_law_position_independent_rows():
    """With the same (p, q) at every slot, P(k - 2 >= j) = beta^j, so
    E[k - 2] = sum_{j=1}^{B-1} beta^j."""
    V, B = 5, 6
    p = synth.prob_rows(3, (V,))
    q = synth.prob_rows(4, (V,))
    N = 40_000
    seq_ids = np.arange(N)
    n = np.full(N, 3)
    it = np.zeros(N, dtype=np.int64)
    p_rows = np.broadcast_to(p, (N, B, V))
    q_rows = np.broadcast_to(q, (N, B - 1, V))
    y = _drafts_from(q_rows, 5, seq_ids, n, it)
    _, n_out = psispec.accept_block(p_rows, q_rows, y, 5, seq_ids, n, it)
    beta = float(np.minimum(p, q).sum())
    acc = n_out.astype(np.float64) - 2
    expect = sum(beta ** j for j in range(1, B))
    assert abs(acc.mean() - expect) < 5 * acc.std() / np.sqrt(N)
    for j in range(1, B):
        assert abs(np.mean(acc >= j) - beta ** j) < 5 * np.sqrt(beta ** j * (1 - beta ** j) / N) + 1e-9


def test_accept_degenerate_cases():
    """p == q accepts every slot (u <= 1 - 2^-24 < 1); p(y) = 0 rejects."""
    V, B, S = 7, 5, 300
    p = synth.prob_rows(8, (S, B, V))
    q = p[:, :-1].copy()
    seq_ids = np.arange(S)
    n = np.arange(S)
    it = np.ones(S, dtype=np.int64)
    y = _drafts_from(q, 1, seq_ids, n, it)
    out, n_out = psispec.accept_block(p, q, y, 1, seq_ids, n, it)
    assert np.all(n_out == B + 1)
    assert np.array_equal(out[:, :B], y)
    # bonus token follows p_{B+1}, drawn with the resample stream at n + B + 1
    for s in range(0, S, 37):
        w = rng.draw_word(1, s, n[s] + B + 1, rng.STREAM_RESAMPLE, 1)
        assert out[s, B] == rng.sample_icdf(p[s, B - 1], w)[0]
    # slot 2 drafted where p_2 = 0: always rejected there
    p0 = p.copy()
    p0[np.arange(S), 0, y[:, 1]] = 0.0
    out0, n0 = psispec.accept_block(p0, q, y, 1, seq_ids, n, it)
    assert np.all(n0 == 2)
    assert np.all(out0[:, 1] != y[:, 1])


def test_first_token_is_ar_exact_and_always_kept(tiny_w):
    """Draft row 0 (gate 0, position n) equals an AR-only single-row forward, and y_1
    is always emitted."""
    pr = synth.prompts(TINY, 2000, 3)
    dec = psispec.Decoder(TINY, tiny_w, [0, 1, 2], 3000, TINY.max_len)
    dec.prefill(list(pr))
    ref = psispec.Decoder(TINY, tiny_w, [0, 1, 2], 3000, TINY.max_len)
    ref.prefill(list(pr))
    for _ in range(4):
        lg, _ = model.forward(TINY, tiny_w, ref.t[:, None], ref.n[:, None], np.zeros((3, 1)),
                              {"k": ref.cache["k"].copy(), "v": ref.cache["v"].copy()})
        r = dec.step()
        assert np.allclose(r["P_d"][:, 0], model.probs(lg)[:, 0], rtol=1e-6, atol=1e-9)
        assert np.array_equal(r["out"][:, 0], r["y"][:, 0])
        ref.__dict__.update(n=dec.n.copy(), t=dec.t.copy(), it=dec.it.copy())
        ref.cache = {"k": dec.cache["k"].copy(), "v": dec.cache["v"].copy()}


@pytest.mark.parametrize("B", [1, 2, 4, 7])
def test_tpf_bounds_and_n_out_range(tiny_w, B):
    cfg = TINY.with_(block_size=B)
    S, N_new = 4, 23
    dec = psispec.Decoder(cfg, tiny_w, np.arange(S), 3000, cfg.prompt_len + N_new + B + 2)
    dec.prefill(list(synth.prompts(cfg, 2000, S)))
    toks, hist, fwd = dec.generate(N_new)
    for h in hist:
        assert np.all((h >= 2) & (h <= B + 1))
    tpf = N_new / fwd
    assert np.all(tpf >= 1.0 - 1e-12) and np.all(tpf <= (B + 1) / 2 + 1e-12)
    assert np.all((toks >= 0) & (toks < cfg.vocab - 1))
    if B == 1:
        assert all(np.all(h == 2) for h in hist)


def test_commit_leaves_exactly_the_ar_cache(tiny_w):
    """After every iteration, cache[0..n) equals the cache an AR-only prefill of the
    committed tokens builds (stale draft/verify entries beyond n are never kept)."""
    S = 3
    pr = synth.prompts(TINY, 2001, S)
    dec = psispec.Decoder(TINY, tiny_w, np.arange(S), 3001, TINY.max_len)
    dec.prefill(list(pr))
    committed = [list(p) for p in pr]
    for _ in range(5):
        r = dec.step()
        for s in range(S):
            committed[s] += list(r["out"][s, : r["n_out"][s]])
        ref = psispec.Decoder(TINY, tiny_w, np.arange(S), 3001, TINY.max_len)
        ref.prefill([np.array(c) for c in committed])
        for s in range(S):
            n = int(dec.n[s])
            assert n == len(committed[s]) - 1 == int(ref.n[s])
            assert int(dec.t[s]) == committed[s][-1]
            assert np.allclose(dec.cache["k"][:, s, :n], ref.cache["k"][:, s, :n], atol=1e-12)
            assert np.allclose(dec.cache["v"][:, s, :n], ref.cache["v"][:, s, :n], atol=1e-12)


def test_keyed_determinism_and_resume(tiny_w):
    """The same (seed, seq_id) yields the same tokens whatever the batch, and a
    decode resumed from committed tokens plus the saved iteration reproduces it."""
    pr = synth.prompts(TINY, 2002, 3)
    a = psispec.Decoder(TINY, tiny_w, [5, 6, 7], 77, TINY.max_len)
    a.prefill(list(pr))
    ta, _, _ = a.generate(20)
    b = psispec.Decoder(TINY, tiny_w, [7], 77, TINY.max_len)
    b.prefill([pr[2]])
    tb, _, _ = b.generate(20)
    assert np.array_equal(ta[2], tb[0])
    # resume: run 3 iterations, rebuild from committed tokens, continue
    c = psispec.Decoder(TINY, tiny_w, [7], 77, TINY.max_len)
    c.prefill([pr[2]])
    emitted = []
    for _ in range(3):
        r = c.step()
        emitted += list(r["out"][0, : r["n_out"][0]])
    d = psispec.Decoder(TINY, tiny_w, [7], 77, TINY.max_len)
    d.prefill([np.concatenate([pr[2], emitted])])
    d.it[:] = c.it
    more, _, _ = d.generate(20 - len(emitted)) if len(emitted) < 20 else (np.zeros((1, 0)), 0, 0)
    assert np.array_equal(np.concatenate([emitted, more[0]])[:20], ta[2])
    # a different seed changes the stream
    e = psispec.Decoder(TINY, tiny_w, [7], 78, TINY.max_len)
    e.prefill([pr[2]])
    te, _, _ = e.generate(20)
    assert not np.array_equal(te[0], ta[2])
