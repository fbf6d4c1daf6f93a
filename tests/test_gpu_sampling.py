"""GPU parity of the keyed sampler and the accept/resample kernel: bit-exact
against the oracle on the same probability tensors and Philox keys."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth
from oracle import psispec, rng
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu


def _sampler_engine(V, max_rows=64, B=4, max_seqs=16):
    cfg = configs.TINY.with_(vocab=V, n_layers=1, block_size=B)
    w = synth.weights_numpy(cfg, 1, with_embed=False)
    return cfg, engine(cfg, w, max_seqs=max_seqs, max_rows=max(max_rows, max_seqs * B), seed=1234)


@pytest.mark.parametrize("V", [32, 2048, 2064, 151936])
def test_sample_bit_exact(V):
    rows = 48
    log(f"sample V={V}")
    cfg, eng = _sampler_engine(V)
    w = synth.prob_rows(V + 1, (rows, V), zero_frac=0.4)
    w[3] = 0.0
    w[3, V - 1] = 1.0            # all mass on the last index (ragged tail chunk)
    w[5] = 0.0
    w[5, 0] = 1.0
    r = np.random.default_rng(V)
    seq = r.integers(0, 1000, rows).astype(np.int32)
    pos = r.integers(0, 10000, rows).astype(np.int32)
    it = r.integers(0, 50, rows).astype(np.int32)
    for stream in (0, 2):
        idx = host(eng.sample(dev(w), dev(seq), dev(pos), dev(it), stream))
        ref, _ = rng.sample_icdf(w, rng.draw_word(1234, seq, pos, stream, it))
        assert np.array_equal(idx, ref.astype(np.int32))
    eng.sync()


def test_sample_zero_row_sets_numeric_flag():
    cfg, eng = _sampler_engine(32)
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, 4] = 1.0
    z = np.zeros(2, dtype=np.int32)
    idx = host(eng.sample(dev(w), dev(z), dev(z), dev(z), 0))
    assert idx[0] == 4 and idx[1] == -1
    with pytest.raises(Exception, match="NUMERIC"):
        eng.sync()


def _accept_case(eng, p, q, y, seq, n, it, seed):
    out, n_out = eng.accept(dev(p), dev(q), dev(y.astype(np.int32)), dev(seq), dev(n), dev(it))
    ro, rn = psispec.accept_block(p, q, y, seed, seq, n, it)
    assert np.array_equal(host(n_out), rn)
    assert np.array_equal(host(out), ro)
    return rn


def test_accept_bit_exact_on_oracle_decode_tensors():
    """Feed the accept kernel the oracle's own p / q from real decode steps."""
    cfg = configs.TINY
    w = synth.weights_numpy(configs.TINY, 1001, lm_head_std=0.35, lora_b_std=0.6)
    S = 16
    dec = psispec.Decoder(cfg, w, np.arange(S), 1234, cfg.max_len)
    dec.prefill(list(synth.prompts(cfg, 2000, S)))
    _, eng = _sampler_engine(cfg.vocab, B=cfg.block_size, max_seqs=S)
    seen = set()
    for step in range(6):
        n0, it0 = dec.n.astype(np.int32), dec.it.astype(np.int32)
        r = dec.step()
        rn = _accept_case(eng, r["P_v"], np.ascontiguousarray(r["P_d"][:, 1:]), r["y"],
                          dec.seq_ids.astype(np.int32), n0, it0, 1234)
        seen.update(rn.tolist())
    log(f"accept lengths seen {sorted(seen)}")
    assert len(seen) >= 2
    eng.sync()


@pytest.mark.parametrize("V,B", [(151936, 16), (2080, 7), (32, 1)])
def test_accept_bit_exact_synthetic(V, B):
    """Synthetic rows at the 8B vocabulary and block size, drafts drawn from q;
    p is a perturbation of q so every accept length occurs."""
    log(f"accept V={V} B={B}")
    S = 12
    _, eng = _sampler_engine(V, B=B, max_seqs=S)
    q = synth.prob_rows(V + B, (S, max(B - 1, 1), V), alpha=0.3)[:, : B - 1]
    noise = synth.prob_rows(V + B + 1, (S, B, V), alpha=0.3)
    base = np.concatenate([q, noise[:, :1]], axis=1) if B > 1 else noise
    mix = np.linspace(0.0, 1.0, S, dtype=np.float32)[:, None, None]
    p = ((1 - mix) * base + mix * noise).astype(np.float32)
    p /= p.sum(-1, keepdims=True)
    p = p.astype(np.float32)
    seq = np.arange(100, 100 + S, dtype=np.int32)
    n = np.arange(S, dtype=np.int32) * 37 + 5
    it = np.arange(S, dtype=np.int32) % 3
    y = np.zeros((S, B), dtype=np.int64)
    y[:, 0] = 7
    for i in range(2, B + 1):
        wd = rng.draw_word(1234, seq, n + i, rng.STREAM_DRAFT, it)
        y[:, i - 1], _ = rng.sample_icdf(q[:, i - 2], wd)
    qq = np.ascontiguousarray(q) if B > 1 else np.zeros((S, 1, V), np.float32)
    _accept_case(eng, np.ascontiguousarray(p), qq, y, seq, n, it, 1234)
    # degenerate: p == q everywhere -> every slot accepted, bonus drawn from p_{B+1}
    if B > 1:
        p2 = np.concatenate([q, noise[:, :1]], axis=1).astype(np.float32)
        rn = _accept_case(eng, np.ascontiguousarray(p2), qq, y, seq, n, it, 1234)
        assert np.all(rn == B + 1)
        # p_2(y_2) = 0 -> slot 2 always rejected
        p3 = p2.copy()
        p3[np.arange(S), 0, y[:, 1]] = 0.0
        rn = _accept_case(eng, np.ascontiguousarray(p3), qq, y, seq, n, it, 1234)
        assert np.all(rn == 2)
    eng.sync()


def test_accept_nan_sets_numeric_flag():
    cfg = configs.TINY
    _, eng = _sampler_engine(cfg.vocab, B=cfg.block_size, max_seqs=2)
    p = synth.prob_rows(1, (2, 4, 32))
    q = synth.prob_rows(2, (2, 3, 32))
    p[1, 0, :] = np.nan
    y = np.ones((2, 4), dtype=np.int32)
    z = np.zeros(2, dtype=np.int32)
    eng.accept(dev(p), dev(q), dev(y), dev(z), dev(z), dev(z))
    with pytest.raises(Exception, match="NUMERIC"):
        eng.sync()


@pytest.mark.parametrize("V", [32, 2080, 151936])
def test_top_p_bit_exact(V):
    """Top-p truncation (uno_top_p) against the oracle's exact reading, bit for bit:
    softmax rows of several temperatures, rows with many tied values, rows with
    zero entries, and top-p from 0.05 to 1 (identity)."""
    import torch
    from diffusion_drafted_lora_amd import uno
    from oracle import nucleus
    rng = np.random.default_rng(V)
    rows = []
    for scale in (0.5, 2.0, 6.0):
        lg = rng.normal(0.0, scale, size=(3, V))
        p = np.exp(lg - lg.max(-1, keepdims=True))
        rows.append(p / p.sum(-1, keepdims=True))
    ties = np.exp(rng.integers(-4, 3, size=(2, V)) * 0.9)        # heavy ties
    rows.append(ties / ties.sum(-1, keepdims=True))
    sparse = rng.random((2, V)) * (rng.random((2, V)) < 0.3)       # zeros
    sparse[:, 0] = 1.0
    rows.append(sparse / sparse.sum(-1, keepdims=True))
    P = np.concatenate(rows).astype(np.float32)
    for top_p in (0.05, 0.5, 0.9, 0.95, 0.999, 1.0):
        got = host(uno.top_p(dev(P), top_p))
        want = nucleus.filter_rows(P, top_p)
        assert np.array_equal(got, want), f"V={V} top_p={top_p}"
    # in place
    t = dev(P)
    uno.top_p(t, 0.95, out=t)
    assert np.array_equal(host(t), nucleus.filter_rows(P, 0.95))


def test_top_p_exact_boundary_and_errors():
    import torch
    from diffusion_drafted_lora_amd import uno
    from oracle import nucleus
    d = np.array([[0.5, 0.25, 0.125, 0.125], [0.25, 0.25, 0.25, 0.25]], dtype=np.float32)
    got = host(uno.top_p(dev(d), 0.75))
    assert np.array_equal(got, nucleus.filter_rows(d, 0.75))
    assert np.flatnonzero(got[0]).tolist() == [0, 1]
    with pytest.raises(uno.UnoError):
        uno.top_p(dev(d), 0.0)
