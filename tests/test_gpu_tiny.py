"""GPU parity on the tiny fp32 decoder: raw forwards, the paged KV cache, and whole
Psi-Spec iterations against the oracle (logits <= 1e-4 abs, probability TV <=
1e-3, tokens / accept lengths identical, cache equal to the oracle's)."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth
from oracle import model, nucleus, psispec
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

TINY = configs.TINY
LOGIT_TOL = 1e-4
TV_TOL = 1e-3


@pytest.fixture(scope="module")
def w_np():
    return synth.weights_numpy(TINY, 1000)


def _tv(a, b):
    return 0.5 * np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).sum(-1)


def test_forward_logits_hidden_and_cache(w_np):
    log("tiny forward")
    eng = engine(TINY, w_np, max_seqs=2, max_rows=40)
    r = np.random.default_rng(0)
    R = 12
    toks = r.integers(0, TINY.vocab, size=(2, R)).astype(np.int32)
    pos = np.tile(np.arange(R, dtype=np.int32), (2, 1))
    gate = (r.random((2, R)) < 0.5).astype(np.uint8)
    hid, lg = eng.forward([0, 1], R, dev(pos.ravel()), dev(gate.ravel()), tokens=dev(toks.ravel()),
                          want_hidden=True, want_logits=True)
    cache = model.new_cache(TINY, 2, 40)
    ref, xref = model.forward(TINY, w_np, toks, pos, gate, cache)
    g = host(lg).reshape(2, R, -1)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.abs(g[fin] - ref[fin]).max() <= LOGIT_TOL
    assert np.abs(host(hid).reshape(2, R, -1) - xref).max() <= LOGIT_TOL
    # continue both sequences by 4 rows at positions 12..15 (ragged gates)
    toks2 = r.integers(0, TINY.vocab, size=(2, 4)).astype(np.int32)
    pos2 = np.tile(np.arange(R, R + 4, dtype=np.int32), (2, 1))
    gate2 = np.array([[0, 1, 1, 0], [1, 1, 1, 1]], dtype=np.uint8)
    _, lg2 = eng.forward([0, 1], 4, dev(pos2.ravel()), dev(gate2.ravel()),
                         tokens=dev(toks2.ravel()), want_logits=True)
    ref2, _ = model.forward(TINY, w_np, toks2, pos2, gate2, cache)
    g2 = host(lg2).reshape(2, 4, -1)
    fin = np.isfinite(ref2)
    assert np.abs(g2[fin] - ref2[fin]).max() <= LOGIT_TOL
    for s in range(2):
        k, v = eng.kv_export(s, R + 4)
        assert np.abs(host(k) - cache["k"][:, s, : R + 4]).max() <= 1e-5
        assert np.abs(host(v) - cache["v"][:, s, : R + 4]).max() <= 1e-5
    eng.sync()


@pytest.mark.parametrize("stress,top_p", [(False, 0.0), (True, 0.0), (True, 0.9)])
def test_decode_iterations_match_oracle(stress, top_p):
    """prefill + 8 iterations of draft / verify / accept / commit on 5 sequences with
    ragged prompt lengths; every intermediate checked against the oracle (with top_p,
    both sides truncate the draft and verify laws to their nuclei)."""
    log(f"tiny decode stress={stress} top_p={top_p}")
    w = synth.weights_numpy(TINY, 1001, lm_head_std=0.35, lora_b_std=0.6) if stress \
        else synth.weights_numpy(TINY, 1000)
    S, seed = 5, 3000
    lens = [16, 9, 1, 16, 4]
    prompts = [synth.prompts(TINY, 2000 + i, 1, L)[0] for i, L in enumerate(lens)]
    seq_ids = [4, 0, 2, 1, 3]
    eng = engine(TINY, w, max_seqs=S, max_seq_len=TINY.max_len + 40, seed=seed, top_p=top_p)
    eng.prefill(seq_ids, prompts)
    dec = psispec.Decoder(TINY, w, seq_ids, seed, TINY.max_len + 40,
                          top_p=top_p if top_p > 0 else 1.0)
    dec.prefill(prompts)
    hist = []
    for step in range(8):
        y_g, pd_g = eng.draft(seq_ids, want_probs=True)
        out_g, n_g, pv_g = eng.verify(seq_ids, want_probs=True)
        r = dec.step()
        pd, pv = host(pd_g), host(pv_g)
        assert _tv(pd, r["P_d"]).max() <= TV_TOL
        assert _tv(pv, r["P_v"]).max() <= TV_TOL
        assert np.abs(pd - r["P_d"]).max() <= 1e-5
        assert np.array_equal(host(y_g), r["y"].astype(np.int32)), step
        assert np.array_equal(host(n_g), r["n_out"]), step
        assert np.array_equal(host(out_g), r["out"]), step
        hist += r["n_out"].tolist()
    for i, s in enumerate(seq_ids):
        L, t, it = eng.seq_state(s)
        assert (L, t, it) == (int(dec.n[i]), int(dec.t[i]), int(dec.it[i]))
        k, v = eng.kv_export(s, L)
        assert np.abs(host(k) - dec.cache["k"][:, i, :L]).max() <= 1e-5
        assert np.abs(host(v) - dec.cache["v"][:, i, :L]).max() <= 1e-5
    assert min(hist) >= 2 and max(hist) <= TINY.block_size + 1
    log(f"accept lengths {sorted(set(hist))}")
    eng.sync()


@pytest.mark.parametrize("B,laws", [(1, "stress"), (2, "stress"), (7, "stress"), (16, "stress"),
                                     (2, "flat"), (7, "flat"), (16, "flat")])
def test_decode_block_sizes_match_oracle(B, laws):
    """The linear sampler at block sizes other than the tiny model's 4: B = 1 (the
    draft holds only the AR slot, so every iteration emits exactly 2 tokens), B = 2,
    a ragged B = 7 and the 8B workload's B = 16; 6 iterations of 3 ragged sequences,
    tokens, accept lengths, laws and cache against the oracle.  "stress" weights
    give draft laws far from the AR laws (short accepted prefixes); "flat" weights
    (LM head N(0, 1e-3)) make every law nearly uniform, so whole blocks are accepted
    and the bonus token past the block is drawn from the verify law."""
    log(f"tiny decode block size {B}, {laws} laws")
    cfg = TINY.with_(block_size=B)
    w = synth.weights_numpy(cfg, 1001, lm_head_std=0.35, lora_b_std=0.6) if laws == "stress" \
        else synth.weights_numpy(cfg, 1002, lm_head_std=1e-3)
    S, seed, iters = 3, 3100 + B, 6
    lens = [16, 5, 1]
    prompts = [synth.prompts(cfg, 2100 + i, 1, L)[0] for i, L in enumerate(lens)]
    seq_ids = [2, 0, 1]
    max_len = cfg.prompt_len + iters * (B + 1) + B + 2
    eng = engine(cfg, w, max_seqs=S, max_seq_len=max_len, seed=seed)
    eng.prefill(seq_ids, prompts)
    dec = psispec.Decoder(cfg, w, seq_ids, seed, max_len)
    dec.prefill(prompts)
    hist = []
    for step in range(iters):
        y_g, pd_g = eng.draft(seq_ids, want_probs=True)
        out_g, n_g, pv_g = eng.verify(seq_ids, want_probs=True)
        r = dec.step()
        pd, pv = host(pd_g), host(pv_g)
        assert _tv(pd, r["P_d"]).max() <= TV_TOL
        assert _tv(pv, r["P_v"]).max() <= TV_TOL
        assert np.array_equal(host(y_g), r["y"].astype(np.int32)), step
        assert np.array_equal(host(n_g), r["n_out"]), step
        assert np.array_equal(host(out_g), r["out"]), step
        hist += r["n_out"].tolist()
    for i, s in enumerate(seq_ids):
        L, t, it = eng.seq_state(s)
        assert (L, t, it) == (int(dec.n[i]), int(dec.t[i]), int(dec.it[i]))
        k, v = eng.kv_export(s, L)
        assert np.abs(host(k) - dec.cache["k"][:, i, :L]).max() <= 1e-5
        assert np.abs(host(v) - dec.cache["v"][:, i, :L]).max() <= 1e-5
    assert min(hist) >= 2 and max(hist) <= B + 1
    if B == 1:
        assert set(hist) == {2}
    if laws == "flat":
        assert max(hist) == B + 1
    log(f"  accept lengths {sorted(set(hist))}")
    eng.sync()


def test_top_p_config_filters_draft_bit_exact():
    """The top_p config field applies exactly the nucleus rule to the softmax rows:
    two contexts on the same weights and seed, one with top_p 0.9, give draft laws
    that the oracle's filter maps one onto the other bit for bit; the draws stay
    inside the nuclei, and the verify rows are truncated too (zeros beyond the mask
    column, unit mass).  The verify laws themselves are checked against the oracle
    by the decode test with top_p."""
    w = synth.weights_numpy(TINY, 1001, lm_head_std=0.35, lora_b_std=0.6)
    S = 3
    prompts = list(synth.prompts(TINY, 2200, S))
    ids = [0, 1, 2]
    res = []
    for tp in (0.0, 0.9):
        log(f"tiny top_p config {tp}")
        eng = engine(TINY, w, max_seqs=S, seed=77, top_p=tp)
        eng.prefill(ids, prompts)
        y, pd = eng.draft(ids, want_probs=True)
        _, _, pv = eng.verify(ids, want_probs=True)
        res.append((host(y).copy(), host(pd).copy(), host(pv).copy()))
        eng.sync()
    (_, pd0, pv0), (y1, pd1, pv1) = res
    assert np.array_equal(nucleus.filter_rows(pd0, 0.9), pd1)
    assert ((pd1 == 0).sum(-1) > (pd0 == 0).sum(-1)).all()
    drawn = np.take_along_axis(pd1, y1[..., None].astype(np.int64), -1)[..., 0]
    assert (drawn > 0).all()
    assert ((pv1 == 0).sum(-1) > (pv0 == 0).sum(-1).min()).all()
    assert np.abs(pv1.astype(np.float64).sum(-1) - 1).max() <= 1e-5


def test_step_equals_draft_then_verify_and_release(w_np):
    S = 3
    prompts = list(synth.prompts(TINY, 2100, S))
    outs = []
    for mode in ("step", "split"):
        eng = engine(TINY, w_np, max_seqs=S, seed=9)
        eng.prefill([0, 1, 2], prompts)
        seq = []
        for _ in range(4):
            if mode == "step":
                o, n = eng.step([0, 1, 2])
            else:
                eng.draft([0, 1, 2])
                o, n, _ = eng.verify([0, 1, 2])
            seq.append((host(o).copy(), host(n).copy()))
        outs.append(seq)
        free0 = eng.free_pages()
        eng.release(1)
        assert eng.free_pages() > free0
        eng.sync()
    for (a, b), (c, d) in zip(*outs):
        assert np.array_equal(a, c) and np.array_equal(b, d)


def test_state_errors(w_np):
    from diffusion_drafted_lora_amd import uno
    eng = engine(TINY, w_np, max_seqs=2, seed=9)
    with pytest.raises(uno.UnoError) as e:
        eng.draft([0])                       # not prefilled
    assert e.value.status == 3
    eng.prefill([0], [synth.prompts(TINY, 1, 1)[0]])
    with pytest.raises(uno.UnoError) as e:
        eng.verify([0])                      # no draft
    assert e.value.status == 3
    with pytest.raises(uno.UnoError) as e:
        eng.draft([0, 0])                    # duplicate id
    assert e.value.status == 1
    eng.sync()


def test_page_pool_and_length_limits_leave_state_intact():
    """Capacity limits during decode: a step that needs more KV pages than the pool has
    left fails with OUT_OF_PAGES and changes nothing (lengths, pending tokens, cache);
    after the other sequence is released the same sequence steps on and matches an
    oracle decoder of that sequence alone; a step that could write past max_seq_len
    fails with INVALID_ARG, again leaving the state and cache as they were, and no
    device flag is raised.  The pool holds 5 pages of 16 positions for two sequences
    of up to 64 (4 pages each)."""
    from diffusion_drafted_lora_amd import uno
    log("tiny decode at the page-pool and length limits")
    w = synth.weights_numpy(TINY, 1001, lm_head_std=0.35, lora_b_std=0.6)
    seed, max_len = 3300, 64
    prompts = [synth.prompts(TINY, 2300 + i, 1, 16)[0] for i in range(2)]
    eng = engine(TINY, w, max_seqs=2, max_seq_len=max_len, n_pages=5, seed=seed)
    eng.prefill([0, 1], prompts)
    decs = []
    for s in (0, 1):
        d = psispec.Decoder(TINY, w, [s], seed, max_len)
        d.prefill([prompts[s]])
        decs.append(d)

    def states(ids):
        return [eng.seq_state(s) for s in ids]

    def check_step(ids):
        out, n_out = eng.step(ids)
        for j, s in enumerate(ids):
            r = decs[s].step()
            assert int(host(n_out)[j]) == int(r["n_out"][0])
            assert np.array_equal(host(out)[j], r["out"][0])

    for _ in range(60):
        before = states([0, 1])
        try:
            check_step([0, 1])
        except uno.UnoError as e:
            assert e.status == 2, e
            assert states([0, 1]) == before
            break
    else:
        pytest.fail("the 5-page pool never ran out")
    log(f"  pool exhausted at lengths {[b[0] for b in before]}")
    eng.release(1)
    for _ in range(60):
        before = states([0])
        try:
            check_step([0])
        except uno.UnoError as e:
            assert e.status == 1, e
            assert states([0]) == before
            break
    else:
        pytest.fail("max_seq_len was never reached")
    L, t, it = before[0]
    log(f"  length limit at length {L}")
    assert L + TINY.block_size + 1 > max_len
    assert (L, t, it) == (int(decs[0].n[0]), int(decs[0].t[0]), int(decs[0].it[0]))
    k, v = eng.kv_export(0, L)
    assert np.abs(host(k) - decs[0].cache["k"][:, 0, :L]).max() <= 1e-5
    assert np.abs(host(v) - decs[0].cache["v"][:, 0, :L]).max() <= 1e-5
    eng.sync()


def test_timing_records_every_nth_call(w_np):
    """Kernel timing: every call of an enabled class is recorded by default; with
    a period n only the first of every n calls is, and the untimed calls still
    run (same tokens)."""
    S = 2
    prompts = list(synth.prompts(TINY, 2300, S))
    counts, outs = {}, {}
    for every in (1, 3):
        eng = engine(TINY, w_np, max_seqs=S, seed=11)
        eng.prefill([0, 1], prompts)
        eng.timing(["linear", "attention"], every=every)
        o, n = eng.step([0, 1])
        outs[every] = (host(o).copy(), host(n).copy())
        counts[every] = {c: eng.timing_read(c) for c in ("linear", "attention", "lm_head")}
        eng.timing([])
        eng.sync()
    calls = 2 * TINY.n_layers * 3                     # q|k|v, o, down per forward
    assert counts[1]["linear"][0] == calls
    assert counts[3]["linear"][0] == (calls + 2) // 3
    assert counts[1]["attention"][0] == 2 * TINY.n_layers
    assert counts[3]["attention"][0] == (2 * TINY.n_layers + 2) // 3
    assert counts[1]["lm_head"][0] == 0                # class not enabled
    assert counts[1]["linear"][1] > 0 and counts[3]["linear"][1] > 0
    assert np.array_equal(outs[1][0], outs[3][0]) and np.array_equal(outs[1][1], outs[3][1])


def test_huge_activations_set_numeric_flag(w_np):
    """Rows whose sum of squares leaves the exact fixed-point range (here x ~ 1e5,
    sum ~ 6e11) set the numeric flag instead of wrapping silently."""
    eng = engine(TINY, w_np, max_seqs=1, max_rows=8)
    pos = np.arange(4, dtype=np.int32)
    x = np.full((4, TINY.d_model), 1e5, dtype=np.float32)
    eng.forward([0], 4, dev(pos), dev(np.zeros(4, np.uint8)), hidden_in=dev(x), want_hidden=True)
    with pytest.raises(Exception, match="NUMERIC"):
        eng.sync()
