"""GPU parity of the tree sampler (uno_tree_draft / uno_tree_verify / uno_tree_accept)
against the oracle (oracle/tree.py).

* the acceptance kernel is bit-exact on the oracle's own tensors: the tiny model's
  decode steps, and synthetic rows at vocabulary 151936 with B 16 and K 1..4 where
  the laws agree up to a per-sequence depth and then differ, so that the walk
  passes several depths and then rejects every candidate through the integer
  residual chain; with K = 1 it equals the linear accept kernel;
* the chain draws are bit-exact on the GPU's own draft laws;
* on the tiny float32 model, whole tree iterations (K = 3, five ragged sequences)
  match the oracle: verify laws (TV <= 1e-3), chains, emitted tokens, accept
  lengths, the chosen chain, and the KV cache at the committed positions;
* one chain through the tree entry points equals uno_step on the same context;
* call-order errors."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import tree
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

TINY = configs.TINY
TV_TOL = 1e-3


def _tv(a, b):
    return 0.5 * np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).sum(-1)


@pytest.fixture(scope="module")
def stress_w():
    return synth.weights_numpy(TINY, 1001, lm_head_std=0.35, lora_b_std=0.6)


def _i32(a):
    return dev(np.asarray(a, dtype=np.int32))


@pytest.mark.parametrize("B,K,top_p", [(4, 3, 0.0), (4, 3, 0.9), (2, 2, 0.0), (1, 2, 0.0)])
def test_tree_decode_matches_oracle(stress_w, B, K, top_p):
    """Blocks of 4 (with and without top-p 0.9: both sides truncate every draft
    and verify row to its nucleus), 2 and 1 (no drafted depth: y_1 and the bonus)."""
    S, seed = 5, 3300
    lens = [16, 9, 1, 16, 4]
    cfg = TINY.with_(block_size=B)
    prompts = [synth.prompts(cfg, 2300 + i, 1, L)[0] for i, L in enumerate(lens)]
    ids = [4, 0, 2, 1, 3]
    cap = cfg.max_len + 60
    log(f"tiny tree decode B={B} K={K} top_p={top_p}")
    eng = engine(cfg, stress_w, max_seqs=S, max_seq_len=cap, seed=seed,
                 max_rows=S * max(B, 1 + K * (B - 1)), tree_chains=K, top_p=top_p)
    eng.prefill(ids, prompts)
    dec = tree.TreeDecoder(cfg, stress_w, ids, seed, cap, top_p=top_p if top_p > 0 else 1.0)
    dec.prefill(prompts)
    seen_side = False
    for step in range(8):
        n0, it0 = dec.n.copy(), dec.it.copy()
        ch_g, pd_g = eng.tree_draft(ids, K, want_probs=True)
        # the draws, bit-exact on the GPU's own draft laws
        own = tree.draft_chains(host(pd_g), K, seed, ids, n0, it0)
        assert np.array_equal(host(ch_g), own.astype(np.int32)), step
        out_g, n_g, ks_g, pv_g = eng.tree_verify(ids, K, want_probs=True)
        r = dec.step_tree(K)
        assert _tv(host(pd_g), r["P_d"]).max() <= TV_TOL, step
        assert np.array_equal(host(ch_g), r["chains"].astype(np.int32)), step
        assert _tv(host(pv_g), r["P_v"]).max() <= TV_TOL, step
        assert np.array_equal(host(out_g), r["out"]), step
        assert np.array_equal(host(n_g), r["n_out"]), step
        assert np.array_equal(host(ks_g), r["kstar"]), step
        seen_side |= bool(((r["kstar"] > 0) & (r["n_out"] >= 3)).any())
    for i, s in enumerate(ids):
        L, t, it = eng.seq_state(s)
        assert (L, t, it) == (int(dec.n[i]), int(dec.t[i]), int(dec.it[i]))
        k, v = eng.kv_export(s, L)
        assert np.abs(host(k) - dec.cache["k"][:, i, :L]).max() <= 1e-5
        assert np.abs(host(v) - dec.cache["v"][:, i, :L]).max() <= 1e-5
    eng.sync()
    log(f"  a side chain carried the accepted path: {seen_side}")


def test_tree_accept_bit_exact_on_oracle_decode_tensors(stress_w):
    K, S, seed = 3, 4, 3400
    B = TINY.block_size
    prompts = list(synth.prompts(TINY, 2400, S))
    ids = [3, 1, 0, 2]
    dec = tree.TreeDecoder(TINY, stress_w, ids, seed, TINY.max_len + 60)
    dec.prefill(prompts)
    eng = engine(TINY, stress_w, max_seqs=S, seed=seed, max_rows=S * (1 + K * (B - 1)),
                 tree_chains=K)
    for step in range(6):
        n0, it0 = dec.n.copy(), dec.it.copy()
        r = dec.step_tree(K)
        out, n_out, ks = eng.tree_accept(dev(r["P_v"]), dev(r["P_d"]), _i32(r["chains"]), _i32(ids),
                                         _i32(n0), _i32(it0))
        assert np.array_equal(host(out), r["out"]), step
        assert np.array_equal(host(n_out), r["n_out"]), step
        assert np.array_equal(host(ks), r["kstar"]), step
    eng.sync()


def _peaked(seed, S, B, V):
    """Rows with 0.7 of their mass on one random token, so that independent chains
    often agree and several stay live."""
    g = np.random.default_rng(seed)
    w = 0.3 * synth.prob_rows(seed, (S, B, V)).astype(np.float64)
    top = g.integers(0, V, size=(S, B))
    np.put_along_axis(w, top[..., None], np.take_along_axis(w, top[..., None], -1) + 0.7, -1)
    return (w / w.sum(-1, keepdims=True)).astype(np.float32)


def _synthetic(K, B, V, S, seed):
    """Draft laws, chains and verify laws where p = q up to depth D_s of sequence
    s (every first candidate passes there) and a different law after it."""
    g = np.random.default_rng(seed)
    q = _peaked(seed, S, B, V)
    other = _peaked(seed + 1, S, B, V)
    ids = np.arange(S) * 7 + 1
    n = g.integers(100, 5000, size=S)
    it = g.integers(0, 50, size=S)
    chains = tree.draft_chains(q, K, seed, ids, n, it)
    depth = g.integers(2, B + 2, size=S)       # first depth whose law differs (B+1: none)
    depth[:2] = (2, 5)
    Rv = 1 + K * (B - 1)
    P_v = np.empty((S, Rv, V), np.float32)
    for s in range(S):
        for k in range(K):
            for dt in range(1, B + 1):          # row holding depth dt predicts depth dt + 1
                law = q[s, dt] if dt + 1 <= B and dt + 1 < depth[s] else other[s, min(dt, B - 1)]
                P_v[s, tree.verify_row(k, dt, B)] = law
    return q, chains, P_v, ids, n, it


@pytest.mark.parametrize("K", [1, 2, 4])
def test_tree_accept_bit_exact_large_vocab(K):
    B, V, S, seed = 16, 151936, 6, 3500 + K
    log(f"tree accept V={V} B={B} K={K}")
    q, chains, P_v, ids, n, it = _synthetic(K, B, V, S, seed)
    ref_out, ref_n, ref_k = tree.tree_accept(P_v, q, chains, seed, ids, n, it)
    # chains live at each stop: more than one means the residual chain ran
    live_at_stop = [int(np.all(chains[s, :, 1:ref_n[s] - 1] == ref_out[s, 1:ref_n[s] - 1],
                               axis=1).sum()) for s in range(S) if ref_n[s] <= B]
    if K > 1:
        assert max(live_at_stop) > 1, live_at_stop
    eng = _accept_engine(B, V, S, seed)
    out, n_out, ks = eng.tree_accept(dev(P_v), dev(q), _i32(chains), _i32(ids), _i32(n), _i32(it))
    assert np.array_equal(host(out), ref_out)
    assert np.array_equal(host(n_out), ref_n)
    assert np.array_equal(host(ks), ref_k)
    log(f"  accept lengths {ref_n.tolist()}, chains live at the stops {live_at_stop}, "
        f"chosen chains {ref_k.tolist()}")
    if K == 1:
        lin_out, lin_n = eng.accept(dev(P_v[:, :B]), dev(np.ascontiguousarray(q[:, 1:])),
                                    _i32(chains[:, 0]), _i32(ids), _i32(n), _i32(it))
        assert np.array_equal(host(lin_out), ref_out)
        assert np.array_equal(host(lin_n), ref_n)
    eng.sync()


def _accept_engine(B, V, S, seed):
    """A small bf16 context whose vocabulary and block size match the synthetic
    rows (the accept entry reads only the probability tensors)."""
    cfg = configs.TINY.with_(name="accept-only", dtype="bf16", n_layers=1, d_model=64,
                             n_q_heads=2, n_kv_heads=1, head_dim=32, ffn_dim=64, vocab=V,
                             lora_rank=32, lora_alpha=64.0, block_size=B)
    w = synth.weights_numpy(cfg, 9, with_embed=False, with_lora=False)
    return engine(cfg, w, max_seqs=S, seed=seed, max_seq_len=64, tree_chains=4)


@pytest.mark.parametrize("B", [4, 2, 1])
def test_one_chain_equals_the_linear_step(stress_w, B):
    S, seed = 3, 3600
    cfg = TINY.with_(block_size=B)
    prompts = list(synth.prompts(cfg, 2600, S))
    ids = [0, 1, 2]
    lin = engine(cfg, stress_w, max_seqs=S, seed=seed)
    tr = engine(cfg, stress_w, max_seqs=S, seed=seed, max_rows=S * B, tree_chains=1)
    lin.prefill(ids, prompts)
    tr.prefill(ids, prompts)
    for step in range(6):
        a_out, a_n = lin.step(ids)
        b_out, b_n = tr.tree_step(ids, 1)
        assert np.array_equal(host(a_out), host(b_out)), step
        assert np.array_equal(host(a_n), host(b_n)), step
    lin.sync()
    tr.sync()


def test_tree_call_order_errors(stress_w):
    B = TINY.block_size
    eng = engine(TINY, stress_w, max_seqs=2, seed=1, max_rows=2 * (1 + 2 * (B - 1)),
                 tree_chains=2)
    eng.prefill([0, 1], list(synth.prompts(TINY, 2700, 2)))
    with pytest.raises(uno.UnoError) as e:
        eng.tree_verify([0, 1], 2)                 # no draft
    assert e.value.status == 3
    eng.tree_draft([0, 1], 2)
    with pytest.raises(uno.UnoError) as e:
        eng.verify([0, 1])                         # a linear verify of a tree draft
    assert e.value.status == 3
    eng.tree_verify([0, 1], 2)
    with pytest.raises(uno.UnoError) as e:
        eng.tree_draft([0, 1], 3)                  # more chains than tree_chains
    assert e.value.status == 1
    eng.draft([0, 1])
    with pytest.raises(uno.UnoError) as e:
        eng.tree_verify([0, 1], 2)                 # a tree verify of a linear draft
    assert e.value.status == 3
    eng.verify([0, 1])
    eng.sync()
    plain = engine(TINY, stress_w, max_seqs=1, seed=1)
    with pytest.raises(uno.UnoError) as e:
        plain.tree_draft([0], 1)                   # the context has no tree chains
    assert e.value.status == 1


def _exact_chain_laws(cfg, wt, prompt, chains, pos):
    """float64 oracle laws of each chain's block after the prompt, on the same
    (bf16-valued) weights."""
    from oracle import model

    def h(t):
        return t.float().cpu().numpy().astype(np.float64)

    wn = {"embed": h(wt["embed"]), "lm_head": h(wt["lm_head"]), "final_norm": h(wt["final_norm"]),
          "layers": [{"attn_norm": h(lw["attn_norm"]), "mlp_norm": h(lw["mlp_norm"]),
                      "w": {p: h(t) for p, t in lw["w"].items()},
                      "la": {p: h(t) for p, t in lw["la"].items()},
                      "lb": {p: h(t) for p, t in lw["lb"].items()}} for lw in wt["layers"]]}
    cf = cfg.with_(dtype="f32")
    cache = model.new_cache(cf, 1, int(pos.max()) + 2)
    toks = np.asarray(prompt, np.int64)
    model.forward(cf, wn, toks[None], np.arange(len(toks))[None], np.zeros((1, len(toks))), cache,
                  want_logits=False)
    out = []
    for k in range(chains.shape[0]):
        ck = {"k": cache["k"].copy(), "v": cache["v"].copy()}
        lg, _ = model.forward(cf, wn, chains[k][None], pos[k][None], np.zeros((1, len(pos[k]))), ck)
        out.append(model.probs(lg)[0].astype(np.float64))
    return out


def test_tree_verify_bf16_8b_layers_match_plain_forwards():
    """The bf16 kernels at the 8B layer shape (two layers, vocabulary 2048): every
    row of a K = 3 tree verify (46 rows: the few-row GEMMs over three row tiles,
    the windowed ring attention, side-chain KV slots) against the float64 oracle
    of its chain, beside plain causal forwards of the same chains on a second
    context (16-row GEMM tiles, the plain ring).  Both store the same bf16 values;
    their attention rounds P to bf16 against running maxima of different key
    groupings, so they differ from each other by bf16 noise.  The bar: the tree
    rows are no farther from the exact laws than the plain forwards (x 1.25 +
    1e-4), and within 1e-2 of them.  After acceptance the accepted path's K/V sit
    at their positions (within bf16 rounding of the plain forward's)."""
    import torch
    cfg = configs.LAYER8B.with_(n_layers=2, vocab=2048)
    K, B = 3, cfg.block_size
    log("8B-shape bf16 tree verify vs plain forwards and the float64 oracle")
    wt = synth.weights_torch(cfg, 7100, "cuda")
    w = uno.pack_weights(cfg, wt)
    prompt = synth.prompts(cfg, 7101, 1, 300)[0]
    eng = uno.Engine(cfg, w, max_seqs=1, max_seq_len=600, max_rows=64, seed=7102, tree_chains=K)
    ref = uno.Engine(cfg, w, max_seqs=K, max_seq_len=600, max_rows=64, seed=7102)
    eng.prefill([0], [prompt])
    ref.prefill(list(range(K)), [prompt] * K)
    n = len(prompt) - 1
    ch, _ = eng.tree_draft([0], K)
    out, n_out, ks, pv = eng.tree_verify([0], K, want_probs=True)
    ch, pv = host(ch)[0], host(pv)[0].astype(np.float64)
    # reference: the pending token at n, then each chain's block at n+1..n+B
    ids = list(range(K))
    ref.forward(ids, 1, _i32(np.full(K, n)), dev(np.zeros(K, np.uint8)),
                tokens=_i32(np.full(K, prompt[-1])))
    pos = np.tile(np.arange(n + 1, n + 1 + B), (K, 1))
    _, lg = ref.forward(ids, B, _i32(pos.ravel()), dev(np.zeros(K * B, np.uint8)),
                        tokens=_i32(ch.ravel()), want_logits=True)
    lg = host(lg).astype(np.float64).reshape(K, B, -1)
    lg -= lg.max(-1, keepdims=True)
    P = np.exp(lg)
    P /= P.sum(-1, keepdims=True)
    ex = _exact_chain_laws(cfg, wt, prompt, ch.astype(np.int64), pos)
    t_tree = t_plain = t_pair = 0.0
    for k in range(K):
        for dt in range(1, B + 1):
            row = pv[tree.verify_row(k, dt, B)]
            t_tree = max(t_tree, float(_tv(row, ex[k][dt - 1])))
            t_plain = max(t_plain, float(_tv(P[k, dt - 1], ex[k][dt - 1])))
            t_pair = max(t_pair, float(_tv(row, P[k, dt - 1])))
    log(f"  max TV to the exact laws: tree rows {t_tree:.2e}, plain forwards {t_plain:.2e}; "
        f"between them {t_pair:.2e}")
    assert t_tree <= 1.25 * t_plain + 1e-4
    assert t_pair <= 1e-2
    k_out, kstar = int(host(n_out)[0]), int(host(ks)[0])
    L = n + k_out
    assert eng.seq_state(0)[0] == L
    ek, ev = eng.kv_export(0, L)
    rk, rv = ref.kv_export(kstar, n + B + 1)
    for a, b in ((ek, rk), (ev, rv)):
        a = host(a.float())[:, n + 1: L]
        b = host(b.float())[:, n + 1: L]
        assert np.abs(a - b).max() <= 2e-2 * max(1.0, float(np.abs(b).max()))
    eng.sync()
    ref.sync()
