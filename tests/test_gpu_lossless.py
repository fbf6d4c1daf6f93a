"""Losslessness and sequence-slot reuse on the GPU path (the tiny fp32 decoder).

* chi^2: the first two tokens emitted by uno_step for 65,536 sequences that share
  a prompt (stress weights: the draft and AR laws differ by a large total
  variation, so a broken accept / resample would show) follow the exact AR joint
  law enumerated by brute force with the oracle (p > 0.01), and agree token for
  token with the oracle's own Psi-Spec run on the same Philox keys.
* Slot reuse: a sequence released and prefilled again while the previous
  iteration's length snapshot may still be in flight keeps correct page bounds:
  its tokens equal a fresh oracle decoder's, and no device bounds check trips."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import psispec
from tests.gpu_util import dev, engine, host, log
from tests.test_oracle_lossless import STRESS, _chi2_pvalue, _exact_joint2

pytestmark = pytest.mark.gpu

TINY = configs.TINY


def _shared_prompt_engine(w, prompt, n, seed):
    """n sequences (ids 0..n-1) holding the same prefilled prompt: sequence 0 is
    prefilled, the others import its K/V, length, pending token and iteration."""
    eng = engine(TINY, w, max_seqs=n, seed=seed)
    eng.prefill([0], [prompt])
    P = len(prompt)
    k, v = eng.kv_export(0, P - 1)
    for s in range(1, n):
        eng.kv_import(s, k, v, pending=int(prompt[-1]), iteration=0)
    return eng


def test_gpu_lossless_first_two_tokens_stress():
    w = synth.weights_numpy(TINY, 1001, **STRESS)
    prompt = synth.prompts(TINY, 2000, 1)[0]
    joint = _exact_joint2(TINY, w, prompt)
    n, seeds = 16384, (3000, 3001, 3002, 3003)
    obs, same = [], 0
    for seed in seeds:
        log(f"lossless: {n} sequences, seed {seed}")
        eng = _shared_prompt_engine(w, prompt, n, seed)
        out, n_out = eng.step(list(range(n)))
        g = host(out)
        eng.sync()
        eng.close()
        obs.append(g[:, :2])
        # the oracle's iteration on the same keys
        one = psispec.Decoder(TINY, w, [0], seed, len(prompt) + TINY.block_size + 2)
        one.prefill([prompt])
        for a in range(0, n, 8192):
            b = min(n, a + 8192)
            dec = psispec.Decoder(TINY, w, np.arange(a, b), seed, len(prompt) + TINY.block_size + 2)
            dec.cache["k"][:] = one.cache["k"]
            dec.cache["v"][:] = one.cache["v"]
            dec.n[:], dec.t[:] = one.n[0], one.t[0]
            r = dec.step()
            same += int(np.sum(np.all(r["out"] == g[a:b], axis=1)))
    obs = np.concatenate(obs)
    pval = _chi2_pvalue(obs, joint)
    frac = same / (n * len(seeds))
    log(f"lossless: chi^2 p = {pval:.3f} over {len(obs)} sequences; identical to the oracle: "
        f"{100 * frac:.3f}%")
    assert pval > 0.01
    # near-ties of float32 decisions may differ in a handful of sequences
    assert frac >= 0.999


def test_release_and_prefill_again_while_snapshot_in_flight():
    w = synth.weights_numpy(TINY, 1001, **STRESS)
    seed, S = 3100, 4
    max_len = TINY.max_len + 40
    eng = engine(TINY, w, max_seqs=S, max_seq_len=max_len, seed=seed)
    prompts = [synth.prompts(TINY, 2100 + i, 1, 16)[0] for i in range(S)]
    ids = list(range(S))
    eng.prefill(ids, prompts)
    decs = {}
    for s in ids:
        decs[s] = psispec.Decoder(TINY, w, [s], seed, max_len)
        decs[s].prefill([prompts[s]])
    for it in range(6):
        out, n_out = eng.step(ids)
        # the snapshot of this verify is enqueued; replace sequence 1 right away with
        # a prompt whose length puts the next block across a page boundary
        if it % 2 == 0:
            new = synth.prompts(TINY, 2200 + it, 1, 13)[0]
            eng.release(1)
            eng.prefill([1], [new])
        g_out, g_n = host(out), host(n_out)
        for i, s in enumerate(ids):
            r = decs[s].step()
            assert int(g_n[i]) == int(r["n_out"][0]), (it, s)
            assert np.array_equal(g_out[i], r["out"][0]), (it, s)
        if it % 2 == 0:
            decs[1] = psispec.Decoder(TINY, w, [1], seed, max_len)
            decs[1].prefill([new])
    eng.sync()      # raises on a tripped bounds check
    for s in ids:
        assert eng.seq_state(s)[0] == int(decs[s].n[0])
