"""uno_accept_noalloc (accept / resample with its working memory in a static device
array, for callers that cannot allocate) against uno_accept on a context, through
the C ABI: the same accept lengths and emitted tokens bit for bit, on two calls in
a row, the second with fewer sequences and a smaller vocabulary."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

SEED = 4321


def _inputs(n, B, V, seed):
    """p / q rows close enough to accept some slots and reject others."""
    r = np.random.default_rng(seed)
    p = synth.prob_rows(seed, (n, B, V), zero_frac=0.3)
    q = synth.prob_rows(seed + 1, (n, B - 1, V), zero_frac=0.3)
    mix = r.random((n, B - 1, 1)) < 0.6
    q = np.where(mix, p[:, : B - 1], q).astype(np.float32)     # identical laws always accept
    cdf = np.cumsum(p[:, 0].astype(np.float64), axis=-1)
    y = np.stack([np.minimum(np.searchsorted(cdf[i], r.random(B) * cdf[i, -1], side="right"),
                             V - 1) for i in range(n)]).astype(np.int32)
    seq = r.permutation(4 * n)[:n].astype(np.int32)
    pos = r.integers(0, 9000, n).astype(np.int32)
    it = r.integers(0, 500, n).astype(np.int32)
    return p, q, y, seq, pos, it


def _reference(V, B, n, args):
    cfg = configs.TINY.with_(vocab=V, n_layers=1, block_size=B)
    w = synth.weights_numpy(cfg, 1, with_embed=False)
    eng = engine(cfg, w, max_seqs=n, max_rows=n * B, seed=SEED)
    out, n_out = eng.accept(*args)
    o, k = host(out), host(n_out)
    eng.sync()
    eng.close()
    return o, k


@pytest.mark.parametrize("first,second", [((64, 16, 151936), (5, 16, 2080))])
def test_noalloc_matches_context_accept(first, second):
    import torch
    for n, B, V in (first, second):
        log(f"accept_noalloc n={n} B={B} V={V}")
        p, q, y, seq, pos, it = _inputs(n, B, V, 100 + n)
        args = [dev(p), dev(q), dev(y), dev(seq), dev(pos), dev(it)]
        out = torch.full((n, B + 1), -7, dtype=torch.int32, device="cuda")
        n_out = torch.zeros((n,), dtype=torch.int32, device="cuda")
        err = torch.zeros((1,), dtype=torch.int32, device="cuda")
        uno.accept_noalloc(SEED, *args, out, n_out, err)
        got_o, got_k = host(out), host(n_out)
        ref_o, ref_k = _reference(V, B, n, args)
        log(f"  accept lengths {np.bincount(got_k, minlength=B + 2)[2:].tolist()}")
        assert np.array_equal(got_k, ref_k)
        assert np.array_equal(got_o, ref_o)
        assert int(host(err)[0]) == 0
        assert len(set(got_k.tolist())) >= 2
