"""GPU parity on one Qwen3-8B-shaped layer in bf16 (d 4096, 32 q / 8 kv heads of
128, SwiGLU 12288, LoRA r 128 alpha 256 on all seven projections): a 1024-token
KV context, one 16-slot draft forward (slot 0 gate off, the rest on) and one
16-row AR verify forward.  Layer outputs (the residual stream) are compared with
the bf16-storage oracle; the written K/V within one bf16 ulp (plus the absolute
shift of a single upstream rounding flip).

Tolerance (derived from the arithmetic): two bf16-storage evaluations of the same
layer differ by rounding-boundary flips, so they cannot agree more closely than
either agrees with the exact result.  The bound is therefore
max(3e-2, 2 * max |oracle_bf16 - oracle_exact|), where oracle_exact is the same
oracle without storage rounding (measured per case: 3-5e-2 on these N(0,1) rows
whose outputs reach magnitude ~5, i.e. about one bf16 ulp).  A mistake hidden in
that noise is caught by the means: the GPU must sit closer to the bf16 oracle
than the bf16 oracle sits to the exact result, and its own distance to the exact
result must look like bf16 storage noise (within 1.25x of the oracle's)."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth
from oracle import model
from tests.gpu_util import dev, engine, host, log

pytestmark = pytest.mark.gpu

CFG = configs.LAYER8B
TOL = 3e-2
CTX = 1024


@pytest.fixture(scope="module")
def setup():
    import torch
    log("layer8b: generating weights")
    w = synth.weights_numpy(CFG, 1001, with_embed=False)
    kc = synth.normal(5001, (1, CTX, CFG.n_kv_heads, CFG.head_dim))
    vc = synth.normal(5002, (1, CTX, CFG.n_kv_heads, CFG.head_dim))
    kc = torch.from_numpy(kc).to(torch.bfloat16).float().numpy()
    vc = torch.from_numpy(vc).to(torch.bfloat16).float().numpy()
    eng = engine(CFG, w, max_seqs=1, max_seq_len=CTX + 64, max_rows=16)
    eng.kv_import(0, dev(kc, torch.bfloat16), dev(vc, torch.bfloat16), pending=0)
    cache = model.new_cache(CFG, 1, CTX + 64)
    cache["k"][0, 0, :CTX] = kc[0]
    cache["v"][0, 0, :CTX] = vc[0]
    return w, eng, cache


def _run(setup, pos, gate, seed):
    w, eng, cache = setup
    x = synth.normal(seed, (16, CFG.d_model))
    hid, _ = eng.forward([0], 16, dev(pos), dev(gate), hidden_in=dev(x), want_hidden=True)
    exact_cache = {"k": cache["k"].copy(), "v": cache["v"].copy()}
    _, ref = model.forward(CFG, w, None, pos[None], gate[None], cache, hidden_in=x[None],
                           want_logits=False)
    _, ex = model.forward(CFG.with_(dtype="f32"), w, None, pos[None], gate[None], exact_cache,
                          hidden_in=x[None], want_logits=False)
    return host(hid), ref[0], x, ex[0]


def _check(g, ref, ex, what):
    err = np.abs(g - ref)
    noise = np.abs(ref - ex)
    tol = max(TOL, 2.0 * float(noise.max()))
    gex = np.abs(g - ex).mean()
    log(f"{what}: max |gpu-oracle| {err.max():.3e} (bound {tol:.3e}); mean |gpu-oracle| "
        f"{err.mean():.2e}, |gpu-exact| {gex:.2e}, |oracle-exact| {noise.mean():.2e}")
    assert err.max() <= tol
    assert err.mean() <= noise.mean()
    assert gex <= 1.25 * noise.mean()


def test_draft_then_verify_layer_outputs(setup):
    w, eng, cache = setup
    log("layer8b: draft rows")
    pos = np.arange(CTX, CTX + 16, dtype=np.int32)
    gate = np.ones(16, dtype=np.uint8)
    gate[0] = 0
    g, ref, x, ex = _run(setup, pos, gate, 6001)
    _check(g, ref, ex, "draft")
    # the adapter is really applied on gated rows: compare against a gate-0 oracle row
    _, ref0 = model.forward(CFG, w, None, pos[None], np.zeros((1, 16)),
                            {"k": cache["k"].copy(), "v": cache["v"].copy()},
                            hidden_in=x[None], want_logits=False)
    assert np.abs(ref0[0, 1:] - ref[1:]).max() > 10 * TOL
    assert np.abs(ref0[0, 0] - ref[0]).max() == 0.0       # slot 0 is AR-only
    log("layer8b: verify rows")
    pos_v = np.arange(CTX + 1, CTX + 17, dtype=np.int32)
    g2, ref2, _, ex2 = _run(setup, pos_v, np.zeros(16, dtype=np.uint8), 6002)
    _check(g2, ref2, ex2, "verify")
    # K/V written by the verify rows at CTX+1..CTX+16 (and the kept draft row at CTX)
    k, v = eng.kv_export(0, CTX + 17)
    k, v = host(k.float()), host(v.float())
    assert np.array_equal(k[:, :CTX], cache["k"][:, 0, :CTX])
    # one bf16 ulp, plus the absolute shift a single upstream rounding flip (e.g. of
    # one LoRA-intermediate element, ~1 ulp * |B| ~ 3e-4) leaves before rounding
    for got, want in ((k, cache["k"]), (v, cache["v"])):
        o = want[:, 0, CTX:CTX + 17]
        d = np.abs(got[:, CTX:CTX + 17] - o)
        assert np.all(d <= 2.0 ** -7 * np.abs(o) + 2e-3)
        assert np.mean(d > 0) <= 0.1
    eng.sync()


def test_repeat_is_bit_identical(setup):
    """Deterministic reductions: the same forward twice gives identical bits."""
    w, eng, cache = setup
    pos = np.arange(CTX + 1, CTX + 17, dtype=np.int32)
    gate = (np.arange(16) % 3 == 0).astype(np.uint8)
    x = synth.normal(6003, (16, CFG.d_model))
    a, _ = eng.forward([0], 16, dev(pos), dev(gate), hidden_in=dev(x), want_hidden=True)
    b, _ = eng.forward([0], 16, dev(pos), dev(gate), hidden_in=dev(x), want_hidden=True)
    assert np.array_equal(host(a), host(b))


def test_large_m_rows_two_sequences():
    """96 rows (the large-M kernel, with a ragged 128-row tile): two sequences of
    48 rows each against their own contexts, gates mixed, LoRA on."""
    import torch
    log("layer8b: large-M rows")
    w = synth.weights_numpy(CFG, 1001, with_embed=False)
    eng = engine(CFG, w, max_seqs=2, max_seq_len=CTX + 128, max_rows=96)
    cache = model.new_cache(CFG, 2, CTX + 128)
    ctxs = [CTX, CTX - 300]
    for s in range(2):
        kc = torch.from_numpy(synth.normal(7001 + s, (1, ctxs[s], CFG.n_kv_heads, CFG.head_dim)))
        vc = torch.from_numpy(synth.normal(7101 + s, (1, ctxs[s], CFG.n_kv_heads, CFG.head_dim)))
        kc, vc = kc.to(torch.bfloat16), vc.to(torch.bfloat16)
        eng.kv_import(s, dev(kc.float().numpy(), torch.bfloat16), dev(vc.float().numpy(), torch.bfloat16),
                      pending=0)
        cache["k"][0, s, :ctxs[s]] = kc.float().numpy()[0]
        cache["v"][0, s, :ctxs[s]] = vc.float().numpy()[0]
    rows = 48
    pos = np.stack([np.arange(c, c + rows) for c in ctxs]).astype(np.int32)
    gate = (np.arange(2 * rows).reshape(2, rows) % 3 != 0).astype(np.uint8)
    x = synth.normal(7201, (2, rows, CFG.d_model))
    hid, _ = eng.forward([0, 1], rows, dev(pos.ravel()), dev(gate.ravel()),
                         hidden_in=dev(x.reshape(-1, CFG.d_model)), want_hidden=True)
    ex_cache = {"k": cache["k"].copy(), "v": cache["v"].copy()}
    _, ref = model.forward(CFG, w, None, pos, gate, cache, hidden_in=x, want_logits=False)
    _, ex = model.forward(CFG.with_(dtype="f32"), w, None, pos, gate, ex_cache, hidden_in=x,
                          want_logits=False)
    _check(host(hid).reshape(2, rows, -1), ref, ex, "large-M")
    for s in range(2):
        k, v = eng.kv_export(s, ctxs[s] + rows)
        k = host(k.float())[:, ctxs[s]:]
        o = cache["k"][:, s, ctxs[s]:ctxs[s] + rows]
        assert np.all(np.abs(k - o) <= 2.0 ** -7 * np.abs(o) + 2e-3)
    eng.sync()


@pytest.mark.parametrize("n", [128, 125, 64])
def test_batch128_rows_sampled_sequences(n):
    """2048 rows, the batch-128 decode launch configuration: 128 sequences of 16
    rows against their own contexts (1024 down to 1024 - 7 * 127 keys), gates as
    in a draft (slot 0 off).  At this height q|k|v runs 256 x 256 tiles, o and
    down split K in two over 256 x 256 tiles (then the slice-sum residual pass),
    gate/up paired 256 x 256, and the LoRA down-projections the sliced large-M
    path.  125 sequences (2000 rows) take the same paths with a ragged last
    256-row tile; 64 sequences (1024 rows, the height of a prefill chunk) split
    o and down into four K slices.  A row's arithmetic does not depend on the other sequences'
    rows, so the oracle runs on sampled sequences only."""
    import torch
    log(f"layer8b: {n} sequences x 16 rows")
    w = synth.weights_numpy(CFG, 1001, with_embed=False)
    rows = 16
    eng = engine(CFG, w, max_seqs=n, max_seq_len=CTX + 64, max_rows=n * rows)
    ctxs = [CTX - 7 * s for s in range(n)]
    sample = (0, 45, n - 1)
    gen = torch.Generator(device="cuda").manual_seed(7301)
    kept = {}
    for s in range(n):
        shape = (1, ctxs[s], CFG.n_kv_heads, CFG.head_dim)
        kc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        vc = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        eng.kv_import(s, kc, vc, pending=0)
        if s in sample:
            kept[s] = (host(kc.float())[0], host(vc.float())[0])
    pos = np.stack([np.arange(c, c + rows) for c in ctxs]).astype(np.int32)
    gate = (np.arange(n * rows).reshape(n, rows) % rows != 0).astype(np.uint8)
    x = synth.normal(7401, (n, rows, CFG.d_model))
    hid, _ = eng.forward(list(range(n)), rows, dev(pos.ravel()), dev(gate.ravel()),
                         hidden_in=dev(x.reshape(-1, CFG.d_model)), want_hidden=True)
    got = host(hid).reshape(n, rows, -1)
    idx = list(sample)
    cache = model.new_cache(CFG, len(idx), CTX + rows)
    for i, s in enumerate(idx):
        cache["k"][0, i, :ctxs[s]] = kept[s][0]
        cache["v"][0, i, :ctxs[s]] = kept[s][1]
    ex_cache = {"k": cache["k"].copy(), "v": cache["v"].copy()}
    _, ref = model.forward(CFG, w, None, pos[idx], gate[idx], cache, hidden_in=x[idx],
                           want_logits=False)
    _, ex = model.forward(CFG.with_(dtype="f32"), w, None, pos[idx], gate[idx], ex_cache,
                          hidden_in=x[idx], want_logits=False)
    _check(got[idx], ref, ex, f"{n} x 16 rows")
    eng.sync()
