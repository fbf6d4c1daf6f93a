"""The full-size 36-layer Qwen3-8B-shaped model (bf16, LoRA r 128, vocabulary
151936) in two launch configurations the throughput measurement uses: the
distillation forward over one sequence of L = 2048 clean tokens plus 2048 MASK
rows (per sequence), and one batch-1 decode forward of 16 draft rows at a
1024-token context.

* Sampled outputs against the oracle: the first 8 teacher rows (an AR forward of
  x[0..7]) and the first 8 student rows of block 0 (no clean context: 8 MASK rows
  with the adapter on), the oracle run layer by layer over weights copied from
  the device.  Tolerance as in the one-layer test: the bf16 oracle's own distance
  to the unrounded result sets the bound.
* Decode: all 16 rows' 151936 logits against the oracle run layer by layer over
  the same weights and the imported context (the skinny kernels at 16 rows and
  the two-tile LM head with its logits epilogue), same tolerance.
* Properties that hold exactly at any size (bitwise, since every row's arithmetic
  is independent of the other rows): teacher rows do not depend on B; student
  rows never see x[L-1]; with B = L the student rows do not depend on x at all;
  changing x[L-1] changes only the last teacher row; 0 <= TV <= 1 and the block
  TV is the mean of its rows."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import configs, synth, uno
from oracle import distill, model
from tests.gpu_util import host, log, require_gpu

pytestmark = pytest.mark.gpu

CFG = configs.MODEL8B
L = 2048
NS = 8          # sampled rows per side


@pytest.fixture(scope="module")
def full():
    torch = require_gpu()
    dev = torch.device("cuda", 0)
    log("c4 full: generating 36-layer weights on the device")
    w = synth.weights_torch(CFG, 1010, dev)
    eng = uno.Engine(CFG, w, max_seqs=1, max_seq_len=2 * L + 16, max_rows=2 * L, device=dev)
    x = torch.from_numpy(synth.prompts(CFG, 7400, 1, L)).to(dev)
    yield torch, w, eng, x
    eng.close()


def _f64(t):
    import torch
    return t.to(torch.float64).cpu().numpy()


def _oracle_first_rows(w, x0):
    """Logits of teacher rows 0..NS-1 and student rows 0..NS-1 (block 0), bf16
    oracle and unrounded oracle, streaming one layer's weights at a time."""
    one = CFG.with_(n_layers=1)
    one_exact = one.with_(dtype="f32")
    toks = np.stack([x0[:NS], np.full(NS, CFG.mask_id)])
    pos = np.tile(np.arange(NS), (2, 1))
    gate = np.stack([np.zeros(NS), np.ones(NS)])
    E = w["embed"]
    import torch
    rows = E[torch.as_tensor(toks.ravel(), device=E.device).long()]
    h = {"bf16": _f64(rows).reshape(2, NS, -1)}
    h["exact"] = h["bf16"].copy()
    fn = _f64(w["final_norm"])
    for l, lw in enumerate(w["layers"]):
        lw64 = {"attn_norm": _f64(lw["attn_norm"]), "mlp_norm": _f64(lw["mlp_norm"]),
                "w": {p: _f64(t) for p, t in lw["w"].items()},
                "la": {p: _f64(t) for p, t in lw["la"].items()},
                "lb": {p: _f64(t) for p, t in lw["lb"].items()}}
        wl = {"final_norm": fn, "layers": [lw64]}
        for key, cfg in (("bf16", one), ("exact", one_exact)):
            cache = model.new_cache(cfg, 2, NS)
            _, h[key] = model.forward(cfg, wl, None, pos, gate, cache, hidden_in=h[key],
                                      want_logits=False)
        if l % 6 == 5:
            log(f"  oracle layer {l + 1}/{CFG.n_layers}")
    head = {"final_norm": fn, "lm_head": _f64(w["lm_head"])}
    return (model.lm_logits(one, head, h["bf16"]), model.lm_logits(one_exact, head, h["exact"]))


def test_c4_full_size_sampled_rows_match_oracle(full):
    torch, w, eng, x = full
    log("c4 full: GPU forward B=16")
    T, S, tv, tvb = eng.distill_forward(x, 16)
    eng.sync()
    got = np.stack([host(T[0, :NS]), host(S[0, :NS])])
    tv_g = host(tv[0, :NS])
    log("c4 full: oracle rows")
    ref, ex = _oracle_first_rows(w, x[0].cpu().numpy())
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    err = np.abs(got[fin] - ref[fin])
    noise = np.abs(ref[fin] - ex[fin])
    gex = np.abs(got[fin] - ex[fin])
    tol = max(3e-2, 2.0 * float(noise.max()))
    log(f"  logits: max |gpu-oracle| {err.max():.3e} (bound {tol:.3e}); mean {err.mean():.2e}, "
        f"|gpu-exact| {gex.mean():.2e}, |oracle-exact| {noise.mean():.2e}")
    assert err.max() <= tol
    assert err.mean() <= 1.5 * noise.mean()
    assert gex.mean() <= 1.25 * noise.mean()
    p = lambda a: model.probs(a).astype(np.float64)
    tv_o = distill.tv_rows(p(ref[0]), p(ref[1]))
    bound = distill.tv_rows(p(got[0]), p(ref[0])) + distill.tv_rows(p(got[1]), p(ref[1])) + 1e-5
    log(f"  tv rows: max |gpu-oracle| {np.abs(tv_g - tv_o).max():.2e}, bound {bound.min():.2e}"
        f"..{bound.max():.2e}")
    assert np.all(np.abs(tv_g - tv_o) <= bound)


def test_c4_full_size_exact_properties(full):
    torch, w, eng, x = full
    log("c4 full: properties")
    T16, S16, tv16, tvb16 = eng.distill_forward(x, 16)
    T4, S4, _, _ = eng.distill_forward(x, 4)
    eng.sync()
    assert torch.equal(T16, T4), "teacher rows depend on B"
    assert not torch.equal(S16, S4)
    del T4, S4
    # x[L-1] is visible to the last teacher row only
    x2 = x.clone()
    x2[0, L - 1] = (x2[0, L - 1] + 1) % (CFG.vocab - 1)
    T2, S2, _, _ = eng.distill_forward(x2, 16)
    eng.sync()
    assert torch.equal(S16, S2)
    assert torch.equal(T16[:, : L - 1], T2[:, : L - 1])
    assert not torch.equal(T16[:, L - 1], T2[:, L - 1])
    del T2, S2
    # B = L: the student sees no clean token
    x3 = torch.from_numpy(synth.prompts(CFG, 7401, 1, L)).to(x.device)
    _, SL, _, _ = eng.distill_forward(x, L)
    _, SL3, _, _ = eng.distill_forward(x3, L)
    eng.sync()
    assert torch.equal(SL, SL3)
    del SL, SL3
    tvr, tvb = host(tv16)[0], host(tvb16)[0]
    assert np.all(np.isfinite(tvr)) and tvr.min() >= 0.0 and tvr.max() <= 1.0
    assert np.abs(tvb - tvr.astype(np.float64).reshape(-1, 16).mean(-1)).max() <= 1e-6


def test_decode_full_size_logits_match_oracle(full):
    torch, w, _, _ = full
    dev = torch.device("cuda", 0)
    ctx, rows = 1024, 16
    log("decode full: importing a 1024-token context into all 36 layers")
    eng = uno.Engine(CFG, w, max_seqs=1, max_seq_len=ctx + 64, max_rows=rows, device=dev)
    gen = torch.Generator(device=dev).manual_seed(7501)
    shape = (CFG.n_layers, ctx, CFG.n_kv_heads, CFG.head_dim)
    k = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    eng.kv_import(0, k, v, pending=0)
    toks = np.full(rows, CFG.mask_id, dtype=np.int32)
    toks[0] = 1234                       # the pending token, then MASK rows
    pos = np.arange(ctx, ctx + rows, dtype=np.int32)
    gate = np.ones(rows, dtype=np.uint8)
    gate[0] = 0                          # slot 0 is AR-only
    t = lambda a: torch.from_numpy(a).to(dev)
    log("decode full: GPU forward")
    _, lg = eng.forward([0], rows, t(pos), t(gate), tokens=t(toks), want_logits=True)
    got = host(lg)
    eng.close()
    kh, vh = _f64(k), _f64(v)
    del k, v
    log("decode full: oracle")
    one = CFG.with_(n_layers=1)
    one_exact = one.with_(dtype="f32")
    E = w["embed"]
    h0 = _f64(E[torch.as_tensor(toks, device=E.device).long()])[None]
    h = {"bf16": h0, "exact": h0.copy()}
    fn = _f64(w["final_norm"])
    for l, lw in enumerate(w["layers"]):
        lw64 = {"attn_norm": _f64(lw["attn_norm"]), "mlp_norm": _f64(lw["mlp_norm"]),
                "w": {p: _f64(q) for p, q in lw["w"].items()},
                "la": {p: _f64(q) for p, q in lw["la"].items()},
                "lb": {p: _f64(q) for p, q in lw["lb"].items()}}
        wl = {"final_norm": fn, "layers": [lw64]}
        for key, cfg in (("bf16", one), ("exact", one_exact)):
            cache = model.new_cache(cfg, 1, ctx + rows)
            cache["k"][0, 0, :ctx] = kh[l]
            cache["v"][0, 0, :ctx] = vh[l]
            _, h[key] = model.forward(cfg, wl, None, pos[None], gate[None], cache, hidden_in=h[key],
                                      want_logits=False)
        if l % 6 == 5:
            log(f"  oracle layer {l + 1}/{CFG.n_layers}")
    head = {"final_norm": fn, "lm_head": _f64(w["lm_head"])}
    ref = model.lm_logits(one, head, h["bf16"])[0]
    ex = model.lm_logits(one_exact, head, h["exact"])[0]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    err = np.abs(got[fin] - ref[fin])
    noise = np.abs(ref[fin] - ex[fin])
    gex = np.abs(got[fin] - ex[fin])
    tol = max(3e-2, 2.0 * float(noise.max()))
    log(f"  logits: max |gpu-oracle| {err.max():.3e} (bound {tol:.3e}); mean {err.mean():.2e}, "
        f"|gpu-exact| {gex.mean():.2e}, |oracle-exact| {noise.mean():.2e}")
    assert err.max() <= tol
    assert err.mean() <= 1.5 * noise.mean()
    assert gex.mean() <= 1.25 * noise.mean()
