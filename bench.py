#!/usr/bin/env python3
"""Throughput of the Psi-Spec draft-and-verify decode step on one MI355X.

Workload (default): a Qwen3-8B-shaped decoder (36 layers, d 4096, 32 q / 8 kv
heads of 128, SwiGLU 12288, vocab 151936) in bf16 with a gated rank-128 LoRA
(alpha 256) on all seven projections of every layer, random N(0, 0.02) weights
generated on the GPU; batch 1, a 1024-token uniform prompt, block B = 16, the
linear sampler with Philox keys, 16-token KV pages.  A step is one whole
iteration: the draft forward, the draft draws, the verify forward, the accept /
resample test and the commit.  W untimed steps, then exactly K timed steps.

Reported: accepted tokens/s (value), positions/s, tokens per forward, whole-step
algorithmic HBM GB/s, the roofline of the dominant kernel (the gate/up
gated-LoRA linear, timed with HIP events on the library's stream), a per-class
kernel time breakdown, batch-1 and batch-128 windows at contexts 1024, 5120 and 9216
with their integrals over the 1K-in / 8K-out run, the HBM floor of each batch-1
linear launch shape (a read-only stream of its weight bytes), the nucleus (top-p) truncation
kernel at the batch-1 and batch-128 row counts, and the CPU oracle timed on a
bounded sample on the host (with its thread counts and a one-thread figure).
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "accepted tokens/s/GPU (Ψ-Spec linear, 8B-shape) at bs=1 & bs=128; HBM GB/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


ROOFLINE_EVERY = 7
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemm_bf16_gateup_bs1_8b.txt")
KERNEL_SOURCES = ("diffusion_drafted_lora_amd/csrc/k_linear.hip",
                  "diffusion_drafted_lora_amd/csrc/uno_internal.h")


def kernel_source_hash():
    """sha256 over the sources of the gate/up linear kernel and its launcher."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary is missing or
    was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    m_h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def copy_probe(mib):
    """A plain elementwise kernel of known size (reads and writes mib MiB each,
    three launches) whose FETCH_SIZE / WRITE_SIZE counters scale the kernel's."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def model_bytes(cfg):
    """Algorithmic bytes of one forward that do not depend on the context:
    layer weights (+ LoRA) and the LM head, bf16."""
    d, q, kv, f, V, r = (cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim, cfg.vocab,
                         cfg.lora_rank)
    layer = (q * d + 2 * kv * d + d * q + 2 * f * d + d * f) * 2
    lora = ((d + q) * r + 2 * (d + kv) * r + (q + d) * r + 2 * (d + f) * r + (f + d) * r) * 2
    return cfg.n_layers * layer + V * d * 2, cfg.n_layers * lora


def kv_bytes_per_pos(cfg):
    return cfg.n_layers * 2 * cfg.kv_dim * 2


def run_batch(cfg, w, dev, batch, ctx, steps, warmup, prompt_len, log_prefix="bs128"):
    """Large-batch leg: `batch` sequences at context `ctx` (prefilled from uniform
    prompts when ctx <= prompt_len, else filled with seeded synthetic K/V), then
    `warmup` + `steps` timed iterations.  Returns a dict of measurements."""
    import numpy as np
    import torch
    from diffusion_drafted_lora_amd import synth, uno

    B = cfg.block_size
    max_len = ctx + (warmup + steps + 6) * (B + 1) + B + 2
    eng = uno.Engine(cfg, w, max_seqs=batch, max_seq_len=max_len, max_rows=batch * B,
                     seed=3003, device=dev)
    ids = list(range(batch))
    t0 = time.perf_counter()
    if ctx <= prompt_len:
        prompts = synth.prompts(cfg, 2003, batch, ctx + 1)
        log(f"{log_prefix}: prefill {batch} x {ctx + 1} tokens")
        eng.prefill(ids, list(prompts))
    else:
        log(f"{log_prefix}: importing synthetic K/V of {ctx} positions for {batch} sequences")
        g = torch.Generator(device=dev)
        g.manual_seed(4003)
        shape = (cfg.n_layers, ctx, cfg.n_kv_heads, cfg.head_dim)
        k = torch.empty(shape, dtype=torch.float32, device=dev).normal_(0, 1, generator=g).to(torch.bfloat16)
        v = torch.empty(shape, dtype=torch.float32, device=dev).normal_(0, 1, generator=g).to(torch.bfloat16)
        for sq in ids:
            eng.kv_import(sq, k, v, pending=sq % (cfg.vocab - 1))
        del k, v
    eng.sync()
    t_fill = time.perf_counter() - t0
    outs = torch.empty((batch, B + 1), dtype=torch.int32, device=dev)
    nouts = torch.empty((warmup, batch), dtype=torch.int32, device=dev)
    for i in range(warmup):
        eng.step(ids, out=outs, n_out=nouts[i])
    eng.sync()
    cls = ["linear", "linear_swiglu", "lora_down", "lm_head", "attention"]
    # Few sequences: hundreds of short kernels per iteration, whose event pairs would
    # lengthen the timed iterations, so the class breakdown comes from a few extra
    # iterations after them.  Large batch: kernels are long, the same iterations serve.
    separate = batch < 8
    extra = min(4, steps) if separate else 0
    nouts = torch.empty((warmup + steps + extra, batch), dtype=torch.int32, device=dev)
    if not separate:
        eng.timing(cls)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        eng.step(ids, out=outs, n_out=nouts[i])
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    eng.sync()
    tok = int(nouts[warmup:warmup + steps].sum().item())
    if separate:
        eng.timing(cls)
        for i in range(warmup + steps, warmup + steps + extra):
            eng.step(ids, out=outs, n_out=nouts[i])
        eng.sync()
    nb = extra if separate else steps
    gemm_ms = gemm_fl = 0.0
    breakdown = {}
    for c in cls:
        n, ms, b, f = eng.timing_read(c)
        breakdown[c] = {"ms_per_step": ms / nb, "TFLOP/s": f / 1e12 / (ms / 1e3) if ms else None,
                        "GB/s": b / 1e9 / (ms / 1e3) if ms else None}
        if c != "attention":
            gemm_ms += ms
            gemm_fl += f
    eng.timing([])
    eng.close()
    del eng
    torch.cuda.empty_cache()
    mfma_tflops = gemm_fl / 1e12 / (gemm_ms / 1e3)
    # algorithmic HBM bytes of the timed iterations: both forwards' weights, the
    # draft's LoRA, and every sequence's context K/V read by both forwards
    fixed, lora = model_bytes(cfg)
    ctx_mid = ctx + (warmup + steps / 2.0) * tok / max(1, batch * steps)
    it_bytes = 2 * fixed + lora + batch * kv_bytes_per_pos(cfg) * (2 * ctx_mid + 2 * B)
    hbm = it_bytes / 1e9 / (sec / steps)
    return {
        "batch": batch, "context_start": ctx, "steps": steps, "warmup": warmup,
        "accepted_tokens_per_s": tok / sec, "positions_per_s": 2 * B * batch * steps / sec,
        "ms_per_step": 1e3 * sec / steps, "tokens_per_forward": tok / (2.0 * batch * steps),
        "gemm_mfma_tflops": mfma_tflops, "gemm_mfma_frac": mfma_tflops / BF16_PEAK_TFLOPS,
        "hbm_gbs_algorithmic": hbm, "hbm_frac": hbm / HBM_PEAK_GBS,
        "fill_s": t_fill, "breakdown": breakdown,
    }


def run_tree(cfg, w, dev, chains, steps, warmup, prompt_len):
    """Batch-1 tree sampler (uno_tree_step) on the headline's prompt and seed, for
    each chain count K: accepted tokens/s, tokens per forward and the step time
    (its verify forward carries 1 + K (B - 1) rows)."""
    import torch
    from diffusion_drafted_lora_amd import synth, uno

    B = cfg.block_size
    res = []
    for K in chains:
        Rv = 1 + K * (B - 1)
        max_len = prompt_len + (warmup + steps + 2) * (B + 1) + 2 + K * (B - 1) + B
        eng = uno.Engine(cfg, w, max_seqs=1, max_seq_len=max_len, max_rows=max(256, Rv),
                         seed=3002, device=dev, tree_chains=K)
        prompt = synth.prompts(cfg, 2002, 1, prompt_len)[0]
        log(f"tree K={K}: prefill {prompt_len} tokens")
        eng.prefill([0], [prompt])
        outs = torch.empty((1, B + 1), dtype=torch.int32, device=dev)
        nouts = torch.empty((warmup + steps,), dtype=torch.int32, device=dev)
        for i in range(warmup):
            eng.tree_step([0], K, out=outs, n_out=nouts[i:i + 1])
        eng.sync()
        ctx0 = eng.seq_state(0)[0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warmup, warmup + steps):
            eng.tree_step([0], K, out=outs, n_out=nouts[i:i + 1])
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        eng.sync()
        tok = int(nouts[warmup:].sum().item())
        res.append({"chains": K, "verify_rows": Rv, "steps": steps, "warmup": warmup,
                    "context_start": int(ctx0), "accepted_tokens_per_s": tok / sec,
                    "tokens_per_forward": tok / (2.0 * steps), "ms_per_step": 1e3 * sec / steps})
        eng.close()
        del eng
        torch.cuda.empty_cache()
    return res


def run_qk_norm(cfg, w, dev, steps, warmup, prompt_len):
    """Batch-1 decode of the same model with the per-head QK RMSNorm off and on
    (unit gains added to the same weights), on the headline's prompt and seed: step
    time, accepted tokens/s, and the time of the norm kernels (the difference of
    the misc class, where they are timed, between the two runs)."""
    import torch
    from diffusion_drafted_lora_amd import synth, uno

    B = cfg.block_size
    res = {}
    for on in (False, True):
        c = cfg.with_(qk_norm=on)
        wq = w
        if on:
            ones = torch.ones(cfg.head_dim, dtype=torch.bfloat16, device=dev)
            wq = dict(w)
            wq["layers"] = [dict(lw, q_norm=ones, k_norm=ones) for lw in w["layers"]]
        max_len = prompt_len + (warmup + steps + 8) * (B + 1) + B + 2
        eng = uno.Engine(c, wq, max_seqs=1, max_seq_len=max_len, max_rows=256, seed=3002,
                         device=dev)
        prompt = synth.prompts(cfg, 2002, 1, prompt_len)[0]
        log(f"qk-norm {'on' if on else 'off'}: prefill {prompt_len} tokens")
        eng.prefill([0], [prompt])
        outs = torch.empty((1, B + 1), dtype=torch.int32, device=dev)
        nouts = torch.empty((warmup + steps,), dtype=torch.int32, device=dev)
        for i in range(warmup):
            eng.step([0], out=outs, n_out=nouts[i:i + 1])
        eng.sync()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warmup, warmup + steps):
            eng.step([0], out=outs, n_out=nouts[i:i + 1])
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        eng.sync()
        tok = int(nouts[warmup:].sum().item())
        eng.timing(["misc"])
        for i in range(4):
            eng.step([0])
        eng.sync()
        n_m, ms_m, _, _ = eng.timing_read("misc")
        eng.timing([])
        res["on" if on else "off"] = {"ms_per_step": 1e3 * sec / steps,
                                      "accepted_tokens_per_s": tok / sec,
                                      "tokens_per_forward": tok / (2.0 * steps),
                                      "misc_ms_per_step": ms_m / 4, "misc_launches_per_step": n_m / 4}
        eng.close()
        del eng
        torch.cuda.empty_cache()
    extra = res["on"]["misc_launches_per_step"] - res["off"]["misc_launches_per_step"]
    res["norm_kernel_us_per_launch"] = (
        1e3 * (res["on"]["misc_ms_per_step"] - res["off"]["misc_ms_per_step"]) / extra if extra else None)
    res["norm_launches_per_step"] = extra
    res["steps"] = steps
    return res


def run_bytes_per_iteration(cfg, contexts):
    """Mean algorithmic bytes of a batch-1 iteration over contexts [c0, c_last]: both
    forwards' weights, the draft's LoRA and the K/V of the context read twice (the
    context grows linearly, so its mean is the midpoint)."""
    fixed, lora = model_bytes(cfg)
    mid = (contexts[0] + contexts[-1]) / 2.0
    return 2 * fixed + lora + kv_bytes_per_pos(cfg) * (2 * mid + 2 * cfg.block_size)


def integrate_windows(windows, batch, B):
    """Whole-run figures of a batch leg measured in windows at several contexts: the
    iteration time is taken piecewise linear in the context between the windows
    (trapezoid rule), and every iteration emits batch * 2 * TPF tokens, so the
    run's rate is tokens per iteration over the mean iteration time."""
    if len(windows) < 2:
        return None
    ws = sorted(windows, key=lambda d: d["context_start"])
    span = ws[-1]["context_start"] - ws[0]["context_start"]
    if span <= 0:
        return None
    mean_ms = sum((b["context_start"] - a["context_start"]) * (a["ms_per_step"] + b["ms_per_step"]) / 2
                  for a, b in zip(ws, ws[1:])) / span
    tpf = sum(d["tokens_per_forward"] for d in ws) / len(ws)
    return {"contexts": [d["context_start"] for d in ws], "method": "trapezoid over the windows",
            "mean_ms_per_step": mean_ms, "tokens_per_forward": tpf,
            "accepted_tokens_per_s": batch * 2 * tpf / (mean_ms / 1e3),
            "positions_per_s": batch * 2 * B / (mean_ms / 1e3)}


# Tokens per forward of trained Uno models (shibing624 reading notes of the Uno paper,
# "实验" section: 2.25 before and 2.10 after RL with the adapter frozen, part "RL 加速与
# 漂移问题"; 4.21 for Uno_Qwen on MBPP in the comparison with lossy methods, part
# "战线二").  Random-init weights accept far less, so the measured TPF is much lower.
PAGES_TPF = (2.10, 2.25, 4.21)


def tpf_projection(ms_per_step, batch, tpfs=PAGES_TPF):
    """Accepted tokens/s of a leg at the trained models' tokens per forward, holding its
    measured iteration time: an iteration runs the same two forwards of B rows whatever
    is accepted (acceptance only sets how many positions are committed), so the rate
    scales with TPF.  A projection, not a measurement; over a whole 1K-in / 8K-out run a
    higher TPF also means fewer iterations at the same mean context."""
    if not ms_per_step or ms_per_step <= 0:
        return None
    return {"kind": "projection", "basis": "measured ms per iteration x tokens per forward",
            "ms_per_step": ms_per_step,
            "accepted_tokens_per_s": {f"{t:.2f}": batch * 2 * t / (ms_per_step / 1e3) for t in tpfs}}


def run_distill(cfg, w, dev, batch, L, B, reps):
    """The [x, z1] distillation forward: `batch` sequences of L uniform clean tokens
    with L MASK tokens, block size B; teacher and student logits written to
    [batch, L, vocab] float32 buffers, per-row and per-block TV.  Returns ms per
    forward, MFMA TFLOP/s over the dense work and the per-class breakdown."""
    import torch
    from diffusion_drafted_lora_amd import synth, uno

    rows = max(2 * L, min(batch, 2) * 2 * L)
    eng = uno.Engine(cfg, w, max_seqs=batch, max_seq_len=2 * L + 16, max_rows=rows,
                     seed=3004, device=dev)
    x = torch.from_numpy(synth.prompts(cfg, 2004, batch, L)).to(torch.int32).to(dev)
    V = cfg.vocab
    teacher = torch.empty((batch, L, V), dtype=torch.float32, device=dev)
    student = torch.empty((batch, L, V), dtype=torch.float32, device=dev)
    tv_row = torch.empty((batch, L), dtype=torch.float32, device=dev)
    tv_block = torch.empty((batch, L // B), dtype=torch.float32, device=dev)
    log(f"distill: warmup, batch {batch} x [{L} | {L}], B {B}")
    eng.distill_forward(x, B, teacher, student, tv_row, tv_block)
    eng.sync()
    cls = ["linear", "linear_swiglu", "lora_down", "lm_head", "attention", "sampling"]
    eng.timing(cls)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        eng.distill_forward(x, B, teacher, student, tv_row, tv_block)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    eng.sync()
    breakdown = {}
    for c in cls:
        n, ms, b, f = eng.timing_read(c)
        breakdown[c] = {"ms_per_forward": ms / reps,
                        "TFLOP/s": f / 1e12 / (ms / 1e3) if ms and f else None,
                        "GB/s": b / 1e9 / (ms / 1e3) if ms else None}
    eng.timing([])
    tvb = tv_block.float().mean().item()
    eng.close()
    del eng, teacher, student
    torch.cuda.empty_cache()
    d, q, kv, F, r = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim, cfg.lora_rank
    R = batch * 2 * L
    dense = 2.0 * R * (cfg.n_layers * (q * d + 2 * kv * d + d * q + 3 * F * d) + V * d)
    lora = 2.0 * (R / 2) * cfg.n_layers * r * ((d + q) + 2 * (d + kv) + (q + d) + 2 * (d + F) + (F + d))
    attn = 4.0 * batch * cfg.n_q_heads * cfg.head_dim * L * (L + 1) * cfg.n_layers
    total = dense + lora + attn
    return {"batch": batch, "L": L, "B": B, "reps": reps, "ms_per_forward": 1e3 * sec,
            "tflop_per_forward": total / 1e12, "tflops": total / 1e12 / sec,
            "mfma_frac": total / 1e12 / sec / BF16_PEAK_TFLOPS,
            "rows_per_s": R / sec, "mean_tv_block": tvb, "breakdown": breakdown}


def backward_flops(cfg, batch, L, B):
    """Algorithmic flops of one distillation backward over batch x L z1 rows: the
    gate-on forward recompute and the backward of every projection (base input
    gradient, LoRA up / down and both LoRA gradients), attention over the visible
    (z1 row, key) pairs only -- forward, the score / probability gradients, dq and
    the z1 keys' dk, dv -- and the LM head's input gradient."""
    from diffusion_drafted_lora_amd import synth
    N = batch * L
    r = cfg.lora_rank
    shapes = synth.proj_shapes(cfg)
    base = sum(o * i for o, i in shapes.values())
    lora_fwd = sum(r * i + (o * r if p != "down" else 0) for p, (o, i) in shapes.items())
    lora_bwd = sum(2 * r * i + 2 * o * r for o, i in shapes.values())
    # visible keys of z1 row i: bB x keys and i - bB + 1 own keys
    vis = sum((i // B) * B + (i - (i // B) * B + 1) for i in range(L)) * batch
    own = sum(i - (i // B) * B + 1 for i in range(L)) * batch
    hq, hd = cfg.n_q_heads, cfg.head_dim
    attn = 2.0 * hq * hd * (2 * vis + 2 * vis + 2 * own)
    per_layer = 2.0 * N * (2 * base + lora_fwd + lora_bwd) + attn
    return cfg.n_layers * per_layer + 2.0 * N * cfg.vocab * cfg.d_model


def run_distill_backward(cfg, w, dev, batch, L, B, reps):
    """Backward of the distillation step: a checkpointed [x, z1] forward, then
    uno_distill_backward (the L_TV gradient with respect to every LoRA matrix)
    timed with HIP events on the engine's stream.  Returns ms per backward and the
    algorithmic TFLOP/s against the bf16 matrix peak."""
    import torch
    from diffusion_drafted_lora_amd import synth, uno

    rows = max(2 * L, min(batch, 2) * 2 * L)
    eng = uno.Engine(cfg, w, max_seqs=batch, max_seq_len=2 * L + 16, max_rows=rows,
                     seed=3005, device=dev)
    x = torch.from_numpy(synth.prompts(cfg, 2005, batch, L)).to(torch.int32).to(dev)
    V = cfg.vocab
    teacher = torch.empty((batch, L, V), dtype=torch.float32, device=dev)
    student = torch.empty((batch, L, V), dtype=torch.float32, device=dev)
    ck = eng.set_distill_checkpoint(batch, L)
    log(f"distill backward: checkpointed forward, batch {batch} x [{L} | {L}], B {B}")
    eng.distill_forward(x, B, teacher, student)
    eng.set_distill_checkpoint(None, L)
    log("distill backward: warmup")
    loss, tv, ga, gb = eng.distill_backward(B, teacher, student, ck)
    eng.sync()
    st = eng.stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        eng.distill_backward(B, teacher, student, ck)
    e1.record(st)
    eng.sync()
    ms = e0.elapsed_time(e1) / reps
    gnorm = float(sum(ga[p].double().norm() ** 2 + gb[p].double().norm() ** 2 for p in ga) ** 0.5)
    lval = float(loss.item())
    fl = backward_flops(cfg, batch, L, B)
    eng.close()
    del eng, teacher, student, ck, ga, gb
    torch.cuda.empty_cache()
    log(f"distill backward: {ms:.1f} ms, loss {lval:.4f}")
    return {"batch": batch, "L": L, "B": B, "reps": reps, "ms_per_backward": ms,
            "tflop_per_backward": fl / 1e12, "tflops": fl / 1e9 / ms,
            "mfma_frac": fl / 1e9 / ms / BF16_PEAK_TFLOPS, "loss": lval, "grad_norm": gnorm}


def stream_floor_shapes(cfg):
    """(name, bf16 weight bytes, workgroups, threads, weight loads in flight per thread)
    of the batch-1 verify launches of the few-row linear kernel: one workgroup per 16
    output columns (q|k|v, o, down: one 16-column tile; gate/up: a 16-column gate and
    up pair; LM head: two tiles), waves x 64 threads, tiles x blocks in flight."""
    d, F, V = cfg.d_model, cfg.ffn_dim, cfg.vocab
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    return [("q|k|v", qkv * d * 2, qkv // 16, 8 * 64, 1 * 2),
            ("o", d * cfg.n_q_heads * cfg.head_dim * 2, d // 16, 12 * 64, 1 * 2),
            ("gate/up", 2 * F * d * 2, F // 16, 4 * 64, 2 * 4),
            ("down", d * F * 2, d // 16, 12 * 64, 1 * 2),
            ("lm_head", V * d * 2, V // 32, 4 * 64, 2 * 4)]


def run_stream_floor(cfg, reps):
    """HBM floor of each batch-1 linear launch shape: uno_stream_read over the launch's
    weight bytes with its grid (workgroups x threads, weight loads in flight per
    thread), windows rotating over 2 GiB so that no launch is served from a cache;
    `reps` back-to-back launches per shape timed with events on the current stream."""
    import torch
    from diffusion_drafted_lora_amd import uno
    shapes = stream_floor_shapes(cfg)
    total = 2 << 30
    buf = torch.zeros(total, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(max(s[2] for s in shapes), dtype=torch.int32, device="cuda:0")
    out = {}
    for name, nb, wg, th, ld in shapes:
        nb = nb // 16 * 16
        uno.stream_read(buf, nb, wg, th, ld, sink, reps=2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        uno.stream_read(buf, nb, wg, th, ld, sink, reps=reps)     # one call: no host gaps
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        out[name] = {"MB": nb / 1e6, "workgroups": wg, "threads": th, "loads_in_flight": ld,
                     "us_per_launch": us, "GB/s": nb / 1e3 / us}
    del buf, sink
    torch.cuda.empty_cache()
    return out


def run_top_p(V, rows_list, top_p=0.95, reps=20):
    """Nucleus truncation (uno_top_p) on float32 probability rows of the model's
    vocabulary: softmax rows of N(0, 3^2) logits, out of place.  Timed with HIP
    events on the stream the kernel runs on; algorithmic bytes are one read and one
    write of every row (8 V bytes per row)."""
    import torch
    from diffusion_drafted_lora_amd import uno
    out = []
    st = torch.cuda.current_stream()
    for rows in rows_list:
        g = torch.Generator(device="cuda:0").manual_seed(4000 + rows)
        probs = torch.softmax(torch.randn(rows, V, device="cuda:0", generator=g) * 3.0, -1)
        dst = torch.empty_like(probs)
        for _ in range(3):
            uno.top_p(probs, top_p, out=dst)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            uno.top_p(probs, top_p, out=dst)
        e1.record(st)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        kept = float((dst > 0).sum(-1).float().mean())
        byts = 8.0 * rows * V
        out.append({"rows": rows, "vocab": V, "top_p": top_p, "us_per_launch": us,
                    "bytes_per_launch": byts, "GB/s": byts / 1e3 / us,
                    "frac_hbm": byts / 1e3 / us / HBM_PEAK_GBS, "mean_kept": kept})
        log(f"top-p rows {rows}: {us:.1f} us per launch")
        del probs, dst
    return out


def cpu_sample_weights(cfg, w):
    """Host float32 copies of what the CPU baseline runs on: layer 0 and the first
    eighth of the LM head (row-major, before packing)."""
    import numpy as np
    lw = w["layers"][0]
    f32 = lambda t: t.float().cpu().numpy()
    w1 = {"final_norm": np.ones(cfg.d_model, np.float32),
          "layers": [{"attn_norm": f32(lw["attn_norm"]), "mlp_norm": f32(lw["mlp_norm"]),
                      "w": {p: f32(t) for p, t in lw["w"].items()},
                      "la": {p: f32(t) for p, t in lw["la"].items()},
                      "lb": {p: f32(t) for p, t in lw["lb"].items()}}]}
    return w1, f32(w["lm_head"][: cfg.vocab // 8])


def cpu_baseline(cfg, sample_w, tokens_per_iter, ctx=1024):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import model, psispec, rng
    from diffusion_drafted_lora_amd import configs, synth

    one = cfg.with_(n_layers=1)
    w1, W = sample_w
    kc = torch.from_numpy(synth.normal(9001, (1, ctx, cfg.n_kv_heads, cfg.head_dim)))
    kc = kc.to(torch.bfloat16).float().numpy()
    B = cfg.block_size
    cache = model.new_cache(one, 1, ctx + B + 2)
    cache["k"][0, 0, :ctx] = kc[0]
    cache["v"][0, 0, :ctx] = kc[0]
    xd = synth.normal(9002, (1, B, cfg.d_model))
    gate = np.ones((1, B))
    gate[0, 0] = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        model.forward(one, w1, None, np.arange(ctx, ctx + B)[None], gate, cache, hidden_in=xd,
                      want_logits=False)
        model.forward(one, w1, None, np.arange(ctx + 1, ctx + B + 1)[None], np.zeros((1, B)),
                      cache, hidden_in=xd, want_logits=False)
        reps += 1
        if time.perf_counter() - t0 > 8.0 or reps >= 4:
            break
    t_layer = (time.perf_counter() - t0) / reps
    # LM head on 1/8 of the vocabulary, both forwards' rows, scaled by 8
    h = synth.normal(9003, (2 * B, cfg.d_model))
    t0 = time.perf_counter()
    lg = model.bf16_round(h) @ W.T
    model.probs(lg)
    t_lm = (time.perf_counter() - t0) * 8
    # draft draws and one accept / resample over the full vocabulary
    P = synth.prob_rows(9004, (1, B, cfg.vocab))
    t0 = time.perf_counter()
    for j in range(B):
        rng.sample_icdf(P[0, j], rng.draw_word(1, 0, ctx + j, 0, 0))
    y = np.zeros((1, B), dtype=np.int64)
    psispec.accept_block(P, P[:, : B - 1], y, 1, [0], [ctx], [0])
    t_samp = time.perf_counter() - t0
    t_iter = cfg.n_layers * t_layer + t_lm + t_samp
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    # one BLAS thread: the draft forward of the sampled layer, once
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        model.forward(one, w1, None, np.arange(ctx, ctx + B)[None], gate, cache, hidden_in=xd,
                      want_logits=False)
        t_draft1 = time.perf_counter() - t0
    t_iter1 = t_iter * (t_draft1 / (t_layer / 2.0))
    return {
        "value": tokens_per_iter / t_iter, "unit": "tokens/s", "cores": int(threads),
        "host_cpus": os.cpu_count(), "blas_threads": int(threads),
        "one_thread": {"value": tokens_per_iter / t_iter1, "seconds_per_iteration": t_iter1,
                       "sample": "the draft forward of the sampled layer with one BLAS thread, "
                                 "scaled by the multi-threaded iteration's layer share"},
        "kind": "oracle",
        "sample": (f"float64 numpy oracle with bf16 storage rounding: 1 of {cfg.n_layers} layers "
                   f"(16 draft rows + 16 verify rows at context {ctx}) timed {reps}x, the LM head "
                   f"on 1/8 of the vocabulary scaled x8, 16 draft draws and one accept/resample; "
                   f"iteration time = {cfg.n_layers} x layer pair + LM head + sampling = "
                   f"{t_iter:.2f} s; tokens per iteration {tokens_per_iter:.3f} from the GPU run"),
        "seconds_per_iteration": t_iter,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--layers", type=int, default=None, help="(debug) fewer layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-steps", type=int, default=8)
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--bs128-steps", type=int, default=6,
                    help="timed iterations of the batch-128 leg (0 skips it)")
    ap.add_argument("--bs128-ctx", type=str, default="1024,5120,9216",
                    help="comma-separated starting contexts of the batch-128 leg (windows "
                         "over the 1K-in / 8K-out run)")
    ap.add_argument("--bs1-window-steps", type=int, default=40,
                    help="timed iterations of each batch-1 window (0 skips the windows)")
    ap.add_argument("--bs1-ctx", type=str, default="1024,5120,9216",
                    help="comma-separated starting contexts of the batch-1 windows over the "
                         "1K-in / 8K-out run")
    ap.add_argument("--distill", type=str, default="8,2048,16", metavar="BATCH,L,B",
                    help="distillation-forward leg (batch, L, block size); 'none' skips it")
    ap.add_argument("--distill-reps", type=int, default=2)
    ap.add_argument("--distill-backward-reps", type=int, default=1,
                    help="timed backward passes of the distillation leg (0 skips the backward)")
    ap.add_argument("--distill-b-sweep", type=str, default="4,8,32",
                    help="further block sizes of the distillation leg, one timed forward "
                         "each ('none' skips them)")
    ap.add_argument("--tree-steps", type=int, default=40,
                    help="timed steps of the batch-1 tree-sampler leg (0: skip)")
    ap.add_argument("--tree-chains", type=str, default="2,3,4",
                    help="chain counts of the tree-sampler leg")
    ap.add_argument("--qk-norm-steps", type=int, default=40,
                    help="timed steps of the batch-1 QK-norm leg (0: skip)")
    ap.add_argument("--stream-floor-reps", type=int, default=20,
                    help="launches per shape of the read-only stream floor leg (0: skip)")
    ap.add_argument("--no-top-p-leg", dest="top_p_leg", action="store_false",
                    help="skip timing the nucleus truncation at the batch-1 / batch-128 shapes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain elementwise copy of MIB MiB (HBM counter scale)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the Psi-Spec step is data parallel over sequences "
              "with no cross-GPU exchange, and it runs on one MI355X: use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from diffusion_drafted_lora_amd import configs, synth, uno

    cfg = configs.MODEL8B
    if args.layers:
        cfg = cfg.with_(n_layers=args.layers)
    B = cfg.block_size
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.copy_probe:
        copy_probe(args.copy_probe)
    log(f"generating weights ({cfg.n_layers} layers) on the GPU")
    w = synth.weights_torch(cfg, args.seed, dev)
    sample_w = None if args.no_cpu_baseline else cpu_sample_weights(cfg, w)
    w = uno.pack_weights(cfg, w)      # the kernels' fragment-tiled layout, once
    torch.cuda.empty_cache()
    max_new = (args.warmup + args.steps + args.breakdown_steps + 1) * (B + 1)
    if args.prompt + max_new > cfg.prompt_len + cfg.new_tokens + B + 1:
        log("note: steps exceed the 1K/8K protocol length; the context grows beyond 9216")
    max_len = args.prompt + max_new + B + 2
    # 256-row prefill chunks run on the large-M kernel, so the skinny decode kernels
    # only ever see the decode steps' 16-row blocks.
    eng = uno.Engine(cfg, w, max_seqs=1, max_seq_len=max_len, max_rows=256, seed=3002, device=dev)
    prompt = synth.prompts(cfg, 2002, 1, args.prompt)[0]
    log(f"prefill {args.prompt} tokens")
    t0 = time.perf_counter()
    eng.prefill([0], [prompt])
    eng.sync()
    t_prefill = time.perf_counter() - t0
    stream = eng.stream
    K, W = args.steps, args.warmup
    outs = torch.empty((W + K, B + 1), dtype=torch.int32, device=dev)
    nouts = torch.empty((W + K,), dtype=torch.int32, device=dev)
    log(f"warmup {W} steps")
    for i in range(W):
        eng.step([0], out=outs[i], n_out=nouts[i:i + 1])
    eng.sync()
    ctx0 = eng.seq_state(0)[0]
    log(f"timed {K} steps from context {ctx0}")
    # events on one gate/up launch in 7 (7 is prime to the 72 launches of a step,
    # so every layer and both forwards are sampled evenly)
    eng.timing(["linear_swiglu"], every=ROOFLINE_EVERY)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(W, W + K):
        eng.step([0], out=outs[i], n_out=nouts[i:i + 1])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    eng.sync()
    n_sw, ms_sw, b_sw, f_sw = eng.timing_read("linear_swiglu")
    eng.timing([])
    nout = nouts[W:].cpu().numpy().astype(np.int64)
    ctx1 = eng.seq_state(0)[0]
    tokens = int(nout.sum())
    sec = wall
    # algorithmic bytes of the timed steps
    fixed, lora = model_bytes(cfg)
    kvp = kv_bytes_per_pos(cfg)
    ctxs = ctx0 + np.concatenate([[0], np.cumsum(nout)[:-1]])
    step_bytes = 2 * fixed + lora + kvp * (2 * ctxs + 2 * B).astype(np.float64)
    total_bytes = float(step_bytes.sum())

    # per-class breakdown on a few extra steps
    classes = list(uno.KC)
    eng.timing(classes)
    for i in range(args.breakdown_steps):
        eng.step([0])
    eng.sync()
    breakdown = {}
    for c in classes:
        n, ms, b, f = eng.timing_read(c)
        if n:
            breakdown[c] = {"launches_per_step": n / args.breakdown_steps,
                            "ms_per_step": ms / args.breakdown_steps,
                            "GB/s": (b / 1e9) / (ms / 1e3) if ms > 0 else None}
    eng.timing([])

    tpf = tokens / (2.0 * K)
    sw_bytes_per_launch = b_sw / max(n_sw, 1)
    sw_ms = ms_sw / max(n_sw, 1)
    achieved = (sw_bytes_per_launch / 1e9) / (sw_ms / 1e3)
    result = {
        "metric": METRIC,
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": 1e3 * sec / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random N(0,0.02) weights generated on the GPU, uniform prompt)",
        "config": {"workload": "qwen3-8b-shape 36L bf16 + gated LoRA r128, batch 1, "
                               f"prompt {args.prompt}, B {B}, linear Psi-Spec, paged KV (16)",
                   "batch": 1, "block": B, "layers": cfg.n_layers,
                   "context_start": int(ctx0), "context_end": int(ctx1)},
        "positions_per_s": 2 * B * K / sec,
        "iterations_per_s": K / sec,
        "tokens_per_forward": tpf,
        "step_gpu_ms": gpu_ms / K,
        "hbm_gbs_step_algorithmic": total_bytes / 1e9 / sec,
        "hbm_frac_step": total_bytes / 1e9 / sec / HBM_PEAK_GBS,
        "prefill_s": t_prefill,
        "roofline": {
            "kernel": "gated-LoRA gate/up linear + SwiGLU (k_gemm_bf16<2,4,4>)",
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
            "bytes_per_launch": sw_bytes_per_launch, "us_per_launch": 1e3 * sw_ms,
            "launches": n_sw, "sampled_every": ROOFLINE_EVERY,
        },
        "breakdown": breakdown,
        "tpf_projection": tpf_projection(1e3 * sec / K, 1),
    }
    eng.close()
    del eng
    torch.cuda.empty_cache()
    if args.bs1_window_steps > 0:
        result["bs1_windows"] = [run_batch(cfg, w, dev, 1, int(c), args.bs1_window_steps, 4,
                                           args.prompt, log_prefix="bs1")
                                 for c in args.bs1_ctx.split(",")]
        result["bs1_run"] = integrate_windows(result["bs1_windows"], 1, B)
        if result["bs1_run"]:
            run = result["bs1_run"]
            run["hbm_gbs_algorithmic"] = run_bytes_per_iteration(cfg, run["contexts"]) / 1e9 / \
                (run["mean_ms_per_step"] / 1e3)
            run["hbm_frac"] = run["hbm_gbs_algorithmic"] / HBM_PEAK_GBS
            run["tpf_projection"] = tpf_projection(run["mean_ms_per_step"], 1)
    if args.qk_norm_steps > 0:
        result["qk_norm"] = run_qk_norm(cfg, w, dev, args.qk_norm_steps, 4, args.prompt)
    if args.tree_steps > 0:
        result["tree"] = run_tree(cfg, w, dev, [int(k) for k in args.tree_chains.split(",")],
                                  args.tree_steps, 4, args.prompt)
    if args.bs128_steps > 0:
        result["bs128"] = [run_batch(cfg, w, dev, 128, int(c), args.bs128_steps, 2, args.prompt)
                           for c in args.bs128_ctx.split(",")]
        result["bs128_run"] = integrate_windows(result["bs128"], 128, B)
        if result["bs128_run"]:
            result["bs128_run"]["tpf_projection"] = tpf_projection(
                result["bs128_run"]["mean_ms_per_step"], 128)
    if args.distill != "none":
        db, dl, dbs = (int(v) for v in args.distill.split(","))
        result["distill"] = run_distill(cfg, w, dev, db, dl, dbs, args.distill_reps)
        if args.distill_b_sweep != "none":
            keys = ("B", "ms_per_forward", "tflops", "mfma_frac", "rows_per_s", "mean_tv_block")
            result["distill_b_sweep"] = [
                {k: d[k] for k in keys}
                for d in (run_distill(cfg, w, dev, db, dl, int(b), 1)
                          for b in args.distill_b_sweep.split(","))]
        if args.distill_backward_reps > 0:
            result["distill_backward"] = run_distill_backward(cfg, w, dev, db, dl, dbs,
                                                              args.distill_backward_reps)
    if args.stream_floor_reps > 0:
        log("stream floor of the batch-1 linear launch shapes")
        result["stream_floor"] = run_stream_floor(cfg, args.stream_floor_reps)
    if args.top_p_leg:
        # one launch filters the B draft (or verify) rows of every sequence
        result["top_p"] = run_top_p(cfg.vocab, [B, 128 * B])
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(cfg, sample_w, tokens / K)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
