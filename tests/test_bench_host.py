"""Host-side logic of bench.py (no GPU): integrating the batch windows over a run,
reporting counter traffic only for the kernel sources it was measured on, and the
projection of a leg to the trained models' tokens per forward."""
import bench


def _win(ctx, ms, tpf=1.25):
    return {"context_start": ctx, "ms_per_step": ms, "tokens_per_forward": tpf}


def test_integrate_windows_linear_time_is_exact():
    # t(n) = 40 + 0.01 n ms: the mean over [1024, 9216] is t(5120) exactly
    ws = [_win(n, 40 + 0.01 * n) for n in (9216, 1024, 5120)]      # any order
    r = bench.integrate_windows(ws, 128, 16)
    assert r["contexts"] == [1024, 5120, 9216]
    assert abs(r["mean_ms_per_step"] - (40 + 0.01 * 5120)) < 1e-9
    assert abs(r["accepted_tokens_per_s"] - 128 * 2 * 1.25 / (r["mean_ms_per_step"] / 1e3)) < 1e-6
    assert abs(r["positions_per_s"] - 128 * 2 * 16 / (r["mean_ms_per_step"] / 1e3)) < 1e-6


def test_integrate_windows_unequal_spacing_and_degenerate():
    # trapezoid with unequal spans: (1000 * (10 + 20) / 2 + 3000 * (20 + 60) / 2) / 4000
    ws = [_win(0, 10), _win(1000, 20), _win(4000, 60)]
    r = bench.integrate_windows(ws, 1, 16)
    assert abs(r["mean_ms_per_step"] - (15000 + 120000) / 4000) < 1e-12
    assert bench.integrate_windows([_win(1024, 80)], 128, 16) is None
    assert bench.integrate_windows([_win(1024, 80), _win(1024, 90)], 128, 16) is None


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() is None                       # no summary
    f.write_text(f"traffic_bytes_per_launch: 123456\nkernel_source_sha256: {'0' * 64}\n")
    assert bench.measured_traffic() is None                       # other sources
    f.write_text(f"traffic_bytes_per_launch: 123456\n"
                 f"kernel_source_sha256: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic() == 123456.0


def test_run_bytes_per_iteration_counts_weights_lora_and_mean_context():
    from diffusion_drafted_lora_amd import configs
    cfg = configs.MODEL8B
    fixed, lora = bench.model_bytes(cfg)
    # the 8B shape: 15.136 GB of weights per forward, 0.698 GB of LoRA, 147,456 B of K/V
    # per position over 36 layers
    assert abs(fixed / 1e9 - 15.136) < 1e-3 and abs(lora / 1e9 - 0.698) < 1e-3
    assert bench.kv_bytes_per_pos(cfg) == 147456
    b = bench.run_bytes_per_iteration(cfg, [1024, 5120, 9216])
    assert abs(b - (2 * fixed + lora + 147456 * (2 * 5120 + 32))) < 1


def test_stream_floor_shapes_match_the_batch1_launches():
    """The read-only streams mirror the few-row launches of the 8B shape: the grids the
    kernel trace shows (q|k|v 384 x 512 threads, o and down 256 x 768, gate/up 768 x 256,
    LM head 4748 x 256) and each launch's weight bytes."""
    from diffusion_drafted_lora_amd import configs
    cfg = configs.MODEL8B
    sh = {n: (b, wg, th, ld) for n, b, wg, th, ld in bench.stream_floor_shapes(cfg)}
    assert sh["q|k|v"] == (6144 * 4096 * 2, 384, 512, 2)
    assert sh["o"] == (4096 * 4096 * 2, 256, 768, 2)
    assert sh["gate/up"] == (2 * 12288 * 4096 * 2, 768, 256, 8)
    assert sh["down"] == (12288 * 4096 * 2, 256, 768, 2)
    assert sh["lm_head"] == (151936 * 4096 * 2, 4748, 256, 8)
    # every shape's bytes split into whole 16-byte words over whole waves
    for b, wg, th, ld in sh.values():
        assert b % 16 == 0 and th % 64 == 0 and ld in (1, 2, 4, 8)


def test_tpf_projection_scales_the_measured_iteration():
    # 8 ms per iteration at batch 1: TPF 2.10 -> 2 * 2.10 tokens per 8 ms = 525 tokens/s
    p = bench.tpf_projection(8.0, 1)
    assert p["kind"] == "projection"
    assert set(p["accepted_tokens_per_s"]) == {"2.10", "2.25", "4.21"}
    assert abs(p["accepted_tokens_per_s"]["2.10"] - 525.0) < 1e-9
    # batch 128 at 100 ms: 128 * 2 * 4.21 / 0.1 s
    q = bench.tpf_projection(100.0, 128)
    assert abs(q["accepted_tokens_per_s"]["4.21"] - 128 * 2 * 4.21 / 0.1) < 1e-6
    # every projection stays within the method's bound TPF <= (B + 1) / 2 at B = 16
    assert max(bench.PAGES_TPF) <= (16 + 1) / 2
    assert bench.tpf_projection(0.0, 1) is None
