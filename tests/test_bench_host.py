"""Host-side logic of bench.py (no GPU): integrating the batch windows over a run,
and reporting counter traffic only for the kernel sources it was measured on."""
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
