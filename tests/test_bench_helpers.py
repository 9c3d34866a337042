"""bench.py's counting helpers against the counts stated for the workloads
(counted flops per token of the chunked form, the recurrence's own count, the
decode step's bytes), its timing summary and the clock report."""
import bench


def test_counted_flops_per_token_at_d128():
    f = bench.flops_per_token(128, 64, 30)
    assert f["scan"] == 65536 and f["cg_iter"] == 50688 and f["out"] == 49408
    assert f["total"] == 1635584  # 857.5 GFLOP over the 524,288 token-heads of workload 3
    assert round(f["total"] * 8 * 16 * 4096 / 1e9, 1) == 857.5


def test_recurrent_form_count():
    # (3d^2 + 3d^2) + n (2d^2 + 10d) + 2d^2 at d = 128, 30 steps: about 1.15 MFLOP per token
    assert bench.recurrent_flops_per_token(128, 30) == 1152512


def test_decode_bytes_per_step():
    # H and G read and written in fp32 plus the token's vectors: 1.079 GB for 4096 pairs
    per_pair = bench.decode_bytes_per_pair(128, 2)
    assert per_pair == 2 * 4 * 2 * 128 * 128 + 3 * 2 * 128 + 8 + 4 * 128 + 4
    total = 4096 * per_pair + 16 * 128 * 4  # lambda once per head
    assert total == 1079042048


def test_spread():
    s = bench.spread([1.0, 2.0, 3.0, 4.0, 5.0])
    assert s == {"median": 3.0, "p25": 2.0, "p75": 4.0, "iqr": 2.0, "n": 5}


def test_clock_report():
    # the nominal 2.5 PFLOP/s is quoted at 2.4 GHz: at 2.0 GHz the same kernel
    # has 2.5 * 2.0 / 2.4 = 2.083 PFLOP/s to reach
    assert bench.clock_report(None, 775.0) is None
    c = {"gfx_mhz_median": 2000.0, "gfx_mhz_min": 1950.0, "gfx_mhz_max": 2050.0, "samples": 9, "steps_run": 960}
    r = bench.clock_report(c, 775.0)
    assert r["nominal_mhz"] == 2400.0 and r["samples"] == 9
    assert r["cg_frac_of_peak_at_that_clock"] == round(775.0 / (2500.0 * 2000.0 / 2400.0), 4) == 0.372
