"""Host-side checks of bench.py's accounting (no GPU): the roofline takes the
bound that the algorithmic FLOPs and bytes make binding at the published
peaks, and the per-workload byte and FLOP counts follow their definitions."""
import numpy as np
import pytest

import bench
from mixture_experts_ffn_sqrt_amd.synth import CONFIGS


def test_roofline_takes_the_binding_bound():
    # 1 TFLOP and 1 GB in 1 ms: 1 PF/s against 2.5 PF (0.4 ms ideal) and
    # 1 TB/s against 8 TB/s (0.125 ms ideal): the matrix cores bind
    r = bench.roofline_of(1e12, 1e9, 1.0, 2500.0, 2000.0, 6000.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0) and r["frac"] == pytest.approx(0.4)
    assert r["measured_peak"] == 2000.0 and r["frac_of_measured_peak"] == pytest.approx(0.5)
    assert r["other_bound"]["bound"] == "hbm"
    assert r["other_bound"]["frac"] == pytest.approx(1000.0 / 8000.0)
    # 1 TFLOP and 8 GB: 0.4 ms against 1 ms ideal: HBM binds
    r = bench.roofline_of(1e12, 8e9, 2.0, 2500.0, 2000.0, 6000.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(4000.0) and r["frac"] == pytest.approx(0.5)
    assert r["measured_peak"] == 6000.0
    assert r["other_bound"]["bound"] == "mfma"
    # no measured ceiling: no fraction of it
    assert bench.roofline_of(1e12, 1e9, 1.0, 2500.0, None, None)["frac_of_measured_peak"] is None


def test_up_gemm_bounds_of_the_prefill_and_decode_shapes():
    """Mixtral's 8 large groups sit far above the ridge; DeepSeek-V3's ~256 rows
    per expert below it (the weights take longer to stream than to multiply);
    V4-Flash decode far below it."""
    def bound(name, rows_per_expert):
        lc = CONFIGS[name]
        counts = np.full(lc.E, rows_per_expert)
        a = bench.accounting(lc, counts)
        r = bench.roofline_of(a["up_routed_flops"], a["up_routed_bytes"], 1.0,
                              bench.PEAK_TFLOPS[lc.dtype], None, None)
        return r["bound"]
    mix, ds = CONFIGS["mixtral_prefill"], CONFIGS["dsv3_prefill"]
    assert bound("mixtral_prefill", mix.T * mix.k // mix.E) == "mfma"
    assert bound("dsv3_prefill", ds.T * ds.k // ds.E) == "hbm"
    assert bound("v4flash_decode", 2) == "hbm"


def test_accounting_counts():
    lc = CONFIGS["mixtral_prefill"]
    counts = np.zeros(lc.E, dtype=np.int64)
    counts[:3] = [lc.T * lc.k - 2, 1, 1]
    a = bench.accounting(lc, counts)
    d, F, rows = lc.d, lc.d_ff, lc.T * lc.k
    assert a["up_routed_flops"] == 4 * d * F * rows
    assert a["up_routed_bytes"] == (3 * 2 * F * d + rows * d + rows * F) * 2
    f, nb = bench.lowp_accounting(lc, counts, "fp8")
    assert f == a["up_routed_flops"]
    w = 2 * F * d + (2 * F // 128) * (d // 128) * 4
    assert nb == 3 * w + rows * (d + d // 128 * 4) + rows * (F + F // 128 * 4)


def test_layer_roofline_fraction_is_t_roof_over_t():
    # 1 TFLOP and 2 GB in 1 ms: t_roof = max(0.4, 0.25) ms -> 0.4 of the roof
    r = bench.layer_roofline(1e12, 2e9, 1.0, "bf16")
    assert r["mfma_frac"] == pytest.approx(0.4) and r["hbm_frac"] == pytest.approx(0.25)
    assert r["roof_frac"] == pytest.approx(0.4)
    r = bench.layer_roofline(1e11, 4e9, 1.0, "bf16")
    assert r["roof_frac"] == pytest.approx(0.5)


def test_kernel_hash_ignores_comments_only():
    a = "int f(int x) {  // twice\n  return 2 * x; /* doubled */\n}\n"
    b = "/* header */\nint f(int x) {\n  // two times x\n  return 2 * x;\n}"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(a.replace("2 * x", "3 * x"))
    assert len(bench.kernel_source_sha("fp8")) == 64
