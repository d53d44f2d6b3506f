"""The roofline denominators (mxfp4_bit_attention_amd/probes.py over csrc/probes.hip)
run on the GPU and give physically possible figures: clocks within the part's range,
an fp4 MFMA rate below the 10.1 PFLOP/s spec peak, a tile mix slower than either of
its parts alone and faster than both back to back, HBM rates below 8 TB/s on a buffer
four times the size of the last-level cache."""
import pytest

from _gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def test_probe_figures_are_physical():
    torch, _ = require_gpu()
    from mxfp4_bit_attention_amd import probes

    den = probes.measure(torch, hbm_bytes=1 << 30)  # four times the last-level cache
    assert den["compute_units"] == 256 and den["wall_clock_kHz"] > 0
    for key in ("mfma_fp4_32x32x64", "mfma_fp4_32x32x64_random_operands"):
        mf = den[key]
        assert 1000 < mf["clock_MHz"] < 2600, key
        assert 0.4 * 10100 < mf["TFLOPs"] < 10100, key
        # one 32x32x64 fp4 MFMA keeps a SIMD's matrix pipe busy for 32 cycles
        assert 30 < mf["cycles_per_mfma_per_simd"] < 40, key
    for name, row in den["valu_cycles_per_instruction_per_simd"].items():
        # three waves per SIMD issue at least as fast as one (3% allowed for timing noise)
        assert 1.5 < row["cycles_3w"] <= 1.03 * row["cycles_1w"] and row["cycles_1w"] < 16, name
        assert 1000 < row["clock_MHz_3w"] < 2600, name
    for key, nm in (("attention_tile_mix", 18), ("attention_tile_mix_d64", 10)):
        m = den[key]
        assert m["per_trip"]["mfma_32x32x64"] == nm
        assert 1000 < m["clock_MHz"] < 2600
    m = den["attention_tile_mix"]
    whole, valu, mfma = m["cycles_per_trip_per_wave"], m["valu_only_cycles"], m["mfma_only_cycles"]
    assert 18 * 30 < mfma < 18 * 40
    assert max(valu, mfma) < whole < 1.02 * (valu + mfma)
    assert 0.0 < m["mfma_hidden"] < 1.0
    r = m["random_operands"]
    assert 1000 < r["clock_MHz"] < 2600 and 0.9 * whole < r["cycles_per_trip_per_wave"] < 1.1 * whole
    # the tile mix at d = 64 has 8 fewer MFMAs and the same vector work
    assert den["attention_tile_mix_d64"]["cycles_per_trip_per_wave"] < whole
    hbm = den["hbm"]
    assert 1000 < hbm["read_GBs"] < 8000 and 1000 < hbm["copy_GBs"] < 8000
