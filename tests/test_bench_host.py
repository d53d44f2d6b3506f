"""Host-side checks of bench.py (CPU only): the single-GPU guard, the metric's
arithmetic and the algorithmic byte counts it prices the kernels with."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_attention_work_and_bytes_at_the_headline_shape():
    """4 B H N^2 d flop; per head-row: Q^ and K^ 64 code bytes + 4 scale bytes each,
    O 256 bytes (bf16), V^T 0.5 + 1/32 bytes per element of the 128-padded token axis."""
    w = synth.WAN_720P
    assert (w.B, w.H, w.N, w.d) == (1, 40, 75600, 128)
    assert w.flops == 4 * 40 * 75600 ** 2 * 128
    rows = 40 * 75600
    pad = 75648  # 591 tiles of 128
    want = rows * (64 + 4) * 2 + rows * 256 + 40 * pad * 128 // 2 + 40 * pad * 128 // 32
    assert bench.attn_algorithmic_bytes(w) == want == 1391170560


def test_quantize_pass_bytes():
    """bf16 read (2 B) + codes (0.5 B) + one scale byte per 32 elements."""
    n = 40 * 75600 * 128
    assert bench.quant_algorithmic_bytes(synth.QUANT_720P) == 2 * n + n // 2 + n // 32 == 979776000


def test_traffic_is_ignored_for_other_kernel_sources(tmp_path, monkeypatch):
    """The counter-measured traffic is reported only for the kernel source it was taken on."""
    import json
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"kernel_source_sha256_16": "0" * 16, "bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic(1) is None
    f.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_source_hash(), "bytes_per_launch": 123.0}))
    assert bench.read_traffic(1) == 123.0


def test_ceilings_from_the_probe_figures():
    """The tile-mix ceiling is the wave-tile's flops on every SIMD at the mix's clock and
    cycles (and again for the mix on pseudo-random operands); the vector-issue floor prices
    64 exponentials and FMAs and 32 conversions and max3 per wave-tile."""
    den = {
        "compute_units": 256,
        "attention_tile_mix": {"cycles_per_trip_per_wave": 1400.0, "clock_MHz": 2000.0,
                               "random_operands": {"cycles_per_trip_per_wave": 1600.0, "clock_MHz": 1600.0}},
        "valu_cycles_per_instruction_per_simd": {
            k: {"cycles_3w": c, "clock_MHz_3w": 2000.0}
            for k, c in (("v_exp_f32", 8.0), ("v_cvt_scalef32_pk_fp4_f32", 8.0), ("v_fma_f32", 2.0), ("v_max3_f32", 4.0))},
    }
    flop_tile = 4.0 * 32 * 128 * 128
    tm = bench.tile_mix_ceiling(den, 128, achieved=1000.0)
    peak = flop_tile * 1024 * 2.0e9 / 1400.0 / 1e12
    assert tm["peak_TFLOPs"] == pytest.approx(peak, abs=0.05) and tm["frac"] == pytest.approx(1000.0 / peak, abs=1e-4)
    rp = flop_tile * 1024 * 1.6e9 / 1600.0 / 1e12
    assert tm["random_operands"]["peak_TFLOPs"] == pytest.approx(rp, abs=0.05)
    fl = bench.alu_floor(den, 128)
    assert fl["cycles_per_wave_tile"] == 64 * (8 + 2) + 32 * (8 + 4)
    assert fl["peak_TFLOPs"] == pytest.approx(flop_tile * 1024 * 2.0e9 / fl["cycles_per_wave_tile"] / 1e12, abs=0.05)
