"""Measured roofline denominators (ctypes binding of libmxattn_probes.so).

The microbenchmarks of csrc/probes.hip, run on the current GPU: the dense fp4
block-scaled MFMA rate (32x32x64, E8M0 scales) with the core clock it sustains, the
issue rate of each vector instruction the attention kernel's softmax uses
(v_exp_f32, v_cvt_scalef32_pk_fp4_f32, v_fma_f32, v_max3_f32) in cycles per wave64
instruction per SIMD, and HBM streaming read and copy bandwidth.  Measurement support
for the benchmark only: nothing on the attention path calls it.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES_PATH = os.path.join(HERE, "libmxattn_probes.so")

VALU_KINDS = {"v_exp_f32": 0, "v_cvt_scalef32_pk_fp4_f32": 1, "v_fma_f32": 2, "v_max3_f32": 3}
MFMA_FLOP = 2 * 32 * 32 * 64          # one 32x32x64 MFMA
VALU_OPS_PER_TRIP = 32                # instructions per wave per loop trip (csrc/probes.hip)
MFMA_PER_TRIP = 4


def _load():
    if not os.path.exists(PROBES_PATH):
        raise ImportError(f"{PROBES_PATH} is not built; run `python mxfp4_bit_attention_amd/build.py`")
    lib = ctypes.CDLL(PROBES_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    lib.mxprobe_cu_count.restype = i32
    lib.mxprobe_wall_clock_khz.restype = i32
    lib.mxprobe_mfma_fp4.restype = i32
    lib.mxprobe_mfma_fp4.argtypes = [i64, i32, vp, vp]
    lib.mxprobe_valu.restype = i32
    lib.mxprobe_valu.argtypes = [i32, i64, i32, vp, vp]
    lib.mxprobe_hbm_read.restype = i32
    lib.mxprobe_hbm_read.argtypes = [vp, u64, vp, vp]
    lib.mxprobe_hbm_copy.restype = i32
    lib.mxprobe_hbm_copy.argtypes = [vp, vp, u64, vp]
    return lib


def _timed(torch, launch, stream, reps: int = 1) -> float:
    """ms of `reps` back-to-back launches, HIP events on `stream`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        rc = launch()
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1)


def _clock(stats, wall_khz: int) -> tuple[float, float]:
    """(core clock in MHz, mean s_memtime cycles per wave) from a probe's stats."""
    cyc, ticks, waves = (int(v) for v in stats[:3])
    return cyc / ticks * wall_khz / 1e3, cyc / max(waves, 1)


def measure(torch, device=None, hbm_bytes: int = 1 << 31) -> dict:
    lib = _load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus, wall_khz = lib.mxprobe_cu_count(), lib.mxprobe_wall_clock_khz()
    simds = 4 * cus
    out = {"compute_units": cus, "wall_clock_kHz": wall_khz}

    # --- fp4 MFMA: two waves per SIMD keep the matrix pipe issuing back to back
    iters, wps = 20000, 2
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda: lib.mxprobe_mfma_fp4(iters, wps, ctypes.c_void_p(stats.data_ptr()), sp)
    _timed(torch, run, stream)                                   # warm up (clock ramp)
    stats.zero_()
    ms = _timed(torch, run, stream)
    st = stats.tolist()
    clk, cyc_wave = _clock(st, wall_khz)
    n_mfma = simds * wps * iters * MFMA_PER_TRIP
    out["mfma_fp4_32x32x64"] = {
        "TFLOPs": round(n_mfma * MFMA_FLOP / (ms * 1e-3) / 1e12, 1),
        "clock_MHz": round(clk, 1),
        "cycles_per_mfma_per_simd": round(cyc_wave / (iters * MFMA_PER_TRIP * wps), 2),
        "ms": round(ms, 3), "waves_per_simd": wps,
    }

    # --- vector instructions: cycles per wave64 instruction per SIMD, 1 and 3 waves per SIMD
    valu = {}
    for name, kind in VALU_KINDS.items():
        row = {}
        for wps in (1, 3):
            it = 4000
            stats = torch.zeros(4, dtype=torch.int64, device=dev)
            run = lambda: lib.mxprobe_valu(kind, it, wps, ctypes.c_void_p(stats.data_ptr()), sp)
            _timed(torch, run, stream)
            stats.zero_()
            _timed(torch, run, stream)
            clk_v, cyc_wave = _clock(stats.tolist(), wall_khz)
            row[f"cycles_{wps}w"] = round(cyc_wave / (it * VALU_OPS_PER_TRIP) / wps, 2)
            row[f"clock_MHz_{wps}w"] = round(clk_v, 1)
        valu[name] = row
    out["valu_cycles_per_instruction_per_simd"] = valu

    # --- HBM streaming
    n = hbm_bytes
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    rd = lambda: lib.mxprobe_hbm_read(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), sp)
    cp = lambda: lib.mxprobe_hbm_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, sp)
    _timed(torch, rd, stream, 2)
    ms_r = _timed(torch, rd, stream, 10) / 10
    _timed(torch, cp, stream, 2)
    ms_c = _timed(torch, cp, stream, 10) / 10
    out["hbm"] = {"bytes": n, "read_GBs": round(n / (ms_r * 1e-3) / 1e9, 1),
                  "copy_GBs": round(2 * n / (ms_c * 1e-3) / 1e9, 1)}
    del src, dst
    return out
