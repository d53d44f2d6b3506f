"""Measured roofline denominators (ctypes binding of libmxattn_probes.so).

The microbenchmarks of csrc/probes.hip, run on the current GPU: the dense fp4
block-scaled MFMA rate (32x32x64, E8M0 scales) with the core clock it sustains, on one
constant operand pattern and on pseudo-random operands (the clock the part sustains
depends on how much the operands toggle), the
issue rate of each vector instruction the attention kernel's softmax uses
(v_exp_f32, v_cvt_scalef32_pk_fp4_f32, v_fma_f32, v_max3_f32) in cycles per wave64
instruction per SIMD, whether exponentials and FMAs overlap, and HBM streaming read
and copy bandwidth (the best of a few launch shapes, as a stream benchmark reports).
Cycles are the kernel's HIP-event time times the core clock (s_memtime against the
constant-rate s_memrealtime, read by every wave), divided by the instructions each
SIMD issued.  Measurement support for the benchmark only: nothing on the attention
path calls it.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES_PATH = os.path.join(HERE, "libmxattn_probes.so")

VALU_KINDS = {"v_exp_f32": 0, "v_cvt_scalef32_pk_fp4_f32": 1, "v_fma_f32": 2, "v_max3_f32": 3}
EXP_FMA_KIND = 4
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
    lib.mxprobe_mfma_fp4.argtypes = [i64, i32, i32, vp, vp]
    lib.mxprobe_valu.restype = i32
    lib.mxprobe_valu.argtypes = [i32, i64, i32, vp, vp]
    lib.mxprobe_hbm_read.restype = i32
    lib.mxprobe_hbm_read.argtypes = [vp, u64, i32, vp, vp]
    lib.mxprobe_hbm_copy.restype = i32
    lib.mxprobe_hbm_copy.argtypes = [vp, vp, u64, i32, i32, vp]
    lib.mxprobe_mix.restype = i32
    lib.mxprobe_mix.argtypes = [i64, i32, i32, vp, vp]
    lib.mxprobe_hbm_dma.restype = i32
    lib.mxprobe_hbm_dma.argtypes = [vp, vp, u64, i32, i32, vp, vp]
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


def _clock(stats, wall_khz: int) -> float:
    """Core clock in MHz from a probe's stats: summed s_memtime cycles over summed
    s_memrealtime ticks of every wave, times the tick rate."""
    cyc, ticks = int(stats[0]), int(stats[1])
    return cyc / ticks * wall_khz / 1e3


def _run(torch, lib_call, stream, dev, wall_khz):
    """Warm up once, then time one launch; returns (ms, clock MHz)."""
    stats = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda: lib_call(ctypes.c_void_p(stats.data_ptr()))
    _timed(torch, run, stream)
    stats.zero_()
    ms = _timed(torch, run, stream)
    return ms, _clock(stats.tolist(), wall_khz)


def measure(torch, device=None, hbm_bytes: int = 1 << 31) -> dict:
    lib = _load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus, wall_khz = lib.mxprobe_cu_count(), lib.mxprobe_wall_clock_khz()
    simds = 4 * cus
    out = {"compute_units": cus, "wall_clock_kHz": wall_khz}

    # --- fp4 MFMA, one and two waves per SIMD (four independent accumulator chains each), with
    # one constant operand pattern and with pseudo-random operands (real data's toggling)
    for rnd, key in ((0, "mfma_fp4_32x32x64"), (1, "mfma_fp4_32x32x64_random_operands")):
        best = None
        for wps in (1, 2):
            iters = 50000 // wps
            ms, clk = _run(torch, lambda st: lib.mxprobe_mfma_fp4(iters, wps, rnd, st, sp), stream, dev, wall_khz)
            per_simd = wps * iters * MFMA_PER_TRIP
            row = {"waves_per_simd": wps, "TFLOPs": round(simds * per_simd * MFMA_FLOP / (ms * 1e-3) / 1e12, 1),
                   "clock_MHz": round(clk, 1),
                   "cycles_per_mfma_per_simd": round(ms * 1e-3 * clk * 1e6 / per_simd, 2), "ms": round(ms, 3)}
            if best is None or row["TFLOPs"] > best["TFLOPs"]:
                best = row
        out[key] = best

    # --- vector instructions: cycles per wave64 instruction per SIMD, 1 and 3 waves per SIMD
    def valu(kind, wps, it=6000):
        ms, clk = _run(torch, lambda st: lib.mxprobe_valu(kind, it, wps, st, sp), stream, dev, wall_khz)
        return ms * 1e-3 * clk * 1e6 / (wps * it * VALU_OPS_PER_TRIP), clk

    table = {}
    for name, kind in VALU_KINDS.items():
        row = {}
        for wps in (1, 3):
            cyc, clk = valu(kind, wps)
            row[f"cycles_{wps}w"] = round(cyc, 2)
            row[f"clock_MHz_{wps}w"] = round(clk, 1)
        table[name] = row
    out["valu_cycles_per_instruction_per_simd"] = table
    mix, _ = valu(EXP_FMA_KIND, 3)
    apart = 0.5 * (table["v_exp_f32"]["cycles_3w"] + table["v_fma_f32"]["cycles_3w"])
    out["exp_fma_interleaved"] = {"cycles_per_instruction_3w": round(mix, 2), "apart_mean": round(apart, 2),
                                  "overlap": "none" if mix >= 0.97 * apart else "partial"}

    # --- the attention tile's instruction mix alone (three waves per SIMD), d = 128 and 64,
    # and its two parts on their own: the vector instructions only, the MFMAs only
    it = 2000

    def mix(d, part):
        ms, clk = _run(torch, lambda st: lib.mxprobe_mix(it, d, part, st, sp), stream, dev, wall_khz)
        return ms, clk, ms * 1e-3 * clk * 1e6 / (3 * it)

    for d, key in ((128, "attention_tile_mix"), (64, "attention_tile_mix_d64")):
        ms, clk, cyc = mix(d, 0)
        out[key] = {
            "per_trip": {"mfma_32x32x64": 18 if d == 128 else 10, "v_exp_f32": 65, "fp4_cvt": 32, "v_fma_f32": 65,
                         "v_maximum3_f32": 34},
            "cycles_per_trip_per_wave": round(cyc, 1),
            "clock_MHz": round(clk, 1), "ms": round(ms, 3)}
    _, _, valu_only = mix(128, 1)
    _, _, mfma_only = mix(128, 2)
    _, clk_rand, cyc_rand = mix(128, 3)
    out["attention_tile_mix"]["random_operands"] = {"cycles_per_trip_per_wave": round(cyc_rand, 1),
                                                    "clock_MHz": round(clk_rand, 1)}
    whole = out["attention_tile_mix"]["cycles_per_trip_per_wave"]
    out["attention_tile_mix"]["valu_only_cycles"] = round(valu_only, 1)
    out["attention_tile_mix"]["mfma_only_cycles"] = round(mfma_only, 1)
    # share of the MFMA time that runs under the vector work
    out["attention_tile_mix"]["mfma_hidden"] = round((valu_only + mfma_only - whole) / mfma_only, 3)

    # --- HBM streaming, best of a few launch shapes
    n = hbm_bytes
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    read, copy = {}, {}
    for bpc in (8, 16, 32):
        rd = lambda: lib.mxprobe_hbm_read(p(src), n, bpc, p(sink), sp)
        _timed(torch, rd, stream, 2)
        read[f"{bpc}wg"] = round(n / (_timed(torch, rd, stream, 10) / 10 * 1e-3) / 1e9, 1)
        for nt in (0, 1):
            cp = lambda: lib.mxprobe_hbm_copy(p(src), p(dst), n, bpc, nt, sp)
            _timed(torch, cp, stream, 2)
            copy[f"{bpc}wg{'_nt' if nt else ''}"] = round(2 * n / (_timed(torch, cp, stream, 10) / 10 * 1e-3) / 1e9, 1)
    for bpc in (4, 8):
        for cp_ in (0, 1):
            run = lambda: lib.mxprobe_hbm_dma(p(src), p(dst), n, bpc, cp_, p(sink), sp)
            _timed(torch, run, stream, 2)
            gbs = (2 if cp_ else 1) * n / (_timed(torch, run, stream, 10) / 10 * 1e-3) / 1e9
            (copy if cp_ else read)[f"{bpc}wg_lds_dma"] = round(gbs, 1)
    out["hbm"] = {"bytes": n, "read_GBs": max(read.values()), "copy_GBs": max(copy.values()),
                  "read_by_shape": read, "copy_by_shape": copy}
    del src, dst
    return out
