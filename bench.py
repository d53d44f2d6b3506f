#!/usr/bin/env python3
"""Benchmark of the MXFP4 UOS + PNQ attention pipeline on one MI355X.

One step = the whole hot path on the Wan2.2-720p-shaped self-attention
(B=1, H=40, N_q=N_kv=75,600, d=128, bf16 inputs resident in HBM): Hadamard +
UOS quantisation of K along d, UOS quantisation of V along tokens, the re-ordering
of their scale bytes into the attention kernel's per-tile operand order, and the
fused MXFP4 flash attention with PNQ, which rotates and quantises Q itself as it
loads its query rows.  Throughput is 4 B H N_q N_kv d per step time, in TFLOP/s.
Each of the K timed steps is bracketed by its own HIP events on the launch stream
(median, min and max reported beside the mean that gives `value`).

Printed as one JSON line, with:
  roofline       the attention kernel (dominant) against the dense MXFP4 MFMA
                 peak -- the metric's denominator -- timed alone (through
                 mxattn_forward_arranged, the same kernel binary) with HIP events
                 on its stream, plus HBM traffic from the committed rocprofv3
                 counter summary when it was taken on the current kernel source
                 (else null); `frac_measured` prices it against the fp4 MFMA rate
                 measured on this board, and `alu_floor` against the issue-time
                 floor of its softmax instructions (what binds it);
  denominators   the microbenchmarks behind those figures (libmxattn_probes.so):
                 fp4 MFMA rate and clock, per-instruction issue cycles, HBM
                 read / copy bandwidth;
  quantize_pass  the standalone Hadamard + quantise pass on 40 x 75,600 x 128
                 bf16 (the seeded host law the parity test checks bit for bit)
                 against HBM bandwidth (UOS, OCP and q = 6);
  rule_ablation  the full step under each shared-exponent rule (UOS, OCP, TFS,
                 OAS and CEIL 7.5; the same rule for Q, K, V and P~);
  other_shapes   the full step at d = 64, at B = 2 x H = 20, with 512 keys
                 (cross-attention-like), at 2,048 / 4,096 / 8,192 tokens, and on
                 the Wan2.2-480p and HunyuanVideo-720p workloads;
  cpu_baseline   the CPU oracle timed on a bounded sample of the same workload
                 on this host, extrapolated to the full workload (and, under
                 cpu_baseline_other, the same for Wan2.2-480p and for
                 HunyuanVideo-720p's 256 text rows).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline] [--no-extras]
    python bench.py --traffic-probe     (one copy of known size + one attention
                                         launch, for rocprofv3 --pmc runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "MXFP4-attn TFLOP/s & % of MXFP4 MFMA peak at H=40,N=75,600,d=128"
PEAK_MXFP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA (published)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E (published)
KERNEL_SOURCES = ["mxfp4_bit_attention_amd/csrc/attention.hip", "mxfp4_bit_attention_amd/csrc/mx_device.h",
                  "mxfp4_bit_attention_amd/csrc/launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_wan720p_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attn_algorithmic_bytes(w) -> int:
    """Bytes the attention kernel must move once: Q^ and K^ codes + scales, V^T codes +
    scales (padded to the kv tile), O in bf16."""
    n_q = w.B * w.H * w.N * w.d
    pad = -(-w.N // 128) * 128
    n_v = w.B * w.H * pad * w.d
    return n_q // 2 + n_q // 32 + n_q // 2 + n_q // 32 + n_v // 2 + n_v // 32 + n_q * 2


def quant_algorithmic_bytes(w) -> int:
    n = w.H * w.N * w.d
    return n * 2 + n // 2 + n // 32


def read_traffic(attn_launch_bytes: int):
    """HBM bytes per attention launch from the committed counter summary, or None when
    it is missing or was taken on different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def time_launches(torch, fn, iters: int, stream) -> float:
    """Average ms per call of fn(), HIP events on `stream` around `iters` back-to-back calls."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def time_each(torch, fn, iters: int, stream) -> list:
    """ms of each of `iters` back-to-back calls of fn(): one HIP event between calls on
    `stream` (the events do not stall the stream), synchronised on both sides."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(iters):
        fn()
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]


def spread(ms: list) -> dict:
    srt = sorted(ms)
    n = len(srt)
    med = srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])
    return {"mean": round(sum(ms) / n, 3), "median": round(med, 3), "min": round(srt[0], 3),
            "max": round(srt[-1], 3), "n": n}


def alu_floor(den: dict, d: int) -> dict:
    """Issue-time floor of the attention kernel's softmax: per score one FMA ((S - m')
    scale log2 e), one exponential, half an fp4 conversion (two codes per instruction)
    and half a max3 (two values per instruction of the block-max tree), at the cycles
    per wave64 instruction per SIMD measured with three waves per SIMD.  A SIMD's wave
    handles 64 scores per lane per 32-query x 128-key tile; the floor is the TFLOP/s
    at which that issue time alone fills every SIMD at the probes' clock."""
    v = den["valu_cycles_per_instruction_per_simd"]
    c = {k: v[k]["cycles_3w"] for k in v}
    per_tile = 64 * (c["v_exp_f32"] + c["v_fma_f32"]) + 32 * (c["v_cvt_scalef32_pk_fp4_f32"] + c["v_max3_f32"])
    clock = 0.5 * (v["v_exp_f32"]["clock_MHz_3w"] + v["v_cvt_scalef32_pk_fp4_f32"]["clock_MHz_3w"]) * 1e6
    simds = 4 * den["compute_units"]
    flop_per_tile = 4.0 * 32 * 128 * d
    return {"cycles_per_wave_tile": round(per_tile, 1), "clock_MHz": round(clock / 1e6, 1),
            "peak_TFLOPs": round(flop_per_tile * simds * clock / per_tile / 1e12, 1)}


def tile_mix_ceiling(den: dict, d: int, achieved: float) -> dict:
    """The attention tile's own instruction mix timed alone (no memory, LDS or barrier;
    three waves per SIMD as the kernel runs): the TFLOP/s the kernel would reach if every
    32-query x 128-key wave-tile cost only that, at the clock that mix sustains."""
    m = den["attention_tile_mix" if d == 128 else "attention_tile_mix_d64"]
    simds = 4 * den["compute_units"]
    peak = 4.0 * 32 * 128 * d * simds * m["clock_MHz"] * 1e6 / m["cycles_per_trip_per_wave"] / 1e12
    out = {"cycles_per_wave_tile": m["cycles_per_trip_per_wave"], "clock_MHz": m["clock_MHz"],
           "peak_TFLOPs": round(peak, 1), "frac": round(achieved / peak, 4)}
    for k in ("valu_only_cycles", "mfma_only_cycles", "mfma_hidden"):
        if k in m:
            out[k] = m[k]
    if "random_operands" in m:
        # the same mix with pseudo-random MFMA operands, at the clock it sustains then
        r = m["random_operands"]
        rp = 4.0 * 32 * 128 * d * simds * r["clock_MHz"] * 1e6 / r["cycles_per_trip_per_wave"] / 1e12
        out["random_operands"] = {"cycles_per_wave_tile": r["cycles_per_trip_per_wave"], "clock_MHz": r["clock_MHz"],
                                  "peak_TFLOPs": round(rp, 1), "frac": round(achieved / rp, 4)}
    return out


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing or failing: report the affinity count
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, rows: int = 1024, row_start: int = 0) -> dict:
    """The oracle on head 0: K and V quantisation of the full head, Q quantisation and
    flash attention for `rows` query rows (from `row_start`) against all N_kv keys;
    extrapolated to every row block and head."""
    import numpy as np
    from oracle import attention as ora
    from oracle import mxfp4
    blas = _blas_threads()
    Q = synth.attn_head(w, synth.Q_ID, 0)[row_start:row_start + rows]
    K = synth.attn_head(w, synth.K_ID, 0)
    V = synth.attn_head(w, synth.V_ID, 0)
    P = -(-w.N // 128) * 128
    t = time.perf_counter()
    Kc, Ks = ora.quantize_qk(K, mxfp4.UOS, True)
    t_k = time.perf_counter() - t
    t = time.perf_counter()
    Vc, Vs = ora.quantize_v(V, mxfp4.UOS, P)
    t_v = time.perf_counter() - t
    t = time.perf_counter()
    Qc, Qs = ora.quantize_qk(Q, mxfp4.UOS, True)
    t_q = time.perf_counter() - t
    t = time.perf_counter()
    ora.flash_attention_mx(Qc, Qs, Kc, Ks, Vc, Vs, w.N, float(np.float32(w.softmax_scale)), True, mxfp4.UOS, 128)
    t_a = time.perf_counter() - t
    row_blocks = w.N / rows
    per_head = t_k + t_v + t_q * row_blocks + t_a * row_blocks
    total = per_head * w.H * w.B
    return {
        "value": w.flops / total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"head 0 of {w.name}: Hadamard+UOS quantise of K ({w.N}x{w.d}) {t_k:.2f}s, token-axis "
                   f"quantise of V {t_v:.2f}s, Q quantise of {rows} rows (from row {row_start}) {t_q:.3f}s, "
                   f"PNQ flash attention of those {rows} query rows x {w.N} keys {t_a:.2f}s; extrapolated "
                   f"x{row_blocks:.1f} row blocks x{w.H * w.B} heads to {total:.0f}s for the full step. NumPy "
                   f"elementwise work is single-threaded; BLAS matmuls used up to {blas} threads; "
                   f"host os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}"),
    }


# Shared-exponent rules of the ablation: UOS (CEIL 7.25), OCP floor, TFS (CEIL 6), OAS (CEIL 7)
# and CEIL 7.5 (Pith review of MXAttention, referee report: the missing Qmax sweep).
ABLATION_RULES = (("uos", "uos"), ("ocp", "ocp"), ("tfs_q6", ("ceil", 6.0)), ("oas_q7", ("ceil", 7.0)),
                  ("q7.5", ("ceil", 7.5)))


def extras(torch, mx, w, q, k, v, out, ws, stream, iters: int = 5) -> dict:
    """Scale-rule ablation of the full step at the headline shape (the same rule for
    Q, K, V and the P~ tiles), and the step at other shapes the boundary takes: d = 64,
    two batch entries, a short key sequence (text-like cross-attention), and the
    Wan2.2-480p and HunyuanVideo-720p workloads."""
    res = {}
    ab = {}
    for name, rule in ABLATION_RULES:
        fn = lambda rule=rule: mx.mxattn_forward(q, k, v, float(w.softmax_scale), hadamard=True, pnq=True,
                                                 rule=rule, out=out, workspace=ws)
        fn()
        ms = time_launches(torch, fn, iters, stream)
        ab[name] = {"ms_per_step": round(ms, 3), "TFLOPs": round(w.flops / (ms * 1e-3) / 1e12, 1)}
    res["rule_ablation"] = {"workload": w.name, "pnq": True, "hadamard": True, "rules": ab}

    shapes = {}
    other = (("d64", dict(B=1, H=40, Nq=w.N, Nkv=w.N, d=64)),
             ("B2_H20", dict(B=2, H=20, Nq=w.N, Nkv=w.N, d=128)),
             ("cross_Nkv512", dict(B=1, H=40, Nq=w.N, Nkv=512, d=128)),
             ("N2048", dict(B=1, H=40, Nq=2048, Nkv=2048, d=128)),
             ("N4096", dict(B=1, H=40, Nq=4096, Nkv=4096, d=128)),
             ("N8192", dict(B=1, H=40, Nq=8192, Nkv=8192, d=128)))
    for name, sh in other:
        g = torch.Generator(device=q.device).manual_seed(7)
        mk = lambda n: torch.randn((sh["B"], sh["H"], n, sh["d"]), generator=g, device=q.device).to(torch.bfloat16)
        qq, kk, vv = mk(sh["Nq"]), mk(sh["Nkv"]), mk(sh["Nkv"])
        oo = torch.empty_like(qq)
        wsz = mx.mxattn_forward_workspace_bytes(sh["B"], sh["H"], sh["Nq"], sh["Nkv"], sh["d"])
        wws = torch.empty(wsz, dtype=torch.uint8, device=q.device)
        sc = 1.0 / math.sqrt(sh["d"])
        fn = lambda: mx.mxattn_forward(qq, kk, vv, sc, hadamard=True, pnq=True, rule="uos", out=oo, workspace=wws)
        fn()
        # short steps are timed over more launches so that each timing spans several ms
        ms = time_launches(torch, fn, iters if sh["Nq"] * sh["Nkv"] > 1 << 26 else 20 * iters, stream)
        flops = 4.0 * sh["B"] * sh["H"] * sh["Nq"] * sh["Nkv"] * sh["d"]
        shapes[name] = dict(sh, ms_per_step=round(ms, 3), TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1))
        del qq, kk, vv, oo, wws
    # the pages' other two workloads, full step on their synthetic tensors
    for wl in (synth.WAN_480P, synth.HUNYUAN_720P):
        qq, kk, vv = (synth.device_attn_tensor(wl, t, q.device) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
        oo = torch.empty_like(qq)
        wws = torch.empty(mx.mxattn_forward_workspace_bytes(wl.B, wl.H, wl.N, wl.N, wl.d), dtype=torch.uint8,
                          device=q.device)
        fn = lambda: mx.mxattn_forward(qq, kk, vv, float(wl.softmax_scale), hadamard=True, pnq=True, rule="uos",
                                       out=oo, workspace=wws)
        fn()
        ms = time_launches(torch, fn, iters, stream)
        shapes[wl.name] = dict(B=wl.B, H=wl.H, Nq=wl.N, Nkv=wl.N, d=wl.d, ms_per_step=round(ms, 3),
                               TFLOPs=round(wl.flops / (ms * 1e-3) / 1e12, 1))
        del qq, kk, vv, oo, wws
    res["other_shapes"] = shapes
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize-pass", action="store_true")
    ap.add_argument("--no-denominators", action="store_true",
                    help="skip the microbenchmarks behind the measured roofline denominators")
    ap.add_argument("--traffic-probe", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the scale-rule ablation and the other-shape lines")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path runs on a single MI355X); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-GPU; do not launch it with more than one rank", file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp4_bit_attention_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WAN_720P
    scale = float(w.softmax_scale)
    q = synth.device_attn_tensor(w, synth.Q_ID, dev)
    k = synth.device_attn_tensor(w, synth.K_ID, dev)
    v = synth.device_attn_tensor(w, synth.V_ID, dev)
    out = torch.empty_like(q)
    ws = torch.empty(mx.mxattn_forward_workspace_bytes(w.B, w.H, w.N, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # attention-only operands: mxattn_forward_arranged launches the kernel mxattn_forward
    # ends with (same binary; Q^ read instead of quantised in its prologue)
    qc, qs = mx.mxattn_quantize(q.view(-1, w.N, w.d), rule="uos", axis="last", hadamard=True)
    kc, ks = mx.mxattn_quantize(k.view(-1, w.N, w.d), rule="uos", axis="last", hadamard=True)
    vc, vs = mx.mxattn_quantize(v.view(-1, w.N, w.d), rule="uos", axis="rows")
    shp = (w.B, w.H)
    qc, qs, kc, ks = (t.view(*shp, *t.shape[1:]) for t in (qc, qs, kc, ks))
    vc, vs = (t.view(*shp, *t.shape[1:]) for t in (vc, vs))
    ksa, vsa = mx.mxattn_arrange_scales(ks, vs, w.N)
    out_a = torch.empty_like(q)

    def attn_only():
        mx.mxattn_forward_arranged(qc, qs, kc, ksa, vc, vsa, w.N, scale, pnq=True, p_rule="uos", out=out_a)

    if args.traffic_probe:
        # a plain copy of known size (the counter scale reference), then one attention launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        attn_only()
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": src.numel(),
                          "attn_algorithmic_bytes": attn_algorithmic_bytes(w),
                          "kernel_source_sha256_16": kernel_source_hash()}))
        return

    def step():
        mx.mxattn_forward(q, k, v, scale, hadamard=True, pnq=True, rule="uos", out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    steps_ms = time_each(torch, step, args.steps, stream)
    torch.cuda.synchronize()
    t_wall = (time.perf_counter() - t_wall) / args.steps * 1e3
    ms_step = sum(steps_ms) / len(steps_ms)
    value = w.flops / (ms_step * 1e-3) / 1e12

    # dominant kernel alone, same launch configuration
    for _ in range(2):
        attn_only()
    attn_ms = time_each(torch, attn_only, args.steps, stream)
    ms_attn = sum(attn_ms) / len(attn_ms)
    achieved = w.flops / (ms_attn * 1e-3) / 1e12
    abytes = attn_algorithmic_bytes(w)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_MXFP4_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MXFP4_TFLOPS, 4), "traffic": read_traffic(abytes),
                "kernel": "k_attn<d=128, arranged scales, PNQ>", "ms_per_launch": spread(attn_ms),
                "algorithmic_bytes": abytes,
                "bound_note": ("'mfma' is the metric's denominator (dense fp4 MFMA peak); the SQ counters show the "
                               "kernel bound by vector-ALU issue of its softmax (exp and fp4 conversion), priced "
                               "under alu_floor")}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4(e2m1+e8m0)->fp32",
        "data": "synthetic (seeded device generator, outlier-channel Gaussian law)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N, "N_kv": w.N, "d": w.d,
                   "input_dtype": "bf16", "hadamard": True, "rule": "uos", "pnq": True,
                   "kv_tile": mx.mxattn_kv_tile()},
        "pct_of_mxfp4_peak": round(100.0 * value / PEAK_MXFP4_TFLOPS, 2),
        "step_ms": spread(steps_ms),
        "wall_ms_per_step": round(t_wall, 3),
        "roofline": roofline,
    }
    del qc, qs, kc, ks, vc, vs, ksa, vsa

    def denominators():
        from mxfp4_bit_attention_amd import probes
        den = probes.measure(torch, dev)
        result["denominators"] = den
        mf = den["mfma_fp4_32x32x64"]["TFLOPs"]
        roofline["peak_measured"] = mf
        roofline["frac_measured"] = round(achieved / mf, 4)
        # the same MFMA loop on pseudo-random operands: the rate the part sustains on data that
        # toggles as real operands do
        mfr = den["mfma_fp4_32x32x64_random_operands"]["TFLOPs"]
        roofline["peak_measured_random_operands"] = mfr
        roofline["frac_measured_random_operands"] = round(achieved / mfr, 4)
        fl = alu_floor(den, w.d)
        fl["frac"] = round(achieved / fl["peak_TFLOPs"], 4)
        roofline["alu_floor"] = fl
        roofline["tile_mix"] = tile_mix_ceiling(den, w.d, achieved)

    def quantize_pass():
        qw = synth.QUANT_720P
        # the seeded host law, as the whole-tensor parity test draws it
        xh = synth.quant_tensor_bf16(qw, threads=min(16, len(os.sched_getaffinity(0))))
        x = torch.from_numpy(xh.view("int16")).view(torch.bfloat16).to(dev)
        del xh
        qbytes = quant_algorithmic_bytes(qw)
        c = torch.empty((qw.H, qw.N, qw.d // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((qw.H, qw.N, qw.d // 32), dtype=torch.uint8, device=dev)
        qp = {"workload": qw.name, "algorithmic_bytes": qbytes, "peak_GBs": PEAK_HBM_GBS,
              "input": "seeded host generator (synth.quant_tensor_bf16)"}
        if "denominators" in result:
            # measured stream model: the pass's reads at the probe's read rate plus its writes at
            # the write rate a copy implies (copy time = n / read + n / write)
            rd = result["denominators"]["hbm"]["read_GBs"]
            cp = result["denominators"]["hbm"]["copy_GBs"]
            wr = 1.0 / (2.0 / cp - 1.0 / rd)
            n = qw.H * qw.N * qw.d
            qp["stream_read_GBs"], qp["stream_copy_GBs"], qp["stream_write_GBs"] = rd, cp, round(wr, 1)
            qp["stream_model_us"] = round((2 * n / rd + (n // 2 + n // 32) / wr) / 1e3, 1)
        # right after the attention runs the first ~10 ms of quantize launches run ~5%
        # slower: warm the pass up for ~17 ms before timing any rule
        for _ in range(100):
            mx.mxattn_quantize(x, rule="uos", axis="last", hadamard=True, codes=c, scales=s)
        for name, rule in (("uos", "uos"), ("ocp", "ocp"), ("q6", ("ceil", 6.0))):
            fn = lambda rule=rule: mx.mxattn_quantize(x, rule=rule, axis="last", hadamard=True, codes=c, scales=s)
            for _ in range(10):
                fn()
            ms = time_launches(torch, fn, max(args.steps, 50), stream)
            gbs = qbytes / (ms * 1e-3) / 1e9
            qp[name] = {"us": round(ms * 1e3, 1), "GBs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
            if "stream_model_us" in qp:
                qp[name]["frac_of_stream_model"] = round(qp["stream_model_us"] / (ms * 1e3), 4)
        result["quantize_pass"] = qp

    def other_shapes():
        result.update(extras(torch, mx, w, q, k, v, out, ws, stream))
        if "denominators" in result:
            d64 = result["other_shapes"]["d64"]
            d64["tile_mix"] = tile_mix_ceiling(result["denominators"], 64, d64["TFLOPs"])

    def cpu_baselines():
        result["cpu_baseline"] = cpu_baseline(w)
        hy = synth.HUNYUAN_720P
        result["cpu_baseline_other"] = {
            synth.WAN_480P.name: cpu_baseline(synth.WAN_480P, rows=512),
            hy.name + " (text rows)": cpu_baseline(hy, rows=hy.text_rows, row_start=hy.N - hy.text_rows),
        }

    # the sections after the headline figures: a Python-level failure in one is reported in
    # the line (as <section>_error) instead of losing the figures already measured
    for skip, name, fn in ((args.no_denominators, "denominators", denominators),
                           (args.no_quantize_pass, "quantize_pass", quantize_pass),
                           (args.no_extras, "other_shapes", other_shapes),
                           (args.no_cpu_baseline, "cpu_baseline", cpu_baselines)):
        if skip:
            continue
        try:
            fn()
        except Exception as e:  # reported in the line and on stderr, not swallowed
            result[name + "_error"] = f"{type(e).__name__}: {e}"[:400]
            print(f"bench.py: the {name} section failed: {e!r}", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
