#!/usr/bin/env python3
"""Mechanism diagnostics of MXFP4 scale rules on the GPU (a study script, like bench.py).

The Pith review's referee report notes that the optimality of the UOS constant
q = 7.25 is argued for a model density of block maxima, and that per-block Qmax
sweeps on real tensors -- P~ tiles included -- are not shown.  These helpers run
those sweeps on any tensor with the library's own kernels:

  qmax_sweep(x, qs, ...)        relative MSE of CEIL(q) block quantisation for each q
                                (x along its last axis, optionally after the Hadamard
                                rotation; or along its rows, as V is quantised);
  p_tile_sweep(...)             the attention output's relative L2 error against exact
                                attention when only the P~ tiles' rule varies;
  rowsum_decomposition(...)     how quantising P~ moves each row's normaliser, split
                                into zeroed, saturated, rounded-down and rounded-up
                                elements (from the kernel's P^ dump);
  global_scaling(...)           the post-normalisation arm with one global factor g
                                applied to P before quantisation: the row sums of the
                                quantised tile for each g, and the g that brings their
                                average closest to one (Figure 7, panel C).

Quantisation and attention run in libmxattn through the binding; the references these
studies compare against (softmax on dequantised operands, a replay of the unquantised
P~, row sums) are reductions in torch here, outside the product package, which holds
only the binding of the HIP path.

    python diagnostics.py          (one JSON line on the Wan2.2-720p-shaped tensors)
"""
from __future__ import annotations

import numpy as np

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from mxfp4_bit_attention_amd import (mxattn_forward_quantized, mxattn_kv_tile,  # noqa: E402
                                     mxattn_padded_tokens, mxattn_quant_error, mxattn_quantize)

SWEEP_QS = tuple(round(6.0 + 0.05 * i, 2) for i in range(41))  # 6.00, 6.05, ..., 8.00


def qmax_sweep(x, qs=SWEEP_QS, axis: str = "last", hadamard: bool = False, extra_rules=("ocp",)):
    """Relative MSE sum (v - dequant v)^2 / sum v^2 of block quantisation of x under
    CEIL(q) for every q in qs (plus the named extra rules).  Returns {label: rel_mse}."""
    import torch
    out = {}
    sums = torch.empty(3, dtype=torch.float64, device=x.device)
    rules = [(f"q{q:.2f}", ("ceil", float(q))) for q in qs] + [(r, r) for r in extra_rules]
    for label, rule in rules:
        mxattn_quant_error(x, rule=rule, axis=axis, hadamard=hadamard, sums=sums)
        e2, r2, nf = sums.tolist()
        out[label] = {"rel_mse": e2 / r2 if r2 > 0 else float("nan"), "nonfinite_blocks": int(nf)}
    return out


def argmin_q(sweep: dict) -> float:
    """The q of the smallest relative MSE among the CEIL(q) entries of a sweep."""
    best = min((v["rel_mse"], k) for k, v in sweep.items() if k.startswith("q"))
    return float(best[1][1:])


E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _dequant_last(c, s):
    """Packed codes [R, C/2] and E8M0 scales [R, C/32] (device) -> fp32 values [R, C]."""
    import torch
    lut = torch.from_numpy(np.concatenate([E2M1, -E2M1])).to(c.device)
    lo, hi = (c & 15).long(), (c >> 4).long()
    vals = torch.stack([lut[lo], lut[hi]], dim=-1).reshape(c.shape[0], -1)
    return vals * torch.pow(2.0, s.float() - 127.0).repeat_interleave(32, dim=1)


def _quantized_head(q, k, v, rule, hadamard):
    qc, qsc = mxattn_quantize(q, rule=rule, axis="last", hadamard=hadamard)
    kc, ksc = mxattn_quantize(k, rule=rule, axis="last", hadamard=hadamard)
    vc, vsc = mxattn_quantize(v, rule=rule, axis="rows")
    return qc, qsc, kc, ksc, vc, vsc


def p_tile_sweep(q, k, v, softmax_scale: float, qs=SWEEP_QS, rows=None, rule="uos", hadamard: bool = True):
    """One head (q, k, v: [N, d] on the GPU).  Q, K, V are quantised once with `rule`;
    the attention then runs with CEIL(q') on the P~ tiles for every q' in qs (and OCP).
    Returns {label: relative L2 error of O[rows]} against softmax attention on the same
    dequantised Q^, K^, V^ with P left unquantised, so only the P~ tiles' rule differs."""
    import torch
    n, d = q.shape
    nkv = k.shape[0]
    rows = torch.arange(n, device=q.device) if rows is None else torch.as_tensor(rows, device=q.device)
    qc, qsc, kc, ksc, vc, vsc = _quantized_head(q, k, v, rule, hadamard)
    qd = _dequant_last(qc[rows], qsc[rows])
    kd = _dequant_last(kc, ksc)
    vd = _dequant_last(vc, vsc).t()[:nkv].contiguous()
    pr = torch.softmax((qd @ kd.t().contiguous()) * softmax_scale, dim=-1)
    ref = pr @ vd
    sh = lambda t: t.reshape(1, 1, *t.shape)
    qc, qsc, kc, ksc, vc, vsc = map(sh, (qc, qsc, kc, ksc, vc, vsc))
    out = {}
    labels = [(f"q{x:.2f}", ("ceil", float(x))) for x in qs] + [("ocp", "ocp")]
    for label, prule in labels:
        o = mxattn_forward_quantized(qc, qsc, kc, ksc, vc, vsc, nkv, softmax_scale, pnq=True,
                                     p_rule=prule)[0, 0][rows]
        out[label] = float(torch.linalg.norm(o - ref) / torch.linalg.norm(ref))
    return out




def rowsum_decomposition(q, k, v, softmax_scale: float, p_rule="uos", rule="uos", hadamard: bool = True,
                         rows=None):
    """One head.  Replays the kernel's kv tiles for the given query rows from the
    dequantised operands (fp32 on the GPU), takes the kernel's own P^ dump, and splits
    sum_j (P^ - P~) -- the change of each row's normaliser that quantising P~ makes,
    rescaled to the final running max as the kernel rescales l -- by element class:
    zeroed (code 0 for P~ > 0), saturated (P~ / 2^e >= 7, which round-to-nearest would
    send to 8 and the format clips to 6), rounded down, rounded up.  Returns each class's
    share of the change as a mean fraction of l~ = sum P~ over the rows.  The P^ dump
    covers every row ([Nq, P/2] bytes), so keep N moderate (a few thousand tokens)."""
    import torch
    dev = q.device
    n, d = q.shape
    nkv = k.shape[0]
    rows = torch.arange(n, device=dev) if rows is None else torch.as_tensor(rows, device=dev)
    qc, qsc, kc, ksc, vc, vsc = _quantized_head(q, k, v, rule, hadamard)
    sh = lambda t: t.reshape(1, 1, *t.shape)
    _, pc, ps = mxattn_forward_quantized(*map(sh, (qc, qsc, kc, ksc, vc, vsc)), nkv, softmax_scale, pnq=True,
                                         p_rule=p_rule, dump_p=True)
    deq_last = _dequant_last

    qd = deq_last(qc[rows], qsc[rows])
    kd = deq_last(kc, ksc)
    P = mxattn_padded_tokens(nkv)
    s = (qd @ kd.t().contiguous()) * softmax_scale  # [R, Nkv] fp32
    s = torch.cat([s, torch.full((s.shape[0], P - nkv), -float("inf"), device=dev)], dim=1)
    bc = mxattn_kv_tile()
    m = torch.full((s.shape[0], 1), -float("inf"), device=dev)
    ptil = torch.empty_like(s)
    mt = torch.empty((s.shape[0], P // bc), device=dev)
    for j in range(P // bc):
        sl = slice(j * bc, (j + 1) * bc)
        m = torch.maximum(m, s[:, sl].max(dim=1, keepdim=True).values)
        ptil[:, sl] = torch.exp2((s[:, sl] - m) * 1.4426950408889634)
        mt[:, j] = m[:, 0]
    phat = deq_last(pc[0, 0][rows], ps[0, 0][rows])
    # rescale every tile to the final running max, as the kernel's running state is
    w = torch.exp2((mt - m) * 1.4426950408889634).repeat_interleave(bc, dim=1)
    scale_e = torch.pow(2.0, ps[0, 0][rows].float() - 127.0).repeat_interleave(32, dim=1)
    diff = (phat - ptil) * w
    zeroed = (phat == 0) & (ptil > 0)
    satur = (ptil / scale_e >= 7.0) & ~zeroed
    down = (diff < 0) & ~zeroed & ~satur
    up = diff > 0
    lt = (ptil * w).sum(dim=1)
    frac = lambda mask: float(((diff * mask).sum(dim=1) / lt).mean())
    return {"zeroed": frac(zeroed), "saturated": frac(satur), "rounded_down": frac(down), "rounded_up": frac(up),
            "total": float(((diff).sum(dim=1) / lt).mean()), "rows": int(rows.numel())}


GAMMAS = tuple(1.0 + i / 512 for i in range(256))  # 1.000, 1.002, ..., 1.498


def probabilities(q, k, v, softmax_scale: float, rows=None, rule="uos", hadamard: bool = True):
    """One head.  P = softmax(S) in fp32 for the given query rows, with S from the
    dequantised Q^ and K^ that the library's quantiser makes (the post-normalisation
    arm materialises P; this is that P).  Returns P [rows, Nkv] on the GPU."""
    import torch
    n = q.shape[0]
    rows = torch.arange(n, device=q.device) if rows is None else torch.as_tensor(rows, device=q.device)
    qc, qsc, kc, ksc, _, _ = _quantized_head(q, k, v, rule, hadamard)
    qd = _dequant_last(qc[rows], qsc[rows])
    kd = _dequant_last(kc, ksc)
    return torch.softmax((qd @ kd.t().contiguous()) * softmax_scale, dim=-1).contiguous()


def global_scaling_rowsums(P, p_rule="uos", gammas=GAMMAS):
    """P [rows, n] fp32 on the GPU.  For each g: y = g * P (fp32), block-quantised along
    each row by the library's quantiser, dequantised and summed per row in float64 (the
    factor stays in the weights: it compensates the average loss of quantisation).
    Returns a float64 tensor [len(gammas), rows]."""
    import torch
    rows, n = P.shape
    pad = -(-n // 32) * 32
    y = torch.zeros((rows, pad), dtype=torch.float32, device=P.device)
    out = torch.empty((len(gammas), rows), dtype=torch.float64, device=P.device)
    for i, g in enumerate(gammas):
        y[:, :n] = P * float(np.float32(g))
        c, s = mxattn_quantize(y, rule=p_rule, axis="last")
        out[i] = _dequant_last(c, s).double().sum(dim=1)
    return out


def global_scaling(P, p_rule="uos", gammas=GAMMAS):
    """Summary of global_scaling_rowsums: the g whose mean row sum is closest to one, and
    the mean, standard deviation and largest |row sum - 1| at g = 1 and at that g."""
    rs = global_scaling_rowsums(P, p_rule, gammas)
    mean = rs.mean(dim=1)
    best = int((mean - 1.0).abs().argmin())
    stats = lambda r: {"mean": float(r.mean()), "std": float(r.std()), "max_abs_dev": float((r - 1).abs().max())}
    return {"g_best": gammas[best], "at_g1": stats(rs[0]), "at_g_best": stats(rs[best]),
            "mean_curve": [round(float(x), 6) for x in mean]}


def main() -> None:
    """The diagnostics on the Wan2.2-720p-shaped synthetic tensors (one JSON line): the
    Qmax sweep of Q and K (rotated, along d) and V (along tokens) over all 40 heads, the
    P~-tile sweep on head 0 (1024 sampled query rows against exact attention), the row-sum
    decomposition on the first 8192 tokens of head 0 (512 rows), and the global-scaling arm
    on 256 rows of head 0's materialised P (all 75,600 keys)."""
    import json
    import torch
    import synth
    w = synth.WAN_720P
    dev = torch.device("cuda:0")
    q, k, v = (synth.device_attn_tensor(w, t, dev).view(-1, w.N, w.d) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
    res = {"workload": w.name}
    for name, x, axis, had in (("Q", q, "last", True), ("K", k, "last", True), ("V", v, "rows", False)):
        sw = qmax_sweep(x, axis=axis, hadamard=had)
        res[f"qmax_sweep_{name}"] = {"argmin_q": argmin_q(sw), "q7.25": sw["q7.25"]["rel_mse"],
                                     "q6.00": sw["q6.00"]["rel_mse"], "q7.00": sw["q7.00"]["rel_mse"],
                                     "q8.00": sw["q8.00"]["rel_mse"], "ocp": sw["ocp"]["rel_mse"],
                                     "curve": {kk: round(vv["rel_mse"], 7) for kk, vv in sw.items()}}
    rows = torch.linspace(0, w.N - 1, 1024, device=dev).long()
    ps = p_tile_sweep(q[0], k[0], v[0], float(w.softmax_scale), rows=rows)
    best = min((e, kk) for kk, e in ps.items() if kk.startswith("q"))
    res["p_tile_sweep"] = {"rows": 1024, "argmin_q": float(best[1][1:]), "q7.25": ps["q7.25"],
                           "ocp": ps["ocp"], "curve": {kk: round(vv, 6) for kk, vv in ps.items()}}
    n = 8192
    sub = lambda t: t[0, :n].contiguous()
    rrows = torch.linspace(0, n - 1, 512, device=dev).long()
    res["rowsum_decomposition"] = {
        r: rowsum_decomposition(sub(q), sub(k), sub(v), float(w.softmax_scale), p_rule=r, rule=r, rows=rrows)
        for r in ("uos", "ocp")}
    P = probabilities(q[0], k[0], v[0], float(w.softmax_scale), rows=torch.linspace(0, w.N - 1, 256, device=dev).long())
    res["global_scaling"] = {"rows": 256, **{r: global_scaling(P, p_rule=r) for r in ("uos", "ocp")}}
    del P
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
