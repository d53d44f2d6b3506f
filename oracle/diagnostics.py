"""Oracle of the scale-rule diagnostics (test infrastructure only, like all of oracle/).

quant_rel_mse         relative MSE of MXFP4 block quantisation of a tensor under a rule:
                      sum (x - dequant(quant(x)))^2 / sum x^2, float64, over finite blocks.
rowsum_decomposition  replays the PNQ online softmax of one head (the tile recurrence of
                      attention.flash_attention_mx) and splits sum (P^ - P~), rescaled to
                      the final running max like the normaliser l, by element class:
                      zeroed (code 0 for P~ > 0), saturated (P~ / 2^e >= 7: round-to-
                      nearest heads for 8 and the format clips to 6), rounded down,
                      rounded up; each as a mean fraction of l~ = sum P~ over the rows.
global_scaling_rowsums  the post-normalisation arm with pre-quantisation global scaling:
                      the materialised probabilities P (fp32) are multiplied by one scalar
                      g and quantised in 32-key blocks; returns the row sums of the
                      dequantised tile for each g (Pith review, Figure 7 caption, panel C:
                      such a global factor can bring the *average* row sum back to one,
                      which leaves each row's own error in place).

The question they answer is the one the Pith review's referee report raises: the UOS
constant is derived for a model density of block maxima, and per-block Qmax sweeps on
real tensors, P~ tiles included, are not shown (Referee Report, major comments; the
explainer's account of why the softmax tile's normaliser drifts).
"""
from __future__ import annotations

import numpy as np

from . import hadamard, mxfp4


def quant_rel_mse(x, rule, axis: str = "last", hadamard_on: bool = False):
    """x [..., rows, cols] fp32 values.  axis 'last': blocks along cols (after the fp32
    Hadamard rotation when asked); axis 'rows': blocks down the rows of each [rows, cols]
    slice, zero-padded.  Returns (sum of squared errors, sum of squares, non-finite blocks)."""
    x = np.asarray(x, dtype=np.float32)
    if axis == "last":
        y = hadamard.fwht_fp32(x) if hadamard_on else x
        codes, scales = mxfp4.quantize_blocks_lastaxis(y, rule)
        deq = mxfp4.dequantize_blocks_lastaxis(codes, scales)
        ref = y.astype(np.float64)
        blocks_ok = np.repeat(scales != 0xFF, mxfp4.BLOCK, axis=-1)
        nonfinite = int((scales == 0xFF).sum())
    elif axis == "rows":
        if hadamard_on:
            raise ValueError("the rows axis takes no rotation")
        xt = np.swapaxes(x, -1, -2)                      # [..., cols, rows]
        pad = -(-xt.shape[-1] // mxfp4.BLOCK) * mxfp4.BLOCK
        xp = np.zeros(xt.shape[:-1] + (pad,), dtype=np.float32)
        xp[..., : xt.shape[-1]] = xt
        codes, scales = mxfp4.quantize_blocks_lastaxis(xp, rule)
        deq = mxfp4.dequantize_blocks_lastaxis(codes, scales)
        ref = xp.astype(np.float64)
        blocks_ok = np.repeat(scales != 0xFF, mxfp4.BLOCK, axis=-1)
        nonfinite = int((scales == 0xFF).sum())
    else:
        raise ValueError("axis must be 'last' or 'rows'")
    err = np.where(blocks_ok, ref - deq, 0.0)
    sq = np.where(blocks_ok, ref, 0.0)
    return float((err * err).sum()), float((sq * sq).sum()), nonfinite


def rowsum_decomposition(Qc, Qs, Kc, Ks, Nkv: int, softmax_scale: float, p_rule, Bc: int):
    """One head, MXFP4 operands as in attention.flash_attention_mx.  Returns the mean
    fractions {zeroed, saturated, rounded_down, rounded_up, total} of sum (P^ - P~)
    relative to l~ = sum P~, both rescaled to the final running max of each row."""
    Qd = mxfp4.dequantize_blocks_lastaxis(Qc, Qs)
    Kd = mxfp4.dequantize_blocks_lastaxis(Kc, Ks)[:Nkv]
    nr = Qd.shape[0]
    n_tiles = -(-Nkv // Bc)
    m = np.full(nr, -np.inf)
    classes = ("zeroed", "saturated", "rounded_down", "rounded_up")
    acc = {c: np.zeros(nr) for c in classes}
    lt = np.zeros(nr)
    for t in range(n_tiles):
        j0, j1 = t * Bc, min((t + 1) * Bc, Nkv)
        S = softmax_scale * (Qd @ Kd[j0:j1].T)
        m_new = np.maximum(m, S.max(axis=1))
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        P = np.zeros((nr, Bc), dtype=np.float32)
        P[:, : j1 - j0] = np.exp(S - m_new[:, None]).astype(np.float32)
        pc, ps = mxfp4.quantize_blocks_lastaxis(P, p_rule)
        P_hat = mxfp4.dequantize_blocks_lastaxis(pc, ps)
        Pd = P.astype(np.float64)
        diff = P_hat - Pd
        scaled = Pd / np.repeat(np.exp2(ps.astype(np.float64) - 127.0), mxfp4.BLOCK, axis=1)
        zeroed = (P_hat == 0) & (Pd > 0)
        satur = (scaled >= 7.0) & ~zeroed
        down = (diff < 0) & ~zeroed & ~satur
        up = diff > 0
        for c, mask in zip(classes, (zeroed, satur, down, up)):
            acc[c] = alpha * acc[c] + (diff * mask).sum(axis=1)
        lt = alpha * lt + Pd.sum(axis=1)
        m = m_new
    out = {c: float((acc[c] / lt).mean()) for c in classes}
    out["total"] = float((sum(acc[c] for c in classes) / lt).mean())
    return out


def global_scaling_rowsums(P, p_rule, gammas):
    """P [rows, n] fp32 probabilities (each row a softmax).  For every g in gammas:
    y = fl32(g * P) (one IEEE fp32 multiply), quantised in 32-key blocks along each row
    under p_rule and dequantised (exact in float64).  Returns the float64 row sums
    [len(gammas), rows] of the dequantised y: the factor is a compensation that stays in
    the weights, chosen to pull the average row sum of the quantised tile back to one."""
    P = np.asarray(P, dtype=np.float32)
    out = np.empty((len(gammas), P.shape[0]), dtype=np.float64)
    for i, g in enumerate(gammas):
        y = (np.float32(g) * P).astype(np.float32)
        codes, scales = mxfp4.quantize_blocks_lastaxis(y, p_rule)
        out[i] = mxfp4.dequantize_blocks_lastaxis(codes, scales)[:, : P.shape[1]].sum(axis=1)
    return out
