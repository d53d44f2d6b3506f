"""MXFP4 attention forward with Pre-Normalization Quantization (CPU oracle; test infrastructure).

Sources (page titles and sections):
  * Pith review of MXAttention, Figure 4 caption: (A) standard attention forms
    the normalised P before O = P V; (B) FlashAttention keeps the running row
    sum l_i and the unnormalised accumulator O~_i, both updated from the same
    exponential tile P~_ij; (C) a direct placement updates l_i from the
    unquantised P~_ij but O~_i from the quantised P^_ij.  PNQ quantises P~_ij
    once and feeds that same tile to both updates.
  * Same review, Core claim and Axiom ledger (FlashAttention-2 online softmax:
    unnormalised accumulator and row sum, O = diag(l)^-1 O~, P never
    materialised); Referee summary (Proposition 1: the induced weights sum to
    one by construction); Figure 7 caption (quantising the normalised P makes
    the mean row sum fall below one).
  * Same review, Figure 1 caption: UOS applies to all MXFP4-quantised
    attention tensors; the Hadamard rotation is applied to Q/K only.
  * 10100.com explainer of MXAttention: PNQ quantises the not-yet-normalised
    exponentials first and uses that one result for both the normaliser and
    the output update.

Readings where the pages are silent:
  * Blocks run along the contraction axis: d for Q and K, tokens for V, kv
    for P~ (aligned to kv index 0).  Ragged tails are zero-padded; padded
    keys get P~ = 0.
  * S = softmax_scale * (Q^ K^^T): the scale multiplies the logits, Q is
    quantised unscaled.
  * kv tiles of width Bc (a multiple of 32) are visited in increasing order;
    P^ depends on Bc because the running max decides which values are
    quantised, so the caller passes the Bc the GPU uses.  Every tile rescales
    with the exact FA-2 rule (no conditional or lazy rescaling).
  * P~ uses the same scale rule as Q/K/V.  P~ = exp(S - m') is evaluated in
    float64 and rounded once to fp32 before its block max and codes are
    decided, since fp32 is the precision the kernel decides them in.
  * pnq=False is the direct placement of Figure 4(C): l sums the unquantised
    P~ (the same fp32-rounded values), O~ uses P^.
  * The non-flash post-normalisation arm (Figure 4(A) with a quantised P) is
    `postnorm_attention`, a diagnostic only.
"""
from __future__ import annotations

import numpy as np

from . import hadamard, mxfp4


def exact_attention(Q, K, V, softmax_scale: float) -> np.ndarray:
    """Textbook softmax attention in float64: softmax(scale Q K^T) V (per leading index)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S = softmax_scale * (Q @ np.swapaxes(K, -1, -2))
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=-1, keepdims=True)
    return P @ V


def flash_attention_f64(Q, K, V, softmax_scale: float, Bc: int) -> np.ndarray:
    """FlashAttention-2 online softmax in float64 with no quantisation (pins the recurrence)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Nq, Nkv = Q.shape[-2], K.shape[-2]
    m = np.full(Q.shape[:-1], -np.inf)
    l = np.zeros(Q.shape[:-1])
    O = np.zeros(Q.shape[:-1] + (V.shape[-1],))
    for j0 in range(0, Nkv, Bc):
        S = softmax_scale * (Q @ np.swapaxes(K[..., j0:j0 + Bc, :], -1, -2))
        m_new = np.maximum(m, S.max(axis=-1))
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        P = np.exp(S - m_new[..., None])
        l = alpha * l + P.sum(axis=-1)
        O = alpha[..., None] * O + P @ V[..., j0:j0 + Bc, :]
        m = m_new
    return O / l[..., None]


def quantize_qk(x, rule, hadamard_on: bool):
    """Q or K [..., N, d]: optional fp32 Hadamard, then blocks along d.

    Returns (codes [..., N, d] one code per element, scales [..., N, d/32])."""
    x32 = np.asarray(x, dtype=np.float32)
    y = hadamard.fwht_fp32(x32) if hadamard_on else x32
    return mxfp4.quantize_blocks_lastaxis(y, rule)


def quantize_v(v, rule, pad_to: int):
    """V [..., N, d] -> V^T codes [..., d, Np] and scales [..., d, Np/32], blocks along tokens."""
    return mxfp4.quantize_rows_transposed(np.asarray(v, dtype=np.float32), rule, pad_to=pad_to)


def flash_attention_mx(Qc, Qs, Kc, Ks, VTc, VTs, Nkv: int, softmax_scale: float,
                       pnq: bool, p_rule, Bc: int, rows=None, return_p: bool = False):
    """Online-softmax attention on MXFP4 operands for one head.

    Qc [Nq, d] codes + Qs [Nq, d/32]; Kc [>=Nkv, d] + Ks; VTc [d, Np] + VTs
    [d, Np/32] (Np >= Nkv, multiple of 32).  `rows` selects query rows (each
    row's recurrence is independent of the others).  Returns O [rows, d] in
    float64 and, if asked, the P^ codes [rows, Np_bc] and scales
    [rows, Np_bc/32] of every tile, Np_bc being Nkv rounded up to Bc.
    """
    if Bc % mxfp4.BLOCK:
        raise ValueError("Bc must be a multiple of 32")
    Qd = mxfp4.dequantize_blocks_lastaxis(Qc, Qs)
    Kd = mxfp4.dequantize_blocks_lastaxis(Kc, Ks)[:Nkv]
    VT = mxfp4.dequantize_blocks_lastaxis(VTc, VTs)
    V = VT.T[:Nkv]
    if rows is not None:
        Qd = Qd[np.asarray(rows)]
    nr, d = Qd.shape
    n_tiles = -(-Nkv // Bc)
    m = np.full(nr, -np.inf)
    l = np.zeros(nr)
    O = np.zeros((nr, V.shape[1]))
    if return_p:
        pc_all = np.zeros((nr, n_tiles * Bc), dtype=np.uint8)
        ps_all = np.zeros((nr, n_tiles * Bc // mxfp4.BLOCK), dtype=np.uint8)
    for t in range(n_tiles):
        j0, j1 = t * Bc, min((t + 1) * Bc, Nkv)
        S = softmax_scale * (Qd @ Kd[j0:j1].T)                      # [nr, <=Bc] float64
        m_new = np.maximum(m, S.max(axis=1))
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        P = np.zeros((nr, Bc), dtype=np.float32)                   # padded keys: P~ = 0
        P[:, : j1 - j0] = np.exp(S - m_new[:, None]).astype(np.float32)
        pc, ps = mxfp4.quantize_blocks_lastaxis(P, p_rule)
        P_hat = mxfp4.dequantize_blocks_lastaxis(pc, ps)
        row_sum = P_hat.sum(axis=1) if pnq else P.astype(np.float64).sum(axis=1)
        l = alpha * l + row_sum
        O = alpha[:, None] * O + P_hat[:, : j1 - j0] @ V[j0:j1]
        m = m_new
        if return_p:
            pc_all[:, j0: j0 + Bc] = pc
            ps_all[:, j0 // mxfp4.BLOCK: (j0 + Bc) // mxfp4.BLOCK] = ps
    O = O / l[:, None]
    if return_p:
        return O, pc_all, ps_all
    return O


def postnorm_attention(Qc, Qs, Kc, Ks, VTc, VTs, Nkv: int, softmax_scale: float, p_rule,
                       rows=None):
    """Diagnostic arm: materialise P = softmax(S) in float64, quantise P in 32-kv blocks,
    O = P^ V^ (Figure 4(A) with a quantised P).  Returns (O, row sums of P^)."""
    Qd = mxfp4.dequantize_blocks_lastaxis(Qc, Qs)
    Kd = mxfp4.dequantize_blocks_lastaxis(Kc, Ks)[:Nkv]
    V = mxfp4.dequantize_blocks_lastaxis(VTc, VTs).T[:Nkv]
    if rows is not None:
        Qd = Qd[np.asarray(rows)]
    S = softmax_scale * (Qd @ Kd.T)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=1, keepdims=True)
    pc, ps = mxfp4.quantize_blocks_lastaxis(P, p_rule)
    P_hat = mxfp4.dequantize_blocks_lastaxis(pc, ps)[:, :Nkv]
    return P_hat @ V, P_hat.sum(axis=1)


def mx_attention_pipeline(Q, K, V, softmax_scale: float, hadamard_on: bool, pnq: bool, rule,
                          Bc: int, v_pad: int, rows=None, return_p: bool = False):
    """The whole path for one head: rotate + quantise Q and K along d, quantise V along
    tokens, then flash_attention_mx.  Q [Nq, d], K and V [Nkv, d] (fp32 values)."""
    Qc, Qs = quantize_qk(Q, rule, hadamard_on)
    Kc, Ks = quantize_qk(K, rule, hadamard_on)
    VTc, VTs = quantize_v(V, rule, v_pad)
    return flash_attention_mx(Qc, Qs, Kc, Ks, VTc, VTs, np.asarray(K).shape[0], softmax_scale,
                              pnq, rule, Bc, rows=rows, return_p=return_p)
