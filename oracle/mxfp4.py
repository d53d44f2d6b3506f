"""MXFP4 number format and block quantiser (CPU oracle; test infrastructure).

Sources (the pages' titles and sections):
  * Pith review of "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
    Quantization for MXFP4 Attention", Axiom & Free-Parameter Ledger, axiom 1:
    32-element blocks, one shared E8M0 power-of-two scale, E2M1 elements on the
    grid {0, +-0.5, ..., +-6}, round-to-nearest with saturation.
  * Same review, Figure 3 caption: the OCP floor rule maps block maxima to
    [4, 8); TFS uses (3, 6]; UOS uses (3.625, 7.25].  Referee minor comment 6:
    e_elem^max = 2 is the exponent of the grid value 4 (Eq. 11).
  * Same review, Core claim / What carries the argument: UOS is the
    ceiling-based power-of-two rule with boundary Qmax = 7.25.
  * Same review, Figure 2 caption and Appendix G fragment (Eq. 96): the ceiling
    rule with q = 7 (OAS) against q = 6 (TFS).
  * 10100.com explainer of MXAttention: 32 elements per group share one E8M0
    factor; E2M1 max finite value is 6; under OCP a scaled max above 7 rounds
    towards the unrepresentable 8 and saturates to 6; UOS only changes how the
    shared factor is chosen.
  * Appendix A opening (Pith review, end of the reference list): the all-zero
    block and out-of-range exponents are left to the MXFP4 conversion routine.

Readings taken where the pages are silent:
  * Grid {0, .5, 1, 1.5, 2, 3, 4, 6}; code = sign << 3 | magnitude index
    (the OCP E2M1 bit layout, where the index is the magnitude's rank).
  * Rounding: nearest grid point; a tie goes to the even code.  Values above
    the grid saturate to 6 (their nearest grid point).
  * The code's sign bit is the sign bit of the value (so -0.0 and small
    negatives that round to zero give 0x8).
  * CEIL(q): e is the smallest integer with M <= q * 2**e.  OCP: e =
    floor(log2 M) - 2.  M = 0 gives e = -127.  e is clamped to [-127, 127].
    A block holding Inf or NaN gets E8M0 0xFF and all codes 0.
  * E8M0 byte = e + 127 (value 2**e).
  * Two codes per byte, the even element in the low nibble.

Everything here is plain NumPy in float64 on exactly representable values: the
scaling by 2**-e is exact in float64, and rounding is a brute nearest-point
search over the eight grid magnitudes.
"""
from __future__ import annotations

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
BLOCK = 32
E8M0_NAN = 0xFF
E_MIN, E_MAX = -127, 127

# Rule descriptors: ("ocp", None) or ("ceil", q).
UOS = ("ceil", 7.25)
TFS = ("ceil", 6.0)
OAS = ("ceil", 7.0)
OCP = ("ocp", None)


def rule_ceil(q: float):
    return ("ceil", float(q))


def e2m1_encode(v) -> np.ndarray:
    """Round already-scaled values to E2M1 codes (uint8 in 0..15).

    Nearest of the eight grid magnitudes; ties to the even code; the sign bit
    copies the sign bit of v.  NaN is not accepted here (the block quantiser
    handles non-finite blocks before calling this).
    """
    v = np.asarray(v, dtype=np.float64)
    # Saturation: every magnitude above 6 has 6 as its nearest grid point.  Clamping
    # to 7 first keeps the distances meaningful for huge values (at 1e30 all eight
    # float64 distances would be equal).
    a = np.minimum(np.abs(v), 7.0)
    dist = np.abs(a[..., None] - E2M1_GRID)          # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                # one, or two adjacent codes on a tie
    n_cand = cand.sum(axis=-1)
    first = np.argmax(cand, axis=-1)                   # lowest candidate code
    # on a tie the two candidates are `first` and `first + 1`; keep the even one
    mag = np.where((n_cand > 1) & (first % 2 == 1), first + 1, first)
    sign = np.signbit(v).astype(np.uint8)
    return (sign << 3 | mag.astype(np.uint8)).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def scale_exponent(M, rule) -> np.ndarray:
    """Shared exponent e for block maxima M (non-negative finite float64 values).

    ("ceil", q): the smallest integer e with M <= q * 2**e, so M / 2**e lies in
    (q/2, q].  ("ocp", None): e = floor(log2 M) - 2, so M / 2**e lies in [4, 8).
    M == 0 gives -127; the result is clamped to [-127, 127].
    """
    M = np.asarray(M, dtype=np.float64)
    kind, q = rule
    pos = M > 0
    Ms = np.where(pos, M, 1.0)
    if kind == "ocp":
        _, E = np.frexp(Ms)                  # Ms = f * 2**E, f in [0.5, 1)  =>  floor(log2 Ms) = E - 1
        e = (E - 1) - 2
    elif kind == "ceil":
        if not (q > 0):
            raise ValueError("ceil rule needs q > 0")
        e = np.ceil(np.log2(Ms / q)).astype(np.int64)
        # make it exact: smallest e with Ms <= q * 2**e (ldexp is exact here)
        for _ in range(3):
            e = np.where(Ms > np.ldexp(q, e), e + 1, e)
        for _ in range(3):
            e = np.where(Ms <= np.ldexp(q, e - 1), e - 1, e)
    else:
        raise ValueError(f"unknown rule {rule!r}")
    e = np.where(pos, e, E_MIN)
    return np.clip(e, E_MIN, E_MAX).astype(np.int64)


def quantize_blocks_lastaxis(x, rule):
    """Quantise x[..., n] (fp32 or fp64 values) in 32-element blocks along the last axis.

    The last axis is zero-padded to a multiple of 32 (zeros never change a
    block max).  Returns (codes uint8 [..., n_pad] one code per element,
    scales uint8 [..., n_pad / 32] E8M0 bytes).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    n_pad = -(-n // BLOCK) * BLOCK
    if n_pad != n:
        pad = [(0, 0)] * (x.ndim - 1) + [(0, n_pad - n)]
        x = np.pad(x, pad)
    blocks = x.reshape(x.shape[:-1] + (n_pad // BLOCK, BLOCK))
    finite = np.isfinite(blocks).all(axis=-1)
    M = np.where(finite, np.abs(np.where(np.isfinite(blocks), blocks, 0.0)).max(axis=-1), 0.0)
    e = scale_exponent(M, rule)
    scaled = np.ldexp(np.where(np.isfinite(blocks), blocks, 0.0), -e[..., None])
    codes = e2m1_encode(scaled)
    codes = np.where(finite[..., None], codes, 0).astype(np.uint8)
    scales = np.where(finite, e + 127, E8M0_NAN).astype(np.uint8)
    return codes.reshape(x.shape[:-1] + (n_pad,)), scales


def dequantize_blocks_lastaxis(codes, scales) -> np.ndarray:
    """Inverse of quantize_blocks_lastaxis (0xFF scales give NaN)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    n = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    s = np.where(scales == E8M0_NAN, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    return (vals * s[..., None]).reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """[..., n] codes (n even) -> [..., n/2] bytes, even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def quantize_rows_transposed(x, rule, pad_to: int = BLOCK):
    """Quantise x[..., N, C] in 32-row blocks down each column (the token axis).

    Returns codes [..., C, Np] and scales [..., C, Np/32], where Np is N
    rounded up to a multiple of `pad_to` (a multiple of 32) and the padding
    rows are zeros, so every block past the data has M = 0 (E8M0 0x00).
    """
    if pad_to % BLOCK:
        raise ValueError("pad_to must be a multiple of 32")
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[-2]
    Np = -(-N // pad_to) * pad_to
    xt = np.swapaxes(x, -1, -2)
    if Np != N:
        pad = [(0, 0)] * (xt.ndim - 1) + [(0, Np - N)]
        xt = np.pad(xt, pad)
    return quantize_blocks_lastaxis(xt, rule)
