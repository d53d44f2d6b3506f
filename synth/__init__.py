"""Seeded synthetic inputs shaped like the video-DiT self-attention workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no arithmetic of the quantisation or attention method: it
only draws random tensors of the stated shapes and laws, and rounds fp32 to
bf16 (round-to-nearest-even on the bit pattern) when a workload is bf16.

Every (workload, tensor, head) has its own generator, seeded with
``[workload_seed, tensor_id, head]``, so one head can be regenerated alone
(tensor ids: Q=0, K=1, V=2, standalone quantiser input X=3).  Outlier
channels are drawn by a second generator seeded ``[workload_seed,
10 + tensor_id, head]``; Q and K draw theirs independently.

Shapes come from the latent grids of the two video models the MXAttention
paper evaluates (abstract; pith.science review, referee report summary):
Wan2.2 at 480p (21 latent frames x 30x52 patches) and 720p (21 x 45x80), and
HunyuanVideo at 720p (33 x 45x80 video tokens plus 256 text tokens).  The
value laws (Gaussian with a few heavy head-dim channels, which is what the
fixed Hadamard rotation targets) are this repository's stand-in for real
activations; the pages give no tensor statistics beyond that.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

Q_ID, K_ID, V_ID, X_ID = 0, 1, 2, 3


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    seed: int
    B: int
    H: int
    N: int            # N_q == N_kv for every self-attention workload here
    d: int
    dtype: str        # "f32" or "bf16"
    softmax_scale: float
    outlier_k: int    # number of outlier head-dim channels per head (Q and K)
    outlier_mult: float
    text_rows: int = 0        # trailing rows drawn N(0, text_sigma^2) for Q, K and V
    text_sigma: float = 1.0

    @property
    def flops(self) -> float:
        return 4.0 * self.B * self.H * self.N * self.N * self.d


@dataclass(frozen=True)
class QuantWorkload:
    name: str
    seed: int
    H: int
    N: int
    d: int
    dtype: str
    outlier_k: int
    outlier_mult: float
    spike_p: float
    spike_mult: float


TINY = AttnWorkload("tiny-h2-n256-d64", seed=0, B=1, H=2, N=256, d=64, dtype="f32",
                    softmax_scale=1.0 / 8.0, outlier_k=2, outlier_mult=20.0)
WAN_480P = AttnWorkload("wan2.2-480p-h40-n32760-d128", seed=2, B=1, H=40, N=32760, d=128,
                        dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
                        outlier_k=3, outlier_mult=16.0)
WAN_720P = AttnWorkload("wan2.2-720p-h40-n75600-d128", seed=3, B=1, H=40, N=75600, d=128,
                        dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
                        outlier_k=3, outlier_mult=16.0)
HUNYUAN_720P = AttnWorkload("hunyuanvideo-720p-h24-n119056-d128", seed=4, B=1, H=24, N=119056,
                            d=128, dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
                            outlier_k=3, outlier_mult=16.0, text_rows=256, text_sigma=2.0)
QUANT_720P = QuantWorkload("quantize-h40-n75600-d128", seed=5, H=40, N=75600, d=128, dtype="bf16",
                           outlier_k=3, outlier_mult=16.0, spike_p=1e-3, spike_mult=100.0)
# standalone quantiser check of the tiny workload: 4096 x 128 fp32 N(0,1)
TINY_QUANT = QuantWorkload("quantize-tiny-4096x128", seed=0, H=1, N=4096, d=128, dtype="f32",
                           outlier_k=0, outlier_mult=1.0, spike_p=0.0, spike_mult=1.0)

ATTN_WORKLOADS = {w.name: w for w in (TINY, WAN_480P, WAN_720P, HUNYUAN_720P)}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even on the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _head_gaussian(seed: int, tid: int, h: int, n: int, d: int) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, h])
    return rng.standard_normal((n, d), dtype=np.float32)


def outlier_channels(seed: int, tid: int, h: int, d: int, k: int) -> np.ndarray:
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    return np.random.default_rng([seed, 10 + tid, h]).choice(d, k, replace=False)


def attn_head(w: AttnWorkload, tid: int, h: int, b: int = 0) -> np.ndarray:
    """One head of Q (tid 0), K (1) or V (2) as fp32 values [N, d].

    For bf16 workloads the values are already bf16-representable (rounded RNE).
    Batch index b > 0 offsets the head seed by b * H.
    """
    hh = b * w.H + h
    x = _head_gaussian(w.seed, tid, hh, w.N, w.d)
    if tid in (Q_ID, K_ID) and w.outlier_k:
        ch = outlier_channels(w.seed, tid, hh, w.d, w.outlier_k)
        x[:, ch] *= np.float32(w.outlier_mult)
    if w.text_rows:
        t = w.text_rows
        rng = np.random.default_rng([w.seed, 20 + tid, hh])
        x[w.N - t:, :] = rng.standard_normal((t, w.d), dtype=np.float32) * np.float32(w.text_sigma)
    if w.dtype == "bf16":
        x = bf16_to_f32(round_to_bf16(x))
    return x


def attn_head_rows(w: AttnWorkload, tid: int, h: int, rows: np.ndarray, b: int = 0) -> np.ndarray:
    """Selected rows of one head (regenerates the head, then slices)."""
    return attn_head(w, tid, h, b)[np.asarray(rows)]


def attn_tensor(w: AttnWorkload, tid: int, heads=None, threads: int = 8) -> np.ndarray:
    """Q/K/V for all (or the listed) heads: fp32 [B, H', N, d]."""
    heads = list(range(w.H)) if heads is None else list(heads)
    out = np.empty((w.B, len(heads), w.N, w.d), dtype=np.float32)

    def fill(job):
        b, i, h = job
        out[b, i] = attn_head(w, tid, h, b)

    jobs = [(b, i, h) for b in range(w.B) for i, h in enumerate(heads)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, jobs))
    return out


def attn_tensor_bf16(w: AttnWorkload, tid: int, heads=None, threads: int = 8) -> np.ndarray:
    """Same as attn_tensor but as bf16 bit patterns (uint16), for device upload."""
    heads = list(range(w.H)) if heads is None else list(heads)
    out = np.empty((w.B, len(heads), w.N, w.d), dtype=np.uint16)

    def fill(job):
        b, i, h = job
        out[b, i] = round_to_bf16(attn_head(w, tid, h, b))

    jobs = [(b, i, h) for b in range(w.B) for i, h in enumerate(heads)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, jobs))
    return out


def quant_head(w: QuantWorkload, h: int) -> np.ndarray:
    """One head of the standalone quantiser input as fp32 values [N, d]."""
    x = _head_gaussian(w.seed, X_ID, h, w.N, w.d)
    if w.outlier_k:
        ch = outlier_channels(w.seed, X_ID, h, w.d, w.outlier_k)
        x[:, ch] *= np.float32(w.outlier_mult)
    if w.spike_p > 0:
        mask = np.random.default_rng([w.seed, 30 + X_ID, h]).random((w.N, w.d)) < w.spike_p
        x[mask] *= np.float32(w.spike_mult)
    if w.dtype == "bf16":
        x = bf16_to_f32(round_to_bf16(x))
    return x


def quant_tensor_bf16(w: QuantWorkload, heads=None, threads: int = 8) -> np.ndarray:
    heads = list(range(w.H)) if heads is None else list(heads)
    out = np.empty((len(heads), w.N, w.d), dtype=np.uint16)

    def fill(job):
        i, h = job
        out[i] = round_to_bf16(quant_head(w, h))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, list(enumerate(heads))))
    return out


def special_values_f32() -> np.ndarray:
    """Every bf16 bit pattern (65,536 values, as fp32) for exhaustive quantiser checks."""
    return bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))


# ---------------------------------------------------------------------------
# Device-side generators with the same laws, for full-size benchmark inputs
# (hundreds of millions of values).  They draw from torch's seeded device
# generator, so their values differ from the host generators above; the
# outlier channels are the same ones the host law picks.

def device_attn_tensor(w: AttnWorkload, tid: int, device="cuda"):
    import torch
    g = torch.Generator(device=device).manual_seed(1000 * w.seed + tid)
    x = torch.randn((w.B, w.H, w.N, w.d), generator=g, device=device, dtype=torch.float32)
    if tid in (Q_ID, K_ID) and w.outlier_k:
        for b in range(w.B):
            for h in range(w.H):
                ch = torch.from_numpy(outlier_channels(w.seed, tid, b * w.H + h, w.d, w.outlier_k)).to(device)
                x[b, h][:, ch] *= w.outlier_mult
    if w.text_rows:
        t = w.text_rows
        x[:, :, w.N - t:, :] = torch.randn((w.B, w.H, t, w.d), generator=g, device=device) * w.text_sigma
    return x.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)


def device_quant_tensor(w: QuantWorkload, device="cuda"):
    import torch
    g = torch.Generator(device=device).manual_seed(1000 * w.seed + X_ID)
    x = torch.randn((w.H, w.N, w.d), generator=g, device=device, dtype=torch.float32)
    for h in range(w.H):
        if w.outlier_k:
            ch = torch.from_numpy(outlier_channels(w.seed, X_ID, h, w.d, w.outlier_k)).to(device)
            x[h][:, ch] *= w.outlier_mult
    if w.spike_p > 0:
        spikes = torch.rand((w.H, w.N, w.d), generator=g, device=device) < w.spike_p
        x[spikes] *= w.spike_mult
    return x.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)
