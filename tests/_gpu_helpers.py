"""Helpers for the GPU parity tests: device upload, oracle comparison metrics."""
from __future__ import annotations

import numpy as np

import synth
from oracle import mxfp4


def require_gpu():
    import pytest
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_bit_attention_amd as mx  # raises if the library is not built
    return torch, mx


def to_device(x: np.ndarray, dtype: str):
    """fp32 numpy values -> a device tensor of dtype 'f32' or 'bf16' (bf16 values must be representable)."""
    import torch
    if dtype == "bf16":
        x32 = np.ascontiguousarray(x, dtype=np.float32)
        bits = synth.round_to_bf16(x32)
        same = synth.bf16_to_f32(bits).view(np.uint32) == x32.view(np.uint32)
        assert same.all(), "values are not bf16-representable"
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def u8(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.uint8)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def p_code_mismatch(gpu_pc_packed: np.ndarray, gpu_ps: np.ndarray, ora_pc: np.ndarray, ora_ps: np.ndarray,
                    nkv: int):
    """Fraction of the P^ codes of the first nkv keys that differ, a changed block
    exponent counting as all of that block's codes among those keys.  Keys past nkv
    (padding, code 0 on both sides) are left out of numerator and denominator alike."""
    g = mxfp4.unpack_nibbles(gpu_pc_packed)
    n = g.shape[-1]
    assert ora_pc.shape[-1] == n and 0 < nkv <= n
    nb = -(-nkv // 32)
    gb = g[..., : nb * 32].reshape(g.shape[:-1] + (nb, 32))
    ob = ora_pc[..., : nb * 32].reshape(ora_pc.shape[:-1] + (nb, 32))
    real = np.minimum(32, nkv - 32 * np.arange(nb))            # real keys in each block
    keep = np.arange(32)[None, :] < real[:, None]               # [nb, 32]
    scale_diff = gpu_ps[..., :nb] != ora_ps[..., :nb]
    code_diff = ((gb != ob) & keep).sum(axis=-1)
    bad = np.where(scale_diff, real, code_diff).sum()
    return float(bad) / (np.prod(g.shape[:-1]) * nkv)


RULES = {"uos": ("uos", mxfp4.UOS), "ocp": ("ocp", mxfp4.OCP), "tfs": (("ceil", 6.0), mxfp4.TFS),
         "oas": (("ceil", 7.0), mxfp4.OAS), "q7.5": (("ceil", 7.5), ("ceil", 7.5))}
