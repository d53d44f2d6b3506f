"""Pins for oracle/hadamard.py: Sylvester structure, orthogonality, and the fp32
butterfly against the plain float64 definition x @ H / sqrt(d)."""
import math

import numpy as np
import pytest

from oracle import hadamard


@pytest.mark.parametrize("d", [32, 64, 128])
def test_sylvester_is_hadamard(d):
    H = hadamard.sylvester(d)
    assert (np.abs(H) == 1).all()
    assert (H @ H.T == d * np.eye(d, dtype=np.int64)).all()
    assert (H == H.T).all() and (H[0] == 1).all() and (H[:, 0] == 1).all()
    # Sylvester recursion H_2n = [[H, H], [H, -H]]
    h = d // 2
    Hh = hadamard.sylvester(h)
    assert (H[:h, :h] == Hh).all() and (H[:h, h:] == Hh).all() and (H[h:, h:] == -Hh).all()


def test_scaling_constants():
    assert hadamard.inv_sqrt_f32(64) == np.float32(0.125)
    assert hadamard.inv_sqrt_f32(128).view(np.uint32) == 0x3DB504F3


@pytest.mark.parametrize("d", [64, 128])
def test_unit_vectors_give_hadamard_rows(d):
    c = hadamard.inv_sqrt_f32(d)
    H = hadamard.sylvester(d)
    for j in (0, 1, d // 2 + 3, d - 1):
        x = np.zeros(d, np.float32)
        x[j] = 1.0
        y = hadamard.fwht_fp32(x)
        assert (y == (H[j].astype(np.float32) * c)).all()


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_butterfly_within_rounding_of_definition(d):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, d)).astype(np.float32)
    x[:, 5] *= 40.0
    y32 = hadamard.fwht_fp32(x).astype(np.float64)
    y64 = hadamard.rotate_f64(x)
    # each of log2(d) stages rounds once (<= 2^-24 of a partial sum of |x|), plus the
    # final multiply and the rounding of c: |err| <= (log2 d + 2) 2^-24 ||x||_1 / sqrt(d)
    bound = (math.log2(d) + 2) * 2.0 ** -24 * np.abs(x).sum(axis=1, dtype=np.float64) / math.sqrt(d)
    assert (np.abs(y32 - y64).max(axis=1) <= bound).all()
    # and it is not exact in general (so the fp32 definition matters)
    assert (y32 != y64).any()


def test_rotation_preserves_logits():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((64, 128)).astype(np.float32)
    k = rng.standard_normal((64, 128)).astype(np.float32)
    s_rot = hadamard.fwht_fp32(q).astype(np.float64) @ hadamard.fwht_fp32(k).astype(np.float64).T
    s = q.astype(np.float64) @ k.astype(np.float64).T
    assert np.abs(s_rot - s).max() < 1e-4 * np.abs(s).max()
    n = np.linalg.norm(q.astype(np.float64), axis=1)
    n_rot = np.linalg.norm(hadamard.fwht_fp32(q).astype(np.float64), axis=1)
    assert np.allclose(n, n_rot, rtol=1e-6)


def test_rotation_spreads_an_outlier_channel():
    # the reason for the rotation: a heavy channel is spread over all d outputs
    x = np.zeros((1, 128), np.float32)
    x[0, 17] = 100.0
    y = hadamard.fwht_fp32(x)
    assert np.allclose(np.abs(y), 100.0 / math.sqrt(128), rtol=1e-6)
