"""The seeded input generators: shapes, laws, determinism, bf16 representability."""
import numpy as np

import synth


def test_workload_shapes_and_flops():
    assert synth.WAN_720P.N == 21 * 45 * 80 and synth.WAN_480P.N == 21 * 30 * 52
    assert synth.HUNYUAN_720P.N == 33 * 45 * 80 + 256
    assert synth.WAN_720P.flops == 4 * 40 * 75600 ** 2 * 128


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38], np.float32)
    b = synth.round_to_bf16(x)
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0                 # tie -> even
    assert back[2] == np.float32(1.0 + 2 ** -7)              # 1.5 ulp -> up
    assert back[3] == -2.5
    allb = synth.special_values_f32()
    assert (synth.round_to_bf16(allb[np.isfinite(allb)]) == np.arange(65536)[np.isfinite(allb)]).all()


def test_heads_deterministic_and_independent():
    w = synth.TINY
    a = synth.attn_head(w, synth.Q_ID, 1)
    b = synth.attn_head(w, synth.Q_ID, 1)
    c = synth.attn_head(w, synth.K_ID, 1)
    assert (a == b).all() and not (a == c).all()
    full = synth.attn_tensor(w, synth.Q_ID)
    assert full.shape == (1, 2, 256, 64) and (full[0, 1] == a).all()


def test_outlier_law():
    w = synth.WAN_480P
    q = synth.attn_head(w, synth.Q_ID, 3)
    assert (synth.bf16_to_f32(synth.round_to_bf16(q)) == q).all()
    ch = synth.outlier_channels(w.seed, synth.Q_ID, 3, w.d, w.outlier_k)
    std = q.std(axis=0)
    assert len(ch) == 3 and np.allclose(std[ch], 16.0, rtol=0.05)
    rest = np.setdiff1d(np.arange(w.d), ch)
    assert np.allclose(std[rest], 1.0, rtol=0.05)
    # K draws its channels from its own generator
    kch = synth.outlier_channels(w.seed, synth.K_ID, 3, w.d, w.outlier_k)
    assert len(kch) == 3 and len(set(kch)) == 3


def test_text_rows_and_spikes():
    w = synth.HUNYUAN_720P
    import dataclasses
    small = dataclasses.replace(w, N=2048)
    v = synth.attn_head(small, synth.V_ID, 0)
    assert np.allclose(v[-256:].std(), 2.0, rtol=0.05) and np.allclose(v[:-256].std(), 1.0, rtol=0.05)
    qw = dataclasses.replace(synth.QUANT_720P, N=4096)
    x = synth.quant_head(qw, 0)
    assert np.abs(x).max() > 100
