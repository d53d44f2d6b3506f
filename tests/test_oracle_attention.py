"""Pins for oracle/attention.py.

* FA-2 exactness: with quantisation off, the online-softmax recurrence equals
  textbook softmax attention for any tile width.
* Proposition 1 (PNQ): induced weights sum to one, so V = 1 gives O = 1, and
  any V whose rows are all equal gives exactly that row.
* Direct placement (Figure 4(C)) and post-normalisation (Figure 4(A), Figure
  7(A)) visibly break the sum-to-one property.
* Convexity: with PNQ, O is a convex combination of the dequantised V rows.
* Single tile: at Bc >= N_kv the running max is the global max.
* Structural invariants: row independence, scale equivariance.
"""
import numpy as np
import pytest

import synth
from oracle import attention, hadamard, mxfp4

RULES = {"uos": mxfp4.UOS, "ocp": mxfp4.OCP, "tfs": mxfp4.TFS}


def _tiny_inputs(h=0):
    w = synth.TINY
    return (synth.attn_head(w, synth.Q_ID, h), synth.attn_head(w, synth.K_ID, h),
            synth.attn_head(w, synth.V_ID, h), w)


@pytest.mark.parametrize("Bc", [32, 64, 100, 256, 1000])
def test_flash_recurrence_equals_softmax_attention(Bc):
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((3, 50, 64)) * 2.0
    K = rng.standard_normal((3, 300, 64)) * 2.0
    V = rng.standard_normal((3, 300, 64))
    O1 = attention.flash_attention_f64(Q, K, V, 0.125, Bc)
    O2 = attention.exact_attention(Q, K, V, 0.125)
    assert np.abs(O1 - O2).max() < 1e-12


def _quantized(Q, K, V, rule, had, v_pad=128):
    Qc, Qs = attention.quantize_qk(Q, rule, had)
    Kc, Ks = attention.quantize_qk(K, rule, had)
    Vc, Vs = attention.quantize_v(V, rule, v_pad)
    return Qc, Qs, Kc, Ks, Vc, Vs


@pytest.mark.parametrize("rule", list(RULES))
@pytest.mark.parametrize("Bc", [32, 128])
def test_pnq_rows_sum_to_one(rule, Bc):
    Q, K, V, w = _tiny_inputs()
    ones = np.ones_like(V)
    q = _quantized(Q, K, ones, RULES[rule], True)
    assert (mxfp4.dequantize_blocks_lastaxis(q[4], q[5])[:, : w.N] == 1.0).all()   # V^ = 1 exactly
    O = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, RULES[rule], Bc)
    assert np.abs(O - 1.0).max() < 1e-12
    Od = attention.flash_attention_mx(*q, w.N, w.softmax_scale, False, RULES[rule], Bc)
    assert np.abs(Od - 1.0).max() > 1e-2                       # direct placement: rows do not sum to one
    _, rs = attention.postnorm_attention(*q, w.N, w.softmax_scale, RULES[rule])
    assert rs.mean() < 1.0                                     # Figure 7(A): mean row sum below one


def test_pnq_constant_rows_are_reproduced_exactly():
    Q, K, _, w = _tiny_inputs(1)
    v_row = np.array([mxfp4.E2M1_GRID[i % 8] * 2.0 ** (i % 5 - 2) * (-1) ** i for i in range(w.d)])
    V = np.tile(v_row, (w.N, 1))
    q = _quantized(Q, K, V, mxfp4.UOS, True)
    O = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.UOS, 64)
    assert np.abs(O - v_row).max() < 1e-12


def test_pnq_output_is_convex_combination():
    Q, K, V, w = _tiny_inputs()
    q = _quantized(Q, K, V, mxfp4.UOS, True)
    O = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.UOS, 64)
    Vd = mxfp4.dequantize_blocks_lastaxis(q[4], q[5]).T[: w.N]
    assert (O <= Vd.max(axis=0) + 1e-12).all() and (O >= Vd.min(axis=0) - 1e-12).all()


def test_single_tile_uses_global_max():
    Q, K, V, w = _tiny_inputs()
    q = _quantized(Q, K, V, mxfp4.UOS, True)
    O, pc, ps = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.UOS, 256,
                                             return_p=True)
    # with one tile, the row max of P~ is exactly 1, and under UOS a block holding
    # P~ = 1 gets the scale 2^-2 (1 / 2^-2 = 4 <= 7.25 < 8)
    Qd = mxfp4.dequantize_blocks_lastaxis(q[0], q[1])
    Kd = mxfp4.dequantize_blocks_lastaxis(q[2], q[3])
    S = w.softmax_scale * Qd @ Kd.T
    jmax = S.argmax(axis=1)
    blk_scale = ps[np.arange(w.N), jmax // 32]
    assert (blk_scale == 127 - 2).all()
    assert (pc[np.arange(w.N), jmax] == 6).all()               # 1 * 4 = 4 -> code 6


def test_on_grid_operands_quantise_exactly():
    # operands already on the E2M1 grid (times a power of two) re-quantise exactly under
    # UOS, so the only error left in O is that of P^ (a sanity bound on its size)
    rng = np.random.default_rng(9)
    g = mxfp4.E2M1_GRID
    Qv = rng.choice(np.concatenate([g, -g]), (64, 64)) * 0.25
    Kv = rng.choice(np.concatenate([g, -g]), (128, 64)) * 0.25
    Vv = rng.choice(np.concatenate([g, -g]), (128, 64))
    q = _quantized(Qv, Kv, Vv, mxfp4.UOS, False)
    Qd = mxfp4.dequantize_blocks_lastaxis(q[0], q[1])
    assert (Qd == Qv).all()
    O = attention.flash_attention_mx(*q, 128, 0.125, True, mxfp4.UOS, 64)
    Kd = mxfp4.dequantize_blocks_lastaxis(q[2], q[3])
    Vd = mxfp4.dequantize_blocks_lastaxis(q[4], q[5]).T[:128]
    assert (Kd == Kv).all() and (Vd == Vv).all()
    Oe = attention.exact_attention(Qd, Kd, Vd, 0.125)
    rel = np.linalg.norm(O - Oe) / np.linalg.norm(Oe)
    assert 0 < rel < 0.5


def test_rows_are_independent_and_selectable():
    Q, K, V, w = _tiny_inputs()
    q = _quantized(Q, K, V, mxfp4.OCP, False)
    O = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.OCP, 64)
    rows = np.array([255, 3, 100])
    Or = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.OCP, 64, rows=rows)
    assert (Or == O[rows]).all()
    perm = np.random.default_rng(0).permutation(w.N)
    Op = attention.flash_attention_mx(q[0][perm], q[1][perm], *q[2:], w.N, w.softmax_scale, True,
                                      mxfp4.OCP, 64)
    assert (Op == O[perm]).all()


def test_scale_equivariance():
    # doubling Q only moves its E8M0 scales; halving softmax_scale undoes it exactly
    Q, K, V, w = _tiny_inputs()
    q = _quantized(Q, K, V, mxfp4.UOS, True)
    q2 = _quantized(2 * Q, K, V, mxfp4.UOS, True)
    assert (q2[0] == q[0]).all() and (q2[1] == q[1] + 1).all()
    O = attention.flash_attention_mx(*q, w.N, w.softmax_scale, True, mxfp4.UOS, 64)
    O2 = attention.flash_attention_mx(*q2, w.N, w.softmax_scale / 2, True, mxfp4.UOS, 64)
    assert np.abs(O - O2).max() < 1e-13


def test_ragged_kv_tail_padded_keys_are_ignored():
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((40, 64)).astype(np.float32)
    K = rng.standard_normal((200, 64)).astype(np.float32)
    V = rng.standard_normal((200, 64)).astype(np.float32)
    q = _quantized(Q, K, V, mxfp4.UOS, True, v_pad=256)
    O, pc, ps = attention.flash_attention_mx(*q, 200, 0.125, True, mxfp4.UOS, 128, return_p=True)
    assert pc.shape == (40, 256) and (pc[:, 200:] == 0).all()
    # adding garbage keys beyond N_kv must not change anything
    K2 = np.concatenate([K, 50 * np.ones((56, 64), np.float32)])
    q2 = _quantized(Q, K2, V, mxfp4.UOS, True, v_pad=256)
    O2 = attention.flash_attention_mx(q2[0], q2[1], q2[2], q2[3], *q[4:], 200, 0.125, True,
                                      mxfp4.UOS, 128)
    assert (O2 == O).all()


def test_pipeline_hadamard_changes_codes_not_logits():
    Q, K, V, w = _tiny_inputs()
    O_h = attention.mx_attention_pipeline(Q, K, V, w.softmax_scale, True, True, mxfp4.UOS, 64, 128)
    O_n = attention.mx_attention_pipeline(Q, K, V, w.softmax_scale, False, True, mxfp4.UOS, 64, 128)
    Oe = attention.exact_attention(Q, K, V, w.softmax_scale)
    e_h = np.linalg.norm(O_h - Oe) / np.linalg.norm(Oe)
    e_n = np.linalg.norm(O_n - Oe) / np.linalg.norm(Oe)
    assert 0 < e_h < 1.5 and 0 < e_n < 1.5 and e_h != e_n
    assert np.abs(hadamard.fwht_fp32(Q) @ hadamard.fwht_fp32(K).T - Q @ K.T).max() < 1e-2
