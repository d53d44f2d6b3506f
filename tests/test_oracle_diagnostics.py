"""Pins of the diagnostics oracle (oracle/diagnostics.py) -- CPU only."""
import numpy as np
import pytest

from oracle import attention as ora
from oracle import diagnostics as od
from oracle import hadamard, mxfp4

RULES = [mxfp4.UOS, mxfp4.OCP, mxfp4.TFS, ("ceil", 7.5)]


@pytest.mark.parametrize("rule", RULES)
def test_representable_blocks_have_zero_error(rule):
    """Blocks of E2M1 grid values whose maximum is 4 * 2^k: every rule here picks
    e = k for them (4 lies in the target interval of CEIL(q) for q in (4, 8] and of
    OCP), so quantisation is exact."""
    rng = np.random.default_rng(1)
    grid = mxfp4.E2M1_GRID
    x = rng.choice(np.concatenate([grid[:6], -grid[:6]]), size=(64, 128)).astype(np.float32)
    x[:, ::32] = 4.0                                   # every block's max is 4
    x *= np.exp2(rng.integers(-20, 20, size=(64, 1))).astype(np.float32)
    e2, r2, nf = od.quant_rel_mse(x, rule)
    assert e2 == 0.0 and r2 > 0 and nf == 0


@pytest.mark.parametrize("rule", RULES)
def test_power_of_two_scaling_leaves_relative_error_unchanged(rule):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((128, 64)).astype(np.float32)
    e2, r2, _ = od.quant_rel_mse(x, rule)
    e2s, r2s, _ = od.quant_rel_mse(x * np.float32(2.0 ** 9), rule)
    assert e2s / r2s == pytest.approx(e2 / r2, rel=1e-12)


def test_rows_axis_is_the_last_axis_of_the_transpose():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((100, 64)).astype(np.float32)   # 100 rows: a ragged last block
    xt = np.zeros((64, 128), dtype=np.float32)
    xt[:, :100] = x.T
    assert od.quant_rel_mse(x, mxfp4.UOS, axis="rows") == od.quant_rel_mse(xt, mxfp4.UOS)


def test_rotation_variant_quantises_the_fwht_output():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    assert od.quant_rel_mse(x, mxfp4.UOS, hadamard_on=True) == od.quant_rel_mse(hadamard.fwht_fp32(x), mxfp4.UOS)


def test_nonfinite_blocks_are_counted_and_left_out():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    ref = od.quant_rel_mse(x, mxfp4.UOS)
    y = x.copy()
    y[0, 3] = np.nan
    y[5, 100] = np.inf
    e2, r2, nf = od.quant_rel_mse(y, mxfp4.UOS)
    assert nf == 2
    assert e2 < ref[0] and r2 < ref[1]


def _head(n_q, n_kv, d, seed):
    rng = np.random.default_rng(seed)
    Q = (rng.standard_normal((n_q, d)) * 1.5).astype(np.float32)
    K = (rng.standard_normal((n_kv, d)) * 1.5).astype(np.float32)
    return Q, K


@pytest.mark.parametrize("rule", [mxfp4.UOS, mxfp4.OCP, mxfp4.TFS])
def test_rowsum_total_is_the_direct_placement_drift_with_unit_values(rule):
    """With V = 1 and direct placement (l sums P~, O~ sums P^), O = sum P^ / sum P~ for
    each row, so mean(O - 1) is exactly the total relative change of the normaliser."""
    Q, K = _head(48, 300, 128, 6)
    Bc, scale = 128, float(np.float32(1 / np.sqrt(128)))
    Qc, Qs = ora.quantize_qk(Q, rule, True)
    Kc, Ks = ora.quantize_qk(K, rule, True)
    VTc, VTs = ora.quantize_v(np.ones_like(K), rule, 384)
    O = ora.flash_attention_mx(Qc, Qs, Kc, Ks, VTc, VTs, 300, scale, False, rule, Bc)
    dec = od.rowsum_decomposition(Qc, Qs, Kc, Ks, 300, scale, rule, Bc)
    assert dec["total"] == pytest.approx(float((O[:, 0] - 1.0).mean()), abs=1e-12)
    parts = dec["zeroed"] + dec["saturated"] + dec["rounded_down"] + dec["rounded_up"]
    assert parts == pytest.approx(dec["total"], abs=1e-12)
    assert dec["zeroed"] <= 0 and dec["saturated"] <= 0 and dec["rounded_down"] <= 0 and dec["rounded_up"] >= 0


def test_rowsum_direct_placement_drifts_down():
    """The pages' account: the unquantised normaliser overshoots the quantised weights
    (zeroed small P~ dominate), so sum P^ < sum P~ on average (direct placement's row
    sums fall below one; Figure 7(A) in the Pith review's captions)."""
    Q, K = _head(64, 512, 128, 7)
    scale = float(np.float32(1 / np.sqrt(128)))
    Qc, Qs = ora.quantize_qk(Q, mxfp4.UOS, True)
    Kc, Ks = ora.quantize_qk(K, mxfp4.UOS, True)
    dec = od.rowsum_decomposition(Qc, Qs, Kc, Ks, 512, scale, mxfp4.UOS, 128)
    assert dec["total"] < 0 and dec["zeroed"] < 0
