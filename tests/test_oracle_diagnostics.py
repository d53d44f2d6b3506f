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


def _key_row(logit):
    """A key row of 32 E2M1 values times 2^-4 whose dot product with an all-ones query
    is `logit` (a multiple of 1/32, |logit| <= 12)."""
    t, vals = logit * 16.0, []
    for _ in range(32):
        a = max(x for x in mxfp4.E2M1_GRID if x <= min(abs(t), 6.0))
        vals.append(np.copysign(a, t))
        t -= vals[-1]
    assert t == 0.0
    return np.array(vals) * 2.0 ** -4


# One query row, one kv tile of 64 keys (two 32-key blocks), logits chosen by hand so that
# each element's scaled value P~ / 2^e sits well inside one rounding class.  Block 0 holds
# the row max (P~ = 1, UOS exponent -2: scaled values are 4 P~); block 1's largest P~ is
# exp(-0.125) = 0.882, whose UOS exponent is -3 (0.882 * 8 = 7.06 <= 7.25).  Each entry:
# (logit, block, P^ value from the E2M1 table, class).
CLASS_TILE = [
    (10.0, 0, 1.0, None),                        # scaled 4      -> 4, exact
    (7.0, 0, 0.0, "zeroed"),                     # scaled 0.199  -> 0
    (8.71875, 0, 1.0 * 2 ** -2, "rounded_down"),  # scaled 1.110  -> 1
    (9.59375, 0, 3.0 * 2 ** -2, "rounded_up"),    # scaled 2.664  -> 3
    (8.09375, 0, 0.5 * 2 ** -2, "rounded_down"),  # scaled 0.594  -> 0.5
    (7.5625, 0, 0.5 * 2 ** -2, "rounded_up"),     # scaled 0.350  -> 0.5
    (9.875, 1, 6.0 * 2 ** -3, "saturated"),       # scaled 7.06   -> 8 unbounded, 6 in E2M1
    (9.8125, 1, 6.0 * 2 ** -3, "rounded_down"),   # scaled 6.63   -> 6 (below the tie at 7)
    (9.625, 1, 6.0 * 2 ** -3, "rounded_up"),      # scaled 5.50   -> 6
    (9.40625, 1, 4.0 * 2 ** -3, "rounded_down"),  # scaled 4.42   -> 4
    (5.625, 1, 0.0, "zeroed"),                    # scaled 0.101  -> 0
]


def test_rowsum_classes_on_a_hand_built_tile():
    """Each class of rowsum_decomposition against sums written out from the table above:
    the class of an element is fixed by its scaled value (zeroed: code 0 for P~ > 0;
    saturated: scaled >= 7, where round-to-nearest heads for 8 and the format clips to
    6; otherwise the sign of P^ - P~), so a shifted boundary or a swapped class fails."""
    n0 = sum(1 for e in CLASS_TILE if e[1] == 0)
    logits = [e[0] for e in CLASS_TILE if e[1] == 0] + [10.0] * (32 - n0) + [e[0] for e in CLASS_TILE if e[1] == 1]
    nkv = len(logits)                                     # keys 37..63 of the tile are padding
    K = np.stack([_key_row(x) for x in logits])
    Q = np.ones((1, 32))
    Qc, Qs = mxfp4.quantize_blocks_lastaxis(Q, mxfp4.UOS)
    Kc, Ks = mxfp4.quantize_blocks_lastaxis(K, mxfp4.UOS)
    assert (mxfp4.dequantize_blocks_lastaxis(Kc, Ks) @ Q[0] == np.array(logits)).all()
    dec = od.rowsum_decomposition(Qc, Qs, Kc, Ks, nkv, 1.0, mxfp4.UOS, 64)
    P = {x: float(np.float32(np.exp(x - 10.0))) for x in logits}
    lt = sum(P[x] for x in logits)
    want = {c: 0.0 for c in ("zeroed", "saturated", "rounded_down", "rounded_up")}
    for logit, _, ph, cls in CLASS_TILE:
        if cls:
            want[cls] += ph - P[logit]
    for c, v in want.items():
        assert dec[c] == pytest.approx(v / lt, rel=1e-12, abs=1e-15), c
    assert dec["total"] == pytest.approx(sum(want.values()) / lt, rel=1e-12)


# ---- global-scaling arm (post-normalisation P, one factor g before quantisation)

def test_global_scaling_one_hot_rows_closed_form():
    """A one-hot row holds the single value g, whose block max is g.  Under UOS
    (smallest e with g <= 7.25 * 2^e) the scaled value g / 2^e rounds to a grid point G,
    and the row sum is G * 2^e.  Worked by hand:
      g = 1   : e = -2, 4.0 -> 4 : 1
      g = 1.1 : e = -2, 4.4 -> 4 : 1
      g = 1.3 : e = -2, 5.2 -> 6 : 1.5
      g = 1.9 : e = -1, 3.8 -> 4 : 2"""
    P = np.zeros((3, 96), np.float32)
    P[0, 0] = P[1, 40] = P[2, 95] = 1.0
    rs = od.global_scaling_rowsums(P, mxfp4.UOS, [1.0, 1.1, 1.3, 1.9])
    for i, w in enumerate([1.0, 1.0, 1.5, 2.0]):
        assert np.all(rs[i] == w), (i, rs[i], w)


def test_global_scaling_power_of_two_factor_scales_the_sums():
    """A power-of-two g moves every block scale by the same power: the row sums scale
    by g exactly."""
    rng = np.random.default_rng(7)
    S = rng.standard_normal((16, 200)) * 3
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P = (P / P.sum(axis=1, keepdims=True)).astype(np.float32)
    for rule in (mxfp4.UOS, mxfp4.OCP):
        rs = od.global_scaling_rowsums(P, rule, [1.0, 2.0, 0.25, 1024.0])
        for i, g in enumerate([1.0, 2.0, 0.25, 1024.0]):
            assert np.array_equal(rs[i], rs[0] * g)


def test_global_scaling_grid_rows_and_ties():
    """[1/2, 1/4, 1/8, 1/8]: block max 1/2, UOS e = -3 (1/2 <= 7.25/8), scaled values
    4, 2, 1, 1 -- grid points -- so the row sum is exactly 1 at g = 1.  At g = 1.25 the
    block max is 0.625, e = -3 again, scaled values 5, 2.5, 1.25, 1.25 are all ties that
    go to the even code: 4, 2, 1, 1, so the sum is (4 + 2 + 1 + 1) / 8 = 1 although the
    weights were scaled up by 1.25.  At g = 1.5: 6, 3, 1.5, 1.5, all on the grid: 1.5."""
    P = np.zeros((1, 32), np.float32)
    P[0, :4] = [0.5, 0.25, 0.125, 0.125]
    rs = od.global_scaling_rowsums(P, mxfp4.UOS, [1.0, 1.25, 1.5])
    assert rs[0, 0] == 1.0 and rs[1, 0] == 1.0 and rs[2, 0] == 1.5


def test_global_scaling_moves_the_mean_not_the_rows():
    """On softmax rows of Gaussian logits the quantised rows sum to less than one on
    average; a factor g a little above one brings the average back to one, and the rows'
    spread around their mean stays of the same size."""
    rng = np.random.default_rng(11)
    S = rng.standard_normal((64, 512)) * 2.5
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P = (P / P.sum(axis=1, keepdims=True)).astype(np.float32)
    gs = [1.0 + i / 256 for i in range(64)]
    rs = od.global_scaling_rowsums(P, mxfp4.UOS, gs)
    mean = rs.mean(axis=1)
    assert mean[0] < 0.97 and mean.max() > 1.0
    best = int(np.abs(mean - 1).argmin())
    assert abs(mean[best] - 1) < 0.005
    assert rs[best].std() > 0.5 * rs[0].std()
