"""Pins for oracle/mxfp4.py: the E2M1 grid, rounding, the scale rules and the block quantiser.

Each test checks the oracle against something other than itself: values the
pages state (tests/golden/page_values.json), a rounding derived another way
(NumPy's round-half-even on the uniformly spaced stretches of the grid), exact
interval properties of each rule, or Eq. 96's cross-rule identity.
"""
import json
import os

import numpy as np
import pytest

from oracle import mxfp4
from synth import special_values_f32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_grid_matches_pages():
    assert mxfp4.E2M1_GRID.tolist() == GOLD["e2m1_positive_grid"]["value"]
    assert mxfp4.BLOCK == GOLD["block_size"]["value"]
    assert mxfp4.E2M1_GRID.max() == GOLD["e2m1_max_finite"]["value"]
    dec = mxfp4.e2m1_decode(np.arange(16))
    assert dec[:8].tolist() == GOLD["e2m1_positive_grid"]["value"]
    assert (dec[8:] == -dec[:8]).all() and np.signbit(dec[8:]).all()


def test_roundtrip_all_codes():
    c = np.arange(16, dtype=np.uint8)
    assert (mxfp4.e2m1_encode(mxfp4.e2m1_decode(c)) == c).all()


def test_tie_and_saturation_table():
    # ties go to the even code; |v| above the grid saturates to 6 (code 7)
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             6.5: 7, 7.0: 7, 7.25: 7, 8.0: 7, 100.0: 7, 1e30: 7}
    for v, code in table.items():
        assert mxfp4.e2m1_encode(v) == code, v
        assert mxfp4.e2m1_encode(-v) == code | 8, v
    ex = GOLD["ocp_overflow_example"]["value"]
    v = np.nextafter(ex["scaled_max_above"], 8.0)           # just above 7: nearest *unbounded* point is 8
    assert mxfp4.e2m1_decode(mxfp4.e2m1_encode(v)) == ex["saturates_to"]


def test_signed_zero_reading():
    assert mxfp4.e2m1_encode(-0.0) == 8
    assert mxfp4.e2m1_encode(-0.1) == 8
    assert mxfp4.e2m1_encode(0.0) == 0


def _round_by_stretches(v):
    """E2M1 rounding derived another way: the grid is uniform on [0,2] (step .5), [2,4]
    (step 1) and [4,6] (step 2); on each stretch numpy's round-half-even of the step
    count gives the code, and even step counts are even codes."""
    a = np.abs(v)
    out = np.where(a <= 2.0, np.round(a * 2.0),                  # codes 0..4
          np.where(a <= 4.0, 2.0 + np.round(a),                  # codes 4..6 (2 + value)
          np.where(a <= 6.0, 4.0 + np.round(a / 2.0),            # codes 6..7 (value 4 or 6)
                   7.0)))
    # at the stretch joins (2, 4) both formulas agree; above 6 everything saturates
    return (np.signbit(v).astype(np.uint8) << 3 | out.astype(np.uint8)).astype(np.uint8)


def test_encode_matches_stretch_rounding_on_dense_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-8, 8, 200_000), np.arange(-8, 8.0001, 0.125),
                        np.arange(-7, 7.0001, 1 / 1024)])
    assert (mxfp4.e2m1_encode(v) == _round_by_stretches(v)).all()


def test_encode_is_nearest_point_on_all_bf16_values():
    x = special_values_f32()
    x = x[np.isfinite(x)]
    for k in (0, -3, 5):                     # a few scalings of every bf16 pattern
        v = np.ldexp(x.astype(np.float64), k)
        c = mxfp4.e2m1_encode(v)
        err = np.abs(np.abs(v) - mxfp4.E2M1_GRID[c & 7])
        others = np.abs(np.abs(v)[:, None] - mxfp4.E2M1_GRID[None, :]).min(axis=1)
        assert (err <= others).all()
        assert ((c >> 3) == np.signbit(v)).all()
        # real ties sit at grid midpoints (<= 5); far above the grid float64 distances
        # all round to the same number, so only look for ties where they are exact
        tie = ((np.abs(np.abs(v)[:, None] - mxfp4.E2M1_GRID[None, :]) == err[:, None]).sum(1) > 1) \
            & (np.abs(v) < 64)
        assert tie.sum() > 0 and ((c[tie] & 1) == 0).all()
        assert (c[np.abs(v) > 6] & 7 == 7).all()


@pytest.mark.parametrize("name,rule", [("ocp", mxfp4.OCP), ("tfs", mxfp4.TFS), ("uos", mxfp4.UOS)])
def test_rule_intervals_match_figure3(name, rule):
    rng = np.random.default_rng(7)
    M = np.exp2(rng.uniform(-40, 40, 1_000_000)).astype(np.float32).astype(np.float64)
    e = mxfp4.scale_exponent(M, rule)
    x = np.ldexp(M, -e)
    r = GOLD["normalised_max_ranges"]["value"][name]
    lo_ok = x >= r["lo"] if r["lo_closed"] else x > r["lo"]
    hi_ok = x <= r["hi"] if r["hi_closed"] else x < r["hi"]
    assert lo_ok.all() and hi_ok.all()


def test_ceil_rule_is_smallest_exponent_at_boundaries():
    q = GOLD["uos_boundary"]["value"]["decimal"]
    assert mxfp4.scale_exponent(q, mxfp4.UOS) == 0
    assert mxfp4.scale_exponent(np.nextafter(np.float32(q), np.float32(8)).astype(np.float64), mxfp4.UOS) == 1
    assert mxfp4.scale_exponent(q * 2.0 ** -40, mxfp4.UOS) == -40
    # exact powers of two: OCP puts M = 1 at 4, ceil(8) at 8
    assert mxfp4.scale_exponent(1.0, mxfp4.OCP) == -2
    assert mxfp4.scale_exponent(1.0, mxfp4.rule_ceil(8.0)) == -3
    # M = 0 and clamping
    assert mxfp4.scale_exponent(0.0, mxfp4.UOS) == -127
    assert mxfp4.scale_exponent(2.0 ** -140, mxfp4.UOS) == -127


def test_eq96_oas_versus_tfs():
    g = GOLD["oas_eq96"]["value"]
    rng = np.random.default_rng(3)
    M = np.exp2(rng.uniform(-20, 20, 200_000))
    e6 = mxfp4.scale_exponent(M, mxfp4.TFS)
    e7 = mxfp4.scale_exponent(M, mxfp4.OAS)
    x6 = np.ldexp(M, -e6)
    lo, hi = g["halves_scale_when_x6_in"]
    band = (x6 > lo) & (x6 <= hi)
    assert (e7[band] == e6[band] - 1).all()
    assert (e7[~band] == e6[~band]).all()
    x7 = np.ldexp(M[band], -e7[band])
    assert (x7 > g["maps_to"][0]).all() and (x7 <= g["maps_to"][1]).all()


def test_block_quantiser_uos_vs_ocp_on_overflow_block():
    # one block whose max scales to 7.5 under OCP: saturates to 6; UOS moves it to the next scale
    x = np.zeros(32)
    x[0] = 7.5
    x[1] = 0.3
    c_ocp, s_ocp = mxfp4.quantize_blocks_lastaxis(x, mxfp4.OCP)
    c_uos, s_uos = mxfp4.quantize_blocks_lastaxis(x, mxfp4.UOS)
    assert s_ocp[0] == 127 and mxfp4.dequantize_blocks_lastaxis(c_ocp, s_ocp)[0] == 6.0
    assert s_uos[0] == 128 and mxfp4.dequantize_blocks_lastaxis(c_uos, s_uos)[0] == 8.0
    # the small element: OCP keeps 0.5 resolution (0.3 -> 0.5), UOS at scale 2 rounds 0.15 -> 0
    assert mxfp4.dequantize_blocks_lastaxis(c_ocp, s_ocp)[1] == 0.5
    assert mxfp4.dequantize_blocks_lastaxis(c_uos, s_uos)[1] == 0.0


def test_block_edge_cases():
    z = np.zeros((2, 64))
    c, s = mxfp4.quantize_blocks_lastaxis(z, mxfp4.UOS)
    assert (c == 0).all() and (s == 0).all()
    bad = np.ones((1, 64))
    bad[0, 3] = np.inf
    bad[0, 40] = np.nan
    c, s = mxfp4.quantize_blocks_lastaxis(bad, mxfp4.UOS)
    assert s.tolist() == [[0xFF, 0xFF]] and (c == 0).all()
    # padding never changes the codes of real elements
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 75)).astype(np.float32)
    c1, s1 = mxfp4.quantize_blocks_lastaxis(x, mxfp4.UOS)
    xp = np.concatenate([x, np.zeros((5, 21), np.float32)], axis=1)
    c2, s2 = mxfp4.quantize_blocks_lastaxis(xp, mxfp4.UOS)
    assert (c1 == c2).all() and (s1 == s2).all()


def test_dequant_error_bound_per_rule():
    # |x - Q(x)| <= half a grid step of the scaled value, except saturation above 6
    rng = np.random.default_rng(5)
    x = rng.standard_normal((512, 128)).astype(np.float32)
    for rule in (mxfp4.UOS, mxfp4.OCP, mxfp4.TFS):
        c, s = mxfp4.quantize_blocks_lastaxis(x, rule)
        xq = mxfp4.dequantize_blocks_lastaxis(c, s)
        scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
        v = np.abs(x) / scale
        step = np.where(v <= 2, 0.5, np.where(v <= 4, 1.0, 2.0))
        bound = np.where(v <= 6, step / 2, v - 6) * scale
        assert (np.abs(x - xq) <= bound + 1e-12).all()


def test_uos_lowers_gaussian_quantisation_error():
    # the clipping/underflow trade-off: on Gaussian blocks UOS beats both OCP and q = 6
    rng = np.random.default_rng([0, 3, 0])
    x = rng.standard_normal((4096, 128)).astype(np.float32)
    def rel_mse(rule):
        c, s = mxfp4.quantize_blocks_lastaxis(x, rule)
        return float(((mxfp4.dequantize_blocks_lastaxis(c, s) - x) ** 2).sum() / (x.astype(np.float64) ** 2).sum())
    u, o, t = rel_mse(mxfp4.UOS), rel_mse(mxfp4.OCP), rel_mse(mxfp4.TFS)
    assert u < o and u < t


def test_pack_unpack_and_transposed_layout():
    rng = np.random.default_rng(2)
    c = rng.integers(0, 16, (3, 64), dtype=np.uint8)
    p = mxfp4.pack_nibbles(c)
    assert p.shape == (3, 32) and (p[:, 0] == (c[:, 0] | c[:, 1] << 4)).all()
    assert (mxfp4.unpack_nibbles(p) == c).all()
    v = rng.standard_normal((70, 8)).astype(np.float32)
    vc, vs = mxfp4.quantize_rows_transposed(v, mxfp4.UOS, pad_to=128)
    assert vc.shape == (8, 128) and vs.shape == (8, 4)
    assert (vs[:, 3] == 0).all() and (vc[:, 70:] == 0).all()
    c0, s0 = mxfp4.quantize_blocks_lastaxis(v[:32, 5], mxfp4.UOS)
    assert (vc[5, :32] == c0).all() and vs[5, 0] == s0[0]
