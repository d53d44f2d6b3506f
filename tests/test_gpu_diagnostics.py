"""GPU parity of the scale-rule diagnostics (mxattn_quant_error and the helpers of
diagnostics.py) against oracle/diagnostics.py and the oracle's
attention.  The quantisers are bit-exact, so the error sums differ from the oracle's
float64 sums only by the kernel's fp32 per-block accumulation."""
import numpy as np
import pytest

import synth
from oracle import attention as ora
from oracle import diagnostics as od
from oracle import mxfp4
from _gpu_helpers import RULES, require_gpu, to_device

pytestmark = pytest.mark.gpu
SUM_REL = 2e-5


def _gpu_sums(mx, x, dtype, rule, axis, had):
    s = mx.mxattn_quant_error(to_device(x, dtype), rule=rule, axis=axis, hadamard=had)
    return s.cpu().numpy()


@pytest.mark.parametrize("rule", ["uos", "ocp", "tfs", "oas", "q7.5"])
@pytest.mark.parametrize("had", [False, True])
def test_quant_error_last_axis(rule, had):
    torch, mx = require_gpu()
    x = synth.quant_head(synth.TINY_QUANT, 0)                 # 4096 x 128 fp32 N(0,1)
    g = _gpu_sums(mx, x, "f32", RULES[rule][0], "last", had)
    e2, r2, nf = od.quant_rel_mse(x, RULES[rule][1], "last", had)
    assert g[2] == nf == 0
    assert g[0] == pytest.approx(e2, rel=SUM_REL) and g[1] == pytest.approx(r2, rel=SUM_REL)


@pytest.mark.parametrize("rule", ["uos", "ocp"])
def test_quant_error_bf16_outliers_rotated_and_rows(rule):
    torch, mx = require_gpu()
    w = synth.QUANT_720P
    x = synth.quant_head(w, 0)[:3000]                          # bf16 values with spikes and outlier channels
    for axis, had in (("last", True), ("last", False), ("rows", False)):
        g = _gpu_sums(mx, x, "bf16", RULES[rule][0], axis, had)
        e2, r2, nf = od.quant_rel_mse(x, RULES[rule][1], axis, had)
        assert g[2] == nf == 0, (axis, had)
        assert g[0] == pytest.approx(e2, rel=SUM_REL), (axis, had)
        assert g[1] == pytest.approx(r2, rel=SUM_REL), (axis, had)


def test_quant_error_counts_nonfinite_blocks():
    torch, mx = require_gpu()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3, 5] = np.nan
    x[10, 70] = np.inf
    x[10, 71] = -np.inf
    for axis, had in (("last", False), ("last", True), ("rows", False)):
        g = _gpu_sums(mx, x, "f32", "uos", axis, had)
        e2, r2, nf = od.quant_rel_mse(x, mxfp4.UOS, axis, had)
        assert g[2] == nf, (axis, had, g[2], nf)
        assert g[0] == pytest.approx(e2, rel=SUM_REL) and g[1] == pytest.approx(r2, rel=SUM_REL)


def test_qmax_sweep_matches_oracle():
    torch, mx = require_gpu()
    import diagnostics as dg
    x = synth.quant_head(synth.TINY_QUANT, 0)
    qs = (6.0, 6.5, 7.0, 7.25, 7.5, 8.0)
    sw = dg.qmax_sweep(to_device(x, "f32"), qs=qs, hadamard=True)
    for q in qs:
        e2, r2, _ = od.quant_rel_mse(x, ("ceil", q), "last", True)
        assert sw[f"q{q:.2f}"]["rel_mse"] == pytest.approx(e2 / r2, rel=SUM_REL)
    e2, r2, _ = od.quant_rel_mse(x, mxfp4.OCP, "last", True)
    assert sw["ocp"]["rel_mse"] == pytest.approx(e2 / r2, rel=SUM_REL)


def test_p_tile_sweep_matches_oracle():
    torch, mx = require_gpu()
    import diagnostics as dg
    w = synth.TINY
    Q, K, V = (synth.attn_head(w, t, 0) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
    scale = float(np.float32(w.softmax_scale))
    qs = (6.0, 7.25, 8.0)
    sw = dg.p_tile_sweep(*(to_device(a, "f32") for a in (Q, K, V)), scale, qs=qs)
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(w.N)
    Qc, Qs = ora.quantize_qk(Q, mxfp4.UOS, True)
    Kc, Ks = ora.quantize_qk(K, mxfp4.UOS, True)
    VTc, VTs = ora.quantize_v(V, mxfp4.UOS, P)
    # reference: softmax attention on the dequantised operands, P left unquantised
    deq = mxfp4.dequantize_blocks_lastaxis
    ex = ora.exact_attention(deq(Qc, Qs), deq(Kc, Ks), deq(VTc, VTs).T[: w.N], scale)
    for q in qs:
        O = ora.flash_attention_mx(Qc, Qs, Kc, Ks, VTc, VTs, w.N, scale, True, ("ceil", q), Bc)
        err = float(np.linalg.norm(O - ex) / np.linalg.norm(ex))
        assert abs(sw[f"q{q:.2f}"] - err) < 5e-3, (q, sw[f"q{q:.2f}"], err)


@pytest.mark.parametrize("rule", ["uos", "ocp"])
def test_rowsum_decomposition_matches_oracle(rule):
    torch, mx = require_gpu()
    import diagnostics as dg
    rng = np.random.default_rng(12)
    n, d = 700, 128
    Q = (rng.standard_normal((n, d)) * 1.5).astype(np.float32)
    K = (rng.standard_normal((n, d)) * 1.5).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    g = dg.rowsum_decomposition(*(to_device(a, "f32") for a in (Q, K, V)), scale, p_rule=RULES[rule][0],
                                rule=RULES[rule][0])
    Qc, Qs = ora.quantize_qk(Q, RULES[rule][1], True)
    Kc, Ks = ora.quantize_qk(K, RULES[rule][1], True)
    o = od.rowsum_decomposition(Qc, Qs, Kc, Ks, n, scale, RULES[rule][1], mx.mxattn_kv_tile())
    for c in ("zeroed", "saturated", "rounded_down", "rounded_up", "total"):
        assert abs(g[c] - o[c]) < 1e-4 + 1e-3 * abs(o[c]), (c, g[c], o[c])


@pytest.mark.parametrize("rule", ["uos", "ocp"])
def test_global_scaling_matches_oracle(rule):
    """The global-scaling arm: the GPU's row sums of the quantised g * P equal the
    oracle's on the same fp32 P (the quantiser is bit-exact; only the float64 summation
    order differs), for a few g and for the g the sweep picks."""
    torch, mx = require_gpu()
    import diagnostics as dg
    w = synth.TINY
    Q, K, V = (synth.attn_tensor(w, t) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
    q, k, v = (to_device(x[0, 0], "f32") for x in (Q, K, V))
    P = dg.probabilities(q, k, v, float(np.float32(w.softmax_scale)), rule=RULES[rule][0])
    gs = (1.0, 1.03, 1.0625, 1.3, 2.0)
    g_rs = dg.global_scaling_rowsums(P, p_rule=RULES[rule][0], gammas=gs).cpu().numpy()
    o_rs = od.global_scaling_rowsums(P.cpu().numpy(), RULES[rule][1], gs)
    np.testing.assert_allclose(g_rs, o_rs, rtol=1e-12, atol=0)
    summary = dg.global_scaling(P, p_rule=RULES[rule][0])
    o_all = od.global_scaling_rowsums(P.cpu().numpy(), RULES[rule][1], dg.GAMMAS)
    best = int(np.abs(o_all.mean(axis=1) - 1).argmin())
    assert summary["g_best"] == dg.GAMMAS[best]
    assert summary["at_g1"]["mean"] == pytest.approx(o_all[0].mean(), rel=1e-12)
