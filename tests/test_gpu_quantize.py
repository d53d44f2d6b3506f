"""GPU parity: the HIP quantisers must be bit-exact to the oracle (codes and E8M0 bytes).

Cases: every bf16 bit pattern in three block arrangements (sequential, shuffled,
and spread over six binades within each block), hand-built tie and saturation
blocks, the tiny workload's Q/K (d = 64, fp32) with and without the Hadamard
rotation, the 4096 x 128 fp32 N(0,1) tensor, outlier-law bf16 heads with the
rotation, the transposed token-axis layout of V with ragged token counts, and
every head of the full 40 x 75,600 x 128 standalone quantise pass.
"""
import os

import numpy as np
import pytest

import synth
from oracle import attention as ora_attn
from oracle import hadamard, mxfp4
from _gpu_helpers import RULES, require_gpu, to_device, u8

pytestmark = pytest.mark.gpu
RULE_NAMES = ["uos", "ocp", "tfs", "oas"]


def _gpu_last(x32: np.ndarray, dtype: str, rule_name: str, had: bool):
    torch, mx = require_gpu()
    xd = to_device(x32, dtype)
    c, s = mx.mxattn_quantize(xd, rule=RULES[rule_name][0], axis="last", hadamard=had)
    torch.cuda.synchronize()
    return mxfp4.unpack_nibbles(u8(c)), u8(s)


def _oracle_last(x32: np.ndarray, rule_name: str, had: bool):
    y = hadamard.fwht_fp32(x32) if had else np.asarray(x32, np.float32)
    return mxfp4.quantize_blocks_lastaxis(y, RULES[rule_name][1])


def _assert_same(gc, gs, oc, os_, what):
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first at {bad_s[:3].tolist()}"
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} codes differ, first at {bad_c[:3].tolist()}"


@pytest.mark.parametrize("rule", RULE_NAMES)
@pytest.mark.parametrize("arrangement", ["sequential", "shuffled", "spread"])
def test_every_bf16_pattern(rule, arrangement):
    v = synth.special_values_f32().reshape(-1, 32)          # 2048 blocks of 32
    if arrangement == "shuffled":
        v = v.reshape(-1)[np.random.default_rng(0).permutation(65536)].reshape(-1, 32)
        dtype = "bf16"
    elif arrangement == "spread":
        # scale element j of every block by 2^-(j % 6): scaled values fill [0, 8]
        v = (v * np.exp2(-(np.arange(32) % 6))).astype(np.float32)
        dtype = "f32"
    else:
        dtype = "bf16"
    gc, gs = _gpu_last(v, dtype, rule, False)
    oc, os_ = _oracle_last(v, rule, False)
    _assert_same(gc, gs, oc, os_, f"{arrangement}/{rule}")


@pytest.mark.parametrize("rule", RULE_NAMES)
def test_ties_saturation_and_boundaries(rule):
    blocks = []
    q = 7.25
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.0]
    for e in (-130, -126, -60, -3, 0, 5, 100, 125):
        for M in (q, np.nextafter(np.float32(q), np.float32(8)), 7.0, 6.0, 4.0, 8.0 - 2 ** -21, 3.625):
            b = np.zeros(32, np.float64)
            b[0] = M
            b[1:1 + len(ties)] = ties
            b[12:12 + len(ties)] = [-t for t in ties]
            b[25] = -0.0
            b[26] = 0.2500001
            blocks.append(np.ldexp(b, e))
    x = np.array(blocks).astype(np.float32)                  # exact: values have few bits
    gc, gs = _gpu_last(x, "f32", rule, False)
    oc, os_ = _oracle_last(x, rule, False)
    _assert_same(gc, gs, oc, os_, f"ties/{rule}")


def test_special_blocks():
    x = np.zeros((4, 32), np.float32)
    x[1, 3] = np.inf
    x[2, 7] = np.nan
    x[2, 8] = 3.0
    x[3, :] = -0.0
    gc, gs = _gpu_last(x, "f32", "uos", False)
    oc, os_ = _oracle_last(x, "uos", False)
    _assert_same(gc, gs, oc, os_, "special")
    assert gs[:, 0].tolist() == [0, 0xFF, 0xFF, 0]


@pytest.mark.parametrize("rule", RULE_NAMES)
@pytest.mark.parametrize("had", [False, True])
def test_tiny_workload_q_k(rule, had):
    w = synth.TINY
    for tid in (synth.Q_ID, synth.K_ID):
        x = synth.attn_tensor(w, tid).reshape(-1, w.d)       # [2 * 256, 64] fp32
        gc, gs = _gpu_last(x, "f32", rule, had)
        oc, os_ = _oracle_last(x, rule, had)
        _assert_same(gc, gs, oc, os_, f"tiny tid={tid} had={had} {rule}")


@pytest.mark.parametrize("rule", RULE_NAMES)
@pytest.mark.parametrize("had", [False, True])
def test_gaussian_4096x128_fp32(rule, had):
    x = np.random.default_rng([0, 3, 0]).standard_normal((4096, 128), dtype=np.float32)
    gc, gs = _gpu_last(x, "f32", rule, had)
    oc, os_ = _oracle_last(x, rule, had)
    _assert_same(gc, gs, oc, os_, f"gauss had={had} {rule}")


@pytest.mark.parametrize("rule", RULE_NAMES)
@pytest.mark.parametrize("nrows", [1, 127, 129, 5000])
def test_outlier_bf16_rows_with_rotation(rule, nrows):
    import dataclasses
    w = dataclasses.replace(synth.QUANT_720P, N=nrows)
    x = synth.quant_head(w, 3)
    gc, gs = _gpu_last(x, "bf16", rule, True)
    oc, os_ = _oracle_last(x, rule, True)
    _assert_same(gc, gs, oc, os_, f"outlier n={nrows} {rule}")


@pytest.mark.parametrize("rule", ["uos", "ocp", "tfs"])
@pytest.mark.parametrize("N,C,dtype", [(256, 64, "f32"), (200, 128, "bf16"), (1000, 128, "bf16"),
                                       (32760 // 8, 128, "bf16"), (33, 64, "bf16"), (1, 128, "f32"),
                                       (300, 6, "f32")])
def test_token_axis_transposed(rule, N, C, dtype):
    torch, mx = require_gpu()
    rng = np.random.default_rng(N * 7 + C)
    x = rng.standard_normal((2, N, C)).astype(np.float32)
    if dtype == "bf16":
        x = synth.bf16_to_f32(synth.round_to_bf16(x))
    xd = to_device(x, dtype)
    c, s = mx.mxattn_quantize(xd, rule=RULES[rule][0], axis="rows")
    torch.cuda.synchronize()
    gc, gs = mxfp4.unpack_nibbles(u8(c)), u8(s)
    P = mx.mxattn_padded_tokens(N)
    oc, os_ = ora_attn.quantize_v(x, RULES[rule][1], P)
    assert gc.shape == oc.shape == (2, C, P)
    _assert_same(gc, gs, oc, os_, f"rows N={N} C={C} {rule}")


DIGESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_720p_digests.json")


def test_full_size_quantize_pass_every_head():
    """The whole standalone quantize workload: 40 x 75,600 x 128 bf16 drawn by the seeded
    host law (outlier channels and spikes), Hadamard + quantise in one launch per rule
    (UOS, OCP, TFS).  Every head's packed codes and scale bytes are hashed and compared
    with the oracle's digests (tests/golden/make_quant_digests.py, which runs only the
    oracle); a head whose digest differs is recomputed with the oracle here and its first
    differing codes and scales are reported."""
    import hashlib
    import json
    torch, mx = require_gpu()
    w = synth.QUANT_720P
    with open(DIGESTS) as f:
        doc = json.load(f)
    assert doc["workload"]["N"] == w.N and doc["workload"]["H"] == w.H and doc["workload"]["seed"] == w.seed
    xh = synth.quant_tensor_bf16(w, threads=16)                  # bf16 bit patterns [H, N, d]
    x = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda()
    for rule in ("uos", "ocp", "tfs"):
        c, s = mx.mxattn_quantize(x, rule=RULES[rule][0], axis="last", hadamard=True)
        torch.cuda.synchronize()
        cc, ss = u8(c), u8(s)
        bad = [h for h in range(w.H)
               if hashlib.sha256(cc[h].tobytes() + ss[h].tobytes()).hexdigest() != doc["rules"][rule][h]]
        if bad:
            h = bad[0]
            oc, os_ = _oracle_last(synth.quant_head(w, h), rule, True)
            _assert_same(mxfp4.unpack_nibbles(cc[h]), ss[h], oc, os_, f"full head={h} {rule}")
        assert not bad, f"{rule}: heads {bad} differ from the oracle's digests"


@pytest.mark.parametrize("axis,had", [("last", True), ("last", False), ("rows", False)])
def test_repeatable_bitwise(axis, had):
    """Each quantiser ten times on the same input: bitwise identical codes and scales (a
    race on the LDS staging buffers would show as a run-to-run difference)."""
    torch, mx = require_gpu()
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((8, 3000, 128), generator=g, device="cuda").to(torch.bfloat16)
    outs = [mx.mxattn_quantize(x, rule="uos", axis=axis, hadamard=had) for _ in range(10)]
    torch.cuda.synchronize()
    for c, s in outs[1:]:
        assert torch.equal(c, outs[0][0]) and torch.equal(s, outs[0][1])
