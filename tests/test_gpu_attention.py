"""GPU parity of the fused MXFP4 attention against the oracle.

Bars: O within relative L2 5e-3 of the oracle on identical quantised Q/K/V
(the quantisers are bit-exact, so the whole pipeline shares its operands with
the oracle); fewer than 1e-3 of the P^ codes differ (a changed block exponent
counts as all 32 codes of the block); V = 1 gives O = 1 within 1e-6 with PNQ
and visibly not without.  The oracle replays the kernel's kv tile width.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import attention as ora
from oracle import mxfp4
from _gpu_helpers import RULES, p_code_mismatch, rel_l2, require_gpu, to_device, u8

pytestmark = pytest.mark.gpu
REL_L2 = 5e-3
P_MISMATCH = 1e-3


def _oracle_inputs(Q, K, V, rule, had, P):
    Qc, Qs = ora.quantize_qk(Q, rule, had)
    Kc, Ks = ora.quantize_qk(K, rule, had)
    Vc, Vs = ora.quantize_v(V, rule, P)
    return Qc, Qs, Kc, Ks, Vc, Vs


def _device_quantized(q):
    """Oracle-quantised operands (one head) -> packed device tensors [1, 1, ...]."""
    import torch
    Qc, Qs, Kc, Ks, Vc, Vs = q
    pk = lambda c: torch.from_numpy(mxfp4.pack_nibbles(c)[None, None].copy()).cuda()
    sc = lambda s: torch.from_numpy(np.ascontiguousarray(s)[None, None].copy()).cuda()
    return pk(Qc), sc(Qs), pk(Kc), sc(Ks), pk(Vc), sc(Vs)


@pytest.mark.parametrize("rule", ["uos", "ocp", "tfs"])
@pytest.mark.parametrize("pnq", [True, False])
@pytest.mark.parametrize("had", [True, False])
def test_tiny_pipeline(rule, pnq, had):
    """The tiny workload (H=2, N=256, d=64, fp32) through mxattn_forward."""
    torch, mx = require_gpu()
    w = synth.TINY
    Q, K, V = (synth.attn_tensor(w, t) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
    scale = float(np.float32(w.softmax_scale))
    O = mx.mxattn_forward(to_device(Q, "f32"), to_device(K, "f32"), to_device(V, "f32"), scale,
                          hadamard=had, pnq=pnq, rule=RULES[rule][0])
    torch.cuda.synchronize()
    Og = O.cpu().numpy()
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(w.N)
    for h in range(w.H):
        Oo = ora.mx_attention_pipeline(Q[0, h], K[0, h], V[0, h], scale, had, pnq, RULES[rule][1], Bc, P)
        err = rel_l2(Og[0, h], Oo)
        assert err < REL_L2, f"head {h}: rel-L2 {err:.2e}"


@pytest.mark.parametrize("rule", ["uos", "ocp", "tfs"])
@pytest.mark.parametrize("Nq,Nkv,d", [(256, 256, 64), (300, 1000, 128), (64, 33, 128), (1, 129, 64),
                                      (517, 1, 128), (2048, 4096, 128)])
def test_quantized_entry_p_codes(rule, Nq, Nkv, d):
    """mxattn_forward_quantized on oracle-quantised operands: O and the P^ dump."""
    torch, mx = require_gpu()
    rng = np.random.default_rng(Nq * 31 + Nkv + d)
    Q = rng.standard_normal((Nq, d)).astype(np.float32) * 1.5
    K = rng.standard_normal((Nkv, d)).astype(np.float32) * 1.5
    V = rng.standard_normal((Nkv, d)).astype(np.float32)
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = _oracle_inputs(Q, K, V, RULES[rule][1], True, P)
    O, pc, ps = mx.mxattn_forward_quantized(*_device_quantized(q), Nkv, scale, pnq=True,
                                            p_rule=RULES[rule][0], dump_p=True)
    torch.cuda.synchronize()
    Oo, opc, ops = ora.flash_attention_mx(*q, Nkv, scale, True, RULES[rule][1], Bc, return_p=True)
    err = rel_l2(O.cpu().numpy()[0, 0], Oo)
    assert err < REL_L2, f"rel-L2 {err:.2e}"
    mm = p_code_mismatch(u8(pc)[0, 0], u8(ps)[0, 0], opc, ops, Nkv)
    assert mm < P_MISMATCH, f"P^ code mismatch {mm:.2e}"


@pytest.mark.parametrize("rule", ["uos", "ocp"])
@pytest.mark.parametrize("Nq,Nkv,d", [(300, 1000, 128), (64, 33, 64), (129, 4096, 128)])
def test_direct_placement_p_codes(rule, Nq, Nkv, d):
    """pnq = False (the direct placement of Figure 4(C): l sums the unquantised P~, O~
    uses P^): the dumped P^ codes and O against the oracle's direct-placement arm."""
    torch, mx = require_gpu()
    rng = np.random.default_rng(Nq * 13 + Nkv + d)
    Q = rng.standard_normal((Nq, d)).astype(np.float32) * 1.5
    K = rng.standard_normal((Nkv, d)).astype(np.float32) * 1.5
    V = rng.standard_normal((Nkv, d)).astype(np.float32)
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = _oracle_inputs(Q, K, V, RULES[rule][1], True, P)
    O, pc, ps = mx.mxattn_forward_quantized(*_device_quantized(q), Nkv, scale, pnq=False,
                                            p_rule=RULES[rule][0], dump_p=True)
    torch.cuda.synchronize()
    Oo, opc, ops = ora.flash_attention_mx(*q, Nkv, scale, False, RULES[rule][1], Bc, return_p=True)
    err = rel_l2(O.cpu().numpy()[0, 0], Oo)
    assert err < REL_L2, f"rel-L2 {err:.2e}"
    mm = p_code_mismatch(u8(pc)[0, 0], u8(ps)[0, 0], opc, ops, Nkv)
    assert mm < P_MISMATCH, f"P^ code mismatch {mm:.2e}"


@pytest.mark.parametrize("rule", ["oas", "q7.5"])
@pytest.mark.parametrize("Nq,Nkv,d", [(300, 1000, 128), (64, 33, 64)])
def test_ablation_rules_p_codes(rule, Nq, Nkv, d):
    """The other CEIL rules of the scale-rule ablation (q = 7 and 7.5) on the P~ tiles."""
    test_quantized_entry_p_codes(rule, Nq, Nkv, d)


@pytest.mark.parametrize("rule", ["uos"])
def test_long_kv_sequence_p_codes(rule):
    """Five query rows against 150,001 keys (1,172 kv tiles, a ragged last one): every
    output row and every P^ code against the oracle, so the running max and the rescale
    are exercised over a sequence twice as long as the headline one."""
    test_quantized_entry_p_codes(rule, 5, 150001, 128)


@pytest.mark.parametrize("B,H,Nq,Nkv,d,dtype", [(2, 2, 300, 700, 128, "bf16"), (3, 1, 129, 257, 64, "f32"),
                                                (1, 1, 5, 150001, 128, "bf16")])
def test_batched_cross_shape_pipeline(B, H, Nq, Nkv, d, dtype):
    """B > 1 and N_q != N_kv through mxattn_forward (Hadamard, UOS, PNQ); every row of
    every (batch, head) against the oracle pipeline."""
    torch, mx = require_gpu()
    rng = np.random.default_rng(B * 1000 + Nq + Nkv + d)
    Q = rng.standard_normal((B, H, Nq, d)).astype(np.float32)
    K = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    V = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    if dtype == "bf16":
        Q, K, V = (synth.bf16_to_f32(synth.round_to_bf16(a)) for a in (Q, K, V))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    O = mx.mxattn_forward(*(to_device(a, dtype) for a in (Q, K, V)), scale, hadamard=True, pnq=True, rule="uos")
    torch.cuda.synchronize()
    Og = O.float().cpu().numpy()
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    for b in range(B):
        for h in range(H):
            Oo = ora.mx_attention_pipeline(Q[b, h], K[b, h], V[b, h], scale, True, True, mxfp4.UOS, Bc, P)
            err = rel_l2(Og[b, h], Oo)
            assert err < REL_L2, f"batch {b} head {h}: rel-L2 {err:.2e}"


@pytest.mark.parametrize("rule", ["uos", "ocp", "tfs"])
def test_pnq_sum_to_one_on_gpu(rule):
    """V = 1: PNQ gives O = 1 within 1e-6; direct placement visibly does not."""
    torch, mx = require_gpu()
    w = synth.TINY
    Q, K = (synth.attn_tensor(w, t) for t in (synth.Q_ID, synth.K_ID))
    ones = np.ones_like(Q)
    args = [to_device(a, "f32") for a in (Q, K, ones)]
    O1 = mx.mxattn_forward(*args, w.softmax_scale, hadamard=True, pnq=True, rule=RULES[rule][0])
    O0 = mx.mxattn_forward(*args, w.softmax_scale, hadamard=True, pnq=False, rule=RULES[rule][0])
    torch.cuda.synchronize()
    assert (O1 - 1).abs().max().item() < 1e-6
    assert (O0 - 1).abs().max().item() > 1e-2


def test_mid_size_bf16_all_rows():
    """B=1, H=2, N=4096, d=128, bf16 outlier law, whole pipeline, every row compared."""
    torch, mx = require_gpu()
    w = dataclasses.replace(synth.WAN_480P, H=2, N=4096)
    Q, K, V = (synth.attn_tensor(w, t) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
    O = mx.mxattn_forward(to_device(Q, "bf16"), to_device(K, "bf16"), to_device(V, "bf16"),
                          float(np.float32(w.softmax_scale)), hadamard=True, pnq=True, rule="uos")
    torch.cuda.synchronize()
    Og = O.float().cpu().numpy()
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(w.N)
    for h in range(w.H):
        Oo = ora.mx_attention_pipeline(Q[0, h], K[0, h], V[0, h], float(np.float32(w.softmax_scale)),
                                       True, True, mxfp4.UOS, Bc, P)
        err = rel_l2(Og[0, h], Oo)
        assert err < REL_L2, f"head {h}: rel-L2 {err:.2e}"


def _full_size_case(w, rows_per_head=32, rule="uos", pnq=True):
    """Full-size workload on the device; heads 0 and H-1 come from the seeded host
    generator (the oracle compares sampled rows of those), the other heads are
    filled on the device with the same Gaussian law."""
    gpu_rule, ora_rule = RULES[rule]
    torch, mx = require_gpu()
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    dev = [torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3)]
    heads = [0, w.H - 1]
    host = {}
    for tid in (synth.Q_ID, synth.K_ID, synth.V_ID):
        for h in heads:
            x = synth.attn_head(w, tid, h)
            host[tid, h] = x
            dev[tid][0, h] = to_device(x, "bf16")
    scale = float(np.float32(w.softmax_scale))
    O = mx.mxattn_forward(*dev, scale, hadamard=True, pnq=pnq, rule=gpu_rule)
    torch.cuda.synchronize()
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(w.N)
    rng = np.random.default_rng(w.seed)
    for h in heads:
        rows = np.sort(rng.choice(w.N, rows_per_head, replace=False))
        rows = np.unique(np.concatenate([rows, [0, w.N - 1]]))
        Og = O[0, h, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        # quantisation is row-local, so quantising only the sampled query rows is exact
        Qc, Qs = ora.quantize_qk(host[synth.Q_ID, h][rows], ora_rule, True)
        Kc, Ks = ora.quantize_qk(host[synth.K_ID, h], ora_rule, True)
        Vc, Vs = ora.quantize_v(host[synth.V_ID, h], ora_rule, P)
        Oo = ora.flash_attention_mx(Qc, Qs, Kc, Ks, Vc, Vs, w.N, scale, pnq, ora_rule, Bc)
        err = rel_l2(Og, Oo)
        assert err < REL_L2, f"{w.name} {rule} head {h}: rel-L2 {err:.2e}"


def test_full_size_wan480p_sampled_rows():
    _full_size_case(synth.WAN_480P)


def test_full_size_wan720p_sampled_rows():
    _full_size_case(synth.WAN_720P)


@pytest.mark.parametrize("rule", ["ocp", "tfs"])
def test_full_size_wan720p_sampled_rows_other_rules(rule):
    """The benchmark's rule ablation runs the full Wan2.2-720p step under every rule; the
    OCP floor rule and TFS (q = 6) against the oracle at that size too."""
    _full_size_case(synth.WAN_720P, rows_per_head=16, rule=rule)


def test_full_size_wan720p_sampled_rows_direct_placement():
    """Direct placement (pnq = 0: the row sum from the unquantised P~) at full size."""
    _full_size_case(synth.WAN_720P, rows_per_head=16, pnq=False)


def test_full_size_hunyuan720p_sampled_rows():
    _full_size_case(synth.HUNYUAN_720P)


def test_full_size_d64_sampled_rows():
    """The Wan2.2-720p token count at head dim 64 (the d = 64 kernel at full length)."""
    w = dataclasses.replace(synth.WAN_720P, d=64, softmax_scale=0.125, name="wan2.2-720p-h40-n75600-d64")
    _full_size_case(w)


@pytest.mark.parametrize("B,H,Nq,Nkv", [(2, 20, 75_600, 75_600), (1, 40, 75_600, 512), (1, 40, 2048, 2048),
                                        (1, 40, 8192, 8192)])
def test_benchmark_extra_shapes_sampled_rows(B, H, Nq, Nkv):
    """The further shapes the benchmark times (B = 2 x H = 20, a 512-key cross-attention
    shape, 2,048 and 8,192 tokens), on the same seeded unit-Gaussian bf16 inputs and through
    the same call: sampled rows of the first and the last head against the oracle."""
    torch, mx = require_gpu()
    d = 128
    gen = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda n: torch.randn((B, H, n, d), generator=gen, device="cuda").to(torch.bfloat16)
    q, k, v = mk(Nq), mk(Nkv), mk(Nkv)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    O = mx.mxattn_forward(q, k, v, scale, hadamard=True, pnq=True, rule="uos")
    torch.cuda.synchronize()
    gpu_rule, ora_rule = RULES["uos"]
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    rng = np.random.default_rng(1000 * B + Nkv)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = np.unique(np.concatenate([rng.choice(Nq, 16, replace=False), [0, Nq - 1]]))
        host = lambda t: t[b, h].float().cpu().numpy()
        Og = O[b, h, torch.from_numpy(rows).cuda()].float().cpu().numpy()
        Qc, Qs = ora.quantize_qk(host(q)[rows], ora_rule, True)
        Kc, Ks = ora.quantize_qk(host(k), ora_rule, True)
        Vc, Vs = ora.quantize_v(host(v), ora_rule, P)
        Oo = ora.flash_attention_mx(Qc, Qs, Kc, Ks, Vc, Vs, Nkv, scale, True, ora_rule, Bc)
        err = rel_l2(Og, Oo)
        assert err < REL_L2, f"B={B} H={H} Nq={Nq} Nkv={Nkv} head ({b}, {h}): rel-L2 {err:.2e}"


@pytest.mark.parametrize("d", [128, 64])
def test_repeatable_bitwise(d):
    """The forward ten times, and the quantised entry with its P^ dump ten times, on the
    same inputs: bitwise identical outputs and dumps (a race on the three-stage LDS ring,
    its DMAs or the barrier would show as a run-to-run difference)."""
    torch, mx = require_gpu()
    g = torch.Generator(device="cuda").manual_seed(1)
    q, k, v = (torch.randn((1, 3, 3000, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    outs = [mx.mxattn_forward(q, k, v, d ** -0.5, hadamard=True, pnq=True, rule="uos") for _ in range(10)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    ops = _device_operands(1, 2, 700, 1500, d, seed=d)
    dumps = [mx.mxattn_forward_quantized(*ops, 1500, d ** -0.5, pnq=True, p_rule="uos", dump_p=True) for _ in range(10)]
    torch.cuda.synchronize()
    for o, pc, ps in dumps[1:]:
        assert torch.equal(o, dumps[0][0]) and torch.equal(pc, dumps[0][1]) and torch.equal(ps, dumps[0][2])


@pytest.mark.parametrize("dtype,d,had,rule", [("bf16", 128, True, "uos"), ("bf16", 128, False, "ocp"),
                                              ("f32", 64, True, "tfs"), ("f32", 128, True, "q7.5")])
def test_fused_q_quantisation_is_bitwise_the_quantiser(dtype, d, had, rule):
    """mxattn_forward rotates and quantises Q inside the attention kernel: its output is
    bitwise the output of mxattn_quantize(Q) followed by mxattn_forward_quantized on the
    same K^ and V^ (a row holding NaN and Inf included).  Nq = 300 leaves one wave with
    both real and padded query rows, and the ragged last kv tile (105 keys) has keys in
    both of its 64-key chunks, so the last P^V MFMAs run right before the epilogue's
    divergent branch."""
    torch, mx = require_gpu()
    rng = np.random.default_rng(d + (7 if had else 0))
    B, H, Nq, Nkv = 1, 3, 300, 617
    Q = (rng.standard_normal((B, H, Nq, d)) * 2).astype(np.float32)
    K = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    V = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    Q[0, 1, 7, 3] = np.nan
    Q[0, 2, 11, 100 % d] = np.inf
    if dtype == "bf16":
        Q, K, V = (synth.bf16_to_f32(synth.round_to_bf16(a)) for a in (Q, K, V))
    q, k, v = (to_device(a, dtype) for a in (Q, K, V))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    r = RULES[rule][0]
    O = mx.mxattn_forward(q, k, v, scale, hadamard=had, pnq=True, rule=r)
    qc, qs = mx.mxattn_quantize(q.view(-1, Nq, d), rule=r, axis="last", hadamard=had)
    kc, ks = mx.mxattn_quantize(k.view(-1, Nkv, d), rule=r, axis="last", hadamard=had)
    vc, vs = mx.mxattn_quantize(v.view(-1, Nkv, d), rule=r, axis="rows")
    sh = lambda t: t.view(B, H, *t.shape[1:])
    O2 = mx.mxattn_forward_quantized(sh(qc), sh(qs), sh(kc), sh(ks), sh(vc), sh(vs), Nkv, scale, pnq=True,
                                     p_rule=r, out_dtype=O.dtype)
    torch.cuda.synchronize()
    iv = torch.int16 if O.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(O.view(iv), O2.view(iv))


@pytest.mark.parametrize("d,Nkv", [(128, 617), (128, 200_000), (64, 617), (64, 400_000)])
def test_forward_joint_and_separate_kv_quantisation(d, Nkv):
    """The forward quantises a small K and V (up to 128 MiB each) in one joint launch and a
    larger one in two launches (200,000 and 400,000 keys x 3 heads in bf16 are above that
    size at d = 128 and 64): either way its output is bitwise that of mxattn_quantize on
    Q, K and V followed by mxattn_forward_quantized."""
    torch, mx = require_gpu()
    B, H, Nq = 1, 3, 300
    g = torch.Generator(device="cuda").manual_seed(d + Nkv)
    q, k, v = (torch.randn((B, H, n, d), generator=g, device="cuda").to(torch.bfloat16) for n in (Nq, Nkv, Nkv))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    O = mx.mxattn_forward(q, k, v, scale, hadamard=True, pnq=True, rule="uos")
    qc, qs = mx.mxattn_quantize(q.view(-1, Nq, d), rule="uos", axis="last", hadamard=True)
    kc, ks = mx.mxattn_quantize(k.view(-1, Nkv, d), rule="uos", axis="last", hadamard=True)
    vc, vs = mx.mxattn_quantize(v.view(-1, Nkv, d), rule="uos", axis="rows")
    sh = lambda t: t.view(B, H, *t.shape[1:])
    O2 = mx.mxattn_forward_quantized(sh(qc), sh(qs), sh(kc), sh(ks), sh(vc), sh(vs), Nkv, scale, pnq=True,
                                     p_rule="uos", out_dtype=O.dtype)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16))


def _arranged_reference(ks, vts, Nkv, d):
    """The order mxattn_arrange_scales documents, written out on the host: per head and
    kv tile j, dword 2 lane + s byte t of K = key 128 j + kappa(t, lane % 32), block
    2s + lane // 32; dword 2 lane + c byte ct of V = channel 32 ct + lane % 32, block
    4 j + 2c + lane // 32."""
    B, H = ks.shape[:2]
    ntiles = vts.shape[-1] // 4
    ka = np.zeros((B, H, ntiles, 64, 2, 4), np.uint8)
    va = np.zeros((B, H, ntiles, 64, 2, 4), np.uint8)
    tiles = np.arange(ntiles)
    for lane in range(64):
        i, g = lane % 32, lane // 32
        for t in range(4):
            kap = 64 * (t // 2) + 32 * ((i // 4) % 2) + 16 * (t % 2) + 4 * (i // 8) + i % 4
            keys = 128 * tiles + kap
            ok = keys < Nkv
            for s in range(d // 64):
                ka[:, :, ok, lane, s, t] = ks[:, :, keys[ok], 2 * s + g]
        for c in range(2):
            for ct in range(d // 32):
                va[:, :, :, lane, c, ct] = vts[:, :, 32 * ct + i, 4 * tiles + 2 * c + g]
    return ka.reshape(B, H, -1), va.reshape(B, H, -1)


def _device_operands(B, H, Nq, Nkv, d, seed):
    torch, mx = require_gpu()
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g, device="cuda") * 1.5
    k = torch.randn((B, H, Nkv, d), generator=g, device="cuda") * 1.5
    v = torch.randn((B, H, Nkv, d), generator=g, device="cuda")
    qc, qs = mx.mxattn_quantize(q.view(-1, Nq, d), rule="uos", axis="last", hadamard=True)
    kc, ks = mx.mxattn_quantize(k.view(-1, Nkv, d), rule="uos", axis="last", hadamard=True)
    vc, vs = mx.mxattn_quantize(v.view(-1, Nkv, d), rule="uos", axis="rows")
    sh = lambda t: t.view(B, H, *t.shape[1:])
    return tuple(map(sh, (qc, qs, kc, ks, vc, vs)))


@pytest.mark.parametrize("B,H,Nkv,d", [(1, 1, 1, 64), (2, 3, 300, 128), (1, 2, 1000, 64), (1, 1, 4096, 128)])
def test_arranged_scales_follow_the_documented_order(B, H, Nkv, d):
    torch, mx = require_gpu()
    qc, qs, kc, ks, vc, vs = _device_operands(B, H, 4, Nkv, d, seed=Nkv + d)
    ksa, vsa = mx.mxattn_arrange_scales(ks, vs, Nkv)
    torch.cuda.synchronize()
    ka, va = _arranged_reference(ks.cpu().numpy(), vs.cpu().numpy(), Nkv, d)
    assert np.array_equal(ksa.cpu().numpy(), ka)
    assert np.array_equal(vsa.cpu().numpy(), va)


@pytest.mark.parametrize("pnq", [True, False])
@pytest.mark.parametrize("B,H,Nq,Nkv,d", [(1, 1, 300, 1000, 128), (2, 2, 64, 33, 64), (1, 1, 1, 129, 64),
                                          (1, 3, 517, 1, 128), (1, 2, 2048, 4096, 128)])
def test_arranged_entry_is_bitwise_the_quantized_entry(B, H, Nq, Nkv, d, pnq):
    """mxattn_forward_arranged runs the kernel variant mxattn_forward uses (scale operands
    loaded directly); on the same operands it must give exactly the caller-layout entry's O."""
    torch, mx = require_gpu()
    qc, qs, kc, ks, vc, vs = _device_operands(B, H, Nq, Nkv, d, seed=Nq * 7 + Nkv + d)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ksa, vsa = mx.mxattn_arrange_scales(ks, vs, Nkv)
    for rule in ("uos", "ocp"):
        o1 = mx.mxattn_forward_quantized(qc, qs, kc, ks, vc, vs, Nkv, scale, pnq=pnq, p_rule=rule)
        o2 = mx.mxattn_forward_arranged(qc, qs, kc, ksa, vc, vsa, Nkv, scale, pnq=pnq, p_rule=rule)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all()
        assert torch.equal(o1, o2), rule


@pytest.mark.parametrize("where", ["q", "k", "v"])
@pytest.mark.parametrize("entry,dtype", [("forward", "f32"), ("forward", "bf16"), ("quantized", "f32")])
def test_non_finite_blocks_propagate_like_the_oracle(where, entry, dtype):
    """A 32-element block holding Inf or NaN is quantised to scale 0xFF (NaN), codes 0
    (Pith review, Axiom ledger axiom 1; Appendix A opening leaves such values to the
    conversion routine).  The oracle, doing IEEE arithmetic on the dequantised operands,
    makes NaN exactly the outputs such a block reaches: a query row's block -> that row;
    a key's block -> every row of the head; a V block (32 tokens of one channel) -> that
    channel in every row.  The GPU must give the same NaN pattern, match the oracle
    everywhere else, and (quantised entry) dump the same P^ codes, NaN rows as 0xFF."""
    torch, mx = require_gpu()
    rng = np.random.default_rng({"q": 1, "k": 2, "v": 3}[where])
    B, H, Nq, Nkv, d = 1, 2, 200, 300, 128
    Q = rng.standard_normal((B, H, Nq, d)).astype(np.float32)
    K = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    V = rng.standard_normal((B, H, Nkv, d)).astype(np.float32)
    if dtype == "bf16":
        Q, K, V = (synth.bf16_to_f32(synth.round_to_bf16(a)) for a in (Q, K, V))
    if where == "q":
        Q[0, 1, 37, 5] = np.nan
    elif where == "k":
        K[0, 0, 250, 70] = np.inf                 # head 0 only: head 1 stays finite
    else:
        V[0, 1, 100, 17] = -np.inf
    scale = float(np.float32(1.0 / np.sqrt(d)))
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    with np.errstate(invalid="ignore", over="ignore"):
        if entry == "forward":
            O = mx.mxattn_forward(*(to_device(a, dtype) for a in (Q, K, V)), scale, hadamard=True, pnq=True,
                                  rule="uos")
            torch.cuda.synchronize()
            Og = O.float().cpu().numpy()
            Oo = np.stack([ora.mx_attention_pipeline(Q[0, h], K[0, h], V[0, h], scale, True, True, mxfp4.UOS, Bc, P)
                           for h in range(H)])[None]
        else:
            qs = [_oracle_inputs(Q[0, h], K[0, h], V[0, h], mxfp4.UOS, True, P) for h in range(H)]
            dev = [torch.cat([_device_quantized(q)[i] for q in qs], dim=1) for i in range(6)]
            O, pc, ps = mx.mxattn_forward_quantized(*dev, Nkv, scale, pnq=True, p_rule="uos", dump_p=True)
            torch.cuda.synchronize()
            Og = O.cpu().numpy()
            res = [ora.flash_attention_mx(*q, Nkv, scale, True, mxfp4.UOS, Bc, return_p=True) for q in qs]
            Oo = np.stack([r[0] for r in res])[None]
            for h in range(H):
                mm = p_code_mismatch(u8(pc)[0, h], u8(ps)[0, h], res[h][1], res[h][2], Nkv)
                assert mm < P_MISMATCH, f"head {h}: P^ code mismatch {mm:.2e}"
    nan_o = np.isnan(Oo)
    expect = {"q": (0, 1, [37], slice(None)), "k": (0, 0, slice(None), slice(None)), "v": (0, 1, slice(None), [17])}
    b, h, rows, cols = expect[where]
    assert nan_o[b, h][rows][:, cols].all()           # the oracle's own reading, checked first
    assert nan_o.sum() == nan_o[b, h][rows][:, cols].size
    assert np.array_equal(np.isnan(Og), nan_o), f"NaN pattern differs: {np.argwhere(np.isnan(Og) != nan_o)[:4]}"
    fin = ~nan_o
    err = rel_l2(Og[fin], Oo[fin])
    assert err < REL_L2, f"finite outputs: rel-L2 {err:.2e}"


@pytest.mark.parametrize("rule", ["uos", "ocp"])
@pytest.mark.parametrize("Nkv", [1, 77, 300])
def test_equal_logits_average_v_exactly(rule, Nkv):
    """Degenerate case of the method: with K = 0 every logit is 0, every P~ = exp(0 - 0)
    is exactly 1 and (a block of ones quantises exactly under every rule here) every P^ is
    1, so PNQ's O is the plain average of the dequantised V^ rows, to fp32 rounding of the
    sums.  Checked against that closed form and against the oracle."""
    torch, mx = require_gpu()
    rng = np.random.default_rng(Nkv)
    Nq, d = 70, 128
    Q = rng.standard_normal((Nq, d)).astype(np.float32)
    K = np.zeros((Nkv, d), np.float32)
    V = rng.standard_normal((Nkv, d)).astype(np.float32)
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    q = _oracle_inputs(Q, K, V, RULES[rule][1], True, P)
    O, pc, ps = mx.mxattn_forward_quantized(*_device_quantized(q), Nkv, 0.125, pnq=True, p_rule=RULES[rule][0],
                                            dump_p=True)
    torch.cuda.synchronize()
    Og = O.cpu().numpy()[0, 0]
    Vd = mxfp4.dequantize_blocks_lastaxis(q[4], q[5]).T[:Nkv]
    mean = Vd.mean(axis=0)
    assert np.abs(Og - mean).max() <= 1e-5 * max(1.0, np.abs(mean).max())
    Oo, opc, ops = ora.flash_attention_mx(*q, Nkv, 0.125, True, RULES[rule][1], Bc, return_p=True)
    assert rel_l2(Og, Oo) < 1e-6
    assert p_code_mismatch(u8(pc)[0, 0], u8(ps)[0, 0], opc, ops, Nkv) == 0.0


def test_largest_query_count():
    """N_q = 2^24, the most query rows per head the ABI accepts (131,072 query tiles in one
    launch, a 2 GiB bf16 Q), against 300 keys: sampled rows -- the first, the last, both
    sides of 2^23 and random ones -- against the oracle on the same inputs."""
    torch, mx = require_gpu()
    Nq, Nkv, d = 1 << 24, 300, 64
    g = torch.Generator(device="cuda").manual_seed(24)
    q = torch.randn((1, 1, Nq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, 1, Nkv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 1, Nkv, d), generator=g, device="cuda").to(torch.bfloat16)
    scale = 0.125
    O = mx.mxattn_forward(q, k, v, scale, hadamard=True, pnq=True, rule="uos")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, (1 << 23) - 1, 1 << 23, Nq - 1],
                                     np.random.default_rng(24).choice(Nq, 27, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Og = O[0, 0, ridx].float().cpu().numpy()
    Qh = q[0, 0, ridx].float().cpu().numpy()
    Kh, Vh = k[0, 0].float().cpu().numpy(), v[0, 0].float().cpu().numpy()
    del q, O
    Bc, P = mx.mxattn_kv_tile(), mx.mxattn_padded_tokens(Nkv)
    Oo = ora.mx_attention_pipeline(Qh, Kh, Vh, scale, True, True, mxfp4.UOS, Bc, P)
    err = rel_l2(Og, Oo)
    assert err < REL_L2, f"rel-L2 {err:.2e}"
