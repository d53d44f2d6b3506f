"""Host-only checks of the Python binding's argument validation.

The C ABI receives plain pointers and cannot see tensor sizes, so the binding is
the one place that can refuse a caller buffer of the wrong shape, dtype or device
before a kernel writes past it.  Shape and dtype checks run before the device
check, so every rejection here is exercised with CPU tensors; a call whose every
shape is right is then refused for not being on the GPU.
"""
import os

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mx():
    lib = os.path.join(ROOT, "mxfp4_bit_attention_amd", "libmxattn.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()
    import mxfp4_bit_attention_amd as m
    return m


u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16


def z(*shape, dtype=u8):
    return torch.zeros(shape, dtype=dtype)


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_quantize_rejects_wrong_buffers(mx):
    x = z(2, 100, 64, dtype=f32)
    raises("x must be float32, bfloat16", mx.mxattn_quantize, z(2, 100, 64, dtype=torch.float16))
    raises("x must be 2-D or 3-D", mx.mxattn_quantize, z(1, 2, 100, 64, dtype=f32))
    raises(r"codes must have shape \(2, 100, 32\)", mx.mxattn_quantize, x, codes=z(2, 100, 31))
    raises(r"scales must have shape \(2, 100, 2\)", mx.mxattn_quantize, x, scales=z(2, 100, 4))
    raises("codes must be uint8", mx.mxattn_quantize, x, codes=z(2, 100, 32, dtype=f32))
    # the transposed token-axis layout: P = 128 padded tokens
    raises(r"codes must have shape \(2, 64, 64\)", mx.mxattn_quantize, x, axis="rows", codes=z(2, 64, 50))
    raises(r"scales must have shape \(2, 64, 4\)", mx.mxattn_quantize, x, axis="rows", scales=z(2, 64, 3))
    raises("axis must be", mx.mxattn_quantize, x, axis="cols")
    raises("tensors must be on the GPU", mx.mxattn_quantize, x, codes=z(2, 100, 32), scales=z(2, 100, 2))


def test_quantize_2d_input_takes_2d_or_3d_outputs(mx):
    x = z(100, 64, dtype=f32)
    raises(r"codes must have shape \(100, 32\)", mx.mxattn_quantize, x, codes=z(100, 33))
    raises(r"codes must have shape \(1, 100, 32\)", mx.mxattn_quantize, x, codes=z(2, 100, 32))
    raises("tensors must be on the GPU", mx.mxattn_quantize, x, codes=z(100, 32))
    raises("tensors must be on the GPU", mx.mxattn_quantize, x, codes=z(1, 100, 32))


def test_quant_error_rejects_wrong_sums(mx):
    x = z(4, 64, dtype=bf16)
    raises(r"sums must have shape \(3,\)", mx.mxattn_quant_error, x, sums=z(4, dtype=torch.float64))
    raises("sums must be float64", mx.mxattn_quant_error, x, sums=z(3, dtype=f32))
    raises("tensors must be on the GPU", mx.mxattn_quant_error, x, sums=z(3, dtype=torch.float64))


def test_forward_rejects_wrong_buffers(mx):
    B, H, Nq, Nkv, d = 1, 2, 10, 33, 64
    q, k, v = z(B, H, Nq, d, dtype=bf16), z(B, H, Nkv, d, dtype=bf16), z(B, H, Nkv, d, dtype=bf16)
    f = mx.mxattn_forward
    raises(r"v must have shape \(1, 2, 33, 64\)", f, q, k, z(B, H, Nkv + 1, d, dtype=bf16), 0.125)
    raises("k must be bfloat16", f, q, z(B, H, Nkv, d, dtype=f32), v, 0.125)
    raises(r"out must have shape \(1, 2, 10, 64\)", f, q, k, v, 0.125, out=z(B, H, Nq, 32, dtype=bf16))
    # the kernel writes O in q's dtype: a float32 out for bf16 q would hold packed bf16 bits
    raises("out must be bfloat16", f, q, k, v, 0.125, out=z(B, H, Nq, d, dtype=f32))
    wsb = mx.mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d)
    raises("workspace must be a 1-D uint8 tensor", f, q, k, v, 0.125, workspace=z(wsb // 4, dtype=f32))
    raises(f"workspace has {wsb - 1} bytes, needs {wsb}", f, q, k, v, 0.125, workspace=z(wsb - 1))
    raises("tensors must be on the GPU", f, q, k, v, 0.125, out=z(B, H, Nq, d, dtype=bf16), workspace=z(wsb))


def _quantized(B=1, H=2, Nq=10, Nkv=200, d=128):
    P = -(-Nkv // 128) * 128
    return dict(qc=z(B, H, Nq, d // 2), qs=z(B, H, Nq, d // 32), kc=z(B, H, Nkv, d // 2),
                ks=z(B, H, Nkv, d // 32), vtc=z(B, H, d, P // 2), vts=z(B, H, d, P // 32)), P


@pytest.mark.parametrize("bad,match", [
    ("qs", r"qs must have shape \(1, 2, 10, 4\)"),
    ("kc", r"kc must have shape \(1, 2, 200, 64\)"),
    ("ks", r"ks must have shape \(1, 2, 200, 4\)"),
    ("vtc", r"vtc must have shape \(1, 2, 128, 128\)"),
    ("vts", r"vts must have shape \(1, 2, 128, 8\)"),
])
def test_forward_quantized_rejects_each_operand(mx, bad, match):
    ops, _ = _quantized()
    ops[bad] = z(*ops[bad].shape[:-1], ops[bad].shape[-1] + 1)
    raises(match, mx.mxattn_forward_quantized, *ops.values(), 200, 0.125)


def test_forward_quantized_checks_nkv_against_the_operands(mx):
    ops, _ = _quantized()
    raises(r"kc must have shape \(1, 2, 201, 64\)", mx.mxattn_forward_quantized, *ops.values(), 201, 0.125)
    # 129 keys would need two kv tiles of V^T: 256 padded tokens
    ops2, _ = _quantized(Nkv=129)
    ops2["vtc"] = z(1, 2, 128, 64)
    raises(r"vtc must have shape \(1, 2, 128, 128\)", mx.mxattn_forward_quantized, *ops2.values(), 129, 0.125)
    raises("Nkv must be >= 1", mx.mxattn_forward_quantized, *ops.values(), 0, 0.125)


def test_forward_quantized_rejects_wrong_out_and_dtype(mx):
    ops, _ = _quantized()
    f = mx.mxattn_forward_quantized
    raises("out must be bfloat16", f, *ops.values(), 200, 0.125, out_dtype=bf16, out=z(1, 2, 10, 128, dtype=f32))
    raises(r"out must have shape \(1, 2, 10, 128\)", f, *ops.values(), 200, 0.125, out=z(1, 2, 10, 64, dtype=f32))
    raises("out_dtype must be float32 or bfloat16", f, *ops.values(), 200, 0.125, out_dtype=torch.float16)
    bad = dict(ops, qc=z(1, 2, 10, 64, dtype=torch.int8))
    raises("qc must be uint8", f, *bad.values(), 200, 0.125)
    raises("tensors must be on the GPU", f, *ops.values(), 200, 0.125)


def test_arrange_scales_and_arranged_entry_reject_wrong_buffers(mx):
    ops, P = _quantized()
    raises(r"vts must have shape \(1, 2, 128, 8\)", mx.mxattn_arrange_scales, ops["ks"], z(1, 2, 128, 7), 200)
    raises(r"ks must have shape \(1, 2, 201, 4\)", mx.mxattn_arrange_scales, ops["ks"], ops["vts"], 201)
    raises("tensors must be on the GPU", mx.mxattn_arrange_scales, ops["ks"], ops["vts"], 200)
    f = mx.mxattn_forward_arranged
    args = [ops["qc"], ops["qs"], ops["kc"], z(1, 2, P * 4), ops["vtc"], z(1, 2, P * 4)]
    raises(r"ksa must have shape \(1, 2, 1024\)", f, *args[:3], z(1, 2, P), *args[4:], 200, 0.125)
    raises(r"vtsa must have shape \(1, 2, 1024\)", f, *args[:5], z(1, 2, P * 4 + 16), 200, 0.125)
    raises("tensors must be on the GPU", f, *args, 200, 0.125)
