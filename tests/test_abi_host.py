"""Host-only checks of the C ABI: the library loads, exports every entry point that
include/mxattn.h declares, and rejects bad arguments before any HIP call (so these
run without a GPU).  Device pointers here are fake, aligned addresses: every call
below must fail validation and never reach the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxattn.h")


@pytest.fixture(scope="module")
def mx():
    lib = os.path.join(ROOT, "mxfp4_bit_attention_amd", "libmxattn.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()
    import mxfp4_bit_attention_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mxattn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("mxattn_quantize", "mxattn_forward", "mxattn_forward_quantized",
              "mxattn_forward_workspace_bytes", "mxattn_kv_tile", "mxattn_padded_tokens",
              "mxattn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(mx):
    lib = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(mx.EXPORTED)


def test_constants(mx):
    assert mx.mxattn_kv_tile() == 128
    assert mx.mxattn_padded_tokens(75600) == 75648
    assert mx.mxattn_padded_tokens(128) == 128 and mx.mxattn_padded_tokens(1) == 128
    assert mx.mxattn_padded_tokens(-1) == -1
    ws = mx.mxattn_forward_workspace_bytes(1, 40, 75600, 75600, 128)
    n = 40 * 75600 * 128
    r256 = lambda b: -(-b // 256) * 256
    # K^ codes, V^T codes (128-padded tokens), and both scale sets in the attention kernel's
    # operand order (4 bytes per padded key per head each), every piece 256-byte aligned
    assert ws == r256(n // 2) + r256(40 * 128 * 75648 // 2) + 2 * r256(40 * 75648 * 4)
    assert ws % 256 == 0
    assert mx.mxattn_forward_workspace_bytes(1, 1, 1, 1, 96) == 0
    assert mx.mxattn_forward_workspace_bytes(0, 1, 1, 1, 64) == 0


FAKE = 1 << 20      # an aligned address that is never dereferenced
MISALIGNED = FAKE + 4


def q_call(mx, x=FAKE, dtype=1, batch=1, rows=4, cols=128, axis=0, kind=0, qmax=7.25, had=0,
           codes=FAKE, scales=FAKE):
    return mx.LIB.mxattn_quantize(ctypes.c_void_p(x), dtype, batch, rows, cols, axis, kind, qmax, had,
                                  ctypes.c_void_p(codes), ctypes.c_void_p(scales), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=0), -1, "null"),
    (dict(codes=0), -1, "null"),
    (dict(dtype=7), -1, "dtype"),
    (dict(x=MISALIGNED), -1, "aligned"),
    (dict(rows=0), -1, ">= 1"),
    (dict(cols=48), -1, "multiple of 32"),
    (dict(cols=96, had=1), -2, "64 or 128"),
    (dict(axis=5), -1, "axis"),
    (dict(axis=1, had=1), -1, "Hadamard"),
    (dict(axis=1, cols=7), -1, "even"),
    (dict(axis=1, cols=1 << 17), -1, "cols <= 65536"),
    (dict(kind=9), -1, "rule"),
    (dict(kind=2, qmax=3.0), -1, "(4, 8]"),
    (dict(kind=2, qmax=float("nan")), -1, "(4, 8]"),
    (dict(rows=1 << 40), -1, "too large"),
])
def test_quantize_rejects_bad_arguments(mx, kw, status, msg):
    assert q_call(mx, **kw) == status
    assert msg in mx.mxattn_last_error()


def f_call(mx, Q=FAKE, dtype=1, B=1, H=2, Nq=256, Nkv=256, d=128, scale=0.125, had=1, pnq=1, kind=0,
           qmax=0.0, O=FAKE, ws=FAKE * 2, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = mx.mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d) if d in (64, 128) else 1 << 30
    p = ctypes.c_void_p
    return mx.LIB.mxattn_forward(p(Q), p(FAKE), p(FAKE), dtype, B, H, Nq, Nkv, d, scale, had, pnq, kind,
                                 qmax, p(O), p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=0), -1, "null"),
    (dict(O=MISALIGNED), -1, "aligned"),
    (dict(ws=FAKE + 16), -1, "256-byte"),
    (dict(d=96), -2, "64 or 128"),
    (dict(Nkv=0), -1, ">= 1"),
    (dict(scale=0.0), -1, "softmax_scale"),
    (dict(scale=float("inf")), -1, "softmax_scale"),
    (dict(ws_bytes=100), -3, "workspace"),
    (dict(kind=2, qmax=9.0), -1, "(4, 8]"),
    (dict(H=70000), -1, "65535"),
    (dict(Nkv=(1 << 24) + 1), -1, "tokens per head"),
    (dict(Nq=(1 << 24) + 1), -1, "tokens per head"),
])
def test_forward_rejects_bad_arguments(mx, kw, status, msg):
    assert f_call(mx, **kw) == status
    assert msg in mx.mxattn_last_error()


def test_quant_error_rejects_bad_arguments(mx):
    p = ctypes.c_void_p
    L = mx.LIB
    assert L.mxattn_quant_error(p(FAKE), 1, 1, 4, 128, 0, 0, 7.25, 0, None, None) == -1
    assert "null" in mx.mxattn_last_error()
    assert L.mxattn_quant_error(p(FAKE), 1, 1, 4, 128, 0, 0, 7.25, 0, p(FAKE + 4), None) == -1
    assert "8-byte" in mx.mxattn_last_error()
    assert L.mxattn_quant_error(p(FAKE), 1, 1, 4, 96, 0, 0, 7.25, 1, p(FAKE), None) == -2
    assert L.mxattn_quant_error(p(FAKE), 1, 1, 4, 128, 1, 0, 7.25, 1, p(FAKE), None) == -1
    assert "Hadamard" in mx.mxattn_last_error()


def test_forward_quantized_rejects_bad_arguments(mx):
    p = ctypes.c_void_p
    L = mx.LIB
    args = [p(FAKE)] * 6 + [1, 1, 16, 16, 128, 0.1, 1, 0, 0.0, p(FAKE), 1, None, None, None]
    assert L.mxattn_forward_quantized(*args[:6], *args[6:17], p(FAKE), None, None) == -1
    assert "both" in mx.mxattn_last_error()
    bad = list(args)
    bad[0] = p(0)
    assert L.mxattn_forward_quantized(*bad) == -1
    bad = list(args)
    bad[16] = 3
    assert L.mxattn_forward_quantized(*bad) == -1 and "out_dtype" in mx.mxattn_last_error()
    bad = list(args)
    bad[10] = 32
    assert L.mxattn_forward_quantized(*bad) == -2


def test_arrange_scales_rejects_bad_arguments(mx):
    p = ctypes.c_void_p
    L = mx.LIB
    args = [p(FAKE), p(FAKE), 1, 2, 300, 128, p(FAKE), p(FAKE), None]
    bad = list(args)
    bad[6] = None
    assert L.mxattn_arrange_scales(*bad) == -1 and "null" in mx.mxattn_last_error()
    bad = list(args)
    bad[1] = p(MISALIGNED)
    assert L.mxattn_arrange_scales(*bad) == -1 and "aligned" in mx.mxattn_last_error()
    bad = list(args)
    bad[5] = 96
    assert L.mxattn_arrange_scales(*bad) == -2
    bad = list(args)
    bad[4] = 0
    assert L.mxattn_arrange_scales(*bad) == -1 and ">= 1" in mx.mxattn_last_error()
    bad = list(args)
    bad[4] = (1 << 24) + 1
    assert L.mxattn_arrange_scales(*bad) == -1 and "tokens per head" in mx.mxattn_last_error()


def test_forward_arranged_rejects_bad_arguments(mx):
    p = ctypes.c_void_p
    L = mx.LIB
    args = [p(FAKE)] * 6 + [1, 1, 16, 16, 128, 0.1, 1, 0, 0.0, p(FAKE), 1, None]
    bad = list(args)
    bad[3] = None
    assert L.mxattn_forward_arranged(*bad) == -1 and "null" in mx.mxattn_last_error()
    bad = list(args)
    bad[5] = p(MISALIGNED)
    assert L.mxattn_forward_arranged(*bad) == -1 and "aligned" in mx.mxattn_last_error()
    bad = list(args)
    bad[16] = 3
    assert L.mxattn_forward_arranged(*bad) == -1 and "out_dtype" in mx.mxattn_last_error()
    bad = list(args)
    bad[10] = 32
    assert L.mxattn_forward_arranged(*bad) == -2
    bad = list(args)
    bad[11] = -1.0
    assert L.mxattn_forward_arranged(*bad) == -1 and "softmax_scale" in mx.mxattn_last_error()
    bad = list(args)
    bad[13] = 7
    assert L.mxattn_forward_arranged(*bad) == -1 and "rule" in mx.mxattn_last_error()


def test_binding_rule_parsing(mx):
    assert mx.rule_args("uos") == (0, 7.25)
    assert mx.rule_args("OCP")[0] == 1
    assert mx.rule_args(("ceil", 6.0)) == (2, 6.0)
    with pytest.raises(ValueError):
        mx.rule_args("nearest")


def n_call(mx, Q=FAKE, dtype=1, B=1, H=2, Nq=256, Nkv=256, d=128, scale=0.125, kind=0, qmax=0.0, O=FAKE):
    p = ctypes.c_void_p
    return mx.LIB.mxattn_forward_noalloc(p(Q), p(FAKE), p(FAKE), dtype, B, H, Nq, Nkv, d, scale, 1, 1, kind,
                                         qmax, p(O), None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Q=0), -1, "null"),
    (dict(O=MISALIGNED), -1, "aligned"),
    (dict(d=96), -2, "64 or 128"),
    (dict(scale=0.0), -1, "softmax_scale"),
    (dict(kind=2, qmax=9.0), -1, "(4, 8]"),
    # 40 heads x 75,600 keys at d = 128 need about 435 MB of workspace: beyond the array
    (dict(H=40, Nq=75600, Nkv=75600), -3, "bytes of scratch"),
])
def test_forward_noalloc_rejects_before_any_hip_call(mx, kw, status, msg):
    """Every rejection of the allocation-free forward happens on the host, before the
    library's array is looked up or anything is launched (so these run without a GPU)."""
    assert n_call(mx, **kw) == status
    assert msg in mx.mxattn_last_error() and "mxattn_forward_noalloc" in mx.mxattn_last_error()


def test_forward_noalloc_size_limit_matches_the_workspace_size(mx):
    """The largest call the array admits is the one whose mxattn_forward workspace fits in it."""
    limit = mx.NOALLOC_SCRATCH_BYTES
    assert mx.mxattn_forward_workspace_bytes(1, 40, 32760, 32760, 128) <= limit       # Wan2.2-480p fits
    assert mx.mxattn_forward_workspace_bytes(1, 40, 75600, 75600, 128) > limit        # Wan2.2-720p does not
    src = open(HEADER).read()
    assert "#define MXATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)" in src and limit == 256 << 20
