"""Python binding of libmxattn (MXFP4 UOS + PNQ attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmxattn.so`` behind the C ABI declared in ``include/mxattn.h``.
PyTorch supplies device memory and the current stream.  The library must be
built first (``python mxfp4_bit_attention_amd/build.py``); importing this
module raises if it is missing, and nothing here falls back to a CPU path.

Names mirror the C entry points: ``mxattn_quantize``, ``mxattn_quant_error``, ``mxattn_forward``,
``mxattn_forward_quantized``, ``mxattn_arrange_scales``, ``mxattn_forward_arranged``,
``mxattn_forward_noalloc``, ``mxattn_forward_workspace_bytes``,
``mxattn_kv_tile``, ``mxattn_padded_tokens``, ``mxattn_last_error``.
Rules are given as ``"uos"``, ``"ocp"`` or ``("ceil", q)``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxattn.so")

MXATTN_OK = 0
MXATTN_E_INVALID = -1
MXATTN_E_UNSUPPORTED = -2
MXATTN_E_WORKSPACE = -3
MXATTN_E_HIP = -4
MXATTN_F32, MXATTN_BF16 = 0, 1
MXATTN_RULE_UOS, MXATTN_RULE_OCP, MXATTN_RULE_CEIL = 0, 1, 2
MXATTN_AXIS_LAST, MXATTN_AXIS_ROWS = 0, 1

EXPORTED = (
    "mxattn_kv_tile", "mxattn_padded_tokens", "mxattn_quantize", "mxattn_forward_workspace_bytes",
    "mxattn_forward", "mxattn_forward_quantized", "mxattn_last_error", "mxattn_quant_error",
    "mxattn_arrange_scales", "mxattn_forward_arranged", "mxattn_forward_noalloc",
)
# bytes of the library's own workspace array behind mxattn_forward_noalloc
NOALLOC_SCRATCH_BYTES = 256 << 20


class MxattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python mxfp4_bit_attention_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes
    vp, i32, i64, u32, f32, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_uint32, c.c_float, c.c_size_t
    lib.mxattn_kv_tile.restype = i32
    lib.mxattn_kv_tile.argtypes = []
    lib.mxattn_padded_tokens.restype = i64
    lib.mxattn_padded_tokens.argtypes = [i64]
    lib.mxattn_last_error.restype = c.c_char_p
    lib.mxattn_last_error.argtypes = []
    lib.mxattn_quantize.restype = c.c_int
    lib.mxattn_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, u32, vp, vp, vp]
    lib.mxattn_quant_error.restype = c.c_int
    lib.mxattn_quant_error.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, u32, vp, vp]
    lib.mxattn_forward_workspace_bytes.restype = sz
    lib.mxattn_forward_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.mxattn_forward.restype = c.c_int
    lib.mxattn_forward.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, f32, u32, u32, i32, f32,
                                   vp, vp, sz, vp]
    lib.mxattn_forward_quantized.restype = c.c_int
    lib.mxattn_forward_quantized.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, u32,
                                             i32, f32, vp, i32, vp, vp, vp]
    lib.mxattn_arrange_scales.restype = c.c_int
    lib.mxattn_arrange_scales.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
    lib.mxattn_forward_noalloc.restype = c.c_int
    lib.mxattn_forward_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, f32, u32, u32, i32, f32, vp, vp]
    lib.mxattn_forward_arranged.restype = c.c_int
    lib.mxattn_forward_arranged.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, u32, i32, f32,
                                            vp, i32, vp]
    return lib


# torch first: libmxattn then binds to the HIP runtime torch already loaded, so
# tensors, streams and the kernels share one runtime whatever the import order
import torch  # noqa: E402,F401

LIB = _load()


def mxattn_last_error() -> str:
    return LIB.mxattn_last_error().decode()


def mxattn_kv_tile() -> int:
    return int(LIB.mxattn_kv_tile())


def mxattn_padded_tokens(n: int) -> int:
    return int(LIB.mxattn_padded_tokens(n))


def mxattn_forward_workspace_bytes(B: int, H: int, Nq: int, Nkv: int, d: int) -> int:
    return int(LIB.mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d))


def _check(status: int):
    if status != MXATTN_OK:
        raise MxattnError(status, mxattn_last_error())


def rule_args(rule):
    """'uos' | 'ocp' | ('ceil', q) | float q  ->  (kind, qmax)."""
    if isinstance(rule, str):
        r = rule.lower()
        if r == "uos":
            return MXATTN_RULE_UOS, 7.25
        if r == "ocp":
            return MXATTN_RULE_OCP, 0.0
        raise ValueError(f"unknown rule {rule!r}")
    if isinstance(rule, (tuple, list)) and len(rule) == 2 and rule[0] == "ceil":
        return MXATTN_RULE_CEIL, float(rule[1])
    if isinstance(rule, (int, float)):
        return MXATTN_RULE_CEIL, float(rule)
    raise ValueError(f"unknown rule {rule!r}")


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MXATTN_F32
    if t.dtype == torch.bfloat16:
        return MXATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _expect(t, name: str, shape, dtypes):
    """Shape and dtype of one caller tensor (checked before anything touches the GPU)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        names = ", ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be {names}, got {str(t.dtype).replace('torch.', '')}")


def _on_device(device, **named):
    """Every named tensor contiguous and on `device` (a CUDA device)."""
    if device.type != "cuda":
        raise ValueError("tensors must be on the GPU")
    for name, t in named.items():
        if t is None:
            continue
        if t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _float_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


def _u8():
    return (_torch().uint8,)


def _as3(x):
    if x.dim() == 2:
        return x.unsqueeze(0), True
    if x.dim() == 3:
        return x, False
    raise ValueError("x must be 2-D or 3-D")


def _quant_shapes(b, r, c, axis):
    if axis == "last":
        return MXATTN_AXIS_LAST, (b, r, c // 2), (b, r, c // 32)
    if axis == "rows":
        P = mxattn_padded_tokens(r)
        return MXATTN_AXIS_ROWS, (b, c, P // 2), (b, c, P // 32)
    raise ValueError("axis must be 'last' or 'rows'")


def mxattn_quantize(x, rule="uos", axis: str = "last", hadamard: bool = False, codes=None, scales=None):
    """Block-quantise x [batch, rows, cols] (or [rows, cols]) on the GPU.

    axis="last": codes [batch, rows, cols/2], scales [batch, rows, cols/32].
    axis="rows": codes [batch, cols, P/2], scales [batch, cols, P/32], P = mxattn_padded_tokens(rows).
    codes / scales, when given, must have exactly those shapes (uint8, contiguous, on x's device).
    """
    torch = _torch()
    x3, squeeze = _as3(x)
    _expect(x3, "x", x3.shape, _float_dtypes())
    b, r, c = x3.shape
    ax, cshape, sshape = _quant_shapes(b, r, c, axis)
    # a 2-D x takes 2-D (or leading-1 3-D) codes and scales
    if codes is not None:
        _expect(codes, "codes", cshape[1:] if squeeze and codes.dim() == 2 else cshape, _u8())
    if scales is not None:
        _expect(scales, "scales", sshape[1:] if squeeze and scales.dim() == 2 else sshape, _u8())
    _on_device(x.device, x=x3, codes=codes, scales=scales)
    codes = codes.view(cshape) if codes is not None else None
    scales = scales.view(sshape) if scales is not None else None
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    kind, q = rule_args(rule)
    _check(LIB.mxattn_quantize(_ptr(x3), _dtype_code(x3), b, r, c, ax, kind, q, int(bool(hadamard)),
                               _ptr(codes), _ptr(scales), _stream(x.device)))
    if squeeze:
        return codes[0], scales[0]
    return codes, scales


def mxattn_quant_error(x, rule="uos", axis: str = "last", hadamard: bool = False, sums=None):
    """Quantisation error of mxattn_quantize(x, rule, axis, hadamard) without storing codes.

    Returns a float64 device tensor [3]: sum (value - dequantised)^2 and sum value^2 over
    finite blocks, and the number of non-finite blocks (values are the rotated ones
    when hadamard is set).
    """
    torch = _torch()
    x3, _ = _as3(x)
    _expect(x3, "x", x3.shape, _float_dtypes())
    b, r, c = x3.shape
    ax = _quant_shapes(b, r, c, axis)[0]
    if sums is not None:
        _expect(sums, "sums", (3,), (torch.float64,))
    _on_device(x.device, x=x3, sums=sums)
    if sums is None:
        sums = torch.empty(3, dtype=torch.float64, device=x.device)
    kind, q = rule_args(rule)
    _check(LIB.mxattn_quant_error(_ptr(x3), _dtype_code(x3), b, r, c, ax, kind, q, int(bool(hadamard)),
                                  _ptr(sums), _stream(x.device)))
    return sums


def mxattn_forward(q, k, v, softmax_scale: float, hadamard: bool = True, pnq: bool = True, rule="uos",
                   out=None, workspace=None):
    """O = MXFP4 attention of q [B,H,Nq,d], k, v [B,H,Nkv,d] (fp32 or bf16), same dtype out.

    out, when given: [B,H,Nq,d] in q's dtype.  workspace, when given: uint8, at least
    mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d) elements.  All on q's device, contiguous."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    _expect(q, "q", q.shape, _float_dtypes())
    _expect(k, "k", (B, H, Nkv, d), (q.dtype,))
    _expect(v, "v", (B, H, Nkv, d), (q.dtype,))
    if out is not None:
        _expect(out, "out", (B, H, Nq, d), (q.dtype,))
    wsb = mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        if workspace.numel() < wsb:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {wsb}")
    _on_device(q.device, q=q, k=k, v=v, out=out, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    kind, qm = rule_args(rule)
    _check(LIB.mxattn_forward(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, Nq, Nkv, d,
                              float(softmax_scale), int(bool(hadamard)), int(bool(pnq)), kind, qm,
                              _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out


def mxattn_forward_noalloc(q, k, v, softmax_scale: float, out, hadamard: bool = True, pnq: bool = True,
                           rule="uos"):
    """mxattn_forward with the library's own workspace array: nothing is allocated on the
    device (the caller supplies out [B,H,Nq,d] in q's dtype).  Calls that overlap in time on
    one GPU share that array and race."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    _expect(q, "q", q.shape, _float_dtypes())
    _expect(k, "k", (B, H, Nkv, d), (q.dtype,))
    _expect(v, "v", (B, H, Nkv, d), (q.dtype,))
    _expect(out, "out", (B, H, Nq, d), (q.dtype,))
    _on_device(q.device, q=q, k=k, v=v, out=out)
    kind, qm = rule_args(rule)
    _check(LIB.mxattn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, Nq, Nkv, d,
                                      float(softmax_scale), int(bool(hadamard)), int(bool(pnq)), kind, qm,
                                      _ptr(out), _stream(q.device)))
    return out


def _quantized_operands(qc, qs, kc, kscales, vtc, vscales, Nkv: int, arranged: bool):
    """Shapes of the MXFP4 operands of the attention entries: (B, H, Nq, d)."""
    if qc is None or qc.dim() != 4:
        raise ValueError("qc must be [B, H, Nq, d/2]")
    B, H, Nq, dh = qc.shape
    d = 2 * dh
    Nkv = int(Nkv)
    if Nkv < 1:
        raise ValueError("Nkv must be >= 1")
    P = mxattn_padded_tokens(Nkv)
    u8 = _u8()
    _expect(qc, "qc", (B, H, Nq, d // 2), u8)
    _expect(qs, "qs", (B, H, Nq, d // 32), u8)
    _expect(kc, "kc", (B, H, Nkv, d // 2), u8)
    _expect(vtc, "vtc", (B, H, d, P // 2), u8)
    if arranged:
        _expect(kscales, "ksa", (B, H, P * 4), u8)
        _expect(vscales, "vtsa", (B, H, P * 4), u8)
    else:
        _expect(kscales, "ks", (B, H, Nkv, d // 32), u8)
        _expect(vscales, "vts", (B, H, d, P // 32), u8)
    return B, H, Nq, d


def _attn_out(out, out_dtype, shape, device):
    torch = _torch()
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in _float_dtypes():
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is not None:
        _expect(out, "out", shape, (out_dtype,))
    return out, out_dtype


def mxattn_forward_quantized(qc, qs, kc, ks, vtc, vts, Nkv: int, softmax_scale: float, pnq: bool = True,
                             p_rule="uos", out_dtype=None, out=None, dump_p: bool = False):
    """Attention on MXFP4 operands in the layouts of mxattn_quantize.

    qc [B,H,Nq,d/2], qs [B,H,Nq,d/32], kc [B,H,Nkv,d/2], ks [B,H,Nkv,d/32], vtc [B,H,d,P/2],
    vts [B,H,d,P/32] (uint8, P = mxattn_padded_tokens(Nkv)).  Returns O [B,H,Nq,d] (and, with
    dump_p, the P^ codes [B,H,Nq,P/2] and scales [B,H,Nq,P/32]).
    """
    torch = _torch()
    B, H, Nq, d = _quantized_operands(qc, qs, kc, ks, vtc, vts, Nkv, arranged=False)
    out, out_dtype = _attn_out(out, out_dtype, (B, H, Nq, d), qc.device)
    _on_device(qc.device, qc=qc, qs=qs, kc=kc, ks=ks, vtc=vtc, vts=vts, out=out)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=qc.device)
    P = mxattn_padded_tokens(Nkv)
    pc = ps = None
    if dump_p:
        pc = torch.zeros((B, H, Nq, P // 2), dtype=torch.uint8, device=qc.device)
        ps = torch.zeros((B, H, Nq, P // 32), dtype=torch.uint8, device=qc.device)
    kind, qm = rule_args(p_rule)
    _check(LIB.mxattn_forward_quantized(_ptr(qc), _ptr(qs), _ptr(kc), _ptr(ks), _ptr(vtc), _ptr(vts),
                                        B, H, Nq, Nkv, d, float(softmax_scale), int(bool(pnq)), kind, qm,
                                        _ptr(out), _dtype_code(out), _ptr(pc), _ptr(ps),
                                        _stream(qc.device)))
    if dump_p:
        return out, pc, ps
    return out


def mxattn_arrange_scales(ks, vts, Nkv: int):
    """ks [B,H,Nkv,d/32], vts [B,H,d,P/32] -> (ksa, vtsa), uint8 [B,H,P*4] each, in the
    per-kv-tile order of the attention kernel's MFMA scale operands."""
    torch = _torch()
    if ks is None or ks.dim() != 4:
        raise ValueError("ks must be [B, H, Nkv, d/32]")
    B, H, _, dg = ks.shape
    d = dg * 32
    Nkv = int(Nkv)
    if Nkv < 1:
        raise ValueError("Nkv must be >= 1")
    P = mxattn_padded_tokens(Nkv)
    _expect(ks, "ks", (B, H, Nkv, d // 32), _u8())
    _expect(vts, "vts", (B, H, d, P // 32), _u8())
    _on_device(ks.device, ks=ks, vts=vts)
    ksa = torch.empty((B, H, P * 4), dtype=torch.uint8, device=ks.device)
    vtsa = torch.empty((B, H, P * 4), dtype=torch.uint8, device=ks.device)
    _check(LIB.mxattn_arrange_scales(_ptr(ks), _ptr(vts), B, H, Nkv, d, _ptr(ksa), _ptr(vtsa),
                                     _stream(ks.device)))
    return ksa, vtsa


def mxattn_forward_arranged(qc, qs, kc, ksa, vtc, vtsa, Nkv: int, softmax_scale: float, pnq: bool = True,
                            p_rule="uos", out_dtype=None, out=None):
    """mxattn_forward_quantized on scales from mxattn_arrange_scales (no P^ dump):
    ksa and vtsa are uint8 [B,H,P*4]."""
    torch = _torch()
    B, H, Nq, d = _quantized_operands(qc, qs, kc, ksa, vtc, vtsa, Nkv, arranged=True)
    out, out_dtype = _attn_out(out, out_dtype, (B, H, Nq, d), qc.device)
    _on_device(qc.device, qc=qc, qs=qs, kc=kc, ksa=ksa, vtc=vtc, vtsa=vtsa, out=out)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=qc.device)
    kind, qm = rule_args(p_rule)
    _check(LIB.mxattn_forward_arranged(_ptr(qc), _ptr(qs), _ptr(kc), _ptr(ksa), _ptr(vtc), _ptr(vtsa),
                                       B, H, Nq, Nkv, d, float(softmax_scale), int(bool(pnq)), kind, qm,
                                       _ptr(out), _dtype_code(out), _stream(qc.device)))
    return out
