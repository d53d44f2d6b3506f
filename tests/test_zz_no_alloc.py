"""mxattn_forward_noalloc, the forward for callers that cannot allocate device memory,
against mxattn_forward (which takes a caller workspace): through the C ABI, two calls in
a row on the same library array, the second with a smaller input, each output bitwise
equal to mxattn_forward's on the same inputs."""
import numpy as np
import pytest

from _gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

# (B, H, Nq, Nkv, d, dtype, hadamard, pnq, rule): the second call is smaller in every size
CALLS = [(2, 3, 300, 1000, 128, "bf16", True, True, "uos"),
         (1, 2, 100, 129, 64, "f32", False, False, "ocp")]


def test_noalloc_matches_forward_on_two_calls_second_smaller():
    torch, mx = require_gpu()
    for B, H, Nq, Nkv, d, dtype, had, pnq, rule in CALLS:
        print(f"noalloc call B={B} H={H} Nq={Nq} Nkv={Nkv} d={d} {dtype}", flush=True)
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        g = torch.Generator(device="cuda").manual_seed(Nq * 7 + Nkv)
        q, k, v = (torch.randn((B, H, n, d), generator=g, device="cuda").to(dt) * 2 for n in (Nq, Nkv, Nkv))
        scale = float(np.float32(1.0 / np.sqrt(d)))
        ref = mx.mxattn_forward(q, k, v, scale, hadamard=had, pnq=pnq, rule=rule)
        out = torch.full_like(q, float("nan"))
        mx.mxattn_forward_noalloc(q, k, v, scale, out, hadamard=had, pnq=pnq, rule=rule)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        iv = torch.int16 if dt == torch.bfloat16 else torch.int32
        assert torch.equal(out.view(iv), ref.view(iv))
