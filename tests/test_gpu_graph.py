"""The library's calls inside a HIP graph (torch.cuda.CUDAGraph): a serving loop can
capture mxattn_forward once and replay it.  Every replay, with eager work on the same
buffers between replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest

from _gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


def _capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_replays_bitwise(dtype):
    torch, mx = require_gpu()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(5)
    B, H, Nq, Nkv, d = 1, 3, 700, 901, 128
    q = torch.randn((B, H, Nq, d), generator=gen, device="cuda").to(dt)
    k = torch.randn((B, H, Nkv, d), generator=gen, device="cuda").to(dt)
    v = torch.randn((B, H, Nkv, d), generator=gen, device="cuda").to(dt)
    ws = torch.empty(mx.mxattn_forward_workspace_bytes(B, H, Nq, Nkv, d), dtype=torch.uint8, device="cuda")
    ref = mx.mxattn_forward(q, k, v, 1.0 / np.sqrt(d), hadamard=True, pnq=True, rule="uos", workspace=ws)
    out = torch.empty_like(q)
    g = _capture(torch, lambda: mx.mxattn_forward(q, k, v, 1.0 / np.sqrt(d), hadamard=True, pnq=True, rule="uos",
                                                  out=out, workspace=ws))
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(i + 1)  # the workspace is scratch: its old contents must not matter
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"


def test_quant_error_replays_clear_their_sums():
    """mxattn_quant_error zeroes its sums with a kernel, so a captured call starts from
    zero on every replay whatever the buffer held."""
    torch, mx = require_gpu()
    gen = torch.Generator(device="cuda").manual_seed(6)
    x = torch.randn((2, 1000, 128), generator=gen, device="cuda").to(torch.bfloat16)
    ref = mx.mxattn_quant_error(x, rule="uos", axis="last", hadamard=True).clone()
    sums = torch.empty(3, dtype=torch.float64, device="cuda")
    g = _capture(torch, lambda: mx.mxattn_quant_error(x, rule="uos", axis="last", hadamard=True, sums=sums))
    for i in range(4):
        sums.fill_(1e30 * (i + 1))
        g.replay()
        torch.cuda.synchronize()
        torch.testing.assert_close(sums, ref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("d,Nkv", [(128, 1000), (64, 300)])
def test_noalloc_forward_replays_on_new_inputs(d, Nkv):
    """mxattn_forward_noalloc is the entry point for callers that cannot allocate, graph
    capture among them: its captured call, replayed on new inputs copied into the captured
    buffers, is bitwise the allocating mxattn_forward on those inputs every time."""
    torch, mx = require_gpu()
    B, H, Nq = 1, 2, 257
    scale = float(1.0 / np.sqrt(d))
    gen = torch.Generator(device="cuda").manual_seed(d + Nkv)
    sets = [tuple(torch.randn((B, H, n, d), generator=gen, device="cuda").to(torch.bfloat16)
                  for n in (Nq, Nkv, Nkv)) for _ in range(3)]
    q, k, v = (t.clone() for t in sets[0])
    out = torch.empty_like(q)
    g = _capture(torch, lambda: mx.mxattn_forward_noalloc(q, k, v, scale, out=out))
    for i, (qs, ks, vs) in enumerate(sets[1:] + sets[:1] + sets[1:2]):
        q.copy_(qs)
        k.copy_(ks)
        v.copy_(vs)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = mx.mxattn_forward(qs, ks, vs, scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
