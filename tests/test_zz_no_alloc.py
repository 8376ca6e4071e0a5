"""mxfp4_linear_bf16_noalloc (the linear call for callers that cannot
allocate: its quantized activations live in the library's static per-GPU
scratch) against mxfp4_linear_bf16 with a caller workspace, through the C
ABI: bit for bit, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's bytes, which must not leak into the second),
then on one-launch shapes that need no scratch, and the size limit."""
import pytest
import torch

import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def weight(mx, N, K, seed):
    w = synth.bf16_normal((N, K), 0.02, seed=seed, device=dev())
    c, s, g = synth.nvfp4_from_bf16(w)
    return mx.mxfp4_requant_from_nvfp4(c, s, g.reshape(1))


def both(mx, x, wc, ws, bias=None, out_dtype=torch.bfloat16, rule="ocp"):
    M, N = x.shape[0], wc.shape[0]
    y0 = torch.full((M, N), float("nan"), dtype=out_dtype, device=dev())
    y1 = torch.full((M, N), float("nan"), dtype=out_dtype, device=dev())
    mx.mxfp4_linear_bf16(x, wc, ws, y0, bias=bias, scale_rule=rule)
    mx.mxfp4_linear_bf16_noalloc(x, wc, ws, y1, bias=bias, scale_rule=rule)
    torch.cuda.synchronize()
    return y0, y1


def test_noalloc_equals_workspace_call_twice_then_smaller(mx):
    K, N = 4096, 2048
    wc, ws = weight(mx, N, K, seed=71)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(72)) * 0.5).to(
        torch.bfloat16).to(dev())
    for M, xseed in ((3000, 73), (200, 74)):          # the second call smaller
        say(f"noalloc linear M={M} N={N} K={K}")
        x = synth.activations(M, K, seed=xseed, outlier_seed=xseed + 1, device=dev())
        assert mx.mxfp4_linear_workspace_size(M, N, K) > 0        # uses the scratch
        y0, y1 = both(mx, x, wc, ws, bias=bias)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), f"M={M} bf16"
        y0, y1 = both(mx, x, wc, ws, out_dtype=torch.float32, rule="uos")
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"M={M} fp32 uos"


def test_noalloc_one_launch_shapes_and_the_limit(mx):
    K, N = 4096, 1024
    wc, ws = weight(mx, N, K, seed=81)
    for M in (1, 16, 17, 64):
        say(f"noalloc linear M={M}")
        x = synth.activations(M, K, seed=82 + M, device=dev())
        y0, y1 = both(mx, x, wc, ws)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), f"M={M}"
    # just past the limit: rejected before anything is launched, y untouched
    Kbig = 14336
    M = mx.MXFP4_NOALLOC_SCRATCH_BYTES // (Kbig // 2 + Kbig // 32) + 1
    wbc = torch.zeros((16, Kbig // 2), dtype=torch.uint8, device=dev())
    wbs = torch.full((16, Kbig // 32), 127, dtype=torch.uint8, device=dev())
    x = torch.zeros((M, Kbig), dtype=torch.bfloat16, device=dev())
    y = torch.full((M, 16), 7.0, dtype=torch.bfloat16, device=dev())
    assert mx.mxfp4_linear_workspace_size(M, 16, Kbig) > mx.MXFP4_NOALLOC_SCRATCH_BYTES
    with pytest.raises(mx.Mxfp4Error) as e:
        mx.mxfp4_linear_bf16_noalloc(x, wbc, wbs, y)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert (y == 7.0).all()
