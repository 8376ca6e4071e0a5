"""GPU parity of the W4A8 path (MXFP8 activations x MXFP4 weights) against the
CPU oracle: the MXFP8 activation quantization bit for bit, and the mixed
FP8 x FP4 GEMM (with and without the row bias) within the W4A8 bar: the GEMM
bar (1e-5 * sum_k |a_k b_k|) plus the MFMA's own truncation inside each MX
block, bounded from the block's operand maxima (gpu_util)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (Guarded, assert_w4a8, bf16_bits, dev, f32, say, u8, w4a8_block_maxima,
                      w4a8_truncation_bound)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def quant8_both(mx, x_cpu, row_index=None, K=None):
    M = x_cpu.shape[0] if row_index is None else row_index.shape[0]
    K = x_cpu.shape[1] if K is None else K
    gc = Guarded((M, K), torch.uint8)
    gs = Guarded((M, K // 32), torch.uint8)
    ri = None if row_index is None else torch.from_numpy(row_index).to(dev())
    mx.mxfp8_quantize_act(x_cpu.to(dev()), gc.view, gs.view, row_index=ri, K=K)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the output"
    oc, os_ = oracle.quantize_act_fp8(bf16_bits(x_cpu), K=K, row_index=row_index)
    return (u8(gc.view), u8(gs.view)), (oc, os_)


def assert_same(gpu, ref, what):
    (gc, gs), (oc, os_) = gpu, ref
    if not np.array_equal(gs, os_):
        i = tuple(np.argwhere(gs != os_)[0])
        raise AssertionError(f"{what}: scale byte mismatch at {i}: gpu {gs[i]} oracle {os_[i]}")
    if not np.array_equal(gc, oc):
        i = tuple(np.argwhere(gc != oc)[0])
        raise AssertionError(f"{what}: code mismatch at {i}: gpu {gc[i]:#04x} oracle {oc[i]:#04x}")


# ---- MXFP8 activation quantization ---------------------------------------------
@pytest.mark.parametrize("M,K", [(1, 32), (16, 512), (37, 544), (5, 4096), (64, 4096)])
def test_act_quant_fp8_ragged_with_outliers(mx, M, K):
    say(f"act_quant_fp8 M={M} K={K}")
    x = synth.activations(M, K, seed=M + K, outlier_seed=K + 1)
    g, o = quant8_both(mx, x)
    assert_same(g, o, f"M={M} K={K}")


def test_act_quant_fp8_gather_and_wide_rows(mx):
    say("act_quant_fp8 gather, ldx > K")
    x = synth.activations(50, 1024, seed=5, outlier_seed=6)
    idx = np.random.default_rng(2).integers(0, 50, size=77).astype(np.int32)
    g, o = quant8_both(mx, x, row_index=idx)
    assert_same(g, o, "gather")
    g, o = quant8_both(mx, x, K=512)
    assert_same(g, o, "ldx>K")


def test_act_quant_fp8_special_values(mx):
    """Random bit patterns (NaN, Inf, subnormals), subnormal-only blocks,
    signed zeros, and E4M3 tie points at many scales."""
    say("act_quant_fp8 specials")
    rng = np.random.default_rng(11)
    K = 256
    bits = rng.integers(0, 2 ** 16, size=(40, K), dtype=np.uint32).astype(np.uint16)
    bits[8:16] = rng.integers(0, 0x80, size=(8, K)).astype(np.uint16) | \
        (rng.integers(0, 2, size=(8, K)).astype(np.uint16) << 15)
    bits[16:24] = rng.choice(np.array([0, 0x8000], dtype=np.uint16), size=(8, K))
    for r in range(24, 40):
        # multiples of 2^-4 between 0 and 2 against an anchor of 1: q = 256 v
        # lands on every E4M3 tie in [64, 512) and saturates above 448
        v = rng.integers(0, 33, size=K).astype(np.float32) / 16
        v[::32] = 1.0
        v *= np.float32(2.0 ** rng.integers(-100, 100)) * rng.choice([-1, 1], size=K)
        bits[r] = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    g, o = quant8_both(mx, x)
    assert_same(g, o, "specials")


def exhaustive_fp8_input():
    """Every bf16 magnitude (both signs) against every scale byte b it can meet:
    element 0 of each block is the anchor 256 * 2^(b-127) = 2^(b-119), the
    others lie below 512 * 2^(b-127), so the block's byte is b."""
    vals = []
    for b in range(0, 247):
        anchor = (b + 8) << 7
        mags = np.arange(0, (b + 9) << 7, dtype=np.uint32)
        v = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        nblk = -(-v.size // 31)
        body = np.concatenate([v, np.zeros(nblk * 31 - v.size, np.uint16)]).reshape(nblk, 31)
        head = np.full((nblk, 1), anchor, dtype=np.uint16)
        head[1::2] |= 0x8000
        vals.append(np.concatenate([head, body], axis=1))
    blocks = np.concatenate(vals)
    per_row = 128
    nrow = -(-blocks.shape[0] // per_row)
    pad = np.zeros((nrow * per_row - blocks.shape[0], 32), dtype=np.uint16)
    return np.concatenate([blocks, pad]).reshape(nrow, per_row * 32)


def test_act_quant_fp8_exhaustive_encoder(mx):
    say("act_quant_fp8 exhaustive: all bf16 magnitudes x all scale bytes")
    bits = exhaustive_fp8_input()
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    g, o = quant8_both(mx, x)
    assert_same(g, o, "exhaustive")
    assert set(np.unique(o[1])) >= set(range(0, 247)), "every scale byte is met"


# ---- the FP8 x FP4 GEMM ----------------------------------------------------------
def mxfp8_operand(M, K, seed):
    """Random MXFP8 operand: every finite E4M3 code (0x7F / 0xFF excluded),
    scale bytes 117..137 (the GEMM's exact-sum domain)."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 0x7F, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)
    s = rng.integers(117, 138, (M, K // 32))
    return torch.from_numpy(c.astype(np.uint8)), torch.from_numpy(s.astype(np.uint8))


@pytest.mark.parametrize("M,N,K", [(1, 256, 4096), (8, 1000, 4096), (33, 520, 2048),
                                   (48, 300, 4096), (64, 300, 4096), (5, 260, 1024),
                                   (20, 96, 96), (200, 520, 1056), (128, 256, 512),
                                   (300, 1000, 1024), (520, 776, 2048), (5, 12500, 2048)])
def test_gemm_w4a8_against_oracle(mx, M, N, K):
    """Skinny (M <= 64, K = 2048/4096), the LDS-staged tiled kernel (M >= 128,
    K % 512 == 0; ragged M and N), and the 16x16x128 tile kernel (other K,
    small M), fp32 and bf16 output, with and without the bias."""
    say(f"gemm_w4a8 M={M} N={N} K={K}")
    ac, as_ = mxfp8_operand(M, K, seed=M + N)
    bc, bs = synth.canonical_mxfp4(N, K, seed=N + K)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(N)) * 4).to(torch.bfloat16)
    y, s = oracle.gemm_w4a8(u8(ac), u8(as_), u8(bc), u8(bs))
    yb, sb = oracle.add_row_bias(y, s, bf16_bits(bias))
    amax, bmax = w4a8_block_maxima(u8(ac), u8(as_), u8(bc), u8(bs))
    pm, pn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    bound = w4a8_truncation_bound(amax, bmax, pm, pn)
    A = [t.to(dev()) for t in (ac, as_, bc, bs)]
    for dt in (torch.float32, torch.bfloat16):
        for use_bias, (yy, ss) in ((False, (y, s)), (True, (yb, sb))):
            gy = Guarded((M, N), dt)
            mx.mxfp4_gemm_w4a8(*A, gy.view, bias=bias.to(dev()) if use_bias else None)
            torch.cuda.synchronize()
            assert gy.intact(), "write outside y"
            assert_w4a8(gy.view, yy, ss, bound, f"w4a8 {dt} bias={use_bias}")
    # the bar stays far below what a misplaced operand byte or scale costs (O(S)):
    # full-range E4M3 operands span 2^18 inside a block, so the worst-case
    # truncation allowance is a few tenths of a percent of S here
    assert np.median(bound / np.maximum(s, 1e-300)) < 2.0 ** -6


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_linear_w4a8_decode_full_size(mx, M):
    """The decode-shaped layer (W [12288, 4096]) through the W4A8 linear call
    with a bias: the MXFP8 activations bit for bit, the output against the
    oracle on sampled columns, and the call equal to its two launches."""
    say(f"linear w4a8 M={M} N=12288 K=4096")
    N, K = 12288, 4096
    x = synth.activations(M, K, seed=12, outlier_seed=13)
    w = synth.bf16_normal((N, K), 0.02, seed=11)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()))
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(3)) * 0.5).to(torch.bfloat16)
    yl = mx.mxfp4_linear_w4a8_bf16(x.to(dev()), wc, ws, bias=bias.to(dev()),
                                   out_dtype=torch.float32)
    xc, xs = mx.mxfp8_quantize_act(x.to(dev()))
    y2 = mx.mxfp4_gemm_w4a8(xc, xs, wc, ws, bias=bias.to(dev()), out_dtype=torch.float32)
    assert torch.equal(yl, y2)
    oc, os_ = oracle.quantize_act_fp8(bf16_bits(x))
    assert np.array_equal(u8(xc), oc) and np.array_equal(u8(xs), os_)
    wo = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, 600)]))
    pm, pn = np.repeat(np.arange(M), cols.size), np.tile(cols, M)
    y, s = oracle.gemm_w4a8(oc, os_, wo[0], wo[1], pm, pn)
    bv = bias.double().numpy()[pn]
    amax, bmax = w4a8_block_maxima(oc, os_, wo[0], wo[1])
    bound = w4a8_truncation_bound(amax, bmax, pm, pn)
    assert_w4a8(yl.cpu()[pm, pn], y + bv, s + np.abs(bv), bound, "linear w4a8")


def test_gemm_w4a8_tiled_large_sampled(mx):
    """A prefill-sized W4A8 GEMM ([4096, 4096] x [1024, 4096]) through the tiled
    kernel, checked on sampled rows (every tile row and the last)."""
    M, N, K = 4096, 1024, 4096
    say(f"gemm_w4a8 tiled M={M} N={N} K={K} sampled")
    ac, as_ = mxfp8_operand(M, K, seed=91)
    bc, bs = synth.canonical_mxfp4(N, K, seed=92)
    gy = mx.mxfp4_gemm_w4a8(*[t.to(dev()) for t in (ac, as_, bc, bs)], out_dtype=torch.float32)
    rows = np.unique(np.concatenate([np.arange(0, M, 128) + np.arange(M // 128) % 128, [M - 1]]))
    pm, pn = np.repeat(rows, N), np.tile(np.arange(N), rows.size)
    y, s = oracle.gemm_w4a8(u8(ac), u8(as_), u8(bc), u8(bs), pm, pn)
    amax, bmax = w4a8_block_maxima(u8(ac), u8(as_), u8(bc), u8(bs))
    bound = w4a8_truncation_bound(amax, bmax, pm, pn)
    assert_w4a8(gy.cpu()[pm, pn], y, s, bound, "tiled large")



def test_gemm_w4a8_persistent_sampled(mx):
    """More than one round of tiles ([4000, 2048] x [2600, 2048]: 32 x 11 tiles
    of 128 x 256, ragged in M and N) takes the persistent walk; fp32 and bf16
    output with the bias, checked on sampled rows (one per tile row, the
    ragged tail included) and every column."""
    M, N, K = 4000, 2600, 2048
    say(f"gemm_w4a8 persistent M={M} N={N} K={K} sampled")
    ac, as_ = mxfp8_operand(M, K, seed=93)
    bc, bs = synth.canonical_mxfp4(N, K, seed=94)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(95)) * 4).to(torch.bfloat16)
    rows = np.unique(np.concatenate([np.arange(0, M, 128) + np.arange((M + 127) // 128) * 5 % 128,
                                     [M - 1]]))
    rows = rows[rows < M]
    pm, pn = np.repeat(rows, N), np.tile(np.arange(N), rows.size)
    y, s = oracle.gemm_w4a8(u8(ac), u8(as_), u8(bc), u8(bs), pm, pn)
    bv = bias.double().numpy()[pn]
    amax, bmax = w4a8_block_maxima(u8(ac), u8(as_), u8(bc), u8(bs))
    bound = w4a8_truncation_bound(amax, bmax, pm, pn)
    A = [t.to(dev()) for t in (ac, as_, bc, bs)]
    for dt in (torch.float32, torch.bfloat16):
        gy = Guarded((M, N), dt)
        mx.mxfp4_gemm_w4a8(*A, gy.view, bias=bias.to(dev()))
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        assert_w4a8(gy.view.cpu()[pm, pn], y + bv, s + np.abs(bv), bound, f"persistent {dt}")

def test_w4a8_graph_replay_matches_eager(mx):
    """The W4A8 act-quant and GEMM (skinny and tiled, with bias) captured in a
    HIP graph give the eager results on every replay."""
    say("w4a8: graph replay vs eager")
    d = dev()
    K, N = 4096, 512
    xs_ = synth.activations(8, K, seed=41).to(d)
    xl = synth.activations(256, K, seed=42).to(d)
    bc, bs = [t.to(d) for t in synth.canonical_mxfp4(N, K, seed=43)]
    bias = torch.randn(N, generator=torch.Generator().manual_seed(44)).to(torch.bfloat16).to(d)
    qs = (torch.empty((8, K), dtype=torch.uint8, device=d),
          torch.empty((8, K // 32), dtype=torch.uint8, device=d))
    ql = (torch.empty((256, K), dtype=torch.uint8, device=d),
          torch.empty((256, K // 32), dtype=torch.uint8, device=d))
    ys = torch.empty((8, N), dtype=torch.bfloat16, device=d)
    yl = torch.empty((256, N), dtype=torch.float32, device=d)

    def step():
        mx.mxfp8_quantize_act(xs_, *qs)
        mx.mxfp8_quantize_act(xl, *ql)
        mx.mxfp4_gemm_w4a8(*qs, bc, bs, ys, bias=bias)
        mx.mxfp4_gemm_w4a8(*ql, bc, bs, yl, bias=bias)

    outs = (*qs, *ql, ys, yl)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in outs:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)
        step()
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,K", [(2, 512), (130, 512)])
def test_w4a8_in_block_truncation_model(mx, M, K):
    """Pins, through the C-ABI, the hardware arithmetic the W4A8 bar rests on:
    inside one 32-element block the E4M3 x E2M1 products are summed 13 bits
    below the block's largest (448 + x keeps x truncated to a multiple of
    2^-5), while separate blocks add without that loss.  B = 1.0 everywhere,
    all scales 2^0; row r puts 448 at k = 0 and x_r at k = 1 (same block) and
    x_r at k = 32 + r % 32 in row r's copy for the other-block case.  (The
    16x16x128 tile kernel at M = 2, the tiled kernel at M = 130.)"""
    say(f"w4a8 truncation model M={M} K={K}")
    xs = np.array([2.0 ** -9, 0.0234375, 0.05859375, 0.140625, 0.25, 1.0], dtype=np.float32)
    codes8 = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(torch.from_numpy(codes8).view(torch.float8_e4m3fn).float().numpy(), xs)
    ac = np.zeros((M, K), dtype=np.uint8)
    ac[:, 0] = 0x7E                                   # 448
    pick = np.arange(M) % xs.size
    same = np.arange(M) % 2 == 0
    ac[same, 1] = codes8[pick[same]]                  # same block as the 448
    ac[~same, 32] = codes8[pick[~same]]               # next block
    as_ = np.full((M, K // 32), 127, dtype=np.uint8)
    bc = np.full((8, K // 2), 0x22, dtype=np.uint8)   # E2M1 1.0 in both nibbles
    bs = np.full((8, K // 32), 127, dtype=np.uint8)
    y = mx.mxfp4_gemm_w4a8(*[torch.from_numpy(t).to(dev()) for t in (ac, as_, bc, bs)],
                           out_dtype=torch.float32).cpu().numpy()
    x = xs[pick].astype(np.float64)
    want = np.where(same, 448 + np.floor(x / 2.0 ** -5) * 2.0 ** -5, 448 + x)
    assert np.array_equal(y, np.repeat(want[:, None], 8, axis=1))
    # and the W4A8 bar covers what the truncation drops
    amax, bmax = w4a8_block_maxima(ac, as_, bc, bs)
    pm, pn = np.repeat(np.arange(M), 8), np.tile(np.arange(8), M)
    bound = w4a8_truncation_bound(amax, bmax, pm, pn)
    exact = np.repeat((448 + x)[:, None], 8, axis=1).reshape(-1)
    assert (np.abs(y.reshape(-1) - exact) <= bound).all()



def observed_error(gpu, y, s, bound):
    """Largest |gpu - exact| relative to S = sum_k |a_k b_k|, to the W4A8
    bar's truncation allowance, and to |exact| (outputs above 1e-3 of the
    largest), and the fraction of outputs beyond the W4A4 bar 1e-5 * S."""
    err = np.abs(f32(gpu.float()).astype(np.float64).reshape(y.shape) - y)
    big = np.abs(y) > 1e-3 * np.abs(y).max()
    return dict(max_err_over_S=float((err / np.maximum(s, 1e-300)).max()),
                max_err_over_allowance=float((err / np.maximum(bound, 1e-300)).max()),
                max_rel_err=float((err[big] / np.abs(y[big])).max()),
                frac_beyond_w4a4_bar=float((err > oracle.GEMM_FP32_RTOL * s).mean()))


def test_w4a8_error_observed_on_the_bench_shapes(mx):
    """The W4A8 error as it comes out on the bench's data (NVFP4-derived
    weights N(0, 0.02), activations N(0, 1) with 1% outlier channels x50):
    the decode layer W [12288, 4096] at M = 64 (every row, 1000 sampled
    columns) and a [4096]^3 GEMM (16 sampled rows, every column), fp32 out.
    Reported (run with -s), and held inside the bar; the bar itself is a
    worst case over full-range operands, far above what such data reaches."""
    cases = []
    w = synth.bf16_normal((12288, 4096), 0.02, seed=11)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    wo = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    x = synth.activations(64, 4096, seed=12, outlier_seed=13)
    cols = np.random.default_rng(7).choice(12288, 1000, replace=False)
    cases.append(("decode M=64 N=12288 K=4096", x, wo, np.repeat(np.arange(64), cols.size),
                  np.tile(cols, 64)))
    w2 = synth.bf16_normal((4096, 4096), 0.02, seed=21)
    c2, s2, g2 = synth.nvfp4_from_bf16(w2)
    wo2 = oracle.requant(u8(c2), u8(s2), np.atleast_1d(g2.numpy()))
    x2 = synth.activations(4096, 4096, seed=24, outlier_seed=26)
    rows = np.unique(np.concatenate([np.arange(0, 4096, 273), [4095]]))
    cases.append(("prefill [4096]^3", x2, wo2, np.repeat(rows, 4096), np.tile(np.arange(4096), rows.size)))
    for label, xx, (bc, bs), pm, pn in cases:
        oc, os_ = oracle.quantize_act_fp8(bf16_bits(xx))
        gy = mx.mxfp4_gemm_w4a8(torch.from_numpy(oc).to(dev()), torch.from_numpy(os_).to(dev()),
                                torch.from_numpy(bc).to(dev()), torch.from_numpy(bs).to(dev()),
                                out_dtype=torch.float32)
        y, s = oracle.gemm_w4a8(oc, os_, bc, bs, pm, pn)
        amax, bmax = w4a8_block_maxima(oc, os_, bc, bs)
        bound = w4a8_truncation_bound(amax, bmax, pm, pn)
        got = gy.cpu()[pm, pn]
        assert_w4a8(got, y, s, bound, label)
        obs = observed_error(got, y, s, bound)
        say(f"  {label}: {obs} "
            f"(allowance median {np.median(bound / np.maximum(s, 1e-300)):.2e} of S)")
        # on these seeded inputs the truncation costs about 3e-5 * S at most
        # (0.5% of its allowance): a change in the arithmetic that kept inside
        # the worst-case bar but lost more would show here
        assert obs["max_err_over_S"] < 1e-4, obs


@pytest.mark.parametrize("M,N,K,ldx", [(1, 1000, 4096, 4096), (5, 300, 2048, 2048),
                                       (16, 2048, 4096, 4104), (8, 520, 2048, 2056),
                                       (17, 300, 4096, 4096)])
def test_linear_w4a8_one_launch_matches_two(mx, M, N, K, ldx):
    """The one-launch W4A8 decode call (M <= 16, K = 2048/4096: MXFP8 quantized
    inside the GEMM kernel) equals mxfp8_quantize_act followed by
    mxfp4_gemm_w4a8 bit for bit -- rows wider than K, NaN and Inf in x, the
    bias, both output types; M = 17 takes the two-launch form."""
    say(f"linear w4a8 fused M={M} N={N} K={K} ldx={ldx}")
    d = dev()
    x = synth.activations(M, ldx, seed=M + N, outlier_seed=K + 5).to(d)
    if M >= 5:
        x[1, 40] = float("nan")
        x[2, K - 1] = float("inf")
        x[4, 64:96] = 0.0
    bc, bs = [t.to(d) for t in synth.canonical_mxfp4(N, K, seed=N + 3)]
    bias = torch.randn(N, generator=torch.Generator().manual_seed(N)).to(torch.bfloat16).to(d)
    assert (mx.mxfp4_linear_w4a8_workspace_size(M, N, K) == 0) == (M <= 16)
    xc, xs_ = mx.mxfp8_quantize_act(x, K=K)
    for dt in (torch.bfloat16, torch.float32):
        ref = mx.mxfp4_gemm_w4a8(xc, xs_, bc, bs, bias=bias, out_dtype=dt)
        gy = Guarded((M, N), dt)
        mx.mxfp4_linear_w4a8_bf16(x, bc, bs, gy.view, bias=bias, K=K)
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        a, b = gy.view.float().cpu(), ref.float().cpu()
        nan = torch.isnan(a) & torch.isnan(b)
        assert bool(((a.view(torch.int32) == b.view(torch.int32)) | nan).all()), dt


def test_gemm_w4a8_at_the_32bit_offset_limit(mx):
    """The W4A8 tiled kernel takes MXFP8 activations under 2 GiB (one byte an
    element): 524287 rows at K = 4096 run tiled, 524288 rows (exactly 2^31
    bytes) go to the 16x16x128 tile kernel.  Sampled rows, the last ones
    included; operands made on the GPU."""
    K, N = 4096, 256
    d = dev()
    m_over = (1 << 31) // K
    g = torch.Generator(device=d)
    g.manual_seed(81)
    ac = (torch.randint(0, 0x7F, (m_over, K), generator=g, device=d, dtype=torch.int32) |
          (torch.randint(0, 2, (m_over, K), generator=g, device=d, dtype=torch.int32) << 7)
          ).to(torch.uint8)
    as_ = torch.randint(117, 138, (m_over, K // 32), generator=g, device=d,
                        dtype=torch.int32).to(torch.uint8)
    bc, bs = synth.canonical_mxfp4(N, K, seed=82, device=d)
    b_cpu = (u8(bc.cpu()), u8(bs.cpu()))
    rng = np.random.default_rng(83)
    for M in (m_over - 1, m_over):
        say(f"gemm_w4a8 at the offset limit M={M} N={N} K={K}")
        y = torch.empty((M, N), dtype=torch.float32, device=d)
        mx.mxfp4_gemm_w4a8(ac[:M], as_[:M], bc, bs, y)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, 1], np.arange(M - 40, M), rng.integers(0, M, 24)]))
        ri = torch.from_numpy(rows).to(d)
        a_cpu = (u8(ac[ri].cpu()), u8(as_[ri].cpu()))
        yo, s = oracle.gemm_w4a8(*a_cpu, *b_cpu)
        amax, bmax = w4a8_block_maxima(*a_cpu, *b_cpu)
        pm, pn = np.meshgrid(np.arange(rows.size), np.arange(N), indexing="ij")
        bound = w4a8_truncation_bound(amax, bmax, pm, pn)
        assert_w4a8(y[ri].cpu(), yo, s, bound, f"w4a8 offset limit M={M}")
        del y
