"""GPU parity of the MXFP4 GEMM calls against the CPU oracle.

Bar: fp32 output within 1e-5 * sum_k |a_k b_k| per element; bf16 output at
most one bf16 ulp (ordered-bit distance) from the oracle's exact result
rounded to bf16.  Operands of the dense/grouped pipelines are produced on each
side by that side's own requant / act-quant from the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (Guarded, assert_gemm_bf16, assert_gemm_fp32, bf16_bits, dev, f32, say,
                      u8)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def to_dev(*ts):
    return [t.to(dev()) if isinstance(t, torch.Tensor) else torch.from_numpy(t).to(dev())
            for t in ts]


# ---- random operands, every tile edge ------------------------------------------------
SHAPES = [(1, 1, 32), (1, 300, 4096), (7, 17, 96), (16, 256, 512), (33, 200, 544),
          (64, 129, 1024), (65, 260, 1056), (100, 64, 4096), (130, 131, 2080),
          # weight-streaming kernel: every activation-block count, K = 2048 and 4096,
          # ragged N, four and eight wavefronts
          (5, 1000, 2048), (16, 16, 4096), (17, 300, 4096), (40, 72, 2048), (48, 257, 4096),
          (64, 4099, 4096), (61, 1040, 2048),
          # more weight tiles than a grid's slots hold at once (over 16 x 3 x 256
          # rows): each slot is refilled as it is consumed
          (3, 13000, 2048), (64, 12352, 2048),
          # the weight-streaming kernel at other K: 1..4 super-steps a wave, those
          # past K masked off (K = 512: seven of eight waves idle), 1..3 tiles in
          # flight, refilled slots past 256 tiles
          (1, 300, 512), (64, 1040, 512), (40, 200, 1536), (17, 333, 3584), (64, 1000, 4608),
          (33, 520, 8192), (32, 260, 12288), (5, 4200, 10240), (16, 4200, 14336),
          (9, 300, 16384),
          # too few 256 x 256 tiles to fill the chip: 128-row tiles (ragged M and
          # N, K of 2, 3 and 16 stages)
          (520, 520, 2048), (1000, 2000, 1536), (256, 1030, 4096),
          # 64 < M <= 128: the decode kernel once per 64-row slice
          (96, 300, 4096), (128, 520, 2048), (127, 1000, 8192), (65, 4200, 4096),
          # more tiles than one round on the chip (ragged M and N), K of 4 and 2
          # stages (the 8-wave pipeline's loads past the last stage); the last
          # round at most half full, so the tiles of each XCD's first slots run
          # as half tiles: ragged last tile row (its bottom half partly, or
          # wholly, past M) and whole tile rows
          (2200, 7700, 1024), (2200, 7700, 512), (1400, 12288, 512), (1536, 12288, 512),
          # the last round more than half full: whole tiles only
          (2500, 12288, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_random_operands_fp32(mx, M, N, K):
    say(f"gemm random M={M} N={N} K={K}")
    a, sa = synth.canonical_mxfp4(M, K, seed=M * 7 + K)
    b, sb = synth.canonical_mxfp4(N, K, seed=N * 11 + K + 1)
    y, s = oracle.gemm(u8(a), u8(sa), u8(b), u8(sb))
    A, SA, B, SB = to_dev(a, sa, b, sb)
    gy = Guarded((M, N), torch.float32)
    mx.mxfp4_gemm(A, SA, B, SB, gy.view)
    yb = mx.mxfp4_gemm(A, SA, B, SB, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert gy.intact(), "write outside y"
    assert_gemm_fp32(gy.view, y, s, f"{M}x{N}x{K}")
    # the bf16 epilogue is the RNE of the same fp32 accumulator
    assert np.array_equal(bf16_bits(yb), bf16_bits(gy.view.to(torch.bfloat16)))


def test_gemm_wide_scale_range(mx):
    """E8M0 bytes over most of the range that keeps every product fp32-normal
    (byte sums >= 130) and every partial sum finite (byte sums <= 366 at K=512)."""
    say("gemm wide scale range")
    M, N, K = 40, 72, 512
    a, sa = synth.canonical_mxfp4(M, K, seed=1, scale_lo=65, scale_hi=183)
    b, sb = synth.canonical_mxfp4(N, K, seed=2, scale_lo=65, scale_hi=183)
    y, s = oracle.gemm(u8(a), u8(sa), u8(b), u8(sb))
    assert s.max() < 3.0e38
    A, SA, B, SB = to_dev(a, sa, b, sb)
    out = mx.mxfp4_gemm(A, SA, B, SB, out_dtype=torch.float32)
    assert_gemm_fp32(out, y, s, "wide scales")


def test_gemm_overflow_saturates_to_inf(mx):
    """When every product has the same sign and the exact sum exceeds the fp32
    range, the fp32 result is +-inf (the RNE image of an overflowing value)."""
    say("gemm fp32 overflow")
    K = 256
    a = torch.full((2, K // 2), 0x77, dtype=torch.uint8)          # all codes 6.0
    sa = torch.full((2, K // 32), 250, dtype=torch.uint8)
    b = torch.full((3, K // 2), 0x77, dtype=torch.uint8)
    b[1] = 0xFF                                                    # all codes -6.0
    sb = torch.full((3, K // 32), 127, dtype=torch.uint8)
    sb[2] = 1                                                      # tiny: finite result
    y, s = oracle.gemm(u8(a), u8(sa), u8(b), u8(sb))
    A, SA, B, SB = to_dev(a, sa, b, sb)
    out = f32(mx.mxfp4_gemm(A, SA, B, SB, out_dtype=torch.float32))
    assert np.all(out[:, 0] == np.inf) and np.all(out[:, 1] == -np.inf)
    assert np.all(np.isfinite(out[:, 2]))
    assert oracle.gemm_fp32_ok(out[:, 2].astype(np.float64), y[:, 2], s[:, 2]).all()


def test_gemm_deterministic_and_finite(mx):
    say("gemm determinism / finiteness over mixed M")
    K, N = 1024, 384
    b, sb = synth.canonical_mxfp4(N, K, seed=5)
    B, SB = to_dev(b, sb)
    for M in (1, 3, 16, 31, 64, 65, 200):
        a, sa = synth.canonical_mxfp4(M, K, seed=M)
        A, SA = to_dev(a, sa)
        y1 = mx.mxfp4_gemm(A, SA, B, SB, out_dtype=torch.float32)
        y2 = mx.mxfp4_gemm(A, SA, B, SB, out_dtype=torch.float32)
        assert torch.equal(y1, y2)
        assert torch.isfinite(y1).all()


# ---- the pipeline: requant + act-quant + GEMM on each side ------------------------------
def pipeline_weight(N, K, seed):
    """NVFP4 weight from bf16 N(0, 0.02); GPU requant on the device, oracle requant
    on the host, each from the same NVFP4 bytes."""
    w = synth.bf16_normal((N, K), 0.02, seed=seed)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    oc, os_ = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    return (codes, scales, g), (oc, os_)


def gpu_weight(mx, nv):
    codes, scales, g = nv
    C, S, G = to_dev(codes, scales, g.reshape(1))
    return mx.mxfp4_requant_from_nvfp4(C, S, G)


@pytest.fixture(scope="module")
def decode_weight(mx):
    say("building decode weight [12288,4096] seed 11")
    nv, (oc, os_) = pipeline_weight(12288, 4096, seed=11)
    wc, ws = gpu_weight(mx, nv)
    return (wc, ws), (oc, os_)


def test_gemm_tiny_pipeline(mx):
    say("tiny pipeline 16x256x512")
    nv, (oc, os_) = pipeline_weight(256, 512, seed=1)
    wc, ws = gpu_weight(mx, nv)
    x = synth.activations(16, 512, seed=2)
    xc, xs = mx.mxfp4_quantize_act(x.to(dev()))
    yg = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.bfloat16)
    ac, as_ = oracle.quantize_act(bf16_bits(x))
    y, s = oracle.gemm(ac, as_, oc, os_)
    assert_gemm_bf16(yg, y, "tiny bf16")
    yf = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.float32)
    assert_gemm_fp32(yf, y, s, "tiny fp32")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_gemm_decode_pipeline_full(mx, decode_weight, M):
    say(f"decode pipeline M={M} N=12288 K=4096 (all outputs)")
    (wc, ws), (oc, os_) = decode_weight
    x = synth.activations(64, 4096, seed=12, outlier_seed=13)[:M].contiguous()
    xc, xs = mx.mxfp4_quantize_act(x.to(dev()))
    yg = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.bfloat16)
    yf = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.float32)
    ac, as_ = oracle.quantize_act(bf16_bits(x))
    y, s = oracle.gemm(ac, as_, oc, os_)
    assert_gemm_bf16(yg, y, f"decode M={M} bf16")
    assert_gemm_fp32(yf, y, s, f"decode M={M} fp32")


# ---- grouped GEMM -------------------------------------------------------------------
def test_grouped_gemm_ragged_and_empty_experts(mx):
    say("grouped gemm ragged/empty experts")
    E, N, K = 6, 72, 544
    counts = np.array([5, 0, 37, 1, 0, 70])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    a, sa = synth.canonical_mxfp4(M, K, seed=1)
    b, sb = synth.canonical_mxfp4(E * N, K, seed=2)
    b, sb = b.reshape(E, N, K // 2), sb.reshape(E, N, K // 32)
    y, s = oracle.grouped_gemm(u8(a), u8(sa), u8(b), u8(sb), offsets)
    A, SA, B, SB, OFF = to_dev(a, sa, b, sb, offsets)
    gy = Guarded((M, N), torch.float32)
    mx.mxfp4_grouped_gemm(A, SA, B, SB, OFF, gy.view)
    torch.cuda.synchronize()
    assert gy.intact()
    assert_gemm_fp32(gy.view, y, s, "grouped")


def test_grouped_gemm_bad_offsets_stay_inside_y(mx):
    """A malformed offset table (decreasing, negative, past total_M) may give wrong
    rows, but the kernel clamps every range: nothing outside y is written."""
    say("grouped gemm malformed offsets")
    E, N, K, M = 4, 32, 64, 50
    a, sa = synth.canonical_mxfp4(M, K, seed=3)
    b, sb = synth.canonical_mxfp4(E * N, K, seed=4)
    A, SA, B, SB = to_dev(a, sa, b.reshape(E, N, K // 2), sb.reshape(E, N, K // 32))
    for table in ([0, 60, 10, -5, 50], [-100, 0, 1000, 20, 50], [0, 0, 0, 0, 0]):
        OFF = torch.tensor(table, dtype=torch.int32, device=dev())
        gy = Guarded((M, N), torch.float32)
        mx.mxfp4_grouped_gemm(A, SA, B, SB, OFF, gy.view)
        torch.cuda.synchronize()
        assert gy.intact(), table


def grouped_case(mx, counts, N, K, seed, out_dtype):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    a, sa = synth.canonical_mxfp4(M, K, seed=seed)
    b, sb = synth.canonical_mxfp4(E * N, K, seed=seed + 1)
    b, sb = b.reshape(E, N, K // 2), sb.reshape(E, N, K // 32)
    y, s = oracle.grouped_gemm(u8(a), u8(sa), u8(b), u8(sb), offsets)
    A, SA, B, SB, OFF = to_dev(a, sa, b, sb, offsets)
    gy = Guarded((M, N), out_dtype)
    mx.mxfp4_grouped_gemm(A, SA, B, SB, OFF, gy.view)
    torch.cuda.synchronize()
    assert gy.intact(), "write outside y"
    return gy.view, y, s


# Expert sizes ending in each 32-row block of a 128-row tile or spanning
# several; the second set averages more than 96 rows an expert, which gives
# the register-streamed kernel its 160-row tile: sizes ending in each of its
# five blocks and spanning two and three tiles.
ROW_BLOCK_COUNTS = {"tile128": [0, 1, 31, 32, 33, 97, 128, 129, 257, 300, 0],
                    "tile160": [0, 1, 31, 32, 33, 97, 128, 129, 159, 160, 161, 257, 300, 320,
                                321, 0]}


@pytest.mark.parametrize("K", [1024, 1536, 3072])
@pytest.mark.parametrize("rows", ["tile128", "tile160"])
def test_grouped_gemm_tiled_row_blocks(mx, K, rows):
    """Expert sizes that end in each 32-row block of a tile, span several
    tiles, or are empty; N with a partial 256-row weight tile.  The bf16
    output is the RNE of the same fp32 accumulator (random scales make
    cancellation common, so the oracle bound is the fp32 one).  K = 1024 and
    3072 take the kernel with the weights streamed into registers (an item
    of 4 stages, and of 12: its steady loop), K = 1536 the one that stages
    them in LDS."""
    counts = ROW_BLOCK_COUNTS[rows]
    say(f"grouped tiled row blocks counts={counts} N=300 K={K}")
    gy, y, s = grouped_case(mx, counts, 300, K, 51, torch.float32)
    assert_gemm_fp32(gy, y, s, "grouped tiled")
    yb, _, _ = grouped_case(mx, counts, 300, K, 51, torch.bfloat16)
    assert np.array_equal(bf16_bits(yb), bf16_bits(gy.to(torch.bfloat16)))


@pytest.mark.parametrize("N", [296, 352])
def test_grouped_gemm_stream_partial_wave_columns(mx, N):
    """bf16 and fp32 out with N a multiple of 8 but not of 64, so that in the
    last weight tile one wave owns 40 (N = 296) or 32 (N = 352) valid columns
    and the waves past it none: the register-streamed kernel's epilogue
    drops the pieces past N through its store descriptor.  Expert sizes as
    in the 160-row tile case, K = 1024; fp32 against the oracle, bf16 equal
    to the RNE of the fp32 result."""
    counts = ROW_BLOCK_COUNTS["tile160"]
    say(f"grouped stream partial wave columns N={N}")
    gy, y, s = grouped_case(mx, counts, N, 1024, 57, torch.float32)
    assert_gemm_fp32(gy, y, s, "grouped stream")
    yb, _, _ = grouped_case(mx, counts, N, 1024, 57, torch.bfloat16)
    assert np.array_equal(bf16_bits(yb), bf16_bits(gy.to(torch.bfloat16)))


def test_grouped_gemm_stream_many_items(mx):
    """More work items than workgroups (480 items of 4 stages over 96 experts),
    so the workgroups walk several: each item's first stages arrive during
    the previous item, whose row count (32-row blocks 1..4) may differ."""
    rng = np.random.default_rng(17)
    counts = rng.integers(0, 160, size=96)
    counts[rng.random(96) < 0.15] = 0
    say(f"grouped stream many items total {counts.sum()} N=1280 K=1024")
    gy, y, s = grouped_case(mx, counts, 1280, 1024, 81, torch.float32)
    assert_gemm_fp32(gy, y, s, "grouped stream many items")


def test_grouped_gemm_tiled_many_small_experts(mx):
    """More experts than a wavefront has lanes (the offset table is scanned in
    pieces), most of them tiny or empty."""
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 6, size=150)
    counts[rng.random(150) < 0.3] = 0
    counts[77] = 140
    say(f"grouped tiled 150 experts total {counts.sum()} N=256 K=512")
    gy, y, s = grouped_case(mx, counts, 256, 512, 61, torch.float32)
    assert_gemm_fp32(gy, y, s, "grouped tiled small experts")


def test_grouped_gemm_tiled_more_than_256_experts(mx):
    """Three hundred experts, mostly with a handful of rows: the expert table
    and the tile walk cross many short experts, under both K-prefetch settings
    (K = 1024 streams the next tile's first stages, K = 512 does not)."""
    rng = np.random.default_rng(9)
    counts = rng.integers(0, 5, size=300)
    counts[[3, 150, 299]] = [130, 257, 40]
    for K in (1024, 512):
        say(f"grouped tiled 300 experts total {counts.sum()} N=256 K={K}")
        gy, y, s = grouped_case(mx, counts, 256, K, 71, torch.float32)
        assert_gemm_fp32(gy, y, s, f"grouped tiled 300 experts K={K}")


def test_preshuffle_matches_the_definition(mx):
    """mxfp4_preshuffle_weights equals the oracle's definition of the layout,
    byte for byte, and writes nothing outside its output."""
    T, N, K = 3, 96, 1536
    say(f"preshuffle T={T} N={N} K={K}")
    codes = torch.randint(0, 256, (T, N, K // 2), dtype=torch.uint8,
                          generator=torch.Generator().manual_seed(5))
    out = Guarded((T, N, K // 2), torch.uint8)
    mx.mxfp4_preshuffle_weights(codes.to(dev()), out.view)
    torch.cuda.synchronize()
    assert out.intact(), "write outside the output"
    assert np.array_equal(u8(out.view), oracle.preshuffle_codes(u8(codes)))


@pytest.mark.parametrize("K", [1024, 3072])
@pytest.mark.parametrize("rows", ["tile128", "tile160"])
def test_grouped_gemm_preshuffled_weights(mx, K, rows):
    """The grouped GEMM reading pre-shuffled weight codes gives the row-major
    call's output bit for bit (fp32 and bf16; every 32-row block of a
    128-row tile, a partial 256-row weight tile, empty experts), and that is
    within the oracle's bar."""
    counts = ROW_BLOCK_COUNTS[rows]
    E, N = len(counts), 320
    say(f"grouped gemm preshuffled counts={counts} N={N} K={K}")
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    a, sa = synth.canonical_mxfp4(M, K, seed=K + 1)
    b, sb = synth.canonical_mxfp4(E * N, K, seed=K + 2)
    b, sb = b.reshape(E, N, K // 2), sb.reshape(E, N, K // 32)
    A, SA, B, SB, OFF = to_dev(a, sa, b, sb, offsets)
    Bs = mx.mxfp4_preshuffle_weights(B)
    for dt in (torch.float32, torch.bfloat16):
        ref = mx.mxfp4_grouped_gemm(A, SA, B, SB, OFF, out_dtype=dt)
        gy = Guarded((M, N), dt)
        mx.mxfp4_grouped_gemm(A, SA, Bs, SB, OFF, gy.view, b_preshuffled=True)
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        assert torch.equal(gy.view, ref), dt
        if dt == torch.float32:
            y, s = oracle.grouped_gemm(u8(a), u8(sa), u8(b), u8(sb), offsets)
            assert_gemm_fp32(gy.view, y, s, "grouped preshuffled")


@pytest.mark.parametrize("K", [512, 1024])
def test_grouped_gemm_tiled_bad_offsets_stay_inside_y(mx, K):
    say(f"grouped tiled gemm malformed offsets K={K}")
    E, N, M = 4, 256, 300
    a, sa = synth.canonical_mxfp4(M, K, seed=13)
    b, sb = synth.canonical_mxfp4(E * N, K, seed=14)
    A, SA, B, SB = to_dev(a, sa, b.reshape(E, N, K // 2), sb.reshape(E, N, K // 32))
    for table in ([0, 400, 10, -5, 300], [-100, 0, 1000, 20, 300], [0, 0, 0, 0, 0],
                  [0, 300, 300, 300, 300], [0, 300, 0, 300, 0], [0, 200, 100, 250, 300]):
        OFF = torch.tensor(table, dtype=torch.int32, device=dev())
        gy = Guarded((M, N), torch.float32)
        mx.mxfp4_grouped_gemm(A, SA, B, SB, OFF, gy.view)
        torch.cuda.synchronize()
        assert gy.intact(), table
        # the tiled kernel reads a table as its row ends clamped to [0, M]
        # and made non-decreasing (a running maximum), so the ranges stay
        # disjoint: rows of that table's experts equal the oracle's
        ends = np.maximum.accumulate(np.clip(np.array(table[1:]), 0, M))
        start = int(np.clip(table[0], 0, M))
        fixed = np.concatenate([[start], np.maximum(ends, start)]).astype(np.int32)
        r0, r1 = int(fixed[0]), int(fixed[-1])
        if r1 > r0:
            y, s = oracle.grouped_gemm(u8(a)[r0:r1], u8(sa)[r0:r1], u8(b).reshape(E, N, K // 2),
                                       u8(sb).reshape(E, N, K // 32), fixed - r0)
            assert_gemm_fp32(gy.view[r0:r1], y, s, f"bad table {table}")


def test_graph_replay_matches_eager(mx):
    """The decode step (requant, act-quant, GEMM) captured in a HIP graph gives
    the eager results on every replay, with eager work in between."""
    say("graph replay vs eager")
    d = dev()
    w = synth.bf16_normal((1024, 4096), 0.02, seed=3)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    C, S, G = to_dev(codes, scales, g.reshape(1))
    x = synth.activations(8, 4096, seed=4).to(d)
    wc = torch.empty((1024, 2048), dtype=torch.uint8, device=d)
    ws = torch.empty((1024, 128), dtype=torch.uint8, device=d)
    xc = torch.empty((8, 2048), dtype=torch.uint8, device=d)
    xs = torch.empty((8, 128), dtype=torch.uint8, device=d)
    y = torch.empty((8, 1024), dtype=torch.bfloat16, device=d)

    def step():
        mx.mxfp4_requant_from_nvfp4(C, S, G, wc, ws)
        mx.mxfp4_quantize_act(x, xc, xs)
        mx.mxfp4_gemm(xc, xs, wc, ws, y)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (wc, ws, xc, xs, y)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in (wc, ws, xc, xs, y):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((wc, ws, xc, xs, y), ref):
            assert torch.equal(a, b)
        step()                          # eager work between replays
        torch.cuda.synchronize()


# ---- act-quant + GEMM in one call ---------------------------------------------------
def same_bits(a, b):
    """Bitwise equality that also accepts NaN against NaN (payloads may differ)."""
    a, b = a.float().cpu(), b.float().cpu()
    both_nan = torch.isnan(a) & torch.isnan(b)
    return bool(((a.view(torch.int32) == b.view(torch.int32)) | both_nan).all())


@pytest.mark.parametrize("M,N,K,ldx", [(1, 1000, 4096, 4096), (2, 12600, 2048, 2048), (5, 300, 2048, 2048),
                                       (16, 12288, 4096, 4096), (17, 257, 4096, 4104),
                                       (33, 1040, 2048, 2056), (64, 4099, 4096, 4096),
                                       (65, 512, 4096, 4096), (200, 300, 1024, 1032),
                                       (8, 256, 1024, 1024)])
def test_linear_bf16_matches_act_quant_then_gemm(mx, M, N, K, ldx):
    """mxfp4_linear_bf16 gives the act-quant call followed by the GEMM bit for
    bit: one launch for the decode shapes (M <= 16, K = 2048/4096), the two
    launches through the workspace otherwise (M = 17 .. 200; K = 1024); rows
    wider than K; both output types; NaN and Inf blocks in x."""
    say(f"linear bf16 M={M} N={N} K={K} ldx={ldx}")
    x = synth.activations(M, ldx, seed=M + N, outlier_seed=K).to(dev())
    if M >= 5:
        x[1, 40] = float("nan")
        x[2, K - 1] = float("inf")
        x[4, 64:96] = 0.0
    w = synth.bf16_normal((N, K), 0.02, seed=N)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()))
    xc, xs = mx.mxfp4_quantize_act(x, K=K)
    for dt in (torch.bfloat16, torch.float32):
        ref = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=dt)
        gy = Guarded((M, N), dt)
        mx.mxfp4_linear_bf16(x, wc, ws, gy.view, K=K)
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        assert same_bits(gy.view, ref), dt


def test_linear_bf16_against_oracle(mx):
    """The one-launch form against the oracle's act-quant and GEMM (decode
    weight, outlier activations, M = 8)."""
    M, N, K = 8, 2048, 4096
    say(f"linear bf16 vs oracle M={M} N={N} K={K}")
    x = synth.activations(M, K, seed=91, outlier_seed=92)
    w = synth.bf16_normal((N, K), 0.02, seed=93)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    oc, os_ = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()))
    y32 = mx.mxfp4_linear_bf16(x.to(dev()), wc, ws, out_dtype=torch.float32)
    yb = mx.mxfp4_linear_bf16(x.to(dev()), wc, ws, out_dtype=torch.bfloat16)
    ac, as_ = oracle.quantize_act(bf16_bits(x))
    y, s = oracle.gemm(ac, as_, oc, os_)
    assert_gemm_fp32(y32, y, s, "linear fp32")
    assert_gemm_bf16(yb, y, "linear bf16")


@pytest.mark.parametrize("M,N,K,ldx", [(1, 1000, 4096, 4096), (5, 300, 2048, 2048),
                                       (16, 2048, 4096, 4104), (17, 257, 4096, 4104),
                                       (200, 300, 1024, 1032)])
def test_linear_bf16_uos_matches_act_quant_then_gemm(mx, M, N, K, ldx):
    """The UOS activation rule through mxfp4_linear_bf16 (one launch and two)
    equals the UOS act-quant call followed by the GEMM, bit for bit."""
    say(f"linear bf16 uos M={M} N={N} K={K} ldx={ldx}")
    x = synth.activations(M, ldx, seed=M + 3 * N, outlier_seed=K + 1).to(dev())
    w = synth.bf16_normal((N, K), 0.02, seed=N + 1)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()),
                                         scale_rule="uos")
    xc, xs = mx.mxfp4_quantize_act(x, K=K, scale_rule="uos")
    _, xs_ocp = mx.mxfp4_quantize_act(x, K=K)
    assert not torch.equal(xs, xs_ocp), "the input does not tell the rules apart"
    for dt in (torch.bfloat16, torch.float32):
        ref = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=dt)
        gy = Guarded((M, N), dt)
        mx.mxfp4_linear_bf16(x, wc, ws, gy.view, K=K, scale_rule="uos")
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        assert same_bits(gy.view, ref), dt


def test_linear_bf16_uos_against_oracle(mx):
    """The one-launch form under UOS against the oracle (both operands under
    the UOS rule)."""
    M, N, K = 8, 2048, 4096
    say(f"linear bf16 uos vs oracle M={M} N={N} K={K}")
    x = synth.activations(M, K, seed=94, outlier_seed=95)
    w = synth.bf16_normal((N, K), 0.02, seed=96)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    oc, os_ = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()), scale_rule="uos")
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()),
                                         scale_rule="uos")
    y32 = mx.mxfp4_linear_bf16(x.to(dev()), wc, ws, out_dtype=torch.float32, scale_rule="uos")
    ac, as_ = oracle.quantize_act(bf16_bits(x), scale_rule="uos")
    y, s = oracle.gemm(ac, as_, oc, os_)
    assert_gemm_fp32(y32, y, s, "linear uos fp32")


@pytest.mark.parametrize("M,N,K", [(1, 1000, 4096), (8, 2048, 4096), (5, 300, 2048),
                                   (33, 1040, 2048), (100, 300, 1024), (150, 260, 800),
                                   (300, 1000, 1024), (4096, 8192, 4096), (20, 13001, 2048),
                                   (1400, 12288, 1024)])
def test_linear_bf16_row_bias(mx, M, N, K):
    """A bf16 row bias through every GEMM path (one-launch decode, skinny, with
    its slots refilled past 12288 rows, generic, tiled with a ragged N,
    several rounds of tiles, half tiles in the last round), against the
    oracle's act-quant, requant and GEMM plus the bias before the one
    rounding.  Sizes the oracle cannot finish whole are checked on sampled
    rows."""
    say(f"linear bf16 + bias M={M} N={N} K={K}")
    x = synth.activations(M, K, seed=M + 7, outlier_seed=K + 7)
    w = synth.bf16_normal((N, K), 0.02, seed=N + 7)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(N)) * 2).to(torch.bfloat16)
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(1).to(dev()))
    oc, os_ = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    ac, as_ = oracle.quantize_act(bf16_bits(x))
    rows = np.arange(M) if M * N <= 2_000_000 else np.unique(
        np.concatenate([[0, M - 1], np.random.default_rng(1).integers(0, M, 24)]))
    pm, pn = np.repeat(rows, N), np.tile(np.arange(N), rows.size)
    y, s = oracle.gemm_at(ac, as_, oc, os_, pm, pn)
    y, s = oracle.add_row_bias(y.reshape(rows.size, N), s.reshape(rows.size, N), bf16_bits(bias))
    for dt in (torch.float32, torch.bfloat16):
        gy = Guarded((M, N), dt)
        mx.mxfp4_linear_bf16(x.to(dev()), wc, ws, gy.view, bias=bias.to(dev()))
        torch.cuda.synchronize()
        assert gy.intact(), "write outside y"
        got = gy.view[torch.from_numpy(rows).to(dev())]
        if dt == torch.float32:
            assert_gemm_fp32(got, y, s, f"bias fp32 M={M}")
        else:
            assert_gemm_bf16(got, y, f"bias bf16 M={M}")


def test_gemm_at_the_32bit_offset_limit(mx):
    """The tiled kernel reaches each operand through a buffer descriptor with
    32-bit offsets, so it takes operands under 2 GiB: A of 2^31 - 2048 bytes
    (1048575 rows at K = 4096) runs tiled; A of exactly 2^31 bytes goes to the
    16x16x128 tile kernel, which addresses with 64 bits.  Both are checked on
    sampled rows, the last 40 included (the largest offsets)."""
    K, N = 4096, 256
    d = dev()
    m_over = (1 << 31) // (K // 2)
    ac, as_ = synth.canonical_mxfp4(m_over, K, seed=71, device=d)
    bc, bs = synth.canonical_mxfp4(N, K, seed=72, device=d)
    b_cpu = (u8(bc.cpu()), u8(bs.cpu()))
    rng = np.random.default_rng(73)
    for M in (m_over - 1, m_over):
        say(f"gemm at the offset limit M={M} N={N} K={K}")
        y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
        mx.mxfp4_gemm(ac[:M], as_[:M], bc, bs, y)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([[0, 1], np.arange(M - 40, M), rng.integers(0, M, 24)]))
        ri = torch.from_numpy(rows).to(d)
        yo, _ = oracle.gemm(u8(ac[ri].cpu()), u8(as_[ri].cpu()), *b_cpu)
        assert_gemm_bf16(y[ri], yo, f"offset limit M={M}")
        del y
