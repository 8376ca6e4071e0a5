"""GPU parity of the MoE expert epilogues against the CPU oracle: the
activation between the two grouped GEMMs (silu(gate) * up, rounded to bf16 and
quantized to MXFP4) and the top-k combine, alone and inside a whole MoE layer.

The activation's codes and scale bytes must match the oracle's exactly, except
where the fp32 value h lies within ULP_WINDOW fp32 ulps of a bf16 rounding
midpoint: the GPU's exp and reciprocal are within about 2 ulp, not correctly
rounded, so there either bf16 neighbour is correct, and the block must equal
the oracle's quantization of one of those choices.  The combine accumulates
topk fp32 fmas, so its error bound is topk * 2^-24 * sum_j |w_j y_j| before
the output rounding (plus half a bf16 ulp for bf16 output)."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bf16_bits, dev, f32, say, u8

pytestmark = pytest.mark.gpu

ULP_WINDOW = 8           # fp32 ulps from a bf16 midpoint that count as a tie
MAX_AMBIGUOUS = 10       # per block; more would mean the inputs are degenerate


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bf16_values(bits):
    return bf16_tensor(bits).double().numpy()


# ---- activation + quantization ----------------------------------------------------
def check_silu_quant(gpu_codes, gpu_scales, gu_bits, I, rule, label):
    hb, hf = oracle.silu_mul(gu_bits, I)
    oc, os_ = oracle.quantize_act(hb, scale_rule=rule)
    M = hb.shape[0]
    nb = I // 32
    diff = (gpu_scales != os_) | (gpu_codes.reshape(M, nb, 16) != oc.reshape(M, nb, 16)).any(-1)
    if not diff.any():
        return 0
    hbits = hf.view(np.uint32)
    low = (hbits & 0xFFFF).astype(np.int64)
    finite = (hbits & 0x7F800000) != 0x7F800000
    ambiguous = (np.abs(low - 0x8000) <= ULP_WINDOW) & finite
    for m, j in np.argwhere(diff):
        sl = slice(32 * j, 32 * j + 32)
        idx = np.nonzero(ambiguous[m, sl])[0]
        assert 0 < idx.size <= MAX_AMBIGUOUS, (
            f"{label}: row {m} block {j} differs and has {idx.size} near-tie values "
            f"(gpu byte {gpu_scales[m, j]} oracle {os_[m, j]})")
        base = hb[m, sl].copy()
        trunc = (hbits[m, sl] >> 16).astype(np.uint16)
        want_c, want_s = gpu_codes[m, 16 * j:16 * j + 16], gpu_scales[m, j]
        found = False
        for pick in itertools.product((0, 1), repeat=idx.size):
            cand = base.copy()
            cand[idx] = trunc[idx] + np.array(pick, dtype=np.uint16)
            c, s = oracle.mx_quantize_block(bf16_values(cand), rule)
            if s == want_s and np.array_equal(c, want_c):
                found = True
                break
        assert found, f"{label}: row {m} block {j} matches no rounding of its near-tie values"
    return int(diff.sum())


def silu_quant_both(mx, gu_cpu, I=None, rule="ocp"):
    M, ldg = gu_cpu.shape
    I = ldg // 2 if I is None else I
    gc = Guarded((M, I // 2), torch.uint8)
    gs = Guarded((M, I // 32), torch.uint8)
    mx.mxfp4_silu_mul_quantize(gu_cpu.to(dev()), gc.view, gs.view, I=I, scale_rule=rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the output"
    return u8(gc.view), u8(gs.view)


def gate_up_input(M, ldg, seed, scale=1.5):
    """gate_up-shaped bf16 rows: N(0, scale^2), 1% of the columns x50."""
    x = synth.activations(M, ldg, seed=seed, outlier_seed=seed + 1).float() * scale
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("M,I,ldg", [(1, 32, 64), (37, 96, 200), (300, 1024, 2048),
                                     (5, 1024, 2056), (64, 4096, 8192)])
def test_silu_mul_quantize_random(mx, M, I, ldg):
    say(f"silu_mul_quantize M={M} I={I} ldg={ldg}")
    gu = gate_up_input(M, ldg, seed=M + I)
    gc, gs = silu_quant_both(mx, gu, I)
    n = check_silu_quant(gc, gs, bf16_bits(gu), I, "ocp", f"M={M} I={I}")
    say(f"  blocks resolved through near-ties: {n}")


def special_gate_up(seed):
    """Every awkward gate value against ordinary and awkward up values."""
    rng = np.random.default_rng(seed)
    M, I = 48, 256
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e30, -1e30, 100.0, -100.0, 88.5,
                         -88.5, 89.0, -89.0, 17.0, -17.0, 1e-40, -1e-40, 2.0 ** -133, 3.0,
                         -3.0, 104.0, -104.0, 105.0, -105.0], dtype=np.float32)
    g = rng.normal(0, 2, (M, I)).astype(np.float32)
    u = rng.normal(0, 2, (M, I)).astype(np.float32)
    pick = rng.random((M, I)) < 0.15
    g[pick] = rng.choice(specials, size=int(pick.sum()))
    pick = rng.random((M, I)) < 0.05
    u[pick] = rng.choice(specials, size=int(pick.sum()))
    # rows 40..47: NaN/Inf-free, so their blocks exercise the finite paths only
    fin = ~np.isfinite(g[40:]) | ~np.isfinite(u[40:])
    g[40:][fin], u[40:][fin] = 1.0, 1.0
    return torch.from_numpy(np.concatenate([g, u], axis=1)).to(torch.bfloat16)


@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_silu_mul_quantize_special_values(mx, rule):
    say(f"silu_mul_quantize specials {rule}")
    gu = special_gate_up(7)
    gc, gs = silu_quant_both(mx, gu, rule=rule)
    check_silu_quant(gc, gs, bf16_bits(gu), gu.shape[1] // 2, rule, f"specials {rule}")


def test_silu_mul_quantize_uos_random(mx):
    say("silu_mul_quantize uos [257, 1024]")
    gu = gate_up_input(257, 2048, seed=71)
    gc, gs = silu_quant_both(mx, gu, rule="uos")
    check_silu_quant(gc, gs, bf16_bits(gu), 1024, "uos", "uos")
    _, ocp_scales = oracle.silu_mul_quantize(bf16_bits(gu))
    assert (ocp_scales != gs).any(), "the input does not tell the rules apart"


def test_silu_mul_quantize_moe_full_size(mx):
    """The MoE configuration's down-projection input: 16384 routed rows of a
    gate_up output [16384, 2048]."""
    say("silu_mul_quantize [16384, 2048] full compare")
    gu = gate_up_input(16384, 2048, seed=81)
    gc, gs = silu_quant_both(mx, gu)
    n = check_silu_quant(gc, gs, bf16_bits(gu), 1024, "ocp", "moe full")
    say(f"  blocks resolved through near-ties: {n} of {gs.size}")


# ---- top-k combine -------------------------------------------------------------
def ulp_bf16(v):
    _, e = np.frexp(np.abs(v))
    return np.maximum(np.ldexp(1.0, e - 8), 2.0 ** -133)


def assert_combine(gpu, out, s, topk, label):
    g = f32(gpu.float()).astype(np.float64)
    nan = np.isnan(out)
    assert np.array_equal(np.isnan(g), nan), f"{label}: NaN positions differ"
    bound = topk * 2.0 ** -24 * s + 1e-45
    if gpu.dtype == torch.bfloat16:
        bound = bound + 0.5 * ulp_bf16(np.maximum(np.abs(g), np.abs(out)))
    err = np.where(nan, 0.0, np.abs(g - np.where(nan, 0.0, out)))
    ok = err <= np.where(nan, 0.0, bound)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} outputs outside the bound; first {i}: "
                             f"gpu {g[i]!r} oracle {out[i]!r} s {s[i]!r}")


def combine_both(mx, y_cpu, rows, weights, H=None, out_dtype=torch.bfloat16):
    T = rows.shape[0]
    H = y_cpu.shape[1] if H is None else H
    go = Guarded((T, H), out_dtype)
    mx.mxfp4_moe_combine(y_cpu.to(dev()), rows.to(dev()), weights.to(dev()), go.view, H=H)
    torch.cuda.synchronize()
    assert go.intact(), "write outside out"
    out, s = oracle.moe_combine(bf16_bits(y_cpu), rows.numpy(), weights.numpy(), H)
    return go.view, out, s


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_moe_combine_full_size(mx, dt):
    """The MoE configuration: 2048 tokens, top-8 of 128 experts, H = 4096."""
    say(f"moe_combine T=2048 topk=8 H=4096 {dt}")
    _, _, rows, w = synth.route_topk_full(2048, 128, 8, seed=34)
    y = synth.activations(2048 * 8, 4096, seed=36)
    gpu, out, s = combine_both(mx, y, rows, w, out_dtype=dt)
    assert_combine(gpu, out, s, 8, f"full {dt}")


@pytest.mark.parametrize("T,topk,H,ldy", [(1, 1, 8, 8), (33, 3, 72, 80), (100, 11, 520, 520),
                                          (7, 64, 2056, 2064), (300, 8, 4096, 4104)])
def test_moe_combine_ragged(mx, T, topk, H, ldy):
    say(f"moe_combine T={T} topk={topk} H={H} ldy={ldy}")
    rng = np.random.default_rng(T + topk)
    R = T * topk + 5
    y = synth.activations(R, ldy, seed=T + 3)
    rows = torch.from_numpy(rng.integers(0, R, (T, topk)).astype(np.int32))
    w = torch.from_numpy(rng.uniform(-1, 1, (T, topk)).astype(np.float32))
    for dt in (torch.bfloat16, torch.float32):
        gpu, out, s = combine_both(mx, y, rows, w, H=H, out_dtype=dt)
        assert_combine(gpu, out, s, topk, f"ragged {dt}")


def test_moe_combine_clamps_rows_and_propagates_nan(mx):
    """Out-of-range row indices are clamped to [0, R) (a bad table reads only
    inside y); a NaN in a routed row reaches exactly its token's column."""
    say("moe_combine clamp + NaN")
    T, topk, H, R = 16, 4, 64, 40
    rng = np.random.default_rng(9)
    y = synth.activations(R, H, seed=10)
    y[5, 17] = float("nan")
    rows = rng.integers(0, R, (T, topk)).astype(np.int32)
    rows[0, 0], rows[1, 2], rows[2, 3] = -7, R + 3, 2 ** 31 - 1
    rows[3, 1] = 5
    w = rng.uniform(0.1, 1, (T, topk)).astype(np.float32)
    go = torch.empty((T, H), dtype=torch.float32, device=dev())
    mx.mxfp4_moe_combine(y.to(dev()), torch.from_numpy(rows).to(dev()),
                         torch.from_numpy(w).to(dev()), go)
    out, s = oracle.moe_combine(bf16_bits(y), np.clip(rows, 0, R - 1), w)
    assert_combine(go, out, s, topk, "clamped")
    assert np.isnan(f32(go)[3, 17])


# ---- a whole MoE layer ----------------------------------------------------------------
# ---- gate_up GEMM with the activation in its epilogue ------------------------------
def interleaved_to_stacked(cols):
    """Column (or weight-row) order of the fused call, 64-groups of 32 gate then
    32 up, -> [gate | up] stacked: index arrays for the last axis."""
    n = cols
    q, r = np.divmod(np.arange(n // 2), 32)
    return np.concatenate([64 * q + r, 64 * q + 32 + r])


def fused_glu_both(mx, E, counts, I, K, seed, rule):
    """The fused call on exact-domain operands (E2M1 codes, scale bytes 126..128:
    every fp32 sum of the GEMM is exact, so the bf16 gate_up values the fused
    epilogue sees are the RNE of the exact sums the oracle computes), checked
    against the oracle from the same inputs and against the two-call path."""
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M, N = int(offsets[-1]), 2 * I
    ac, as_ = synth.canonical_mxfp4(M, K, seed=seed, scale_lo=126, scale_hi=128)
    bc, bs = synth.canonical_mxfp4(E * N, K, seed=seed + 1, scale_lo=126, scale_hi=128)
    bc, bs = bc.reshape(E, N, K // 2), bs.reshape(E, N, K // 32)
    d = dev()
    A = [t.to(d) for t in (ac, as_, bc, bs)] + [torch.from_numpy(offsets).to(d)]
    gc = Guarded((M, I // 2), torch.uint8)
    gs = Guarded((M, I // 32), torch.uint8)
    mx.mxfp4_grouped_gemm_silu_quantize(*A, gc.view, gs.view, scale_rule=rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the outputs"
    # oracle: exact grouped GEMM, bf16 RNE, columns back to [gate | up], activation
    y, _ = oracle.grouped_gemm(u8(ac), u8(as_), u8(bc), u8(bs), offsets)
    assert (np.abs(y) < 2.0 ** 20).all()          # the exact-sum domain
    gu = oracle.bf16_from_double_array(y)[:, interleaved_to_stacked(N)]
    check_silu_quant(u8(gc.view), u8(gs.view), gu, I, rule, f"fused glu {rule}")
    # the two calls it replaces, bit for bit
    y1 = mx.mxfp4_grouped_gemm(*A, out_dtype=torch.bfloat16)
    idx = torch.from_numpy(interleaved_to_stacked(N)).to(d)
    hc, hs = mx.mxfp4_silu_mul_quantize(y1[:, idx].contiguous(), scale_rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(hc, gc.view) and torch.equal(hs, gs.view), "fused != two calls"
    if K % 1024 == 0 and M:
        # the same call on pre-shuffled weight codes
        pc, ps = mx.mxfp4_grouped_gemm_silu_quantize(
            A[0], A[1], mx.mxfp4_preshuffle_weights(A[2]), A[3], A[4], scale_rule=rule,
            b_preshuffled=True)
        torch.cuda.synchronize()
        assert torch.equal(pc, gc.view) and torch.equal(ps, gs.view), "preshuffled"


@pytest.mark.parametrize("E,counts,I,K", [
    (4, [0, 37, 130, 1], 96, 512),             # empty expert, ragged rows, N = 192 < one tile
    (3, [128, 0, 300], 256, 1024),              # a partial tile of waves, the persistent walk
    (8, [64, 200, 5, 0, 129, 256, 17, 90], 512, 2048)])
@pytest.mark.parametrize("rule", ["ocp", "uos"])
def test_grouped_gemm_silu_quantize(mx, E, counts, I, K, rule):
    say(f"grouped gemm + silu quantize E={E} I={I} K={K} {rule}")
    fused_glu_both(mx, E, counts, I, K, seed=E * 7 + I, rule=rule)


def test_grouped_gemm_silu_quantize_moe_size(mx):
    """At the MoE bench's shape (128 experts, 2048 tokens x top-8 routed, H =
    4096, I = 1024; real routing) the fused call equals the two calls, bit for
    bit, on random MXFP4 weights (made on the GPU: 512 MiB of codes) and
    quantized activations."""
    say("grouped gemm + silu quantize, MoE size")
    E, T, TOPK, H, I = 128, 2048, 8, 4096, 1024
    d = dev()
    perm, offsets, _, _ = synth.route_topk_full(T, E, TOPK, seed=61)
    x = synth.activations(T, H, seed=62, outlier_seed=63).to(d)
    wc, ws = synth.canonical_mxfp4(E * 2 * I, H, seed=64, device=d)
    wc, ws = wc.reshape(E, 2 * I, H // 2), ws.reshape(E, 2 * I, H // 32)
    off = offsets.to(d)
    xc, xs = mx.mxfp4_quantize_act(x, row_index=perm.to(d))
    hc, hs = mx.mxfp4_grouped_gemm_silu_quantize(xc, xs, wc, ws, off)
    y1 = mx.mxfp4_grouped_gemm(xc, xs, wc, ws, off, out_dtype=torch.bfloat16)
    idx = torch.from_numpy(interleaved_to_stacked(2 * I)).to(d)
    rc, rs = mx.mxfp4_silu_mul_quantize(y1[:, idx].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(hc, rc) and torch.equal(hs, rs)
    # and the same call on pre-shuffled weight codes
    pc, ps = mx.mxfp4_grouped_gemm_silu_quantize(xc, xs, mx.mxfp4_preshuffle_weights(wc), ws, off,
                                                 b_preshuffled=True)
    torch.cuda.synchronize()
    assert torch.equal(pc, hc) and torch.equal(ps, hs)


def test_moe_layer_end_to_end(mx):
    """Routed tokens through the whole expert path on the GPU: gathered
    act-quant, grouped gate_up GEMM, expert activation + quantization, grouped
    down GEMM, top-k combine (16 experts, 256 tokens, top-4, H = 512, I = 256).
    Every expected value is the oracle's, run on the same seeded inputs:

    * the act-quant bit for bit;
    * the gate_up GEMM bit for bit: the operands sit in the exact-sum domain
      (activations without outlier channels quantize to scale bytes 125..127,
      weights carry 126..128; every fp32 sum is a multiple of 2^-5 below 2^16),
      so the GPU's bf16 output is the RNE of the oracle's exact sum;
    * the activation against the oracle's activation of those bf16 values,
      blocks differing only at near-ties of h;
    * the down GEMM within one bf16 ulp, on the rows whose h equals the
      oracle's (the others carry a near-tie choice into the sum);
    * the combine within its fp32 bound plus the bf16 ulp each routed input
      may carry, for the tokens whose rows were all compared."""
    say("MoE layer end to end")
    E, T, TOPK, H, I = 16, 256, 4, 512, 256
    d = dev()
    perm, offsets, rows, w = synth.route_topk_full(T, E, TOPK, seed=51)
    x = synth.activations(T, H, seed=52)
    wgt = {}
    for name, (N, K), seed in (("gate_up", (2 * I, H), 54), ("down", (H, I), 55)):
        c, sc = synth.canonical_mxfp4(E * N, K, seed=seed, scale_lo=126, scale_hi=128)
        wgt[name] = (c.reshape(E, N, K // 2), sc.reshape(E, N, K // 32))
    off = offsets.to(d)
    xc, xs = mx.mxfp4_quantize_act(x.to(d), row_index=perm.to(d))
    y1 = mx.mxfp4_grouped_gemm(xc, xs, *[t.to(d) for t in wgt["gate_up"]], off,
                               out_dtype=torch.bfloat16)
    hc, hs = mx.mxfp4_silu_mul_quantize(y1)
    y2 = mx.mxfp4_grouped_gemm(hc, hs, *[t.to(d) for t in wgt["down"]], off,
                               out_dtype=torch.bfloat16)
    out = mx.mxfp4_moe_combine(y2, rows.to(d), w.to(d), out_dtype=torch.float32)
    torch.cuda.synchronize()

    # the oracle's chain from the same inputs
    ac, as_ = oracle.quantize_act(bf16_bits(x), row_index=perm.numpy())
    assert np.array_equal(u8(xc), ac) and np.array_equal(u8(xs), as_)
    assert as_.min() >= 125 and as_.max() <= 127, "activation scales left the exact domain"
    y1o, _ = oracle.grouped_gemm(ac, as_, u8(wgt["gate_up"][0]), u8(wgt["gate_up"][1]),
                                 offsets.numpy())
    y1b = oracle.bf16_from_double_array(y1o)
    assert np.array_equal(bf16_bits(y1), y1b), "gate_up: not the RNE of the exact sums"
    check_silu_quant(u8(hc), u8(hs), y1b, I, "ocp", "layer activation")
    hco, hso = oracle.silu_mul_quantize(y1b, I)
    y2o, _ = oracle.grouped_gemm(hco, hso, u8(wgt["down"][0]), u8(wgt["down"][1]),
                                 offsets.numpy())
    same = (u8(hc) == hco).all(1) & (u8(hs) == hso).all(1)
    assert same.sum() >= same.size - 8, f"{int((~same).sum())} rows of h differ"
    ok = oracle.gemm_bf16_ok(bf16_bits(y2)[same], y2o[same])
    assert ok.all(), f"down: {int((~ok).sum())} outputs off by >1 bf16 ulp"
    y2b = oracle.bf16_from_double_array(y2o)
    ref, s = oracle.moe_combine(y2b, rows.numpy(), w.numpy())
    # each routed input may sit one bf16 ulp from the oracle's
    yv = np.abs(bf16_values(y2b))
    carry = np.zeros_like(ref)
    for j in range(TOPK):
        carry += np.abs(w.numpy()[:, j])[:, None] * ulp_bf16(yv[rows.numpy()[:, j]]) * 2
    tok = same[rows.numpy()].all(1)
    g = out.cpu().double().numpy()
    bound = TOPK * 2.0 ** -24 * s + carry + 1e-45
    err = np.abs(g - ref)
    assert (err[tok] <= bound[tok]).all(), "layer combine outside its bound"
    assert tok.sum() >= T - 4 * 8
    assert torch.isfinite(out).all()


def test_moe_epilogues_graph_replay_matches_eager(mx):
    """The expert activation + quantization and the combine captured in a HIP
    graph give the eager results on every replay, with eager work between."""
    say("moe epilogues: graph replay vs eager")
    d = dev()
    gu = gate_up_input(256, 512, seed=97).to(d)
    _, _, rows, w = synth.route_topk_full(64, 16, 4, seed=98)
    y = synth.activations(256, 384, seed=99).to(d)
    rows, w = rows.to(d), w.to(d)
    hc = torch.empty((256, 128), dtype=torch.uint8, device=d)
    hs = torch.empty((256, 8), dtype=torch.uint8, device=d)
    out = torch.empty((64, 384), dtype=torch.bfloat16, device=d)

    def step():
        mx.mxfp4_silu_mul_quantize(gu, hc, hs)
        mx.mxfp4_moe_combine(y, rows, w, out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (hc, hs, out)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in (hc, hs, out):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((hc, hs, out), ref):
            assert torch.equal(a, b)
        step()
        torch.cuda.synchronize()


def test_moe_epilogues_rows_past_one_grid(mx):
    """The activation kernel over 131073 rows and the combine over 65537
    tokens: more than one launch grid's rows, walked with a grid stride."""
    M, I = 2 * 65535 + 3, 32
    say(f"silu_mul_quantize rows past one grid M={M}")
    gu = gate_up_input(M, 2 * I, seed=43)
    gc, gs = silu_quant_both(mx, gu, I)
    check_silu_quant(gc, gs, bf16_bits(gu), I, "ocp", "rows past one grid")
    T, TOPK, H = 65537, 2, 8
    say(f"moe_combine tokens past one grid T={T}")
    _, _, rows, w = synth.route_topk_full(T, 4, TOPK, seed=44)
    y = synth.activations(T * TOPK, H, seed=45)
    go, out, sc = combine_both(mx, y, rows, w)
    assert_combine(go, out, sc, TOPK, "combine past one grid")
