"""Every output at full size: the three prefill GEMMs (M = 4096 tokens;
(N, K) = (4096, 4096), (28672, 4096), (4096, 14336)) and the MoE layer
(128 experts, 2048 tokens, top-8; gate_up [2048, 4096], down [4096, 1024]),
with NVFP4-derived weights (bf16 N(0, 0.02)) and activations N(0, 1) with 1%
outlier channels x50.

The expected values come from the oracle on the same seeded inputs: its
requant and act-quant (the GPU's must equal them bit for bit), then the GEMM
as fp64 dequantize + numpy matmul (oracle.gemm_blas, error about K * 2^-53 *
S).  Each element must meet the GEMM bar (fp32 within 1e-5 * S, bf16 within
one ulp of RNE(y)); an element that misses the bf16 bar against the BLAS sum
is re-checked against the exact integer-sum oracle at that position, and the
exact oracle also checks a sample of positions on every prefill shape.

The expert activation decides quantized codes from bf16 gate/up values that
the GEMM bar lets differ from RNE(y) where y lies near a bf16 rounding
midpoint.  Its check is therefore by intervals: each h value's range over the
admissible gate/up values (and over both neighbours of an h that lies within
a few fp32 ulps of a bf16 midpoint) bounds the block's amax, hence its scale
byte, and each code given the GPU's scale byte.  Nearly every block must also
equal the oracle's chain on RNE(y) bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_bits, dev, f32, say, u8

pytestmark = pytest.mark.gpu

ULP_WINDOW = 8           # fp32 ulps from a bf16 midpoint that count as a tie


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def ordered(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def from_ordered(o):
    o = np.asarray(o, dtype=np.int64)
    return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)


def check_fp32(gpu, y, s, K, label):
    g = np.asarray(gpu, dtype=np.float64)
    tol = oracle.GEMM_FP32_RTOL * s + K * 2.0 ** -52 * s
    bad = ~(np.abs(g - y) <= tol)
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {bad.size} fp32 outputs outside "
                           f"1e-5*S, first at {np.argwhere(bad)[0].tolist()}")


def check_bf16(gpu_bits, y, exact_at, label):
    """gpu_bits vs RNE(y) within one ulp; misses re-checked against the exact
    oracle (exact_at(rows, cols) -> y at those positions).  Returns the number
    of re-checked elements."""
    ok = oracle.gemm_bf16_ok(gpu_bits, y)
    if ok.all():
        return 0
    pm, pn = np.nonzero(~ok)
    assert pm.size <= 1000, f"{label}: {pm.size} bf16 outputs off by >1 ulp of the BLAS sum"
    ye = exact_at(pm, pn)
    ok2 = oracle.gemm_bf16_ok(gpu_bits[pm, pn], ye)
    assert ok2.all(), (f"{label}: {int((~ok2).sum())} bf16 outputs off by >1 ulp of the exact "
                       f"sum, first at {(int(pm[~ok2][0]), int(pn[~ok2][0]))}")
    return int(pm.size)


# ---- prefill --------------------------------------------------------------------------
PREFILL = [(4096, 4096, 21, 24, 26), (28672, 4096, 22, 24, 26), (4096, 14336, 23, 25, 27)]


def sample_positions(M, N, seed, n_random=3000):
    rng = np.random.default_rng(seed)
    pm = [rng.integers(0, M, n_random)]
    pn = [rng.integers(0, N, n_random)]
    for m in (0, 1, 127, 128, 255, 256, M - 1):           # row runs at tile edges
        cols = np.unique(np.concatenate([np.arange(0, min(N, 300)), rng.integers(0, N, 200),
                                         [N - 1]]))
        pm.append(np.full(cols.size, m))
        pn.append(cols)
    return np.concatenate(pm), np.concatenate(pn)


@pytest.mark.parametrize("N,K,wseed,xseed,oseed", PREFILL)
def test_prefill_every_output(mx, N, K, wseed, xseed, oseed):
    M = 4096
    say(f"prefill M={M} N={N} K={K}: every output")
    d = dev()
    w = synth.bf16_normal((N, K), 0.02, seed=wseed)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    del w
    x = synth.activations(M, K, seed=xseed, outlier_seed=oseed)
    oc, os_ = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()))
    ac, as_ = oracle.quantize_act(bf16_bits(x))
    wc, ws = mx.mxfp4_requant_from_nvfp4(codes.to(d), scales.to(d), g.reshape(1).to(d))
    xc, xs = mx.mxfp4_quantize_act(x.to(d))
    yb = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.bfloat16)
    yf = mx.mxfp4_gemm(xc, xs, wc, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(u8(wc), oc) and np.array_equal(u8(ws), os_), "requant"
    assert np.array_equal(u8(xc), ac) and np.array_equal(u8(xs), as_), "act-quant"
    y, s = oracle.gemm_blas(ac, as_, oc, os_)
    check_fp32(f32(yf), y, s, K, f"{N}x{K} fp32")
    n = check_bf16(bf16_bits(yb), y, lambda pm, pn: oracle.gemm_at(ac, as_, oc, os_, pm, pn)[0],
                   f"{N}x{K} bf16")
    pm, pn = sample_positions(M, N, seed=N + K)
    ye, _ = oracle.gemm_at(ac, as_, oc, os_, pm, pn)
    ok = oracle.gemm_bf16_ok(bf16_bits(yb)[pm, pn], ye)
    assert ok.all(), f"{int((~ok).sum())} sampled outputs off the exact oracle by >1 bf16 ulp"
    say(f"  {M * N} outputs checked; {n} re-checked against the exact sum")


# ---- MoE --------------------------------------------------------------------------------
E, T, TOPK, H, I = 128, 2048, 8, 4096, 1024


@pytest.fixture(scope="module")
def moe(mx):
    """The MoE layer's inputs: NVFP4 expert weights drawn on the GPU (synth),
    held on the host as the shared input and requantized by each side; tokens
    with outlier channels; softmax top-8 routing.  The gate_up weight rows are
    read by the fused call as interleaved by 32 (gate, up) and by the oracle
    in the same row order."""
    say("MoE inputs: 128 experts, 2048 tokens, top-8")
    d = dev()
    perm, offsets, rows, weights = synth.route_topk_full(T, E, TOPK, seed=34)
    tokens = synth.activations(T, H, seed=33, outlier_seed=36)
    st = dict(perm=perm.numpy(), offsets=offsets.numpy(), rows=rows.numpy(),
              weights=weights.numpy(), tokens=tokens, gpu={}, orc={})
    for name, (N, K), seed in (("gate_up", (2 * I, H), 31), ("down", (H, I), 32)):
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=d)
        scales = torch.empty((E, N, K // 16), dtype=torch.uint8, device=d)
        gs = torch.empty((E,), dtype=torch.float32, device=d)
        for e in range(E):
            w = synth.bf16_normal((N, K), 0.02, seed=seed * 1000 + e, device=d)
            codes[e], scales[e], gs[e] = synth.nvfp4_from_bf16(w)
        hc, hs, hg = u8(codes), u8(scales), f32(gs)
        st["gpu"][name] = mx.mxfp4_requant_from_nvfp4(codes, scales, gs)
        st["orc"][name] = oracle.requant(hc, hs, hg)
        del codes, scales, gs
    torch.cuda.synchronize()
    for name in ("gate_up", "down"):
        wc, ws = st["gpu"][name]
        assert np.array_equal(u8(wc), st["orc"][name][0]), f"{name} requant codes"
        assert np.array_equal(u8(ws), st["orc"][name][1]), f"{name} requant scales"
    st["ac"], st["as"] = oracle.quantize_act(bf16_bits(tokens), row_index=st["perm"])
    return st


def grouped_blas(ac, as_, wc, ws, offsets):
    """Per expert e: oracle.gemm_blas of its rows against its weights."""
    M, N = ac.shape[0], wc.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            y[r0:r1], s[r0:r1] = oracle.gemm_blas(ac[r0:r1], as_[r0:r1], wc[e], ws[e])
    return y, s


def grouped_exact_at(ac, as_, wc, ws, offsets):
    def at(pm, pn):
        e = np.searchsorted(offsets, pm, side="right") - 1
        out = np.empty(pm.size, dtype=np.float64)
        for i in range(pm.size):
            out[i] = oracle.gemm_at(ac[pm[i]:pm[i] + 1], as_[pm[i]:pm[i] + 1], wc[e[i]],
                                    ws[e[i]], np.array([0]), pn[i:i + 1])[0][0]
        return out
    return at


def test_moe_grouped_gemms_every_output(mx, moe):
    """Both grouped GEMMs over every routed row: gate_up on the gathered token
    rows, down on a synthetic bf16 [16384, 1024] input N(0, 1).  The bench
    runs them on pre-shuffled weights: that call must give the same bytes."""
    d = dev()
    off = moe["offsets"]
    cases = [("gate_up", moe["tokens"], moe["perm"], 35), ("down", None, None, 35)]
    for name, x, perm, seed in cases:
        say(f"MoE grouped {name}: every output")
        if x is None:
            x = synth.activations(T * TOPK, I, seed=seed)
            ac, as_ = oracle.quantize_act(bf16_bits(x))
            xc, xs = mx.mxfp4_quantize_act(x.to(d))
        else:
            ac, as_ = moe["ac"], moe["as"]
            xc, xs = mx.mxfp4_quantize_act(x.to(d), row_index=torch.from_numpy(perm).to(d))
        wc, ws = moe["gpu"][name]
        y = mx.mxfp4_grouped_gemm(xc, xs, wc, ws, torch.from_numpy(off).to(d),
                                  out_dtype=torch.bfloat16)
        ysh = mx.mxfp4_grouped_gemm(xc, xs, mx.mxfp4_preshuffle_weights(wc), ws,
                                    torch.from_numpy(off).to(d), out_dtype=torch.bfloat16,
                                    b_preshuffled=True)
        torch.cuda.synchronize()
        assert torch.equal(ysh, y), f"{name}: pre-shuffled weights"
        del ysh
        assert np.array_equal(u8(xc), ac) and np.array_equal(u8(xs), as_), f"{name} act-quant"
        owc, ows = moe["orc"][name]
        yo, _ = grouped_blas(ac, as_, owc, ows, off)
        n = check_bf16(bf16_bits(y), yo, grouped_exact_at(ac, as_, owc, ows, off), name)
        say(f"  {yo.size} outputs checked; {n} re-checked against the exact sum")


def interleaved_to_stacked(n):
    q, r = np.divmod(np.arange(n // 2), 32)
    return np.concatenate([64 * q + r, 64 * q + 32 + r])


def bf16_candidates(y, s):
    """Ordered-int range [lo, hi] of the bf16 values the GPU may write for an
    exact sum y: RNE of any fp32 within 1e-5 * s of y, and within one ulp of
    RNE(y) (the GEMM bar)."""
    nom = ordered(oracle.bf16_from_double_array(y))
    tol = oracle.GEMM_FP32_RTOL * s
    lo = np.maximum(ordered(oracle.bf16_from_double_array(y - tol)), nom - 1)
    hi = np.minimum(ordered(oracle.bf16_from_double_array(y + tol)), nom + 1)
    return nom, lo, hi


def h_range(gate_up_y, gate_up_s):
    """For each h = bf16(silu(gate) * up): its nominal bits (from RNE(y)) and
    the least and greatest value it can take over the admissible gate/up bf16
    values and both neighbours of a near-tie h."""
    nom, lo, hi = bf16_candidates(gate_up_y, gate_up_s)
    g_idx, u_idx = np.arange(I), np.arange(I, 2 * I)
    hmin = np.full((gate_up_y.shape[0], I), np.inf)
    hmax = np.full((gate_up_y.shape[0], I), -np.inf)
    nominal = None
    for dg in (0, -1, 1):
        for du in (0, -1, 1):
            gsel = from_ordered(np.clip(nom[:, g_idx] + dg, lo[:, g_idx], hi[:, g_idx]))
            usel = from_ordered(np.clip(nom[:, u_idx] + du, lo[:, u_idx], hi[:, u_idx]))
            hb, hf = oracle.silu_mul(np.concatenate([gsel, usel], axis=1), I)
            if nominal is None:
                nominal = hb
            cands = [bf16_values(hb)]
            bits = hf.view(np.uint32)
            near = (np.abs((bits & 0xFFFF).astype(np.int64) - 0x8000) <= ULP_WINDOW)
            if near.any():
                trunc = (bits >> 16).astype(np.uint16)
                cands += [bf16_values(np.where(near, trunc, hb)),
                          bf16_values(np.where(near, trunc + np.uint16(1), hb))]
            for c in cands:
                np.minimum(hmin, c, out=hmin)
                np.maximum(hmax, c, out=hmax)
    return nominal, hmin, hmax


def check_glu_intervals(gpu_codes, gpu_scales, nominal, hmin, hmax, label):
    """Scale bytes within the range the block's amax interval allows; codes
    within the range of their h interval at the GPU's scale byte.  Returns
    the number of blocks that differ from the nominal chain."""
    R = nominal.shape[0]
    nb = I // 32
    assert np.isfinite(hmin).all() and np.isfinite(hmax).all(), f"{label}: non-finite h"
    amin = np.where((hmin <= 0) & (hmax >= 0), 0.0, np.minimum(np.abs(hmin), np.abs(hmax)))
    amax = np.maximum(np.abs(hmin), np.abs(hmax))
    blo = amin.reshape(R, nb, 32).max(-1)
    bhi = amax.reshape(R, nb, 32).max(-1)
    byte_lo = np.vectorize(oracle.shared_exponent)(blo)
    byte_hi = np.vectorize(oracle.shared_exponent)(bhi)
    bad = (gpu_scales < byte_lo) | (gpu_scales > byte_hi)
    assert not bad.any(), f"{label}: {int(bad.sum())} scale bytes outside their range"
    table = np.array([oracle.e2m1_value(c) for c in range(16)])
    nib = np.stack([gpu_codes & 15, gpu_codes >> 4], -1).reshape(R, I)
    got = table[nib]
    byte_el = np.repeat(gpu_scales, 32, axis=1)
    lo_bits = oracle.bf16_from_double_array(hmin)
    hi_bits = oracle.bf16_from_double_array(hmax)
    assert np.array_equal(bf16_values(lo_bits), hmin) and np.array_equal(bf16_values(hi_bits), hmax)
    vlo = np.empty(got.shape)
    vhi = np.empty(got.shape)
    for b in np.unique(byte_el):
        m = byte_el == b
        vlo[m] = table[oracle.e2m1_encode_bf16_at_scale(lo_bits[m], int(b))]
        vhi[m] = table[oracle.e2m1_encode_bf16_at_scale(hi_bits[m], int(b))]
    bad = (got < vlo) | (got > vhi)
    assert not bad.any(), (f"{label}: {int(bad.sum())} codes outside their range, first at "
                           f"{np.argwhere(bad)[0].tolist()}")
    oc, os_ = oracle.quantize_act(nominal)
    same = (gpu_scales == os_) & (gpu_codes.reshape(R, nb, 16) == oc.reshape(R, nb, 16)).all(-1)
    return int((~same).sum()), (oc, os_)


@pytest.fixture(scope="module")
def gate_up_oracle(moe):
    """The oracle's gate_up sums over every routed row, in [gate | up] order."""
    owc, ows = moe["orc"]["gate_up"]
    y, s = grouped_blas(moe["ac"], moe["as"], owc, ows, moe["offsets"])
    idx = interleaved_to_stacked(2 * I)
    return np.ascontiguousarray(y[:, idx]), np.ascontiguousarray(s[:, idx])


def test_moe_layer_every_output(mx, moe, gate_up_oracle):
    """The whole MoE layer on the GPU: act-quant scattered to the routed rows,
    gate_up GEMM with the expert activation and its quantization in the
    epilogue, down GEMM, top-k combine (fp32 out), each stage against the
    oracle.  Stages after the activation are compared on the rows whose h
    equals the oracle's nominal h (the others carry an admissible choice)."""
    say("MoE layer: every output")
    d = dev()
    off = torch.from_numpy(moe["offsets"]).to(d)
    rows = torch.from_numpy(moe["rows"]).to(d)
    R = T * TOPK
    xc = torch.empty((R, H // 2), dtype=torch.uint8, device=d)
    xs = torch.empty((R, H // 32), dtype=torch.uint8, device=d)
    mx.mxfp4_quantize_act_scatter(moe["tokens"].to(d), rows, xc, xs)
    hc, hs = mx.mxfp4_grouped_gemm_silu_quantize(xc, xs, *moe["gpu"]["gate_up"], off)
    y2 = mx.mxfp4_grouped_gemm(hc, hs, *moe["gpu"]["down"], off, out_dtype=torch.bfloat16)
    out = mx.mxfp4_moe_combine(y2, rows, torch.from_numpy(moe["weights"]).to(d),
                               out_dtype=torch.float32)
    # the bench's configuration: both grouped GEMMs on pre-shuffled weights
    (gwc, gws), (dwc, dws) = moe["gpu"]["gate_up"], moe["gpu"]["down"]
    hcs, hss = mx.mxfp4_grouped_gemm_silu_quantize(xc, xs, mx.mxfp4_preshuffle_weights(gwc), gws,
                                                   off, b_preshuffled=True)
    y2s = mx.mxfp4_grouped_gemm(hc, hs, mx.mxfp4_preshuffle_weights(dwc), dws, off,
                                out_dtype=torch.bfloat16, b_preshuffled=True)
    torch.cuda.synchronize()
    assert torch.equal(hcs, hc) and torch.equal(hss, hs), "gate_up: pre-shuffled weights"
    assert torch.equal(y2s, y2), "down: pre-shuffled weights"
    del hcs, hss, y2s
    assert np.array_equal(u8(xc), moe["ac"]) and np.array_equal(u8(xs), moe["as"]), "dispatch"

    nominal, hmin, hmax = h_range(*gate_up_oracle)
    ndiff, (hco, hso) = check_glu_intervals(u8(hc), u8(hs), nominal, hmin, hmax, "activation")
    same = (u8(hc) == hco).all(1) & (u8(hs) == hso).all(1)
    say(f"  activation: {ndiff} of {R * (I // 32)} blocks differ from the nominal chain "
        f"(admissible), {int((~same).sum())} rows")
    assert ndiff <= R * (I // 32) // 100 and same.mean() >= 0.9

    owc, ows = moe["orc"]["down"]
    y2o, _ = grouped_blas(hco, hso, owc, ows, moe["offsets"])
    yb = bf16_bits(y2)
    n = check_bf16(yb[same], y2o[same],
                   lambda pm, pn: grouped_exact_at(hco, hso, owc, ows, moe["offsets"])(
                       np.nonzero(same)[0][pm], pn), "down")
    say(f"  down: {int(same.sum()) * H} outputs checked, {n} re-checked against the exact sum")

    y2b = oracle.bf16_from_double_array(y2o)
    ref, s = oracle.moe_combine(y2b, moe["rows"], moe["weights"])
    yv = np.abs(bf16_values(y2b))
    _, e = np.frexp(yv)
    ulp = np.ldexp(1.0, e - 8)
    carry = np.zeros_like(ref)
    for j in range(TOPK):
        carry += np.abs(moe["weights"][:, j])[:, None] * ulp[moe["rows"][:, j]] * 2
    tok = same[moe["rows"]].all(1)
    bound = TOPK * 2.0 ** -24 * s + carry + 1e-45
    err = np.abs(out.cpu().double().numpy() - ref)
    assert (err[tok] <= bound[tok]).all(), "combine outside its bound"
    assert tok.mean() >= 0.5
    say(f"  combine: {int(tok.sum())} of {T} tokens checked")
