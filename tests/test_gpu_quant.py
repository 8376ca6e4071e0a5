"""GPU parity of the two quantization calls against the CPU oracle: every code
byte and every scale byte must match exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bf16_bits, dev, oracle_requant_from_bf16, say, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def act_quant_both(mx, x_cpu, row_index=None, K=None, scale_rule="ocp"):
    """GPU and oracle act-quant of the same bf16 input; canary-guarded outputs."""
    xg = x_cpu.to(dev())
    M = x_cpu.shape[0] if row_index is None else row_index.shape[0]
    K = x_cpu.shape[1] if K is None else K
    gc = Guarded((M, K // 2), torch.uint8)
    gs = Guarded((M, K // 32), torch.uint8)
    ri = None if row_index is None else torch.from_numpy(row_index).to(dev())
    mx.mxfp4_quantize_act(xg, gc.view, gs.view, row_index=ri, K=K, scale_rule=scale_rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the output"
    oc, os_ = oracle.quantize_act(bf16_bits(x_cpu), K=K, row_index=row_index,
                                  scale_rule=scale_rule)
    return (u8(gc.view), u8(gs.view)), (oc, os_)


def assert_same(gpu, ref, what):
    (gc, gs), (oc, os_) = gpu, ref
    if not np.array_equal(gs, os_):
        i = tuple(np.argwhere(gs != os_)[0])
        raise AssertionError(f"{what}: scale byte mismatch at {i}: gpu {gs[i]} oracle {os_[i]}")
    if not np.array_equal(gc, oc):
        i = tuple(np.argwhere(gc != oc)[0])
        raise AssertionError(f"{what}: code byte mismatch at {i}: gpu {gc[i]:#04x} "
                             f"oracle {oc[i]:#04x}")


# ---- activation quantization --------------------------------------------------
def test_act_quant_tiny(mx):
    say("act_quant tiny [16,512] seed 2")
    x = synth.activations(16, 512, seed=2)
    g, o = act_quant_both(mx, x)
    assert_same(g, o, "tiny")


@pytest.mark.parametrize("M,K", [(1, 32), (37, 544), (5, 4096), (64, 4096)])
def test_act_quant_ragged_with_outliers(mx, M, K):
    say(f"act_quant M={M} K={K} with outliers")
    x = synth.activations(M, K, seed=12, outlier_seed=13)
    g, o = act_quant_both(mx, x)
    assert_same(g, o, f"M={M} K={K}")


def test_act_quant_gather_and_wide_rows(mx):
    say("act_quant gather, ldx > K")
    x = synth.activations(50, 1024, seed=3, outlier_seed=4)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 50, size=131).astype(np.int32)
    g, o = act_quant_both(mx, x, row_index=idx)
    assert_same(g, o, "gather")
    g, o = act_quant_both(mx, x, K=512)
    assert_same(g, o, "ldx>K")


def special_values_input():
    rng = np.random.default_rng(1)
    K = 256
    bits = (rng.integers(0, 2 ** 16, size=(64, K), dtype=np.uint32)).astype(np.uint16)
    # rows 0-7: random bit patterns (NaN, Inf, subnormals all appear)
    # rows 8-15: subnormal-only blocks; rows 16-23: zeros of both signs
    bits[8:16] = rng.integers(0, 0x80, size=(8, K)).astype(np.uint16) | \
        (rng.integers(0, 2, size=(8, K)).astype(np.uint16) << 15)
    bits[16:24] = rng.choice(np.array([0, 0x8000], dtype=np.uint16), size=(8, K))
    # rows 24-31: exact E2M1 tie points times powers of two
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], dtype=np.float32)
    for r in range(24, 32):
        v = rng.choice(ties, size=K) * np.float32(2.0 ** rng.integers(-20, 20))
        v[::32] = 4.0 * np.float32(2.0 ** rng.integers(-20, 20))
        v *= rng.choice(np.array([-1, 1], dtype=np.float32), size=K)
        bits[r] = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def test_act_quant_special_values(mx):
    say("act_quant NaN/Inf/subnormal/ties")
    g, o = act_quant_both(mx, special_values_input())
    assert_same(g, o, "specials")


def exhaustive_encode_input():
    """Every bf16 magnitude p (both signs) paired with every scale byte b it can
    meet: blocks whose element 0 is the anchor 4 * 2^(b-127) and whose other 31
    elements are bf16 values below 8 * 2^(b-127), so every block's amax lies in
    [4, 8) * 2^(b-127) and its scale byte is b."""
    vals = []
    for b in range(0, 253):
        anchor = (b + 2) << 7                            # bf16 bits of 2^(b-125)
        mags = np.arange(0, (b + 3) << 7, dtype=np.uint32)
        v = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        nblk = -(-v.size // 31)
        pad = np.zeros(nblk * 31 - v.size, dtype=np.uint16)
        body = np.concatenate([v, pad]).reshape(nblk, 31)
        head = np.full((nblk, 1), anchor, dtype=np.uint16)
        head[1::2] |= 0x8000
        vals.append(np.concatenate([head, body], axis=1))
    blocks = np.concatenate(vals)
    per_row = 128
    nrow = -(-blocks.shape[0] // per_row)
    pad = np.zeros((nrow * per_row - blocks.shape[0], 32), dtype=np.uint16)
    return np.concatenate([blocks, pad]).reshape(nrow, per_row * 32)


def test_act_quant_exhaustive_encoder(mx):
    say("act_quant exhaustive: all bf16 magnitudes x all scale bytes")
    bits = exhaustive_encode_input()
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    g, o = act_quant_both(mx, x)
    assert_same(g, o, "exhaustive")


@pytest.mark.parametrize("M,K", [(4096, 4096), (4096, 14336)])
def test_act_quant_prefill_full_size(mx, M, K):
    say(f"act_quant prefill [{M},{K}] full compare")
    x = synth.activations(M, K, seed=24 if K == 4096 else 25,
                          outlier_seed=26 if K == 4096 else 27)
    g, o = act_quant_both(mx, x)
    assert_same(g, o, f"prefill {M}x{K}")


def test_act_quant_deterministic(mx):
    x = synth.activations(256, 4096, seed=5).to(dev())
    c1, s1 = mx.mxfp4_quantize_act(x)
    c2, s2 = mx.mxfp4_quantize_act(x)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


# ---- NVFP4 -> MXFP4 requant ------------------------------------------------------
def requant_both(mx, codes, scales, g, bf16_intermediate=False, scale_rule="ocp"):
    T = 1 if codes.dim() == 2 else codes.shape[0]
    N, K = codes.shape[-2], codes.shape[-1] * 2
    shape_c = (T, N, K // 2) if codes.dim() == 3 else (N, K // 2)
    shape_s = (T, N, K // 32) if codes.dim() == 3 else (N, K // 32)
    gc = Guarded(shape_c, torch.uint8)
    gs = Guarded(shape_s, torch.uint8)
    mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()),
                                g.reshape(-1).to(torch.float32).to(dev()),
                                gc.view, gs.view, bf16_intermediate=bf16_intermediate,
                                scale_rule=scale_rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the destination"
    oc, os_ = oracle.requant(u8(codes), u8(scales), g.reshape(-1).numpy().astype(np.float32),
                             bf16_intermediate=bf16_intermediate, scale_rule=scale_rule)
    return (u8(gc.view), u8(gs.view)), (oc.reshape(shape_c), os_.reshape(shape_s))


@pytest.mark.parametrize("bf16_intermediate", [False, True])
def test_requant_tiny(mx, bf16_intermediate):
    say(f"requant tiny [256,512] seed 1 bf16={bf16_intermediate}")
    w = synth.bf16_normal((256, 512), 0.02, seed=1)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    gpu, ref = requant_both(mx, codes, scales, g, bf16_intermediate)
    assert_same(gpu, ref, "tiny requant")


@pytest.mark.parametrize("scale_rule", ["ocp", "uos"])
@pytest.mark.parametrize("bf16_intermediate", [False, True])
def test_requant_random_bytes_many_globals(mx, bf16_intermediate, scale_rule):
    """Arbitrary NVFP4 bytes (every E4M3 byte incl. NaN and subnormals) under
    global scales from 2^-140 to 2^120, so fp32 denormals, overflow to Inf and
    NaN blocks all occur; ragged K (17 MX blocks)."""
    say(f"requant random bytes T=12 N=37 K=544 bf16={bf16_intermediate} {scale_rule}")
    rng = np.random.default_rng(3)
    T, N, K = 12, 37, 544
    codes = torch.from_numpy(rng.integers(0, 256, size=(T, N, K // 2), dtype=np.uint8))
    scales = torch.from_numpy(rng.integers(0, 256, size=(T, N, K // 16), dtype=np.uint8))
    g = torch.tensor([2.0 ** e for e in (-140, -130, -126, -120, -60, -20, -7, 0, 3, 30, 100,
                                         120)], dtype=torch.float32)
    gpu, ref = requant_both(mx, codes, scales, g, bf16_intermediate, scale_rule)
    assert_same(gpu, ref, "random requant")
    g2 = torch.from_numpy(rng.uniform(1e-6, 1e-2, size=T).astype(np.float32))
    gpu, ref = requant_both(mx, codes, scales, g2, bf16_intermediate, scale_rule)
    assert_same(gpu, ref, "random requant, non-power-of-two g")


@pytest.mark.parametrize("scale_rule", ["ocp", "uos"])
@pytest.mark.parametrize("bf16_intermediate", [False, True])
def test_requant_limited_code_range(mx, bf16_intermediate, scale_rule):
    """Each NVFP4 block draws its codes from magnitudes 0..c_max with c_max
    itself random (so the block's largest code varies from 0 to 6), under
    E4M3 scales and global scales of both signs, including zero."""
    say(f"requant limited code range T=8 N=64 K=1024 bf16={bf16_intermediate} {scale_rule}")
    rng = np.random.default_rng(17)
    T, N, K = 8, 64, 1024
    cmax = rng.integers(0, 8, size=(T, N, K // 16, 1))
    mag = np.minimum(rng.integers(0, 8, size=(T, N, K // 16, 16)), cmax)
    nib = (mag | (rng.integers(0, 2, size=mag.shape) << 3)).reshape(T, N, K)
    codes = torch.from_numpy((nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8))
    sc = rng.integers(0, 0x7F, size=(T, N, K // 16)) | (rng.integers(0, 2, size=(T, N, K // 16)) << 7)
    scales = torch.from_numpy(sc.astype(np.uint8))
    g = torch.tensor([1e-3, -2.5e-4, 0.0, -0.0, 3.0e-41, -7.0, 1.0e30, 2.0 ** -149],
                     dtype=torch.float32)
    gpu, ref = requant_both(mx, codes, scales, g, bf16_intermediate, scale_rule)
    assert_same(gpu, ref, "limited code range")


def test_requant_decode_weight_full_size(mx):
    say("requant W [12288,4096] seed 11 full compare")
    w = synth.bf16_normal((12288, 4096), 0.02, seed=11)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    gpu, ref = requant_both(mx, codes, scales, g)
    assert_same(gpu, ref, "decode weight")


def test_requant_layer_shaped_batch(mx):
    """A batch of expert tensors of both MoE shapes, as the layerwise load
    passes them (one call per shape, T tensors each)."""
    for shape, seed in (((6, 2048, 4096), 41), ((6, 4096, 1024), 42)):
        say(f"requant layer batch {shape}")
        w = synth.bf16_normal(shape, 0.02, seed=seed)
        codes, scales, g = synth.nvfp4_from_bf16(w)
        gpu, ref = requant_both(mx, codes, scales, g)
        assert_same(gpu, ref, f"layer batch {shape}")


def test_requant_rerun_is_identical(mx):
    """Re-running a layer's requant into the same destination gives identical
    bytes (a reload can restart from any layer)."""
    w = synth.bf16_normal((3, 512, 1024), 0.02, seed=7).to(dev())
    codes, scales, g = synth.nvfp4_from_bf16(w)
    c1, s1 = mx.mxfp4_requant_from_nvfp4(codes, scales, g.reshape(-1))
    c2 = torch.full_like(c1, 0x5A)
    s2 = torch.full_like(s1, 0x5A)
    mx.mxfp4_requant_from_nvfp4(codes, scales, g.reshape(-1), c2, s2)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


@pytest.mark.parametrize("T,N,K,every", [(8, 256, 1024, (0, 2, 3, 7)), (1100, 16, 64, None)])
def test_requant_subset(mx, T, N, K, every):
    """The subset call converts exactly the listed tensors (bit-exact against
    the oracle) and leaves every other destination slot as it was.  1100 tiny
    tensors with 825 listed take two launches (512 indices a launch)."""
    say(f"requant subset T={T} N={N} K={K}")
    w = synth.bf16_normal((T, N, K), 0.02, seed=T + N)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    sel = list(every) if every else [t for t in range(T) if t % 4 != 1]
    gc = Guarded((T, N, K // 2), torch.uint8)
    gs = Guarded((T, N, K // 32), torch.uint8)
    gc.view.fill_(0x5A)
    gs.view.fill_(0xA5)
    mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(-1).to(dev()),
                                gc.view, gs.view, tensors=sel)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the destination"
    oc, os_ = oracle.requant(u8(codes), u8(scales), g.reshape(-1).numpy().astype(np.float32))
    oc, os_ = oc.reshape(T, N, K // 2), os_.reshape(T, N, K // 32)
    got_c, got_s = u8(gc.view), u8(gs.view)
    rest = [t for t in range(T) if t not in set(sel)]
    assert np.array_equal(got_c[sel], oc[sel]) and np.array_equal(got_s[sel], os_[sel])
    assert (got_c[rest] == 0x5A).all() and (got_s[rest] == 0xA5).all()
    with pytest.raises(mx.Mxfp4Error):
        mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(-1).to(dev()),
                                    gc.view, gs.view, tensors=[1, 0])


# ---- the UOS scale rule (Qmax = 7.25) ------------------------------------------------
def uos_act_inputs(case):
    if case == "outliers":
        return synth.activations(37, 544, seed=61, outlier_seed=62)
    if case == "specials":
        return special_values_input()
    if case == "exhaustive":
        # every bf16 magnitude is some block's amax, at every exponent: every
        # side of every 1.8125 boundary
        bits = exhaustive_encode_input()
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    raise ValueError(case)


@pytest.mark.parametrize("case", ["outliers", "specials", "exhaustive"])
def test_act_quant_uos(mx, case):
    """Act-quant under MXFP4_SCALE_UOS, bit-exact against the oracle's UOS rule;
    the inputs are chosen so that the two rules' scale bytes differ in places."""
    say(f"act_quant uos {case}")
    x = uos_act_inputs(case)
    g, o = act_quant_both(mx, x, scale_rule="uos")
    assert_same(g, o, f"uos {case}")
    _, ocp_scales = oracle.quantize_act(bf16_bits(x))
    assert (ocp_scales != o[1]).any(), "the input does not tell the rules apart"


def test_act_quant_uos_gather(mx):
    say("act_quant uos gather, ldx > K")
    x = synth.activations(50, 1024, seed=63, outlier_seed=64)
    idx = np.random.default_rng(5).integers(0, 50, size=77).astype(np.int32)
    g, o = act_quant_both(mx, x, row_index=idx, scale_rule="uos")
    assert_same(g, o, "uos gather")
    g, o = act_quant_both(mx, x, K=512, scale_rule="uos")
    assert_same(g, o, "uos ldx>K")


def test_act_quant_uos_prefill_full_size(mx):
    """The large-output (non-temporal store) form of the kernel under UOS."""
    say("act_quant uos prefill [4096,14336] full compare")
    x = synth.activations(4096, 14336, seed=65, outlier_seed=66)
    g, o = act_quant_both(mx, x, scale_rule="uos")
    assert_same(g, o, "uos prefill")


@pytest.mark.parametrize("bf16_intermediate", [False, True])
def test_requant_uos_tiny_and_subset(mx, bf16_intermediate):
    """Requant of a realistic weight under UOS, whole and as a subset call."""
    say(f"requant uos T=6 N=256 K=1024 bf16={bf16_intermediate}")
    w = synth.bf16_normal((6, 256, 1024), 0.02, seed=67)
    codes, scales, g = synth.nvfp4_from_bf16(w)
    gpu, ref = requant_both(mx, codes, scales, g, bf16_intermediate, "uos")
    assert_same(gpu, ref, "uos requant")
    _, ocp_scales = oracle.requant(u8(codes), u8(scales), g.reshape(-1).numpy(),
                                   bf16_intermediate=bf16_intermediate)
    assert (ocp_scales.reshape(ref[1].shape) != ref[1]).any()
    sel = [0, 3, 4]
    dc = torch.full((6, 256, 512), 0x5A, dtype=torch.uint8, device=dev())
    ds = torch.full((6, 256, 32), 0xA5, dtype=torch.uint8, device=dev())
    mx.mxfp4_requant_from_nvfp4(codes.to(dev()), scales.to(dev()), g.reshape(-1).to(dev()),
                                dc, ds, bf16_intermediate=bf16_intermediate, tensors=sel,
                                scale_rule="uos")
    got_c, got_s = u8(dc), u8(ds)
    assert np.array_equal(got_c[sel], ref[0][sel]) and np.array_equal(got_s[sel], ref[1][sel])
    assert (got_c[[1, 2, 5]] == 0x5A).all() and (got_s[[1, 2, 5]] == 0xA5).all()



# ---- Smooth pre-scale ------------------------------------------------------------
def smooth_vector(K, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.uniform(0.05, 4, K) * 2.0 ** rng.integers(-3, 4, K))
                            .astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("M,K,gather,rule", [(1, 32, False, "ocp"), (37, 544, False, "ocp"),
                                             (64, 4096, False, "uos"), (50, 1024, True, "ocp"),
                                             (4096, 4096, False, "ocp")])
def test_act_quant_smooth(mx, M, K, gather, rule):
    """Act-quant of bf16(x * smooth), bit-exact against the oracle (gather, both
    scale rules, the large-output form)."""
    say(f"act_quant smooth M={M} K={K} gather={gather} {rule}")
    x = synth.activations(M, K, seed=M + 1, outlier_seed=K + 1)
    sm = smooth_vector(K, seed=K)
    idx = np.random.default_rng(3).integers(0, M, size=2 * M).astype(np.int32) if gather else None
    Mo = M if idx is None else idx.size
    gc = Guarded((Mo, K // 2), torch.uint8)
    gs = Guarded((Mo, K // 32), torch.uint8)
    mx.mxfp4_quantize_act_smooth(x.to(dev()), sm.to(dev()), gc.view, gs.view,
                                 row_index=None if idx is None else torch.from_numpy(idx).to(dev()),
                                 scale_rule=rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact()
    oc, os_ = oracle.quantize_act_smooth(bf16_bits(x), bf16_bits(sm), row_index=idx,
                                         scale_rule=rule)
    assert_same((u8(gc.view), u8(gs.view)), (oc, os_), "smooth")


@pytest.mark.parametrize("M,K", [(5, 4096), (300, 1024)])
def test_act_quant_fp8_smooth(mx, M, K):
    say(f"act_quant_fp8 smooth M={M} K={K}")
    x = synth.activations(M, K, seed=M + 2, outlier_seed=K + 2)
    sm = smooth_vector(K, seed=K + 1)
    c, s = mx.mxfp8_quantize_act_smooth(x.to(dev()), sm.to(dev()))
    oc, os_ = oracle.quantize_act_fp8_smooth(bf16_bits(x), bf16_bits(sm))
    assert_same((u8(c), u8(s)), (oc, os_), "fp8 smooth")


def test_quantizers_rows_past_one_grid(mx):
    """More rows than one launch grid has (65535 workgroup rows of 2 rows
    each): the act-quant kernels walk the rest with a grid stride.  MXFP4 and
    MXFP8 act-quant of 131073 rows, bit for bit against the oracle."""
    M, K = 2 * 65535 + 3, 64
    say(f"act_quant rows past one grid M={M} K={K}")
    x = synth.activations(M, K, seed=41, outlier_seed=42)
    g, o = act_quant_both(mx, x)
    assert_same(g, o, "mxfp4 rows past one grid")
    c8, s8 = mx.mxfp8_quantize_act(x.to(dev()))
    torch.cuda.synchronize()
    oc8, os8 = oracle.quantize_act_fp8(bf16_bits(x))
    assert np.array_equal(u8(c8), oc8) and np.array_equal(u8(s8), os8)


@pytest.mark.parametrize("T,E,topk,K,rule", [(256, 16, 4, 512, "ocp"), (2048, 128, 8, 4096, "ocp"),
                                            (37, 5, 3, 96, "uos")])
def test_act_quant_scatter_equals_the_gather(mx, T, E, topk, K, rule):
    """Each token row quantized once and written to its routed rows: bit for
    bit the oracle's act-quant gathered by the routing's sorted order."""
    say(f"act_quant scatter T={T} E={E} top-{topk} K={K} {rule}")
    perm, _, rows, _ = synth.route_topk_full(T, E, topk, seed=T + K)
    x = synth.activations(T, K, seed=T, outlier_seed=K)
    R = T * topk
    gc = Guarded((R, K // 2), torch.uint8)
    gs = Guarded((R, K // 32), torch.uint8)
    mx.mxfp4_quantize_act_scatter(x.to(dev()), rows.to(dev()), gc.view, gs.view,
                                  scale_rule=rule)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the outputs"
    oc, os_ = oracle.quantize_act(bf16_bits(x), row_index=perm.numpy(), scale_rule=rule)
    assert_same((u8(gc.view), u8(gs.view)), (oc, os_), "scatter")


def test_act_quant_scatter_clamps_bad_rows(mx):
    """Destination rows outside [0, R) are clamped in the kernel: no write
    outside the outputs, and the rows named once by a valid entry are right."""
    say("act_quant scatter with bad destination rows")
    T, fan, K = 64, 2, 256
    R = T * fan
    x = synth.activations(T, K, seed=5)
    dest = np.arange(R, dtype=np.int32).reshape(T, fan)
    dest[3, 0], dest[9, 1], dest[20, 0] = -7, R + 100, 2 ** 31 - 1
    gc = Guarded((R, K // 2), torch.uint8)
    gs = Guarded((R, K // 32), torch.uint8)
    mx.mxfp4_quantize_act_scatter(x.to(dev()), torch.from_numpy(dest).to(dev()), gc.view,
                                  gs.view)
    torch.cuda.synchronize()
    assert gc.intact() and gs.intact(), "write outside the outputs"
    oc, os_ = oracle.quantize_act(bf16_bits(x))
    clamped = np.clip(dest.astype(np.int64), 0, R - 1)
    owners = np.bincount(clamped.ravel(), minlength=R)
    for t in range(T):
        for j in range(fan):
            d = clamped[t, j]
            if owners[d] == 1 and dest[t, j] == d:
                assert np.array_equal(u8(gc.view)[d], oc[t]) and np.array_equal(u8(gs.view)[d], os_[t])


_FIRST_CALLS_IN_CAPTURE = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import w4a4_mxfp4_gemm_amd as mx
d = torch.device("cuda:0")
g = torch.Generator().manual_seed(5)
x = torch.randn((4096, 4096), generator=g).to(torch.bfloat16).to(d)
nc = torch.randint(0, 256, (12288, 2048), dtype=torch.uint8, generator=g).to(d)
ns = torch.randint(0, 127, (12288, 256), dtype=torch.uint8, generator=g).to(d)
ng = torch.tensor([0.25], dtype=torch.float32).to(d)
c, s = torch.empty((4096, 2048), dtype=torch.uint8, device=d), torch.empty((4096, 128), dtype=torch.uint8, device=d)
oc, os_ = torch.empty((12288, 2048), dtype=torch.uint8, device=d), torch.empty((12288, 128), dtype=torch.uint8, device=d)
stream = torch.cuda.Stream()
graph = torch.cuda.CUDAGraph()
with torch.cuda.stream(stream):
    with torch.cuda.graph(graph, stream=stream):
        mx.mxfp4_quantize_act(x, codes=c, scales=s)
        mx.mxfp4_requant_from_nvfp4(nc, ns, ng, mx_codes=oc, mx_scales=os_)
for _ in range(3):
    c.zero_(); oc.zero_()
    graph.replay()
    torch.cuda.synchronize()
    ec, es = mx.mxfp4_quantize_act(x)
    rc, rs = mx.mxfp4_requant_from_nvfp4(nc, ns, ng)
    torch.cuda.synchronize()
    assert torch.equal(c, ec) and torch.equal(s, es), "act-quant replay"
    assert torch.equal(oc, rc) and torch.equal(os_, rs), "requant replay"
print("first calls inside capture ok", flush=True)
"""


def test_first_quantizer_calls_inside_graph_capture(mx, tmp_path):
    """The grid sizing of the act-quant and single-tensor requant queries the
    runtime once, at the first call.  In a fresh process whose first such
    calls are made during HIP graph capture, the calls still succeed, and
    every replay equals the eager result bit for bit (the shapes are the ones
    whose grids are resized: [4096, 4096] activations, one [12288, 4096]
    weight)."""
    import pathlib
    import subprocess
    import sys
    say("first act-quant / requant calls inside graph capture (fresh process)")
    script = tmp_path / "first_calls.py"
    script.write_text(_FIRST_CALLS_IN_CAPTURE)
    root = pathlib.Path(__file__).resolve().parent.parent
    r = subprocess.run([sys.executable, str(script), str(root)], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    assert "first calls inside capture ok" in r.stdout
