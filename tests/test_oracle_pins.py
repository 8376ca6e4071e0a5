"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- torch's fp8/bf16 decode tables, numpy's half-to-even ``rint``,
brute-force searches over whole domains, hand-worked fixtures under
``tests/golden/`` (each cites its source passage), exact round trips and
closed forms.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import parse_float, parse_sparse, read_table


def e2m1_table():
    rows = []
    for line in (__import__("conftest").GOLDEN / "e2m1_values.txt").read_text().splitlines():
        line = line.strip()
        if line and not line.startswith("#"):
            c, v = line.split()
            rows.append((int(c), float(v)))
    assert [c for c, _ in rows] == list(range(16))
    return np.array([v for _, v in rows], dtype=np.float64)


E2M1 = e2m1_table()


# ---- scalar decoders -----------------------------------------------------
def test_e2m1_decode_matches_value_table():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == E2M1[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, E2M1[c])
    assert max(oracle.e2m1_value(c) for c in range(16)) == 6.0


def test_e4m3_decode_matches_torch_all_bytes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = np.array([oracle.e4m3_value(i) for i in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert got[0x7E] == 448.0 and np.isnan(got[0x7F]) and got[0x01] == 2.0 ** -9


def test_e8m0_decode_matches_torch_all_bytes():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = np.array([oracle.e8m0_value(i) for i in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits[::7]])
    r = ref[::7]
    assert np.array_equal(np.isnan(r), np.isnan(got))
    ok = ~np.isnan(r)
    assert np.array_equal(r[ok], got[ok])


# ---- bf16 rounding -------------------------------------------------------
def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add every bf16 midpoint family explicitly: low 16 bits == 0x8000
    mids = (rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, mids.astype(np.uint32)])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_double_array(f.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_rounding_from_double_single_rounding():
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1.0078125: ties-to-even -> 1.0;
    # a hair above it must round up (no double rounding through fp32).
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_from_double(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_from_double(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    # largest finite bf16 and overflow
    assert oracle.bf16_from_double(float.fromhex("0x1.fep127")) == 0x7F7F
    assert oracle.bf16_from_double(float.fromhex("0x1.ffp127")) == 0x7F80
    assert oracle.bf16_from_double(2.0 ** -133) == 0x0001
    assert oracle.bf16_from_double(2.0 ** -134) == 0x0000       # tie -> even (0)
    assert oracle.bf16_from_double(-0.0) == 0x8000
    assert oracle.bf16_from_double(float("nan")) == 0x7FC0


# ---- E2M1 encoder ----------------------------------------------------------
def rint_reference(q):
    """E2M1 RNE written region by region with numpy's half-to-even rint:
    spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; saturate at 6."""
    a = np.abs(q)
    v = np.where(a < 2, np.rint(a * 2) / 2, np.where(a < 4, np.rint(a), 2 * np.rint(a / 2)))
    return np.minimum(v, 6.0)


def test_e2m1_encode_matches_regionwise_rint():
    rng = np.random.default_rng(7)
    grid = np.arange(0, 8.0, 1.0 / 64)           # every tie point and more
    rand = rng.uniform(-8, 8, size=50_000)
    q = np.concatenate([grid, -grid, rand, [6.0, 6.5, 7.0, 7.99, 1e-30, -1e-30]])
    codes = np.array([oracle.e2m1_encode(x) for x in q])
    assert np.array_equal(np.abs(E2M1[codes]), rint_reference(q))
    assert np.array_equal(codes >= 8, np.signbit(q))


def test_e2m1_encode_exhaustive_every_bf16_at_every_scale_byte():
    """The block quantizer's element step over all 65,536 bf16 patterns (NaN
    and Inf aside) at every finite scale byte 0..254: the code equals the
    region-wise rint of |v| / 2^(byte-127), computed here from torch's bf16
    decode, and carries v's sign bit (so negative values that round to zero
    give 0x8)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(v)
    bits, v = bits[finite], v[finite]
    sign = np.signbit(v)
    for byte in range(255):
        codes = oracle.e2m1_encode_bf16_at_scale(bits, byte)
        q = np.ldexp(v, 127 - byte)
        mag = rint_reference(q)
        got = E2M1[codes]
        bad = (np.abs(got) != mag) | ((codes >= 8) != sign)
        assert not bad.any(), (byte, int(bits[np.argmax(bad)]))


def test_e2m1_encode_roundtrip_all_codes():
    for c in range(16):
        assert oracle.e2m1_encode(E2M1[c]) == c


# ---- shared exponent ---------------------------------------------------------
def brute_force_byte(amax):
    """The unique E8M0 byte b with 4 <= amax / 2^(b-127) < 8 (the block max
    lands in E2M1's top binade), clamped to [0, 254] at the ends."""
    if amax < 4 * 2.0 ** -127:
        return 0
    for b in range(255):
        r = amax / 2.0 ** (b - 127)
        if 4 <= r < 8:
            return b
    raise AssertionError(amax)


def test_shared_exponent_bruteforce_all_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)         # positive finite bf16
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    for v in vals[::3]:
        assert oracle.shared_exponent(v) == brute_force_byte(v), v


def test_shared_exponent_fp32_sweep_and_specials():
    rng = np.random.default_rng(3)
    for e in range(-149, 128):
        for m in (1.0, 1.5, 1.999999, float(rng.uniform(1, 2))):
            v = float(np.float32(m * 2.0 ** e))
            if v > 0 and math.isfinite(v):
                assert oracle.shared_exponent(v) == brute_force_byte(v), v
    assert oracle.shared_exponent(0.0) == 0
    assert oracle.shared_exponent(float("nan")) == 255
    assert oracle.shared_exponent(float("inf")) == 255


# ---- hand-worked block fixtures -------------------------------------------------
def uos_exponent_by_fraction(a: float) -> int:
    """UOS exponent from the binary fraction of a (a > 0, finite): with
    a = f * 2^p, f in [1, 2), a / 2^(p-2) = 4f lies in [4, 8) and is at most
    7.25 exactly when f <= 1.8125; otherwise one exponent more is needed."""
    m, x = math.frexp(a)          # a = m * 2^x, m in [0.5, 1)
    f, p = 2.0 * m, x - 1
    e = p - 2 + (1 if f > 1.8125 else 0)
    return min(max(e, -127), 127) + 127


def test_uos_exponent_boundaries():
    """Setting 2 of the vLLM-Omni guide (Single-Scale Block Scaling): the
    exponent is the smallest e with amax <= 7.25 * 2^e; elements still
    saturate at 6."""
    for k in range(-120, 121, 7):
        b = 7.25 * 2.0 ** k
        assert oracle.shared_exponent(b, "uos") == k + 127
        assert oracle.shared_exponent(np.nextafter(b, np.inf), "uos") == k + 128
        assert oracle.shared_exponent(3.625 * 2.0 ** k, "uos") == k + 126
        assert oracle.shared_exponent(np.nextafter(3.625 * 2.0 ** k, np.inf), "uos") == k + 127
    assert oracle.shared_exponent(0.0, "uos") == 0
    assert oracle.shared_exponent(float("nan"), "uos") == 0xFF
    assert oracle.shared_exponent(float("inf"), "uos") == 0xFF
    assert oracle.shared_exponent(3.0e38, "uos") == 125 + 127    # 7.25 * 2^124 < 3e38 <= 7.25 * 2^125
    assert oracle.shared_exponent(1e-44, "uos") == 0             # clamped


def test_uos_exponent_matches_fraction_rule_and_ocp():
    """Random magnitudes over the whole fp32 range, subnormals included: the
    oracle's search agrees with the fraction rule.  Against the OCP exponent
    it is the same or one more, one more exactly when the fraction exceeds
    1.8125 (unless the lower clamp holds both at 0)."""
    rng = np.random.default_rng(7)
    bits = rng.integers(1, 0x7F800000, size=20000, dtype=np.int64).astype(np.uint32)
    vals = bits.view(np.float32).astype(np.float64)
    for a in vals:
        u = oracle.shared_exponent(a, "uos")
        o = oracle.shared_exponent(a)
        assert u == uos_exponent_by_fraction(a), a
        f = 2.0 * math.frexp(a)[0]
        assert u - o in (0, 1), a
        if o > 0:
            assert (u - o == 1) == (f > 1.8125), a


def test_uos_block_worked_example():
    """A block with amax 7.5: OCP picks 2^0 (7.5 saturates to 6); UOS picks 2^1,
    so 7.5 -> 3.75 -> 4 (code 6), -7.5 -> code 14, 1.0 -> 0.5 (code 1),
    0.375 -> 0.1875 -> 0 (code 0), 3.0 -> 1.5 (code 3); the rest 0."""
    v = np.zeros(32)
    v[:5] = [7.5, -7.5, 1.0, 0.375, 3.0]
    codes, s = oracle.mx_quantize_block(v, "uos")
    assert s == 128
    nib = [(codes[i // 2] >> (4 * (i % 2))) & 15 for i in range(32)]
    assert nib[:5] == [6, 14, 1, 0, 3] and all(n == 0 for n in nib[5:])
    codes_o, s_o = oracle.mx_quantize_block(v)
    nib_o = [(codes_o[i // 2] >> (4 * (i % 2))) & 15 for i in range(32)]
    assert s_o == 127 and nib_o[:5] == [7, 15, 2, 1, 5]     # 6, -6, 1, 0.5 (0.375 rounds up), 3


def test_uos_act_quant_and_requant_use_the_rule():
    """The row operations under "uos" equal per-block quantization under the
    same rule (act-quant of bf16 rows; requant of the NVFP4 values)."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 128)) * np.array([1e-3, 1.0, 40.0])[:, None]
    bits = oracle.bf16_from_double_array(x.ravel()).reshape(3, 128)
    c, s = oracle.quantize_act(bits, scale_rule="uos")
    for r in range(3):
        for j in range(4):
            vals = np.array([oracle.bf16_value(int(b)) for b in bits[r, 32 * j:32 * j + 32]])
            cb, sb = oracle.mx_quantize_block(vals, "uos")
            assert sb == s[r, j] and np.array_equal(cb, c[r, 16 * j:16 * j + 16])
    codes = rng.integers(0, 256, size=(8, 64), dtype=np.uint8)
    scales = rng.integers(0x20, 0x60, size=(8, 8), dtype=np.uint8)
    g = np.float32(0.0123)
    mc, ms = oracle.requant(codes, scales, g, scale_rule="uos")
    deq = oracle.nvfp4_dequant(codes, scales, g)
    for r in range(8):
        for j in range(4):
            cb, sb = oracle.mx_quantize_block(deq[r, 32 * j:32 * j + 32].astype(np.float64), "uos")
            assert sb == ms[r, j] and np.array_equal(cb, mc[r, 16 * j:16 * j + 16])


@pytest.mark.parametrize("row", read_table("mx_block_examples.txt"), ids=lambda r: r[0])
def test_mx_block_examples(row):
    name, inputs, byte, codes = row
    v = np.zeros(32)
    for i, x in parse_sparse(inputs, parse_float).items():
        v[i] = x
    want = np.zeros(32, dtype=np.int64)
    for i, c in parse_sparse(codes, int).items():
        want[i] = c
    got_codes, got_byte = oracle.mx_quantize_block(v)
    assert got_byte == int(byte)
    unpacked = np.empty(32, dtype=np.int64)
    unpacked[0::2] = got_codes & 15
    unpacked[1::2] = got_codes >> 4
    assert np.array_equal(unpacked, want)


@pytest.mark.parametrize("row", read_table("requant_examples.txt"), ids=lambda r: r[0])
def test_requant_examples(row):
    name, gbits, s0, s1, codes, bf16, byte, mx = row
    g = np.array([int(gbits, 16)], dtype=np.uint32).view(np.float32)
    nib = np.zeros(32, dtype=np.uint8)
    for i, c in parse_sparse(codes, int).items():
        nib[i] = c
    packed = (nib[0::2] | (nib[1::2] << 4)).reshape(1, 16)
    scales = np.array([[int(s0, 16), int(s1, 16)]], dtype=np.uint8)
    out_codes, out_scales = oracle.requant(packed, scales, g, bf16_intermediate=bool(int(bf16)))
    assert out_scales.shape == (1, 1) and int(out_scales[0, 0]) == int(byte)
    want = np.zeros(32, dtype=np.uint8)
    for i, c in parse_sparse(mx, int).items():
        want[i] = c
    got = np.empty(32, dtype=np.uint8)
    got[0::2] = out_codes[0] & 15
    got[1::2] = out_codes[0] >> 4
    assert np.array_equal(got, want)


# ---- round trips and exactness ---------------------------------------------------
def canonical_blocks(rows, K, seed, lo=2, hi=252):
    """MXFP4 tensors whose blocks re-quantize to themselves: each non-zero block's
    largest |code| is 6 or 7 (4 or 6), scale bytes keep values normal in bf16;
    all-zero blocks carry byte 0."""
    rng = np.random.default_rng(seed)
    nib = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    nb = K // 32
    blk = nib.reshape(rows, nb, 32)
    pos = rng.integers(0, 32, size=(rows, nb))
    top = rng.choice(np.array([6, 7, 14, 15], dtype=np.uint8), size=(rows, nb))
    np.put_along_axis(blk, pos[..., None], top[..., None], axis=2)
    scales = rng.integers(lo, hi + 1, size=(rows, nb), dtype=np.uint8)
    zero = rng.random((rows, nb)) < 0.05
    blk[zero] = rng.choice(np.array([0, 8], dtype=np.uint8), size=(int(zero.sum()), 32))
    scales[zero] = 0
    nib = blk.reshape(rows, K)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return nib, packed, scales


def dequant_to_bf16_bits(nib, scales):
    vals = E2M1[nib] * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    f = vals.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), vals)          # exact
    b = f.view(np.uint32)
    assert not (b & 0xFFFF).any()                             # exact in bf16
    return (b >> 16).astype(np.uint16)


def test_quantize_act_roundtrip_canonical():
    nib, packed, scales = canonical_blocks(64, 1024, seed=11)
    x = dequant_to_bf16_bits(nib, scales)
    codes, sc = oracle.quantize_act(x)
    assert np.array_equal(sc, scales)
    assert np.array_equal(codes, packed)


def test_quantize_act_gather_equals_quantize_then_index():
    rng = np.random.default_rng(4)
    x = torch.randn(40, 256, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    idx = rng.integers(0, 40, size=77).astype(np.int32)
    c_all, s_all = oracle.quantize_act(xb)
    c_g, s_g = oracle.quantize_act(xb, row_index=idx)
    assert np.array_equal(c_g, c_all[idx]) and np.array_equal(s_g, s_all[idx])
    # ldx > K: only the first K columns are read
    wide = np.concatenate([xb, np.full((40, 64), 0x7FC0, dtype=np.uint16)], axis=1)
    c_w, s_w = oracle.quantize_act(wide, K=256)
    assert np.array_equal(c_w, c_all) and np.array_equal(s_w, s_all)


def test_requant_exact_on_representable_input():
    rng = np.random.default_rng(21)
    N, K = 48, 512
    nib, packed, _ = canonical_blocks(N, K, seed=22)
    # both 16-halves of a 32-block share one power-of-two E4M3 scale 2^p
    p = rng.integers(-9, 9, size=(N, K // 32))
    def e4m3_pow2(pp):
        if pp >= -6:
            return (pp + 7) << 3
        return {-7: 0x04, -8: 0x02, -9: 0x01}[pp]
    e4 = np.vectorize(e4m3_pow2)(p).astype(np.uint8)
    nv_scales = np.repeat(e4, 2, axis=1)
    for q in (-3, 0, 5):
        g = np.float32(2.0 ** q)
        codes, scales = oracle.requant(packed, nv_scales, g)
        blk_nonzero = (nib.reshape(N, K // 32, 32) & 7).any(axis=2)
        want_scales = np.where(blk_nonzero, p + q + 127, 0)
        assert np.array_equal(scales, want_scales.astype(np.uint8))
        assert np.array_equal(codes, packed)       # signed zeros included


def test_nvfp4_dequant_matches_numpy_fp32():
    rng = np.random.default_rng(8)
    N, K = 16, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)   # finite, >= 0
    g = np.float32(rng.uniform(1e-5, 3.0))
    nib = np.empty((N, K), dtype=np.uint8)
    nib[:, 0::2] = codes & 15
    nib[:, 1::2] = codes >> 4
    s = torch.from_numpy(scales).view(torch.float8_e4m3fn).float().numpy()
    p = (E2M1[nib].astype(np.float32) * np.repeat(s, 16, axis=1)).astype(np.float32)
    want = p * g                                              # numpy IEEE fp32
    got = oracle.nvfp4_dequant(codes, scales, g)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    got_b = oracle.nvfp4_dequant(codes, scales, g, bf16_intermediate=True)
    want_b = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got_b.view(np.uint32), want_b.view(np.uint32))


def test_requant_bf16_path_equals_act_quant_of_dequant():
    """With the bf16 intermediate, requant == act-quant of the dequantized tensor."""
    rng = np.random.default_rng(12)
    N, K = 32, 512
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    g = np.float32(0.000123)
    deq = oracle.nvfp4_dequant(codes, scales, g, bf16_intermediate=True)
    xb = (deq.view(np.uint32) >> 16).astype(np.uint16)
    c1, s1 = oracle.requant(codes, scales, g, bf16_intermediate=True)
    c2, s2 = oracle.quantize_act(xb)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_requant_fp32_path_equals_blockwise_quantization():
    rng = np.random.default_rng(13)
    N, K = 6, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    g = np.float32(0.37)
    deq = oracle.nvfp4_dequant(codes, scales, g)
    c1, s1 = oracle.requant(codes, scales, g)
    for n in range(N):
        for j in range(K // 32):
            cb, sb = oracle.mx_quantize_block(deq[n, 32 * j:32 * j + 32].astype(np.float64))
            assert sb == s1[n, j]
            assert np.array_equal(cb, c1[n, 16 * j:16 * j + 16])


# ---- GEMM ------------------------------------------------------------------------
def dequant(codes, scales):
    K = codes.shape[-1] * 2
    nib = np.empty(codes.shape[:-1] + (K,), dtype=np.uint8)
    nib[..., 0::2] = codes & 15
    nib[..., 1::2] = codes >> 4
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return E2M1[nib] * np.repeat(sc, 32, axis=-1)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (7, 5, 64), (33, 17, 544), (16, 256, 512)])
def test_gemm_matches_numpy_fp64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    a = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    sa = rng.integers(110, 140, size=(M, K // 32), dtype=np.uint8)
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sb = rng.integers(110, 140, size=(N, K // 32), dtype=np.uint8)
    y, s = oracle.gemm(a, sa, b, sb)
    A, B = dequant(a, sa), dequant(b, sb)
    ref = A @ B.T
    S = np.abs(A) @ np.abs(B).T
    assert np.all(np.abs(y - ref) <= 1e-12 * S + 1e-300)
    assert np.allclose(s, S, rtol=1e-12, atol=0)


def test_gemm_unit_scales_is_integer_product():
    rng = np.random.default_rng(1)
    M, N, K = 9, 11, 320
    a = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ones_a = np.full((M, K // 32), 127, dtype=np.uint8)
    ones_b = np.full((N, K // 32), 127, dtype=np.uint8)
    y, _ = oracle.gemm(a, ones_a, b, ones_b)
    def twice(c):          # 2 * e2m1 value as an integer, from the table fixture
        nib = np.empty((c.shape[0], K), dtype=np.uint8)
        nib[:, 0::2] = c & 15
        nib[:, 1::2] = c >> 4
        return (2 * E2M1[nib]).astype(np.int64)
    ref = twice(a) @ twice(b).T
    assert np.array_equal(y * 4, ref.astype(np.float64))


def test_gemm_one_hot_reproduces_dequantized_column():
    rng = np.random.default_rng(2)
    N, K = 13, 96
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sb = rng.integers(100, 150, size=(N, K // 32), dtype=np.uint8)
    B = dequant(b, sb)
    for k0 in (0, 1, 31, 32, 95):
        a = np.zeros((1, K // 2), dtype=np.uint8)
        a[0, k0 // 2] = 2 << (4 * (k0 % 2))      # code 2 = 1.0
        sa = np.full((1, K // 32), 127, dtype=np.uint8)
        y, s = oracle.gemm(a, sa, b, sb)
        assert np.array_equal(y[0], B[:, k0])
        assert np.array_equal(s[0], np.abs(B[:, k0]))


def test_gemm_nan_scale_propagates():
    a = np.zeros((1, 16), dtype=np.uint8)
    sa = np.array([[255]], dtype=np.uint8)
    b = np.zeros((2, 16), dtype=np.uint8)
    sb = np.full((2, 1), 127, dtype=np.uint8)
    y, _ = oracle.gemm(a, sa, b, sb)
    assert np.isnan(y).all()


def test_gemm_at_matches_full():
    rng = np.random.default_rng(6)
    M, N, K = 20, 30, 128
    a = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    sa = rng.integers(120, 134, size=(M, K // 32), dtype=np.uint8)
    b = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sb = rng.integers(120, 134, size=(N, K // 32), dtype=np.uint8)
    y, s = oracle.gemm(a, sa, b, sb)
    pm = rng.integers(0, M, size=50)
    pn = rng.integers(0, N, size=50)
    yp, sp = oracle.gemm_at(a, sa, b, sb, pm, pn)
    assert np.array_equal(yp, y[pm, pn]) and np.array_equal(sp, s[pm, pn])


def test_grouped_gemm_equals_per_expert_gemm():
    rng = np.random.default_rng(10)
    E, N, K = 5, 24, 96
    counts = np.array([3, 0, 7, 1, 0])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    a = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    sa = rng.integers(120, 134, size=(M, K // 32), dtype=np.uint8)
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sb = rng.integers(120, 134, size=(E, N, K // 32), dtype=np.uint8)
    y, s = oracle.grouped_gemm(a, sa, b, sb, offsets)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ye, se = oracle.gemm(a[r0:r1], sa[r0:r1], b[e], sb[e])
            assert np.array_equal(y[r0:r1], ye) and np.array_equal(s[r0:r1], se)


# ---- the tolerance rules themselves ----------------------------------------------
def test_tolerance_rules_accept_one_ulp_reject_two():
    rng = np.random.default_rng(0)
    y = rng.standard_normal(2000) * 10.0 ** rng.integers(-5, 5, 2000)
    ref = oracle.bf16_from_double_array(y)
    def step(bits, k):
        b = bits.astype(np.int64)
        mag = (b & 0x7FFF) + k
        return ((b & 0x8000) | mag).astype(np.uint16)
    assert oracle.gemm_bf16_ok(ref, y).all()
    assert oracle.gemm_bf16_ok(step(ref, 1), y).all()
    assert not oracle.gemm_bf16_ok(step(ref, 2), y).any()
    assert oracle.gemm_bf16_ok(np.array([0x8000], dtype=np.uint16), np.array([0.0])).all()
    s = np.abs(y) * 3
    assert oracle.gemm_fp32_ok(y + 0.9e-5 * s, y, s).all()
    assert not oracle.gemm_fp32_ok(y + 1.1e-5 * s, y, s).any()
    assert oracle.gemm_fp32_ok(np.array([0.0]), np.array([0.0]), np.array([0.0])).all()
    assert not oracle.gemm_fp32_ok(np.array([1e-30]), np.array([0.0]), np.array([0.0])).any()


# ---- R10: expert activation (silu(gate) * up) before the down projection ------
def bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_silu_mul_against_library_sigmoid():
    """Random bf16 gate/up values: the oracle's fp32 evaluation lies within a
    few fp32 ulps of g * expit(g) * u, with scipy's logistic function as the
    independent sigmoid (a wrong sign in the exponent, a dropped term or the
    gate and up roles swapped are off by far more)."""
    from scipy.special import expit
    rng = np.random.default_rng(101)
    g = torch.from_numpy(rng.uniform(-30, 30, 4000).astype(np.float32)).to(torch.bfloat16)
    u = torch.from_numpy(rng.normal(0, 2, 4000).astype(np.float32)).to(torch.bfloat16)
    g64, u64 = g.double().numpy(), u.double().numpy()
    want = g64 * expit(g64) * u64
    got = np.array([oracle.silu_mul_f32(a, b) for a, b in zip(g64, u64)])
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert (np.abs(got - want) <= 4 * ulp + 1e-44).all()


def test_silu_mul_closed_forms():
    f = oracle.silu_mul_f32
    # silu(g) - silu(-g) = g
    for g in (0.5, 1.0, 2.75, 7.0, 12.5):
        assert abs((f(g, 1.0) - f(-g, 1.0)) - g) <= 4 * np.spacing(np.float32(g))
    assert f(0.0, 3.0) == 0.0
    for g in (17.0, 20.0, 60.0, 1e30):     # e^-g below half an ulp of 1: silu(g) = g
        for u in (0.3, -1.7, 2.0 ** -100):
            assert f(g, u) == float(np.float32(g) * np.float32(u))
    assert f(-100.0, 1.0) == 0.0 and np.signbit(f(-100.0, 1.0))
    assert f(float("inf"), 1.0) == float("inf")
    assert np.isnan(f(float("-inf"), 1.0)) and np.isnan(f(float("nan"), 1.0))


def test_silu_mul_quantize_linear_region_is_act_quant():
    """Where every gate is >= 17 the activation is exactly fl32(g * u): the
    composition must equal the act-quant of those products rounded to bf16
    (rounded here by torch), for both scale rules; the gate and up halves are
    told apart because swapping them leaves that region."""
    rng = np.random.default_rng(102)
    M, I = 6, 96
    g = torch.from_numpy(rng.uniform(17, 400, (M, I)).astype(np.float32)).to(torch.bfloat16)
    u = torch.from_numpy(rng.normal(0, 0.05, (M, I)).astype(np.float32)).to(torch.bfloat16)
    gu = bf16_bits(torch.cat([g, u], dim=1))
    prod = (g.float() * u.float()).to(torch.bfloat16)
    for rule in ("ocp", "uos"):
        want = oracle.quantize_act(bf16_bits(prod), scale_rule=rule)
        got = oracle.silu_mul_quantize(gu, scale_rule=rule)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    hb, hf = oracle.silu_mul(gu)
    assert np.array_equal(hb, bf16_bits(prod))
    assert np.array_equal(hf, (g.float() * u.float()).numpy())


@pytest.mark.parametrize("row", read_table("silu_mul_examples.txt"), ids=lambda r: r[0])
def test_silu_mul_examples(row):
    name, gate, up, hbits, byte, codes = row
    gu = np.zeros((1, 64), dtype=np.float32)
    for i, x in parse_sparse(gate, parse_float).items():
        gu[0, i] = x
    for i, x in parse_sparse(up, parse_float).items():
        gu[0, 32 + i] = x
    bits = bf16_bits(torch.from_numpy(gu).to(torch.bfloat16))
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
                          .numpy(), gu), "fixture inputs must be bf16 values"
    hb, _ = oracle.silu_mul(bits)
    want_h = np.zeros(32, dtype=np.uint16)
    for i, b in parse_sparse(hbits, lambda t: int(t, 16)).items():
        want_h[i] = b
    assert np.array_equal(hb[0], want_h)
    c, s = oracle.silu_mul_quantize(bits)
    assert int(s[0, 0]) == int(byte)
    want = np.zeros(32, dtype=np.int64)
    for i, k in parse_sparse(codes, int).items():
        want[i] = k
    got = np.empty(32, dtype=np.int64)
    got[0::2], got[1::2] = c[0] & 15, c[0] >> 4
    assert np.array_equal(got, want)


# ---- R5 through BLAS, for full-size parity ----------------------------------------
@pytest.mark.parametrize("M,N,K,lo,hi", [(7, 9, 64, 100, 150), (33, 40, 1024, 0, 254),
                                         (64, 17, 4096, 117, 137)])
def test_gemm_blas_matches_the_exact_gemm(M, N, K, lo, hi):
    """The fp64 dequantize + numpy matmul form of the GEMM agrees with the
    exact integer-sum oracle to within K * 2^-52 * s, over random codes and
    scale bytes (the whole E8M0 range in one case), whole or in row chunks."""
    rng = np.random.default_rng(M + N + K)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(lo, hi + 1, (M, K // 32), dtype=np.uint8)
    bs = rng.integers(lo, hi + 1, (N, K // 32), dtype=np.uint8)
    y, s = oracle.gemm(ac, as_, bc, bs)
    yb, sb = oracle.gemm_blas(ac, as_, bc, bs)
    fin = np.isfinite(s)
    assert np.array_equal(fin, np.isfinite(sb))
    assert (np.abs(yb - y)[fin] <= K * 2.0 ** -52 * s[fin]).all()
    assert (np.abs(sb - s)[fin] <= K * 2.0 ** -52 * s[fin]).all()
    yc, _ = oracle.gemm_blas(ac, as_, bc, bs, row_chunk=5)    # BLAS may reorder the sums
    assert (np.abs(yc - y)[fin] <= K * 2.0 ** -52 * s[fin]).all()


def test_gemm_blas_nan_scale_and_decode():
    """Scale byte 0xFF makes its row's results NaN; the dequantized operand is
    the E2M1 value times 2^(byte-127), nibble order R1."""
    ac = np.array([[0x21, 0x00] * 8, [0x7F, 0xF7] * 8], dtype=np.uint8)
    v = oracle.mxfp4_dequant_f64(ac, np.array([[127], [130]], dtype=np.uint8))
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0 and v[0, 2] == 0.0
    assert v[1, 0] == -6 * 8 and v[1, 1] == 6 * 8 and v[1, 2] == 6 * 8 and v[1, 3] == -6 * 8
    bc = np.full((3, 16), 0x22, dtype=np.uint8)
    y, _ = oracle.gemm_blas(ac, np.array([[127], [255]], dtype=np.uint8), bc,
                            np.full((3, 1), 127, dtype=np.uint8))
    assert np.isfinite(y[0]).all() and np.isnan(y[1]).all()
    assert y[0, 0] == 8 * (0.5 * 1 + 1 * 1)


# ---- R11: top-k combine --------------------------------------------------------
def combine_case(seed, T=12, topk=8, H=40, R=None):
    rng = np.random.default_rng(seed)
    R = R or T * topk
    y = torch.from_numpy(rng.normal(0, 1, (R, H)).astype(np.float32)).to(torch.bfloat16)
    rows = rng.permutation(R)[:T * topk].reshape(T, topk).astype(np.int32)
    w = rng.dirichlet(np.ones(topk), size=T).astype(np.float32)
    return bf16_bits(y), y.double().numpy(), rows, w


def test_combine_one_hot_weights_select_rows():
    bits, y, rows, w = combine_case(103)
    w1 = np.zeros_like(w)
    w1[np.arange(w.shape[0]), 3] = 1.0
    out, s = oracle.moe_combine(bits, rows, w1)
    assert np.array_equal(out, y[rows[:, 3]]) and np.array_equal(s, np.abs(out))


def test_combine_per_token_weights_and_rows():
    """Each token has its own weights and rows: token t one-hot at column
    t mod topk returns its own routed row there, and distinct random weights
    give numpy's fp64 weighted sum of the gathered rows.  A weight read from
    the wrong token (w[j] in place of w[t*topk+j]) or a row from the wrong
    token fails both."""
    T, topk, H = 24, 8, 40
    bits, y, rows, w = combine_case(106, T=T, topk=topk, H=H)
    w1 = np.zeros_like(w)
    col = np.arange(T) % topk
    w1[np.arange(T), col] = 1.0
    out, _ = oracle.moe_combine(bits, rows, w1)
    assert np.array_equal(out, y[rows[np.arange(T), col]])
    assert len({tuple(r) for r in w.round(6)}) == T         # the weights differ per token
    out, s = oracle.moe_combine(bits, rows, w)
    ref = np.einsum("tj,tjn->tn", w.astype(np.float64), y[rows])
    assert np.allclose(out, ref, rtol=0, atol=4e-16 * s.max())
    assert not np.allclose(out[1:], ref[0], rtol=0, atol=1e-6)


def test_combine_equal_rows_and_power_of_two_weights():
    """k copies of one row with weights 1/k (k a power of two) return the row
    exactly; weights w and 2w give exactly twice the result."""
    bits, y, rows, w = combine_case(104, topk=8)
    rows_same = np.repeat(rows[:, :1], 8, axis=1)
    out, _ = oracle.moe_combine(bits, rows_same, np.full(w.shape, 0.125, np.float32))
    assert np.array_equal(out, y[rows[:, 0]])
    a, _ = oracle.moe_combine(bits, rows, w)
    b, _ = oracle.moe_combine(bits, rows, 2 * w)
    assert np.array_equal(b, 2 * a)


def test_combine_order_and_linearity_invariants():
    """Permuting a token's k (row, weight) pairs changes nothing beyond fp64
    rounding; the result is linear in the weights; s bounds |out| and equals
    it when every product is non-negative."""
    bits, y, rows, w = combine_case(105)
    out, s = oracle.moe_combine(bits, rows, w)
    perm = np.random.default_rng(6).permutation(rows.shape[1])
    out2, s2 = oracle.moe_combine(bits, rows[:, perm], w[:, perm])
    assert np.allclose(out2, out, rtol=0, atol=1e-15 * s.max())
    assert np.allclose(s2, s, rtol=1e-15, atol=0)
    half = (w / 2).astype(np.float32)
    p, _ = oracle.moe_combine(bits, rows, half)
    q, _ = oracle.moe_combine(bits, rows, w - half)
    assert np.allclose(p + q, out, rtol=0, atol=1e-15 * s.max())
    assert (np.abs(out) <= s).all()
    pos_bits = bits & np.uint16(0x7FFF)
    o3, s3 = oracle.moe_combine(pos_bits, rows, w)
    assert np.array_equal(o3, s3)


# ---- R12: row bias ------------------------------------------------------------------
def test_row_bias_closed_forms():
    """All activation codes zero: the result is the bias itself, on every row;
    a zero bias changes nothing; the bias is one value per weight row (output
    column), not per activation row; s grows by |bias|."""
    rng = np.random.default_rng(120)
    M, N, K = 5, 24, 64
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bs = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    ac = np.zeros((M, K // 2), dtype=np.uint8)
    as_ = np.full((M, K // 32), 127, dtype=np.uint8)
    bias = bf16_bits(torch.from_numpy(rng.normal(0, 3, N).astype(np.float32)).to(torch.bfloat16))
    bval = torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).double().numpy()
    y0, s0 = oracle.gemm(ac, as_, bc, bs)
    y, s = oracle.add_row_bias(y0, s0, bias)
    assert np.array_equal(y, np.broadcast_to(bval, (M, N)))
    assert np.array_equal(s, np.broadcast_to(np.abs(bval), (M, N)))
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    y1, s1 = oracle.gemm(ac, as_, bc, bs)
    yz, sz = oracle.add_row_bias(y1, s1, np.zeros(N, dtype=np.uint16))
    assert np.array_equal(yz, y1) and np.array_equal(sz, s1)
    yb, _ = oracle.add_row_bias(y1, s1, bias)
    # scales 127 on A and B bytes in [120, 135): every term and sum is exact
    assert np.array_equal(yb - y1, np.broadcast_to(bval, (M, N)))


# ---- R13-R15: W4A8 (MXFP8 activations x MXFP4 weights) ---------------------------------
def all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    return v[torch.isfinite(v)]


def test_e4m3_encode_matches_torch_cast_and_saturates():
    """Every finite bf16 value q with |q| <= 448 encodes to torch's
    float32 -> float8_e4m3fn cast (round to nearest even, a library routine);
    448 < |q| < 512 saturates to 0x7E with the sign kept."""
    v = all_bf16_values()
    inside = v[v.abs() <= 448]
    want = inside.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(q) for q in inside.double().numpy()], dtype=np.uint8)
    assert np.array_equal(got, want)
    over = v[(v.abs() > 448) & (v.abs() < 512)].double().numpy()
    assert over.size > 0
    for q in over:
        assert oracle.e4m3_encode(q) == (0xFE if q < 0 else 0x7E)


def test_shared_exponent_fp8_brute_force():
    """The byte is the unique b with 256 <= amax / 2^(b-127) < 512 (a block's
    amax lands in E4M3's top binade), clamped to [0, 254]; NaN/Inf -> 0xFF."""
    v = all_bf16_values().double().numpy()
    v = np.unique(np.abs(v[v != 0]))
    rng = np.random.default_rng(130)
    v = np.concatenate([v, rng.uniform(1, 2, 200) * 2.0 ** rng.integers(-140, 128, 200)])
    for a in v:
        b = oracle.shared_exponent_fp8(a)
        fits = [c for c in range(255) if 256 <= a / 2.0 ** (c - 127) < 512]
        if fits:
            assert b == fits[0]
        else:
            assert b == (0 if a < 2.0 ** -119 else 254)
    assert oracle.shared_exponent_fp8(0.0) == 0
    assert oracle.shared_exponent_fp8(float("nan")) == 0xFF
    assert oracle.shared_exponent_fp8(float("inf")) == 0xFF


@pytest.mark.parametrize("row", read_table("mx8_block_examples.txt"), ids=lambda r: r[0])
def test_mx8_block_examples(row):
    name, inputs, byte, codes = row
    v = np.zeros(32)
    for i, x in parse_sparse(inputs, parse_float).items():
        v[i] = x
    want = np.zeros(32, dtype=np.uint8)
    for i, c in parse_sparse(codes, lambda t: int(t, 16)).items():
        want[i] = c
    got, b = oracle.mx8_quantize_block(v)
    assert b == int(byte) and np.array_equal(got, want)


def test_quantize_act_fp8_round_trip_of_canonical_mxfp8():
    """A canonical MXFP8 tensor (every block's largest |code| in E4M3's top
    binade, scale bytes 20..230) dequantized to bf16 (exact: 4 significant
    bits) quantizes back to the same codes and bytes; a gather picks rows."""
    rng = np.random.default_rng(131)
    M, K = 12, 256
    nb = K // 32
    mag = rng.integers(0, 0x7F, (M, nb, 32))
    mag[:, :, 0] = rng.integers(0x78, 0x7F, (M, nb))          # top binade: exponent 15
    codes = (mag | (rng.integers(0, 2, mag.shape) << 7)).astype(np.uint8).reshape(M, K)
    scales = rng.integers(20, 231, (M, nb)).astype(np.uint8)
    vals = np.array([oracle.e4m3_value(int(c)) for c in codes.reshape(-1)]).reshape(M, nb, 32)
    vals = vals * (2.0 ** (scales.astype(np.float64) - 127))[:, :, None]
    x = torch.from_numpy(vals.reshape(M, K)).to(torch.bfloat16)
    assert np.array_equal(x.double().numpy(), vals.reshape(M, K)), "bf16 must hold them exactly"
    c, s = oracle.quantize_act_fp8(bf16_bits(x))
    assert np.array_equal(s, scales)
    # -0 codes come back as 0x80, +0 as 0x00: compare as values and signs
    assert np.array_equal(c, codes)
    idx = np.array([3, 3, 0, 11], dtype=np.int32)
    cg, sg = oracle.quantize_act_fp8(bf16_bits(x), row_index=idx)
    assert np.array_equal(cg, codes[idx]) and np.array_equal(sg, scales[idx])


def test_gemm_w4a8_against_numpy_and_closed_form():
    """Against an fp64 numpy matmul of operands dequantized by other means
    (torch's float8_e4m3fn decode, the E2M1 golden table); and A = 1.0
    everywhere (code 0x38, scale 127) gives B's row sums."""
    rng = np.random.default_rng(132)
    M, N, K = 7, 9, 96
    ac = rng.integers(0, 0x7F, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)
    ac = ac.astype(np.uint8)
    as_ = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bs = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    a = torch.from_numpy(ac).view(torch.float8_e4m3fn).double().numpy()
    a = a * np.repeat(2.0 ** (as_.astype(np.float64) - 127), 32, axis=1)
    nib = np.stack([bc & 15, bc >> 4], axis=-1).reshape(N, K)
    b = E2M1[nib] * np.repeat(2.0 ** (bs.astype(np.float64) - 127), 32, axis=1)
    y, s = oracle.gemm_w4a8(ac, as_, bc, bs)
    assert np.allclose(y, a @ b.T, rtol=0, atol=1e-12 * s.max())
    assert np.allclose(s, np.abs(a) @ np.abs(b).T, rtol=1e-12, atol=0)
    ones = np.full((M, K), 0x38, dtype=np.uint8)
    y1, _ = oracle.gemm_w4a8(ones, np.full((M, K // 32), 127, np.uint8), bc, bs)
    assert np.array_equal(y1, np.broadcast_to(b.sum(axis=1), (M, N)))
    pm = np.array([0, 6, 3]); pn = np.array([8, 0, 4])
    ys, ss = oracle.gemm_w4a8(ac, as_, bc, bs, pm, pn)
    assert np.array_equal(ys, y[pm, pn]) and np.array_equal(ss, s[pm, pn])


# ---- R17: Smooth pre-scale ----------------------------------------------------------
def test_smooth_rows_matches_torch_bf16_multiply():
    """bf16 x times bf16 smooth through torch's bf16 multiply (fp32 product
    rounded to bf16, a library routine), random values over the whole bf16
    range including subnormal and huge products."""
    rng = np.random.default_rng(140)
    M, K = 9, 96
    x = torch.from_numpy((rng.standard_normal((M, K)) * 2.0 ** rng.integers(-60, 60, (M, K)))
                         .astype(np.float32)).to(torch.bfloat16)
    sm = torch.from_numpy((rng.uniform(0.01, 8, K) * 2.0 ** rng.integers(-70, 70, K))
                          .astype(np.float32)).to(torch.bfloat16)
    want = bf16_bits(x * sm)
    got = oracle.smooth_rows(bf16_bits(x), bf16_bits(sm))
    assert np.array_equal(got, want)


def test_quantize_act_smooth_closed_forms():
    """A Smooth vector of ones changes nothing; a power of two per 32-block
    shifts that block's scale byte by its exponent and keeps its codes (while
    nothing clamps); a gather picks smoothed rows."""
    rng = np.random.default_rng(141)
    M, K = 6, 128
    x = torch.from_numpy(rng.normal(0, 1, (M, K)).astype(np.float32)).to(torch.bfloat16)
    xb = bf16_bits(x)
    ones = bf16_bits(torch.ones(K, dtype=torch.bfloat16))
    for rule in ("ocp", "uos"):
        a = oracle.quantize_act(xb, scale_rule=rule)
        b = oracle.quantize_act_smooth(xb, ones, scale_rule=rule)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c8 = oracle.quantize_act_fp8(xb)
    d8 = oracle.quantize_act_fp8_smooth(xb, ones)
    assert np.array_equal(c8[0], d8[0]) and np.array_equal(c8[1], d8[1])
    e = np.array([3, -5, 0, 9])
    pw = torch.from_numpy(np.repeat(2.0 ** e, 32).astype(np.float32)).to(torch.bfloat16)
    c, s_ = oracle.quantize_act_smooth(xb, bf16_bits(pw))
    c0, s0 = oracle.quantize_act(xb)
    assert np.array_equal(c, c0) and np.array_equal(s_.astype(int), s0.astype(int) + e)
    idx = np.array([5, 0, 5], dtype=np.int32)
    g = oracle.quantize_act_smooth(xb, bf16_bits(pw), row_index=idx)
    assert np.array_equal(g[0], c[idx]) and np.array_equal(g[1], s_[idx])


# ---- the pre-shuffled weight order --------------------------------------------------
def test_preshuffle_piece_by_piece_and_inverse():
    """preshuffle_codes against the piece formula the header states, one
    16-byte piece at a time in a plain loop (lane l, K-step t, stage s, block
    b of piece p; source row 32b + l % 32, bytes 128s + 16(4(l // 32) + t)),
    for two tensors; and the inverse permutation restores the input."""
    rng = np.random.default_rng(3)
    T, N, K = 2, 64, 512
    codes = rng.integers(0, 256, (T, N, K // 2), dtype=np.uint8)
    out = oracle.preshuffle_codes(codes)
    S = K // 256
    for tt in range(T):
        flat = out[tt].reshape(-1)
        for p in range(N * K // 32):
            l, t, s, b = p % 64, (p // 64) % 4, (p // 256) % S, p // (256 * S)
            row, byte = 32 * b + l % 32, 128 * s + 16 * (4 * (l // 32) + t)
            assert np.array_equal(flat[16 * p:16 * p + 16], codes[tt, row, byte:byte + 16]), (tt, p)
    # a 2-D tensor is one tensor
    assert np.array_equal(oracle.preshuffle_codes(codes[1]), out[1])
    # the piece formula maps output bytes one to one onto input bytes, so
    # scattering the output back through it restores the input
    src = np.empty(N * K // 2, dtype=np.int64)
    for p in range(N * K // 32):
        l, t, s, b = p % 64, (p // 64) % 4, (p // 256) % S, p // (256 * S)
        row, byte = 32 * b + l % 32, 128 * s + 16 * (4 * (l // 32) + t)
        src[16 * p:16 * p + 16] = row * (K // 2) + byte + np.arange(16)
    assert np.array_equal(np.sort(src), np.arange(src.size))
    back = np.empty(N * K // 2, dtype=np.uint8)
    back[src] = out[0].reshape(-1)
    assert np.array_equal(back.reshape(N, K // 2), codes[0])
