"""CPU oracle for the block-scaled 4-bit (E2M1) linear-layer path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its binding) never imports, links or calls it, and
it shares no code with that path.

The arithmetic lives in ``mxfp4_oracle.c`` (plain C, fp64, one obvious loop
per definition); this module is a ctypes veneer that moves numpy arrays in and
out.  Source passages for every definition are listed in ``mxfp4_oracle.h``.

Tolerance rules for the GEMM (``gemm_fp32_ok`` / ``gemm_bf16_ok``) restate
the parity bar fixed for this path: per element
``|gpu - y| <= 1e-5 * sum_k |a_k b_k|`` for fp32 output, and at most one bf16
ulp (ordered-bit distance, +0 == -0) from RNE_bf16(y) for bf16 output.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_DIR = pathlib.Path(__file__).resolve().parent
_SRC = _DIR / "mxfp4_oracle.c"
_LIB_PATH = _DIR / "_liboracle.so"
_lib = None

GEMM_FP32_RTOL = 1e-5


def build() -> pathlib.Path:
    """Compile the oracle with the host gcc (no GPU toolchain involved)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
        "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", str(_SRC),
        "-o", str(_LIB_PATH) + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(str(_LIB_PATH) + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        build()
    lib = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint]
    lib.orc_e8m0_value.restype = ctypes.c_double
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_from_double.restype = ctypes.c_uint16
    lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
    lib.orc_e2m1_encode.restype = ctypes.c_uint
    lib.orc_e2m1_encode.argtypes = [ctypes.c_double]
    lib.orc_e2m1_encode_bf16_at_scale.restype = None
    lib.orc_e2m1_encode_bf16_at_scale.argtypes = [P, I, ctypes.c_uint, P]
    lib.orc_shared_exponent.restype = ctypes.c_uint
    lib.orc_shared_exponent.argtypes = [ctypes.c_double]
    lib.orc_shared_exponent_uos.restype = ctypes.c_uint
    lib.orc_shared_exponent_uos.argtypes = [ctypes.c_double]
    lib.orc_mx_quantize_block.restype = None
    lib.orc_mx_quantize_block.argtypes = [P, P, P]
    lib.orc_mx_quantize_block_rule.restype = None
    lib.orc_mx_quantize_block_rule.argtypes = [P, P, P, ctypes.c_int]
    lib.orc_nvfp4_dequant.restype = None
    lib.orc_nvfp4_dequant.argtypes = [P, P, ctypes.c_float, I, I, ctypes.c_int, P]
    lib.orc_requant.restype = None
    lib.orc_requant.argtypes = [P, P, P, I, I, I, ctypes.c_int, P, P]
    lib.orc_requant_rule.restype = None
    lib.orc_requant_rule.argtypes = [P, P, P, I, I, I, ctypes.c_int, ctypes.c_int, P, P]
    lib.orc_quantize_act.restype = None
    lib.orc_quantize_act.argtypes = [P, I, P, I, I, P, P]
    lib.orc_quantize_act_rule.restype = None
    lib.orc_quantize_act_rule.argtypes = [P, I, P, I, I, ctypes.c_int, P, P]
    lib.orc_gemm.restype = None
    lib.orc_gemm.argtypes = [P, P, P, P, I, I, I, P, P]
    lib.orc_gemm_at.restype = None
    lib.orc_gemm_at.argtypes = [P, P, P, P, I, I, I, P, P, I, P, P]
    lib.orc_grouped_gemm.restype = None
    lib.orc_grouped_gemm.argtypes = [P, P, P, P, P, I, I, I, P, P]
    lib.orc_silu_mul_f32.restype = ctypes.c_float
    lib.orc_silu_mul_f32.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.orc_silu_mul.restype = None
    lib.orc_silu_mul.argtypes = [P, I, I, I, P, P]
    lib.orc_silu_mul_quantize.restype = None
    lib.orc_silu_mul_quantize.argtypes = [P, I, I, I, ctypes.c_int, P, P]
    lib.orc_moe_combine.restype = None
    lib.orc_moe_combine.argtypes = [P, I, P, P, I, I, I, P, P]
    lib.orc_smooth_rows.restype = None
    lib.orc_smooth_rows.argtypes = [P, I, P, P, I, I, P]
    lib.orc_e4m3_encode.restype = ctypes.c_uint
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_shared_exponent_fp8.restype = ctypes.c_uint
    lib.orc_shared_exponent_fp8.argtypes = [ctypes.c_double]
    lib.orc_mx8_quantize_block.restype = None
    lib.orc_mx8_quantize_block.argtypes = [P, P, P]
    lib.orc_quantize_act_fp8.restype = None
    lib.orc_quantize_act_fp8.argtypes = [P, I, P, I, I, P, P]
    lib.orc_gemm_w4a8_at.restype = None
    lib.orc_gemm_w4a8_at.argtypes = [P, P, P, P, I, I, I, P, P, I, P, P]
    lib.orc_add_row_bias.restype = None
    lib.orc_add_row_bias.argtypes = [P, P, I, I, P]
    lib.orc_bf16_from_double_array.restype = None
    lib.orc_bf16_from_double_array.argtypes = [P, I, P]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_set_num_threads.restype = None
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the oracle's loops from now on."""
    _load().orc_set_num_threads(int(n))


# ---- scalar codecs (for the pins) ----------------------------------------
def e2m1_value(code: int) -> float:
    return float(_load().orc_e2m1_value(int(code)))


def e4m3_value(byte: int) -> float:
    return float(_load().orc_e4m3_value(int(byte)))


def e8m0_value(byte: int) -> float:
    return float(_load().orc_e8m0_value(int(byte)))


def bf16_value(bits: int) -> float:
    return float(_load().orc_bf16_value(int(bits)))


def bf16_from_double(v: float) -> int:
    return int(_load().orc_bf16_from_double(float(v)))


def bf16_from_double_array(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_bf16_from_double_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_encode(q: float) -> int:
    return int(_load().orc_e2m1_encode(float(q)))


def e2m1_encode_bf16_at_scale(x_bits, byte: int) -> np.ndarray:
    """R4 at a fixed scale byte: the E2M1 code (0..15) of each bf16 value
    divided by 2^(byte - 127), as the block quantizer encodes its elements."""
    x_bits = _c(x_bits, np.uint16)
    out = np.empty(x_bits.shape, dtype=np.uint8)
    _load().orc_e2m1_encode_bf16_at_scale(_ptr(x_bits), x_bits.size, int(byte), _ptr(out))
    return out


# Scale rules: "ocp" (R3, the OCP MX shared exponent) and "uos" (R9, the
# Qmax = 7.25 rule of the vLLM-Omni guide's single-scale setting 2).
_RULES = {"ocp": 0, "uos": 1}


def shared_exponent(amax: float, rule: str = "ocp") -> int:
    fn = _load().orc_shared_exponent_uos if rule == "uos" else _load().orc_shared_exponent
    assert rule in _RULES
    return int(fn(float(amax)))


def mx_quantize_block(v, rule: str = "ocp") -> tuple[np.ndarray, int]:
    v = _c(v, np.float64)
    assert v.shape == (32,)
    codes = np.empty(16, dtype=np.uint8)
    scale = np.empty(1, dtype=np.uint8)
    _load().orc_mx_quantize_block_rule(_ptr(v), _ptr(codes), _ptr(scale), _RULES[rule])
    return codes, int(scale[0])


# ---- the operations of the path -------------------------------------------
def nvfp4_dequant(codes, scales, g, bf16_intermediate=False) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (N, K // 16)
    out = np.empty((N, K), dtype=np.float32)
    _load().orc_nvfp4_dequant(_ptr(codes), _ptr(scales), float(np.float32(g)), N, K,
                              int(bool(bf16_intermediate)), _ptr(out))
    return out


def requant(nv_codes, nv_scales, nv_global, bf16_intermediate=False, scale_rule="ocp"):
    """NVFP4 [T,N,K/2] + [T,N,K/16] + g[T] -> MXFP4 codes [T,N,K/2], E8M0 [T,N,K/32]."""
    nv_codes = _c(nv_codes, np.uint8)
    nv_scales = _c(nv_scales, np.uint8)
    squeeze = nv_codes.ndim == 2
    if squeeze:
        nv_codes = nv_codes[None]
        nv_scales = nv_scales[None]
    g = _c(np.atleast_1d(nv_global), np.float32)
    T, N, Kh = nv_codes.shape
    K = 2 * Kh
    assert K % 32 == 0 and nv_scales.shape == (T, N, K // 16) and g.shape == (T,)
    codes = np.empty((T, N, K // 2), dtype=np.uint8)
    scales = np.empty((T, N, K // 32), dtype=np.uint8)
    _load().orc_requant_rule(_ptr(nv_codes), _ptr(nv_scales), _ptr(g), T, N, K,
                             int(bool(bf16_intermediate)), _RULES[scale_rule],
                             _ptr(codes), _ptr(scales))
    if squeeze:
        return codes[0], scales[0]
    return codes, scales


def quantize_act(x_bits, K=None, row_index=None, scale_rule="ocp"):
    """bf16 bit patterns (uint16) [R, ldx] -> codes [M, K/2], E8M0 [M, K/32]."""
    x_bits = _c(x_bits, np.uint16)
    R, ldx = x_bits.shape
    K = ldx if K is None else int(K)
    assert K % 32 == 0 and K <= ldx
    if row_index is not None:
        row_index = _c(row_index, np.int32)
        M = row_index.shape[0]
        assert M == 0 or (row_index.min() >= 0 and row_index.max() < R)
    else:
        M = R
    codes = np.empty((M, K // 2), dtype=np.uint8)
    scales = np.empty((M, K // 32), dtype=np.uint8)
    if M:
        _load().orc_quantize_act_rule(_ptr(x_bits), ldx, _ptr(row_index), M, K,
                                      _RULES[scale_rule], _ptr(codes), _ptr(scales))
    return codes, scales


def _gemm_operands(a_codes, a_scales, b_codes, b_scales):
    a_codes = _c(a_codes, np.uint8)
    a_scales = _c(a_scales, np.uint8)
    b_codes = _c(b_codes, np.uint8)
    b_scales = _c(b_scales, np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[-2]
    assert K % 32 == 0 and b_codes.shape[-1] * 2 == K
    assert a_scales.shape == (M, K // 32) and b_scales.shape[-1] == K // 32
    return a_codes, a_scales, b_codes, b_scales, M, N, K


def gemm(a_codes, a_scales, b_codes, b_scales):
    """Returns (y, s): fp64 [M,N] result and sum_k |a_k b_k|."""
    a_codes, a_scales, b_codes, b_scales, M, N, K = _gemm_operands(
        a_codes, a_scales, b_codes, b_scales)
    y = np.empty((M, N), dtype=np.float64)
    s = np.empty((M, N), dtype=np.float64)
    _load().orc_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                     M, N, K, _ptr(y), _ptr(s))
    return y, s


def gemm_at(a_codes, a_scales, b_codes, b_scales, pm, pn):
    a_codes, a_scales, b_codes, b_scales, M, N, K = _gemm_operands(
        a_codes, a_scales, b_codes, b_scales)
    pm = _c(pm, np.int64)
    pn = _c(pn, np.int64)
    assert pm.shape == pn.shape and pm.ndim == 1
    assert (pm >= 0).all() and (pm < M).all() and (pn >= 0).all() and (pn < N).all()
    y = np.empty(pm.shape, dtype=np.float64)
    s = np.empty(pm.shape, dtype=np.float64)
    _load().orc_gemm_at(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                        M, N, K, _ptr(pm), _ptr(pn), pm.shape[0], _ptr(y), _ptr(s))
    return y, s


def mxfp4_dequant_f64(codes, scales) -> np.ndarray:
    """MXFP4 codes [rows, K/2] + E8M0 [rows, K/32] -> fp64 values [rows, K]:
    e2m1(code) * 2^(byte - 127), exact in fp64 (the E2M1 table is the C
    oracle's own decode, R1 nibble order); byte 0xFF gives NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows, Kh = codes.shape
    table = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    v = np.empty((rows, 2 * Kh), dtype=np.float64)
    v[:, 0::2] = table[codes & 15]
    v[:, 1::2] = table[codes >> 4]
    f = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    v *= np.repeat(f, 32, axis=1)
    return v


def gemm_blas(a_codes, a_scales, b_codes, b_scales, row_chunk=1024):
    """R5's result through a library matmul, for sizes the exact oracle cannot
    finish in seconds: both operands dequantized exactly to fp64, then
    y = A B^T and s = |A| |B|^T by numpy's BLAS, in row chunks.  Every product
    is exact; the fp64 sums carry an error of at most about K * 2^-53 * s
    (against the 1e-5 * s parity bar).  Returns (y, s) like gemm."""
    M = np.asarray(a_codes).shape[0]
    B = mxfp4_dequant_f64(b_codes, b_scales)
    Bt, Bat = np.ascontiguousarray(B.T), np.ascontiguousarray(np.abs(B).T)
    del B
    y = np.empty((M, Bt.shape[1]), dtype=np.float64)
    s = np.empty_like(y)
    for r0 in range(0, M, row_chunk):
        A = mxfp4_dequant_f64(a_codes[r0:r0 + row_chunk], a_scales[r0:r0 + row_chunk])
        np.matmul(A, Bt, out=y[r0:r0 + A.shape[0]])
        np.matmul(np.abs(A), Bat, out=s[r0:r0 + A.shape[0]])
    return y, s


def grouped_gemm(a_codes, a_scales, b_codes, b_scales, offsets):
    """A [total_M, K/2] expert-sorted, B [E, N, K/2], offsets [E+1]."""
    a_codes, a_scales, b_codes, b_scales, M, N, K = _gemm_operands(
        a_codes, a_scales, b_codes, b_scales)
    offsets = _c(offsets, np.int32)
    E = offsets.shape[0] - 1
    assert b_codes.shape == (E, N, K // 2) and b_scales.shape == (E, N, K // 32)
    assert offsets[0] == 0 and offsets[-1] == M and (np.diff(offsets) >= 0).all()
    y = np.zeros((M, N), dtype=np.float64)
    s = np.zeros((M, N), dtype=np.float64)
    _load().orc_grouped_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                             _ptr(b_scales), _ptr(offsets), E, N, K, _ptr(y), _ptr(s))
    return y, s


# ---- O12: the layerwise load ----------------------------------------------------
def layerwise_requant(sources, excluded, dest, first_layer=0, flags_bf16=False,
                      scale_rule="ocp"):
    """The layerwise load of the AMD blog's pipeline section (Figure 1): the
    model's NVFP4 weights are requantized one layer at a time into a
    destination allocated beforehand, and tensors the producer excluded are
    skipped (the blog's note on producer excludes).  In symbols, for every
    layer l >= first_layer, tensor kind k and tensor t:

        dest[k][l, t] = requant(sources[l][k][t])   unless excluded[l][k][t]

    and every excluded slot keeps whatever it held.

    sources   per layer, per kind: (codes [T,N,K/2], E4M3 [T,N,K/16], g [T])
    excluded  bool [L, kinds, T]
    dest      per kind: (codes [L,T,N,K/2], E8M0 [L,T,N,K/32]), written in place
    Returns the number of tensors requantized.  Peak extra memory is one
    layer's source, which the caller holds; this function holds nothing more
    than one requantized kind of one layer."""
    excluded = np.asarray(excluded, dtype=bool)
    L = len(sources)
    done = 0
    for l in range(first_layer, L):
        for k, (codes, scales, g) in enumerate(sources[l]):
            keep = np.nonzero(~excluded[l, k])[0]
            if keep.size == 0:
                continue
            c, sc = requant(np.asarray(codes)[keep], np.asarray(scales)[keep],
                            np.asarray(g, dtype=np.float32).reshape(-1)[keep],
                            bf16_intermediate=flags_bf16, scale_rule=scale_rule)
            dest[k][0][l, keep] = c
            dest[k][1][l, keep] = sc
            done += keep.size
    return done


# ---- Smooth pre-scale (R17) ---------------------------------------------------------
def smooth_rows(x_bits, smooth_bits, K=None, row_index=None):
    """bf16 bits [R, ldx] times the bf16 Smooth vector [K] (fp32 product, RNE to
    bf16) -> bf16 bits [M, K] (M = R, or len(row_index) with a gather)."""
    x_bits = _c(x_bits, np.uint16)
    R, ldx = x_bits.shape
    K = ldx if K is None else int(K)
    smooth_bits = _c(smooth_bits, np.uint16)
    assert smooth_bits.shape == (K,) and K <= ldx
    if row_index is not None:
        row_index = _c(row_index, np.int32)
        M = row_index.shape[0]
    else:
        M = R
    out = np.empty((M, K), dtype=np.uint16)
    if M and K:
        _load().orc_smooth_rows(_ptr(x_bits), ldx, _ptr(row_index), _ptr(smooth_bits), M, K,
                                _ptr(out))
    return out


def quantize_act_smooth(x_bits, smooth_bits, K=None, row_index=None, scale_rule="ocp"):
    """R17 then R3/R9 + R4: MXFP4 of bf16(x * smooth)."""
    h = smooth_rows(x_bits, smooth_bits, K, row_index)
    return quantize_act(h, scale_rule=scale_rule)


def quantize_act_fp8_smooth(x_bits, smooth_bits, K=None, row_index=None):
    """R17 then R13 + R14: MXFP8 of bf16(x * smooth)."""
    h = smooth_rows(x_bits, smooth_bits, K, row_index)
    return quantize_act_fp8(h)


# ---- W4A8 (R13-R15) -------------------------------------------------------------
def e4m3_encode(q: float) -> int:
    return int(_load().orc_e4m3_encode(float(q)))


def shared_exponent_fp8(amax: float) -> int:
    return int(_load().orc_shared_exponent_fp8(float(amax)))


def mx8_quantize_block(v) -> tuple[np.ndarray, int]:
    """32 values -> (32 E4M3 code bytes, E8M0 byte)."""
    v = _c(v, np.float64)
    assert v.shape == (32,)
    codes = np.empty(32, dtype=np.uint8)
    scale = np.empty(1, dtype=np.uint8)
    _load().orc_mx8_quantize_block(_ptr(v), _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


def quantize_act_fp8(x_bits, K=None, row_index=None):
    """bf16 bit patterns [R, ldx] -> MXFP8 codes [M, K] (E4M3 bytes), E8M0 [M, K/32]."""
    x_bits = _c(x_bits, np.uint16)
    R, ldx = x_bits.shape
    K = ldx if K is None else int(K)
    assert K % 32 == 0 and K <= ldx
    if row_index is not None:
        row_index = _c(row_index, np.int32)
        M = row_index.shape[0]
        assert M == 0 or (row_index.min() >= 0 and row_index.max() < R)
    else:
        M = R
    codes = np.empty((M, K), dtype=np.uint8)
    scales = np.empty((M, K // 32), dtype=np.uint8)
    if M:
        _load().orc_quantize_act_fp8(_ptr(x_bits), ldx, _ptr(row_index), M, K, _ptr(codes),
                                     _ptr(scales))
    return codes, scales


def gemm_w4a8(a_codes, a_scales, b_codes, b_scales, pm=None, pn=None):
    """R15: A MXFP8 [M, K] + [M, K/32], B MXFP4 [N, K/2] + [N, K/32].  Whole
    [M, N] result (y, s), or at the sampled positions (pm, pn)."""
    a_codes = _c(a_codes, np.uint8)
    a_scales = _c(a_scales, np.uint8)
    b_codes = _c(b_codes, np.uint8)
    b_scales = _c(b_scales, np.uint8)
    M, K = a_codes.shape
    N = b_codes.shape[0]
    assert K % 32 == 0 and b_codes.shape == (N, K // 2)
    assert a_scales.shape == (M, K // 32) and b_scales.shape == (N, K // 32)
    if pm is None:
        P = M * N
        y = np.empty((M, N), dtype=np.float64)
        s = np.empty((M, N), dtype=np.float64)
        if P:
            _load().orc_gemm_w4a8_at(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes),
                                     _ptr(b_scales), M, N, K, None, None, P, _ptr(y), _ptr(s))
        return y, s
    pm = _c(pm, np.int64)
    pn = _c(pn, np.int64)
    assert pm.shape == pn.shape and pm.ndim == 1
    assert (pm >= 0).all() and (pm < M).all() and (pn >= 0).all() and (pn < N).all()
    y = np.empty(pm.shape, dtype=np.float64)
    s = np.empty(pm.shape, dtype=np.float64)
    if pm.size:
        _load().orc_gemm_w4a8_at(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales),
                                 M, N, K, _ptr(pm), _ptr(pn), pm.shape[0], _ptr(y), _ptr(s))
    return y, s


def add_row_bias(y, s, bias_bits):
    """R12: (y + bias[n], s + |bias[n]|) for an [M, N] GEMM result (y, s) and
    bf16 bias bits [N].  Returns new arrays."""
    y = np.array(y, dtype=np.float64, order="C", copy=True)
    s = np.array(s, dtype=np.float64, order="C", copy=True)
    bias_bits = _c(bias_bits, np.uint16)
    M, N = y.shape
    assert s.shape == (M, N) and bias_bits.shape == (N,)
    if M and N:
        _load().orc_add_row_bias(_ptr(y), _ptr(s), M, N, _ptr(bias_bits))
    return y, s


# ---- MoE expert epilogues (R10, R11) -------------------------------------------
def silu_mul_f32(g: float, u: float) -> float:
    """silu(g) * u with every step rounded to fp32 (R10)."""
    return float(_load().orc_silu_mul_f32(float(g), float(u)))


def _gate_up(gate_up_bits, I):
    gate_up_bits = _c(gate_up_bits, np.uint16)
    M, ldg = gate_up_bits.shape
    I = ldg // 2 if I is None else int(I)
    assert 2 * I <= ldg
    return gate_up_bits, M, ldg, I


def silu_mul(gate_up_bits, I=None):
    """bf16 bits [M, ldg] (gate = columns [0, I), up = [I, 2I)) ->
    (h bf16 bits [M, I], h fp32 [M, I] before the bf16 rounding)."""
    gate_up_bits, M, ldg, I = _gate_up(gate_up_bits, I)
    hb = np.empty((M, I), dtype=np.uint16)
    hf = np.empty((M, I), dtype=np.float32)
    if M and I:
        _load().orc_silu_mul(_ptr(gate_up_bits), ldg, M, I, _ptr(hb), _ptr(hf))
    return hb, hf


def silu_mul_quantize(gate_up_bits, I=None, scale_rule="ocp"):
    """R10 then act-quant: codes [M, I/2], E8M0 [M, I/32]."""
    gate_up_bits, M, ldg, I = _gate_up(gate_up_bits, I)
    assert I % 32 == 0
    codes = np.empty((M, I // 2), dtype=np.uint8)
    scales = np.empty((M, I // 32), dtype=np.uint8)
    if M and I:
        _load().orc_silu_mul_quantize(_ptr(gate_up_bits), ldg, M, I, _RULES[scale_rule],
                                      _ptr(codes), _ptr(scales))
    return codes, scales


def moe_combine(y_bits, rows, weights, H=None):
    """R11: y bf16 bits [R, ldy], rows int32 [T, topk] (sorted-row index of
    each token's j-th expert), weights fp32 [T, topk] -> (out fp64 [T, H],
    s = sum_j |w * y| [T, H])."""
    y_bits = _c(y_bits, np.uint16)
    R, ldy = y_bits.shape
    H = ldy if H is None else int(H)
    rows = _c(rows, np.int32)
    weights = _c(weights, np.float32)
    T, topk = rows.shape
    assert weights.shape == (T, topk) and H <= ldy
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < R)
    out = np.empty((T, H), dtype=np.float64)
    s = np.empty((T, H), dtype=np.float64)
    if T and H:
        _load().orc_moe_combine(_ptr(y_bits), ldy, _ptr(rows), _ptr(weights), T, topk, H,
                                _ptr(out), _ptr(s))
    return out, s


# ---- pre-shuffled weight order (a layout of this library) -------------------
def preshuffle_codes(codes):
    """The weight-code order of mxfp4_preshuffle_weights.  It is this
    library's own layout (defined where include/mxfp4.h declares that call),
    not something the pages define: a permutation of each tensor's bytes so
    that one 32x32x64 matrix-core operand load is 1 KiB contiguous.  With the
    codes of a tensor viewed as [N/32 blocks b][32 rows q][K/256 stages s]
    [2 halves h][4 K-steps t][16 bytes j] (row 32b + q, byte 128s + 16(4h + t)
    + j of the row), the output lists the same bytes in the order
    [b][s][t][h][q][j]: piece ((b S + s) 4 + t) 64 + 32h + q.  codes:
    [..., N, K/2] uint8, N % 32 == 0, K % 256 == 0."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    *lead, N, half = c.shape
    K = 2 * half
    assert N % 32 == 0 and K % 256 == 0
    n = len(lead)
    v = c.reshape(*lead, N // 32, 32, K // 256, 2, 4, 16)
    axes = list(range(n)) + [n + a for a in (0, 2, 4, 3, 1, 5)]
    return np.ascontiguousarray(v.transpose(axes)).reshape(c.shape)


# ---- parity bar for the GEMM ------------------------------------------------
def gemm_fp32_ok(gpu, y, s, rtol=GEMM_FP32_RTOL) -> np.ndarray:
    """Elementwise: |gpu - y| <= rtol * s (s == 0 requires gpu == 0)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    return np.abs(gpu - y) <= rtol * s


def _bf16_ordered(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def gemm_bf16_ok(gpu_bits, y, max_ulp=1) -> np.ndarray:
    """Elementwise: ordered-bit distance between the GPU's bf16 output and
    RNE_bf16(y) is at most max_ulp (+0 and -0 are the same point)."""
    ref = bf16_from_double_array(y)
    return np.abs(_bf16_ordered(gpu_bits) - _bf16_ordered(ref)) <= max_ulp
