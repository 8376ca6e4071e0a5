"""Shared helpers for the GPU parity tests: host copies, canary-guarded
outputs, and the oracle-side chains that mirror the GPU calls."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

CANARY = 0xA5
PAD = 4096


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def u8(t) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def bf16_bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(t) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


class Guarded:
    """A device buffer with canary bytes before and after the usable view."""

    def __init__(self, shape, dtype, device=None):
        device = device or dev()
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * PAD,), CANARY, dtype=torch.uint8, device=device)
        self.n = n
        self.view = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def intact(self) -> bool:
        r = self.raw.cpu().numpy()
        return bool((r[:PAD] == CANARY).all() and (r[PAD + self.n:] == CANARY).all())


def oracle_requant_from_bf16(w_bf16_cpu, bf16_intermediate=False):
    """synth NVFP4 of a CPU bf16 weight, then the oracle's requant."""
    codes, scales, g = synth.nvfp4_from_bf16(w_bf16_cpu)
    mc, ms = oracle.requant(u8(codes), u8(scales), np.atleast_1d(g.numpy()),
                            bf16_intermediate=bf16_intermediate)
    return (codes, scales, g), (mc, ms)


def assert_gemm_bf16(gpu_y_bf16, y, label=""):
    bits = bf16_bits(gpu_y_bf16)
    ok = oracle.gemm_bf16_ok(bits, y)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{label}: {int((~ok).sum())} of {ok.size} bf16 outputs off by "
                             f">1 ulp, first at {idx.tolist()}")


def assert_gemm_fp32(gpu_y_f32, y, s, label=""):
    g = f32(gpu_y_f32).astype(np.float64)
    ok = oracle.gemm_fp32_ok(g, y, s)
    if not ok.all():
        idx = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} of {ok.size} fp32 outputs outside "
                             f"1e-5*S; first {idx}: gpu {g[idx]!r} oracle {y[idx]!r} S {s[idx]!r}")


# ---- W4A8 GEMM bar ----------------------------------------------------------------
# gfx950's E4M3 x E2M1 block-scaled MFMA sums the 32 products of each MX block
# in fixed point aligned to the block's largest magnitude, keeping 13 bits
# below its leading bit and truncating the rest (measured: 448 + x loses
# every x below 2^-5 and keeps x truncated to a multiple of 2^-5; blocks are
# then combined without loss).  Per block the loss is below 32 grid steps,
# the grid being 2^(floor(log2(max|a| * max|b|)) + 1 - 13) (the product of the
# operand maxima bounds the largest product and its leading bit).
W4A8_WINDOW_BITS = 13
_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def w4a8_block_maxima(a_codes, a_scales, b_codes, b_scales):
    """Per row: max |value| of each MX block of the dequantized MXFP8 A and
    MXFP4 B ([M, K/32], [N, K/32])."""
    M, K = a_codes.shape
    N = b_codes.shape[0]
    a = torch.from_numpy(np.ascontiguousarray(a_codes)).view(torch.float8_e4m3fn).double()
    a = a.abs().numpy().reshape(M, K // 32, 32).max(axis=2)
    a = a * 2.0 ** (np.asarray(a_scales, np.float64) - 127)
    nib = np.stack([b_codes & 15, b_codes >> 4], axis=-1).reshape(N, K // 32, 32)
    b = np.abs(_E2M1[nib]).max(axis=2) * 2.0 ** (np.asarray(b_scales, np.float64) - 127)
    return a, b


def w4a8_truncation_bound(amax, bmax, pm, pn):
    """Sum over blocks of 32 grid steps, at the sampled (m, n) positions."""
    prod = amax[pm] * bmax[pn]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(prod > 0, prod, 1.0)))
    step = np.where(prod > 0, np.ldexp(1.0, (e + 1 - W4A8_WINDOW_BITS).astype(np.int64)), 0.0)
    return 32.0 * step.sum(axis=-1)


def assert_w4a8(gpu, y, s, bound, label=""):
    """fp32: |gpu - y| <= 1e-5 * S + bound.  bf16: one ulp of RNE(y), or that
    fp32 bar plus one bf16 ulp of |y|."""
    g = f32(gpu.float()).astype(np.float64).reshape(y.shape)
    tol = oracle.GEMM_FP32_RTOL * s + bound
    if gpu.dtype == torch.bfloat16:
        _, e = np.frexp(np.abs(y))
        ulp = np.maximum(np.ldexp(1.0, e - 8), 2.0 ** -133)
        ok = oracle.gemm_bf16_ok(bf16_bits(gpu).reshape(y.shape), y) | (np.abs(g - y) <= tol + ulp)
    else:
        ok = np.abs(g - y) <= tol
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} of {ok.size} outside the W4A8 bar; "
                             f"first {i}: gpu {g[i]!r} oracle {y[i]!r} S {s[i]!r} "
                             f"bound {bound[i]!r}")
