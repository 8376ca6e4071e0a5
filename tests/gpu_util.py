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
