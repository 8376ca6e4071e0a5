"""Seeded synthetic inputs for the block-scaled 4-bit linear-layer path.

This module only *draws inputs*.  It contains none of the arithmetic the path
computes (no MXFP4 quantization, no requant, no GEMM) and imports neither the
HIP binding nor the CPU oracle; both of those consume what it returns.

Recipes (workload shapes and distributions as the path is benchmarked):

* bf16 tensors: ``torch.randn`` (fp32) from a seeded ``torch.Generator`` on
  the requested device, times sigma, rounded to bf16.
* outlier channels: ``round(0.01 * K)`` K-channels drawn without replacement
  from their own seed and multiplied by 50 in fp32 before the bf16 rounding.
* NVFP4 weights from bf16 W (the input format the requant consumes):
  g = fp32(amax|W| / (448 * 6)) per tensor; per 16-block along K the E4M3
  scale is torch's fp32 -> float8_e4m3fn cast of min(amax_blk / (6 g), 448);
  each element gets the index of the E2M1 magnitude nearest to |w| / (s g),
  ties toward the smaller magnitude, and the sign bit of w when that index is
  non-zero.  Two codes per byte, even element in the low nibble.  Any byte
  pattern is a valid NVFP4 input, so nothing downstream depends on these
  generator choices.
* MoE routing: logits N(0, 1) [tokens, experts], fp32 softmax, top-k, then a
  stable sort of the (token, expert) pairs by expert: ``perm`` holds the token
  of each routed row and ``offsets[E+1]`` the per-expert row ranges.
* canonical MXFP4 operands (GEMM-only tests): uniformly random codes and
  E8M0 bytes drawn from a stated range.
"""
from __future__ import annotations

import math

import torch

# Half-way points between neighbouring E2M1 magnitudes, used only by the
# input-side NVFP4 encoder above (ties resolve toward the smaller magnitude).
_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(shape, sigma: float, seed: int, device="cpu") -> torch.Tensor:
    x = torch.randn(shape, generator=generator(seed, device), device=device,
                    dtype=torch.float32)
    return (x * sigma).to(torch.bfloat16)


def outlier_channels(K: int, seed: int, frac: float = 0.01) -> torch.Tensor:
    n = int(round(frac * K))
    perm = torch.randperm(K, generator=generator(seed, "cpu"))
    return torch.sort(perm[:n]).values


def activations(M: int, K: int, seed: int, outlier_seed: int | None = None,
                factor: float = 50.0, device="cpu") -> torch.Tensor:
    """bf16 [M, K] ~ N(0, 1), optionally with 1% of K-channels scaled x50."""
    x = torch.randn((M, K), generator=generator(seed, device), device=device,
                    dtype=torch.float32)
    if outlier_seed is not None:
        ch = outlier_channels(K, outlier_seed).to(device)
        x[:, ch] *= factor
    return x.to(torch.bfloat16)


def nvfp4_from_bf16(w: torch.Tensor):
    """bf16 [..., N, K] -> (codes u8 [..., N, K/2], E4M3 u8 [..., N, K/16],
    g fp32 [...]) with one global scale per leading index."""
    assert w.dtype == torch.bfloat16 and w.shape[-1] % 16 == 0
    lead = w.shape[:-2]
    N, K = w.shape[-2], w.shape[-1]
    wf = w.float().reshape(-1, N, K)
    T = wf.shape[0]
    amax = wf.abs().reshape(T, -1).amax(dim=1)
    g = (amax / (448.0 * 6.0)).to(torch.float32)
    g = torch.where(g > 0, g, torch.ones_like(g))
    blk = wf.reshape(T, N, K // 16, 16)
    bmax = blk.abs().amax(dim=-1)
    s_val = torch.clamp(bmax / (6.0 * g.view(T, 1, 1)), max=448.0)
    s_f8 = s_val.to(torch.float8_e4m3fn)
    s_bytes = s_f8.view(torch.uint8)
    s_dec = s_f8.to(torch.float32)
    denom = (s_dec * g.view(T, 1, 1)).unsqueeze(-1)
    safe = torch.where(denom > 0, denom, torch.ones_like(denom))
    r = (blk.abs() / safe).reshape(T, N, K)
    mids = torch.tensor(_MIDPOINTS, device=w.device, dtype=torch.float32)
    idx = torch.bucketize(r.contiguous(), mids, right=False).to(torch.uint8)
    idx = torch.where((denom > 0).expand(T, N, K // 16, 16).reshape(T, N, K), idx,
                      torch.zeros_like(idx))
    neg = (wf < 0) & (idx > 0)
    code = idx | (neg.to(torch.uint8) << 3)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return (packed.reshape(*lead, N, K // 2).contiguous(),
            s_bytes.reshape(*lead, N, K // 16).contiguous(),
            g.reshape(lead) if lead else g.reshape(()))


def canonical_mxfp4(rows: int, K: int, seed: int, scale_lo: int = 117,
                    scale_hi: int = 137, device="cpu"):
    """Random MXFP4 operand: codes u8 [rows, K/2] (all 256 byte values),
    E8M0 bytes u8 [rows, K/32] uniform in [scale_lo, scale_hi]."""
    gen = generator(seed, device)
    codes = torch.randint(0, 256, (rows, K // 2), generator=gen, device=device,
                          dtype=torch.int32).to(torch.uint8)
    scales = torch.randint(scale_lo, scale_hi + 1, (rows, K // 32), generator=gen,
                           device=device, dtype=torch.int32).to(torch.uint8)
    return codes, scales


def route_topk_full(tokens: int, experts: int, topk: int, seed: int, device="cpu"):
    """Softmax top-k routing over N(0,1) logits, ties to the lower expert index.
    Returns (perm int32 [tokens*topk]: token index of each expert-sorted row,
    offsets int32 [experts+1], rows int32 [tokens, topk]: the sorted row
    holding token t's j-th choice, weights fp32 [tokens, topk]: the chosen
    probabilities renormalised to sum to 1 per token)."""
    logits = torch.randn((tokens, experts), generator=generator(seed, device),
                         device=device, dtype=torch.float32)
    probs = torch.softmax(logits, dim=-1)
    top, idx = torch.topk(probs, topk, dim=-1)
    flat_e = idx.reshape(-1)
    flat_t = torch.arange(tokens, device=device).repeat_interleave(topk)
    order = torch.sort(flat_e, stable=True).indices
    perm = flat_t[order].to(torch.int32)
    counts = torch.bincount(flat_e, minlength=experts)
    offsets = torch.zeros(experts + 1, dtype=torch.int64, device=device)
    offsets[1:] = torch.cumsum(counts, 0)
    rows = torch.empty_like(order)
    rows[order] = torch.arange(order.numel(), device=device)
    weights = top / top.sum(dim=-1, keepdim=True)
    return (perm.contiguous(), offsets.to(torch.int32).contiguous(),
            rows.reshape(tokens, topk).to(torch.int32).contiguous(),
            weights.to(torch.float32).contiguous())


def route_topk(tokens: int, experts: int, topk: int, seed: int, device="cpu"):
    """route_topk_full's (perm, offsets)."""
    perm, offsets, _, _ = route_topk_full(tokens, experts, topk, seed, device)
    return perm, offsets


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def nbytes_mxfp4(rows: int, K: int) -> int:
    return rows * (K // 2) + rows * math.ceil(K / 32)
