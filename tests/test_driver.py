"""The layerwise load on the CPU (no GPU).

The AMD blog's pipeline section (Figure 1) requantizes an NVFP4 checkpoint one
layer at a time into a destination allocated beforehand, skipping the tensors
the producer excluded, so that the extra memory the load needs is one layer's
source.  Two things are checked here:

* the oracle's definition of that load (``oracle.layerwise_requant``) against
  independent per-tensor requants, canary bytes in the excluded slots, re-runs
  from a later layer and layers that share one pooled source;
* the product's load plan (``mxfp4_layerwise_plan`` of the C ABI, host code
  only), executed step by step with host copies and the oracle's requant in
  place of the GPU: it must fill the destination exactly as the oracle's
  definition does, touch no excluded slot, and keep every staged byte inside
  the scratch buffer it was given.
"""
import numpy as np
import pytest

import oracle

CANARY = 0xA5
SHAPES = [(64, 128), (96, 64)]          # two tensor kinds (N, K), like gate_up and down


def make_sources(n_pool, T, seed):
    """Pooled NVFP4 layers: random code and E4M3 bytes (every byte pattern is a
    valid NVFP4 input, NaN scales included) and a random fp32 global per tensor."""
    rng = np.random.default_rng(seed)
    pool = []
    for _ in range(n_pool):
        layer = []
        for N, K in SHAPES:
            codes = rng.integers(0, 256, (T, N, K // 2), dtype=np.uint8)
            scales = rng.integers(0, 256, (T, N, K // 16), dtype=np.uint8)
            g = (rng.uniform(0.5, 2.0, T) * 2.0 ** rng.integers(-20, 20, T)).astype(np.float32)
            layer.append((codes, scales, g))
        pool.append(layer)
    return pool


def canary_dest(L, T):
    return [(np.full((L, T, N, K // 2), CANARY, np.uint8),
             np.full((L, T, N, K // 32), CANARY, np.uint8)) for N, K in SHAPES]


def setup(L=5, T=6, n_pool=2, seed=1, frac=0.25):
    pool = make_sources(n_pool, T, seed)
    sources = [pool[l % n_pool] for l in range(L)]
    excluded = np.random.default_rng(seed + 100).random((L, len(SHAPES), T)) < frac
    excluded[0, 0, :] = True                      # a wholly excluded kind
    excluded[1, 1, :] = False                     # a kind with nothing excluded
    return sources, excluded


def test_layerwise_definition_matches_independent_requants():
    """Every slot not excluded holds the requant of exactly its own tensor;
    every excluded slot still holds the canary bytes."""
    sources, excluded = setup()
    L, T = len(sources), excluded.shape[2]
    dest = canary_dest(L, T)
    n = oracle.layerwise_requant(sources, excluded, dest)
    assert n == int((~excluded).sum())
    for l in range(L):
        for k in range(len(SHAPES)):
            codes, scales, g = sources[l][k]
            for t in range(T):
                dc, ds = dest[k][0][l, t], dest[k][1][l, t]
                if excluded[l, k, t]:
                    assert (dc == CANARY).all() and (ds == CANARY).all(), (l, k, t)
                else:
                    c, s = oracle.requant(codes[t], scales[t], g[t:t + 1])
                    assert np.array_equal(dc, c) and np.array_equal(ds, s), (l, k, t)


def test_layerwise_rerun_from_a_later_layer_is_identical():
    """Re-running the load from layer l over a finished destination changes
    no byte; run from l on a fresh destination it writes layers >= l exactly
    as the full run did and leaves the earlier layers alone."""
    sources, excluded = setup(seed=2)
    L, T = len(sources), excluded.shape[2]
    full = canary_dest(L, T)
    oracle.layerwise_requant(sources, excluded, full)
    again = [(c.copy(), s.copy()) for c, s in full]
    oracle.layerwise_requant(sources, excluded, again, first_layer=2)
    for (c0, s0), (c1, s1) in zip(full, again):
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    fresh = canary_dest(L, T)
    oracle.layerwise_requant(sources, excluded, fresh, first_layer=2)
    for (c0, s0), (c1, s1) in zip(full, fresh):
        assert (c1[:2] == CANARY).all() and (s1[:2] == CANARY).all()
        assert np.array_equal(c0[2:], c1[2:]) and np.array_equal(s0[2:], s1[2:])


def test_layerwise_pooled_layers_agree():
    """Layers that share one pooled source give the same bytes in every slot
    both of them convert."""
    sources, excluded = setup(L=6, n_pool=2, seed=3)
    L, T = len(sources), excluded.shape[2]
    dest = canary_dest(L, T)
    oracle.layerwise_requant(sources, excluded, dest)
    for k in range(len(SHAPES)):
        for l in range(2, L):
            both = ~excluded[l, k] & ~excluded[l - 2, k]
            assert np.array_equal(dest[k][0][l, both], dest[k][0][l - 2, both])
            assert np.array_equal(dest[k][1][l, both], dest[k][1][l - 2, both])
