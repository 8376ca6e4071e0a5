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


# ---- the product's plan, executed on the host with the oracle as the backend ----------
def mx_lib():
    return pytest.importorskip("w4a4_mxfp4_gemm_amd")


def flatten(sources, excluded):
    """Parts in load order (layer by layer, kind by kind) for the C ABI."""
    parts, masks, where = [], [], []
    for l, layer in enumerate(sources):
        for k, (codes, _, _) in enumerate(layer):
            T, N, Kh = codes.shape
            parts.append((T, N, 2 * Kh))
            masks.append(excluded[l, k].astype(np.uint8))
            where.append((l, k))
    return parts, masks, where


def execute_plan(plan, slot_bytes, scratch_bytes, sources, excluded, dest, where):
    """Run the plan as the GPU executor would, with a host array as the scratch:
    copy each kept tensor's NVFP4 bytes to its place in the slot, then requant
    from those staged bytes with the oracle.  Returns the tensors converted."""
    scratch = np.full(scratch_bytes, 0x5A, np.uint8)
    converted = []
    for c in plan:
        l, k = where[c["part"]]
        codes, scales, g = sources[l][k]
        T, N, Kh = codes.shape
        cb, sb = N * Kh, N * Kh // 8
        n = c["t1"] - c["t0"]
        lo, hi = c["slot"] * slot_bytes, (c["slot"] + 1) * slot_bytes
        assert c["slot"] in (0, 1) and hi <= scratch_bytes
        assert lo <= c["codes_offset"] and c["codes_offset"] + n * cb <= c["scales_offset"]
        assert c["scales_offset"] + n * sb <= c["global_offset"]
        assert c["global_offset"] + 4 * n <= hi
        assert c["codes_offset"] % 16 == 0 and c["scales_offset"] % 16 == 0
        assert not excluded[l, k, c["t0"]] and not excluded[l, k, c["t1"] - 1]
        kept = [t for t in range(c["t0"], c["t1"]) if not excluded[l, k, t]]
        for t in kept:                                    # the host -> device copies
            i = t - c["t0"]
            scratch[c["codes_offset"] + i * cb:c["codes_offset"] + (i + 1) * cb] = codes[t].ravel()
            scratch[c["scales_offset"] + i * sb:c["scales_offset"] + (i + 1) * sb] = scales[t].ravel()
        scratch[c["global_offset"]:c["global_offset"] + 4 * n] = \
            np.ascontiguousarray(g[c["t0"]:c["t1"]], np.float32).view(np.uint8)
        for t in kept:                                    # the requant, reading the slot
            i = t - c["t0"]
            sc = scratch[c["codes_offset"] + i * cb:c["codes_offset"] + (i + 1) * cb]
            ss = scratch[c["scales_offset"] + i * sb:c["scales_offset"] + (i + 1) * sb]
            sg = scratch[c["global_offset"] + 4 * i:c["global_offset"] + 4 * i + 4].view(np.float32)
            mc, ms = oracle.requant(sc.reshape(N, Kh), ss.reshape(N, Kh // 8), sg)
            dest[k][0][l, t], dest[k][1][l, t] = mc, ms
            converted.append((l, k, t))
    return converted


@pytest.mark.parametrize("scratch_tensors", [2, 3, 7, 1000])
def test_plan_executed_with_the_oracle_equals_the_definition(scratch_tensors):
    """With scratch for 2, 3 or 7 of the larger tensors (slots reused many
    times, chunks cut by exclusions) or for everything at once, the plan
    stages only kept tensors, inside its slots, each exactly once, and yields
    the oracle's layerwise load byte for byte, canaries intact."""
    mx = mx_lib()
    sources, excluded = setup(L=4, T=7, seed=5)
    L, T = len(sources), excluded.shape[2]
    parts, masks, where = flatten(sources, excluded)
    one = max(N * K // 2 + N * K // 16 for _, N, K in parts)
    scratch_bytes = scratch_tensors * (one + 1024)
    plan, slot_bytes = mx.mxfp4_layerwise_plan(parts, masks, scratch_bytes)
    got = canary_dest(L, T)
    converted = execute_plan(plan, slot_bytes, scratch_bytes, sources, excluded, got, where)
    want_list = [(l, k, t) for l in range(L) for k in range(len(SHAPES)) for t in range(T)
                 if not excluded[l, k, t]]
    assert sorted(converted) == want_list                 # each kept tensor exactly once
    want = canary_dest(L, T)
    oracle.layerwise_requant(sources, excluded, want)
    for (c0, s0), (c1, s1) in zip(want, got):
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_plan_at_the_full_load_stays_within_one_layer():
    """48 MoE layers x 128 experts x ([2048, 4096] + [4096, 1024]) with 5% of
    the tensors excluded and a scratch of one layer's NVFP4 bytes: every chunk
    lies inside its slot, no excluded tensor starts or ends a chunk, and every
    kept tensor is covered exactly once."""
    mx = mx_lib()
    L, E = 48, 128
    shapes = [(E, 2048, 4096), (E, 4096, 1024)]
    excluded = np.random.default_rng(42).random((L, 2, E)) < 0.05
    parts = [shapes[k] for _ in range(L) for k in range(2)]
    masks = [excluded[l, k].astype(np.uint8) for l in range(L) for k in range(2)]
    layer_bytes = sum(T * (N * K // 2 + N * K // 16) for T, N, K in shapes)
    plan, slot_bytes = mx.mxfp4_layerwise_plan(parts, masks, layer_bytes)
    assert 2 * slot_bytes <= layer_bytes
    covered = np.zeros((L, 2, E), np.int64)
    for c in plan:
        T, N, K = parts[c["part"]]
        l, k = divmod(c["part"], 2)
        n = c["t1"] - c["t0"]
        assert c["global_offset"] + 4 * n <= (c["slot"] + 1) * slot_bytes
        assert c["codes_offset"] >= c["slot"] * slot_bytes
        assert not excluded[l, k, c["t0"]] and not excluded[l, k, c["t1"] - 1]
        covered[l, k, c["t0"]:c["t1"]] += 1
    assert (covered[~excluded] == 1).all() and (covered[excluded] <= 1).all()


def test_plan_rejects_a_scratch_smaller_than_two_tensors():
    mx = mx_lib()
    with pytest.raises(mx.Mxfp4Error):
        mx.mxfp4_layerwise_plan([(4, 64, 128)], [None], 2 * (64 * 64 + 64 * 8))
