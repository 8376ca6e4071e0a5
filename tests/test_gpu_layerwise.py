"""GPU parity of the layerwise load (mxfp4_requant_layers_from_host) against
the oracle's definition of it: NVFP4 layers in pinned host memory, staged
through a device scratch buffer of at most one layer, requantized into a
preallocated destination whose excluded slots must keep their canary bytes
(AMD blog, pipeline section under Figure 1 and its note on producer
excludes).  Everything is bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, say, u8

pytestmark = pytest.mark.gpu

CANARY = 0xA5


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a4_mxfp4_gemm_amd as m
    return m


def pinned(t):
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


def make_pool(shapes, T, n_pool, seed):
    """Pooled layers on the host: NVFP4 of bf16 N(0, 0.02) weights (the
    workload's recipe), except that the last pooled layer's second kind holds
    random bytes (NaN and subnormal E4M3 scales included)."""
    pool = []
    for p in range(n_pool):
        layer = []
        for k, (N, K) in enumerate(shapes):
            if p == n_pool - 1 and k == 1:
                rng = np.random.default_rng(seed + 7)
                c = torch.from_numpy(rng.integers(0, 256, (T, N, K // 2), dtype=np.uint8))
                s = torch.from_numpy(rng.integers(0, 256, (T, N, K // 16), dtype=np.uint8))
                g = torch.from_numpy(rng.uniform(1e-3, 1.0, T).astype(np.float32))
            else:
                w = synth.bf16_normal((T, N, K), 0.02, seed=seed + 10 * p + k)
                c, s, g = synth.nvfp4_from_bf16(w)
            layer.append((pinned(c), pinned(s), pinned(g.reshape(T).contiguous())))
        pool.append(layer)
    return pool


def build_case(shapes, L, T, n_pool, seed, frac=0.2):
    pool = make_pool(shapes, T, n_pool, seed)
    sources = [pool[l % n_pool] for l in range(L)]
    excluded = np.random.default_rng(seed + 1).random((L, len(shapes), T)) < frac
    excluded[1, 0, :] = True                    # a kind with every tensor excluded
    excluded[0, 1, :] = False                   # and one with none
    return sources, excluded


def device_dest(shapes, L, T):
    d = dev()
    return [(torch.full((L, T, N, K // 2), CANARY, dtype=torch.uint8, device=d),
             torch.full((L, T, N, K // 32), CANARY, dtype=torch.uint8, device=d))
            for N, K in shapes]


def parts_for(sources, excluded, dest, first_layer=0):
    parts = []
    for l in range(first_layer, len(sources)):
        for k, (c, s, g) in enumerate(sources[l]):
            parts.append(dict(nv_codes=c, nv_scales=s, nv_global=g,
                              excluded=torch.from_numpy(excluded[l, k].astype(np.uint8)),
                              mx_codes=dest[k][0][l], mx_scales=dest[k][1][l]))
    return parts


def oracle_load(sources, excluded, shapes, L, T, **kw):
    want = [(np.full((L, T, N, K // 2), CANARY, np.uint8),
             np.full((L, T, N, K // 32), CANARY, np.uint8)) for N, K in shapes]
    np_sources = [[(c.numpy(), s.numpy(), g.numpy()) for c, s, g in layer] for layer in sources]
    oracle.layerwise_requant(np_sources, excluded, want, **kw)
    return want


def assert_same(dest, want, label):
    for k, ((dc, ds), (wc, ws)) in enumerate(zip(dest, want)):
        assert np.array_equal(u8(dc), wc), f"{label}: kind {k} codes differ"
        assert np.array_equal(u8(ds), ws), f"{label}: kind {k} scales differ"


def one_layer_bytes(shapes, T):
    return sum(T * (N * K // 2 + N * K // 16) for N, K in shapes)


SHAPES = [(256, 512), (512, 256)]


@pytest.mark.parametrize("scratch", ["layer", "two_tensors"])
@pytest.mark.parametrize("streams", ["two", "one"])
def test_layerwise_load_equals_the_oracle(mx, scratch, streams):
    """4 layers x 2 kinds x 8 tensors from 2 pooled layers, ~20% excluded; the
    scratch is one layer (two chunks a layer) or just over two of the larger
    tensors (every chunk one or two tensors, slots refilled 30+ times); the
    copies on their own stream or on the compute stream."""
    L, T = 4, 8
    say(f"layerwise load L={L} T={T} scratch={scratch} streams={streams}")
    sources, excluded = build_case(SHAPES, L, T, 2, seed=11)
    dest = device_dest(SHAPES, L, T)
    big = max(N * K // 2 + N * K // 16 for N, K in SHAPES)
    nbytes = one_layer_bytes(SHAPES, T) if scratch == "layer" else 2 * (big + 1024)
    d = dev()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(d)[0]
    base = torch.cuda.memory_allocated(d)
    torch.cuda.reset_peak_memory_stats(d)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=d)
    cs = torch.cuda.Stream(d) if streams == "two" else None
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, dest), buf, copy_stream=cs)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(d) - base
    free1 = torch.cuda.mem_get_info(d)[0]
    assert peak <= nbytes + (1 << 20), f"peak extra memory {peak} > scratch {nbytes}"
    assert free0 - free1 <= nbytes + (64 << 20), "the load took device memory of its own"
    assert nbytes <= one_layer_bytes(SHAPES, T)
    want = oracle_load(sources, excluded, SHAPES, L, T)
    assert_same(dest, want, f"{scratch}/{streams}")


def test_layerwise_load_rerun_from_a_later_layer(mx):
    """Re-running the load from layer 2 over the finished destination changes
    nothing; run from layer 2 on a fresh destination it leaves layers 0-1 as
    canaries and writes the rest as the full load did."""
    L, T = 4, 8
    say("layerwise load re-run from layer 2")
    sources, excluded = build_case(SHAPES, L, T, 2, seed=21)
    buf = torch.empty(one_layer_bytes(SHAPES, T), dtype=torch.uint8, device=dev())
    cs = torch.cuda.Stream(dev())
    full = device_dest(SHAPES, L, T)
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, full), buf, copy_stream=cs)
    torch.cuda.synchronize()
    before = [(c.clone(), s.clone()) for c, s in full]
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, full, 2), buf, copy_stream=cs)
    fresh = device_dest(SHAPES, L, T)
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, fresh, 2), buf, copy_stream=cs)
    torch.cuda.synchronize()
    for (c0, s0), (c1, s1), (c2, s2) in zip(before, full, fresh):
        assert torch.equal(c0, c1) and torch.equal(s0, s1)
        assert (c2[:2] == CANARY).all() and (s2[:2] == CANARY).all()
        assert torch.equal(c0[2:], c2[2:]) and torch.equal(s0[2:], s2[2:])
    assert_same(full, oracle_load(sources, excluded, SHAPES, L, T), "full")


@pytest.mark.parametrize("flags", [dict(bf16_intermediate=True), dict(scale_rule="uos")])
def test_layerwise_load_flags(mx, flags):
    """The requant flags reach the kernel: the bf16 intermediate and the UOS
    scale rule, against the oracle's load under the same reading."""
    L, T = 2, 5
    say(f"layerwise load flags {flags}")
    sources, excluded = build_case(SHAPES, L, T, 2, seed=31)
    dest = device_dest(SHAPES, L, T)
    buf = torch.empty(one_layer_bytes(SHAPES, T), dtype=torch.uint8, device=dev())
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, dest), buf,
                                      copy_stream=torch.cuda.Stream(dev()), **flags)
    torch.cuda.synchronize()
    kw = dict(flags_bf16=flags.get("bf16_intermediate", False),
              scale_rule=flags.get("scale_rule", "ocp"))
    assert_same(dest, oracle_load(sources, excluded, SHAPES, L, T, **kw), str(flags))


def test_layerwise_load_expert_shapes(mx):
    """One layer of the MoE expert shapes at reduced expert count: 6 experts of
    [2048, 4096] and [4096, 1024] (the benchmark's layer shapes), one excluded
    in each kind, the scratch one layer."""
    shapes = [(2048, 4096), (4096, 1024)]
    L, T = 1, 6
    say("layerwise load, expert shapes")
    pool = make_pool(shapes, T, 1, seed=41)
    sources = [pool[0]]
    excluded = np.zeros((L, 2, T), bool)
    excluded[0, 0, 2] = excluded[0, 1, 5] = True
    dest = device_dest(shapes, L, T)
    buf = torch.empty(one_layer_bytes(shapes, T), dtype=torch.uint8, device=dev())
    mx.mxfp4_requant_layers_from_host(parts_for(sources, excluded, dest), buf,
                                      copy_stream=torch.cuda.Stream(dev()))
    torch.cuda.synchronize()
    assert_same(dest, oracle_load(sources, excluded, shapes, L, T), "expert shapes")
