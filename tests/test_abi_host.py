"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
function include/mxfp4.h declares, and rejects malformed arguments before
anything would be launched.  No compute call is made."""
import ctypes
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "mxfp4.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import w4a4_mxfp4_gemm_amd as m
    return m.library()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("mxfp4_requant_from_nvfp4", "mxfp4_quantize_act", "mxfp4_gemm",
              "mxfp4_grouped_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import w4a4_mxfp4_gemm_amd as m
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in m.EXPORTED_SYMBOLS
    assert m.LIBRARY_PATH.exists()


def test_status_strings_and_version(lib):
    import w4a4_mxfp4_gemm_amd as m
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(m.mxfp4_status_string(s), str) and m.mxfp4_status_string(s)
    assert m.mxfp4_version() >= 100
    assert m.mxfp4_gemm_workspace_size(64, 12288, 4096) == 0


# Arguments that are rejected before any HIP call (so these run without a GPU).
FAKE = 0x1000            # 16-byte aligned, never dereferenced
ODD = 0x1001


def call_gemm(lib, **kw):
    a = dict(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, M=16, N=16, K=64, y=FAKE, dt=0,
             ws=None, wsb=0, flags=0)
    a.update(kw)
    return lib.mxfp4_gemm(a["a"], a["sa"], a["b"], a["sb"], a["M"], a["N"], a["K"], a["y"],
                          a["dt"], a["ws"], a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=48), -1), (dict(K=0), -1), (dict(K=-32), -1), (dict(N=0), -1), (dict(M=-1), -1),
    (dict(dt=2), -1), (dict(flags=1), -1), (dict(wsb=64), -1), (dict(a=None), -1),
    (dict(y=None), -1), (dict(a=ODD), -2), (dict(b=ODD), -2), (dict(y=ODD), -2),
    (dict(M=0), 0),
])
def test_gemm_argument_checks(lib, kw, status):
    assert call_gemm(lib, **kw) == status


def test_grouped_gemm_argument_checks(lib):
    f = lib.mxfp4_grouped_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 32, 64, FAKE, 0, None, 0, 0, None]
    bad_e = list(args); bad_e[5] = 0
    assert f(*bad_e) == -1
    no_off = list(args); no_off[4] = None
    assert f(*no_off) == -1
    odd_off = list(args); odd_off[4] = ODD
    assert f(*odd_off) == -2
    empty = list(args); empty[6] = 0
    assert f(*empty) == 0
    badk = list(args); badk[8] = 40
    assert f(*badk) == -1


def test_quantize_act_argument_checks(lib):
    f = lib.mxfp4_quantize_act
    assert f(FAKE, 32, None, 4, 64, FAKE, FAKE, 0, None) == -1           # ldx < K
    assert f(FAKE, 64, None, 4, 48, FAKE, FAKE, 0, None) == -1           # K % 32
    assert f(FAKE, 64, None, 4, 64, FAKE, FAKE, 1, None) == -1           # flags
    assert f(FAKE, 64, None, 4, 64, FAKE, FAKE, 4, None) == -1
    assert f(FAKE, 64, None, 0, 64, FAKE, FAKE, 2, None) == 0            # UOS accepted
    assert f(FAKE, 68, None, 4, 64, FAKE, FAKE, 0, None) == -2           # ldx % 8
    assert f(ODD, 64, None, 4, 64, FAKE, FAKE, 0, None) == -2            # x alignment
    assert f(FAKE, 64, ODD, 4, 64, FAKE, FAKE, 0, None) == -2            # row_index
    assert f(None, 64, None, 4, 64, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, 64, None, 0, 64, FAKE, FAKE, 0, None) == 0            # M == 0


def test_requant_argument_checks(lib):
    f = lib.mxfp4_requant_from_nvfp4
    assert f(FAKE, FAKE, FAKE, 1, 16, 48, FAKE, FAKE, 0, None) == -1     # K % 32
    assert f(FAKE, FAKE, FAKE, 1, 16, 64, FAKE, FAKE, 4, None) == -1     # flags
    # the two known flags pass the flag check and reach the next one
    assert f(None, FAKE, FAKE, 1, 16, 64, FAKE, FAKE, 3, None) == -1     # null source
    assert f(FAKE, FAKE, FAKE, 0, 16, 64, FAKE, FAKE, 3, None) == 0      # T == 0
    assert f(FAKE, FAKE, FAKE, 1, 0, 64, FAKE, FAKE, 0, None) == -1      # N
    assert f(None, FAKE, FAKE, 1, 16, 64, FAKE, FAKE, 0, None) == -1
    assert f(ODD, FAKE, FAKE, 1, 16, 64, FAKE, FAKE, 0, None) == -2
    assert f(FAKE, ODD, FAKE, 1, 16, 64, FAKE, FAKE, 0, None) == -2      # u16 scale loads
    assert f(FAKE, FAKE, FAKE, 0, 16, 64, FAKE, FAKE, 0, None) == 0      # T == 0


def test_requant_subset_argument_checks(lib):
    f = lib.mxfp4_requant_from_nvfp4_subset
    ok = (ctypes.c_int32 * 3)(0, 2, 5)
    bad_order = (ctypes.c_int32 * 3)(0, 2, 2)
    bad_range = (ctypes.c_int32 * 2)(0, 6)
    negative = (ctypes.c_int32 * 1)(-1)
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(bad_order), 3, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(bad_range), 2, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(negative), 1, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, None, 3, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(ok), -1, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, FAKE, FAKE, 6, 16, 48, P(ok), 3, FAKE, FAKE, 0, None) == -1      # K % 32
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(ok), 3, FAKE, FAKE, 4, None) == -1      # flags
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(ok), 0, FAKE, FAKE, 3, None) == 0       # both flags
    assert f(ODD, FAKE, FAKE, 6, 16, 64, P(ok), 3, FAKE, FAKE, 0, None) == -2
    assert f(FAKE, FAKE, FAKE, 6, 16, 64, P(ok), 0, FAKE, FAKE, 0, None) == 0       # empty list


def test_linear_argument_checks(lib):
    f = lib.mxfp4_linear_bf16
    #        x    ldx  M  N    K     b_codes b_scales bias y  dtype ws  ws_bytes flags stream
    assert f(FAKE, 4000, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1   # ldx < K
    assert f(FAKE, 4096, 1, 256, 4080, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1   # K % 32
    assert f(FAKE, 4096, 1, 0, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1      # N
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 7, None, 0, 0, None) == -1    # out_dtype
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 1, None) == -1    # flags
    assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 2, None) == 0     # UOS
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 64, 0, None) == -1   # ws NULL
    assert f(None, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1
    assert f(ODD, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -2
    assert f(FAKE, 4100, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -2    # ldx % 8
    assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == 0     # M == 0
    # the two-launch form needs its workspace
    assert f(FAKE, 1024, 200, 256, 1024, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1
    # a misaligned bias is refused before anything is launched
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, ODD, FAKE, 0, None, 0, 0, None) == -2
    assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE, FAKE, FAKE, 0, None, 0, 0, None) == 0


def test_linear_workspace_size(lib):
    ws = lib.mxfp4_linear_workspace_size
    assert ws(1, 12288, 4096) == 0 and ws(16, 4096, 2048) == 0           # one launch
    assert ws(17, 512, 4096) == (17 * 2048 + 255) // 256 * 256 + 17 * 128
    assert ws(65, 512, 4096) == (65 * 2048 + 255) // 256 * 256 + 65 * 128
    assert ws(8, 256, 1024) == (8 * 512 + 255) // 256 * 256 + 8 * 32     # K = 1024
    assert ws(0, 256, 1024) == 0 and ws(8, 256, 48) == 0                 # nothing to run


def test_silu_mul_quantize_argument_checks(lib):
    f = lib.mxfp4_silu_mul_quantize
    #        gate_up ldg  M  I    codes scales flags stream
    assert f(FAKE, 256, 4, 80, FAKE, FAKE, 0, None) == -1     # I % 32
    assert f(FAKE, 120, 4, 64, FAKE, FAKE, 0, None) == -1     # ldg < 2I
    assert f(FAKE, 128, 4, 64, FAKE, FAKE, 1, None) == -1     # flags
    assert f(FAKE, 128, -1, 64, FAKE, FAKE, 0, None) == -1    # M
    assert f(None, 128, 4, 64, FAKE, FAKE, 0, None) == -1
    assert f(FAKE, 128, 4, 64, None, FAKE, 0, None) == -1
    assert f(ODD, 128, 4, 64, FAKE, FAKE, 0, None) == -2      # gate_up alignment
    assert f(FAKE, 132, 4, 64, FAKE, FAKE, 0, None) == -2     # ldg % 8
    assert f(FAKE, 128, 4, 64, ODD, FAKE, 0, None) == -2      # codes alignment
    assert f(FAKE, 128, 0, 64, FAKE, FAKE, 2, None) == 0      # M == 0, UOS accepted


def test_quantize_act_scatter_argument_checks(lib):
    f = lib.mxfp4_quantize_act_scatter
    def g(x=FAKE, ldx=64, T=4, K=64, dest=FAKE, fan=2, R=8, c=FAKE, sc=FAKE, flags=0):
        return f(x, ldx, T, K, dest, fan, R, c, sc, flags, None)
    assert g(K=48) == -1                 # K % 32
    assert g(ldx=32) == -1               # ldx < K
    assert g(fan=0) == -1
    assert g(fan=70000) == -1
    assert g(R=0) == -1
    assert g(T=-1) == -1
    assert g(flags=1) == -1
    assert g(dest=None) == -1
    assert g(x=None) == -1
    assert g(ldx=68) == -2               # ldx % 8
    assert g(x=ODD) == -2
    assert g(dest=ODD) == -2
    assert g(c=ODD) == -2
    assert g(T=0, flags=2) == 0          # nothing to do; UOS accepted


def test_grouped_gemm_silu_quantize_argument_checks(lib):
    """Every rejected call returns before a launch (the pointers are fake)."""
    f = lib.mxfp4_grouped_gemm_silu_quantize
    def g(a=FAKE, sa=FAKE, b=FAKE, sb=FAKE, off=FAKE, E=4, M=64, I=64, K=512, hc=FAKE,
          hs=FAKE, flags=0):
        return f(a, sa, b, sb, off, E, M, I, K, hc, hs, flags, None)
    assert g(E=0) == -1
    assert g(M=-1) == -1
    assert g(I=80) == -1                 # I % 32
    assert g(I=0) == -1
    assert g(K=48) == -1                 # K % 32
    assert g(flags=1) == -1
    assert g(flags=8) == -1             # 4 is MXFP4_B_PRESHUFFLED
    assert g(off=None) == -1
    assert g(hs=None) == -1
    assert g(a=ODD) == -2
    assert g(hc=ODD) == -2               # 16-byte code stores
    assert g(off=ODD) == -2
    assert g(K=544) == -3                # the tiled kernel needs K % 512 == 0
    assert g(sa=ODD) == -3               # ... and 4-byte aligned scales
    assert g(E=4096) == -3               # more experts than its table holds
    assert g(M=0, flags=2) == 0          # nothing to do; UOS accepted


def test_moe_combine_argument_checks(lib):
    f = lib.mxfp4_moe_combine
    #        y    ldy  R   rows weights T  topk H    out  dtype flags stream
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 8, 60, FAKE, 0, 0, None) == -1    # H % 8
    assert f(FAKE, 56, 16, FAKE, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -1    # ldy < H
    assert f(FAKE, 64, 0, FAKE, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -1     # R
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 0, 64, FAKE, 0, 0, None) == -1    # topk
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 65, 64, FAKE, 0, 0, None) == -1   # topk > 64
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 8, 64, FAKE, 5, 0, None) == -1    # out dtype
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 8, 64, FAKE, 0, 1, None) == -1    # flags
    assert f(FAKE, 64, 16, None, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -1    # rows
    assert f(ODD, 64, 16, FAKE, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -2
    assert f(FAKE, 68, 16, FAKE, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -2    # ldy % 8
    assert f(FAKE, 64, 16, FAKE, FAKE, 2, 8, 64, FAKE + 8, 0, 0, None) == -2  # out
    assert f(FAKE, 64, 16, ODD, FAKE, 2, 8, 64, FAKE, 0, 0, None) == -2     # rows
    assert f(FAKE, 64, 16, FAKE, FAKE, 0, 8, 64, FAKE, 1, 0, None) == 0     # T == 0


def test_w4a8_argument_checks(lib):
    q = lib.mxfp8_quantize_act
    assert q(FAKE, 32, None, 4, 64, FAKE, FAKE, 0, None) == -1           # ldx < K
    assert q(FAKE, 64, None, 4, 48, FAKE, FAKE, 0, None) == -1           # K % 32
    assert q(FAKE, 64, None, 4, 64, FAKE, FAKE, 2, None) == -1           # flags (no UOS)
    assert q(FAKE, 68, None, 4, 64, FAKE, FAKE, 0, None) == -2           # ldx % 8
    assert q(FAKE, 64, None, 4, 64, ODD, FAKE, 0, None) == -2            # codes alignment
    assert q(FAKE, 64, None, 0, 64, FAKE, FAKE, 0, None) == 0            # M == 0
    g = lib.mxfp4_gemm_w4a8
    #        a     sa    b     sb    M  N   K   bias  y     dt flags stream
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 48, None, FAKE, 0, 0, None) == -1    # K % 32
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 64, None, FAKE, 3, 0, None) == -1    # out dtype
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 64, None, FAKE, 0, 1, None) == -1    # flags
    assert g(None, FAKE, FAKE, FAKE, 4, 16, 64, None, FAKE, 0, 0, None) == -1
    assert g(ODD, FAKE, FAKE, FAKE, 4, 16, 64, None, FAKE, 0, 0, None) == -2
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 16, 64, ODD, FAKE, 0, 0, None) == -2     # bias
    assert g(FAKE, FAKE, FAKE, FAKE, 0, 16, 64, None, FAKE, 0, 0, None) == 0     # M == 0
    f = lib.mxfp4_linear_w4a8_bf16
    assert f(FAKE, 4096, 17, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == -1  # ws
    assert f(FAKE, 4096, 8, 256, 4096, FAKE, FAKE, None, FAKE, 0, FAKE, 1 << 20, 1,
             None) == -1                                                           # flags
    assert f(FAKE, 4096, 8, 256, 4096, FAKE, FAKE, ODD, FAKE, 0, FAKE, 1 << 20, 0,
             None) == -2                                                           # bias
    assert f(FAKE, 4096, 17, 256, 4096, FAKE, FAKE, None, FAKE, 0, ODD, 1 << 20, 0,
             None) == -2                                                           # ws align
    assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE, None, FAKE, 0, None, 0, 0, None) == 0
    ws = lib.mxfp4_linear_w4a8_workspace_size
    assert ws(8, 256, 4096) == 0                    # one launch: no workspace
    assert ws(17, 256, 4096) == 17 * 4096 + 17 * 128
    assert ws(3, 256, 96) == 512 + 9


def test_smooth_quantize_argument_checks(lib):
    for name, good_flag in (("mxfp4_quantize_act_smooth", 2), ("mxfp8_quantize_act_smooth", 0)):
        f = getattr(lib, name)
        #        x     ldx  ri    smooth M  K   codes scales flags stream
        assert f(FAKE, 64, None, FAKE, 4, 48, FAKE, FAKE, 0, None) == -1       # K % 32
        assert f(FAKE, 64, None, None, 4, 64, FAKE, FAKE, 0, None) == -1       # smooth NULL
        assert f(FAKE, 64, None, ODD, 4, 64, FAKE, FAKE, 0, None) == -2        # smooth align
        assert f(FAKE, 64, None, FAKE, 4, 64, FAKE, FAKE, 4, None) == -1       # flags
        assert f(FAKE, 64, None, FAKE, 0, 64, FAKE, FAKE, good_flag, None) == 0
    assert lib.mxfp8_quantize_act_smooth(FAKE, 64, None, FAKE, 4, 64, FAKE, FAKE, 2, None) == -1


def test_linear_weight_scales_must_be_16_byte_aligned(lib):
    """Both linear calls pick the one-launch form by shape alone, so they need
    the alignment that form needs from every caller: b_scales 16-byte aligned
    (else EALIGN before anything is launched), and the workspace query is
    exact for every call it accepts."""
    for f in (lib.mxfp4_linear_bf16, lib.mxfp4_linear_w4a8_bf16):
        for M in (1, 200):                                # one-launch and two-launch shapes
            assert f(FAKE, 4096, M, 256, 4096, FAKE, FAKE + 4, None, FAKE, 0, FAKE, 1 << 24, 0,
                     None) == -2
            assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE + 4, None, FAKE, 0, None, 0, 0,
                     None) == 0
    g = lib.mxfp4_linear_bf16_noalloc
    assert g(FAKE, 4096, 1, 256, 4096, FAKE, FAKE + 4, None, FAKE, 0, 0, None) == -2


def test_noalloc_linear_argument_checks(lib):
    f = lib.mxfp4_linear_bf16_noalloc
    #        x     ldx   M  N    K     b_codes b_scales bias y  dtype flags stream
    assert f(FAKE, 4000, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, 0, None) == -1    # ldx < K
    assert f(FAKE, 4096, 1, 256, 4080, FAKE, FAKE, None, FAKE, 0, 0, None) == -1    # K % 32
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 7, 0, None) == -1    # out_dtype
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, 1, None) == -1    # flags
    assert f(None, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, 0, None) == -1
    assert f(ODD, 4096, 1, 256, 4096, FAKE, FAKE, None, FAKE, 0, 0, None) == -2
    assert f(FAKE, 4096, 1, 256, 4096, FAKE, FAKE, ODD, FAKE, 0, 0, None) == -2     # bias
    assert f(FAKE, 4096, 0, 256, 4096, FAKE, FAKE, None, FAKE, 0, 2, None) == 0     # M == 0
    # one row past what the static scratch holds at K = 14336: MXFP4_ESCRATCH,
    # decided before any HIP call
    K = 14336
    M = (32 << 20) // (K // 2 + K // 32) + 1
    assert lib.mxfp4_linear_workspace_size(M, 256, K) > (32 << 20)
    assert lib.mxfp4_linear_workspace_size(M - 1, 256, K) <= (32 << 20)
    assert f(FAKE, K, M, 256, K, FAKE, FAKE, None, FAKE, 0, 0, None) == -5
    import w4a4_mxfp4_gemm_amd as m
    assert "scratch" in m.mxfp4_status_string(-5)
    assert m.MXFP4_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_layerwise_argument_checks(lib):
    import w4a4_mxfp4_gemm_amd as m
    parts = (m.LoadPart * 2)()
    for p, (T, N, K) in zip(parts, ((4, 64, 128), (0, 32, 64))):
        p.T, p.N, p.K = T, N, K
        p.nv_codes = p.nv_scales = p.nv_global = p.mx_codes = p.mx_scales = FAKE
    P = ctypes.cast(parts, ctypes.c_void_p)
    n = ctypes.c_int64(0)
    plan = lib.mxfp4_layerwise_plan
    assert plan(P, 2, 1 << 20, None, 0, ctypes.byref(n), None) == 0 and n.value == 1
    assert plan(P, 2, 1 << 20, None, 0, None, None) == -1                 # no count
    assert plan(P, -1, 1 << 20, None, 0, ctypes.byref(n), None) == -1
    assert plan(P, 2, 1024, None, 0, ctypes.byref(n), None) == -1          # slot < one tensor
    chunks = (m.LoadChunk * 1)()
    assert plan(P, 2, 1 << 20, ctypes.cast(chunks, ctypes.c_void_p), 0, ctypes.byref(n),
                None) == -1                                                # max_chunks too small
    parts[0].K = 48
    assert plan(P, 2, 1 << 20, None, 0, ctypes.byref(n), None) == -1      # K % 32
    parts[0].K = 128
    run = lib.mxfp4_requant_layers_from_host
    assert run(P, 2, FAKE, 1 << 20, 4, None, None) == -1                   # flags
    assert run(P, 2, None, 1 << 20, 0, None, None) == -1                   # no scratch
    assert run(P, 2, FAKE + 16, 1 << 20, 0, None, None) == -2              # scratch alignment
    assert run(P, 2, FAKE, 1024, 0, None, None) == -1                      # scratch too small
    parts[0].mx_codes = ODD
    assert run(P, 2, FAKE, 1 << 20, 0, None, None) == -2                   # destination alignment
    parts[0].mx_codes = FAKE
    parts[0].nv_global = None
    assert run(P, 2, FAKE, 1 << 20, 0, None, None) == -1                   # a null source
    parts[0].T = 0
    assert run(P, 2, None, 0, 0, None, None) == 0                          # nothing to load


def test_preshuffle_argument_checks(lib):
    f = lib.mxfp4_preshuffle_weights
    #         codes out        T  N   K
    assert f(FAKE, FAKE + 4096, 1, 48, 256, None) == -1          # N % 32
    assert f(FAKE, FAKE + 4096, 1, 32, 384, None) == -1          # K % 256
    assert f(FAKE, FAKE + 4096, -1, 32, 256, None) == -1
    assert f(None, FAKE + 4096, 1, 32, 256, None) == -1
    assert f(FAKE, FAKE + 2048, 1, 32, 256, None) == -1          # overlapping (4 KiB each)
    assert f(FAKE, FAKE, 1, 32, 256, None) == -1                 # in place
    assert f(ODD, FAKE + 8192, 1, 32, 256, None) == -2
    assert f(FAKE, FAKE + 4104, 1, 32, 256, None) == -2          # out alignment
    assert f(FAKE, FAKE, 0, 32, 256, None) == 0                  # nothing to do


def test_grouped_preshuffled_needs_the_register_streamed_kernel(lib):
    """MXFP4_B_PRESHUFFLED is refused (before any launch) where the kernel
    that reads that layout does not run: K % 1024 != 0 or N % 32 != 0."""
    import w4a4_mxfp4_gemm_amd as m
    F = m.MXFP4_B_PRESHUFFLED
    g = lib.mxfp4_grouped_gemm
    #        a     sa    b     sb    off   E  M   N    K     y     dt ws  wsb flags
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 256, 1536, FAKE, 0, None, 0, F, None) == -3
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 240, 1024, FAKE, 0, None, 0, F, None) == -3
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 256, 1024, FAKE, 0, None, 0, 8, None) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 256, 1536, FAKE, 0, None, 0, F, None) == 0
    h = lib.mxfp4_grouped_gemm_silu_quantize
    #        a     sa    b     sb    off   E  M   I    K     hc    hs    flags
    assert h(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 1536, FAKE, FAKE, F, None) == -3
    assert h(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 1536, FAKE, FAKE, F | 2, None) == 0
