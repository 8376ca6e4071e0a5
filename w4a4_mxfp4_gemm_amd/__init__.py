"""Python binding of the gfx950 MXFP4 library (``libmxfp4_cdna4.so``).

The functions below carry the C ABI's names (``include/mxfp4.h``) and do
argument marshalling only: torch tensors supply device memory, the current
torch stream supplies the HIP stream, and every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the shared library is
missing and cannot be built, importing this package raises.
"""
from __future__ import annotations

import ctypes
import pathlib

import torch

_PKG = pathlib.Path(__file__).resolve().parent
LIBRARY_PATH = _PKG / "libmxfp4_cdna4.so"

MXFP4_OUT_BF16 = 0
MXFP4_OUT_FP32 = 1
MXFP4_REQ_INTERMEDIATE_BF16 = 1
MXFP4_SCALE_UOS = 2
MXFP4_B_PRESHUFFLED = 4

_STATUS_NAMES = {0: "MXFP4_OK", -1: "MXFP4_EINVAL", -2: "MXFP4_EALIGN",
                 -3: "MXFP4_EUNSUPPORTED", -4: "MXFP4_EHIP", -5: "MXFP4_ESCRATCH"}

MXFP4_NOALLOC_SCRATCH_BYTES = 32 << 20


class Mxfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_STATUS_NAMES.get(status, status)} "
                         f"({mxfp4_status_string(status)})")


def _load_library() -> ctypes.CDLL:
    if not LIBRARY_PATH.exists():
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(str(LIBRARY_PATH))
    P, I, U32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    lib.mxfp4_requant_from_nvfp4.argtypes = [P, P, P, I, I, I, P, P, U32, P]
    lib.mxfp4_requant_from_nvfp4.restype = ctypes.c_int
    lib.mxfp4_requant_from_nvfp4_subset.argtypes = [P, P, P, I, I, I, P, I, P, P, U32, P]
    lib.mxfp4_requant_from_nvfp4_subset.restype = ctypes.c_int
    lib.mxfp4_quantize_act.argtypes = [P, I, P, I, I, P, P, U32, P]
    lib.mxfp4_quantize_act.restype = ctypes.c_int
    lib.mxfp4_gemm.argtypes = [P, P, P, P, I, I, I, P, ctypes.c_int, P, SZ, U32, P]
    lib.mxfp4_gemm.restype = ctypes.c_int
    lib.mxfp4_grouped_gemm.argtypes = [P, P, P, P, P, I, I, I, I, P, ctypes.c_int, P, SZ, U32, P]
    lib.mxfp4_grouped_gemm.restype = ctypes.c_int
    lib.mxfp4_linear_bf16.argtypes = [P, I, I, I, I, P, P, P, P, ctypes.c_int, P, SZ, U32, P]
    lib.mxfp4_linear_bf16.restype = ctypes.c_int
    lib.mxfp4_quantize_act_scatter.argtypes = [P, I, I, I, P, I, I, P, P, U32, P]
    lib.mxfp4_quantize_act_scatter.restype = ctypes.c_int
    lib.mxfp4_quantize_act_smooth.argtypes = [P, I, P, P, I, I, P, P, U32, P]
    lib.mxfp4_quantize_act_smooth.restype = ctypes.c_int
    lib.mxfp8_quantize_act_smooth.argtypes = [P, I, P, P, I, I, P, P, U32, P]
    lib.mxfp8_quantize_act_smooth.restype = ctypes.c_int
    lib.mxfp8_quantize_act.argtypes = [P, I, P, I, I, P, P, U32, P]
    lib.mxfp8_quantize_act.restype = ctypes.c_int
    lib.mxfp4_gemm_w4a8.argtypes = [P, P, P, P, I, I, I, P, P, ctypes.c_int, U32, P]
    lib.mxfp4_gemm_w4a8.restype = ctypes.c_int
    lib.mxfp4_linear_w4a8_bf16.argtypes = [P, I, I, I, I, P, P, P, P, ctypes.c_int, P, SZ, U32,
                                           P]
    lib.mxfp4_linear_w4a8_bf16.restype = ctypes.c_int
    lib.mxfp4_linear_w4a8_workspace_size.argtypes = [I, I, I]
    lib.mxfp4_linear_w4a8_workspace_size.restype = SZ
    lib.mxfp4_silu_mul_quantize.argtypes = [P, I, I, I, P, P, U32, P]
    lib.mxfp4_silu_mul_quantize.restype = ctypes.c_int
    lib.mxfp4_grouped_gemm_silu_quantize.argtypes = [P, P, P, P, P, I, I, I, I, P, P, U32, P]
    lib.mxfp4_grouped_gemm_silu_quantize.restype = ctypes.c_int
    lib.mxfp4_moe_combine.argtypes = [P, I, I, P, P, I, I, I, P, ctypes.c_int, U32, P]
    lib.mxfp4_moe_combine.restype = ctypes.c_int
    lib.mxfp4_linear_workspace_size.argtypes = [I, I, I]
    lib.mxfp4_linear_workspace_size.restype = SZ
    lib.mxfp4_gemm_workspace_size.argtypes = [I, I, I]
    lib.mxfp4_gemm_workspace_size.restype = SZ
    lib.mxfp4_layerwise_plan.argtypes = [P, I, SZ, P, I, ctypes.POINTER(ctypes.c_int64),
                                         ctypes.POINTER(ctypes.c_uint64)]
    lib.mxfp4_layerwise_plan.restype = ctypes.c_int
    lib.mxfp4_requant_layers_from_host.argtypes = [P, I, P, SZ, U32, P, P]
    lib.mxfp4_requant_layers_from_host.restype = ctypes.c_int
    lib.mxfp4_linear_bf16_noalloc.argtypes = [P, I, I, I, I, P, P, P, P, ctypes.c_int, U32, P]
    lib.mxfp4_linear_bf16_noalloc.restype = ctypes.c_int
    lib.mxfp4_preshuffle_weights.argtypes = [P, P, I, I, I, P]
    lib.mxfp4_preshuffle_weights.restype = ctypes.c_int
    lib.mxfp4_status_string.argtypes = [ctypes.c_int]
    lib.mxfp4_status_string.restype = ctypes.c_char_p
    lib.mxfp4_version.argtypes = []
    lib.mxfp4_version.restype = ctypes.c_int
    return lib


_lib = _load_library()

EXPORTED_SYMBOLS = ("mxfp4_requant_from_nvfp4", "mxfp4_requant_from_nvfp4_subset",
                    "mxfp4_quantize_act", "mxfp4_gemm",
                    "mxfp4_grouped_gemm", "mxfp4_linear_bf16", "mxfp4_gemm_workspace_size",
                    "mxfp4_linear_workspace_size", "mxfp4_silu_mul_quantize",
                    "mxfp4_moe_combine", "mxfp8_quantize_act", "mxfp4_gemm_w4a8",
                    "mxfp4_linear_w4a8_bf16", "mxfp4_linear_w4a8_workspace_size",
                    "mxfp4_quantize_act_smooth", "mxfp8_quantize_act_smooth",
                    "mxfp4_grouped_gemm_silu_quantize", "mxfp4_quantize_act_scatter",
                    "mxfp4_layerwise_plan", "mxfp4_requant_layers_from_host",
                    "mxfp4_linear_bf16_noalloc", "mxfp4_preshuffle_weights",
                    "mxfp4_status_string", "mxfp4_version")


def library() -> ctypes.CDLL:
    return _lib


def mxfp4_status_string(status: int) -> str:
    return _lib.mxfp4_status_string(int(status)).decode()


def mxfp4_version() -> int:
    return int(_lib.mxfp4_version())


def mxfp4_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(_lib.mxfp4_gemm_workspace_size(M, N, K))


# ---- marshalling helpers -------------------------------------------------------
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(fn, status):
    if status != 0:
        raise Mxfp4Error(fn, status)


def _rule_flag(scale_rule):
    if scale_rule == "ocp":
        return 0
    if scale_rule == "uos":
        return MXFP4_SCALE_UOS
    raise ValueError(f"scale_rule must be 'ocp' or 'uos', not {scale_rule!r}")


# ---- the four calls ---------------------------------------------------------------
def mxfp4_requant_from_nvfp4(nv_codes, nv_scales, nv_global, mx_codes=None, mx_scales=None,
                             *, bf16_intermediate=False, tensors=None, scale_rule="ocp",
                             stream=None):
    """NVFP4 ([T,]N,K/2 codes, [T,]N,K/16 E4M3 bytes, fp32 global [T]) -> MXFP4
    ([T,]N,K/2 codes, [T,]N,K/32 E8M0 bytes), written into mx_codes/mx_scales
    (allocated when None).  `tensors` (strictly increasing indices into the T
    tensors) converts only those, in one launch, leaving the other slots of
    the destination untouched.  scale_rule: "ocp" or "uos" (MXFP4_SCALE_UOS).
    Returns (mx_codes, mx_scales)."""
    _need(nv_codes, "nv_codes", torch.uint8)
    dev = nv_codes.device
    _need(nv_scales, "nv_scales", torch.uint8, dev)
    _need(nv_global, "nv_global", torch.float32, dev)
    lead = nv_codes.shape[:-2]
    N, K = nv_codes.shape[-2], nv_codes.shape[-1] * 2
    T = int(torch.tensor(lead).prod().item()) if len(lead) else 1
    if nv_scales.shape != (*lead, N, K // 16):
        raise ValueError(f"nv_scales shape {tuple(nv_scales.shape)} != {(*lead, N, K // 16)}")
    if nv_global.numel() != T:
        raise ValueError(f"nv_global has {nv_global.numel()} entries, expected {T}")
    if mx_codes is None:
        mx_codes = torch.empty((*lead, N, K // 2), dtype=torch.uint8, device=dev)
    if mx_scales is None:
        mx_scales = torch.empty((*lead, N, K // 32), dtype=torch.uint8, device=dev)
    _need(mx_codes, "mx_codes", torch.uint8, dev)
    _need(mx_scales, "mx_scales", torch.uint8, dev)
    if mx_codes.shape != (*lead, N, K // 2) or mx_scales.shape != (*lead, N, K // 32):
        raise ValueError("destination shapes do not match the source")
    flags = (MXFP4_REQ_INTERMEDIATE_BF16 if bf16_intermediate else 0) | _rule_flag(scale_rule)
    if tensors is not None:
        sel = [int(t) for t in tensors]
        arr = (ctypes.c_int32 * max(len(sel), 1))(*sel)
        _check("mxfp4_requant_from_nvfp4_subset", _lib.mxfp4_requant_from_nvfp4_subset(
            _ptr(nv_codes), _ptr(nv_scales), _ptr(nv_global), T, N, K,
            ctypes.cast(arr, ctypes.c_void_p), len(sel),
            _ptr(mx_codes), _ptr(mx_scales), flags, _stream(stream, dev)))
        return mx_codes, mx_scales
    _check("mxfp4_requant_from_nvfp4", _lib.mxfp4_requant_from_nvfp4(
        _ptr(nv_codes), _ptr(nv_scales), _ptr(nv_global), T, N, K,
        _ptr(mx_codes), _ptr(mx_scales), flags, _stream(stream, dev)))
    return mx_codes, mx_scales


class LoadPart(ctypes.Structure):
    """mxfp4_load_part of include/mxfp4.h."""
    _fields_ = [("nv_codes", ctypes.c_void_p), ("nv_scales", ctypes.c_void_p),
                ("nv_global", ctypes.c_void_p), ("excluded", ctypes.c_void_p),
                ("mx_codes", ctypes.c_void_p), ("mx_scales", ctypes.c_void_p),
                ("T", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class LoadChunk(ctypes.Structure):
    """mxfp4_load_chunk of include/mxfp4.h."""
    _fields_ = [("part", ctypes.c_int64), ("t0", ctypes.c_int64), ("t1", ctypes.c_int64),
                ("slot", ctypes.c_int64), ("codes_offset", ctypes.c_uint64),
                ("scales_offset", ctypes.c_uint64), ("global_offset", ctypes.c_uint64)]


def _excluded_u8(excluded, T):
    if excluded is None:
        return None
    e = torch.as_tensor(excluded).to("cpu").reshape(-1).to(torch.uint8).contiguous()
    if e.numel() != T:
        raise ValueError(f"excluded has {e.numel()} entries, expected {T}")
    return e


def mxfp4_layerwise_plan(shapes, excluded, scratch_bytes):
    """The layerwise load's plan (host code only, no GPU needed): shapes is a
    list of (T, N, K) per part, excluded a matching list of [T] masks (or
    None entries).  Returns (chunks, slot_bytes) with each chunk a dict of
    part, t0, t1, slot, codes_offset, scales_offset, global_offset."""
    keep = [_excluded_u8(e, int(T)) for (T, _, _), e in zip(shapes, excluded)]
    parts = (LoadPart * max(len(shapes), 1))()
    for i, ((T, N, K), e) in enumerate(zip(shapes, keep)):
        parts[i].T, parts[i].N, parts[i].K = int(T), int(N), int(K)
        parts[i].excluded = None if e is None else e.data_ptr()
    n = ctypes.c_int64(0)
    slot = ctypes.c_uint64(0)
    _check("mxfp4_layerwise_plan", _lib.mxfp4_layerwise_plan(
        ctypes.cast(parts, ctypes.c_void_p), len(shapes), int(scratch_bytes), None, 0,
        ctypes.byref(n), ctypes.byref(slot)))
    chunks = (LoadChunk * max(n.value, 1))()
    _check("mxfp4_layerwise_plan", _lib.mxfp4_layerwise_plan(
        ctypes.cast(parts, ctypes.c_void_p), len(shapes), int(scratch_bytes),
        ctypes.cast(chunks, ctypes.c_void_p), n.value, ctypes.byref(n), ctypes.byref(slot)))
    out = [{f: int(getattr(chunks[i], f)) for f, _ in LoadChunk._fields_} for i in range(n.value)]
    return out, int(slot.value)


def mxfp4_requant_layers_from_host(parts, scratch, *, copy_stream=None, bf16_intermediate=False,
                                   scale_rule="ocp", stream=None):
    """The layerwise load: each part is a dict with nv_codes [T,N,K/2] u8,
    nv_scales [T,N,K/16] u8, nv_global [T] fp32 (CPU tensors, pinned for the
    copies to overlap), optional excluded [T] mask, and mx_codes [T,N,K/2],
    mx_scales [T,N,K/32] u8 GPU tensors written in place.  scratch: a u8 GPU
    tensor (256-byte aligned; one layer's NVFP4 bytes is enough).  The copies
    run on copy_stream (default: the compute stream), the requant on stream
    (default: the current stream).  The host tensors must stay alive until
    that stream has finished."""
    _need(scratch, "scratch", torch.uint8)
    dev = scratch.device
    keep = []
    arr = (LoadPart * max(len(parts), 1))()
    for i, p in enumerate(parts):
        c, sc, g = p["nv_codes"], p["nv_scales"], p["nv_global"]
        mc, ms = p["mx_codes"], p["mx_scales"]
        for t, name, dt in ((c, "nv_codes", torch.uint8), (sc, "nv_scales", torch.uint8),
                            (g, "nv_global", torch.float32)):
            if t.device.type != "cpu" or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"part {i}: {name} must be a contiguous CPU {dt} tensor")
        _need(mc, "mx_codes", torch.uint8, dev)
        _need(ms, "mx_scales", torch.uint8, dev)
        T, N, K = (int(torch.tensor(c.shape[:-2]).prod().item()) if c.dim() > 2 else 1,
                   c.shape[-2], c.shape[-1] * 2)
        if (sc.numel() != T * N * (K // 16) or g.numel() != T or mc.numel() != T * N * (K // 2)
                or ms.numel() != T * N * (K // 32)):
            raise ValueError(f"part {i}: shapes do not match codes [{T},{N},{K // 2}]")
        e = _excluded_u8(p.get("excluded"), T)
        keep.append(e)
        arr[i].nv_codes, arr[i].nv_scales, arr[i].nv_global = (c.data_ptr(), sc.data_ptr(),
                                                                g.data_ptr())
        arr[i].excluded = None if e is None else e.data_ptr()
        arr[i].mx_codes, arr[i].mx_scales = mc.data_ptr(), ms.data_ptr()
        arr[i].T, arr[i].N, arr[i].K = T, N, K
    flags = (MXFP4_REQ_INTERMEDIATE_BF16 if bf16_intermediate else 0) | _rule_flag(scale_rule)
    s = _stream(stream, dev)
    cs = s if copy_stream is None else _stream(copy_stream, dev)
    _check("mxfp4_requant_layers_from_host", _lib.mxfp4_requant_layers_from_host(
        ctypes.cast(arr, ctypes.c_void_p), len(parts), _ptr(scratch), scratch.numel(), flags,
        cs, s))


def mxfp4_quantize_act(x, codes=None, scales=None, *, row_index=None, K=None,
                       scale_rule="ocp", stream=None):
    """bf16 x [R, ldx] -> MXFP4 codes [M, K/2] and E8M0 bytes [M, K/32] where
    M = R, or len(row_index) with output row i taken from x[row_index[i]].
    K defaults to x's row length; x may have extra columns (ldx >= K).
    scale_rule: "ocp" or "uos"."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, ldx]")
    ldx = x.shape[1]
    K = ldx if K is None else int(K)
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, dev)
        M = row_index.shape[0]
    else:
        M = x.shape[0]
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (M, K // 2) or scales.shape != (M, K // 32):
        raise ValueError("output shapes do not match [M, K/2] / [M, K/32]")
    _check("mxfp4_quantize_act", _lib.mxfp4_quantize_act(
        _ptr(x), ldx, _ptr(row_index), M, K, _ptr(codes), _ptr(scales), _rule_flag(scale_rule),
        _stream(stream, dev)))
    return codes, scales


def _out_dtype(dtype):
    if dtype == torch.bfloat16:
        return MXFP4_OUT_BF16
    if dtype == torch.float32:
        return MXFP4_OUT_FP32
    raise TypeError("out dtype must be torch.bfloat16 or torch.float32")


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, y=None, *, out_dtype=torch.bfloat16,
               stream=None):
    """y [M, N] = A [M, K] * B [N, K]^T over MXFP4 operands."""
    _need(a_codes, "a_codes", torch.uint8)
    dev = a_codes.device
    for t, n in ((a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _need(t, n, torch.uint8, dev)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if b_codes.shape != (N, K // 2) or a_scales.shape != (M, K // 32) or \
            b_scales.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _need(y, "y", y.dtype, dev)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    _check("mxfp4_gemm", _lib.mxfp4_gemm(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
        _ptr(y), _out_dtype(y.dtype), None, 0, 0, _stream(stream, dev)))
    return y


def mxfp4_linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(_lib.mxfp4_linear_workspace_size(M, N, K))


def mxfp4_linear_bf16(x, b_codes, b_scales, y=None, *, bias=None, K=None,
                      out_dtype=torch.bfloat16, workspace=None, scale_rule="ocp", stream=None):
    """y [M, N] = MXFP4(x) [M, K] * B [N, K]^T from bf16 x [M, ldx] (the act-quant
    call followed by the GEMM, bit for bit; one launch for decode shapes).  K
    defaults to x's row length.  A workspace of mxfp4_linear_workspace_size
    bytes is allocated when none is given and one is needed.  bias: bf16 [N],
    added to each fp32 sum before the output rounding.  scale_rule: the
    activations' rule, "ocp" or "uos"."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(b_codes, "b_codes", torch.uint8, dev)
    _need(b_scales, "b_scales", torch.uint8, dev)
    if x.dim() != 2:
        raise ValueError("x must be [M, ldx]")
    M, ldx = x.shape
    K = ldx if K is None else K
    N = b_codes.shape[0]
    if b_codes.shape != (N, K // 2) or b_scales.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _need(y, "y", y.dtype, dev)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    need = mxfp4_linear_workspace_size(M, N, K)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    _check("mxfp4_linear_bf16", _lib.mxfp4_linear_bf16(
        _ptr(x), ldx, M, N, K, _ptr(b_codes), _ptr(b_scales), _ptr(bias), _ptr(y),
        _out_dtype(y.dtype),
        ws_ptr, ws_bytes, _rule_flag(scale_rule), _stream(stream, dev)))
    return y


def mxfp4_linear_bf16_noalloc(x, b_codes, b_scales, y, *, bias=None, K=None, scale_rule="ocp",
                              stream=None):
    """mxfp4_linear_bf16 without a workspace: the library's static per-GPU
    scratch (MXFP4_NOALLOC_SCRATCH_BYTES) holds the quantized activations.
    y [M, N] (bf16 or fp32) is the caller's; nothing is allocated."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(b_codes, "b_codes", torch.uint8, dev)
    _need(b_scales, "b_scales", torch.uint8, dev)
    if x.dim() != 2:
        raise ValueError("x must be [M, ldx]")
    M, ldx = x.shape
    K = ldx if K is None else K
    N = b_codes.shape[0]
    if b_codes.shape != (N, K // 2) or b_scales.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev)
        if bias.shape != (N,):
            raise ValueError("bias must be [N]")
    _need(y, "y", y.dtype, dev)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    _check("mxfp4_linear_bf16_noalloc", _lib.mxfp4_linear_bf16_noalloc(
        _ptr(x), ldx, M, N, K, _ptr(b_codes), _ptr(b_scales), _ptr(bias), _ptr(y),
        _out_dtype(y.dtype), _rule_flag(scale_rule), _stream(stream, dev)))
    return y


def _quantize_smooth(fn, elem_cols, x, smooth, codes, scales, row_index, K, flags, stream):
    _need(x, "x", torch.bfloat16)
    dev = x.device
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, ldx]")
    ldx = x.shape[1]
    K = ldx if K is None else int(K)
    _need(smooth, "smooth", torch.bfloat16, dev)
    if smooth.shape != (K,):
        raise ValueError("smooth must be [K]")
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, dev)
        M = row_index.shape[0]
    else:
        M = x.shape[0]
    if codes is None:
        codes = torch.empty((M, elem_cols(K)), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (M, elem_cols(K)) or scales.shape != (M, K // 32):
        raise ValueError("output shapes do not match")
    _check(fn, getattr(_lib, fn)(_ptr(x), ldx, _ptr(row_index), _ptr(smooth), M, K, _ptr(codes),
                                 _ptr(scales), flags, _stream(stream, dev)))
    return codes, scales


def mxfp4_quantize_act_smooth(x, smooth, codes=None, scales=None, *, row_index=None, K=None,
                              scale_rule="ocp", stream=None):
    """mxfp4_quantize_act of bf16(x * smooth) (smooth: bf16 [K])."""
    return _quantize_smooth("mxfp4_quantize_act_smooth", lambda k: k // 2, x, smooth, codes,
                            scales, row_index, K, _rule_flag(scale_rule), stream)


def mxfp8_quantize_act_smooth(x, smooth, codes=None, scales=None, *, row_index=None, K=None,
                              stream=None):
    """mxfp8_quantize_act of bf16(x * smooth) (smooth: bf16 [K])."""
    return _quantize_smooth("mxfp8_quantize_act_smooth", lambda k: k, x, smooth, codes, scales,
                            row_index, K, 0, stream)


def mxfp8_quantize_act(x, codes=None, scales=None, *, row_index=None, K=None, stream=None):
    """W4A8 activations: bf16 x [R, ldx] -> E4M3 codes [M, K] (one byte each) and
    E8M0 bytes [M, K/32]; M = R, or len(row_index) with row i from x[row_index[i]]."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, ldx]")
    ldx = x.shape[1]
    K = ldx if K is None else int(K)
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, dev)
        M = row_index.shape[0]
    else:
        M = x.shape[0]
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (M, K) or scales.shape != (M, K // 32):
        raise ValueError("output shapes do not match [M, K] / [M, K/32]")
    _check("mxfp8_quantize_act", _lib.mxfp8_quantize_act(
        _ptr(x), ldx, _ptr(row_index), M, K, _ptr(codes), _ptr(scales), 0, _stream(stream, dev)))
    return codes, scales


def _bias_arg(bias, N, dev):
    if bias is None:
        return None
    _need(bias, "bias", torch.bfloat16, dev)
    if bias.shape != (N,):
        raise ValueError("bias must be [N]")
    return bias


def mxfp4_gemm_w4a8(a_codes, a_scales, b_codes, b_scales, y=None, *, bias=None,
                    out_dtype=torch.bfloat16, stream=None):
    """W4A8: y [M, N] = A [M, K] (MXFP8) * B [N, K]^T (MXFP4) + bias."""
    _need(a_codes, "a_codes", torch.uint8)
    dev = a_codes.device
    for t, n in ((a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _need(t, n, torch.uint8, dev)
    M, K = a_codes.shape
    N = b_codes.shape[0]
    if b_codes.shape != (N, K // 2) or a_scales.shape != (M, K // 32) or \
            b_scales.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    bias = _bias_arg(bias, N, dev)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _need(y, "y", y.dtype, dev)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    _check("mxfp4_gemm_w4a8", _lib.mxfp4_gemm_w4a8(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _ptr(bias),
        _ptr(y), _out_dtype(y.dtype), 0, _stream(stream, dev)))
    return y


def mxfp4_linear_w4a8_workspace_size(M: int, N: int, K: int) -> int:
    return int(_lib.mxfp4_linear_w4a8_workspace_size(M, N, K))


def mxfp4_linear_w4a8_bf16(x, b_codes, b_scales, y=None, *, bias=None, K=None,
                           out_dtype=torch.bfloat16, workspace=None, stream=None):
    """W4A8 linear: y [M, N] = MXFP8(x) [M, K] * B [N, K]^T + bias from bf16 x
    [M, ldx] (mxfp8_quantize_act then mxfp4_gemm_w4a8, bit for bit; one launch
    for decode shapes).  A workspace is allocated when one is needed and none
    is given."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(b_codes, "b_codes", torch.uint8, dev)
    _need(b_scales, "b_scales", torch.uint8, dev)
    if x.dim() != 2:
        raise ValueError("x must be [M, ldx]")
    M, ldx = x.shape
    K = ldx if K is None else K
    N = b_codes.shape[0]
    if b_codes.shape != (N, K // 2) or b_scales.shape != (N, K // 32):
        raise ValueError("operand shapes disagree")
    bias = _bias_arg(bias, N, dev)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _need(y, "y", y.dtype, dev)
    if y.shape != (M, N):
        raise ValueError("y must be [M, N]")
    need = mxfp4_linear_w4a8_workspace_size(M, N, K)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel())
    _check("mxfp4_linear_w4a8_bf16", _lib.mxfp4_linear_w4a8_bf16(
        _ptr(x), ldx, M, N, K, _ptr(b_codes), _ptr(b_scales), _ptr(bias), _ptr(y),
        _out_dtype(y.dtype), ws_ptr, ws_bytes, 0, _stream(stream, dev)))
    return y


def mxfp4_silu_mul_quantize(gate_up, codes=None, scales=None, *, I=None, scale_rule="ocp",
                            stream=None):
    """MoE expert activation for the down projection: bf16 gate_up [M, ldg]
    (gate = columns [0, I), up = [I, 2I)) -> MXFP4 codes [M, I/2] and E8M0
    bytes [M, I/32] of bf16(silu(gate) * up).  I defaults to ldg // 2."""
    _need(gate_up, "gate_up", torch.bfloat16)
    dev = gate_up.device
    if gate_up.dim() != 2:
        raise ValueError("gate_up must be 2-D [rows, ldg]")
    M, ldg = gate_up.shape
    I = ldg // 2 if I is None else int(I)
    if codes is None:
        codes = torch.empty((M, I // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, I // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (M, I // 2) or scales.shape != (M, I // 32):
        raise ValueError("output shapes do not match [M, I/2] / [M, I/32]")
    _check("mxfp4_silu_mul_quantize", _lib.mxfp4_silu_mul_quantize(
        _ptr(gate_up), ldg, M, I, _ptr(codes), _ptr(scales), _rule_flag(scale_rule),
        _stream(stream, dev)))
    return codes, scales


def mxfp4_moe_combine(y, rows, weights, out=None, *, H=None, out_dtype=torch.bfloat16,
                      stream=None):
    """out [T, H] = sum_j weights[t, j] * y[rows[t, j], :H] over bf16 y [R, ldy]
    (expert-sorted rows), int32 rows [T, topk], fp32 weights [T, topk]."""
    _need(y, "y", torch.bfloat16)
    dev = y.device
    _need(rows, "rows", torch.int32, dev)
    _need(weights, "weights", torch.float32, dev)
    if y.dim() != 2 or rows.dim() != 2 or weights.shape != rows.shape:
        raise ValueError("y must be [R, ldy]; rows and weights [T, topk]")
    R, ldy = y.shape
    T, topk = rows.shape
    H = ldy if H is None else int(H)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _need(out, "out", out.dtype, dev)
    if out.shape != (T, H):
        raise ValueError("out must be [T, H]")
    _check("mxfp4_moe_combine", _lib.mxfp4_moe_combine(
        _ptr(y), ldy, R, _ptr(rows), _ptr(weights), T, topk, H, _ptr(out),
        _out_dtype(out.dtype), 0, _stream(stream, dev)))
    return out


def mxfp4_grouped_gemm(a_codes, a_scales, b_codes, b_scales, offsets, y=None, *,
                       out_dtype=torch.bfloat16, b_preshuffled=False, stream=None):
    """For each expert e: y[off[e]:off[e+1]] = A[off[e]:off[e+1]] * B[e]^T.
    A [total_M, K/2] expert-sorted, B [E, N, K/2], offsets int32 [E+1].
    b_preshuffled: B's codes as mxfp4_preshuffle_weights wrote them."""
    _need(a_codes, "a_codes", torch.uint8)
    dev = a_codes.device
    for t, n in ((a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _need(t, n, torch.uint8, dev)
    _need(offsets, "offsets", torch.int32, dev)
    total_M, K = a_codes.shape[0], a_codes.shape[1] * 2
    E, N = b_codes.shape[0], b_codes.shape[1]
    if offsets.shape != (E + 1,):
        raise ValueError("offsets must have E+1 entries")
    if b_codes.shape != (E, N, K // 2) or b_scales.shape != (E, N, K // 32) or \
            a_scales.shape != (total_M, K // 32):
        raise ValueError("operand shapes disagree")
    if y is None:
        y = torch.empty((total_M, N), dtype=out_dtype, device=dev)
    _need(y, "y", y.dtype, dev)
    if y.shape != (total_M, N):
        raise ValueError("y must be [total_M, N]")
    _check("mxfp4_grouped_gemm", _lib.mxfp4_grouped_gemm(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), _ptr(offsets),
        E, total_M, N, K, _ptr(y), _out_dtype(y.dtype), None, 0,
        MXFP4_B_PRESHUFFLED if b_preshuffled else 0, _stream(stream, dev)))
    return y


def mxfp4_preshuffle_weights(codes, out=None, *, stream=None):
    """MXFP4 weight codes [T, N, K/2] (or [N, K/2]) -> the same bytes in the
    grouped GEMMs' operand order (for b_preshuffled=True); N % 32 == 0,
    K % 256 == 0."""
    _need(codes, "codes", torch.uint8)
    dev = codes.device
    if codes.dim() not in (2, 3):
        raise ValueError("codes must be [N, K/2] or [T, N, K/2]")
    T = 1 if codes.dim() == 2 else codes.shape[0]
    N, K = codes.shape[-2], codes.shape[-1] * 2
    if out is None:
        out = torch.empty_like(codes)
    _need(out, "out", torch.uint8, dev)
    if out.shape != codes.shape:
        raise ValueError("out must have the shape of codes")
    _check("mxfp4_preshuffle_weights", _lib.mxfp4_preshuffle_weights(
        _ptr(codes), _ptr(out), T, N, K, _stream(stream, dev)))
    return out



def mxfp4_quantize_act_scatter(x, dest_rows, codes=None, scales=None, *, R=None, K=None,
                               scale_rule="ocp", stream=None):
    """MoE dispatch: bf16 x [T, ldx] -> MXFP4 rows written to
    dest_rows[t, j] (int32 [T, fan]) of codes [R, K/2] / scales [R, K/32].
    R defaults to T * fan (every routed row once)."""
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(dest_rows, "dest_rows", torch.int32, dev)
    if x.dim() != 2 or dest_rows.dim() != 2 or dest_rows.shape[0] != x.shape[0]:
        raise ValueError("x must be [T, ldx] and dest_rows [T, fan]")
    T, ldx = x.shape
    fan = dest_rows.shape[1]
    K = ldx if K is None else int(K)
    R = T * fan if R is None else int(R)
    if codes is None:
        codes = torch.empty((R, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((R, K // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (R, K // 2) or scales.shape != (R, K // 32):
        raise ValueError("output shapes do not match [R, K/2] / [R, K/32]")
    _check("mxfp4_quantize_act_scatter", _lib.mxfp4_quantize_act_scatter(
        _ptr(x), ldx, T, K, _ptr(dest_rows), fan, R, _ptr(codes), _ptr(scales),
        _rule_flag(scale_rule), _stream(stream, dev)))
    return codes, scales


def mxfp4_grouped_gemm_silu_quantize(a_codes, a_scales, b_codes, b_scales, offsets,
                                     codes=None, scales=None, *, scale_rule="ocp",
                                     b_preshuffled=False, stream=None):
    """The MoE gate_up grouped GEMM with the expert activation and its MXFP4
    quantization fused in: A [total_M, K/2] expert-sorted, B [E, 2I, K/2] with
    each expert's rows interleaved by 32 (rows 64q..64q+31 gate, 64q+32..64q+63
    up, for h columns 32q..32q+31), offsets int32 [E+1] -> MXFP4 codes
    [total_M, I/2] and E8M0 bytes [total_M, I/32] of bf16(silu(gate) * up)."""
    _need(a_codes, "a_codes", torch.uint8)
    dev = a_codes.device
    for t, n in ((a_scales, "a_scales"), (b_codes, "b_codes"), (b_scales, "b_scales")):
        _need(t, n, torch.uint8, dev)
    _need(offsets, "offsets", torch.int32, dev)
    total_M, K = a_codes.shape[0], a_codes.shape[1] * 2
    E, N = b_codes.shape[0], b_codes.shape[1]
    if offsets.shape != (E + 1,):
        raise ValueError("offsets must have E+1 entries")
    if b_codes.shape != (E, N, K // 2) or b_scales.shape != (E, N, K // 32) or \
            a_scales.shape != (total_M, K // 32):
        raise ValueError("operand shapes disagree")
    if N % 2:
        raise ValueError("B must hold 2I rows per expert")
    I = N // 2
    if codes is None:
        codes = torch.empty((total_M, I // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((total_M, I // 32), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev)
    _need(scales, "scales", torch.uint8, dev)
    if codes.shape != (total_M, I // 2) or scales.shape != (total_M, I // 32):
        raise ValueError("output shapes do not match [total_M, I/2] / [total_M, I/32]")
    _check("mxfp4_grouped_gemm_silu_quantize", _lib.mxfp4_grouped_gemm_silu_quantize(
        _ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), _ptr(offsets),
        E, total_M, I, K, _ptr(codes), _ptr(scales),
        _rule_flag(scale_rule) | (MXFP4_B_PRESHUFFLED if b_preshuffled else 0),
        _stream(stream, dev)))
    return codes, scales


__all__ = ["mxfp4_requant_from_nvfp4", "mxfp4_quantize_act", "mxfp4_gemm",
           "mxfp4_grouped_gemm", "mxfp4_linear_bf16", "mxfp4_gemm_workspace_size",
           "mxfp4_linear_workspace_size", "mxfp4_silu_mul_quantize", "mxfp4_moe_combine",
           "mxfp8_quantize_act", "mxfp4_gemm_w4a8", "mxfp4_linear_w4a8_bf16",
           "mxfp4_linear_w4a8_workspace_size", "mxfp4_quantize_act_smooth",
           "mxfp8_quantize_act_smooth", "mxfp4_grouped_gemm_silu_quantize",
           "mxfp4_quantize_act_scatter", "mxfp4_preshuffle_weights",
           "mxfp4_status_string",
           "mxfp4_version", "Mxfp4Error", "LIBRARY_PATH", "EXPORTED_SYMBOLS",
           "MXFP4_OUT_BF16", "MXFP4_OUT_FP32", "MXFP4_REQ_INTERMEDIATE_BF16",
           "MXFP4_SCALE_UOS", "MXFP4_B_PRESHUFFLED"]
