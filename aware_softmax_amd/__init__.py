"""Python binding of libfa.so, the gfx950 fused exact-attention library.

Argument marshalling only: every step of the forward, backward and decode runs in the HIP
kernels behind the C ABI declared in include/fa.h.  torch supplies device
memory and the current stream.  There is no fallback: if libfa.so is
missing or fails to load, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FaError",
    "fwd",
    "fa_fwd",
    "fa_fwd_gqa",
    "fa_fwd_varlen",
    "fwd_varlen",
    "fwd_fp8",
    "fa_fwd_fp8",
    "bwd_varlen",
    "fa_bwd_varlen",
    "bwd_varlen_workspace_bytes",
    "fa_bwd_gqa",
    "bwd",
    "fa_bwd",
    "bwd_workspace_bytes",
    "bwd_gqa_workspace_bytes",
    "bwd_tile_config",
    "decode",
    "fa_decode",
    "fa_decode_static",
    "decode_static",
    "DECODE_STATIC_SCRATCH_BYTES",
    "decode_plan",
    "decode_workspace_bytes",
    "tile_config",
    "version",
    "mfma_ceiling",
    "MFMA_CEILING_FLOP_PER_ITER_BLOCK",
    "status_string",
    "last_hip_error",
    "library",
    "LIB_PATH",
    "DTYPE_F32",
    "DTYPE_BF16",
    "DTYPE_F16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
FA_OK = 0


class FaError(RuntimeError):
    """A nonzero fa_status_t from the C library."""

    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code


def _load() -> ctypes.CDLL:
    # One HIP runtime per process: torch bundles its own libamdhip64.so.7,
    # and libfa.so, loaded first, would pull in the system copy next to it;
    # kernels launched through the second runtime then fail (it reports no
    # device).  Loading torch first lets libfa.so bind to the runtime already
    # loaded under the same soname.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python aware_softmax_amd/build.py` "
            "(there is no non-HIP fallback)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_fwd_gqa.restype = ci
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_fwd_varlen.restype = ci
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, ci,
                                  ctypes.c_float, ci, vp]
    lib.fa_bwd_varlen.restype = ci
    lib.fa_bwd_varlen_workspace_bytes.argtypes = [ci, ci, ci]
    lib.fa_bwd_varlen_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [ci]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd_tile.argtypes = [ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci), ctypes.POINTER(ci)]
    lib.fa_fwd_tile.restype = ci
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ci, ctypes.c_float,
                               ci, vp]
    lib.fa_bwd_gqa.restype = ci
    lib.fa_bwd_gqa_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
    lib.fa_bwd_gqa_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_tile.argtypes = [ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
    lib.fa_bwd_tile.restype = ci
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, ci, ci, ci, ci, ci, ctypes.c_float, ci, ci, vp]
    lib.fa_decode.restype = ci
    lib.fa_decode_static.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, ci, vp]
    lib.fa_decode_static.restype = ci
    lib.fa_decode_plan.argtypes = [ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci),
                                   ctypes.POINTER(sz)]
    lib.fa_decode_plan.restype = ci
    lib.fa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_last_hip_error.argtypes = [ctypes.POINTER(ctypes.c_char_p)]
    lib.fa_last_hip_error.restype = ci
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ctypes.c_float,
                               ctypes.c_float, ctypes.c_float, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_mfma_ceiling.argtypes = [vp, ci, ci, ci, vp]
    lib.fa_mfma_ceiling.restype = ci
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    return lib


_LIB = _load()


def library() -> ctypes.CDLL:
    return _LIB


def status_string(code: int) -> str:
    return _LIB.fa_status_string(int(code)).decode()


def version() -> str:
    return _LIB.fa_version().decode()


def last_hip_error() -> tuple:
    """(hipError_t code, message) behind the last FA_ERR_HIP on this thread."""
    msg = ctypes.c_char_p()
    code = _LIB.fa_last_hip_error(ctypes.byref(msg))
    return code, (msg.value or b"").decode()


def _check(code: int) -> None:
    if code != FA_OK:
        message = status_string(code)
        if code == 7:  # FA_ERR_HIP: add what the runtime reported
            hip_code, hip_msg = last_hip_error()
            message += f" (hipError_t {hip_code}: {hip_msg})"
        raise FaError(code, message)


def _check_out(name, t, shape, dtype, device) -> None:
    """A caller-supplied output must be a contiguous tensor of the given
    shape and dtype on the inputs' device: the C ABI sees only its address,
    so a wrong size would be written past its end and a host tensor would
    be dereferenced by the kernel."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be a {dtype} tensor of shape {tuple(shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(t, device) -> int:
    """A workspace is a contiguous uint8 device tensor on the inputs'
    device; returns its size in bytes (the library checks the size)."""
    import torch

    if t.dtype != torch.uint8 or t.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"workspace must be a device tensor on {device}")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return t.numel()


def _check_inputs(device, **tensors) -> None:
    for name, t in tensors.items():
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a device tensor on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def tile_config(d: int, dtype: int) -> tuple:
    """(block_q, block_k, waves) that fa_fwd uses for head dim d and dtype."""
    bq, bk, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_LIB.fa_fwd_tile(int(d), int(dtype), ctypes.byref(bq), ctypes.byref(bk), ctypes.byref(w)))
    return bq.value, bk.value, w.value


def fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, causal, scale, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses; returns
    the fa_status_t code."""
    return _LIB.fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(N), int(d),
                       int(bool(causal)), float(scale), int(dtype), stream)


def fa_fwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, causal, scale, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses."""
    return _LIB.fa_fwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(Hkv), int(N), int(d),
                           int(bool(causal)), float(scale), int(dtype), stream)


def fwd(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None, stream=None):
    """O, L = attention forward of [B, H, N, d] device tensors (bf16, fp16 or fp32).

    k and v may have fewer heads, [B, Hkv, N, d] with H a multiple of Hkv
    (grouped heads: query head h reads key/value head h // (H // Hkv)).
    Returns (o, lse): o like q, lse float32 [B, H, N] (natural-log
    logsumexp of each scaled, masked score row).  out / lse may be passed to
    reuse buffers.  Runs on `stream` (default: torch's current stream).
    """
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.float32: DTYPE_F32}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype}; use torch.bfloat16, torch.float16 or torch.float32")
    dtype = dtypes[q.dtype]
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.shape != (B, Hkv, N, d):
            raise ValueError(f"{name} must be [B, Hkv, N, d] with the dtype, B, N and d of q")
    _check_inputs(q.device, q=q, k=k, v=v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, Hkv, N, d, causal, scale, dtype, stream.cuda_stream))
    return out, lse


def fa_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, causal, scale, q_descale, k_descale,
               v_descale, stream) -> int:
    """Raw call of the C entry point with integer device addresses; returns
    the fa_status_t code."""
    return _LIB.fa_fwd_fp8(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, int(B), int(H), int(Hkv), int(N), int(d),
                           int(bool(causal)), float(scale), float(q_descale), float(k_descale), float(v_descale),
                           stream)


def fwd_fp8(q, k, v, q_descale: float, k_descale: float, v_descale: float, causal: bool = True,
            scale: float | None = None, out=None, lse=None, stream=None):
    """O, L = attention forward of e4m3 inputs: q [B, H, N, d] and k, v
    [B, Hkv, N, d] device tensors of torch.float8_e4m3fn (or uint8 holding
    e4m3 bytes), element value = byte value x the tensor's descale factor.
    Returns (o, lse): o bfloat16 [B, H, N, d], lse float32 [B, H, N].
    d 64 or 128."""
    import torch

    allowed = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype not in allowed:
            raise TypeError(f"{name} must be torch.float8_e4m3fn or uint8 e4m3 bytes, not {t.dtype}")
    _check_inputs(q.device, q=q, k=k, v=v)
    for name, t in (("k", k), ("v", v)):
        if t.shape != (B, Hkv, N, d):
            raise ValueError(f"{name} must be [B, Hkv, N, d] with the B, N and d of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out("out", out, (B, H, N, d), torch.bfloat16, q.device)
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d,
                      causal, scale, q_descale, k_descale, v_descale, stream.cuda_stream))
    return out, lse


def bwd_gqa_workspace_bytes(B, H, Hkv, N, d) -> int:
    """Device workspace bytes with which fa_bwd_gqa may split each group's
    heads over several dK/dV workgroups (0 for unsupported sizes)."""
    return int(_LIB.fa_bwd_gqa_workspace_bytes(int(B), int(H), int(Hkv), int(N), int(d)))


def bwd_workspace_bytes(B, H, N, d) -> int:
    """Device workspace bytes fa_bwd needs (0 for unsupported sizes)."""
    return int(_LIB.fa_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def bwd_tile_config(d: int) -> tuple:
    """(keys per workgroup, queries per streamed tile) of the backward."""
    bk, bq = ctypes.c_int(), ctypes.c_int()
    _check(_LIB.fa_bwd_tile(int(d), ctypes.byref(bk), ctypes.byref(bq)))
    return bk.value, bq.value


def fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, ws_bytes,
           B, H, N, d, causal, scale, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses; returns
    the fa_status_t code."""
    return _LIB.fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                       int(ws_bytes), int(B), int(H), int(N), int(d), int(bool(causal)), float(scale),
                       int(dtype), stream)


def fa_bwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, ws_bytes,
               B, H, Hkv, N, d, causal, scale, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses."""
    return _LIB.fa_bwd_gqa(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                           int(ws_bytes), int(B), int(H), int(Hkv), int(N), int(d), int(bool(causal)),
                           float(scale), int(dtype), stream)


def bwd(q, k, v, o, lse, do, causal: bool = True, scale: float | None = None, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """dQ, dK, dV of attention for [B, H, N, d] bf16 or fp16 device tensors.

    k and v (and so dk, dv) may be [B, Hkv, N, d] with H a multiple of Hkv,
    as in fwd(); dk and dv then sum over the query heads of each group.

    o and lse are the outputs of fwd() for the same q, k, v, causal and
    scale; do is the upstream gradient of o.  dq / dk / dv / workspace may
    be passed to reuse buffers (workspace: a uint8 device tensor of at least
    bwd_workspace_bytes(B, H, N, d) bytes; bwd_gqa_workspace_bytes(B, H,
    Hkv, N, d) bytes let grouped heads use the head-split dK/dV pass).  Runs on `stream` (default:
    torch's current stream).
    """
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype} for the backward; use torch.bfloat16 or torch.float16")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        want = (B, Hkv, N, d) if name in ("k", "v") else q.shape
        if t.dtype != q.dtype or t.shape != want:
            raise ValueError(f"{name} must be a {q.dtype} tensor of shape {tuple(want)}")
    _check_inputs(q.device, q=q, k=k, v=v, o=o, do=do)
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_out("dq", dq, q.shape, q.dtype, q.device)
    _check_out("dk", dk, k.shape, q.dtype, q.device)
    _check_out("dv", dv, k.shape, q.dtype, q.device)
    if workspace is None:
        # the grouped-head size enables the head-split dK/dV pass where it applies
        need = bwd_gqa_workspace_bytes(B, H, Hkv, N, d)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_bwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                      ws_bytes, B, H, Hkv, N, d, causal, scale,
                      dtypes[q.dtype], stream.cuda_stream))
    return dq, dk, dv


def decode_plan(B, H, Hkv, N, d, num_splits=0) -> tuple:
    """(splits, keys per split, workspace bytes) that fa_decode uses."""
    sp, ck, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _check(_LIB.fa_decode_plan(int(B), int(H), int(Hkv), int(N), int(d), int(num_splits), ctypes.byref(sp),
                               ctypes.byref(ck), ctypes.byref(ws)))
    return sp.value, ck.value, ws.value


# FLOPs of one loop iteration of one fa_mfma_ceiling workgroup: 4 waves x 4
# MFMA 32x32x16 x 32768 FLOP.
MFMA_CEILING_FLOP_PER_ITER_BLOCK = 4 * 4 * 32768


def mfma_ceiling(sink, iters: int, blocks: int, store: bool = False, stream=None) -> None:
    """Enqueue the matrix-core-only ceiling kernel (a measurement helper):
    `blocks` workgroups each run `iters` iterations of 16 bf16 MFMAs;
    `sink` is an fp32 device tensor of at least blocks * 256 elements."""
    import torch

    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 256:
        raise ValueError("sink must be an fp32 device tensor of blocks * 256 elements")
    stream = stream or torch.cuda.current_stream(sink.device)
    _check(_LIB.fa_mfma_ceiling(sink.data_ptr(), int(iters), int(blocks), int(bool(store)), stream.cuda_stream))


def decode_workspace_bytes(B, H, Hkv, N, d, num_splits=0) -> int:
    """Device workspace bytes fa_decode needs (0 for invalid sizes)."""
    return int(_LIB.fa_decode_workspace_bytes(int(B), int(H), int(Hkv), int(N), int(d), int(num_splits)))


def fa_decode(q_ptr, k_ptr, v_ptr, seqlens_ptr, o_ptr, lse_ptr, ws_ptr, ws_bytes, B, H, Hkv, N, d, scale,
              num_splits, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses; returns
    the fa_status_t code."""
    return _LIB.fa_decode(q_ptr, k_ptr, v_ptr, seqlens_ptr, o_ptr, lse_ptr, ws_ptr, int(ws_bytes), int(B), int(H),
                          int(Hkv), int(N), int(d), float(scale), int(num_splits), int(dtype), stream)


def decode(q, k, v, scale: float | None = None, num_splits: int = 0, out=None, lse=None, workspace=None,
           stream=None, cache_seqlens=None):
    """Split-K decode attention: q [B, H, d] against a cache k, v
    [B, Hkv, N, d] (bf16 or fp16 device tensors, H a multiple of Hkv).

    cache_seqlens (optional int32 device tensor [B]): sequence b attends to
    the first cache_seqlens[b] rows of its cache (default: all N).
    Returns (o [B, H, d] like q, lse [B, H] float32).  num_splits = 0 lets the
    library choose; 1 runs the unsplit kernel.  out / lse / workspace (uint8,
    at least decode_plan(...)[2] bytes) may be passed to reuse buffers.
    Runs on `stream` (default: torch's current stream).
    """
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype} for decode; use torch.bfloat16 or torch.float16")
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, H, d] and k, v [B, Hkv, N, d]")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have the dtype of q")
    _check_inputs(q.device, q=q, k=k, v=v)
    if v.shape != k.shape:
        raise ValueError("v must match k in shape")
    B, H, d = q.shape
    Bk, Hkv, N, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("k, v must be [B, Hkv, N, d] with the B and d of q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_plan(B, H, Hkv, N, d, num_splits)[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (B, H), torch.float32, q.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    seq_ptr = None
    if cache_seqlens is not None:
        _check_out("cache_seqlens", cache_seqlens, (B,), torch.int32, q.device)
        seq_ptr = cache_seqlens.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), seq_ptr, out.data_ptr(), lse.data_ptr(),
                     workspace.data_ptr(), ws_bytes, B, H, Hkv, N, d, scale, num_splits,
                     dtypes[q.dtype], stream.cuda_stream))
    return out, lse


# FA_DECODE_STATIC_SCRATCH_BYTES of include/fa.h
DECODE_STATIC_SCRATCH_BYTES = 16 << 20


def fa_decode_static(q_ptr, k_ptr, v_ptr, seqlens_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, scale, num_splits, dtype,
                     stream) -> int:
    """Raw call of the C entry point with integer device addresses; returns
    the fa_status_t code."""
    return _LIB.fa_decode_static(q_ptr, k_ptr, v_ptr, seqlens_ptr, o_ptr, lse_ptr, int(B), int(H), int(Hkv), int(N),
                                 int(d), float(scale), int(num_splits), int(dtype), stream)


def decode_static(q, k, v, out, lse, scale: float | None = None, num_splits: int = 0, stream=None,
                  cache_seqlens=None):
    """decode() without a workspace: the library's static device scratch
    holds the split partials, so the call allocates nothing (out and lse
    are the caller's).  Calls that overlap in time on one device race on
    that scratch.  Raises FaError (FA_ERR_SCRATCH) when the split partials
    would exceed DECODE_STATIC_SCRATCH_BYTES."""
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype} for decode; use torch.bfloat16 or torch.float16")
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, d] and k, v [B, Hkv, N, d]")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have the dtype of q")
    _check_inputs(q.device, q=q, k=k, v=v)
    B, H, d = q.shape
    Bk, Hkv, N, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("k, v must be [B, Hkv, N, d] with the B and d of q")
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (B, H), torch.float32, q.device)
    seq_ptr = None
    if cache_seqlens is not None:
        _check_out("cache_seqlens", cache_seqlens, (B,), torch.int32, q.device)
        seq_ptr = cache_seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), seq_ptr, out.data_ptr(), lse.data_ptr(), B, H,
                            Hkv, N, d, scale, num_splits, dtypes[q.dtype], stream.cuda_stream))
    return out, lse


def fa_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, B, H, Hkv, total, max_seqlen, d, causal, scale,
                  dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses."""
    return _LIB.fa_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, cu_ptr, int(B), int(H), int(Hkv), int(total),
                              int(max_seqlen), int(d), int(bool(causal)), float(scale), int(dtype), stream)


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = True, scale: float | None = None, out=None,
               lse=None, stream=None):
    """Forward over packed sequences of different lengths.

    q [H, total, d] and k, v [Hkv, total, d] (bf16 or fp16 device tensors)
    hold the rows of all sequences one after another; cu_seqlens is an int32
    device tensor of B + 1 offsets (sequence b = rows cu_seqlens[b] ..
    cu_seqlens[b + 1] - 1) and max_seqlen the longest length (a host int).
    Returns (o [H, total, d], lse [H, total] float32).
    """
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype} for varlen; use torch.bfloat16 or torch.float16")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [H, total, d] and k, v [Hkv, total, d]")
    H, total, d = q.shape
    Hkv = k.shape[0]
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.shape != (Hkv, total, d):
            raise ValueError(f"{name} must be [Hkv, total, d] with the dtype, total and d of q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor of B + 1 offsets")
    _check_inputs(q.device, q=q, k=k, v=v, cu_seqlens=cu_seqlens)
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check_out("out", out, q.shape, q.dtype, q.device)
    _check_out("lse", lse, (H, total), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         cu_seqlens.data_ptr(), B, H, Hkv, total, max_seqlen, d, causal, scale, dtypes[q.dtype],
                         stream.cuda_stream))
    return out, lse


def bwd_varlen_workspace_bytes(H, total, d) -> int:
    return int(_LIB.fa_bwd_varlen_workspace_bytes(int(H), int(total), int(d)))


def fa_bwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, cu_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr, ws_bytes, B,
                  H, Hkv, total, max_seqlen, d, causal, scale, dtype, stream) -> int:
    """Raw call of the C entry point with integer device addresses."""
    return _LIB.fa_bwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, do_ptr, cu_ptr, dq_ptr, dk_ptr, dv_ptr, ws_ptr,
                              int(ws_bytes), int(B), int(H), int(Hkv), int(total), int(max_seqlen), int(d),
                              int(bool(causal)), float(scale), int(dtype), stream)


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen: int, causal: bool = True, scale: float | None = None,
               dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of fwd_varlen (the same packed layouts and cu_seqlens)."""
    import torch

    dtypes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}
    if q.dtype not in dtypes:
        raise TypeError(f"unsupported dtype {q.dtype} for varlen; use torch.bfloat16 or torch.float16")
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [H, total, d] and k, v [Hkv, total, d]")
    H, total, d = q.shape
    Hkv = k.shape[0]
    for name, t in (("o", o), ("do", do)):
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError(f"{name} must match q in dtype and shape")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.shape != (Hkv, total, d):
            raise ValueError(f"{name} must be [Hkv, total, d] with the dtype, total and d of q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    _check_inputs(q.device, q=q, k=k, v=v, o=o, do=do, cu_seqlens=cu_seqlens)
    _check_out("lse", lse, (H, total), torch.float32, q.device)
    B = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_out("dq", dq, q.shape, q.dtype, q.device)
    _check_out("dk", dk, k.shape, q.dtype, q.device)
    _check_out("dv", dv, k.shape, q.dtype, q.device)
    need = bwd_varlen_workspace_bytes(H, total, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    _check(fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                         cu_seqlens.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                         ws_bytes, B, H, Hkv, total, max_seqlen, d, causal,
                         scale, dtypes[q.dtype], stream.cuda_stream))
    return dq, dk, dv
