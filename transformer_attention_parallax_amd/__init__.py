"""Python binding of libparallax, the MI355X Parallax attention library.

Argument marshalling only: shapes, strides, dtypes and the current HIP
stream are read from torch tensors and passed through ctypes to the C ABI
declared in ``include/parallax.h``; every step of the attention path runs in
the HIP kernels of ``libparallax.so``. There is no fallback: if the library
is not built, or the GPU call fails, a ``ParallaxError`` is raised.

Parallax attention (zubnet.ai news item on Parallax, second paragraph):
softmax attention minus the key-value covariance contracted with a learned
probe rho_i = W_R x_i; rho = 0 gives plain softmax attention.

    decode(q, k_cache, v_cache, rho, seqlens=None, scale=None, ...)
        q, rho [B, H, D]; k_cache, v_cache [B, H, Lmax, D]  ->  [B, H, D]
    fwd(q, k, v, rho, causal=True, scale=None, ...)
        q, k, v, rho [B, N, H, D]  ->  [B, N, H, D]
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "ParallaxError", "library", "decode", "decode_noalloc", "fwd", "decode_splits",
    "decode_workspace_size", "fwd_workspace_size", "bwd", "bwd_workspace_size",
    "decode_gqa", "decode_gqa_workspace_size",
    "LIBRARY", "STATUS",
]

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "libparallax.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
STATUS = {OK: "OK", ERR_INVALID_ARG: "ERR_INVALID_ARG",
          ERR_UNSUPPORTED: "ERR_UNSUPPORTED", ERR_WORKSPACE: "ERR_WORKSPACE",
          ERR_HIP: "ERR_HIP"}
F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}

# Exported functions and their ctypes signatures (mirrors include/parallax.h).
_i64, _int, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
SIGNATURES = {
    "parallax_status_string": (ctypes.c_char_p, [_int]),
    "parallax_last_error": (ctypes.c_char_p, []),
    "parallax_decode_splits": (_int, [_int, _int, _int, _int, _int,
                                      ctypes.POINTER(_int)]),
    "parallax_decode_workspace_size": (_int, [_int, _int, _int, _int, _int,
                                              ctypes.POINTER(ctypes.c_size_t)]),
    "parallax_fwd_workspace_size": (_int, [_int, _int, _int, _int, _int,
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "parallax_decode_gqa_workspace_size": (_int, [_int, _int, _int, _int, _int, _int, _int,
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "parallax_decode_gqa": (_int, [
        _vp, _i64, _i64,                 # q
        _vp, _i64, _i64,                 # rho
        _vp, _vp, _i64, _i64, _i64,      # k_cache, v_cache, strides
        _vp, _i64, _int, _int,           # block_table, row stride, page size, pages
        _vp,                             # seqlens
        _vp, _i64, _i64,                 # out
        _int, _int, _int, _int, _int, ctypes.c_float, _int, _int, _int,
        _vp, ctypes.c_size_t, _vp]),
    "parallax_stream_read": (_int, [_vp, _i64, _vp, _vp]),
    "parallax_decode_gqa_splits": (_int, [_int, _int, _int, _int, _int, _int, _int,
                                          ctypes.POINTER(_int)]),
    "parallax_project": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _int,
                                _int, _vp]),
    "parallax_fwd_varlen": (_int, [
        _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,  # q k v rho
        _vp, _i64, _i64,                 # out
        _vp, _int, _int, _int, _int,     # cu_seqlens, B, max_seqlen, H, D
        ctypes.c_float, _int, _int, _int, _vp, ctypes.c_size_t, _vp]),
    "parallax_bwd_workspace_size": (_int, [_int, _int, _int, _int, _int,
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "parallax_bwd": (_int, [
        _vp, _i64, _i64, _i64,           # q
        _vp, _i64, _i64, _i64,           # k
        _vp, _i64, _i64, _i64,           # v
        _vp, _i64, _i64, _i64,           # rho
        _vp, _i64, _i64, _i64,           # dout
        _vp, _i64, _i64, _i64,           # dq
        _vp, _i64, _i64, _i64,           # dk
        _vp, _i64, _i64, _i64,           # dv
        _vp, _i64, _i64, _i64,           # drho
        _int, _int, _int, _int, ctypes.c_float, _int, _int,
        _vp, ctypes.c_size_t, _vp]),
    "parallax_decode": (_int, [
        _vp, _i64, _i64,                 # q
        _vp, _i64, _i64,                 # rho
        _vp, _vp, _i64, _i64, _i64,      # k_cache, v_cache, strides
        _vp,                             # seqlens
        _vp, _i64, _i64,                 # out
        _int, _int, _int, _int, ctypes.c_float,
        _int, _int, _int, _vp, ctypes.c_size_t, _vp]),
    "parallax_decode_noalloc": (_int, [
        _vp, _i64, _i64,                 # q
        _vp, _i64, _i64,                 # rho
        _vp, _vp, _i64, _i64, _i64,      # k_cache, v_cache, strides
        _vp,                             # seqlens
        _vp, _i64, _i64,                 # out
        _int, _int, _int, _int, ctypes.c_float,
        _int, _int, _int, _vp]),
    "parallax_fwd": (_int, [
        _vp, _i64, _i64, _i64,           # q
        _vp, _i64, _i64, _i64,           # k
        _vp, _i64, _i64, _i64,           # v
        _vp, _i64, _i64, _i64,           # rho
        _vp, _i64, _i64, _i64,           # out
        _int, _int, _int, _int, ctypes.c_float, _int, _int, _int,
        _vp, ctypes.c_size_t, _vp]),
    "parallax_fwd_train": (_int, [
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # q, k
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # v, rho
        _vp, _i64, _i64, _i64,           # out
        _vp, _vp,                        # vbar, lse_rbar
        _int, _int, _int, _int, ctypes.c_float, _int, _int, _int,
        _vp, ctypes.c_size_t, _vp]),
    "parallax_bwd_saved": (_int, [
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # q, k
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # v, rho
        _vp, _i64, _i64, _i64,           # dout
        _vp, _i64, _i64, _i64, _int,     # out, its dtype
        _vp, _vp,                        # vbar, lse_rbar
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # dq, dk
        _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,     # dv, drho
        _int, _int, _int, _int, ctypes.c_float, _int, _int,
        _vp, ctypes.c_size_t, _vp]),
}


class ParallaxError(RuntimeError):
    """A libparallax call failed (status code and the library's message)."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


_lib = None


def library(path: Optional[str] = None):
    """Load libparallax.so (raises ParallaxError if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY
    if not os.path.exists(p):
        raise ParallaxError(
            ERR_HIP, f"{p} is not built; run "
            "`python -m transformer_attention_parallax_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _raise_on(status: int, what: str):
    if status != OK:
        msg = library().parallax_last_error().decode(errors="replace")
        raise ParallaxError(status, f"{what}: {msg}")


def decode_splits(B: int, H: int, D: int, Lmax: int, num_splits: int = 0) -> int:
    """Number of KV splits parallax_decode uses for these sizes."""
    out = _int(0)
    _raise_on(library().parallax_decode_splits(B, H, D, Lmax, num_splits,
                                               ctypes.byref(out)),
              "parallax_decode_splits")
    return out.value


def decode_workspace_size(B: int, H: int, D: int, Lmax: int,
                          num_splits: int = 0) -> int:
    """Bytes of device workspace parallax_decode needs for these sizes."""
    out = ctypes.c_size_t(0)
    _raise_on(library().parallax_decode_workspace_size(
        B, H, D, Lmax, num_splits, ctypes.byref(out)),
        "parallax_decode_workspace_size")
    return out.value


def fwd_workspace_size(B: int, N: int, H: int, D: int,
                       dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of device workspace parallax_fwd needs for these sizes."""
    code = {torch.float32: F32, torch.bfloat16: BF16}.get(dtype)
    if code is None:
        raise ParallaxError(ERR_INVALID_ARG, f"unsupported dtype {dtype}")
    out = ctypes.c_size_t(0)
    _raise_on(library().parallax_fwd_workspace_size(
        B, N, H, D, code, ctypes.byref(out)), "parallax_fwd_workspace_size")
    return out.value


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise ParallaxError(ERR_UNSUPPORTED,
                            f"{name}: dtype {t.dtype} (float32 or bfloat16)")
    return _DT[t.dtype]


def _need_gpu(*tensors):
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ParallaxError(ERR_INVALID_ARG, "tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ParallaxError(ERR_INVALID_ARG, "tensors must be on one GPU")


def _stream(device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ParallaxError(ERR_INVALID_ARG, "stream is on another GPU than the tensors")
    return int(stream.cuda_stream)


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   rho: Optional[torch.Tensor], seqlens: Optional[torch.Tensor] = None,
                   scale: Optional[float] = None, out: torch.Tensor = None,
                   num_splits: int = 0,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """parallax_decode_noalloc: ``decode`` without a workspace (split records
    in the library's fixed device scratch). ``out`` ([B, H, D], float32 or
    bfloat16) must be given: the call allocates nothing."""
    if out is None:
        raise ParallaxError(ERR_INVALID_ARG, "decode_noalloc needs out (it allocates nothing)")
    return decode(q, k_cache, v_cache, rho, seqlens, scale=scale, out=out,
                  num_splits=num_splits, stream=stream, _noalloc=True)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           rho: Optional[torch.Tensor], seqlens: Optional[torch.Tensor] = None,
           scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.float32, num_splits: int = 0,
           workspace: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None,
           _noalloc: bool = False) -> torch.Tensor:
    """Parallax decode: one query per sequence against a KV cache.

    q, rho: [B, H, D]; k_cache, v_cache: [B, H, Lmax, D] (innermost stride
    1, K and V with equal strides); seqlens: int32 [B] on the GPU or None.
    rho=None gives plain softmax attention (the rho = 0 output, computed
    without the probe products).
    A caller-owned ``workspace`` (uint8, decode_workspace_size(...) bytes)
    needs no initialisation and may be reused by later calls.
    Returns ``out`` ([B, H, D], float32 unless ``out_dtype`` says bfloat16).
    """
    _need_gpu(q, k_cache, v_cache, rho, seqlens, out, workspace)
    if q.dim() != 3 or (rho is not None and rho.shape != q.shape):
        raise ParallaxError(ERR_INVALID_ARG, "q and rho must be [B, H, D]")
    B, H, D = q.shape
    if k_cache.dim() != 4 or k_cache.shape[:2] != (B, H) or k_cache.shape[3] != D:
        raise ParallaxError(ERR_INVALID_ARG, "k_cache must be [B, H, Lmax, D]")
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ParallaxError(ERR_INVALID_ARG,
                            "v_cache must match k_cache in shape and strides")
    Lmax = k_cache.shape[2]
    dt = _dtype_code(q, "q")
    for name, t in (("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t is not None and t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} dtype differs from q")
    for name, t in (("q", q), ("rho", rho), ("k_cache", k_cache)):
        if t is not None and t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if seqlens is not None:
        if seqlens.dtype != torch.int32 or seqlens.shape != (B,):
            raise ParallaxError(ERR_INVALID_ARG, "seqlens must be int32 [B]")
        seqlens = seqlens.contiguous()
    if out is None:
        out = torch.empty((B, H, D), dtype=out_dtype, device=q.device)
    if out.shape != (B, H, D) or (out.numel() and out.stride(-1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be [B, H, D], inner stride 1")
    odt = _dtype_code(out, "out")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    args = (q.data_ptr(), q.stride(0), q.stride(1),
            rho.data_ptr() if rho is not None else None,
            rho.stride(0) if rho is not None else 0, rho.stride(1) if rho is not None else 0,
            k_cache.data_ptr(), v_cache.data_ptr(),
            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
            seqlens.data_ptr() if seqlens is not None else None,
            out.data_ptr(), out.stride(0), out.stride(1),
            B, H, D, Lmax, scale, dt, odt, int(num_splits))
    if _noalloc:
        st = library().parallax_decode_noalloc(*args, _stream(q.device, stream))
        _raise_on(st, "parallax_decode_noalloc")
        return out
    need = decode_workspace_size(B, H, D, Lmax, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = library().parallax_decode(*args, ws_ptr, ws_bytes, _stream(q.device, stream))
    _raise_on(st, "parallax_decode")
    return out


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
               cu_seqlens: torch.Tensor, max_seqlen: int, causal: bool = True,
               scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               out_dtype: torch.dtype = torch.float32,
               workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Parallax prefill over packed sequences, bf16. q, k, v, rho: [T, H, D]
    (innermost stride 1); cu_seqlens: int32 [B + 1] on the GPU, sequence b
    is rows cu_seqlens[b] .. cu_seqlens[b+1]-1; max_seqlen bounds every
    length. Returns ``out`` [T, H, D] (rows outside every sequence are left
    as they were; a new ``out`` starts zeroed)."""
    _need_gpu(q, k, v, rho, cu_seqlens, out, workspace)
    if q.dim() != 3:
        raise ParallaxError(ERR_INVALID_ARG, "q must be [T, H, D]")
    T, H, D = q.shape
    for name, t in (("k", k), ("v", v), ("rho", rho)):
        if t.shape != q.shape:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} must match q's shape")
        if t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} dtype differs from q")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho)):
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ParallaxError(ERR_INVALID_ARG, "cu_seqlens must be int32 [B + 1]")
    cu_seqlens = cu_seqlens.contiguous()
    B = cu_seqlens.numel() - 1
    dt = _dtype_code(q, "q")
    if out is None:
        out = torch.zeros((T, H, D), dtype=out_dtype, device=q.device)
    if out.shape != (T, H, D) or (out.numel() and out.stride(-1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be [T, H, D], inner stride 1")
    odt = _dtype_code(out, "out")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None:
        need = fwd_workspace_size(B, int(max_seqlen), H, D, q.dtype)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = library().parallax_fwd_varlen(
        q.data_ptr(), q.stride(0), q.stride(1), k.data_ptr(), k.stride(0), k.stride(1),
        v.data_ptr(), v.stride(0), v.stride(1), rho.data_ptr(), rho.stride(0), rho.stride(1),
        out.data_ptr(), out.stride(0), out.stride(1), cu_seqlens.data_ptr(),
        B, int(max_seqlen), H, D, scale, 1 if causal else 0, dt, odt,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(q.device, stream))
    _raise_on(st, "parallax_fwd_varlen")
    return out


def project(x: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """y = x @ w.T in bf16 (fp32 accumulation): x [M, K], w [N, K] (the
    torch Linear weight layout), N a multiple of 256, K of 64."""
    _need_gpu(x, w, out)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ParallaxError(ERR_INVALID_ARG, "x must be [M, K] and w [N, K]")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ParallaxError(ERR_UNSUPPORTED, "project takes bfloat16 tensors")
    for name, t in (("x", x), ("w", w)):
        if t.numel() and t.stride(1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: inner stride must be 1")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if out.shape != (M, N) or out.dtype != torch.bfloat16 or (out.numel() and out.stride(1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be bfloat16 [M, N], inner stride 1")
    st = library().parallax_project(x.data_ptr(), x.stride(0), w.data_ptr(), w.stride(0),
                                    out.data_ptr(), out.stride(0), M, N, K, BF16,
                                    _stream(x.device, stream))
    _raise_on(st, "parallax_project")
    return out


def fuse_qkvr_weight(w_q: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                     w_r: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stack the projection weights (torch Linear layout [out, in]) into the
    one weight `project` takes. w_r = None stacks zeros: the converted layer
    computes plain softmax attention until W_R is trained."""
    if w_r is None:
        w_r = torch.zeros_like(w_q)
    return torch.cat([w_q, w_k, w_v, w_r], dim=0).contiguous()


def split_qkvr(y: torch.Tensor, Hq: int, Hkv: int, D: int):
    """Views q [M, Hq, D], k, v [M, Hkv, D], rho [M, Hq, D] of a projection
    output y [M, (2 Hq + 2 Hkv) D]; no copy."""
    M = y.shape[0]
    widths = (Hq * D, Hkv * D, Hkv * D, Hq * D)
    if y.shape[1] != sum(widths):
        raise ParallaxError(ERR_INVALID_ARG, "y width is not 2 (Hq + Hkv) D")
    parts, o = [], 0
    for wdt, h in zip(widths, (Hq, Hkv, Hkv, Hq)):
        parts.append(y[:, o:o + wdt].view(M, h, D) if y.is_contiguous()
                     else y[:, o:o + wdt].unflatten(1, (h, D)))
        o += wdt
    return tuple(parts)


def stream_read(src: torch.Tensor, sink: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """XOR every 32-bit word of the contiguous tensor ``src`` into the int32
    ``sink`` (one element, on the GPU) with 16-byte streaming loads: the
    plain read rate of device memory, a reference for the decode kernels."""
    _need_gpu(src, sink)
    if not src.is_contiguous():
        raise ParallaxError(ERR_INVALID_ARG, "src must be contiguous")
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ParallaxError(ERR_INVALID_ARG, "sink must be int32 with one element")
    st = library().parallax_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                        sink.data_ptr(), _stream(src.device, stream))
    _raise_on(st, "parallax_stream_read")
    return sink


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
        causal: bool = True, scale: Optional[float] = None,
        out: Optional[torch.Tensor] = None,
        out_dtype: torch.dtype = torch.float32,
        workspace: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Parallax prefill over [B, N, H, D] tensors (innermost stride 1).

    bf16 inputs need a device workspace of fwd_workspace_size(...) bytes;
    one is allocated per call when `workspace` is None."""
    _need_gpu(q, k, v, rho, out, workspace)
    if q.dim() != 4:
        raise ParallaxError(ERR_INVALID_ARG, "q must be [B, N, H, D]")
    B, N, H, D = q.shape
    dt = _dtype_code(q, "q")
    for name, t in (("k", k), ("v", v), ("rho", rho)):
        if t.shape != q.shape:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} must match q's shape")
        if t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} dtype differs from q")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho)):
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=out_dtype, device=q.device)
    if out.shape != q.shape or (out.numel() and out.stride(-1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be [B, N, H, D], inner stride 1")
    odt = _dtype_code(out, "out")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    need = fwd_workspace_size(B, N, H, D, q.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = library().parallax_fwd(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
        v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
        rho.data_ptr(), rho.stride(0), rho.stride(1), rho.stride(2),
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        B, N, H, D, scale, 1 if causal else 0, dt, odt, ws_ptr, ws_bytes,
        _stream(q.device, stream))
    _raise_on(st, "parallax_fwd")
    return out


def bwd_workspace_size(B: int, N: int, H: int, D: int) -> int:
    """Bytes of device workspace parallax_bwd needs (bf16 inputs)."""
    out = ctypes.c_size_t(0)
    _raise_on(library().parallax_bwd_workspace_size(
        B, N, H, D, BF16, ctypes.byref(out)), "parallax_bwd_workspace_size")
    return out.value


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
        dout: torch.Tensor, causal: bool = True, scale: Optional[float] = None,
        grads: Optional[Sequence[torch.Tensor]] = None,
        workspace: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None):
    """Backward of fwd(): (dq, dk, dv, drho) fp32 [B, N, H, D] for bf16
    q, k, v, rho and dout (innermost stride 1). `grads` may supply the four
    output tensors; a workspace of bwd_workspace_size(...) bytes is
    allocated per call when `workspace` is None."""
    _need_gpu(q, k, v, rho, dout, workspace, *(grads or ()))
    if q.dim() != 4:
        raise ParallaxError(ERR_INVALID_ARG, "q must be [B, N, H, D]")
    B, N, H, D = q.shape
    dt = _dtype_code(q, "q")
    for name, t in (("k", k), ("v", v), ("rho", rho), ("dout", dout)):
        if t.shape != q.shape:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} must match q's shape")
        if t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} dtype differs from q")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho), ("dout", dout)):
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if grads is None:
        grads = [torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
                 for _ in range(4)]
    for g in grads:
        if g.shape != q.shape or g.dtype != torch.float32 or (g.numel() and g.stride(-1) != 1):
            raise ParallaxError(ERR_INVALID_ARG, "gradients must be fp32 [B, N, H, D], inner stride 1")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if dt == BF16 and B * N * H:
        need = bwd_workspace_size(B, N, H, D)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = []
    for t in (q, k, v, rho, dout, *grads):
        args += [t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)]
    st = library().parallax_bwd(*args, B, N, H, D, scale, 1 if causal else 0, dt,
                                ws_ptr, ws_bytes, _stream(q.device, stream))
    _raise_on(st, "parallax_bwd")
    return tuple(grads)


def fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
              causal: bool = True, scale: Optional[float] = None,
              out: Optional[torch.Tensor] = None,
              out_dtype: torch.dtype = torch.float32,
              saved: Optional[Sequence[torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None):
    """Training forward (bf16): returns (out, vbar, lse_rbar) with vbar fp32
    [B, N, H, D] and lse_rbar fp32 [B, H, N, 2], the tensors bwd_saved
    takes; `saved` may supply (vbar, lse_rbar)."""
    _need_gpu(q, k, v, rho, out, workspace, *(saved or ()))
    if q.dim() != 4:
        raise ParallaxError(ERR_INVALID_ARG, "q must be [B, N, H, D]")
    B, N, H, D = q.shape
    dt = _dtype_code(q, "q")
    for name, t in (("k", k), ("v", v), ("rho", rho)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} must match q's shape and dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho)):
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=out_dtype, device=q.device)
    if out.shape != q.shape or (out.numel() and out.stride(-1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be [B, N, H, D], inner stride 1")
    if saved is None:
        saved = (torch.empty((B, N, H, D), dtype=torch.float32, device=q.device),
                 torch.empty((B, H, N, 2), dtype=torch.float32, device=q.device))
    vbar, lse_rbar = saved
    if (vbar.shape != (B, N, H, D) or lse_rbar.shape != (B, H, N, 2)
            or vbar.dtype != torch.float32 or lse_rbar.dtype != torch.float32
            or not vbar.is_contiguous() or not lse_rbar.is_contiguous()):
        raise ParallaxError(ERR_INVALID_ARG,
                            "saved must be contiguous fp32 [B, N, H, D] and [B, H, N, 2]")
    odt = _dtype_code(out, "out")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None:
        workspace = torch.empty(max(16, fwd_workspace_size(B, N, H, D, q.dtype)),
                                dtype=torch.uint8, device=q.device)
    st = library().parallax_fwd_train(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
        k.data_ptr(), k.stride(0), k.stride(1), k.stride(2),
        v.data_ptr(), v.stride(0), v.stride(1), v.stride(2),
        rho.data_ptr(), rho.stride(0), rho.stride(1), rho.stride(2),
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        vbar.data_ptr(), lse_rbar.data_ptr(),
        B, N, H, D, scale, 1 if causal else 0, dt, odt,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(q.device, stream))
    _raise_on(st, "parallax_fwd_train")
    return out, vbar, lse_rbar


def bwd_saved(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rho: torch.Tensor,
              dout: torch.Tensor, out: torch.Tensor, vbar: torch.Tensor,
              lse_rbar: torch.Tensor, causal: bool = True, scale: Optional[float] = None,
              grads: Optional[Sequence[torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None,
              stream: Optional[torch.cuda.Stream] = None):
    """bwd() from fwd_train()'s saved (out, vbar, lse_rbar): no second
    forward pass. Returns (dq, dk, dv, drho) fp32 [B, N, H, D]."""
    _need_gpu(q, k, v, rho, dout, out, vbar, lse_rbar, workspace, *(grads or ()))
    B, N, H, D = q.shape
    dt = _dtype_code(q, "q")
    for name, t in (("k", k), ("v", v), ("rho", rho), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} must match q's shape and dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("rho", rho), ("dout", dout), ("out", out)):
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if out.shape != q.shape:
        raise ParallaxError(ERR_INVALID_ARG, "out must be [B, N, H, D]")
    if (vbar.shape != (B, N, H, D) or lse_rbar.shape != (B, H, N, 2)
            or not vbar.is_contiguous() or not lse_rbar.is_contiguous()):
        raise ParallaxError(ERR_INVALID_ARG, "vbar / lse_rbar as written by fwd_train")
    if grads is None:
        grads = [torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
                 for _ in range(4)]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None and B * N * H:
        workspace = torch.empty(bwd_workspace_size(B, N, H, D), dtype=torch.uint8,
                                device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = []
    for t in (q, k, v, rho, dout, out):
        args += [t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)]
    args += [_dtype_code(out, "out"), vbar.data_ptr(), lse_rbar.data_ptr()]
    for t in grads:
        args += [t.data_ptr(), t.stride(0), t.stride(1), t.stride(2)]
    st = library().parallax_bwd_saved(*args, B, N, H, D, scale, 1 if causal else 0, dt,
                                      ws_ptr, ws_bytes, _stream(q.device, stream))
    _raise_on(st, "parallax_bwd_saved")
    return tuple(grads)


def decode_gqa_splits(B: int, Hq: int, Hkv: int, D: int, Lmax: int,
                      num_splits: int = 0, paged: bool = False) -> int:
    """Number of KV splits parallax_decode_gqa uses for these sizes (paged:
    the call has a block table)."""
    out = _int(0)
    _raise_on(library().parallax_decode_gqa_splits(B, Hq, Hkv, D, Lmax, int(bool(paged)),
                                                   num_splits, ctypes.byref(out)),
              "parallax_decode_gqa_splits")
    return out.value


def decode_gqa_workspace_size(B: int, Hq: int, Hkv: int, D: int, Lmax: int,
                              num_splits: int = 0, paged: bool = False) -> int:
    """Bytes of device workspace parallax_decode_gqa needs (paged: the call
    has a block table)."""
    out = ctypes.c_size_t(0)
    _raise_on(library().parallax_decode_gqa_workspace_size(
        B, Hq, Hkv, D, Lmax, int(bool(paged)), num_splits, ctypes.byref(out)),
        "parallax_decode_gqa_workspace_size")
    return out.value


def decode_gqa(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               rho: torch.Tensor, seqlens: Optional[torch.Tensor] = None,
               block_table: Optional[torch.Tensor] = None,
               scale: Optional[float] = None, num_splits: int = 0,
               out: Optional[torch.Tensor] = None,
               out_dtype: torch.dtype = torch.float32,
               workspace: Optional[torch.Tensor] = None,
               stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Grouped-query decode, bf16. q, rho [B, Hq, D].

    Without block_table the caches are [B, Hkv, Lmax, D]; with it they are
    paged [num_pages, page_size, Hkv, D], block_table int32 [B, max_pages]
    and seqlens int32 [B] is required (Lmax = max_pages * page_size)."""
    _need_gpu(q, k_cache, v_cache, rho, seqlens, block_table, out, workspace)
    if q.dim() != 3 or rho.shape != q.shape:
        raise ParallaxError(ERR_INVALID_ARG, "q and rho must be [B, Hq, D]")
    B, Hq, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ParallaxError(ERR_INVALID_ARG, "k_cache and v_cache must match, 4-D")
    dt = _dtype_code(q, "q")
    for name, t in (("rho", rho), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != q.dtype:
            raise ParallaxError(ERR_INVALID_ARG, f"{name} dtype differs from q")
        if t.numel() and t.stride(-1) != 1:
            raise ParallaxError(ERR_UNSUPPORTED, f"{name}: head_dim stride must be 1")
    if block_table is None:
        _, Hkv, Lmax, _ = k_cache.shape
        kv_sb, kv_sh, kv_sl = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
        bt_ptr, bt_sb, page, npages = None, 0, 0, 0
    else:
        npages, page, Hkv, _ = k_cache.shape
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ParallaxError(ERR_INVALID_ARG, "block_table must be int32 [B, max_pages]")
        if seqlens is None:
            raise ParallaxError(ERR_INVALID_ARG, "a paged cache needs seqlens")
        Lmax = block_table.shape[1] * page
        kv_sb, kv_sl, kv_sh = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
        bt_ptr, bt_sb = block_table.data_ptr(), block_table.stride(0)
    if k_cache.shape[-1] != D:
        raise ParallaxError(ERR_INVALID_ARG, "head_dim mismatch")
    if seqlens is not None:
        if seqlens.dtype != torch.int32 or seqlens.shape != (B,) or not seqlens.is_contiguous():
            raise ParallaxError(ERR_INVALID_ARG, "seqlens must be contiguous int32 [B]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    if out.shape != (B, Hq, D) or (out.numel() and out.stride(-1) != 1):
        raise ParallaxError(ERR_INVALID_ARG, "out must be [B, Hq, D], inner stride 1")
    odt = _dtype_code(out, "out")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if Hkv <= 0 or Hq % Hkv:
        raise ParallaxError(ERR_INVALID_ARG, "Hq must be a multiple of Hkv")
    need = decode_gqa_workspace_size(B, Hq, Hkv, D, Lmax, num_splits,
                                     paged=block_table is not None)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = library().parallax_decode_gqa(
        q.data_ptr(), q.stride(0), q.stride(1),
        rho.data_ptr(), rho.stride(0), rho.stride(1),
        k_cache.data_ptr(), v_cache.data_ptr(), kv_sb, kv_sh, kv_sl,
        bt_ptr, bt_sb, page, npages,
        seqlens.data_ptr() if seqlens is not None else None,
        out.data_ptr(), out.stride(0), out.stride(1),
        B, Hq, Hkv, D, Lmax, scale, dt, odt, int(num_splits),
        ws_ptr, ws_bytes, _stream(q.device, stream))
    _raise_on(st, "parallax_decode_gqa")
    return out
