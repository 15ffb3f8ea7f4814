"""Python binding of librelattn (relation-aware self-attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of librelattn.so, reached through its C ABI (include/relattn.h).
PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "validate", "fwd_offset_bias", "validate_offset_bias", "decode",
           "decode_workspace_size", "debug_indices",
           "RelattnError", "library_path",
           "OK", "INVALID_ARGUMENT", "UNSUPPORTED", "NO_DEVICE", "LAUNCH_FAILED"]

OK, INVALID_ARGUMENT, UNSUPPORTED, NO_DEVICE, LAUNCH_FAILED = 0, -1, -2, -3, -4
_F32, _BF16 = 0, 1

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librelattn.so")


class RelattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 4),
                ("stride", ctypes.c_int64 * 4)]


class _Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("key_lens", ctypes.c_void_p)]


class _T5(ctypes.Structure):
    _fields_ = [("num_buckets", ctypes.c_int32), ("max_distance", ctypes.c_int32),
                ("bidirectional", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is not built; run `python -m relative_position_encoding_amd.build`")
    lib = ctypes.CDLL(library_path)
    P = ctypes.POINTER
    args = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor),
            P(_T5), ctypes.c_int32, ctypes.c_float, P(_Mask), P(_Tensor)]
    lib.relattn_fwd.argtypes = args + [ctypes.c_void_p]
    lib.relattn_fwd.restype = ctypes.c_int
    lib.relattn_validate.argtypes = args
    lib.relattn_validate.restype = ctypes.c_int
    dec = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor),
           P(_T5), ctypes.c_int32, ctypes.c_float]
    lib.relattn_decode.argtypes = dec + [ctypes.c_void_p, P(_Tensor), ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    lib.relattn_decode.restype = ctypes.c_int
    lib.relattn_decode_workspace_size.argtypes = dec + [P(_Tensor), P(ctypes.c_size_t)]
    lib.relattn_decode_workspace_size.restype = ctypes.c_int
    ob = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_float,
          P(_Mask), P(_Tensor)]
    lib.relattn_fwd_offset_bias.argtypes = ob + [ctypes.c_void_p]
    lib.relattn_fwd_offset_bias.restype = ctypes.c_int
    lib.relattn_validate_offset_bias.argtypes = ob
    lib.relattn_validate_offset_bias.restype = ctypes.c_int
    lib.relattn_debug_indices.argtypes = [ctypes.c_int32, ctypes.c_int32, P(_T5),
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.relattn_debug_indices.restype = ctypes.c_int
    lib.relattn_strerror.argtypes = [ctypes.c_int]
    lib.relattn_strerror.restype = ctypes.c_char_p
    lib.relattn_last_error.argtypes = []
    lib.relattn_last_error.restype = ctypes.c_char_p
    lib.relattn_version.argtypes = []
    lib.relattn_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return _F32
    if t.dtype == torch.bfloat16:
        return _BF16
    return 99  # rejected by the library


def _view(t):
    if t is None:
        return None
    v = _Tensor()
    v.data = t.data_ptr() or None
    v.dtype = _dtype_code(t)
    v.ndim = t.dim()
    for i in range(min(t.dim(), 4)):
        v.shape[i] = t.shape[i]
        v.stride[i] = t.stride(i)
    return v


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
          max_distance, bidirectional, scale, out):
    keep = []  # keep ctypes objects alive through the call
    views = [_view(x) for x in (q, k, v, wK, wV, t5_bias)]
    keep += views
    t5 = None
    if t5_bias is not None:
        t5 = _T5(int(num_buckets), int(max_distance), 1 if bidirectional else 0)
    mask = None
    if causal or key_lens is not None:
        mask = _Mask(1 if causal else 0, key_lens.data_ptr() if key_lens is not None else None)
    outv = _view(out)
    keep += [t5, mask, outv]
    args = [_ref(x) for x in views] + [_ref(t5), int(clip),
                                        float(0.0 if scale is None else scale),
                                        _ref(mask), _ref(outv)]
    return args, keep


def _raise(lib, status):
    msg = lib.relattn_last_error().decode() or lib.relattn_strerror(status).decode()
    raise RelattnError(status, f"relattn: {lib.relattn_strerror(status).decode()}: {msg}")


def fwd(q, k, v, wK=None, wV=None, *, clip=0, causal=False, key_lens=None,
        t5_bias=None, num_buckets=32, max_distance=128, bidirectional=True,
        scale=None, out=None, stream=None):
    """Relation-aware self-attention forward (or T5 bias when t5_bias is given).

    q, k, v: [B, H, n, d] CUDA(HIP) tensors (float32 or bfloat16);
    wK, wV: [H or 1, 2*clip+1, d] tables of the same dtype (None = absent);
    key_lens: int32 [B] device tensor; t5_bias: float32 [num_buckets, H].
    Enqueued on ``stream`` (default: torch's current stream); returns ``out``.
    """
    import torch
    lib = _load()
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: key_lens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    args, keep = _args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                       max_distance, bidirectional, scale, out)
    st = lib.relattn_fwd(*args, ctypes.c_void_p(stream))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


def validate(q, k, v, wK=None, wV=None, *, clip=0, causal=False, key_lens=None,
             t5_bias=None, num_buckets=32, max_distance=128, bidirectional=True,
             scale=None, out=None):
    """Host-only argument check of ``fwd``; returns the library status code."""
    lib = _load()
    if out is None:
        out = q
    args, keep = _args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                       max_distance, bidirectional, scale, out)
    st = lib.relattn_validate(*args)
    del keep
    return st


def last_error() -> str:
    return _load().relattn_last_error().decode()


def debug_indices(n, clip=0, *, t5=False, num_buckets=32, max_distance=128,
                  bidirectional=True, device="cuda", stream=None):
    """Per-offset integer indices computed on the GPU by the kernels' own index
    functions: entry delta + n - 1 holds clip(delta, clip) + clip, or the T5
    bucket of delta when ``t5`` is true."""
    import torch
    lib = _load()
    out = torch.empty(2 * n - 1, dtype=torch.int32, device=device)
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    t5p = _T5(int(num_buckets), int(max_distance), 1 if bidirectional else 0) if t5 else None
    st = lib.relattn_debug_indices(int(n), int(clip), _ref(t5p), ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(stream))
    if st != OK:
        _raise(lib, st)
    return out


def _dec_args(q, k, v, wK, wV, t5_bias, clip, num_buckets, max_distance, bidirectional,
              scale):
    keep = []
    views = [_view(x) for x in (q, k, v, wK, wV, t5_bias)]
    t5 = None
    if t5_bias is not None:
        t5 = _T5(int(num_buckets), int(max_distance), 1 if bidirectional else 0)
    keep += views + [t5]
    args = [_ref(x) for x in views] + [_ref(t5), int(clip),
                                        float(0.0 if scale is None else scale)]
    return args, keep


def decode_workspace_size(q, k, v, wK=None, wV=None, *, clip=0, t5_bias=None,
                          num_buckets=32, max_distance=128, bidirectional=True, scale=None,
                          out=None):
    """Workspace bytes ``decode`` needs (host-only check of its arguments);
    raises RelattnError on invalid arguments."""
    lib = _load()
    args, keep = _dec_args(q, k, v, wK, wV, t5_bias, clip, num_buckets, max_distance,
                           bidirectional, scale)
    outv = _view(q if out is None else out)
    nbytes = ctypes.c_size_t(0)
    st = lib.relattn_decode_workspace_size(*args, ctypes.byref(outv), ctypes.byref(nbytes))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(nbytes.value)


def decode(q, k, v, wK=None, wV=None, *, clip=0, cache_lens=None, t5_bias=None,
           num_buckets=32, max_distance=128, bidirectional=True, scale=None, out=None,
           workspace=None, stream=None):
    """Incremental decoding: q [B, H, Tq, d] holds the newest Tq positions of
    each sequence, k and v [B, H, L, d] its cache; query t of batch b sits at
    position cache_lens[b] - Tq + t (cache_lens: int32 [B] device tensor, None
    = L) and sees the keys up to it.  Tables and T5 arguments as for ``fwd``.
    ``workspace`` (a device tensor of at least ``decode_workspace_size`` bytes)
    is allocated through torch when not given.  Returns ``out``."""
    import torch
    lib = _load()
    if cache_lens is not None and cache_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: cache_lens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    need = decode_workspace_size(q, k, v, wK, wV, clip=clip, t5_bias=t5_bias,
                                 num_buckets=num_buckets, max_distance=max_distance,
                                 bidirectional=bidirectional, scale=scale, out=out)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    args, keep = _dec_args(q, k, v, wK, wV, t5_bias, clip, num_buckets, max_distance,
                           bidirectional, scale)
    outv = _view(out)
    st = lib.relattn_decode(*args,
                            ctypes.c_void_p(cache_lens.data_ptr() if cache_lens is not None
                                            else None),
                            ctypes.byref(outv), ctypes.c_void_p(workspace.data_ptr()),
                            ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                            ctypes.c_void_p(stream))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


def _ob_args(q, k, v, bias, window, causal, key_lens, scale, out):
    views = [_view(x) for x in (q, k, v, bias)]
    mask = None
    if causal or key_lens is not None:
        mask = _Mask(1 if causal else 0, key_lens.data_ptr() if key_lens is not None else None)
    outv = _view(out)
    args = [_ref(x) for x in views] + [int(window), float(0.0 if scale is None else scale),
                                        _ref(mask), _ref(outv)]
    return args, views + [mask, outv]


def fwd_offset_bias(q, k, v, bias, window, *, causal=False, key_lens=None, scale=None,
                    out=None, stream=None):
    """Attention with a scalar bias by clipped offset: bias [H or 1, 2*window+1]
    float32, entry window + delta for offset delta = j - i (ALiBi:
    -m_h * |delta|).  Other arguments as for ``fwd``; returns ``out``."""
    import torch
    lib = _load()
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: key_lens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    args, keep = _ob_args(q, k, v, bias, window, causal, key_lens, scale, out)
    st = lib.relattn_fwd_offset_bias(*args, ctypes.c_void_p(stream))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


def validate_offset_bias(q, k, v, bias, window, *, causal=False, key_lens=None, scale=None,
                         out=None):
    """Host-only argument check of ``fwd_offset_bias``; returns the status code."""
    lib = _load()
    args, keep = _ob_args(q, k, v, bias, window, causal, key_lens, scale, q if out is None else out)
    st = lib.relattn_validate_offset_bias(*args)
    del keep
    return st
