"""Python binding of librelattn (relation-aware self-attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of librelattn.so, reached through its C ABI (include/relattn.h).
PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os

__all__ = ["fwd", "validate", "fwd_offset_bias", "validate_offset_bias", "decode",
           "decode_workspace_size", "decode_noalloc", "debug_indices", "fwd_lse", "fwd_offset_bias_lse",
           "bwd", "bwd_workspace_size", "bwd_offset_bias", "bwd_offset_bias_workspace_size",
           "attention", "attention_offset_bias", "fwd_xl", "validate_xl", "fwd_grid_bias",
           "validate_grid_bias", "fwd_grid_bias_lse", "bwd_grid_bias",
           "bwd_grid_bias_workspace_size", "attention_grid_bias", "fwd_edge_bias",
           "fwd_edge_bias_lse", "bwd_edge_bias", "bwd_edge_bias_workspace_size",
           "attention_edge_bias", "fwd_xl_lse", "bwd_xl", "bwd_xl_workspace_size", "attention_xl",
           "fwd_edge_tables_lse", "bwd_edge_tables", "bwd_edge_tables_workspace_size",
           "attention_edge_tables", "validate_edge_bias", "edge_label_buffer",
           "fwd_edge_tables", "validate_edge_tables", "decode_offset_bias",
           "decode_offset_bias_workspace_size", "decode_xl", "decode_xl_workspace_size",
           "RelattnError", "library_path",
           "OK", "INVALID_ARGUMENT", "UNSUPPORTED", "NO_DEVICE", "LAUNCH_FAILED"]

OK, INVALID_ARGUMENT, UNSUPPORTED, NO_DEVICE, LAUNCH_FAILED = 0, -1, -2, -3, -4
_F32, _BF16, _U8 = 0, 1, 2

# RELATTN_LIBRARY names another build of the same library (e.g. the host-sanitized one)
library_path = os.environ.get("RELATTN_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "librelattn.so")


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
    lib.relattn_decode_noalloc.argtypes = dec + [ctypes.c_void_p, P(_Tensor), ctypes.c_void_p]
    lib.relattn_decode_noalloc.restype = ctypes.c_int
    decob = [P(_Tensor)] * 4 + [ctypes.c_int32, ctypes.c_float]
    lib.relattn_decode_offset_bias.argtypes = decob + [ctypes.c_void_p, P(_Tensor),
                                                       ctypes.c_void_p, ctypes.c_size_t,
                                                       ctypes.c_void_p]
    lib.relattn_decode_offset_bias.restype = ctypes.c_int
    lib.relattn_decode_offset_bias_workspace_size.argtypes = decob + [P(_Tensor),
                                                                      P(ctypes.c_size_t)]
    lib.relattn_decode_offset_bias_workspace_size.restype = ctypes.c_int
    decxl = [P(_Tensor)] * 6 + [ctypes.c_int32, ctypes.c_float]
    lib.relattn_decode_xl.argtypes = decxl + [ctypes.c_void_p, P(_Tensor), ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p]
    lib.relattn_decode_xl.restype = ctypes.c_int
    lib.relattn_decode_xl_workspace_size.argtypes = decxl + [P(_Tensor), P(ctypes.c_size_t)]
    lib.relattn_decode_xl_workspace_size.restype = ctypes.c_int
    ob = [P(_Tensor), P(_Tensor), P(_Tensor), P(_Tensor), ctypes.c_int32, ctypes.c_float,
          P(_Mask), P(_Tensor)]
    lib.relattn_fwd_offset_bias.argtypes = ob + [ctypes.c_void_p]
    lib.relattn_fwd_offset_bias.restype = ctypes.c_int
    lib.relattn_validate_offset_bias.argtypes = ob
    lib.relattn_validate_offset_bias.restype = ctypes.c_int
    lib.relattn_fwd_lse.argtypes = args + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_lse.restype = ctypes.c_int
    lib.relattn_fwd_offset_bias_lse.argtypes = ob + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_offset_bias_lse.restype = ctypes.c_int
    # q k v wK wV t5_bias t5 clip scale mask out dout lse dq dk dv dwK dwV dbias
    bw = args + [P(_Tensor)] * 8
    lib.relattn_bwd.argtypes = bw + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.relattn_bwd.restype = ctypes.c_int
    lib.relattn_bwd_workspace_size.argtypes = bw + [P(ctypes.c_size_t)]
    lib.relattn_bwd_workspace_size.restype = ctypes.c_int
    # q k v bias window scale mask out dout lse dq dk dv dbias
    obw = ob + [P(_Tensor)] * 6
    lib.relattn_bwd_offset_bias.argtypes = obw + [ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p]
    lib.relattn_bwd_offset_bias.restype = ctypes.c_int
    lib.relattn_bwd_offset_bias_workspace_size.argtypes = obw + [P(ctypes.c_size_t)]
    lib.relattn_bwd_offset_bias_workspace_size.restype = ctypes.c_int
    xl = [P(_Tensor)] * 6 + [ctypes.c_int32, ctypes.c_float, P(_Mask), P(_Tensor)]
    lib.relattn_fwd_xl.argtypes = xl + [ctypes.c_void_p]
    lib.relattn_fwd_xl.restype = ctypes.c_int
    lib.relattn_validate_xl.argtypes = xl
    lib.relattn_validate_xl.restype = ctypes.c_int
    lib.relattn_fwd_xl_lse.argtypes = xl + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_xl_lse.restype = ctypes.c_int
    # q k v R u v window scale mask out dout lse dq dk dv dR du dv_bias
    xlw = xl + [P(_Tensor)] * 8
    lib.relattn_bwd_xl.argtypes = xlw + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.relattn_bwd_xl.restype = ctypes.c_int
    lib.relattn_bwd_xl_workspace_size.argtypes = xlw + [P(ctypes.c_size_t)]
    lib.relattn_bwd_xl_workspace_size.restype = ctypes.c_int
    lib.relattn_fwd_grid_bias.argtypes = ob + [ctypes.c_void_p]
    lib.relattn_fwd_grid_bias.restype = ctypes.c_int
    lib.relattn_validate_grid_bias.argtypes = ob
    lib.relattn_validate_grid_bias.restype = ctypes.c_int
    lib.relattn_fwd_grid_bias_lse.argtypes = ob + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_grid_bias_lse.restype = ctypes.c_int
    lib.relattn_bwd_grid_bias.argtypes = obw + [ctypes.c_void_p, ctypes.c_size_t,
                                                ctypes.c_void_p]
    lib.relattn_bwd_grid_bias.restype = ctypes.c_int
    lib.relattn_bwd_grid_bias_workspace_size.argtypes = obw + [P(ctypes.c_size_t)]
    lib.relattn_bwd_grid_bias_workspace_size.restype = ctypes.c_int
    edge = [P(_Tensor)] * 5 + [ctypes.c_float, P(_Mask), P(_Tensor)]
    lib.relattn_fwd_edge_bias.argtypes = edge + [ctypes.c_void_p]
    lib.relattn_fwd_edge_bias.restype = ctypes.c_int
    lib.relattn_validate_edge_bias.argtypes = edge
    lib.relattn_validate_edge_bias.restype = ctypes.c_int
    lib.relattn_fwd_edge_bias_lse.argtypes = edge + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_edge_bias_lse.restype = ctypes.c_int
    # q k v labels bias scale mask out dout lse dq dk dv dbias
    edgew = edge + [P(_Tensor)] * 6
    lib.relattn_bwd_edge_bias.argtypes = edgew + [ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p]
    lib.relattn_bwd_edge_bias.restype = ctypes.c_int
    lib.relattn_bwd_edge_bias_workspace_size.argtypes = edgew + [P(ctypes.c_size_t)]
    lib.relattn_bwd_edge_bias_workspace_size.restype = ctypes.c_int
    edget = [P(_Tensor)] * 6 + [ctypes.c_float, P(_Mask), P(_Tensor)]
    lib.relattn_fwd_edge_tables.argtypes = edget + [ctypes.c_void_p]
    lib.relattn_fwd_edge_tables.restype = ctypes.c_int
    lib.relattn_validate_edge_tables.argtypes = edget
    lib.relattn_validate_edge_tables.restype = ctypes.c_int
    lib.relattn_fwd_edge_tables_lse.argtypes = edget + [P(_Tensor), ctypes.c_void_p]
    lib.relattn_fwd_edge_tables_lse.restype = ctypes.c_int
    # q k v labels wK wV scale mask out dout lse dq dk dv dwK dwV
    edgetw = edget + [P(_Tensor)] * 7
    lib.relattn_bwd_edge_tables.argtypes = edgetw + [ctypes.c_void_p, ctypes.c_size_t,
                                                     ctypes.c_void_p]
    lib.relattn_bwd_edge_tables.restype = ctypes.c_int
    lib.relattn_bwd_edge_tables_workspace_size.argtypes = edgetw + [P(ctypes.c_size_t)]
    lib.relattn_bwd_edge_tables_workspace_size.restype = ctypes.c_int
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
    if t.dtype == torch.uint8:
        return _U8
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


def _on_stream(fn):
    """Run a binding call with the stream it enqueues on as torch's current
    stream.  Every tensor the binding allocates for the call (outputs,
    workspace) then comes from the caching allocator's pool of that stream, so
    a workspace dropped when the call returns is handed out again only to work
    ordered after the kernels that use it, whichever stream the caller names.
    A raw hipStream_t handle is wrapped as an external torch stream."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        import torch
        if not hasattr(stream, "cuda_stream"):
            stream = torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return call


@_on_stream
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


@_on_stream
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


@_on_stream
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


def decode_noalloc(q, k, v, wK=None, wV=None, *, clip=0, cache_lens=None, t5_bias=None,
                   num_buckets=32, max_distance=128, bidirectional=True, scale=None, out,
                   stream=None):
    """``decode`` through the entry point that allocates nothing on the device:
    the library's static per-device scratch stands in for the workspace (at
    most 4 MiB of it; larger shapes raise UNSUPPORTED).  ``out`` must be given
    (the caller owns every buffer).  Calls on one device share the scratch:
    calls that overlap in time race.  Returns ``out``."""
    import torch
    lib = _load()
    if cache_lens is not None and cache_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: cache_lens must be int32")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    args, keep = _dec_args(q, k, v, wK, wV, t5_bias, clip, num_buckets, max_distance,
                           bidirectional, scale)
    outv = _view(out)
    st = lib.relattn_decode_noalloc(*args,
                                    ctypes.c_void_p(cache_lens.data_ptr() if cache_lens is not None
                                                    else None),
                                    ctypes.byref(outv), ctypes.c_void_p(stream))
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


@_on_stream
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


# ---------------------------------------------------------------------------
# training: forward with row statistics, backward
# ---------------------------------------------------------------------------

def _stream_of(q, stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream(q.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check_lens(key_lens):
    import torch
    if key_lens is not None and key_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: key_lens must be int32")


def _new_lse(q):
    import torch
    return torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)


@_on_stream
def fwd_lse(q, k, v, wK=None, wV=None, *, clip=0, causal=False, key_lens=None,
            t5_bias=None, num_buckets=32, max_distance=128, bidirectional=True,
            scale=None, out=None, lse=None, stream=None):
    """``fwd`` that also writes each row's log-sum-exp of its logits (natural
    log, float32 [B, H, n]; -inf for a row that sees no key), the statistic
    ``bwd`` takes.  Returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                       max_distance, bidirectional, scale, out)
    lv = _view(lse)
    st = lib.relattn_fwd_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


@_on_stream
def fwd_offset_bias_lse(q, k, v, bias, window, *, causal=False, key_lens=None, scale=None,
                        out=None, lse=None, stream=None):
    """``fwd_offset_bias`` with the row log-sum-exp; returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _ob_args(q, k, v, bias, window, causal, key_lens, scale, out)
    lv = _view(lse)
    st = lib.relattn_fwd_offset_bias_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


def _bwd_outputs(q, wK, wV, bias, dq, dk, dv, dwK, dwV, dbias, want_dwk, want_dwv,
                 want_dbias):
    import torch

    def new_like_q(x):
        return x if x is not None else torch.empty_like(q, memory_format=torch.contiguous_format)

    def new_f32(x, ref, want):
        if x is not None or ref is None or not want:
            return x
        return torch.empty(ref.shape, dtype=torch.float32, device=q.device)
    return (new_like_q(dq), new_like_q(dk), new_like_q(dv), new_f32(dwK, wK, want_dwk),
            new_f32(dwV, wV, want_dwv), new_f32(dbias, bias, want_dbias))


def _bwd_args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets, max_distance,
              bidirectional, scale, out, dout, lse, grads):
    args, keep = _args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                       max_distance, bidirectional, scale, out)
    extra = [_view(x) for x in (dout, lse) + tuple(grads)]
    return args + [_ref(x) for x in extra], keep + extra


def bwd_workspace_size(q, k, v, wK=None, wV=None, *, out, dout, lse, clip=0, causal=False,
                       key_lens=None, t5_bias=None, num_buckets=32, max_distance=128,
                       bidirectional=True, scale=None, dq=None, dk=None, dv=None, dwK=None,
                       dwV=None, dbias=None, want_dwk=True, want_dwv=True, want_dbias=True):
    """Workspace bytes ``bwd`` needs for these shapes (host only)."""
    lib = _load()
    grads = _bwd_outputs(q, wK, wV, t5_bias, dq if dq is not None else q,
                         dk if dk is not None else q, dv if dv is not None else q, dwK, dwV,
                         dbias, want_dwk, want_dwv, want_dbias)
    args, keep = _bwd_args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                           max_distance, bidirectional, scale, out, dout, lse, grads)
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd(q, k, v, wK=None, wV=None, *, out, dout, lse, clip=0, causal=False, key_lens=None,
        t5_bias=None, num_buckets=32, max_distance=128, bidirectional=True, scale=None,
        dq=None, dk=None, dv=None, dwK=None, dwV=None, dbias=None, want_dwk=True,
        want_dwv=True, want_dbias=True, workspace=None, stream=None):
    """Gradients of sum(dout * out) for the attention ``fwd_lse`` computed.

    out, lse: the forward's output and row log-sum-exp; dout: dL/d out.
    Returns (dq, dk, dv, dwK, dwV, dbias): dq, dk, dv like q; table gradients
    float32 like wK / wV (None when the table is absent or not wanted); dbias
    float32 like t5_bias.  ``workspace``: a uint8 device tensor of at least
    ``bwd_workspace_size`` bytes (allocated here when None)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    grads = _bwd_outputs(q, wK, wV, t5_bias, dq, dk, dv, dwK, dwV, dbias, want_dwk,
                         want_dwv, want_dbias)
    args, keep = _bwd_args(q, k, v, wK, wV, t5_bias, clip, causal, key_lens, num_buckets,
                           max_distance, bidirectional, scale, out, dout, lse, grads)
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd(*args, ctypes.c_void_p(workspace.data_ptr()),
                         ctypes.c_size_t(workspace.numel()),
                         ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return grads


def _bwd_ob_args(q, k, v, bias, window, causal, key_lens, scale, out, dout, lse, grads):
    args, keep = _ob_args(q, k, v, bias, window, causal, key_lens, scale, out)
    extra = [_view(x) for x in (dout, lse) + tuple(grads)]
    return args + [_ref(x) for x in extra], keep + extra


def bwd_offset_bias_workspace_size(q, k, v, bias, window, *, out, dout, lse, causal=False,
                                   key_lens=None, scale=None, want_dbias=True):
    """Workspace bytes ``bwd_offset_bias`` needs (host only)."""
    lib = _load()
    db = _bwd_outputs(q, None, None, bias, q, q, q, None, None, None, False, False,
                      want_dbias)[5]
    args, keep = _bwd_ob_args(q, k, v, bias, window, causal, key_lens, scale, out, dout, lse,
                              (q, q, q, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_offset_bias_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd_offset_bias(q, k, v, bias, window, *, out, dout, lse, causal=False, key_lens=None,
                    scale=None, dq=None, dk=None, dv=None, dbias=None, want_dbias=True,
                    workspace=None, stream=None):
    """Gradients for ``fwd_offset_bias_lse``: returns (dq, dk, dv, dbias); dbias
    float32 like ``bias`` (None when not wanted, e.g. fixed ALiBi slopes)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    dq, dk, dv, _, _, db = _bwd_outputs(q, None, None, bias, dq, dk, dv, None, None, dbias,
                                        False, False, want_dbias)
    args, keep = _bwd_ob_args(q, k, v, bias, window, causal, key_lens, scale, out, dout, lse,
                              (dq, dk, dv, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_offset_bias_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd_offset_bias(*args, ctypes.c_void_p(workspace.data_ptr()),
                                     ctypes.c_size_t(workspace.numel()),
                                     ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return dq, dk, dv, db


def _autograd_fn():
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, wK, wV, t5_bias, opts):
            out, lse = fwd_lse(q, k, v, wK, wV, t5_bias=t5_bias, **opts)
            ctx.save_for_backward(q, k, v, wK, wV, t5_bias, out, lse)
            ctx.opts = opts
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, wK, wV, t5_bias, out, lse = ctx.saved_tensors
            dout = dout.contiguous()
            g = bwd(q, k, v, wK, wV, t5_bias=t5_bias, out=out, dout=dout, lse=lse,
                    want_dwk=ctx.needs_input_grad[3], want_dwv=ctx.needs_input_grad[4],
                    want_dbias=ctx.needs_input_grad[5], **ctx.opts)
            dq, dk, dv, dwK, dwV, db = g
            cast = lambda x, ref: None if x is None else x.to(ref.dtype)
            return dq, dk, dv, cast(dwK, wK), cast(dwV, wV), db, None

    class _AttentionOB(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, bias, window, opts):
            out, lse = fwd_offset_bias_lse(q, k, v, bias, window, **opts)
            ctx.save_for_backward(q, k, v, bias, out, lse)
            ctx.window, ctx.opts = window, opts
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, bias, out, lse = ctx.saved_tensors
            dq, dk, dv, db = bwd_offset_bias(q, k, v, bias, ctx.window, out=out,
                                             dout=dout.contiguous(), lse=lse,
                                             want_dbias=ctx.needs_input_grad[3], **ctx.opts)
            return dq, dk, dv, db, None, None

    return _Attention, _AttentionOB


_fns = None


def attention(q, k, v, wK=None, wV=None, *, clip=0, causal=False, key_lens=None,
              t5_bias=None, num_buckets=32, max_distance=128, bidirectional=True, scale=None):
    """Differentiable ``fwd`` (torch.autograd): the forward runs ``fwd_lse``,
    the backward ``bwd``; gradients flow to q, k, v, the tables and t5_bias."""
    global _fns
    if _fns is None:
        _fns = _autograd_fn()
    opts = dict(clip=clip, causal=causal, key_lens=key_lens, scale=scale)
    if t5_bias is not None:
        opts.update(num_buckets=num_buckets, max_distance=max_distance,
                    bidirectional=bidirectional)
    return _fns[0].apply(q, k, v, wK, wV, t5_bias, opts)


def attention_offset_bias(q, k, v, bias, window, *, causal=False, key_lens=None, scale=None):
    """Differentiable ``fwd_offset_bias``."""
    global _fns
    if _fns is None:
        _fns = _autograd_fn()
    return _fns[1].apply(q, k, v, bias, window,
                         dict(causal=causal, key_lens=key_lens, scale=scale))


# ---------------------------------------------------------------------------
# Transformer-XL relative logits
# ---------------------------------------------------------------------------

def _xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out):
    views = [_view(x) for x in (q, k, v, R, u, vb)]
    mask = None
    if causal or key_lens is not None:
        mask = _Mask(1 if causal else 0, key_lens.data_ptr() if key_lens is not None else None)
    outv = _view(out)
    args = [_ref(x) for x in views] + [int(window), float(0.0 if scale is None else scale),
                                        _ref(mask), _ref(outv)]
    return args, views + [mask, outv]


@_on_stream
def fwd_xl(q, k, v, R, u, vb, window, *, causal=False, key_lens=None, scale=None, out=None,
           stream=None):
    """Transformer-XL relative logits: e_ij = s[(q_i + u).k_j + (q_i + vb).R_{i-j}].

    R: [H or 1, 2*window+1, d], row window + (i - j) for distance i - j; u, vb:
    [H or 1, d] global biases; all in the dtype of q.  Returns ``out``."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, keep = _xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out)
    st = lib.relattn_fwd_xl(*args, ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


def validate_xl(q, k, v, R, u, vb, window, *, causal=False, key_lens=None, scale=None,
                out=None):
    """Host-only argument check of ``fwd_xl``; returns the status code."""
    lib = _load()
    args, keep = _xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale,
                          q if out is None else out)
    st = lib.relattn_validate_xl(*args)
    del keep
    return st


@_on_stream
def fwd_xl_lse(q, k, v, R, u, vb, window, *, causal=False, key_lens=None, scale=None,
               out=None, lse=None, stream=None):
    """``fwd_xl`` with the row log-sum-exp; returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out)
    lv = _view(lse)
    st = lib.relattn_fwd_xl_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


def _xl_grads(q, R, u, vb, dq, dk, dv, dR, du, dvb, want_dR, want_du, want_dvb):
    import torch

    def f32(x, ref, want):
        if x is not None or not want:
            return x
        return torch.empty(ref.shape, dtype=torch.float32, device=q.device)
    base = _bwd_outputs(q, None, None, None, dq, dk, dv, None, None, None, False, False, False)
    return base[:3] + (f32(dR, R, want_dR), f32(du, u, want_du), f32(dvb, vb, want_dvb))


def _bwd_xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out, dout, lse, grads):
    args, keep = _xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out)
    extra = [_view(x) for x in (dout, lse) + tuple(grads)]
    return args + [_ref(x) for x in extra], keep + extra


def bwd_xl_workspace_size(q, k, v, R, u, vb, window, *, out, dout, lse, causal=False,
                          key_lens=None, scale=None, want_dR=True, want_du=True, want_dvb=True):
    """Workspace bytes ``bwd_xl`` needs (host only)."""
    lib = _load()
    g = _xl_grads(q, R, u, vb, q, q, q, None, None, None, want_dR, want_du, want_dvb)
    args, keep = _bwd_xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out, dout,
                              lse, g)
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_xl_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd_xl(q, k, v, R, u, vb, window, *, out, dout, lse, causal=False, key_lens=None,
           scale=None, dq=None, dk=None, dv=None, dR=None, du=None, dvb=None, want_dR=True,
           want_du=True, want_dvb=True, workspace=None, stream=None):
    """Gradients for ``fwd_xl_lse``: returns (dq, dk, dv, dR, du, dvb), the
    last three float32 like R, u and vb (None when not wanted)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    g = _xl_grads(q, R, u, vb, dq, dk, dv, dR, du, dvb, want_dR, want_du, want_dvb)
    args, keep = _bwd_xl_args(q, k, v, R, u, vb, window, causal, key_lens, scale, out, dout,
                              lse, g)
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_xl_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd_xl(*args, ctypes.c_void_p(workspace.data_ptr()),
                            ctypes.c_size_t(workspace.numel()),
                            ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return g


_xl_fn = None


def attention_xl(q, k, v, R, u, vb, window, *, causal=False, key_lens=None, scale=None):
    """Differentiable ``fwd_xl``: gradients to q, k, v, R, u and vb."""
    global _xl_fn
    if _xl_fn is None:
        import torch

        class _AttentionXL(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, R, u, vb, window, opts):
                out, lse = fwd_xl_lse(q, k, v, R, u, vb, window, **opts)
                ctx.save_for_backward(q, k, v, R, u, vb, out, lse)
                ctx.window, ctx.opts = window, opts
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, R, u, vb, out, lse = ctx.saved_tensors
                need = ctx.needs_input_grad
                dq, dk, dv, dR, du, dvb = bwd_xl(q, k, v, R, u, vb, ctx.window, out=out,
                                                 dout=dout.contiguous(), lse=lse,
                                                 want_dR=need[3], want_du=need[4],
                                                 want_dvb=need[5], **ctx.opts)
                cast = lambda x, ref: None if x is None else x.to(ref.dtype)
                return dq, dk, dv, cast(dR, R), cast(du, u), cast(dvb, vb), None, None

        _xl_fn = _AttentionXL
    return _xl_fn.apply(q, k, v, R, u, vb, window,
                        dict(causal=causal, key_lens=key_lens, scale=scale))


# ---------------------------------------------------------------------------
# 2-D window bias (Swin)
# ---------------------------------------------------------------------------

@_on_stream
def fwd_grid_bias(q, k, v, bias, window_side, *, key_lens=None, scale=None, out=None,
                  stream=None):
    """Relative position bias on an M x M window (n = M*M raster tokens): bias
    [H or 1, (2M-1)^2] float32, entry (dy + M - 1)(2M - 1) + (dx + M - 1) for the
    key-minus-query offset (dy, dx).  Returns ``out``."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, keep = _ob_args(q, k, v, bias, window_side, False, key_lens, scale, out)
    st = lib.relattn_fwd_grid_bias(*args, ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


def validate_grid_bias(q, k, v, bias, window_side, *, causal=False, key_lens=None,
                       scale=None, out=None):
    """Host-only argument check of ``fwd_grid_bias``; returns the status code."""
    lib = _load()
    args, keep = _ob_args(q, k, v, bias, window_side, causal, key_lens, scale,
                          q if out is None else out)
    st = lib.relattn_validate_grid_bias(*args)
    del keep
    return st


@_on_stream
def fwd_grid_bias_lse(q, k, v, bias, window_side, *, key_lens=None, scale=None, out=None,
                      lse=None, stream=None):
    """``fwd_grid_bias`` with the row log-sum-exp; returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _ob_args(q, k, v, bias, window_side, False, key_lens, scale, out)
    lv = _view(lse)
    st = lib.relattn_fwd_grid_bias_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


def bwd_grid_bias_workspace_size(q, k, v, bias, window_side, *, out, dout, lse, key_lens=None,
                                 scale=None, want_dbias=True):
    """Workspace bytes ``bwd_grid_bias`` needs (host only)."""
    lib = _load()
    db = _bwd_outputs(q, None, None, bias, q, q, q, None, None, None, False, False,
                      want_dbias)[5]
    args, keep = _bwd_ob_args(q, k, v, bias, window_side, False, key_lens, scale, out, dout,
                              lse, (q, q, q, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_grid_bias_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd_grid_bias(q, k, v, bias, window_side, *, out, dout, lse, key_lens=None, scale=None,
                  dq=None, dk=None, dv=None, dbias=None, want_dbias=True, workspace=None,
                  stream=None):
    """Gradients for ``fwd_grid_bias_lse``: returns (dq, dk, dv, dbias); dbias
    float32 like ``bias`` (None when not wanted)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    dq, dk, dv, _, _, db = _bwd_outputs(q, None, None, bias, dq, dk, dv, None, None, dbias,
                                        False, False, want_dbias)
    args, keep = _bwd_ob_args(q, k, v, bias, window_side, False, key_lens, scale, out, dout,
                              lse, (dq, dk, dv, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_grid_bias_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd_grid_bias(*args, ctypes.c_void_p(workspace.data_ptr()),
                                   ctypes.c_size_t(workspace.numel()),
                                   ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return dq, dk, dv, db


_grid_fn = None


def attention_grid_bias(q, k, v, bias, window_side, *, key_lens=None, scale=None):
    """Differentiable ``fwd_grid_bias``: the forward runs ``fwd_grid_bias_lse``,
    the backward ``bwd_grid_bias``."""
    global _grid_fn
    if _grid_fn is None:
        import torch

        class _AttentionGrid(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, bias, window_side, opts):
                out, lse = fwd_grid_bias_lse(q, k, v, bias, window_side, **opts)
                ctx.save_for_backward(q, k, v, bias, out, lse)
                ctx.window_side, ctx.opts = window_side, opts
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, bias, out, lse = ctx.saved_tensors
                dq, dk, dv, db = bwd_grid_bias(q, k, v, bias, ctx.window_side, out=out,
                                               dout=dout.contiguous(), lse=lse,
                                               want_dbias=ctx.needs_input_grad[3], **ctx.opts)
                return dq, dk, dv, db, None, None

        _grid_fn = _AttentionGrid
    return _grid_fn.apply(q, k, v, bias, window_side, dict(key_lens=key_lens, scale=scale))


def edge_label_buffer(B, n, device=None):
    """A zeroed uint8 [B, n, n] view whose rows are n rounded up to 16 bytes
    apart, the layout ``fwd_edge_bias`` reads its labels in."""
    import torch
    n16 = (n + 15) // 16 * 16
    return torch.zeros((B, n, n16), dtype=torch.uint8, device=device)[:, :, :n]


def _edge_args(q, k, v, labels, bias, causal, key_lens, scale, out, tables=None):
    import torch
    n = labels.shape[1] if labels.dim() == 3 else 0
    if labels.dtype == torch.uint8 and labels.dim() == 3 and labels.numel() > 0:
        # every row must be readable to n rounded up to 16 bytes
        n16 = (n + 15) // 16 * 16
        last = (labels.storage_offset() + (labels.shape[0] - 1) * labels.stride(0)
                + (n - 1) * labels.stride(1) + n16)
        if last > labels.untyped_storage().nbytes():
            raise RelattnError(INVALID_ARGUMENT,
                               "relattn: labels rows must be readable to n rounded up to 16 "
                               "bytes (see edge_label_buffer)")
    views = [_view(x) for x in ((q, k, v, labels, bias) if tables is None
                                 else (q, k, v, labels) + tuple(tables))]
    mask = None
    if causal or key_lens is not None:
        mask = _Mask(1 if causal else 0, key_lens.data_ptr() if key_lens is not None else None)
    outv = _view(out)
    args = [_ref(x) for x in views] + [float(0.0 if scale is None else scale), _ref(mask),
                                        _ref(outv)]
    return args, views + [mask, outv]


@_on_stream
def fwd_edge_bias(q, k, v, labels, bias, *, causal=False, key_lens=None, scale=None, out=None,
                  stream=None):
    """Attention with a scalar bias by a per-pair label: labels uint8 [B, n, n]
    (rows padded to 16 bytes, e.g. from ``edge_label_buffer``), bias float32
    [H or 1, NL]; e_ij = scale * q_i.k_j + bias[h, labels[b, i, j]].  Returns
    ``out``."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, keep = _edge_args(q, k, v, labels, bias, causal, key_lens, scale, out)
    st = lib.relattn_fwd_edge_bias(*args, ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


@_on_stream
def fwd_edge_bias_lse(q, k, v, labels, bias, *, causal=False, key_lens=None, scale=None,
                      out=None, lse=None, stream=None):
    """``fwd_edge_bias`` with the row log-sum-exp; returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _edge_args(q, k, v, labels, bias, causal, key_lens, scale, out)
    lv = _view(lse)
    st = lib.relattn_fwd_edge_bias_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


def _bwd_edge_args(q, k, v, labels, bias, causal, key_lens, scale, out, dout, lse, grads):
    args, keep = _edge_args(q, k, v, labels, bias, causal, key_lens, scale, out)
    extra = [_view(x) for x in (dout, lse) + tuple(grads)]
    return args + [_ref(x) for x in extra], keep + extra


def bwd_edge_bias_workspace_size(q, k, v, labels, bias, *, out, dout, lse, causal=False,
                                 key_lens=None, scale=None, want_dbias=True):
    """Workspace bytes ``bwd_edge_bias`` needs (host only)."""
    lib = _load()
    db = _bwd_outputs(q, None, None, bias, q, q, q, None, None, None, False, False,
                      want_dbias)[5]
    args, keep = _bwd_edge_args(q, k, v, labels, bias, causal, key_lens, scale, out, dout, lse,
                                (q, q, q, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_edge_bias_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd_edge_bias(q, k, v, labels, bias, *, out, dout, lse, causal=False, key_lens=None,
                  scale=None, dq=None, dk=None, dv=None, dbias=None, want_dbias=True,
                  workspace=None, stream=None):
    """Gradients for ``fwd_edge_bias_lse``: returns (dq, dk, dv, dbias); dbias
    float32 like ``bias`` (None when not wanted)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    dq, dk, dv, _, _, db = _bwd_outputs(q, None, None, bias, dq, dk, dv, None, None, dbias,
                                        False, False, want_dbias)
    args, keep = _bwd_edge_args(q, k, v, labels, bias, causal, key_lens, scale, out, dout, lse,
                                (dq, dk, dv, db))
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_edge_bias_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd_edge_bias(*args, ctypes.c_void_p(workspace.data_ptr()),
                                   ctypes.c_size_t(workspace.numel()),
                                   ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return dq, dk, dv, db


_edge_fn = None


def attention_edge_bias(q, k, v, labels, bias, *, causal=False, key_lens=None, scale=None):
    """Differentiable ``fwd_edge_bias`` (gradients to q, k, v and bias; the
    labels are integers)."""
    global _edge_fn
    if _edge_fn is None:
        import torch

        class _AttentionEdge(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, labels, bias, opts):
                out, lse = fwd_edge_bias_lse(q, k, v, labels, bias, **opts)
                ctx.save_for_backward(q, k, v, labels, bias, out, lse)
                ctx.opts = opts
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, labels, bias, out, lse = ctx.saved_tensors
                dq, dk, dv, db = bwd_edge_bias(q, k, v, labels, bias, out=out,
                                               dout=dout.contiguous(), lse=lse,
                                               want_dbias=ctx.needs_input_grad[4], **ctx.opts)
                return dq, dk, dv, None, db, None

        _edge_fn = _AttentionEdge
    return _edge_fn.apply(q, k, v, labels, bias,
                          dict(causal=causal, key_lens=key_lens, scale=scale))


def validate_edge_bias(q, k, v, labels, bias, *, causal=False, key_lens=None, scale=None,
                       out=None):
    """Host-only argument check of ``fwd_edge_bias``; returns the status code."""
    lib = _load()
    args, keep = _edge_args(q, k, v, labels, bias, causal, key_lens, scale,
                            q if out is None else out)
    st = lib.relattn_validate_edge_bias(*args)
    del keep
    return st


@_on_stream
def fwd_edge_tables(q, k, v, labels, wK=None, wV=None, *, causal=False, key_lens=None,
                    scale=None, out=None, stream=None):
    """Relation-aware attention over a labeled graph: labels uint8 [B, n, n]
    (layout of ``fwd_edge_bias``), wK / wV [H or 1, NL, d] in the dtype of q;
    e_ij = scale * q_i.(k_j + wK[E_ij]), z_i = sum_j alpha_ij (v_j + wV[E_ij]).
    Returns ``out``."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    args, keep = _edge_args(q, k, v, labels, None, causal, key_lens, scale, out, (wK, wV))
    st = lib.relattn_fwd_edge_tables(*args, ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return out


@_on_stream
def fwd_edge_tables_lse(q, k, v, labels, wK=None, wV=None, *, causal=False, key_lens=None,
                        scale=None, out=None, lse=None, stream=None):
    """``fwd_edge_tables`` with the row log-sum-exp; returns (out, lse)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = _new_lse(q)
    args, keep = _edge_args(q, k, v, labels, None, causal, key_lens, scale, out, (wK, wV))
    lv = _view(lse)
    st = lib.relattn_fwd_edge_tables_lse(*args, _ref(lv), ctypes.c_void_p(_stream_of(q, stream)))
    del keep, lv
    if st != OK:
        _raise(lib, st)
    return out, lse


def _bwd_edget_args(q, k, v, labels, wK, wV, causal, key_lens, scale, out, dout, lse, grads):
    args, keep = _edge_args(q, k, v, labels, None, causal, key_lens, scale, out, (wK, wV))
    extra = [_view(x) for x in (dout, lse) + tuple(grads)]
    return args + [_ref(x) for x in extra], keep + extra


def bwd_edge_tables_workspace_size(q, k, v, labels, wK=None, wV=None, *, out, dout, lse,
                                   causal=False, key_lens=None, scale=None, want_dwk=True,
                                   want_dwv=True):
    """Workspace bytes ``bwd_edge_tables`` needs (host only)."""
    lib = _load()
    g = _bwd_outputs(q, wK, wV, None, q, q, q, None, None, None, want_dwk, want_dwv, False)
    args, keep = _bwd_edget_args(q, k, v, labels, wK, wV, causal, key_lens, scale, out, dout,
                                 lse, g[:5])
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_edge_tables_workspace_size(*args, ctypes.byref(n))
    del keep
    if st != OK:
        _raise(lib, st)
    return int(n.value)


@_on_stream
def bwd_edge_tables(q, k, v, labels, wK=None, wV=None, *, out, dout, lse, causal=False,
                    key_lens=None, scale=None, dq=None, dk=None, dv=None, dwK=None, dwV=None,
                    want_dwk=True, want_dwv=True, workspace=None, stream=None):
    """Gradients for ``fwd_edge_tables_lse``: returns (dq, dk, dv, dwK, dwV), the
    table gradients float32 like the tables (None when absent or not wanted)."""
    import torch
    lib = _load()
    _check_lens(key_lens)
    g = _bwd_outputs(q, wK, wV, None, dq, dk, dv, dwK, dwV, None, want_dwk, want_dwv, False)
    args, keep = _bwd_edget_args(q, k, v, labels, wK, wV, causal, key_lens, scale, out, dout,
                                 lse, g[:5])
    n = ctypes.c_size_t(0)
    st = lib.relattn_bwd_edge_tables_workspace_size(*args, ctypes.byref(n))
    if st != OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    st = lib.relattn_bwd_edge_tables(*args, ctypes.c_void_p(workspace.data_ptr()),
                                     ctypes.c_size_t(workspace.numel()),
                                     ctypes.c_void_p(_stream_of(q, stream)))
    del keep
    if st != OK:
        _raise(lib, st)
    return g[:5]


_edget_fn = None


def attention_edge_tables(q, k, v, labels, wK=None, wV=None, *, causal=False, key_lens=None,
                          scale=None):
    """Differentiable ``fwd_edge_tables``: gradients to q, k, v and the tables."""
    global _edget_fn
    if _edget_fn is None:
        import torch

        class _AttentionEdgeTables(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, labels, wK, wV, opts):
                out, lse = fwd_edge_tables_lse(q, k, v, labels, wK, wV, **opts)
                ctx.save_for_backward(q, k, v, labels, wK, wV, out, lse)
                ctx.opts = opts
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, labels, wK, wV, out, lse = ctx.saved_tensors
                need = ctx.needs_input_grad
                dq, dk, dv, dwK, dwV = bwd_edge_tables(
                    q, k, v, labels, wK, wV, out=out, dout=dout.contiguous(), lse=lse,
                    want_dwk=need[4], want_dwv=need[5], **ctx.opts)
                cast = lambda x, ref: None if x is None else x.to(ref.dtype)
                return dq, dk, dv, None, cast(dwK, wK), cast(dwV, wV), None

        _edget_fn = _AttentionEdgeTables
    return _edget_fn.apply(q, k, v, labels, wK, wV,
                           dict(causal=causal, key_lens=key_lens, scale=scale))


def validate_edge_tables(q, k, v, labels, wK=None, wV=None, *, causal=False, key_lens=None,
                         scale=None, out=None):
    """Host-only argument check of ``fwd_edge_tables``; returns the status code."""
    lib = _load()
    args, keep = _edge_args(q, k, v, labels, None, causal, key_lens, scale,
                            q if out is None else out, (wK, wV))
    st = lib.relattn_validate_edge_tables(*args)
    del keep
    return st


def decode_offset_bias_workspace_size(q, k, v, bias, window, *, scale=None, out=None):
    """Workspace bytes ``decode_offset_bias`` needs for these shapes (host only)."""
    lib = _load()
    views = [_view(x) for x in (q, k, v, bias)]
    outv = _view(q if out is None else out)
    nbytes = ctypes.c_size_t(0)
    st = lib.relattn_decode_offset_bias_workspace_size(
        *[_ref(x) for x in views], int(window), float(0.0 if scale is None else scale),
        ctypes.byref(outv), ctypes.byref(nbytes))
    if st != OK:
        _raise(lib, st)
    return nbytes.value


@_on_stream
def decode_offset_bias(q, k, v, bias, window, *, cache_lens=None, scale=None, out=None,
                       workspace=None, stream=None):
    """Incremental decoding (positions as for ``decode``) with a scalar bias by
    clipped offset: bias float32 [H or 1, 2*window+1], entry window + delta for
    offset delta = j - i (ALiBi: -m_h * |delta|).  Returns ``out``."""
    import torch
    lib = _load()
    if cache_lens is not None and cache_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: cache_lens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    need = decode_offset_bias_workspace_size(q, k, v, bias, window, scale=scale, out=out)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    views = [_view(x) for x in (q, k, v, bias)]
    outv = _view(out)
    st = lib.relattn_decode_offset_bias(
        *[_ref(x) for x in views], int(window), float(0.0 if scale is None else scale),
        ctypes.c_void_p(cache_lens.data_ptr() if cache_lens is not None else None),
        ctypes.byref(outv), ctypes.c_void_p(workspace.data_ptr()),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        ctypes.c_void_p(_stream_of(q, stream)))
    del views, outv
    if st != OK:
        _raise(lib, st)
    return out


def decode_xl_workspace_size(q, k, v, R, u, vb, window, *, scale=None, out=None):
    """Workspace bytes ``decode_xl`` needs for these shapes (host only)."""
    lib = _load()
    views = [_view(x) for x in (q, k, v, R, u, vb)]
    outv = _view(q if out is None else out)
    nbytes = ctypes.c_size_t(0)
    st = lib.relattn_decode_xl_workspace_size(
        *[_ref(x) for x in views], int(window), float(0.0 if scale is None else scale),
        ctypes.byref(outv), ctypes.byref(nbytes))
    if st != OK:
        _raise(lib, st)
    return nbytes.value


@_on_stream
def decode_xl(q, k, v, R, u, vb, window, *, cache_lens=None, scale=None, out=None,
              workspace=None, stream=None):
    """Incremental decoding (positions as for ``decode``) with Transformer-XL
    relative logits: R [H or 1, 2*window+1, d] by distance i - j, u and vb
    [H or 1, d] (arguments of ``fwd_xl``).  Returns ``out``."""
    import torch
    lib = _load()
    if cache_lens is not None and cache_lens.dtype != torch.int32:
        raise RelattnError(INVALID_ARGUMENT, "relattn: cache_lens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    need = decode_xl_workspace_size(q, k, v, R, u, vb, window, scale=scale, out=out)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    views = [_view(x) for x in (q, k, v, R, u, vb)]
    outv = _view(out)
    st = lib.relattn_decode_xl(
        *[_ref(x) for x in views], int(window), float(0.0 if scale is None else scale),
        ctypes.c_void_p(cache_lens.data_ptr() if cache_lens is not None else None),
        ctypes.byref(outv), ctypes.c_void_p(workspace.data_ptr()),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        ctypes.c_void_p(_stream_of(q, stream)))
    del views, outv
    if st != OK:
        _raise(lib, st)
    return out
