"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/relattn.h, and its host-only validation rejects bad
arguments with the documented status codes."""
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ra():
    import relative_position_encoding_amd as ra
    if not os.path.exists(ra.library_path):
        from relative_position_encoding_amd import build
        build.build()
    return ra


def declared_functions():
    src = open(os.path.join(ROOT, "include", "relattn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(relattn_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(ra):
    import ctypes
    lib = ctypes.CDLL(ra.library_path)
    names = declared_functions()
    assert {"relattn_fwd", "relattn_validate", "relattn_debug_indices"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strerror(ra):
    lib = ra._load()
    assert lib.relattn_version() == 1
    for st in (ra.OK, ra.INVALID_ARGUMENT, ra.UNSUPPORTED, ra.NO_DEVICE, ra.LAUNCH_FAILED):
        assert lib.relattn_strerror(st)
    assert lib.relattn_strerror(12345) == b"unknown status"


def T(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def qkv(B=2, H=3, n=40, d=64, dtype=torch.bfloat16):
    return T(B, H, n, d, dtype=dtype), T(B, H, n, d, dtype=dtype), T(B, H, n, d, dtype=dtype)


def test_valid_arguments(ra):
    q, k, v = qkv()
    assert ra.validate(q, k, v) == ra.OK
    assert ra.validate(q, k, v, T(3, 9, 64), T(3, 9, 64), clip=4, causal=True) == ra.OK
    assert ra.validate(q, k, v, T(1, 9, 64), None, clip=4) == ra.OK   # shared table
    assert ra.validate(q, k, v, None, T(3, 9, 64), clip=4) == ra.OK   # value table only
    assert ra.validate(q, k, v, t5_bias=T(32, 3, dtype=torch.float32)) == ra.OK
    qf, kf, vf = qkv(dtype=torch.float32, d=16)
    assert ra.validate(qf, kf, vf, T(3, 1, 16, dtype=torch.float32), clip=0) == ra.OK


@pytest.mark.parametrize("case", [
    "dtype_mix", "shape_mix", "table_rows", "table_heads", "table_dtype", "neg_clip",
    "t5_and_tables", "t5_odd_buckets", "t5_small_distance", "t5_bias_shape",
    "t5_bias_dtype", "ndim", "nan_scale"])
def test_invalid_arguments(ra, case):
    q, k, v = qkv()
    kw = {}
    args = [q, k, v]
    if case == "dtype_mix":
        args[1] = k.float()
    elif case == "shape_mix":
        args[2] = T(2, 3, 41, 64)
    elif case == "table_rows":
        args += [T(3, 8, 64)]; kw["clip"] = 4
    elif case == "table_heads":
        args += [T(2, 9, 64)]; kw["clip"] = 4
    elif case == "table_dtype":
        args += [T(3, 9, 64, dtype=torch.float32)]; kw["clip"] = 4
    elif case == "neg_clip":
        args += [T(3, 1, 64)]; kw["clip"] = -1
    elif case == "t5_and_tables":
        args += [T(3, 9, 64)]; kw.update(clip=4, t5_bias=T(32, 3, dtype=torch.float32))
    elif case == "t5_odd_buckets":
        kw.update(t5_bias=T(31, 3, dtype=torch.float32), num_buckets=31)
    elif case == "t5_small_distance":
        kw.update(t5_bias=T(32, 3, dtype=torch.float32), max_distance=8)
    elif case == "t5_bias_shape":
        kw.update(t5_bias=T(32, 4, dtype=torch.float32))
    elif case == "t5_bias_dtype":
        kw.update(t5_bias=T(32, 3))
    elif case == "ndim":
        args = [T(3, 40, 64)] * 3
    elif case == "nan_scale":
        kw["scale"] = float("nan")
    assert ra.validate(*args, **kw) == ra.INVALID_ARGUMENT, ra.last_error()
    assert ra.last_error()


@pytest.mark.parametrize("n,causal", [(2 ** 21 + 5, False), (2 ** 22, True), (2 ** 22, False)])
def test_window_past_32bit_layout_is_unsupported(ra, n, causal):
    """Label windows of millions of rows (n and clip of order 2^21-2^22, given
    as expanded stride-0 views so nothing large is allocated): the plan rejects
    them before sizing any LDS layout, whose byte offsets are 32-bit."""
    x = torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16).expand(1, 1, n, 64)
    tab = torch.zeros(1, 1, 64, dtype=torch.bfloat16).expand(1, 2 * n + 1, 64)
    assert ra.validate(x, x, x, tab, tab, clip=n, causal=causal) == ra.UNSUPPORTED
    assert "fit" in ra.last_error()
    bias = torch.zeros(1, 2 * n + 1)
    assert ra.validate_offset_bias(x, x, x, bias, n, causal=causal) == ra.UNSUPPORTED


@pytest.mark.parametrize("case", ["head_size", "noncontig_d", "misaligned_stride",
                                  "huge_label_window", "fp16"])
def test_unsupported_arguments(ra, case):
    q, k, v = qkv()
    args, kw = [q, k, v], {}
    if case == "head_size":
        args = list(qkv(d=48))
    elif case == "noncontig_d":
        args = [T(2, 3, 40, 128)[..., ::2]] * 3
    elif case == "misaligned_stride":
        x = T(2, 3, 40, 68)[..., :64]  # row stride 136 bytes
        args = [x, x, x]
    elif case == "huge_label_window":
        q, k, v = qkv(n=5000, B=1, H=1)
        c = 4000
        args = [q, k, v, T(1, 2 * c + 1, 64)]
        kw["clip"] = c
    elif case == "fp16":
        args = list(qkv(dtype=torch.float16))
    st = ra.validate(*args, **kw)
    expected = ra.INVALID_ARGUMENT if case == "fp16" else ra.UNSUPPORTED
    assert st == expected, ra.last_error()


def test_empty_problem_validates(ra):
    for shape in [(0, 2, 8, 64), (2, 0, 8, 64), (2, 2, 0, 64)]:
        x = T(*shape)
        assert ra.validate(x, x, x, clip=2) == ra.OK


def test_no_device_status():
    """relattn_fwd reports NO_DEVICE when HIP sees no device (forced from the
    host by hiding every device from the child process)."""
    code = r"""
import sys, torch
sys.path.insert(0, %r)
import relative_position_encoding_amd as ra
q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
lib = ra._load()
args, keep = ra._args(q, q, q, None, None, None, 0, False, None, 32, 128, True, None, q)
st = lib.relattn_fwd(*args, None)
print(st)
""" % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip().splitlines()[-1]) == -3


def test_plan_cache_keeps_every_check():
    """relattn_fwd keeps recent plans per thread, keyed on shapes, strides,
    dtypes, scalars and pointer alignment.  After a valid call is cached, calls
    that differ only in a misaligned pointer, a dtype, a table shape, the key
    lengths' alignment or the clip still fail their checks, and the valid call
    still reaches the device check (no device is visible to the child)."""
    code = r"""
import sys, torch
sys.path.insert(0, %r)
import relative_position_encoding_amd as ra
lib = ra._load()
bf = torch.bfloat16
q = torch.zeros(2, 3, 40, 64, dtype=bf)
tab = torch.zeros(3, 9, 64, dtype=bf)
lens = torch.zeros(4, dtype=torch.int32)
def call(q=q, k=q, v=q, wK=tab, wV=tab, clip=4, causal=True, key_lens=None, out=q):
    args, keep = ra._args(q, k, v, wK, wV, None, clip, causal, key_lens, 32, 128, True, None,
                          out)
    return lib.relattn_fwd(*args, None)
mis = torch.zeros(2 * 3 * 40 * 64 + 8, dtype=bf)[1:1 + 2 * 3 * 40 * 64].view(2, 3, 40, 64)
class Mis:  # key lengths at an address that is not 4-byte aligned (never read)
    def data_ptr(self):
        return lens.data_ptr() + 2
res = [call(), call(), call(q=mis), call(out=q.float()), call(wK=torch.zeros(3, 8, 64, dtype=bf)),
       call(key_lens=Mis()), call(clip=-1), call(), call(key_lens=lens[:2])]
print(" ".join(map(str, res)))
""" % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stderr
    got = [int(x) for x in r.stdout.strip().splitlines()[-1].split()]
    assert got == [-3, -3, -2, -1, -1, -1, -1, -3, -3], got


# ---------------------------------------------------------------------------
# relattn_decode: host-only checks through relattn_decode_workspace_size
# ---------------------------------------------------------------------------

def test_decode_workspace_size(ra):
    B, H, Tq, L, d, c = 2, 3, 1, 1000, 64, 16
    q, k, v = T(B, H, Tq, d), T(B, H, L, d), T(B, H, L, d)
    ch = 32768 // (2 * d)                       # keys per decode workgroup (bf16)
    nch = -(-L // ch)
    rows = B * H * Tq
    base = -(-(rows * nch * 2 * 4) // 16) * 16 + rows * nch * d * 4
    # value table: one raw logit per single-key label (min(c, L) of them) per row
    want = -(-(base + rows * c * 4) // 16) * 16
    assert ra.decode_workspace_size(q, k, v, T(H, 2 * c + 1, d), T(H, 2 * c + 1, d),
                                    clip=c) == want
    assert ra.decode_workspace_size(q, k, v, T(H, 2 * c + 1, d), clip=c) == -(-base // 16) * 16
    assert ra.decode_workspace_size(q, k, v, t5_bias=T(32, H, dtype=torch.float32)) > 0
    e = T(0, H, Tq, d)
    assert ra.decode_workspace_size(e, T(0, H, L, d), T(0, H, L, d)) == 0


@pytest.mark.parametrize("case", ["cache_mismatch", "head_mismatch", "dtype_mix",
                                  "table_rows", "t5_and_tables", "head_size"])
def test_decode_rejects(ra, case):
    H, d, c = 3, 64, 4
    q, k, v = T(2, H, 1, d), T(2, H, 50, d), T(2, H, 50, d)
    args, kw = [q, k, v], {}
    code = ra.INVALID_ARGUMENT
    if case == "cache_mismatch":
        args[2] = T(2, H, 49, d)
    elif case == "head_mismatch":
        args[1] = T(2, H + 1, 50, d)
    elif case == "dtype_mix":
        args[2] = T(2, H, 50, d, dtype=torch.float32)
    elif case == "table_rows":
        args += [T(H, 2 * c, d)]; kw["clip"] = c
    elif case == "t5_and_tables":
        args += [T(H, 2 * c + 1, d)]; kw.update(clip=c, t5_bias=T(32, H, dtype=torch.float32))
    elif case == "head_size":
        args = [T(2, H, 1, 48), T(2, H, 50, 48), T(2, H, 50, 48)]
        code = ra.UNSUPPORTED
    with pytest.raises(ra.RelattnError) as ei:
        ra.decode_workspace_size(*args, **kw)
    assert ei.value.status == code


# ---------------------------------------------------------------------------
# relattn_fwd_offset_bias: host-only checks
# ---------------------------------------------------------------------------

def test_offset_bias_validation(ra):
    q, k, v = qkv()
    F = lambda *s: T(*s, dtype=torch.float32)
    assert ra.validate_offset_bias(q, k, v, F(3, 9), 4) == ra.OK
    assert ra.validate_offset_bias(q, k, v, F(1, 9), 4, causal=True) == ra.OK
    assert ra.validate_offset_bias(q, k, v, F(3, 1), 0) == ra.OK
    assert ra.validate_offset_bias(q, k, v, F(3, 8), 4) == ra.INVALID_ARGUMENT      # 2w+1
    assert ra.validate_offset_bias(q, k, v, F(2, 9), 4) == ra.INVALID_ARGUMENT      # heads
    assert ra.validate_offset_bias(q, k, v, T(3, 9), 4) == ra.INVALID_ARGUMENT      # dtype
    assert ra.validate_offset_bias(q, k, v, F(3, 1), -1) == ra.INVALID_ARGUMENT     # window
    big = 40000
    qb, kb, vb = qkv(B=1, H=1, n=50000)
    assert ra.validate_offset_bias(qb, kb, vb, F(1, 2 * big + 1), big) == ra.UNSUPPORTED


# ---------------------------------------------------------------------------
# backward: host-only checks of relattn_bwd_workspace_size (no HIP call)
# ---------------------------------------------------------------------------

def _ws_expected(B, H, n, d, nr, tables, nb=0, brq=128):
    """Workspace bytes from the sections the library documents: per query, lse
    and D (+64 floats of slack); per query tile of the dq kernel, the partial
    gradient of each table ([nr, d]) and of the bias ([nb]); each section
    rounded up to 256 bytes."""
    up = lambda floats: (floats * 4 + 255) // 256 * 256
    n_pad = (n + 63) // 64 * 64
    nqt = (n + brq - 1) // brq
    total = up(B * H * 2 * n_pad + 64)
    total += tables * up(B * H * nqt * nr * d)
    if nb:
        total += up(B * H * nqt * nb)
    return total


def _bwd_ws(ra, q, k, v, wK=None, wV=None, **kw):
    B, H, n, d = q.shape
    out = torch.zeros_like(q)
    lse = T(B, H, n, dtype=torch.float32)
    return ra.bwd_workspace_size(q, k, v, wK, wV, out=out, dout=torch.zeros_like(q), lse=lse,
                                 **kw)


def test_bwd_workspace_size(ra):
    q, k, v = qkv(B=2, H=3, n=300, d=64)
    # causal: labels -4..0 reachable (nr = 5); non-causal: all 9
    assert _bwd_ws(ra, q, k, v, T(3, 9, 64), T(3, 9, 64), clip=4, causal=True) == \
        _ws_expected(2, 3, 300, 64, 5, 2)
    assert _bwd_ws(ra, q, k, v, T(3, 9, 64), None, clip=4) == _ws_expected(2, 3, 300, 64, 9, 1)
    assert _bwd_ws(ra, q, k, v) == _ws_expected(2, 3, 300, 64, 1, 0)
    t5 = T(32, 3, dtype=torch.float32)
    assert _bwd_ws(ra, q, k, v, t5_bias=t5) == _ws_expected(2, 3, 300, 64, 1, 0, nb=32)
    assert _bwd_ws(ra, q, k, v, t5_bias=t5, want_dbias=False) == _ws_expected(2, 3, 300, 64, 1, 0)
    q0, k0, v0 = qkv(B=0)
    assert _bwd_ws(ra, q0, k0, v0) == 0


@pytest.mark.parametrize("case", ["dout_shape", "lse_dtype", "lse_shape", "dq_dtype",
                                  "dwk_without_wk", "dwk_shape", "dwk_dtype",
                                  "dbias_without_bias"])
def test_bwd_rejects(ra, case):
    q, k, v = qkv(n=50)
    B, H, n, d = q.shape
    wK = T(3, 9, 64)
    out, dout = torch.zeros_like(q), torch.zeros_like(q)
    lse = T(B, H, n, dtype=torch.float32)
    kw = dict(clip=4)
    tabs = [wK, None]
    if case == "dout_shape":
        dout = T(B, H, n + 1, d)
    elif case == "lse_dtype":
        lse = T(B, H, n)
    elif case == "lse_shape":
        lse = T(B, H, n - 1, dtype=torch.float32)
    elif case == "dq_dtype":
        kw["dq"] = torch.zeros_like(q).float()
    elif case == "dwk_without_wk":
        tabs = [None, None]
        kw["dwK"] = T(3, 9, 64, dtype=torch.float32)
    elif case == "dwk_shape":
        kw["dwK"] = T(3, 7, 64, dtype=torch.float32)
    elif case == "dwk_dtype":
        kw["dwK"] = T(3, 9, 64)
    elif case == "dbias_without_bias":
        kw["dbias"] = T(32, 3, dtype=torch.float32)
    with pytest.raises(ra.RelattnError) as e:
        ra.bwd_workspace_size(q, k, v, *tabs, out=out, dout=dout, lse=lse, **kw)
    assert e.value.status == ra.INVALID_ARGUMENT, case


def test_bwd_offset_bias_window_checks(ra):
    """A bias gradient needs per-workgroup sums over 2*min(W, n-1)+1 offsets on
    chip: too wide is UNSUPPORTED; without the bias gradient it is accepted."""
    q, k, v = qkv(B=1, H=2, n=600, d=64)
    out, dout = torch.zeros_like(q), torch.zeros_like(q)
    lse = T(1, 2, 600, dtype=torch.float32)
    bias = T(2, 2 * 599 + 1, dtype=torch.float32)
    with pytest.raises(ra.RelattnError) as e:
        ra.bwd_offset_bias_workspace_size(q, k, v, bias, 599, out=out, dout=dout, lse=lse)
    assert e.value.status == ra.UNSUPPORTED
    assert ra.bwd_offset_bias_workspace_size(q, k, v, bias, 599, out=out, dout=dout, lse=lse,
                                             want_dbias=False) > 0
    small = T(2, 11, dtype=torch.float32)
    assert ra.bwd_offset_bias_workspace_size(q, k, v, small, 5, out=out, dout=dout,
                                             lse=lse) > 0


def test_edge_bias_validation(ra):
    """Label layout and bias-table checks of relattn_validate_edge_bias."""
    B, H, n = 2, 3, 40
    q, k, v = qkv(B, H, n)
    bias = T(H, 7, dtype=torch.float32)
    lab = ra.edge_label_buffer(B, n)
    assert lab.stride(1) == 48
    assert ra.validate_edge_bias(q, k, v, lab, bias) == ra.OK
    assert ra.validate_edge_bias(q, k, v, lab, T(1, 7, dtype=torch.float32)) == ra.OK
    kl = torch.zeros(B, dtype=torch.int32)
    assert ra.validate_edge_bias(q, k, v, lab, bias, causal=True, key_lens=kl) == ra.OK
    assert ra.validate_edge_bias(q, k, v, lab, T(H, 256, dtype=torch.float32)) == ra.OK
    # one label matrix for every batch entry (batch stride 0)
    shared = lab[:1].expand(B, n, n)
    assert ra.validate_edge_bias(q, k, v, shared, bias) == ra.OK
    # rows closer than n rounded up to 16, or not a multiple of 16 bytes apart
    tight = torch.zeros(B * n * n + 16, dtype=torch.uint8).as_strided((B, n, n), (n * n, n, 1))
    assert ra.validate_edge_bias(q, k, v, tight, bias) == ra.UNSUPPORTED
    buf = torch.zeros(B * n * 64, dtype=torch.uint8)
    assert ra.validate_edge_bias(q, k, v, buf.as_strided((B, n, n), (n * 32, 32, 1)),
                                 bias) == ra.UNSUPPORTED
    # a contiguous matrix whose n is a multiple of 16 needs no padding
    q48, k48, v48 = qkv(B, H, 48)
    assert ra.validate_edge_bias(q48, k48, v48, torch.zeros(B, 48, 48, dtype=torch.uint8),
                                 bias) == ra.OK
    # wrong label dtype or shape, bad bias tables
    assert ra.validate_edge_bias(q, k, v, lab.to(torch.int32), bias) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_bias(q, k, v, ra.edge_label_buffer(B, n + 1)[:, :n, :n],
                                 bias) == ra.OK
    assert ra.validate_edge_bias(q, k, v, ra.edge_label_buffer(B + 1, n)[:, :, :],
                                 bias) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_bias(q, k, v, lab, T(H, 0, dtype=torch.float32)) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_bias(q, k, v, lab, T(H, 257, dtype=torch.float32)) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_bias(q, k, v, lab, T(H, 7)) == ra.INVALID_ARGUMENT   # bf16 bias
    assert ra.validate_edge_bias(q, k, v, lab, T(2, 7, dtype=torch.float32)) == ra.INVALID_ARGUMENT
    # the last row must be readable to n rounded up to 16 (checked by the binding)
    short = torch.zeros(B * n * 48 - 8, dtype=torch.uint8).as_strided((B, n, n), (n * 48, 48, 1))
    with pytest.raises(ra.RelattnError):
        ra.validate_edge_bias(q, k, v, short, bias)
    # empty problems validate
    q0, k0, v0 = qkv(0, H, n)
    assert ra.validate_edge_bias(q0, k0, v0, ra.edge_label_buffer(0, n), bias) == ra.OK


def test_edge_tables_validation(ra):
    """Table checks of relattn_validate_edge_tables (label layout as for the bias)."""
    B, H, n, d = 2, 3, 40, 64
    q, k, v = qkv(B, H, n, d)
    lab = ra.edge_label_buffer(B, n)
    wK, wV = T(H, 9, d), T(1, 9, d)
    assert ra.validate_edge_tables(q, k, v, lab, wK, wV) == ra.OK
    assert ra.validate_edge_tables(q, k, v, lab, wK, None, causal=True) == ra.OK
    assert ra.validate_edge_tables(q, k, v, lab, None, wV) == ra.OK
    assert ra.validate_edge_tables(q, k, v, lab, T(H, 256, d), None) == ra.OK
    assert ra.validate_edge_tables(q, k, v, lab, None, None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, wK, T(H, 8, d)) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, T(H, 257, d), None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, T(H, 0, d), None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, T(2, 9, d), None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, T(H, 9, 32), None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab, T(H, 9, d, dtype=torch.float32),
                                   None) == ra.INVALID_ARGUMENT
    assert ra.validate_edge_tables(q, k, v, lab.to(torch.int32), wK, None) == ra.INVALID_ARGUMENT
    tight = torch.zeros(B * n * n + 16, dtype=torch.uint8).as_strided((B, n, n), (n * n, n, 1))
    assert ra.validate_edge_tables(q, k, v, tight, wK, None) == ra.UNSUPPORTED


def test_decode_offset_bias_checks(ra):
    """Workspace size and argument checks of the offset-bias decode (host only)."""
    B, H, L, d = 2, 3, 64, 64
    q = T(B, H, 1, d)
    k, v = T(B, H, L, d), T(B, H, L, d)
    bias = T(H, 2 * 10 + 1, dtype=torch.float32)
    n1 = ra.decode_offset_bias_workspace_size(q, k, v, bias, 10)
    n0 = ra.decode_workspace_size(q, k, v, t5_bias=T(32, H, dtype=torch.float32))
    assert n1 == n0     # the same plan as the T5 bias: no value term
    assert ra.decode_offset_bias_workspace_size(q, k, v, T(1, 21, dtype=torch.float32), 10) == n1
    for bad, win in ((T(H, 20, dtype=torch.float32), 10), (T(2, 21, dtype=torch.float32), 10),
                     (T(H, 21), 10), (bias, -1)):
        with pytest.raises(ra.RelattnError) as e:
            ra.decode_offset_bias_workspace_size(q, k, v, bad, win)
        assert e.value.status == ra.INVALID_ARGUMENT


def test_missing_library_fails_loudly():
    """Without the built library every entry point raises: there is no CPU
    fallback behind the binding."""
    code = r"""
import sys, torch
sys.path.insert(0, %r)
import relative_position_encoding_amd as ra
ra.library_path = "/nonexistent/librelattn.so"
q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
for call in (lambda: ra.fwd(q, q, q), lambda: ra.validate(q, q, q),
             lambda: ra.fwd_edge_bias(q, q, q, ra.edge_label_buffer(1, 8), torch.zeros(1, 4)),
             lambda: ra.decode(q, q, q)):
    try:
        call()
    except RuntimeError as e:
        assert "not built" in str(e), e
    else:
        raise SystemExit("no error")
print("ok")
""" % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "ok"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_xl_checks(ra):
    """Workspace size and argument checks of the Transformer-XL decode (host only)."""
    B, H, L, d, W = 2, 3, 64, 64, 70
    q = T(B, H, 1, d)
    k, v = T(B, H, L, d), T(B, H, L, d)
    R, u = T(H, 2 * W + 1, d), T(H, d)
    n1 = ra.decode_xl_workspace_size(q, k, v, R, u, u, W)
    assert n1 == ra.decode_workspace_size(q, k, v, R, None, clip=W)
    for args in ((R, u.float(), u, W), (R, u, T(H, 32), W), (R[:, :-1], u, u, W),
                 (R, T(2, d), u, W)):
        with pytest.raises(ra.RelattnError) as e:
            ra.decode_xl_workspace_size(q, k, v, *args)
        assert e.value.status == ra.INVALID_ARGUMENT


def test_edge_tables_vocabulary_too_wide_for_chip(ra):
    """At d = 128 the rows of 256 labels (label logits and two weight sums per
    query) do not fit beside the K/V ring: UNSUPPORTED from the host plan."""
    B, H, n = 1, 2, 64
    q = T(B, H, n, 128)
    lab = ra.edge_label_buffer(B, n)
    assert ra.validate_edge_tables(q, q, q, lab, T(H, 200, 128), T(H, 200, 128)) == ra.OK
    assert ra.validate_edge_tables(q, q, q, lab, T(H, 256, 128), T(H, 256, 128)) == ra.UNSUPPORTED


def test_bwd_grid_bias_window_checks(ra):
    """The grid backward holds the head's (2M-1)^2 entries on chip, and with a
    bias gradient a sum over them per wave: head size 64 in bf16 reaches M = 40
    with the gradient and M = 74 without; one more is UNSUPPORTED."""
    def ws(M, want):
        q = T(1, 2, M * M, 64)
        bias = T(2, (2 * M - 1) ** 2, dtype=torch.float32)
        lse = T(1, 2, M * M, dtype=torch.float32)
        return ra.bwd_grid_bias_workspace_size(q, q, q, bias, M, out=q, dout=q, lse=lse,
                                               want_dbias=want)
    assert ws(40, True) > 0 and ws(74, False) > 0
    for M, want in ((41, True), (75, False)):
        with pytest.raises(ra.RelattnError) as e:
            ws(M, want)
        assert e.value.status == ra.UNSUPPORTED
    # the bias gradient's partial sums: one row of (2M-1)^2 per query tile
    M = 7
    assert ws(M, True) == _ws_expected(1, 2, M * M, 64, 1, 0, nb=(2 * M - 1) ** 2)
    assert ws(M, False) == _ws_expected(1, 2, M * M, 64, 1, 0)


def test_bwd_xl_window_checks(ra):
    """The Transformer-XL backward holds one row of relative logits per query
    over the reachable distances on chip: every distance of a 512-token causal
    segment fits in bf16 at d = 64 (one-wave query tiles); at d = 128 or over
    1024 tokens it is UNSUPPORTED, before any launch; the gradient buffers of
    u and v need the biases they belong to."""
    def ws(n, d, W, dtype=torch.bfloat16):
        q = T(1, 2, n, d, dtype=dtype)
        R, u = T(2, 2 * W + 1, d, dtype=dtype), T(2, d, dtype=dtype)
        lse = T(1, 2, n, dtype=torch.float32)
        return ra.bwd_xl_workspace_size(q, q, q, R, u, u, W, out=q, dout=q, lse=lse, causal=True)
    assert ws(512, 64, 511) > 0
    for n, d in ((512, 128), (1024, 64)):
        with pytest.raises(ra.RelattnError) as e:
            ws(n, d, n - 1)
        assert e.value.status == ra.UNSUPPORTED
    # partials of du and dv: 2 d floats per one-wave query tile of each head
    n, d, W = 512, 64, 511
    no_biases = ra.bwd_xl_workspace_size(
        T(1, 2, n, d), T(1, 2, n, d), T(1, 2, n, d), T(2, 2 * W + 1, d), T(2, d), T(2, d), W,
        out=T(1, 2, n, d), dout=T(1, 2, n, d), lse=T(1, 2, n, dtype=torch.float32),
        causal=True, want_du=False, want_dvb=False)
    up = lambda floats: (floats * 4 + 255) // 256 * 256
    assert ws(n, d, W) - no_biases == up(1 * 2 * (n // 32) * 2 * d)


def test_bwd_edge_tables_checks(ra):
    """The edge-table backward keeps per query row the label sums of dS and P on
    chip: key and value tables of 64 labels fit in bf16 at d = 64, 128 do not
    (UNSUPPORTED before any launch); a key table alone reaches 256 labels; the
    table gradients have the tables' NL rows."""
    B, H, n, d = 1, 2, 100, 64
    q = T(B, H, n, d)
    lab = ra.edge_label_buffer(B, n)
    lse = T(B, H, n, dtype=torch.float32)

    def ws(wK, wV, **kw):
        return ra.bwd_edge_tables_workspace_size(q, q, q, lab, wK, wV, out=q, dout=q, lse=lse,
                                                 **kw)
    assert ws(T(H, 64, d), T(H, 64, d)) > 0
    assert ws(T(H, 256, d), None) > 0
    with pytest.raises(ra.RelattnError) as e:
        ws(T(H, 128, d), T(H, 128, d))
    assert e.value.status == ra.UNSUPPORTED
    with pytest.raises(ra.RelattnError) as e:
        ra.bwd_edge_tables(q, q, q, lab, T(H, 16, d), None, out=q, dout=q, lse=lse,
                           dwK=T(H, 17, d, dtype=torch.float32))
    assert e.value.status == ra.INVALID_ARGUMENT
