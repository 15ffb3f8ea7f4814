"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test here runs librelattn's kernels on the GPU and compares with the
oracle on the same seeded inputs.  Bars: bit-exact for integer indices;
max-abs 1e-5 for fp32 and 2e-2 for bf16 inputs with fp32 accumulation.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


@pytest.fixture(scope="module")
def ra():
    import relative_position_encoding_amd as ra
    if not os.path.exists(ra.library_path):
        from relative_position_encoding_amd import build
        build.build()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return ra


@pytest.fixture(autouse=True)
def _announce(request):
    # name the case before any GPU work, so a crash still says which one
    sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


DEV = "cuda"


def to_dev(x):
    return None if x is None else x.to(DEV)


def gen(B, H, n, d, dtype, seed, ntab=None, std=1.0, tstd=0.1, shared=False):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g)
    q, k, v = (r(B, H, n, d) * std for _ in range(3))
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if ntab is not None:
        Ht = 1 if shared else H
        out += [(r(Ht, ntab, d) * tstd).to(dtype), (r(Ht, ntab, d) * tstd).to(dtype)]
    return out


def run_shaw(ra, q, k, v, wK, wV, c, causal=False, lens=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = ra.fwd(to_dev(q), to_dev(k), to_dev(v), to_dev(wK), to_dev(wV), clip=c,
                 causal=causal, key_lens=lens_d, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b))) if np.size(b) else 0.0


# ---------------------------------------------------------------------------
# integer indices: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,c", [(1, 0), (7, 0), (32, 4), (100, 16), (300, 64), (50, 70)])
def test_clip_indices_bit_exact(ra, n, c):
    got = ra.debug_indices(n, c).cpu().numpy()
    want = np.array([oracle.clip(d, c) + c for d in range(-(n - 1), n)])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B,D,bidir", [(32, 128, True), (32, 128, False), (8, 8, True),
                                       (8, 8, False), (16, 64, True), (64, 300, True)])
def test_t5_bucket_indices_bit_exact(ra, B, D, bidir):
    n = 1500
    got = ra.debug_indices(n, t5=True, num_buckets=B, max_distance=D,
                           bidirectional=bidir).cpu().numpy()
    want = np.array([oracle.t5_bucket(d, B, D, bidir) for d in range(-(n - 1), n)])
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# moderate sizes, full oracle: several tiles and a ragged tail
# ---------------------------------------------------------------------------

SHAW_CASES = []
for dtype in (torch.float32, torch.bfloat16):
    for d in (16, 32, 64, 128):
        for which in ("kv", "k", "v", "none"):
            for mask in ("none", "causal", "lens", "causal+lens"):
                SHAW_CASES.append((dtype, d, which, mask))


@pytest.mark.parametrize("dtype,d,which,mask", SHAW_CASES,
                         ids=lambda x: str(x).replace("torch.", ""))
def test_shaw_parity_moderate(ra, dtype, d, which, mask):
    B, H, n, c = 2, 3, 157, 5 + d % 7
    seed = 1000 + d + len(which) * 10 + len(mask)
    q, k, v, wK, wV = gen(B, H, n, d, dtype, seed, 2 * c + 1, tstd=0.3)
    wK = wK if "k" in which else None
    wV = wV if "v" in which else None
    causal = "causal" in mask
    lens = [101, 157] if "lens" in mask else None
    got = run_shaw(ra, q, k, v, wK, wV, c, causal, lens)
    want = oracle.relattn_factored(q, k, v, wK, wV, c, causal=causal, key_lens=lens)
    assert maxerr(got, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n,c", [(1, 0), (2, 1), (33, 0), (65, 64), (70, 75), (129, 200)])
def test_shaw_clip_extremes(ra, dtype, n, c):
    """k = 0 (one label), k >= n-1 (no clipping) and tiny n."""
    q, k, v, wK, wV = gen(1, 2, n, 64, dtype, 7 + n + c, 2 * c + 1, tstd=0.3)
    for causal in (False, True):
        got = run_shaw(ra, q, k, v, wK, wV, c, causal)
        want = oracle.relattn_factored(q, k, v, wK, wV, c, causal=causal)
        assert maxerr(got, want) <= TOL[dtype], (causal,)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
def test_t5_parity_moderate(ra, dtype, bidir, mask):
    B, H, n, d = 2, 3, 301, 64
    q, k, v = gen(B, H, n, d, dtype, 77, std=0.5)
    g = torch.Generator().manual_seed(78)
    bias = torch.randn(32, H, generator=g)
    causal = mask == "causal"
    lens = [150, 301] if mask == "lens" else None
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = ra.fwd(q.to(DEV), k.to(DEV), v.to(DEV), t5_bias=bias.to(DEV), num_buckets=32,
                 max_distance=64, bidirectional=bidir, causal=causal, key_lens=lens_d)
    torch.cuda.synchronize()
    want = oracle.t5_attention(q, k, v, bias, 32, 64, bidir, causal=causal, key_lens=lens)
    assert maxerr(out.float().cpu().numpy(), want) <= TOL[dtype]


def test_explicit_scale(ra):
    q, k, v, wK, wV = gen(2, 2, 90, 32, torch.bfloat16, 5, 9, tstd=0.3)
    got = run_shaw(ra, q, k, v, wK, wV, 4, scale=0.05)
    want = oracle.relattn_factored(q, k, v, wK, wV, 4, scale=0.05)
    assert maxerr(got, want) <= 2e-2


def test_strided_views(ra):
    """q, k, v as [B, H, n, d] views of [B, n, H, d] storage; out strided too."""
    B, H, n, d, c = 2, 4, 77, 64, 6
    g = torch.Generator().manual_seed(11)
    base = [torch.randn(B, n, H, d, generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (x.permute(0, 2, 1, 3) for x in base)
    wK = (torch.randn(H, 2 * c + 1, d, generator=g) * 0.3).to(torch.bfloat16)
    wV = (torch.randn(H, 2 * c + 1, d, generator=g) * 0.3).to(torch.bfloat16)
    outbuf = torch.empty(B, n, H, d, dtype=torch.bfloat16, device=DEV)
    out = outbuf.permute(0, 2, 1, 3)
    ra.fwd(q.to(DEV), k.to(DEV), v.to(DEV), wK.to(DEV), wV.to(DEV), clip=c, causal=True,
           out=out)
    torch.cuda.synchronize()
    want = oracle.relattn_factored(q, k, v, wK, wV, c, causal=True)
    assert maxerr(out.float().cpu().numpy(), want) <= 2e-2


# ---------------------------------------------------------------------------
# properties that hold at any size (bit-exact on the GPU)
# ---------------------------------------------------------------------------

def test_deterministic(ra):
    q, k, v, wK, wV = (to_dev(x) for x in gen(2, 4, 333, 64, torch.bfloat16, 3, 33))
    a = ra.fwd(q, k, v, wK, wV, clip=16, causal=True)
    b = ra.fwd(q, k, v, wK, wV, clip=16, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_causal_ignores_positive_offset_rows(ra):
    c = 8
    q, k, v, wK, wV = (to_dev(x) for x in gen(2, 2, 200, 64, torch.bfloat16, 4, 2 * c + 1))
    wK2, wV2 = wK.clone(), wV.clone()
    wK2[:, c + 1:] += 3.0
    wV2[:, c + 1:] -= 2.0
    a = ra.fwd(q, k, v, wK, wV, clip=c, causal=True)
    b = ra.fwd(q, k, v, wK2, wV2, clip=c, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_shared_tables_equal_replicated(ra):
    c, H = 8, 3
    q, k, v, wK, wV = (to_dev(x) for x in gen(2, H, 150, 64, torch.bfloat16, 6, 2 * c + 1,
                                               shared=True))
    a = ra.fwd(q, k, v, wK, wV, clip=c)
    b = ra.fwd(q, k, v, wK.expand(H, -1, -1).contiguous(), wV.expand(H, -1, -1).contiguous(),
               clip=c)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_zero_length_rows_output_zero(ra):
    q, k, v, wK, wV = gen(3, 2, 64, 32, torch.float32, 8, 9)
    lens = [0, 64, 1]
    got = run_shaw(ra, q, k, v, wK, wV, 4, lens=lens)
    assert np.all(got[0] == 0)
    want = oracle.relattn_factored(q, k, v, wK, wV, 4, key_lens=lens)
    assert maxerr(got, want) <= 1e-5


def test_empty_problem_is_noop(ra):
    for shape in [(0, 2, 8, 64), (2, 0, 8, 64), (2, 2, 0, 64)]:
        q = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        out = ra.fwd(q, q, q, clip=3)
        assert out.shape == q.shape


def test_unsupported_head_size_raises(ra):
    q = torch.zeros(1, 1, 8, 48, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ra.RelattnError) as e:
        ra.fwd(q, q, q)
    assert e.value.status == ra.UNSUPPORTED


# ---------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench times
# ---------------------------------------------------------------------------

def _run_workload(ra, name):
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    g = {key: to_dev(t) for key, t in x.items()}
    if w.t5 is None:
        out = ra.fwd(g["q"], g["k"], g["v"], g["key_table"], g["value_table"], clip=w.clip,
                     causal=w.causal, key_lens=g["key_lens"])
    else:
        out = ra.fwd(g["q"], g["k"], g["v"], t5_bias=g["t5_bias"], causal=w.causal,
                     key_lens=g["key_lens"], **w.t5)
    torch.cuda.synchronize()
    return w, x, out.float().cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "base", "big_causal_k", "big_causal_kv"])
def test_workload_full_oracle(ra, name):
    w, x, got = _run_workload(ra, name)
    want = oracle.relattn_factored(x["q"], x["k"], x["v"], x["key_table"], x["value_table"],
                                   w.clip, causal=w.causal, key_lens=x["key_lens"])
    err = maxerr(got, want)
    print(f"{name}: max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


def test_workload_t5_full_oracle(ra):
    w, x, got = _run_workload(ra, "t5")
    want = oracle.t5_attention(x["q"], x["k"], x["v"], x["t5_bias"], causal=w.causal,
                               key_lens=x["key_lens"], **w.t5)
    err = maxerr(got, want)
    print(f"t5: max abs err {err:.3g}")
    assert err <= TOL[w.dtype]


def test_workload_long_full_oracle(ra):
    """n = 4096, clip 64, causal: every output row against the factored fp64
    oracle (Eq. 5 form, itself pinned to brute force), so every query tile, the
    heaviest-first tile order and the chunked table staging are all compared."""
    w, x, got = _run_workload(ra, "long")
    want = oracle.relattn_factored(x["q"], x["k"], x["v"], x["key_table"], x["value_table"],
                                   w.clip, causal=w.causal, key_lens=x["key_lens"])
    assert want.shape == got.shape
    err = maxerr(got, want)
    print(f"long: max abs err over all {got.shape[0] * got.shape[1] * got.shape[2]} rows {err:.3g}")
    assert err <= TOL[w.dtype]


def test_workload_long_sampled_rows(ra):
    """n = 4096: 64 sampled rows against the brute-force row oracle (the
    materialised n x n x d form of Eq. 3 and Eq. 4, row by row), including rows
    at the clip boundary and the last row."""
    w, x, got = _run_workload(ra, "long")
    rng = np.random.default_rng(4)
    c, n = w.clip, w.n
    rows = [(b, h, i) for b, h, i in zip(rng.integers(0, w.batch, 59),
                                         rng.integers(0, w.heads, 59),
                                         rng.integers(0, n, 59))]
    rows += [(0, 0, 0), (1, 3, c - 1), (0, 5, c), (1, 7, c + 1), (1, 15, n - 1)]
    want = oracle.relattn_rows(x["q"], x["k"], x["v"], x["key_table"], x["value_table"],
                               c, causal=True, rows=rows)
    gotr = np.stack([got[b, h, i] for b, h, i in rows])
    err = maxerr(gotr, want)
    print(f"long: max abs err over {len(rows)} rows {err:.3g}")
    assert err <= 2e-2
    assert np.isfinite(got).all()
