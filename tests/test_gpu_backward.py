"""GPU parity of the backward pass (relattn_fwd_lse + relattn_bwd through the C
ABI) against the fp64 oracle's chain-rule gradients (oracle.relattn_backward,
oracle.t5_backward), on the same seeded inputs.

Bar: for every gradient, max|gpu - oracle| <= TOL * max(max|oracle|, 1):
TOL = 1e-4 for fp32 (fp32 products and sums) and 3e-2 for bf16 (operands of
the weight and dS products rounded to bf16, 2^-9 relative each, and the
outputs dq, dk, dv rounded to bf16).  The normalisation by the largest
gradient entry, not by each entry, is deliberate: table gradients are sums
over many pairs that cancel (they sum to zero over the labels).  The floor of
1 (inputs are O(1)) covers gradients that vanish identically (one key per
row, one label for every pair): D_i = dz_i.z_i uses the forward's output z
as stored, and its rounding is then all that remains."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}
DEV = "cuda"


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
    sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield


def gen(shape, dtype, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(dtype)


def dev(x):
    return None if x is None else x.to(DEV)


def nerr(got, want):
    want = np.asarray(want, np.float64)
    got = got.double().cpu().numpy()
    return float(np.max(np.abs(got - want))) / max(float(np.max(np.abs(want))), 1.0)


def run_shaw(ra, q, k, v, wK, wV, dz, clip, causal=False, lens=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, wkd, wvd, dzd = (dev(x) for x in (q, k, v, wK, wV, dz))
    out, lse = ra.fwd_lse(qd, kd, vd, wkd, wvd, clip=clip, causal=causal, key_lens=lens_d,
                          scale=scale)
    g = ra.bwd(qd, kd, vd, wkd, wvd, out=out, dout=dzd, lse=lse, clip=clip, causal=causal,
               key_lens=lens_d, scale=scale)
    torch.cuda.synchronize()
    return g


def check(got, want, dtype, names=("dq", "dk", "dv", "dwK", "dwV")):
    for name, g, w in zip(names, got, want):
        if w is None:
            assert g is None, name
            continue
        e = nerr(g, w)
        assert e <= TOL[dtype], f"{name}: normalised error {e:.3g} > {TOL[dtype]}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
def test_shaw_backward_parity(ra, dtype, d, mask):
    B, H, n, clip = 2, 2, 200, 5
    q, k, v, dz = (gen((B, H, n, d), dtype, 100 + d + i) for i in range(4))
    wK = gen((H, 2 * clip + 1, d), dtype, 105, 0.5)
    wV = gen((H, 2 * clip + 1, d), dtype, 106, 0.5)
    causal = mask == "causal"
    lens = [n, 131] if mask == "lens" else None
    got = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal, lens)
    want = oracle.relattn_backward(q, k, v, wK, wV, clip, dz, causal=causal, key_lens=lens)
    check(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("tables", ["k", "v", "none", "shared"])
@pytest.mark.parametrize("causal", [False, True])
def test_shaw_backward_tables(ra, dtype, tables, causal):
    B, H, n, d, clip = 2, 3, 150, 32, 16
    q, k, v, dz = (gen((B, H, n, d), dtype, 200 + i) for i in range(4))
    Ht = 1 if tables == "shared" else H
    wK = gen((Ht, 2 * clip + 1, d), dtype, 205, 0.5) if tables in ("k", "shared") else None
    wV = gen((Ht, 2 * clip + 1, d), dtype, 206, 0.5) if tables in ("v", "shared") else None
    got = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal)
    want = oracle.relattn_backward(q, k, v, wK, wV, clip, dz, causal=causal)
    check(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n,clip", [(1, 0), (1, 3), (37, 0), (37, 60), (64, 63), (129, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_shaw_backward_edges(ra, dtype, n, clip, causal):
    """clip 0 (one label), clip >= n (only 2n - 1 labels reachable), one row,
    ragged n and tile boundaries."""
    B, H, d = 1, 2, 64
    q, k, v, dz = (gen((B, H, n, d), dtype, 300 + n + clip + i) for i in range(4))
    wK = gen((H, 2 * clip + 1, d), dtype, 305, 0.5)
    wV = gen((H, 2 * clip + 1, d), dtype, 306, 0.5)
    got = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal)
    want = oracle.relattn_backward(q, k, v, wK, wV, clip, dz, causal=causal)
    check(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_backward_empty_rows(ra, dtype):
    """key length 0 for one sequence: its rows see no key, every gradient
    through them is 0; a length of 1 keeps one key per row."""
    B, H, n, d, clip = 3, 2, 90, 64, 4
    q, k, v, dz = (gen((B, H, n, d), dtype, 400 + i) for i in range(4))
    wK = gen((H, 2 * clip + 1, d), dtype, 405, 0.5)
    wV = gen((H, 2 * clip + 1, d), dtype, 406, 0.5)
    lens = [0, 1, 90]
    got = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal=True, lens=lens)
    want = oracle.relattn_backward(q, k, v, wK, wV, clip, dz, causal=True, key_lens=lens)
    check(got, want, dtype)
    for g in got[:3]:
        assert torch.count_nonzero(g[0]).item() == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("bidir", [True, False])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
def test_t5_backward_parity(ra, dtype, bidir, mask):
    B, H, n, d, nb, maxd = 2, 3, 180, 64, 32, 64
    q, k, v, dz = (gen((B, H, n, d), dtype, 500 + i) for i in range(4))
    bias = gen((nb, H), torch.float32, 505)
    causal = mask == "causal"
    lens = [n, 100] if mask == "lens" else None
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, bd, dzd = (dev(x) for x in (q, k, v, bias, dz))
    out, lse = ra.fwd_lse(qd, kd, vd, t5_bias=bd, num_buckets=nb, max_distance=maxd,
                          bidirectional=bidir, causal=causal, key_lens=lens_d)
    dq, dk, dv, _, _, db = ra.bwd(qd, kd, vd, t5_bias=bd, num_buckets=nb, max_distance=maxd,
                                  bidirectional=bidir, causal=causal, key_lens=lens_d, out=out,
                                  dout=dzd, lse=lse)
    torch.cuda.synchronize()
    want = oracle.t5_backward(q, k, v, bias, nb, maxd, bidir, dz, causal=causal, key_lens=lens)
    check((dq, dk, dv, db), want, dtype, names=("dq", "dk", "dv", "dbias"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [32, 64])
def test_forward_lse(ra, dtype, d):
    """The row statistic of fwd_lse: log sum over visible keys of exp(e_ij).
    In bf16 the row sum is taken over the weights as rounded to bf16 for the
    value product (the normaliser of the output), each within a relative 2^-9
    of its exact value, so the statistic is within ln(1 + 2^-9) < 2^-9 of the
    exact one (plus fp32 rounding of the logits)."""
    B, H, n, clip = 2, 2, 100, 6
    q, k, v = (gen((B, H, n, d), dtype, 600 + i) for i in range(3))
    wK = gen((H, 2 * clip + 1, d), dtype, 605, 0.5)
    lens = [n, 0]
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = ra.fwd_lse(dev(q), dev(k), dev(v), dev(wK), None, clip=clip, causal=True,
                          key_lens=lens_d)
    torch.cuda.synchronize()
    want = np.full((B, H, n), -np.inf)
    for b in range(B):
        ok = oracle.visible(n, True, lens[b])
        for h in range(H):
            e = oracle.shaw_logits(q[b, h], k[b, h], wK[h], clip)
            for i in range(n):
                if ok[i].any():
                    x = e[i][ok[i]]
                    want[b, h, i] = x.max() + np.log(np.exp(x - x.max()).sum())
    got = lse.double().cpu().numpy()
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.max(np.abs(got[fin] - want[fin])) <= (1e-5 if dtype == torch.float32 else 2.0 ** -9 + 1e-4)


def test_backward_deterministic(ra):
    """Two calls on the same inputs give bitwise equal gradients."""
    B, H, n, d, clip = 2, 4, 256, 64, 16
    dtype = torch.bfloat16
    q, k, v, dz = (gen((B, H, n, d), dtype, 700 + i) for i in range(4))
    wK = gen((1, 2 * clip + 1, d), dtype, 705, 0.5)
    wV = gen((1, 2 * clip + 1, d), dtype, 706, 0.5)
    a = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal=True)
    b = run_shaw(ra, q, k, v, wK, wV, dz, clip, causal=True)
    for x, y in zip(a, b):
        assert (x is None and y is None) or torch.equal(x, y)
    assert a[5] is None and a[3] is not None


def test_autograd_wrapper(ra):
    """torch.autograd through ra.attention matches the explicit bwd call."""
    B, H, n, d, clip = 1, 2, 70, 32, 3
    dtype = torch.float32
    q, k, v, dz = (gen((B, H, n, d), dtype, 800 + i).to(DEV) for i in range(4))
    wK = gen((H, 2 * clip + 1, d), dtype, 805, 0.5).to(DEV)
    wV = gen((H, 2 * clip + 1, d), dtype, 806, 0.5).to(DEV)
    leaves = [x.clone().requires_grad_(True) for x in (q, k, v, wK, wV)]
    out = ra.attention(*leaves, clip=clip, causal=True)
    out.backward(dz)
    want = oracle.relattn_backward(q.cpu(), k.cpu(), v.cpu(), wK.cpu(), wV.cpu(), clip,
                                   dz.cpu(), causal=True)
    check([x.grad for x in leaves], want, dtype)


@pytest.mark.parametrize("shape", ["big_causal_kv", "base"])
def test_backward_full_size_sampled(ra, shape):
    """The workload shapes at full size in one call; dq, dk, dv of a few sampled
    (batch, head) pairs against the oracle run on those heads alone, and the
    table gradients against their closed-form sums (weights per row sum to 1:
    sum_r dw^V_r = sum over all rows of dz_i; dS per row sums to 0:
    sum_r dw^K_r = 0)."""
    import workloads
    w = workloads.WORKLOADS[shape]
    x = workloads.make_inputs(w)
    dtype = x["q"].dtype
    B, H, n, d = x["q"].shape
    dz = gen((B, H, n, d), dtype, 900)
    lens = x["key_lens"]
    g = run_shaw(ra, x["q"], x["k"], x["v"], x["key_table"], x["value_table"], dz, w.clip,
                 w.causal, None if lens is None else lens.tolist())
    rng = np.random.default_rng(901)
    for _ in range(3):
        b, h = int(rng.integers(B)), int(rng.integers(H))
        sl = lambda t: t[b:b + 1, h:h + 1]
        tk = x["key_table"][h:h + 1] if x["key_table"].shape[0] > 1 else x["key_table"]
        tv = x["value_table"][h:h + 1] if x["value_table"].shape[0] > 1 else x["value_table"]
        want = oracle.relattn_backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), tk, tv, w.clip,
                                       sl(dz), causal=w.causal,
                                       key_lens=None if lens is None else [int(lens[b])])
        check([sl(t) for t in g[:3]], want[:3], dtype, names=("dq", "dk", "dv"))
    dwk, dwv = g[3].double().cpu().numpy(), g[4].double().cpu().numpy()
    assert np.max(np.abs(dwk.sum(axis=1))) <= 0.1 * max(np.abs(dwk).max(), 1e-3)
    # rows that see at least one key contribute their dz to the value-table sum
    zsum = np.zeros((dwv.shape[0], d))
    for b in range(B):
        L = n if lens is None else int(lens[b])
        rows = dz[b, :, :n if L > 0 else 0].double().numpy()
        if dwv.shape[0] == 1:
            zsum[0] += rows.sum(axis=(0, 1))
        else:
            zsum += rows.sum(axis=1)
    assert np.max(np.abs(dwv.sum(axis=1) - zsum)) <= 0.02 * np.abs(zsum).max()


@pytest.mark.parametrize("shape", ["big_causal_kv", "base"])
def test_backward_full_size_table_gradients(ra, shape):
    """The workload shapes at full size in one call; for two sampled heads h,
    the table gradients dw^K[h] and dw^V[h] element by element against the
    oracle summed over every batch entry of that head (the tables are per head,
    so their gradient is the sum over the batch of Eq. 3 and Eq. 4's bucketed
    terms), and dq, dk, dv of every batch entry of those heads."""
    import workloads
    w = workloads.WORKLOADS[shape]
    x = workloads.make_inputs(w)
    dtype = x["q"].dtype
    B, H, n, d = x["q"].shape
    assert x["key_table"].shape[0] == H and x["value_table"].shape[0] == H
    dz = gen((B, H, n, d), dtype, 900)
    lens = x["key_lens"]
    lens_l = None if lens is None else lens.tolist()
    g = run_shaw(ra, x["q"], x["k"], x["v"], x["key_table"], x["value_table"], dz, w.clip,
                 w.causal, lens_l)
    rng = np.random.default_rng(902)
    heads = [int(h) for h in rng.choice(H, size=2, replace=False)]
    for h in heads:
        hs = slice(h, h + 1)
        want = oracle.relattn_backward(x["q"][:, hs], x["k"][:, hs], x["v"][:, hs],
                                       x["key_table"][hs], x["value_table"][hs], w.clip,
                                       dz[:, hs], causal=w.causal, key_lens=lens_l)
        got = [t[:, hs] for t in g[:3]] + [g[3][hs], g[4][hs]]
        errs = {name: nerr(a, b) for name, a, b in
                zip(("dq", "dk", "dv", "dwK", "dwV"), got, want)}
        print(f"{shape} head {h}: normalised errors " +
              ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))
        check(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
@pytest.mark.parametrize("window,shared", [(0, False), (5, True), (20, False)])
def test_offset_bias_backward_parity(ra, dtype, mask, window, shared):
    """Scalar bias by clipped offset: dq, dk, dv and the table gradient."""
    B, H, n, d = 2, 3, 150, 64
    q, k, v, dz = (gen((B, H, n, d), dtype, 1000 + window + i) for i in range(4))
    bias = gen((1 if shared else H, 2 * window + 1), torch.float32, 1005)
    causal = mask == "causal"
    lens = [n, 77] if mask == "lens" else None
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, bd, dzd = (dev(x) for x in (q, k, v, bias, dz))
    out, lse = ra.fwd_offset_bias_lse(qd, kd, vd, bd, window, causal=causal, key_lens=lens_d)
    got = ra.bwd_offset_bias(qd, kd, vd, bd, window, out=out, dout=dzd, lse=lse, causal=causal,
                             key_lens=lens_d)
    torch.cuda.synchronize()
    want = oracle.offset_bias_backward(q, k, v, bias, window, dz, causal=causal, key_lens=lens)
    if window == 0 and dtype == torch.bfloat16:
        # one entry for every pair: a constant per head, which the softmax
        # ignores, so the true gradient is 0.  What remains is the rounding of
        # D_i = dz_i.z_i taken with the stored bf16 output: per row
        # |sum_j dS_ij| = |D_exact - D_used| <= 2^-9 sum_d |dz_id| |z_id|
        # (2^-8 below covers the sums' own rounding)
        check(got[:3], want[:3], dtype, names=("dq", "dk", "dv"))
        z = oracle.offset_bias_attention(q, k, v, bias, window, causal=causal, key_lens=lens)
        per_head = 2.0 ** -8 * (np.abs(dz.double().numpy()) * np.abs(z)).sum(axis=(0, 2, 3))
        bound = per_head if bias.shape[0] > 1 else per_head.sum(keepdims=True)
        err = np.abs(got[3].double().cpu().numpy()[:, 0] - want[3][:, 0])
        assert np.all(err <= bound), (err, bound)
    else:
        check(got, want, dtype, names=("dq", "dk", "dv", "dbias"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_alibi_backward_without_bias_gradient(ra, dtype):
    """Causal ALiBi over the whole sequence (window n - 1, fixed slopes): the
    bias gradient is not asked for; dq, dk, dv against the oracle."""
    B, H, n, d = 2, 4, 200, 64
    q, k, v, dz = (gen((B, H, n, d), dtype, 1100 + i) for i in range(4))
    W = n - 1
    slopes = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    bias = torch.tensor([[-m * abs(x) for x in range(-W, W + 1)] for m in slopes])
    qd, kd, vd, bd, dzd = (dev(x) for x in (q, k, v, bias, dz))
    out, lse = ra.fwd_offset_bias_lse(qd, kd, vd, bd, W, causal=True)
    dq, dk, dv, db = ra.bwd_offset_bias(qd, kd, vd, bd, W, out=out, dout=dzd, lse=lse,
                                        causal=True, want_dbias=False)
    torch.cuda.synchronize()
    assert db is None
    want = oracle.offset_bias_backward(q, k, v, bias, W, dz, causal=True)
    check((dq, dk, dv), want[:3], dtype, names=("dq", "dk", "dv"))


def test_backward_rejects_bias_gradient_too_wide(ra):
    """A bias gradient over 2n - 1 offsets does not fit on chip: UNSUPPORTED,
    reported before any launch."""
    B, H, n, d = 1, 2, 600, 64
    q, k, v, dz = (gen((B, H, n, d), torch.bfloat16, 1200 + i).to(DEV) for i in range(4))
    bias = torch.zeros(H, 2 * (n - 1) + 1, device=DEV)
    out, lse = ra.fwd_offset_bias_lse(q, k, v, bias, n - 1)
    with pytest.raises(ra.RelattnError) as e:
        ra.bwd_offset_bias(q, k, v, bias, n - 1, out=out, dout=dz, lse=lse)
    assert e.value.status == ra.UNSUPPORTED
