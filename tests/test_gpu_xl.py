"""GPU parity of Transformer-XL relative logits (relattn_fwd_xl, through the C
ABI) against the fp64 oracle (oracle.xl_attention).  Bars: max-abs 1e-5 (fp32)
and 2e-2 (bf16; q + u and q + v are rounded once to bf16 like every operand)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
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


def run(ra, q, k, v, R, u, vb, window, causal=False, lens=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = ra.fwd_xl(*(x.to(DEV) for x in (q, k, v, R, u, vb)), window, causal=causal,
                    key_lens=lens_d, scale=scale)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
@pytest.mark.parametrize("window", ["full", 16])
def test_xl_parity(ra, dtype, d, mask, window):
    B, H, n = 2, 3, 150
    W = n - 1 if window == "full" else window
    q, k, v = (gen((B, H, n, d), dtype, 1300 + d + i) for i in range(3))
    R = gen((H, 2 * W + 1, d), dtype, 1303, 0.5)
    u, vb = gen((H, d), dtype, 1304, 0.5), gen((H, d), dtype, 1305, 0.5)
    causal = mask == "causal"
    lens = [n, 93] if mask == "lens" else None
    got = run(ra, q, k, v, R, u, vb, W, causal, lens)
    # the oracle takes q + u and q + v exactly; the kernel rounds each sum once
    # to the input dtype, which the bf16 bar covers
    want = oracle.xl_attention(q, k, v, R, u, vb, W, causal=causal, key_lens=lens)
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_xl_shared_and_scale(ra, dtype):
    """R, u and v shared by all heads; an explicit scale; a ragged small n."""
    B, H, n, d, W = 2, 4, 37, 64, 40
    q, k, v = (gen((B, H, n, d), dtype, 1400 + i) for i in range(3))
    R = gen((1, 2 * W + 1, d), dtype, 1403, 0.5)
    u, vb = gen((1, d), dtype, 1404, 0.5), gen((1, d), dtype, 1405, 0.5)
    got = run(ra, q, k, v, R, u, vb, W, causal=True, scale=0.2)
    want = oracle.xl_attention(q, k, v, R, u, vb, W, scale=0.2, causal=True)
    assert float(np.max(np.abs(got - want))) <= TOL[dtype]


def test_xl_zero_biases_match_shaw_with_reversed_table(ra):
    """u = v = 0: relattn_fwd with the table reversed computes the same
    attention.  At bf16 and d = 64 the two calls run different kernels (the
    Shaw call takes the lean kernel, whose normaliser sums the bf16-rounded
    weights), so they agree to the output rounding: one bf16 step (2^-8
    relative) either way, 2^-7 of the largest output; both meet the oracle."""
    B, H, n, d, W = 2, 2, 130, 64, 129
    dtype = torch.bfloat16
    qc, kc, vc = (gen((B, H, n, d), dtype, 1500 + i) for i in range(3))
    Rc = gen((H, 2 * W + 1, d), dtype, 1503, 0.5)
    q, k, v, R = (t.to(DEV) for t in (qc, kc, vc, Rc))
    zero = torch.zeros(H, d, dtype=dtype, device=DEV)
    a = ra.fwd_xl(q, k, v, R, zero, zero, W, causal=True)
    b = ra.fwd(q, k, v, R.flip(1).contiguous(), None, clip=W, causal=True)
    torch.cuda.synchronize()
    a, b = a.float().cpu().numpy(), b.float().cpu().numpy()
    assert float(np.max(np.abs(a - b))) <= 2.0 ** -7 * max(float(np.abs(b).max()), 1.0)
    want = oracle.relattn_factored(qc, kc, vc, Rc.flip(1).contiguous(), None, W, causal=True)
    assert float(np.max(np.abs(a - want))) <= TOL[dtype]
    assert float(np.max(np.abs(b - want))) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n", [1, 33, 97])
@pytest.mark.parametrize("causal", [False, True])
def test_xl_small_rows_d16(ra, dtype, n, causal):
    """Short and ragged segments at d = 16 (a single partial key tile, tiles
    whose distance block reaches past both ends of the table)."""
    B, H, d, W = 2, 2, 16, 20
    q, k, v = (gen((B, H, n, d), dtype, 1700 + n + i) for i in range(3))
    R = gen((H, 2 * W + 1, d), dtype, 1703, 0.5)
    u, vb = gen((H, d), dtype, 1704, 0.5), gen((H, d), dtype, 1705, 0.5)
    got = run(ra, q, k, v, R, u, vb, W, causal, [n, max(1, n - 7)])
    want = oracle.xl_attention(q, k, v, R, u, vb, W, causal=causal, key_lens=[n, max(1, n - 7)])
    assert float(np.max(np.abs(got - want))) <= TOL[dtype]


@pytest.mark.parametrize("name,slices", [("xl", ((0, 0), (3, 9), (7, 15))),
                                         ("xl128", ((0, 0), (4, 3), (7, 7)))])
def test_xl_full_size(ra, name, slices):
    """The benchmark segments (B8 H16 n512 d64 and B8 H8 n512 d128, causal, every
    distance), in the launch configuration the benchmark times, against the
    oracle on sampled (batch, head) slices."""
    import workloads
    w = workloads.XL_WORKLOADS[name]
    x = workloads.make_xl_inputs(w)
    out = ra.fwd_xl(*(x[key].to(DEV) for key in ("q", "k", "v", "R", "u", "vb")), x["window"],
                    causal=True)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    for b, h in slices:
        sl = lambda t: t[b:b + 1, h:h + 1]
        want = oracle.xl_attention(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["R"][h:h + 1],
                                   x["u"][h:h + 1], x["vb"][h:h + 1], x["window"], causal=True)
        err = float(np.max(np.abs(out[b:b + 1, h:h + 1] - want)))
        assert err <= TOL[torch.bfloat16], (b, h, err)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_xl_long_segment(ra, d):
    """n = 2048 with every distance (fused mode: 32 key tiles per row, table
    rows read across the whole window)."""
    B, H, n = 1, 2, 2048
    W = n - 1
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 1800 + d + i) for i in range(3))
    R = gen((H, 2 * W + 1, d), torch.bfloat16, 1803, 0.5)
    u, vb = gen((H, d), torch.bfloat16, 1804, 0.5), gen((H, d), torch.bfloat16, 1805, 0.5)
    got = run(ra, q, k, v, R, u, vb, W, causal=True, lens=[2000])
    want = oracle.xl_attention(q, k, v, R, u, vb, W, causal=True, key_lens=[2000])
    assert float(np.max(np.abs(got - want))) <= TOL[torch.bfloat16]


def test_xl_rejects(ra):
    q = gen((1, 2, 16, 64), torch.bfloat16, 1600).to(DEV)
    R = gen((2, 9, 64), torch.bfloat16, 1601).to(DEV)
    u = gen((2, 64), torch.bfloat16, 1602).to(DEV)
    assert ra.validate_xl(q, q, q, R, u, u, 4) == ra.OK
    assert ra.validate_xl(q, q, q, R, u.float(), u, 4) == ra.INVALID_ARGUMENT
    assert ra.validate_xl(q, q, q, R, u[:, :32].contiguous(), u, 4) == ra.INVALID_ARGUMENT
    assert ra.validate_xl(q, q, q, R, u, u, 5) == ra.INVALID_ARGUMENT  # R rows != 2W + 1


# ---------------------------------------------------------------------------
# backward: relattn_fwd_xl_lse + relattn_bwd_xl against the oracle's
# chain-rule gradients (oracle.xl_backward).  Bar as for the other backward
# passes: max|gpu - oracle| <= BTOL * max(max|oracle|, 1), BTOL = 1e-4 (fp32)
# and 3e-2 (bf16: the product operands rounded to bf16, 2^-9 relative each,
# q + u and q + v rounded once like every operand, and dq, dk, dv rounded to
# bf16).
# ---------------------------------------------------------------------------

BTOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}
XL_GRADS = ("dq", "dk", "dv", "dR", "du", "dv_bias")


def bcheck(got, want, dtype, names=XL_GRADS):
    for name, g, w in zip(names, got, want):
        w = np.asarray(w, np.float64)
        e = float(np.max(np.abs(g.double().cpu().numpy() - w))) / max(float(np.abs(w).max()), 1.0)
        assert e <= BTOL[dtype], f"{name}: normalised error {e:.3g} > {BTOL[dtype]}"


def xl_grads(ra, q, k, v, R, u, vb, W, dz, causal=False, lens=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, Rd, ud, vbd, dzd = (x.to(DEV) for x in (q, k, v, R, u, vb, dz))
    out, lse = ra.fwd_xl_lse(qd, kd, vd, Rd, ud, vbd, W, causal=causal, key_lens=lens_d)
    g = ra.bwd_xl(qd, kd, vd, Rd, ud, vbd, W, out=out, dout=dzd, lse=lse, causal=causal,
                  key_lens=lens_d)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
@pytest.mark.parametrize("window", ["full", 9])
def test_xl_backward_parity(ra, dtype, d, mask, window):
    """Every gradient, per-head R, u and v, the full distance range and a
    clipped one (end rows shared by the far pairs), under every mask (fp32 at
    d = 128 over 64 tokens: the 199 rows of 100 would not fit on chip)."""
    B, H = 2, 2
    n = 64 if (dtype == torch.float32 and d == 128) else 100
    W = n - 1 if window == "full" else window
    q, k, v, dz = (gen((B, H, n, d), dtype, 3400 + d + i) for i in range(4))
    R = gen((H, 2 * W + 1, d), dtype, 3404, 0.5)
    u, vb = gen((H, d), dtype, 3405, 0.5), gen((H, d), dtype, 3406, 0.5)
    causal = mask == "causal"
    lens = [n, 61] if mask == "lens" else None
    got = xl_grads(ra, q, k, v, R, u, vb, W, dz, causal, lens)
    want = oracle.xl_backward(q, k, v, R, u, vb, W, dz, causal=causal, key_lens=lens)
    bcheck(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_xl_backward_shared_and_empty(ra, dtype):
    """One R, u and v for every head (gradients summed over the heads), an
    explicit scale, and a sequence with no visible key (its gradients 0)."""
    B, H, n, d, W = 3, 3, 70, 64, 20
    q, k, v, dz = (gen((B, H, n, d), dtype, 3500 + i) for i in range(4))
    R = gen((1, 2 * W + 1, d), dtype, 3504, 0.5)
    u, vb = gen((1, d), dtype, 3505, 0.5), gen((1, d), dtype, 3506, 0.5)
    lens = [n, 0, 33]
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, Rd, ud, vbd, dzd = (x.to(DEV) for x in (q, k, v, R, u, vb, dz))
    out, lse = ra.fwd_xl_lse(qd, kd, vd, Rd, ud, vbd, W, causal=True, key_lens=lens_d,
                             scale=0.3)
    got = ra.bwd_xl(qd, kd, vd, Rd, ud, vbd, W, out=out, dout=dzd, lse=lse, causal=True,
                    key_lens=lens_d, scale=0.3)
    torch.cuda.synchronize()
    want = oracle.xl_backward(q, k, v, R, u, vb, W, dz, scale=0.3, causal=True, key_lens=lens)
    bcheck(got, want, dtype)
    for g in got[:3]:
        assert torch.count_nonzero(g[1]).item() == 0


def test_xl_backward_autograd(ra):
    """torch.autograd through attention_xl matches the oracle (fp32)."""
    B, H, n, d, W = 2, 2, 40, 32, 12
    q, k, v, dz = (gen((B, H, n, d), torch.float32, 3600 + i) for i in range(4))
    R = gen((H, 2 * W + 1, d), torch.float32, 3604, 0.5)
    u, vb = gen((H, d), torch.float32, 3605, 0.5), gen((H, d), torch.float32, 3606, 0.5)
    leaves = [x.to(DEV).requires_grad_(True) for x in (q, k, v, R, u, vb)]
    out = ra.attention_xl(*leaves, W, causal=True)
    out.backward(dz.to(DEV))
    want = oracle.xl_backward(q, k, v, R, u, vb, W, dz, causal=True)
    bcheck([x.grad for x in leaves], want, torch.float32)


def test_xl_backward_full_segment(ra):
    """The language-model segment at full size (B8 H16 n512 d64, every
    distance, causal, bf16): one row of relative logits per query over 512
    distances takes the one-wave query tiles.  dq, dk, dv of sampled (batch,
    head) pairs against the oracle on those heads; dR, du and dv of two sampled
    heads element by element against the oracle summed over the batch."""
    import workloads
    x = workloads.make_xl_inputs("xl")
    q, k, v, R, u, vb, W = (x[t] for t in ("q", "k", "v", "R", "u", "vb", "window"))
    B, H, n, d = q.shape
    dz = gen(q.shape, q.dtype, 3700)
    got = xl_grads(ra, q, k, v, R, u, vb, W, dz, causal=True)
    rng = np.random.default_rng(3701)
    for h in (int(z) for z in rng.choice(H, size=2, replace=False)):
        hs = slice(h, h + 1)
        want = oracle.xl_backward(q[:, hs], k[:, hs], v[:, hs], R[hs], u[hs], vb[hs], W,
                                  dz[:, hs], causal=True)
        bcheck([got[3][hs], got[4][hs], got[5][hs]], want[3:], torch.bfloat16,
               names=("dR", "du", "dv_bias"))
        for b in (int(z) for z in rng.choice(B, size=2, replace=False)):
            bcheck([t[b:b + 1, hs] for t in got[:3]], [w[b:b + 1] for w in want[:3]],
                   torch.bfloat16, names=("dq", "dk", "dv"))


def test_shaw_backward_widest_window(ra):
    """The key table alone over every offset of a 512-token causal sequence
    (bf16, d = 64): the one-wave query tiles, against the oracle on sampled
    heads."""
    B, H, n, d, c = 2, 4, 512, 64, 511
    q, k, v, dz = (gen((B, H, n, d), torch.bfloat16, 3800 + i) for i in range(4))
    wK = gen((H, 2 * c + 1, d), torch.bfloat16, 3804, 0.5)
    qd, kd, vd, wkd, dzd = (x.to(DEV) for x in (q, k, v, wK, dz))
    out, lse = ra.fwd_lse(qd, kd, vd, wkd, None, clip=c, causal=True)
    got = ra.bwd(qd, kd, vd, wkd, None, out=out, dout=dzd, lse=lse, clip=c, causal=True)
    torch.cuda.synchronize()
    for h in (0, 3):
        hs = slice(h, h + 1)
        want = oracle.relattn_backward(q[:, hs], k[:, hs], v[:, hs], wK[hs], None, c, dz[:, hs],
                                       causal=True)
        bcheck([got[0][:, hs], got[1][:, hs], got[2][:, hs], got[3][hs]], want[:4],
               torch.bfloat16, names=("dq", "dk", "dv", "dwK"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n,causal", [(1, True), (33, True), (97, False)])
def test_xl_backward_d16(ra, dtype, n, causal):
    """Head size 16, short segments (one row, a ragged tail), every distance."""
    B, H, d = 2, 2, 16
    W = max(n - 1, 0)
    q, k, v, dz = (gen((B, H, n, d), dtype, 3900 + n + i) for i in range(4))
    R = gen((H, 2 * W + 1, d), dtype, 3904, 0.5)
    u, vb = gen((H, d), dtype, 3905, 0.5), gen((H, d), dtype, 3906, 0.5)
    got = xl_grads(ra, q, k, v, R, u, vb, W, dz, causal)
    want = oracle.xl_backward(q, k, v, R, u, vb, W, dz, causal=causal)
    bcheck(got, want, dtype)
