"""GPU parity of the 2-D window (Swin) relative position bias
(relattn_fwd_grid_bias, through the C ABI) against the fp64 oracle
(oracle.grid_bias_attention).  Bars: max-abs 1e-5 (fp32), 2e-2 (bf16)."""
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("M", [1, 4, 7, 8, 12])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("shared", [False, True])
def test_grid_bias_parity(ra, dtype, M, d, shared):
    n = M * M
    B, H = 5, 3
    q, k, v = (gen((B, H, n, d), dtype, 1700 + M + d + i) for i in range(3))
    bias = gen((1 if shared else H, (2 * M - 1) ** 2), torch.float32, 1703)
    lens = [n, max(1, n - 3), n, 1, n]
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = ra.fwd_grid_bias(q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), M, key_lens=lens_d)
    torch.cuda.synchronize()
    want = oracle.grid_bias_attention(q, k, v, bias, M, key_lens=lens)
    err = float(np.max(np.abs(out.double().cpu().numpy() - want)))
    assert err <= TOL[dtype], err


def test_grid_bias_full_size_windows(ra):
    """A stage of a windowed vision transformer: 2048 windows of 7 x 7 tokens,
    3 heads, d = 32 (bf16), against the oracle on sampled windows."""
    B, H, M, d = 2048, 3, 7, 32
    n = M * M
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 1800 + i) for i in range(3))
    bias = gen((H, (2 * M - 1) ** 2), torch.float32, 1803)
    out = ra.fwd_grid_bias(q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), M)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    for b in (0, 777, 2047):
        want = oracle.grid_bias_attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], bias, M)
        assert float(np.max(np.abs(out[b:b + 1] - want))) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("B,H,M,d", [(2045, 3, 7, 32), (49200, 3, 7, 32), (16387, 2, 8, 64),
                                     (3001, 4, 5, 64)])
def test_grid_bias_long_runs(ra, B, H, M, d):
    """Many windows per launch (bf16): each workgroup walks a run of
    (window, head) items that crosses head boundaries, and runs of more than 64
    items restage their key lengths; sampled windows (every head) against the
    oracle, with ragged key lengths."""
    n = M * M
    g = torch.Generator(device=DEV).manual_seed(2100 + B)
    q, k, v = (torch.randn(B, H, n, d, generator=g, device=DEV).to(torch.bfloat16)
               for _ in range(3))
    bias = gen((H, (2 * M - 1) ** 2), torch.float32, 2104)
    lens = torch.randint(1, n + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    out = ra.fwd_grid_bias(q, k, v, bias.to(DEV), M, key_lens=lens)
    torch.cuda.synchronize()
    lens_h = lens.cpu().tolist()
    for b in sorted({0, 1, 63, 64, 65, B // 3, B // 2 + 7, B - 65, B - 2, B - 1}):
        want = oracle.grid_bias_attention(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(),
                                          bias, M, key_lens=[lens_h[b]])
        err = float(np.max(np.abs(out[b:b + 1].double().cpu().numpy() - want)))
        assert err <= TOL[torch.bfloat16], (b, err)


@pytest.mark.parametrize("d", [32, 64])
def test_grid_bias_window_layouts(ra, d):
    """Small windows (bf16) from strided operands: q a head-interleaved
    [B, n, H, d] buffer seen as [B, H, n, d], k and v slices of wider rows, the
    table rows of a wider table, the output written into a strided view;
    windows with no visible key (length 0) give zero rows, like the oracle's."""
    B, H, M = 37, 3, 7
    n = M * M
    g = torch.Generator(device=DEV).manual_seed(2200 + d)
    qb = torch.randn(B, n, H, d, generator=g, device=DEV).to(torch.bfloat16)
    q = qb.permute(0, 2, 1, 3)
    kb = torch.randn(B, H, n, 2 * d, generator=g, device=DEV).to(torch.bfloat16)
    vb = torch.randn(B, H, n, d + 16, generator=g, device=DEV).to(torch.bfloat16)
    k, v = kb[..., d:], vb[..., 8:8 + d]
    nb = (2 * M - 1) ** 2
    bias_w = gen((H, nb + 12), torch.float32, 2204).to(DEV)
    bias = bias_w[:, 4:4 + nb]  # rows of a wider table
    lens = torch.randint(0, n + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    lens[0], lens[1], lens[2] = 0, n, 1
    ob = torch.full((B, H, n, d + 16), float("nan"), device=DEV, dtype=torch.bfloat16)
    out = ob[..., 8:8 + d]  # (operands start on 16-byte boundaries)
    ra.fwd_grid_bias(q, k, v, bias, M, key_lens=lens, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(ob[..., :8]).all() and torch.isnan(ob[..., 8 + d:]).all()
    want = oracle.grid_bias_attention(q.cpu(), k.cpu(), v.cpu(), bias.cpu(), M,
                                      key_lens=lens.cpu().tolist())
    err = float(np.max(np.abs(out.double().cpu().numpy() - want)))
    assert err <= TOL[torch.bfloat16], err
    assert not torch.isnan(out).any()
    assert float(out[0].abs().max()) == 0.0


def test_grid_bias_rejects(ra):
    q = gen((1, 2, 49, 32), torch.bfloat16, 1900).to(DEV)
    bias = torch.zeros(2, 169, device=DEV)
    assert ra.validate_grid_bias(q, q, q, bias, 7) == ra.OK
    assert ra.validate_grid_bias(q, q, q, bias, 6) == ra.INVALID_ARGUMENT       # n != M*M
    assert ra.validate_grid_bias(q, q, q, bias[:, :100], 7) == ra.INVALID_ARGUMENT
    assert ra.validate_grid_bias(q, q, q, bias, 7, causal=True) == ra.INVALID_ARGUMENT
    assert ra.validate_grid_bias(q, q, q, bias, 0) == ra.INVALID_ARGUMENT


# ---------------------------------------------------------------------------
# backward: relattn_fwd_grid_bias_lse + relattn_bwd_grid_bias against the
# oracle's chain-rule gradients (oracle.grid_bias_backward).  Bar as for the
# other backward passes: max|gpu - oracle| <= BTOL * max(max|oracle|, 1), with
# BTOL = 1e-4 (fp32) and 3e-2 (bf16: operands of the weight and dS products
# rounded to bf16, 2^-9 relative each, and dq, dk, dv rounded to bf16).
# ---------------------------------------------------------------------------

BTOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}


def bcheck(got, want, dtype, names=("dq", "dk", "dv", "dbias")):
    for name, g, w in zip(names, got, want):
        w = np.asarray(w, np.float64)
        e = float(np.max(np.abs(g.double().cpu().numpy() - w))) / max(float(np.abs(w).max()), 1.0)
        assert e <= BTOL[dtype], f"{name}: normalised error {e:.3g} > {BTOL[dtype]}"


def grid_grads(ra, q, k, v, bias, M, dz, lens=None, want_dbias=True):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd, bd, dzd = (x.to(DEV) for x in (q, k, v, bias, dz))
    out, lse = ra.fwd_grid_bias_lse(qd, kd, vd, bd, M, key_lens=lens_d)
    g = ra.bwd_grid_bias(qd, kd, vd, bd, M, out=out, dout=dzd, lse=lse, key_lens=lens_d,
                         want_dbias=want_dbias)
    torch.cuda.synchronize()
    return out, lse, g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("M", [1, 4, 7, 8, 12])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("shared", [False, True])
def test_grid_bias_backward_parity(ra, dtype, M, d, shared):
    """dq, dk, dv and the table gradient, ragged key lengths (one window with
    none visible: its gradients are 0)."""
    n = M * M
    B, H = 5, 3
    q, k, v, dz = (gen((B, H, n, d), dtype, 2300 + M + d + i) for i in range(4))
    bias = gen((1 if shared else H, (2 * M - 1) ** 2), torch.float32, 2305)
    lens = [n, max(1, n - 3), 0, 1, n]
    out, lse, got = grid_grads(ra, q, k, v, bias, M, dz, lens)
    want = oracle.grid_bias_backward(q, k, v, bias, M, dz, key_lens=lens)
    bcheck(got, want, dtype)
    for g in got[:3]:
        assert torch.count_nonzero(g[2]).item() == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_grid_bias_lse(ra, dtype):
    """The row statistic of the forward (window kernel for bf16 windows of at
    most 64 tokens, the general kernel otherwise): natural-log log-sum-exp of
    each row's visible logits, -inf for a row that sees none."""
    for M, d in ((7, 32), (8, 64), (9, 64)):
        n = M * M
        B, H = 6, 2
        q, k, v = (gen((B, H, n, d), dtype, 2400 + M + i) for i in range(3))
        bias = gen((H, (2 * M - 1) ** 2), torch.float32, 2404)
        lens = [n, 0, 1, n - 5, n, 2]
        lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
        out, lse = ra.fwd_grid_bias_lse(q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), M,
                                        key_lens=lens_d)
        torch.cuda.synchronize()
        want_out = oracle.grid_bias_attention(q, k, v, bias, M, key_lens=lens)
        assert float(np.max(np.abs(out.double().cpu().numpy() - want_out))) <= TOL[dtype]
        qq, kk = q.double().numpy(), k.double().numpy()
        y, x = np.divmod(np.arange(n), M)
        ent = (y[None, :] - y[:, None] + M - 1) * (2 * M - 1) + (x[None, :] - x[:, None] + M - 1)
        got = lse.double().cpu().numpy()
        for b in range(B):
            for h in range(H):
                e = (qq[b, h] @ kk[b, h].T) / np.sqrt(d) + bias[h].double().numpy()[ent]
                L = lens[b]
                if L == 0:
                    assert np.all(np.isneginf(got[b, h])), (M, b, h)
                    continue
                m = e[:, :L].max(axis=1)
                ref = m + np.log(np.exp(e[:, :L] - m[:, None]).sum(axis=1))
                # bf16: the weights are summed as rounded to bf16 (2^-9 each)
                tol = 1e-5 if dtype == torch.float32 else 2.0 ** -9 + 1e-4
                assert np.max(np.abs(got[b, h] - ref)) <= tol, (M, b, h)


def test_grid_bias_backward_without_bias_gradient(ra):
    """A fixed table: no bias gradient asked for; dq, dk, dv as with one."""
    B, H, M, d = 4, 2, 6, 64
    n = M * M
    q, k, v, dz = (gen((B, H, n, d), torch.bfloat16, 2500 + i) for i in range(4))
    bias = gen((H, (2 * M - 1) ** 2), torch.float32, 2505)
    _, _, got = grid_grads(ra, q, k, v, bias, M, dz, want_dbias=False)
    assert got[3] is None
    want = oracle.grid_bias_backward(q, k, v, bias, M, dz)
    bcheck(got[:3], want[:3], torch.bfloat16, names=("dq", "dk", "dv"))


def test_grid_bias_autograd(ra):
    """torch.autograd through attention_grid_bias matches the oracle (fp32)."""
    B, H, M, d = 3, 2, 5, 32
    n = M * M
    q, k, v, dz = (gen((B, H, n, d), torch.float32, 2600 + i) for i in range(4))
    bias = gen((H, (2 * M - 1) ** 2), torch.float32, 2605)
    leaves = [x.to(DEV).requires_grad_(True) for x in (q, k, v, bias)]
    out = ra.attention_grid_bias(*leaves, M)
    out.backward(dz.to(DEV))
    want = oracle.grid_bias_backward(q, k, v, bias, M, dz)
    bcheck([x.grad for x in leaves], want, torch.float32)


@pytest.mark.parametrize("shared", [False, True])
def test_grid_bias_backward_full_size(ra, shared):
    """A stage of a windowed vision transformer at full size in one call
    (2048 windows of 7 x 7 tokens, 3 heads, d = 32, bf16): the table gradient,
    a sum over every window, element by element against the oracle over all
    windows; dq, dk, dv of sampled windows."""
    B, H, M, d = 2048, 3, 7, 32
    n = M * M
    q, k, v, dz = (gen((B, H, n, d), torch.bfloat16, 2700 + i) for i in range(4))
    bias = gen((1 if shared else H, (2 * M - 1) ** 2), torch.float32, 2705)
    _, _, got = grid_grads(ra, q, k, v, bias, M, dz)
    want = oracle.grid_bias_backward(q, k, v, bias, M, dz)
    bcheck(got[3:], want[3:], torch.bfloat16, names=("dbias",))
    for b in (0, 1023, 2047):
        sl = slice(b, b + 1)
        bcheck([t[sl] for t in got[:3]], [w[sl] for w in want[:3]], torch.bfloat16,
               names=("dq", "dk", "dv"))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [16, 128])
def test_grid_bias_backward_head_sizes(ra, dtype, d):
    """Head sizes 16 and 128 (the general kernel's other register layouts),
    per-head table, ragged key lengths."""
    M, B, H = 6, 4, 2
    n = M * M
    q, k, v, dz = (gen((B, H, n, d), dtype, 2800 + d + i) for i in range(4))
    bias = gen((H, (2 * M - 1) ** 2), torch.float32, 2804)
    lens = [n, 20, 1, n - 1]
    _, _, got = grid_grads(ra, q, k, v, bias, M, dz, lens)
    want = oracle.grid_bias_backward(q, k, v, bias, M, dz, key_lens=lens)
    bcheck(got, want, dtype)
