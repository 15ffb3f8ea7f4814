"""GPU parity of relation-aware attention over a labeled graph
(relattn_fwd_edge_tables, through the C ABI: key and value tables indexed by a
per-pair label) against the fp64 oracle (oracle.edge_label_relattn).  Bars:
max-abs 1e-5 (fp32), 2e-2 (bf16), as for the other forward arms."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

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


def labels_of(ra, E):
    B, n, _ = E.shape
    lab = ra.edge_label_buffer(B, n, DEV)
    lab.copy_(torch.as_tensor(E).to(torch.uint8))
    return lab


def run(ra, q, k, v, E, wK, wV, causal=False, lens=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    dev = lambda t: None if t is None else t.to(DEV)
    out = ra.fwd_edge_tables(q.to(DEV), k.to(DEV), v.to(DEV), labels_of(ra, E), dev(wK), dev(wV),
                             causal=causal, key_lens=lens_d, scale=scale)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n", [1, 37, 130])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("tables", ["KV", "K", "V"])
@pytest.mark.parametrize("mask", ["none", "causal+lens", "lens"])
def test_edge_tables_parity(ra, dtype, n, d, tables, mask):
    B, H, NL = 3, 2, 20
    q, k, v = (gen((B, H, n, d), dtype, 3000 + n + d + i) for i in range(3))
    wK = gen((H, NL, d), dtype, 3003, 0.5) if "K" in tables else None
    wV = gen((H, NL, d), dtype, 3004, 0.5) if "V" in tables else None
    E = np.random.default_rng(3005 + n).integers(0, NL, (B, n, n))
    causal = mask.startswith("causal")
    lens = [n, max(1, n // 2), max(1, n - 3)] if "lens" in mask else None
    got = run(ra, q, k, v, E, wK, wV, causal, lens)
    want = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=causal, key_lens=lens)
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 16), (torch.bfloat16, 128),
                                     (torch.float32, 16), (torch.float32, 128)], ids=str)
@pytest.mark.parametrize("NL,shared", [(1, False), (7, True), (100, False)])
def test_edge_tables_head_sizes_and_vocabularies(ra, dtype, d, NL, shared):
    B, H, n = 2, 3, 75
    q, k, v = (gen((B, H, n, d), dtype, 3100 + d + NL + i) for i in range(3))
    wK = gen((1 if shared else H, NL, d), dtype, 3103 + NL, 0.5)
    wV = gen((1 if shared else H, NL, d), dtype, 3104 + NL, 0.5)
    E = np.random.default_rng(3105 + NL).integers(0, NL, (B, n, n))
    got = run(ra, q, k, v, E, wK, wV, causal=True, lens=[n, 40])
    want = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=True, key_lens=[n, 40])
    assert float(np.max(np.abs(got - want))) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_edge_tables_large_logits_rescale_the_sums(ra, dtype):
    """Logits that grow along the row (keys scaled up with j) force the running
    max, and with it the per-label weight sums, to be rescaled tile after tile."""
    B, H, n, d, NL = 2, 2, 256, 64, 12
    q = gen((B, H, n, d), dtype, 3200)
    k = (gen((B, H, n, d), torch.float32, 3201) * torch.linspace(0.1, 3.0, n)[:, None]).to(dtype)
    v = gen((B, H, n, d), dtype, 3202)
    wK, wV = gen((H, NL, d), dtype, 3203, 0.5), gen((H, NL, d), dtype, 3204, 0.5)
    E = np.random.default_rng(3205).integers(0, NL, (B, n, n))
    got = run(ra, q, k, v, E, wK, wV)
    want = oracle.edge_label_relattn(q, k, v, E, wK, wV)
    assert float(np.max(np.abs(got - want))) <= TOL[dtype]


def test_edge_tables_of_clipped_offsets_match_shaw(ra):
    """Labels clip(j - i, c) + c with the 2c+1-row tables: the same logits as
    relattn_fwd (the relative rows are the same MFMA products), and outputs
    within the bar of each other (the value term sums the weights in another
    order)."""
    B, H, n, d, c = 2, 4, 200, 64, 16
    dtype = torch.bfloat16
    q, k, v = (gen((B, H, n, d), dtype, 3300 + i).to(DEV) for i in range(3))
    wK = gen((H, 2 * c + 1, d), dtype, 3303, 0.5).to(DEV)
    wV = gen((H, 2 * c + 1, d), dtype, 3304, 0.5).to(DEV)
    E = np.stack([oracle.relative_labels(n, c) + c] * B)
    lens = torch.tensor([n, 150], dtype=torch.int32, device=DEV)
    a = ra.fwd_edge_tables(q, k, v, labels_of(ra, E), wK, wV, causal=True, key_lens=lens)
    b = ra.fwd(q, k, v, wK, wV, clip=c, causal=True, key_lens=lens)
    torch.cuda.synchronize()
    assert float((a.float() - b.float()).abs().max()) <= TOL[dtype]


def test_edge_tables_labels_past_the_table_read_the_last_row(ra):
    B, H, n, d, NL = 2, 2, 50, 32, 5
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 3400 + i) for i in range(3))
    wK, wV = gen((H, NL, d), torch.bfloat16, 3403, 0.5), gen((H, NL, d), torch.bfloat16, 3404, 0.5)
    E = np.random.default_rng(3405).integers(0, 256, (B, n, n))
    got = run(ra, q, k, v, E, wK, wV)
    want = oracle.edge_label_relattn(q, k, v, np.minimum(E, NL - 1), wK, wV)
    assert float(np.max(np.abs(got - want))) <= TOL[torch.bfloat16]


def test_edge_tables_one_matrix_for_the_batch(ra):
    B, H, n, d, NL = 3, 2, 70, 64, 9
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 3500 + i) for i in range(3))
    wK, wV = gen((H, NL, d), torch.bfloat16, 3503, 0.5), gen((H, NL, d), torch.bfloat16, 3504, 0.5)
    E1 = np.random.default_rng(3505).integers(0, NL, (1, n, n))
    lab = labels_of(ra, E1).expand(B, n, n)
    out = ra.fwd_edge_tables(q.to(DEV), k.to(DEV), v.to(DEV), lab, wK.to(DEV), wV.to(DEV))
    torch.cuda.synchronize()
    want = oracle.edge_label_relattn(q, k, v, np.repeat(E1, B, axis=0), wK, wV)
    assert float(np.max(np.abs(out.double().cpu().numpy() - want))) <= TOL[torch.bfloat16]


def test_edge_tables_full_size(ra):
    """The benchmark shape (B16 H16 n256 d64, 64 labels uniform per pair, key and
    value tables), in the launch configuration the benchmark times, against the
    oracle on sampled (batch, head) slices."""
    w = workloads.EDGE_WORKLOADS["edge_kv"]
    x = workloads.make_edge_inputs(w)
    E = x["labels"].numpy()
    out = ra.fwd_edge_tables(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), labels_of(ra, E),
                             x["wK"].to(DEV), x["wV"].to(DEV))
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    for b, h in ((0, 0), (9, 4), (15, 15)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        want = oracle.edge_label_relattn(sl(x["q"]), sl(x["k"]), sl(x["v"]), E[b:b + 1],
                                         x["wK"][h:h + 1], x["wV"][h:h + 1])
        err = float(np.max(np.abs(out[b:b + 1, h:h + 1] - want)))
        assert err <= TOL[torch.bfloat16], (b, h, err)


def test_edge_tables_empty_problems(ra):
    wK = torch.zeros(2, 4, 32, dtype=torch.bfloat16, device=DEV)
    for B, n in ((0, 16), (2, 0)):
        q = torch.zeros(B, 2, n, 32, dtype=torch.bfloat16, device=DEV)
        out = ra.fwd_edge_tables(q, q, q, ra.edge_label_buffer(B, n, DEV), wK, wK)
        assert out.shape == q.shape


@pytest.mark.parametrize("causal", [False, True])
def test_edge_tables_long_rows(ra, causal):
    """n = 600 (ten key tiles per row, several weight-sum rescales), 48 labels."""
    B, H, n, d, NL = 1, 2, 600, 32, 48
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 3600 + i) for i in range(3))
    wK, wV = gen((H, NL, d), torch.bfloat16, 3603, 0.5), gen((H, NL, d), torch.bfloat16, 3604, 0.5)
    E = np.random.default_rng(3605).integers(0, NL, (B, n, n))
    got = run(ra, q, k, v, E, wK, wV, causal=causal, lens=[555])
    want = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=causal, key_lens=[555])
    assert float(np.max(np.abs(got - want))) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("d,NL", [(64, 256), (128, 200)])
def test_edge_tables_largest_vocabulary(ra, d, NL):
    """The largest vocabularies that fit (256 labels, all the uint8 labels
    address, at d = 64; 200 at d = 128): the per-query label rows and weight
    sums take most of the LDS, the plan falls back to smaller workgroups and
    staged value tables."""
    B, H, n = 2, 2, 150
    q, k, v = (gen((B, H, n, d), torch.bfloat16, 3700 + d + i) for i in range(3))
    wK, wV = gen((H, NL, d), torch.bfloat16, 3703, 0.5), gen((H, NL, d), torch.bfloat16, 3704, 0.5)
    E = np.random.default_rng(3705).integers(0, NL, (B, n, n))
    got = run(ra, q, k, v, E, wK, wV, causal=True, lens=[n, 120])
    want = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=True, key_lens=[n, 120])
    assert float(np.max(np.abs(got - want))) <= TOL[torch.bfloat16]


# ---------------------------------------------------------------------------
# backward: relattn_fwd_edge_tables_lse + relattn_bwd_edge_tables against the
# oracle's chain-rule gradients (oracle.edge_label_relattn_backward).  Bar as
# for the other backward passes: max|gpu - oracle| <= BTOL * max(max|oracle|,
# 1), BTOL = 1e-4 (fp32) and 3e-2 (bf16: the product operands rounded to bf16,
# 2^-9 relative each, and dq, dk, dv rounded to bf16).
# ---------------------------------------------------------------------------

BTOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}
GRADS = ("dq", "dk", "dv", "dwK", "dwV")


def bcheck(got, want, dtype, names=GRADS):
    for name, g, w in zip(names, got, want):
        if w is None:
            assert g is None, name
            continue
        w = np.asarray(w, np.float64)
        e = float(np.max(np.abs(g.double().cpu().numpy() - w))) / max(float(np.abs(w).max()), 1.0)
        assert e <= BTOL[dtype], f"{name}: normalised error {e:.3g} > {BTOL[dtype]}"


def edge_table_grads(ra, q, k, v, E, wK, wV, dz, causal=False, lens=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    dev = lambda x: None if x is None else x.to(DEV)
    qd, kd, vd, wkd, wvd, dzd = (dev(x) for x in (q, k, v, wK, wV, dz))
    lab = labels_of(ra, E)
    out, lse = ra.fwd_edge_tables_lse(qd, kd, vd, lab, wkd, wvd, causal=causal, key_lens=lens_d)
    g = ra.bwd_edge_tables(qd, kd, vd, lab, wkd, wvd, out=out, dout=dzd, lse=lse, causal=causal,
                           key_lens=lens_d)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("n", [1, 37, 130])
@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("tables", ["KV", "K", "V"])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
def test_edge_tables_backward_parity(ra, dtype, n, d, tables, mask):
    """dq, dk, dv and the table gradients; some labels lie past the tables
    (read as the last row, as the oracle is given them)."""
    B, H, NL = 2, 2, 24
    q, k, v, dz = (gen((B, H, n, d), dtype, 3900 + n + d + i) for i in range(4))
    wK = gen((H, NL, d), dtype, 3904, 0.5) if "K" in tables else None
    wV = gen((H, NL, d), dtype, 3905, 0.5) if "V" in tables else None
    E = np.random.default_rng(3906 + n).integers(0, NL + 4, (B, n, n))
    causal = mask == "causal"
    lens = [n, max(1, n // 2)] if mask == "lens" else None
    got = edge_table_grads(ra, q, k, v, E, wK, wV, dz, causal, lens)
    want = oracle.edge_label_relattn_backward(q, k, v, np.minimum(E, NL - 1), wK, wV, dz,
                                              causal=causal, key_lens=lens)
    bcheck(got, want, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d,NL,tables", [(16, 1, "KV"), (128, 7, "KV"), (64, 64, "KV"),
                                         (64, 256, "K"), (32, 100, "V")])
def test_edge_tables_backward_shapes(ra, dtype, d, NL, tables):
    """Head sizes 16 and 128, one label, the longest tables that fit (every
    label for the key table alone, through the one-wave query tiles), shared
    tables (gradients summed over the heads) and an empty sequence."""
    if dtype == torch.float32 and (d, NL) in ((64, 256), (128, 7)):
        NL = 32  # fp32 rows take twice the room
    B, H, n = 3, 3, 70
    q, k, v, dz = (gen((B, H, n, d), dtype, 4000 + d + NL + i) for i in range(4))
    wK = gen((1, NL, d), dtype, 4004, 0.5) if "K" in tables else None
    wV = gen((1, NL, d), dtype, 4005, 0.5) if "V" in tables else None
    E = np.random.default_rng(4006 + NL).integers(0, NL, (B, n, n))
    lens = [n, 0, 33]
    got = edge_table_grads(ra, q, k, v, E, wK, wV, dz, True, lens)
    want = oracle.edge_label_relattn_backward(q, k, v, E, wK, wV, dz, causal=True, key_lens=lens)
    if NL == 1 and dtype == torch.bfloat16:
        # one label for every pair: dwK = s sum_i (sum_j dS_ij) q_i vanishes
        # identically; what remains is the rounding of D_i = dz_i.z_i taken
        # with the stored bf16 output, |sum_j dS_ij| <= 2^-9 sum_d |dz_id| |z_id|
        # per row (2^-8 below covers the sums' own rounding)
        bcheck(got[:3] + (None, got[4]), want[:3] + (None, want[4]), dtype)
        z = oracle.edge_label_relattn(q, k, v, E, wK, wV, causal=True, key_lens=lens)
        qq, zz = q.double().numpy(), dz.double().numpy()
        row = 2.0 ** -8 * (np.abs(zz) * np.abs(z)).sum(axis=3, keepdims=True)  # [B, H, n, 1]
        bound = (row * np.abs(qq)).sum(axis=(0, 1, 2)) / np.sqrt(d)
        err = np.abs(got[3].double().cpu().numpy()[0, 0] - want[3][0, 0])
        assert np.all(err <= bound), (err.max(), bound.min())
    else:
        bcheck(got, want, dtype)
    for g in got[:3]:
        assert torch.count_nonzero(g[1]).item() == 0


def test_edge_tables_backward_is_shaw_backward_on_offset_labels(ra):
    """Labels clip(j - i, k) + k with the 2k+1-row tables: the same gradients as
    relattn_bwd with the clipped offset (fp32, within rounding)."""
    B, H, n, d, c = 2, 2, 90, 64, 6
    q, k, v, dz = (gen((B, H, n, d), torch.float32, 4100 + i) for i in range(4))
    wK, wV = gen((H, 2 * c + 1, d), torch.float32, 4104, 0.5), gen((H, 2 * c + 1, d),
                                                                  torch.float32, 4105, 0.5)
    E = np.stack([oracle.relative_labels(n, c) + c] * B)
    got = edge_table_grads(ra, q, k, v, E, wK, wV, dz, True)
    qd, kd, vd, wkd, wvd, dzd = (x.to(DEV) for x in (q, k, v, wK, wV, dz))
    out, lse = ra.fwd_lse(qd, kd, vd, wkd, wvd, clip=c, causal=True)
    ref = ra.bwd(qd, kd, vd, wkd, wvd, out=out, dout=dzd, lse=lse, clip=c, causal=True)
    torch.cuda.synchronize()
    for name, a, b_ in zip(GRADS, got, ref[:5]):
        e = float((a - b_).abs().max()) / max(float(b_.abs().max()), 1.0)
        assert e <= 1e-4, (name, e)


def test_edge_tables_autograd(ra):
    """torch.autograd through attention_edge_tables matches the oracle (fp32)."""
    B, H, n, d, NL = 2, 2, 40, 32, 9
    q, k, v, dz = (gen((B, H, n, d), torch.float32, 4200 + i) for i in range(4))
    wK, wV = gen((H, NL, d), torch.float32, 4204, 0.5), gen((H, NL, d), torch.float32, 4205, 0.5)
    E = np.random.default_rng(4206).integers(0, NL, (B, n, n))
    leaves = [x.to(DEV).requires_grad_(True) for x in (q, k, v, wK, wV)]
    out = ra.attention_edge_tables(leaves[0], leaves[1], leaves[2], labels_of(ra, E), leaves[3],
                                   leaves[4], causal=True)
    out.backward(dz.to(DEV))
    want = oracle.edge_label_relattn_backward(q, k, v, E, wK, wV, dz, causal=True)
    bcheck([x.grad for x in leaves], want, torch.float32)


def test_edge_tables_backward_full_size(ra):
    """The labeled-graph workload at full size in one call (B16 H16 n256 d64, 64
    labels uniform per pair, key and value tables, bf16): dq, dk, dv of sampled
    (batch, head) pairs against the oracle on those heads, and the table
    gradients of two sampled heads element by element against the oracle
    summed over the batch."""
    x = workloads.make_edge_inputs("edge_kv")
    q, k, v, wK, wV = (x[t] for t in ("q", "k", "v", "wK", "wV"))
    E = x["labels"].numpy()
    B, H, n, d = q.shape
    dz = gen(q.shape, q.dtype, 4300)
    got = edge_table_grads(ra, q, k, v, E, wK, wV, dz)
    rng = np.random.default_rng(4301)
    for h in (int(z) for z in rng.choice(H, size=2, replace=False)):
        hs = slice(h, h + 1)
        want = oracle.edge_label_relattn_backward(q[:, hs], k[:, hs], v[:, hs], E, wK[hs],
                                                  wV[hs], dz[:, hs])
        bcheck([got[3][hs], got[4][hs]], want[3:], torch.bfloat16, names=("dwK", "dwV"))
        for b in (int(z) for z in rng.choice(B, size=2, replace=False)):
            bcheck([t[b:b + 1, hs] for t in got[:3]], [w[b:b + 1] for w in want[:3]],
                   torch.bfloat16, names=("dq", "dk", "dv"))
