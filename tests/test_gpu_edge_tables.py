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
