"""GPU parity of attention with a scalar bias by clipped offset
(relattn_fwd_offset_bias, through the C ABI) against the fp64 oracle; ALiBi is
such a table.  Bars: max-abs 1e-5 (fp32) and 2e-2 (bf16)."""
import math
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


def gen(B, H, n, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, n, d, generator=g).to(dtype) for _ in range(3)]


def alibi(H, window):
    """-m_h |delta| with geometric slopes (one common choice; the pages leave the
    slopes to the model)."""
    m = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)]
    return torch.tensor([[-mh * abs(x) for x in range(-window, window + 1)] for mh in m],
                        dtype=torch.float32)


def run(ra, q, k, v, bias, window, causal=False, lens=None, scale=None):
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = ra.fwd_offset_bias(q.to(DEV), k.to(DEV), v.to(DEV), bias.to(DEV), window,
                             causal=causal, key_lens=lens_d, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b)))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "lens"])
@pytest.mark.parametrize("window", [0, 5, 140])
def test_offset_bias_parity(ra, dtype, d, mask, window):
    B, H, n = 2, 3, 140
    q, k, v = gen(B, H, n, d, dtype, 10 + d + window)
    g = torch.Generator().manual_seed(20 + window)
    bias = torch.randn(H, 2 * window + 1, generator=g)
    causal = mask == "causal"
    lens = [n, 77] if mask == "lens" else None
    got = run(ra, q, k, v, bias, window, causal, lens)
    want = oracle.offset_bias_attention(q, k, v, bias, window, causal=causal, key_lens=lens)
    assert maxerr(got, want) <= TOL[dtype], maxerr(got, want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_alibi_parity(ra, dtype):
    """ALiBi without clipping (window n - 1), causal, shared-free per-head slopes."""
    B, H, n, d = 2, 8, 300, 64
    q, k, v = gen(B, H, n, d, dtype, 30)
    bias = alibi(H, n - 1)
    got = run(ra, q, k, v, bias, n - 1, causal=True)
    want = oracle.offset_bias_attention(q, k, v, bias, n - 1, causal=True)
    assert maxerr(got, want) <= TOL[dtype]


def test_offset_bias_shared_row_and_scale(ra):
    q, k, v = gen(2, 4, 90, 64, torch.bfloat16, 40)
    bias = torch.randn(1, 21, generator=torch.Generator().manual_seed(41))
    got = run(ra, q, k, v, bias, 10, scale=0.3)
    want = oracle.offset_bias_attention(q, k, v, bias, 10, scale=0.3)
    assert maxerr(got, want) <= 2e-2


def test_offset_bias_window_beyond_sequence(ra):
    """A window longer than the sequence: only offsets up to n - 1 are read."""
    q, k, v = gen(1, 2, 50, 64, torch.float32, 50)
    bias = torch.randn(2, 2 * 400 + 1, generator=torch.Generator().manual_seed(51))
    got = run(ra, q, k, v, bias, 400)
    want = oracle.offset_bias_attention(q, k, v, bias, 400)
    assert maxerr(got, want) <= 1e-5


def test_offset_bias_equals_t5_with_bucket_table(ra):
    """Two HIP paths on the same inputs: T5 buckets, and a table by offset
    filled with each offset's bucket bias."""
    B, H, n, d = 2, 4, 200, 64
    g = torch.Generator().manual_seed(60)
    q, k, v = [(torch.randn(B, H, n, d, generator=g) / 8).to(torch.float32) for _ in range(3)]
    t5 = torch.randn(32, H, generator=g)
    W = n - 1
    table = torch.tensor([[t5[oracle.t5_bucket(x, 32, 128, True), h].item()
                           for x in range(-W, W + 1)] for h in range(H)])
    a = ra.fwd(q.to(DEV), k.to(DEV), v.to(DEV), t5_bias=t5.to(DEV), num_buckets=32,
               max_distance=128, bidirectional=True)
    b = ra.fwd_offset_bias(q.to(DEV), k.to(DEV), v.to(DEV), table.to(DEV), W, scale=1.0)
    torch.cuda.synchronize()
    assert maxerr(a.cpu().numpy(), b.cpu().numpy().astype(np.float64)) <= 1e-5


def test_alibi_workload_full_oracle(ra):
    """The T5 shape (B8 H12 n1024 d64, bf16) with causal ALiBi, every output
    against the oracle."""
    B, H, n, d = 8, 12, 1024, 64
    q, k, v = gen(B, H, n, d, torch.bfloat16, 70)
    bias = alibi(H, n - 1)
    got = run(ra, q, k, v, bias, n - 1, causal=True)
    want = oracle.offset_bias_attention(q, k, v, bias, n - 1, causal=True)
    assert maxerr(got, want) <= 2e-2
