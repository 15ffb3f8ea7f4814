"""The decode entry point that allocates nothing (relattn_decode_noalloc,
through the C ABI) against relattn_decode with a caller's workspace: the same
kernels on the same inputs, so the outputs must be bit-identical.  Two calls
in a row on the static scratch, the second with a smaller input, plus the
size limit of the scratch."""
import os
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
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


def gen(B, H, L, d, c, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g)
    q, k, v = r(B, H, 1, d), r(B, H, L, d), r(B, H, L, d)
    wK, wV = r(H, 2 * c + 1, d) * 0.1, r(H, 2 * c + 1, d) * 0.1
    return [x.to(dtype).to(DEV) for x in (q, k, v, wK, wV)]


@pytest.mark.parametrize("t5", [False, True])
def test_noalloc_matches_decode_twice(ra, t5):
    c = 8
    for B, H, L, d, lens in [(2, 3, 3000, 64, [3000, 1711]), (1, 2, 900, 32, [640])]:
        q, k, v, wK, wV = gen(B, H, L, d, c, 77 + L)
        lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
        if t5:
            bias = torch.randn(32, H, generator=torch.Generator().manual_seed(5)).to(DEV)
            kw = dict(t5_bias=bias)
            tabs = (None, None)
        else:
            kw = dict(clip=c)
            tabs = (wK, wV)
        need = ra.decode_workspace_size(q, k, v, *tabs, **kw)
        assert 0 < need <= 4 << 20, "the case must use the scratch"
        want = ra.decode(q, k, v, *tabs, cache_lens=lens_d, **kw)
        got = torch.full_like(want, float("nan"))
        ra.decode_noalloc(q, k, v, *tabs, cache_lens=lens_d, out=got, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (B, H, L, d)


def test_noalloc_rejects_shapes_beyond_the_scratch(ra):
    """960 split rows whose band logits (a clip of 1100 keys) need more than
    4 MiB of workspace: UNSUPPORTED, before any launch.  The cache and the
    tables are expanded views (nothing large is allocated or read)."""
    B, H, L, d, c = 8, 120, 1100, 32, 1100
    z = lambda *shape: torch.zeros(*([1] * (len(shape) - 1)), shape[-1], dtype=torch.bfloat16,
                                   device=DEV).expand(*shape)
    q, kv, tab = z(B, H, 1, d), z(B, H, L, d), z(1, 2 * c + 1, d)
    need = ra.decode_workspace_size(q, kv, kv, tab, tab, clip=c)
    assert need > 4 << 20, need
    out = torch.empty(B, H, 1, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ra.RelattnError) as e:
        ra.decode_noalloc(q, kv, kv, tab, tab, clip=c, out=out)
    assert e.value.status == ra.UNSUPPORTED
