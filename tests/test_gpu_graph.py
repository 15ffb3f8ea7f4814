"""Calls captured into a HIP graph and replayed: every replay, with eager work of
the program in between, gives the eager result bit for bit (the kernels read
only their inputs and write only their outputs; nothing in these paths records
a memset).  Forward on the lean and the general kernel, decoding with its
workspace, and the backward."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ra():
    import os
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


def gen(shape, seed, std=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(dtype).to(DEV)


def replay_matches(run, eager):
    """Capture run() (which writes into fixed outputs), replay it three times with
    eager work between the replays, compare each replay with `eager`."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the plan caches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        outs = run()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))  # the replay must rewrite every element
        junk = torch.randn(1 << 20, device=DEV) * 3.0  # eager work between replays
        junk.sum().item()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"


@pytest.mark.parametrize("shape", [(2, 3, 256, 64, 16, True),     # lean kernel, causal
                                   (2, 2, 200, 128, 8, False)])   # general kernel, d = 128
def test_forward_graph_replays(ra, shape):
    B, H, n, d, c, causal = shape
    q, k, v = gen((B, H, n, d), 1), gen((B, H, n, d), 2), gen((B, H, n, d), 3)
    wK, wV = gen((H, 2 * c + 1, d), 4, 0.3), gen((H, 2 * c + 1, d), 5, 0.3)
    lens = torch.tensor([n, n - 37], dtype=torch.int32, device=DEV)
    eager = ra.fwd(q, k, v, wK, wV, clip=c, causal=causal, key_lens=lens)
    torch.cuda.synchronize()
    out = torch.empty_like(q)

    def run():
        ra.fwd(q, k, v, wK, wV, clip=c, causal=causal, key_lens=lens, out=out)
        return [out]
    replay_matches(run, [eager])


def test_decode_graph_replays(ra):
    B, H, L, d, c = 2, 2, 3000, 64, 8
    q, k, v = gen((B, H, 1, d), 11), gen((B, H, L, d), 12), gen((B, H, L, d), 13)
    wK, wV = gen((H, 2 * c + 1, d), 14, 0.1), gen((H, 2 * c + 1, d), 15, 0.1)
    lens = torch.tensor([L, 2100], dtype=torch.int32, device=DEV)
    eager = ra.decode(q, k, v, wK, wV, clip=c, cache_lens=lens)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)

    def run():
        ra.decode(q, k, v, wK, wV, clip=c, cache_lens=lens, out=out)
        return [out]
    replay_matches(run, [eager])


def test_backward_graph_replays(ra):
    B, H, n, d, c = 2, 2, 192, 64, 6
    q, k, v, dz = (gen((B, H, n, d), 20 + i) for i in range(4))
    wK, wV = gen((H, 2 * c + 1, d), 25, 0.3), gen((H, 2 * c + 1, d), 26, 0.3)
    out, lse = ra.fwd_lse(q, k, v, wK, wV, clip=c, causal=True)
    eager = [g for g in ra.bwd(q, k, v, wK, wV, out=out, dout=dz, lse=lse, clip=c, causal=True)
             if g is not None]
    torch.cuda.synchronize()

    def run():
        return [g for g in ra.bwd(q, k, v, wK, wV, out=out, dout=dz, lse=lse, clip=c, causal=True)
                if g is not None]
    replay_matches(run, eager)
