"""Calls enqueued on a stream other than torch's current one (a torch side
stream, or its raw hipStream_t handle): the workspace and outputs the binding
allocates must not be handed to other work before the kernels on that stream
have used them.  Each call is followed at once by allocations of the same size
on the current stream that are filled with garbage; results are compared with
the fp64 oracle after the side stream finishes.  Bars as elsewhere: 2e-2
max-abs for bf16 forward and decoding, the backward's normalised 3e-2."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

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


def gen(shape, seed, std=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(dtype)


def scribble(nbytes, rounds=4):
    """Allocate and overwrite memory on the current stream while the side
    stream may still be running."""
    keep = []
    for r in range(rounds):
        t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
        t.fill_(0x7f + r)
        keep.append(t)
    return keep


@pytest.mark.parametrize("handle", ["stream", "raw"])
def test_decode_on_side_stream(ra, handle):
    """Few rows over a long cache: the rows are split over workgroups that
    combine through the workspace."""
    B, H, Tq, L, d, c = 2, 2, 1, 3000, 64, 8
    q, k, v = gen((B, H, Tq, d), 1), gen((B, H, L, d), 2), gen((B, H, L, d), 3)
    wK, wV = gen((H, 2 * c + 1, d), 4, 0.1), gen((H, 2 * c + 1, d), 5, 0.1)
    lens = [L, 2100]
    g = [x.to(DEV) for x in (q, k, v, wK, wV)]
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    need = ra.decode_workspace_size(*g, clip=c)
    assert need > 0, "the case must use a workspace"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        out = ra.decode(*g, clip=c, cache_lens=lens_d,
                        stream=side if handle == "stream" else side.cuda_stream)
        outs.append(out)
        junk = scribble(need)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    want = oracle.relattn_decode(q, k, v, wK, wV, c, cache_lens=lens)
    for out in outs:
        err = float(np.max(np.abs(out.float().cpu().numpy() - want)))
        assert err <= 2e-2, err


@pytest.mark.parametrize("handle", ["stream", "raw"])
def test_backward_on_side_stream(ra, handle):
    B, H, n, d, c = 2, 3, 200, 64, 6
    q, k, v, dz = (gen((B, H, n, d), 10 + i) for i in range(4))
    wK, wV = gen((H, 2 * c + 1, d), 15, 0.3), gen((H, 2 * c + 1, d), 16, 0.3)
    g = [x.to(DEV) for x in (q, k, v, wK, wV)]
    dzd = dz.to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    s = side if handle == "stream" else side.cuda_stream
    out, lse = ra.fwd_lse(*g, clip=c, causal=True, stream=s)
    need = ra.bwd_workspace_size(*g, out=out, dout=dzd, lse=lse, clip=c, causal=True)
    assert need > 0, "the case must use a workspace"
    grads = ra.bwd(*g, out=out, dout=dzd, lse=lse, clip=c, causal=True, stream=s)
    junk = scribble(need)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    want = oracle.relattn_backward(q, k, v, wK, wV, c, dz, causal=True)
    for name, a, w in zip(("dq", "dk", "dv", "dwK", "dwV"), grads, want):
        w = np.asarray(w, np.float64)
        e = float(np.max(np.abs(a.double().cpu().numpy() - w))) / max(float(np.abs(w).max()), 1.0)
        assert e <= 3e-2, f"{name}: {e:.3g}"
