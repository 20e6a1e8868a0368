"""Streams and graph capture through the C ABI.

The library keeps no global state and enqueues all work on the stream it is
given: calls on different streams with different workspaces may overlap, and
the cold path (prepare with k-means, then forward) issues no host
synchronisation and no memset, so it can be captured in a HIP graph and
replayed.  Both must give results bit-identical to plain eager calls."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gpu_common as G  # noqa: E402

import precision_fp8_attention_amd as vc  # noqa: E402
from synthetic import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vc.lib()


def _case(seed, flags=vc.DEFAULT_FLAGS):
    B, H, N, C_ = 1, 3, 1000, 8
    p = G.lib_params(B, H, N, C_, seed=seed, rho=0.02, flags=flags)
    q, k, v = inputs.make_custom(B, H, N, seed=seed)
    return p, G.to_device(q, k, v)


def test_two_streams_overlap_bit_identical():
    import torch
    cases = [_case(11), _case(12, vc.DEFAULT_FLAGS | vc.V4 | vc.FP8_SCORES)]
    G.log("[case] two streams: eager references on the current stream")
    ref = []
    for p, (qd, kd, vd) in cases:
        _, o = G.run(p, qd, kd, vd)
        ref.append(o.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    wss = [vc.alloc_workspace(p) for p, _ in cases]
    outs = [torch.empty_like(c[1][0]) for c in cases]
    torch.cuda.synchronize()
    G.log("[case] two streams: both cases enqueued on their own streams")
    for rep in range(3):
        for (p, (qd, kd, vd)), s, ws, o in zip(cases, streams, wss, outs):
            with torch.cuda.stream(s):
                o.zero_()
                vc.prepare(p, qd, kd, vd, ws)
                vc.forward(p, ws, o)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], ref[i]), f"stream case {i}, repetition {rep}"


def test_graph_replay_matches_eager():
    """Capture prepare + forward once; replay with new inputs copied into the
    captured buffers, eager library calls and synchronisations in between; every
    replay must equal the eager result for the same inputs."""
    import torch
    p, (qd, kd, vd) = _case(21, vc.DEFAULT_FLAGS | vc.FP8_SCORES)  # the benchmark's kernel
    ws = vc.alloc_workspace(p)
    o = torch.empty_like(qd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on the capture's stream
        vc.prepare(p, qd, kd, vd, ws)
        vc.forward(p, ws, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    G.log("[case] graph: capture prepare + forward")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vc.prepare(p, qd, kd, vd, ws)
        vc.forward(p, ws, o)
    torch.cuda.synchronize()
    ws_e = vc.alloc_workspace(p)
    for rep, seed in enumerate((21, 22, 23, 22)):
        q, k, v = inputs.make_custom(1, 3, 1000, seed=seed)
        new = G.to_device(q, k, v)
        for dst, src in zip((qd, kd, vd), new):
            dst.copy_(src)
        torch.cuda.synchronize()
        G.log(f"[case] graph: replay {rep} (inputs seed {seed})")
        g.replay()
        torch.cuda.synchronize()
        o_eager = torch.empty_like(o)
        vc.prepare(p, *new, ws_e)
        vc.forward(p, ws_e, o_eager)
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), f"replay {rep} differs from eager"
        ho, he = o.float().cpu().numpy(), o_eager.float().cpu().numpy()
        assert np.all(np.isfinite(ho)) and np.array_equal(ho, he)
