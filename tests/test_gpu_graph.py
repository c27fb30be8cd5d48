"""A whole step (rc_compress + rc_decompress) captured in a HIP graph.

The library launches kernels only (no allocation, no host synchronisation, no
memset nodes inside a call), so a serving loop can capture a step once and
replay it. Each replay here follows eager work (a new input copied into the
graph's static buffer) and must give exactly the state that the same calls made
eagerly give, for every scheme, over several replays in a row.
"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, bits, say, synth, to_device
from activation_residual_compression_amd import librescomp as rc

pytestmark = pytest.mark.gpu


def _setup(scheme):
    if scheme == "bs":
        wl = synth.LatentWorkload(batch=2, height=16, width=32, m=64, steps=6)
        return wl, dict(grid_w=32, keep_blocks=3)
    wl = synth.FluxWorkload(batch=2, n=100, m=256, steps=6)
    kw = {"q1": dict(group=64), "q2": dict(group=128), "nm": dict(nm_keep=2, nm_block=16),
          "lr": dict(rank=16, iters=2, q0=wl.q0(16))}[scheme]
    return wl, kw


@pytest.mark.parametrize("scheme", ["q1", "q2", "nm", "lr", "bs"])
def test_graph_replays_equal_eager(scheme):
    wl, kw = _setup(scheme)
    frames = [wl.next()[1] for _ in range(wl.steps)]
    shape = (wl.nb, wl.n, wl.m)
    say("[gpu] graph %s" % scheme)
    with rc.Plan(shape, "bf16", scheme, **kw) as pg, rc.Plan(shape, "bf16", scheme, **kw) as pe:
        a_static = to_device(frames[0], "bf16")
        start = a_static.float()
        g_ahat, g_e, g_rec = start.clone(), torch.zeros_like(start), start.clone()
        e_ahat, e_e, e_rec = start.clone(), torch.zeros_like(start), start.clone()
        g_pk = torch.zeros(pg.packed_bytes, dtype=torch.uint8, device=DEV)
        e_pk = torch.zeros_like(g_pk)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                pg.compress(a_static, g_ahat, g_e, g_pk)
                pg.decompress(g_pk, g_rec)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        # capture ran nothing: the state is still the start state
        assert np.array_equal(bits(g_ahat.cpu().numpy()), bits(start.cpu().numpy()))
        for t in range(1, wl.steps):
            a_t = to_device(frames[t], "bf16")
            a_static.copy_(a_t)
            graph.replay()
            pe.compress(a_t, e_ahat, e_e, e_pk)
            pe.decompress(e_pk, e_rec)
            torch.cuda.synchronize()
            for x, y in ((g_pk, e_pk), (g_ahat, e_ahat), (g_e, e_e), (g_rec, e_rec)):
                assert np.array_equal(bits(x.cpu().numpy()), bits(y.cpu().numpy())), t
