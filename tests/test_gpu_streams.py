"""Independent plans on independent streams.

A plan owns its workspace and round state, and every entry point only enqueues
kernels on the caller's stream, so plans driven from different streams at the
same time must give exactly what they give one after the other: here a 2-bit, a
low-rank and a block-selection plan, three steps each, interleaved over three
streams, against the same calls made in sequence on one stream.
"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, bits, say, synth, to_device
from activation_residual_compression_amd import librescomp as rc

pytestmark = pytest.mark.gpu

STEPS = 3


def _cases():
    fl = synth.FluxWorkload(batch=3, n=160, m=512, steps=STEPS + 1)
    lr = synth.FluxWorkload(batch=2, n=200, m=320, steps=STEPS + 1)
    bs = synth.LatentWorkload(batch=2, height=32, width=64, m=64, steps=STEPS + 1)
    return [("q2", fl, dict(group=128)),
            ("lr", lr, dict(rank=32, iters=2, q0=lr.q0(32))),
            ("bs", bs, dict(grid_w=64, keep_blocks=5))]


def _frames(wl):
    return [to_device(wl.next()[1], wl.dtype) for _ in range(STEPS + 1)]


def _run(cases, frames, streams):
    """Run every case for STEPS steps; streams[i] is case i's stream (one stream
    for all = in sequence). Returns per case the packed bytes and states."""
    plans, states = [], []
    for (scheme, wl, kw), fr in zip(cases, frames):
        plans.append(rc.Plan((wl.nb, wl.n, wl.m), wl.dtype, scheme, **kw))
        start = fr[0].float()
        states.append(dict(ahat=start.clone(), e=torch.zeros_like(start), recon=start.clone(),
                           packed=torch.zeros(plans[-1].packed_bytes, dtype=torch.uint8, device=DEV)))
    torch.cuda.synchronize()
    for t in range(1, STEPS + 1):
        for i, (plan, st) in enumerate(zip(plans, states)):
            s = streams[i]
            plan.compress(frames[i][t], st["ahat"], st["e"], st["packed"], s)
            plan.decompress(st["packed"], st["recon"], s)
    torch.cuda.synchronize()
    out = [{k: v.cpu().numpy() for k, v in st.items()} for st in states]
    for p in plans:
        p.close()
    return out


def test_plans_on_separate_streams_match_sequential_run():
    cases = _cases()
    frames = [_frames(wl) for _, wl, _ in cases]
    say("[gpu] streams: sequential")
    one = torch.cuda.Stream()
    seq = _run(cases, frames, [one] * len(cases))
    say("[gpu] streams: concurrent")
    streams = [torch.cuda.Stream() for _ in cases]
    par = _run(cases, frames, streams)
    for (scheme, _, _), a, b in zip(cases, seq, par):
        for key in ("packed", "ahat", "e", "recon"):
            assert np.array_equal(bits(a[key]) if key != "packed" else a[key],
                                  bits(b[key]) if key != "packed" else b[key]), (scheme, key)
        assert np.array_equal(bits(a["recon"]), bits(a["ahat"])), scheme


def test_lowrank_two_stream_compress_matches_one_stream():
    # batch >= 2: by default half of the batch runs on the plan's own stream;
    # RC_LR_ONE_STREAM keeps it on the caller's. Both must give the same bits,
    # and an odd batch splits unevenly (3 + 2 tensors).
    wl = synth.FluxWorkload(batch=5, n=200, m=320, steps=STEPS + 1)
    fr = _frames(wl)
    q0 = wl.q0(32)
    out = []
    for flags in (0, rc.RC_LR_ONE_STREAM):
        say("[gpu] streams: low rank flags %d" % flags)
        s = torch.cuda.Stream()
        with rc.Plan((wl.nb, wl.n, wl.m), wl.dtype, "lr", rank=32, iters=2, q0=q0, flags=flags) as p:
            ahat = fr[0].float().clone()
            e = torch.zeros_like(ahat)
            recon = ahat.clone()
            packed = torch.zeros(p.packed_bytes, dtype=torch.uint8, device=DEV)
            steps = []
            for t in range(1, STEPS + 1):
                p.compress(fr[t], ahat, e, packed, s)
                p.decompress(packed, recon, s)
                s.synchronize()
                steps.append((packed.cpu().numpy(), bits(ahat.cpu().numpy()), bits(e.cpu().numpy()),
                              bits(recon.cpu().numpy())))
            out.append(steps)
    for t, (a, b) in enumerate(zip(*out)):
        for i, key in enumerate(("packed", "ahat", "e", "recon")):
            assert np.array_equal(a[i], b[i]), (t, key)
        assert np.array_equal(a[1], a[3]), t
