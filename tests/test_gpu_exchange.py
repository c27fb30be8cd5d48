"""GPU checks of the exchange-side entry points.

rc_compress_send compresses the batch in chunks and queues a copy of each
chunk's packed bytes on a second stream while the next chunk is compressed
(CompactFusion notes, Key designs / System co-design: compression overlapped
with communication). Its packed stream, the copy at the destination (device
buffer or pinned host memory) and the sender state must equal those of one
rc_compress call bit for bit, whatever the chunk size.

rc_decompress_many decodes several peers' packed streams into their receiver
states (Overall framework: each GPU rebuilds every peer's activation); it must
equal one rc_decompress per peer bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, lib_view_f32, say, to_device
from activation_residual_compression_amd import librescomp as rc
from activation_residual_compression_amd import synth

pytestmark = pytest.mark.gpu

SCHEMES = [("q2", "bf16", dict(group=128)), ("q1", "f32", dict(group=64)),
           ("nm", "bf16", dict(nm_keep=2, nm_block=16)), ("lr", "bf16", dict(rank=16, iters=2))]


def _inputs(scheme, dtype, kw, B, n, m, seed_tensors=None):
    wl = synth.FluxWorkload(batch=B, n=n, m=m, steps=2)
    _, a0 = wl.next()
    _, a1 = wl.next()
    params = dict(kw)
    if scheme == "lr":
        params["q0"] = wl.q0(kw["rank"])
    if dtype == "f32":
        a0, a1 = lib_view_f32(a0, "bf16"), lib_view_f32(a1, "bf16")
    return params, a0, a1


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("scheme,dtype,kw", SCHEMES)
@pytest.mark.parametrize("chunk", [1, 2, 5, 7])
@pytest.mark.parametrize("dest", ["device", "host"])
def test_compress_send_equals_compress(scheme, dtype, kw, chunk, dest):
    B, n, m = 5, 72, 256
    params, a0, a1 = _inputs(scheme, dtype, kw, B, n, m)
    say("[gpu] compress_send %s %s chunk %d -> %s" % (scheme, dtype, chunk, dest))
    with rc.Plan((B, n, m), dtype, scheme, **params) as plan:
        a = to_device(a1, dtype)
        start = to_device(a0, dtype).float()
        ahat_ref, e_ref = start.clone(), torch.zeros_like(start)
        ahat_s, e_s = start.clone(), torch.zeros_like(start)
        packed_ref = torch.full((plan.packed_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
        packed_out = torch.full((plan.packed_bytes,), 0x5A, dtype=torch.uint8, device=DEV)
        if dest == "device":
            packed_dst = torch.full((plan.packed_bytes,), 0x3C, dtype=torch.uint8, device=DEV)
        else:
            packed_dst = torch.full((plan.packed_bytes,), 0x3C, dtype=torch.uint8, pin_memory=True)
        plan.compress(a, ahat_ref, e_ref, packed_ref)
        torch.cuda.synchronize()
        copy_stream = torch.cuda.Stream()
        plan.compress_send(a, ahat_s, e_s, packed_out, packed_dst, chunk, copy_stream)
        copy_stream.synchronize()
        torch.cuda.synchronize()
        ref = _bits(packed_ref)
        assert np.array_equal(_bits(packed_out), ref)
        assert np.array_equal(packed_dst.cpu().numpy(), ref)
        assert np.array_equal(_bits(ahat_s), _bits(ahat_ref))
        assert np.array_equal(_bits(e_s), _bits(e_ref))


@pytest.mark.parametrize("scheme,dtype,kw", SCHEMES)
@pytest.mark.parametrize("npeers", [1, 3, 8])
def test_decompress_many_equals_one_call_per_peer(scheme, dtype, kw, npeers):
    B, n, m = 3, 40, 256
    params, a0, a1 = _inputs(scheme, dtype, kw, B * npeers, n, m)
    say("[gpu] decompress_many %s %s peers %d" % (scheme, dtype, npeers))
    if scheme == "lr":
        params["q0"] = params["q0"][:B]
    with rc.Plan((B, n, m), dtype, scheme, **params) as plan:
        packed, states = [], []
        for p in range(npeers):
            sl = slice(p * B, (p + 1) * B)
            a = to_device(a1[sl], dtype)
            ahat = to_device(a0[sl], dtype).float()
            e = torch.zeros_like(ahat)
            pk = torch.empty(plan.packed_bytes, dtype=torch.uint8, device=DEV)
            plan.compress(a, ahat, e, pk)
            packed.append(pk)
            # each receiver starts from its own state (here: the peer's step-0 activation)
            states.append(to_device(a0[sl], dtype).float())
        seq = [s.clone() for s in states]
        many = [s.clone() for s in states]
        for p in range(npeers):
            plan.decompress(packed[p], seq[p])
        plan.decompress_many(packed, many)
        torch.cuda.synchronize()
        for p in range(npeers):
            assert np.array_equal(_bits(many[p]), _bits(seq[p])), p
            assert not np.array_equal(_bits(many[p]), _bits(states[p])), p  # something was applied
