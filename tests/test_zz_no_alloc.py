"""rc_compress_lowrank_noalloc (the low-rank sender step without a plan and
without allocation, its workspace in a fixed device array) against
rc_compress on a plan with the same parameters: packed bytes, e and ahat equal
bit for bit, on two calls in a row, the second with a smaller input, with
start matrices given on the device and drawn from a seed; shapes whose
workspace exceeds the fixed array are rejected before anything runs."""
import numpy as np
import pytest
import torch

from gpu_harness import DEV, bits, say, synth, to_device
from activation_residual_compression_amd import librescomp as rc

pytestmark = pytest.mark.gpu


def _case(B, n, m, rank, seed_only):
    wl = synth.FluxWorkload(batch=B, n=n, m=m, steps=2)
    _, a0 = wl.next()
    _, a1 = wl.next()
    q0 = None if seed_only else torch.from_numpy(wl.q0(rank)).to(DEV)
    return wl, a0, a1, q0


@pytest.mark.parametrize("seed_only", [False, True])
@pytest.mark.parametrize("factors", ["int4", "bf16"])
def test_noalloc_equals_plan_on_two_calls(seed_only, factors):
    flags = rc.RC_LR_BF16_FACTORS if factors == "bf16" else 0
    for (B, n, m, rank) in ((3, 200, 320, 32), (2, 100, 192, 16)):   # the second call is smaller
        wl, a0, a1, q0 = _case(B, n, m, rank, seed_only)
        say("[gpu] noalloc %s %s shape %s rank %d" % (factors, "seed" if seed_only else "q0", (B, n, m), rank))
        kw = dict(rank=rank, iters=2, flags=flags, seed=wl.seed)
        if q0 is not None:
            kw["q0"] = q0
        a = to_device(a1, "bf16")
        outs = []
        with rc.Plan((B, n, m), "bf16", "lr", **kw) as plan:
            for use_plan in (True, False):
                ahat = to_device(a0, "bf16").float()
                e = torch.full_like(ahat, 7.0)
                pk = torch.full((plan.packed_bytes,), 0xA5, dtype=torch.uint8, device=DEV)
                if use_plan:
                    plan.compress(a, ahat, e, pk)
                else:
                    params = rc.make_params("lr", **kw)
                    st = rc.rc_state_t(ahat.data_ptr(), e.data_ptr())
                    rc.rc_compress_lowrank_noalloc((B, n, m), "bf16", params, None, a, st, pk)
                torch.cuda.synchronize()
                outs.append((pk.cpu().numpy(), bits(ahat.cpu().numpy()), bits(e.cpu().numpy())))
        for x, y in zip(*outs):
            assert np.array_equal(x, y)


def test_noalloc_rejects_oversized_and_bad_arguments():
    # the full flux batch needs about 0.5 GB of workspace: more than the fixed array
    params = rc.make_params("lr", rank=32, iters=2, seed=1)
    st = rc.rc_state_t(4096, 4096)
    with pytest.raises(rc.RcError) as ei:
        rc.rc_compress_lowrank_noalloc((57, 1152, 3072), "bf16", params, None, 4096, st, 4096)
    assert ei.value.status == rc.RC_ERR_UNSUPPORTED
    for bad, status in ((dict(rank=24), rc.RC_ERR_UNSUPPORTED),
                        (dict(flags=rc.RC_LR_CHECK_NUMERIC), rc.RC_ERR_INVALID_ARG),
                        (dict(flags=rc.RC_LR_ONE_STREAM), rc.RC_ERR_INVALID_ARG)):
        kw = dict(rank=16, iters=2, seed=1)
        kw.update(bad)
        with pytest.raises(rc.RcError) as ei:
            rc.rc_compress_lowrank_noalloc((2, 100, 192), "bf16", rc.make_params("lr", **kw), None,
                                           4096, st, 4096)
        assert ei.value.status == status
    with pytest.raises(rc.RcError) as ei:   # misaligned a_t
        rc.rc_compress_lowrank_noalloc((2, 100, 192), "bf16", rc.make_params("lr", rank=16, iters=2),
                                       None, 4100, st, 4096)
    assert ei.value.status == rc.RC_ERR_ALIGNMENT
