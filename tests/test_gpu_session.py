"""GPU runs of whole sequences through the session driver.

CompactFusion notes, Overall framework and Error feedback: the closed loop, and
the two ablations (noef: residual against the previous activation with the
dropped part discarded; direct: the activation itself compressed). For the
bit-exact schemes every free-running GPU trajectory equals the oracle's
free-running trajectory (oracle.run_trajectory) bit for bit (direct: value for
value, since the receiver adds C(a_t) to a zeroed state). The pages' claims are
then checked on the GPU trajectories: with feedback the error stays bounded,
without it it grows, direct compression is far worse. A schedule that switches
scheme mid-sequence keeps sender and receiver identical.
"""
import numpy as np
import pytest
import torch

from gpu_harness import bits, lib_view_f32, oracle, relF, say, synth, to_device
from activation_residual_compression_amd.session import Schedule, Session

pytestmark = pytest.mark.gpu


def _frames(wl):
    out = []
    for _ in range(wl.steps):
        out.append(wl.next()[1])
    return out


@pytest.mark.parametrize("scheme,params", [("q1", dict(group=64)), ("q2", dict(group=128)),
                                           ("nm", dict(nm_keep=2, nm_block=16))])
@pytest.mark.parametrize("mode", ["closed", "noef", "direct"])
def test_modes_match_oracle_trajectory(scheme, params, mode):
    wl = synth.FluxWorkload(batch=2, n=48, m=256, steps=8)
    frames = _frames(wl)
    okw = {} if scheme == "nm" else dict(group=params["group"])
    with Session((2, 48, 256), "bf16", {scheme: (scheme, params)}, Schedule([(1, scheme)]),
                 mode=mode) as s:
        gpu = []
        for a in frames:
            s.step(to_device(a, "bf16"))
            torch.cuda.synchronize()
            gpu.append(s.recon.cpu().numpy())
        if mode == "closed":
            assert np.array_equal(bits(s.recon.cpu().numpy()), bits(s.ahat.cpu().numpy()))
    for b in range(2):
        ref = oracle.run_trajectory(mode, scheme, [lib_view_f32(f[b], "bf16") for f in frames], **okw)
        for t, (g, o) in enumerate(zip(gpu, ref)):
            if mode == "direct":
                assert np.array_equal(g[b], o), (t, b)
            else:
                assert np.array_equal(bits(g[b]), bits(o)), (t, b)
    say("[gpu] %s %s trajectory equals the oracle's" % (scheme, mode))


def test_feedback_bounded_noef_grows_direct_worse():
    # random walk with per-channel scales (fp32), 1-bit residuals, 28 steps
    wl = synth.WalkWorkload(batch=1, n=64, m=512, steps=28)
    frames = _frames(wl)
    err = {}
    for mode in ("closed", "noef", "direct"):
        with Session((1, 64, 512), "f32", {"q1": ("q1", dict(group=64))}, Schedule([(1, "q1")]),
                     mode=mode) as s:
            e = []
            for a in frames:
                s.step(to_device(a, "f32"))
                torch.cuda.synchronize()
                e.append(relF(a[0], s.recon.cpu().numpy()[0]))
            err[mode] = np.array(e[1:])
    say("[gpu] final relative error closed %.4f noef %.4f direct %.4f" %
        (err["closed"][-1], err["noef"][-1], err["direct"][-1]))
    tail = err["closed"][len(err["closed"]) // 2:]
    assert tail.max() <= 1.5 * tail.min()                      # bounded: flat second half
    sq = err["noef"] ** 2                                        # open loop: error energy grows
    t = np.arange(1, sq.size + 1)
    r2 = np.corrcoef(t, sq)[0, 1] ** 2
    assert sq[-1] > 4 * sq[2] and r2 > 0.9
    assert err["direct"].min() > 4 * err["closed"].max()


def test_schedule_switch_keeps_receiver_equal():
    wl = synth.FluxWorkload(batch=2, n=100, m=192, steps=8)
    frames = _frames(wl)
    schemes = {"lr": ("lr", dict(rank=16, iters=2, q0=wl.q0(16))), "q1": ("q1", dict(group=64)),
               "nm": ("nm", dict(nm_keep=2, nm_block=16))}
    sched = Schedule([(2, "lr"), (4, "q1"), (6, "nm")], full_steps=2)
    with Session((2, 100, 192), "bf16", schemes, sched) as s:
        prev = None
        for t, a in enumerate(frames):
            info = s.step(to_device(a, "bf16"))
            torch.cuda.synchronize()
            ah, rh = s.ahat.cpu().numpy(), s.recon.cpu().numpy()
            assert info["kind"] == sched.at(t)
            assert np.array_equal(bits(ah), bits(rh)), t
            af = lib_view_f32(a, "bf16")
            if info["kind"] == "full":
                assert np.array_equal(ah, af)
            elif info["kind"] in ("q1", "nm"):
                for b in range(2):
                    o = oracle.compress_tensor(info["kind"], af[b], prev[b],
                                               **({"group": 64} if info["kind"] == "q1" else {}))
                    assert np.array_equal(bits(ah[b]), bits(o["ahat"])), (t, b)
            prev = ah


@pytest.mark.parametrize("mode", ["noef", "direct"])
def test_lowrank_ablation_modes_match_oracle_trajectory(mode):
    """Low rank in the two ablation modes against oracle.run_trajectory. The
    compression input of both modes does not depend on the state (noef: the
    step change a_t - a_{t-1}; direct: a_t), so the GPU and the oracle compress
    the same residuals every step and the relative errors of the receiver
    state agree within the per-step 1e-3."""
    wl = synth.FluxWorkload(batch=2, n=96, m=256, steps=6)
    frames = _frames(wl)
    q0 = wl.q0(16)
    schemes = {"lr": ("lr", dict(rank=16, iters=2, q0=q0))}
    with Session((2, 96, 256), "bf16", schemes, Schedule([(1, "lr")]), mode=mode) as s:
        gpu = []
        for a in frames:
            s.step(to_device(a, "bf16"))
            torch.cuda.synchronize()
            gpu.append(s.recon.cpu().numpy())
    for b in range(2):
        fr = [lib_view_f32(f[b], "bf16") for f in frames]
        ref = oracle.run_trajectory(mode, "lr", fr, rank=16, iters=2, q0=q0[b])
        for t in range(1, len(frames)):
            eg, eo = relF(fr[t], gpu[t][b]), relF(fr[t], ref[t])
            say("[gpu] lr %s t=%d b=%d eps gpu %.5f oracle %.5f" % (mode, t, b, eg, eo))
            assert abs(eg - eo) <= 1e-3, (t, b, eg, eo)


@pytest.mark.parametrize("scheme,params", [("q2", dict(group=128)), ("bs", dict(grid_w=32, keep_blocks=4))])
@pytest.mark.parametrize("mode", ["closed", "noef", "direct"])
def test_session_on_a_side_stream_equals_current_stream(scheme, params, mode):
    """Session.step(stream=s) with s not the current stream: the state updates
    around the library calls run on s too, so the results equal those of the
    same steps on the current stream bit for bit."""
    if scheme == "bs":
        wl = synth.LatentWorkload(batch=2, height=16, width=32, m=64, steps=6)
    else:
        wl = synth.FluxWorkload(batch=2, n=48, m=256, steps=6)
    frames = _frames(wl)
    sched = Schedule([(1, scheme)], full_steps=1)
    out = []
    for use_side in (False, True):
        side = torch.cuda.Stream() if use_side else None
        with Session((2, wl.n, wl.m), "bf16", {scheme: (scheme, params)}, sched, mode=mode) as s:
            inputs = []   # kept alive until the side stream has read them
            for a in frames:
                inputs.append(to_device(a, "bf16"))
                if side is not None:
                    side.wait_stream(torch.cuda.current_stream())
                s.step(inputs[-1], stream=side)
            torch.cuda.synchronize()
            out.append((s.recon.cpu().numpy(), s.ahat.cpu().numpy(), s.e.cpu().numpy()))
    for x, y in zip(out[0], out[1]):
        assert np.array_equal(bits(x), bits(y))
    say("[gpu] session %s %s on a side stream: identical" % (scheme, mode))
