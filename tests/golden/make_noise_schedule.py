"""Writes noise_schedule_eps.json: the relative error of the receiver copy,
eps_t = |a_t - ahat_t|_F / |a_t|_F, over a sequence whose early steps change
sharply, for four per-step schedules.

Calls only the CPU oracle and the seeded input generator. Page: "Accelerating
Parallel Diffusion Model Serving with Residual Compression" (CompactFusion
notes), Limitations: extreme low rank may fail at the steps where the noise
level changes sharply, such as the first few, and those steps can be sent in
full or with a finer scheme first. Input: NoiseScheduleWorkload, tensor 0 of
the FLUX-like share (1152 x 3072 bf16), 12 steps. Schedules (closed loop,
rank-r low rank with 2 subspace iterations and INT4 factors, seeded start
matrices):
  full1     -- step 0 in full, rank 32 from step 1;
  full3     -- steps 0-2 in full, rank 32 from step 3;
  rank64x3  -- step 0 in full, rank 64 for steps 1-3, rank 32 from step 4;
  q1x3      -- step 0 in full, 1-bit (group 64) for steps 1-3, rank 32 from step 4.
Also records the bytes each step sends (packed tensor sizes of the layouts)
and, per schedule, how far a second run parts from the first when the state
after the first compressed step is moved by one fp32 ulp per element in a
random direction (the size of the difference between fp32 and fp64 factor
arithmetic): max over steps of |eps' - eps| / eps.
Run: python tests/golden/make_noise_schedule.py  (about 4 minutes, one core)
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from activation_residual_compression_amd import synth  # noqa: E402

N, M, STEPS = 1152, 3072, 12
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "noise_schedule_eps.json")


def schedules(q0):
    lr = lambda r: ("lr", dict(rank=r, iters=2, q0=q0[r]))  # noqa: E731
    q1 = ("q1", dict(group=64))
    return {
        "full1": [None] + [lr(32)] * (STEPS - 1),
        "full3": [None] * 3 + [lr(32)] * (STEPS - 3),
        "rank64x3": [None] + [lr(64)] * 3 + [lr(32)] * (STEPS - 4),
        "q1x3": [None] + [q1] * 3 + [lr(32)] * (STEPS - 4),
    }


def step_bytes(kind):
    if kind is None:
        return N * M * 2
    scheme, p = kind
    if scheme == "lr":
        return oracle.tensor_bytes("lr", N, M, rank=p["rank"])
    return oracle.tensor_bytes(scheme, N, M, group=p["group"])


def eps(a, ahat):
    a = a.astype(np.float64)
    return float(np.linalg.norm(a - ahat.astype(np.float64)) / np.linalg.norm(a))


def main():
    wl = synth.NoiseScheduleWorkload(batch=1, n=N, m=M, steps=STEPS)
    frames = [synth.bf16_bits_to_f32(wl.next()[1])[0].copy() for _ in range(STEPS)]
    q0 = {r: wl.q0(r)[0] for r in (32, 64)}
    result = dict(workload="NoiseScheduleWorkload tensor 0", shape=[N, M], steps=STEPS,
                  white=[wl.white(t) for t in range(1, STEPS)], schedules={})
    rng = np.random.default_rng(2)
    for name, kinds in schedules(q0).items():
        out = oracle.run_schedule(frames, kinds)
        e = [eps(frames[t], out[t]) for t in range(STEPS)]
        # perturbed run: continue from the first compressed step's state moved by one ulp
        t1 = next(t for t, k in enumerate(kinds) if k is not None)
        ahat = out[t1].copy()
        ahat = np.nextafter(ahat, np.where(rng.random(ahat.shape) < 0.5, -np.inf, np.inf).astype(np.float32))
        assert np.all(ahat != out[t1]) and ahat.dtype == np.float32
        ep = e[:t1 + 1]
        for t in range(t1 + 1, STEPS):
            ahat = oracle.run_schedule([ahat, frames[t]], [None, kinds[t]])[1]
            ep.append(eps(frames[t], ahat))
        gap = max(abs(x - y) / y for x, y in zip(ep[t1 + 1:], e[t1 + 1:]))
        result["schedules"][name] = dict(eps=e, bytes=[step_bytes(k) for k in kinds],
                                         perturbed_eps=ep, max_rel_gap=gap)
        print(name, " ".join("%.4f" % x for x in e), "gap %.2e" % gap, flush=True)
    with open(OUT, "w") as f:
        json.dump(result, f, indent=1)


if __name__ == "__main__":
    main()
