"""Sequence driver around the library: warm-up, per-step scheme schedule, and
the ablation modes.

"Accelerating Parallel Diffusion Model Serving with Residual Compression"
(CompactFusion notes):
  * Limitations: step 0 has no history and is sent in full; the first few steps,
    where the noise level changes fastest, carry the largest residuals, so a
    schedule may send them in full or with a finer scheme before switching to
    the cheap one (`Schedule`).
  * Overall framework / Error feedback: the normative loop is `closed`
    (r = a_t - ahat_{t-1}, e kept by the sender); the ablations of the notes are
    `noef` (residual against the previous activation, the dropped part
    discarded) and `direct` (the activation itself compressed, no residual).

Every mode runs through the C ABI unchanged: the mode only decides what the
sender's state buffer holds before the call (ahat, the previous activation, or
zeros). This module holds host logic and device buffer copies only; all
arithmetic of the method runs in librescomp's kernels.
"""
from __future__ import annotations

import bisect

from activation_residual_compression_amd import librescomp as rc

MODES = ("closed", "noef", "direct")


class Schedule:
    """Which scheme each step uses.

    full_steps: steps 0 .. full_steps-1 are sent in full (at least step 0).
    phases: [(first_step, scheme_name), ...] sorted by first_step; step t >=
    full_steps uses the last phase whose first_step <= t.
    """

    def __init__(self, phases, full_steps=1):
        if full_steps < 1:
            raise ValueError("step 0 is always sent in full")
        self.full_steps = int(full_steps)
        self.phases = sorted((int(s), str(n)) for s, n in phases)
        if not self.phases or self.phases[0][0] > self.full_steps:
            raise ValueError("no scheme for step %d" % self.full_steps)
        self._starts = [s for s, _ in self.phases]

    def at(self, t):
        """'full' or the scheme name for step t."""
        if t < self.full_steps:
            return "full"
        return self.phases[bisect.bisect_right(self._starts, t) - 1][1]


class Session:
    """One sender and one receiver for a batch of tensors [batch, rows, cols].

    schemes: {name: (scheme, params)} with params as for librescomp.Plan (a
    low-rank entry needs q0). Buffers live on `device`; step() takes a_t as a
    device tensor of the plan dtype (torch.bfloat16 / torch.float32).
    """

    def __init__(self, shape, dtype, schemes, schedule, mode="closed", device="cuda:0"):
        import torch
        if mode not in MODES:
            raise ValueError("mode must be one of %s" % (MODES,))
        self.shape, self.dtype, self.mode, self.schedule = tuple(shape), dtype, mode, schedule
        self.plans = {name: rc.Plan(self.shape, dtype, sch, **dict(params))
                      for name, (sch, params) in schemes.items()}
        for _, name in schedule.phases:
            if name not in self.plans:
                raise ValueError("schedule names unknown scheme %r" % name)
        dev = torch.device(device)
        self.ahat = torch.zeros(self.shape, dtype=torch.float32, device=dev)   # sender state
        self.e = torch.zeros_like(self.ahat)
        self.recon = torch.zeros_like(self.ahat)                                # receiver state
        self.sref = torch.zeros_like(self.ahat)   # noef / direct: what the sender compresses against
        self.packed = torch.empty(max(p.packed_bytes for p in self.plans.values()),
                                  dtype=torch.uint8, device=dev)
        self.t = -1
        self.sent_bytes = 0

    def step(self, a_t, stream=None):
        """Advance one step; returns dict(t, kind, bytes).

        Everything the step does -- the library calls and the copies and clears
        of the state buffers around them -- is enqueued on `stream` (a
        torch.cuda.Stream or a raw hipStream_t; None: torch's current stream),
        in that order, so no update can overtake a kernel that reads the same
        buffer. a_t must be ready on that stream."""
        import torch
        if stream is None:
            s = torch.cuda.current_stream()
        elif isinstance(stream, int):
            s = torch.cuda.ExternalStream(stream)
        else:
            s = stream
        with torch.cuda.stream(s):
            return self._step(a_t, s)

    def _step(self, a_t, stream):
        self.t += 1
        kind = self.schedule.at(self.t)
        if kind == "full":
            self.ahat.copy_(a_t)
            self.recon.copy_(a_t)
            self.e.zero_()
            self.sref.copy_(a_t)
            nbytes = a_t.numel() * a_t.element_size()
            for p in self.plans.values():
                p.reset_state(stream)
        else:
            plan = self.plans[kind]
            if self.mode == "closed":
                plan.compress(a_t, self.ahat, self.e, self.packed, stream)
                plan.decompress(self.packed, self.recon, stream)
            elif self.mode == "noef":
                # r = a_t - a_{t-1}; the sender's copy is overwritten next step
                plan.compress(a_t, self.sref, self.e, self.packed, stream)
                plan.decompress(self.packed, self.recon, stream)
                self.sref.copy_(a_t)
            else:  # direct: C(a_t) replaces the receiver's copy
                self.sref.zero_()
                plan.compress(a_t, self.sref, self.e, self.packed, stream)
                self.recon.zero_()
                plan.decompress(self.packed, self.recon, stream)
            nbytes = plan.packed_bytes
        self.sent_bytes += nbytes
        return dict(t=self.t, kind=kind, bytes=nbytes)

    def close(self):
        for p in self.plans.values():
            p.close()
        self.plans = {}

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
