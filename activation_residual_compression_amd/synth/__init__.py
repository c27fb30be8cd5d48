"""Seeded synthetic activation sequences (inputs only; no compression arithmetic).

Both the GPU library's tests/benchmarks and the CPU oracle consume the arrays made
here, so the two sides always see identical inputs. Every array comes from one
counter-based generator (SplitMix64 -> uniform -> Box-Muller, see ``gen.c``), so
a tensor of a batch can be generated alone and equals the same tensor of the full
batch.

Workloads (shapes and statistics follow the experimental setting of the page
"Accelerating Parallel Diffusion Model Serving with Residual Compression":
FLUX.1-dev sequence-parallel shares on 4 GPUs and CogVideoX-2b; the models,
prompts and datasets are not used, the activations are synthetic stand-ins):

* ``tiny``  : 1 fp32 matrix 256x64, 10 steps, random walk with step 0.1*s_c,
  s_c ~ LogNormal(0, 0.5).
* ``flux``  : 57 bf16 tensors [1152 tokens x 3072 hidden], 28 steps;
  s_c ~ LogNormal(0,1) with 1% outlier channels x20; step change of std 0.1*s_c
  split equally between white noise and a persistent rank-8 drift.
* ``flux_sched``: the flux shape whose white step change follows a noise
  schedule, 20x larger at step 1 and decaying with time constant 1.5 steps
  (NoiseScheduleWorkload).
* ``video`` : 30 bf16 tensors [4444 tokens x 1920 hidden], 50 steps; share 0 of a
  226-text + 13x30x45-patch token sequence split 4 ways; AR(1) with rho = 0.98
  and Gaussian-blurred (sigma = 2 tokens) spatial noise.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")

SEED_BASE = 0x5EED0000


def build(force: bool = True) -> str:
    """Compile the generator library in place (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _VideoGeom(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int), ("frames", ctypes.c_int), ("height", ctypes.c_int),
                ("width", ctypes.c_int), ("share", ctypes.c_int), ("n", ctypes.c_int),
                ("blur_sigma", ctypes.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                                  ctypes.c_void_p)
        lib.sg_key.restype = u64
        lib.sg_key.argtypes = [u64, u64, u64, u64]
        lib.sg_u64.restype = u64
        lib.sg_u64.argtypes = [u64, u64]
        lib.sg_uniform.argtypes = [u64, u64, i64, vp]
        lib.sg_normal.argtypes = [u64, u64, i64, vp]
        lib.sg_normal_f32.argtypes = [u64, u64, i64, vp]
        lib.sg_to_bf16.argtypes = [i64, vp, vp]
        lib.sg_walk_init.argtypes = [u64, i32, i32, i32, dbl, vp, vp]
        lib.sg_walk_step.argtypes = [u64, i32, i32, i32, i32, dbl, vp, vp]
        lib.sg_flux_init.argtypes = [u64, i32, i32, i32, i32, dbl, i32, vp, vp, vp, vp]
        lib.sg_flux_step.argtypes = [u64, i32, i32, i32, i32, dbl, i32, vp, vp, vp, vp]
        lib.sg_flux_step_mix.argtypes = [u64, i32, i32, i32, i32, dbl, dbl, i32, vp, vp, vp, vp]
        lib.sg_video_init.argtypes = [u64, i32, ctypes.POINTER(_VideoGeom), i32, vp, vp]
        lib.sg_video_step.argtypes = [u64, i32, i32, ctypes.POINTER(_VideoGeom), i32, dbl, vp, vp, vp]
        lib.sg_q0.argtypes = [u64, i32, i32, i32, vp]
        lib.sg_latent_init.argtypes = [u64, i32, i32, i32, i32, vp, vp]
        lib.sg_latent_step.argtypes = [u64, i32, i32, i32, i32, i32, dbl, dbl, dbl, vp, vp, vp]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- primitives
def normal(key: int, first: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float64)
    _load().sg_normal(key, first, count, _p(out))
    return out


def uniform(key: int, first: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float64)
    _load().sg_uniform(key, first, count, _p(out))
    return out


def key(seed: int, role: int, tensor: int = 0, step: int = 0) -> int:
    return int(_load().sg_key(seed, role, tensor, step))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) as uint16 bit patterns."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().sg_to_bf16(x.size, _p(x), _p(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- workloads
@dataclass
class Workload:
    """A seeded sequence of activation batches a_0 .. a_{steps-1}.

    ``next()`` returns (t, a) where ``a`` is what the library sees for step t:
    float32 [nb, n, m] for dtype 'f32', uint16 bf16 bit patterns for 'bf16'.
    ``tensors`` selects a subset of the batch (default: all).
    """

    name: str
    batch: int
    n: int
    m: int
    steps: int
    dtype: str
    seed: int
    tensors: list = field(default=None)

    def __post_init__(self):
        if self.tensors is None:
            self.tensors = list(range(self.batch))
        self.tensors = [int(b) for b in self.tensors]
        for b in self.tensors:
            if not 0 <= b < self.batch:
                raise ValueError("tensor index %d outside batch %d" % (b, self.batch))
        self.reset()

    @property
    def nb(self) -> int:
        return len(self.tensors)

    def reset(self):
        self._t = -1
        self._state = None

    def _init(self):  # pragma: no cover - per workload
        raise NotImplementedError

    def _step(self, t):  # pragma: no cover - per workload
        raise NotImplementedError

    def next(self):
        self._t += 1
        if self._t >= self.steps:
            raise StopIteration
        if self._t == 0:
            self._init()
        else:
            self._step(self._t)
        af = self._state  # fp32 [nb, n, m]
        if self.dtype == "f32":
            return self._t, af.copy()
        return self._t, to_bf16_bits(af)

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        """Library-view activations as float32 values."""
        return a.astype(np.float32) if self.dtype == "f32" else bf16_bits_to_f32(a)

    def q0(self, rank: int) -> np.ndarray:
        """Seeded N(0,1) start matrices, float32 [nb, m, rank]."""
        return start_matrices(self.seed, self.tensors, self.m, rank)


def start_matrices(seed: int, tensors, m: int, rank: int) -> np.ndarray:
    """N(0,1) start matrices of the subspace iteration for the given seed,
    float32 [len(tensors), m, rank]: element (b, c, j) is the (c*rank + j)-th
    normal of stream key(seed, 7, b, 0) (Workload.q0 is this with the workload's
    seed)."""
    out = np.empty((len(tensors), m, rank), np.float32)
    for i, b in enumerate(tensors):
        _load().sg_q0(int(seed), int(b), m, rank, _p(out[i]))
    return out


class WalkWorkload(Workload):
    def __init__(self, name="tiny", batch=1, n=256, m=64, steps=10, seed=SEED_BASE + 0,
                 scale_sigma=0.5, step_sigma=0.1, tensors=None):
        self.scale_sigma, self.step_sigma = scale_sigma, step_sigma
        super().__init__(name, batch, n, m, steps, "f32", seed, tensors)

    def _init(self):
        lib = _load()
        self._sc = np.empty((self.nb, self.m), np.float32)
        self._state = np.empty((self.nb, self.n, self.m), np.float32)
        for i, b in enumerate(self.tensors):
            lib.sg_walk_init(self.seed, b, self.n, self.m, self.scale_sigma, _p(self._sc[i]),
                             _p(self._state[i]))

    def _step(self, t):
        lib = _load()
        for i, b in enumerate(self.tensors):
            lib.sg_walk_step(self.seed, b, t, self.n, self.m, self.step_sigma, _p(self._sc[i]),
                             _p(self._state[i]))


class FluxWorkload(Workload):
    def __init__(self, name="flux", batch=57, n=1152, m=3072, steps=28, seed=SEED_BASE + 1,
                 outlier_frac=0.01, outlier_mult=20.0, sigma=0.1, drift_rank=8, tensors=None):
        self.n_outlier = int(round(outlier_frac * m))
        self.outlier_mult, self.sigma, self.drift_rank = outlier_mult, sigma, drift_rank
        super().__init__(name, batch, n, m, steps, "bf16", seed, tensors)

    def _init(self):
        lib = _load()
        nb, n, m, r = self.nb, self.n, self.m, self.drift_rank
        self._sc = np.empty((nb, m), np.float32)
        self._A = np.empty((nb, n, r), np.float32)
        self._B = np.empty((nb, m, r), np.float32)
        self._state = np.empty((nb, n, m), np.float32)
        for i, b in enumerate(self.tensors):
            lib.sg_flux_init(self.seed, b, n, m, self.n_outlier, self.outlier_mult, r,
                             _p(self._sc[i]), _p(self._A[i]), _p(self._B[i]), _p(self._state[i]))

    def _step(self, t):
        lib = _load()
        for i, b in enumerate(self.tensors):
            lib.sg_flux_step(self.seed, b, t, self.n, self.m, self.sigma, self.drift_rank,
                             _p(self._sc[i]), _p(self._A[i]), _p(self._B[i]), _p(self._state[i]))


class NoiseScheduleWorkload(FluxWorkload):
    """The FLUX-like share whose step change follows a noise schedule.

    The page "Accelerating Parallel Diffusion Model Serving with Residual
    Compression" (CompactFusion notes, Limitations) names the steps where the
    noise level changes sharply, such as the first few, as those where extreme
    low-rank compression may fail. Here the white (full-rank) part of the step
    change has std
        white(t) = sigma / sqrt(2) * (1 + (early_ratio - 1) * exp(-(t - 1) / tau))
    times s_c, so step 1 moves the activation by about its own size (early_ratio
    20: 1.4 s_c) and the change decays to the FLUX-like white part within about
    six steps; the persistent rank-8 drift keeps std sigma / sqrt(2) throughout.
    Scales, outliers and a_0 are drawn as in FluxWorkload.
    """

    def __init__(self, name="flux_sched", batch=57, n=1152, m=3072, steps=28,
                 seed=SEED_BASE + 6, early_ratio=20.0, tau=1.5, **kw):
        self.early_ratio, self.tau = float(early_ratio), float(tau)
        super().__init__(name=name, batch=batch, n=n, m=m, steps=steps, seed=seed, **kw)

    def white(self, t: int) -> float:
        """Std of the white part of the step change at step t >= 1, in units of s_c."""
        return self.sigma / math.sqrt(2.0) * (1.0 + (self.early_ratio - 1.0) * math.exp(-(t - 1) / self.tau))

    def _step(self, t):
        lib = _load()
        for i, b in enumerate(self.tensors):
            lib.sg_flux_step_mix(self.seed, b, t, self.n, self.m, self.white(t),
                                 self.sigma / math.sqrt(2.0), self.drift_rank, _p(self._sc[i]),
                                 _p(self._A[i]), _p(self._B[i]), _p(self._state[i]))


class VideoWorkload(Workload):
    def __init__(self, name="video", batch=30, m=1920, steps=50, seed=SEED_BASE + 4, share=0,
                 n_shares=4, n_text=226, frames=13, height=30, width=45, blur_sigma=2.0, rho=0.98,
                 tensors=None):
        total = n_text + frames * height * width
        if total % n_shares:
            raise ValueError("token count %d not divisible by %d shares" % (total, n_shares))
        n = total // n_shares
        self.rho = rho
        self._geom = _VideoGeom(n_text, frames, height, width, share, n, blur_sigma)
        super().__init__(name, batch, n, m, steps, "bf16", seed, tensors)

    def _init(self):
        lib = _load()
        nb, n, m = self.nb, self.n, self.m
        self._sc = np.empty((nb, m), np.float32)
        self._state = np.empty((nb, n, m), np.float32)
        self._scratch = np.empty((n, m), np.float32)
        for i, b in enumerate(self.tensors):
            lib.sg_video_init(self.seed, b, ctypes.byref(self._geom), m, _p(self._sc[i]),
                              _p(self._state[i]))

    def _step(self, t):
        lib = _load()
        for i, b in enumerate(self.tensors):
            lib.sg_video_step(self.seed, b, t, ctypes.byref(self._geom), self.m, self.rho,
                              _p(self._sc[i]), _p(self._state[i]), _p(self._scratch))


class LatentWorkload(Workload):
    """Spatial token grid H x W (raster order) x C channels, bf16; change per step
    concentrated in smooth regions (gen.c, sg_latent_*)."""

    def __init__(self, name="latent", batch=16, height=64, width=128, m=320, steps=50,
                 seed=SEED_BASE + 5, sigma=0.1, gamma=1.0, blur=8.0, tensors=None):
        self.height, self.width = height, width
        self.sigma, self.gamma, self.blur = sigma, gamma, blur
        super().__init__(name, batch, height * width, m, steps, "bf16", seed, tensors)

    def _init(self):
        lib = _load()
        self._sc = np.empty((self.nb, self.m), np.float32)
        self._state = np.empty((self.nb, self.n, self.m), np.float32)
        self._field = np.empty(2 * self.n, np.float64)
        for i, b in enumerate(self.tensors):
            lib.sg_latent_init(self.seed, b, self.height, self.width, self.m, _p(self._sc[i]),
                               _p(self._state[i]))

    def _step(self, t):
        lib = _load()
        for i, b in enumerate(self.tensors):
            lib.sg_latent_step(self.seed, b, t, self.height, self.width, self.m, self.sigma,
                               self.gamma, self.blur, _p(self._sc[i]), _p(self._state[i]),
                               _p(self._field))


# The evaluated settings: (workload factory, scheme, scheme parameters).
CONFIGS = {
    "tiny_q1": dict(workload=lambda **kw: WalkWorkload(**kw), scheme="q1", group=64),
    "flux_q2": dict(workload=lambda **kw: FluxWorkload(**kw), scheme="q2", group=128),
    "flux_nm": dict(workload=lambda **kw: FluxWorkload(**kw), scheme="nm", nm_keep=2, nm_block=16),
    "flux_lr": dict(workload=lambda **kw: FluxWorkload(**kw), scheme="lr", rank=32, iters=2),
    "video_q1": dict(workload=lambda **kw: VideoWorkload(**kw), scheme="q1", group=64),
    "video_lr": dict(workload=lambda **kw: VideoWorkload(**kw), scheme="lr", rank=48, iters=2),
    # Otil-style block selection: 8x8-token blocks, a quarter of them per step
    "latent_bs": dict(workload=lambda **kw: LatentWorkload(**kw), scheme="bs", grid_w=128,
                      keep_blocks=32),
}


def make(config: str, **kw) -> Workload:
    return CONFIGS[config]["workload"](**kw)


def sigma_ratio(a_prev: np.ndarray, a_next: np.ndarray) -> float:
    """std(a_next - a_prev) / std(a_prev) (for checking generator statistics)."""
    d = a_next.astype(np.float64) - a_prev.astype(np.float64)
    return float(d.std() / a_prev.astype(np.float64).std())


__all__ = ["start_matrices", "Workload", "WalkWorkload", "FluxWorkload", "NoiseScheduleWorkload",
           "VideoWorkload", "LatentWorkload", "CONFIGS", "make", "build",
           "normal", "uniform", "key", "to_bf16_bits", "bf16_bits_to_f32", "SEED_BASE",
           "sigma_ratio"]
