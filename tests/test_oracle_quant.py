"""Pins of the CPU oracle's quantisers (1-bit, 2-bit) and bf16 rounding.

Each check ties the oracle to something other than itself: a library routine
(torch's bf16 conversion), an exactly rounded closed form (Fractions), a
least-squares optimality property, a brute-force nearest-level search, or a
hand-built group whose exact answer follows from the definition.
Method: "Accelerating Parallel Diffusion Model Serving with Residual
Compression", Key designs / Residual compression and the Main experiment table
(1-bit = 16x, 2-bit = 8x).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20251203)


def f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even (by comparing neighbours)."""
    d = np.float32(float(fr))
    cands = [np.nextafter(d, np.float32(-np.inf)), d, np.nextafter(d, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(f32_bits(c)) & 1))


# ------------------------------------------------------------------ bf16
def test_bf16_matches_torch_rounding():
    x = np.concatenate([
        RNG.standard_normal(200_000).astype(np.float32) * np.float32(3.0),
        (RNG.standard_normal(1000) * 1e-39).astype(np.float32),       # subnormals
        np.array([3.0e38, -3.3e38, 0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    # exact ties: low 16 bits = 0x8000 with even and odd kept parts
    base = (RNG.integers(0x3F00, 0x4100, 1000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, base.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(f32_bits(got), f32_bits(want))


# ------------------------------------------------------------------ 1-bit
def test_q1_scale_is_exactly_rounded_mean_abs():
    r = (RNG.standard_normal(64 * 40) * np.exp(RNG.standard_normal(64 * 40))).astype(np.float32)
    _, scale = oracle.q1_encode(r, 64)
    for g in range(40):
        exact = sum(Fraction(float(abs(v))) for v in r[g * 64:(g + 1) * 64]) / 64
        assert f32_bits(scale[g]) == f32_bits(round_fraction_to_f32(exact)), g


@pytest.mark.parametrize("group", [32, 64, 128])
def test_q1_scale_exactly_rounded_when_small_terms_decide(group):
    # The first half of the group sums to group * (1 + 2^-24), so the mean is
    # the midpoint between 1 and 1 + 2^-23; the second half adds group/2 terms
    # of 2^-51, pushing the exact mean just above it. The correctly rounded
    # scale is 1 + 2^-23. (Added one at a time to the large running sum, the
    # small terms would vanish and the tie would round down to 1.0.)
    half = group // 2
    g = np.full(group, 2.0)
    g[half - 1] = 2.0 + group * 2.0 ** -24
    g[half:] = 2.0 ** -51
    for k, sign_seed in ((0, 1), (7, 2), (-9, 3)):
        r = (g * 2.0 ** k * np.random.default_rng(sign_seed).choice([-1.0, 1.0], group)).astype(np.float32)
        _, scale = oracle.q1_encode(r, group)
        exact = sum(Fraction(float(abs(v))) for v in r) / group
        assert f32_bits(scale[0]) == f32_bits(round_fraction_to_f32(exact))
        assert scale[0] == np.float32((1 + 2.0 ** -23) * 2.0 ** k)


@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_q1_scale_exactly_rounded_on_wide_magnitude_spans(group):
    # Magnitudes with random exponents over the whole fp32 range (subnormals
    # included) make every floating-point summation order round somewhere;
    # the scale must still be the exactly rounded mean (Fractions).
    for trial in range(60):
        lo = int(RNG.integers(-149, 100))
        span = int(RNG.integers(20, 127 - lo + 1)) if lo < 100 else 20
        ex = RNG.integers(lo, min(lo + span, 127) + 1, group)
        mag = np.ldexp(RNG.uniform(1.0, 2.0, group), ex)
        r = (mag * RNG.choice([-1.0, 1.0], group)).astype(np.float32)
        r[RNG.random(group) < 0.1] = 0.0
        _, scale = oracle.q1_encode(r, group)
        exact = sum(Fraction(float(abs(v))) for v in r) / group
        assert f32_bits(scale[0]) == f32_bits(round_fraction_to_f32(exact)), trial


@pytest.mark.parametrize("group", [32, 64, 128])
def test_q1_scale_on_the_subnormal_grid(group):
    # Means below the smallest normal fp32 round on the subnormal grid 2^-149:
    # k terms of 2^-149 give k/group * 2^-149, which rounds to 0 below one half,
    # ties to even (0) at exactly one half, and to 2^-149 above it.
    tiny = np.float32(2.0 ** -149)
    for k, want in ((1, 0.0), (group // 2, 0.0), (group // 2 + 1, float(tiny)),
                    (3 * group // 2 // 2, float(tiny)), (group, float(tiny))):
        r = np.zeros(group, np.float32)
        r[:k] = tiny
        _, scale = oracle.q1_encode(r, group)
        assert scale[0] == np.float32(want), k
    # one and a half grid steps (3/4 of the group at 2^-148): a tie between
    # 2^-149 and 2^-148, which goes to the even one, 2^-148
    r = np.zeros(group, np.float32)
    r[:3 * group // 4] = np.float32(2.0 ** -148)
    _, scale = oracle.q1_encode(r, group)
    assert scale[0] == np.float32(2.0 ** -148)
    # the largest finite magnitudes do not overflow the exact sum
    r = np.full(group, np.float32(3.4028235e38), np.float32)
    _, scale = oracle.q1_encode(r, group)
    assert scale[0] == np.float32(3.4028235e38)


def test_q1_scale_minimises_squared_error_for_fixed_signs():
    r = RNG.standard_normal(64 * 50).astype(np.float32)
    bits, scale = oracle.q1_encode(r, 64)
    c = oracle.q1_decode(bits, scale, r.size, 64)
    sign = np.sign(c.astype(np.float64))
    for g in range(50):
        sl = slice(g * 64, (g + 1) * 64)
        x, sg = r[sl].astype(np.float64), sign[sl]
        f = lambda s: np.sum((x - sg * s) ** 2)
        s0 = float(scale[g])
        assert f(s0) <= f(s0 * (1 + 1e-3)) and f(s0) <= f(s0 * (1 - 1e-3))
        # signs are those of r (r >= 0 -> +)
        assert np.all((x >= 0) == (sg > 0))


def test_q1_hand_built_groups():
    # alternating signs, magnitudes 1..64 (/64): bits 1,0,1,0,... -> bytes 0x55
    mags = np.arange(1, 65, dtype=np.float64) / 64
    r = np.where(np.arange(64) % 2 == 0, mags, -mags).astype(np.float32)
    bits, scale = oracle.q1_encode(r, 64)
    assert bits.tolist() == [0x55] * 8
    assert scale[0] == np.float32(2080 / 64 / 64)   # sum(1..64)/64 / 64 = 0.5078125 exactly
    bits, _ = oracle.q1_encode(-r, 64)
    assert bits.tolist() == [0xAA] * 8
    # equal magnitudes: lossless
    r = np.where(RNG.random(128) < 0.5, 0.375, -0.375).astype(np.float32)
    bits, scale = oracle.q1_encode(r, 64)
    c = oracle.q1_decode(bits, scale, 128, 64)
    assert np.array_equal(c, r)
    # zero group (with negative zeros): scale 0, all bits 1, c = +-0, e = r
    r = np.zeros(64, np.float32)
    r[::3] = -0.0
    bits, scale = oracle.q1_encode(r, 64)
    assert scale[0] == 0 and bits.tolist() == [0xFF] * 8
    c = oracle.q1_decode(bits, scale, 64, 64)
    e, ahat = oracle.ef_update(r, c, np.full(64, 2.5, np.float32))
    assert np.all(e == 0) and np.all(ahat == 2.5)


def test_q1_packing_is_lsb_first():
    r = np.full(64, -1.0, np.float32)
    r[[0, 9, 17, 63]] = 1.0
    bits, _ = oracle.q1_encode(r, 64)
    want = [0] * 8
    for k in (0, 9, 17, 63):
        want[k // 8] |= 1 << (k % 8)
    assert bits.tolist() == want


# ------------------------------------------------------------------ 2-bit
def test_q2_is_nearest_level_and_within_half_step():
    r = (RNG.standard_normal(128 * 200) * np.exp(RNG.standard_normal(128 * 200))).astype(np.float32)
    codes, mn, d = oracle.q2_encode(r, 128)
    c = oracle.q2_decode(codes, mn, d, r.size, 128)
    for g in range(200):
        sl = slice(g * 128, (g + 1) * 128)
        x = r[sl].astype(np.float64)
        assert mn[g] == r[sl].min()
        assert float(d[g]) == pytest.approx((float(r[sl].max()) - float(mn[g])) / 3, rel=2.5e-7)
        # the 4 levels, each rounded once from mn + q d (exact rationals)
        lv = np.array([float(round_fraction_to_f32(Fraction(float(mn[g])) + q * Fraction(float(d[g]))))
                       for q in range(4)])
        dist = np.abs(x[:, None] - lv[None, :])
        got = np.abs(x - c[sl].astype(np.float64))
        assert np.all(np.isin(c[sl].astype(np.float64), lv))
        # brute force: the chosen level is the nearest one (up to a relative 1e-5 step near ties)
        assert np.all(got <= dist.min(axis=1) + 1e-5 * float(d[g]))
        assert np.all(got <= 0.5 * float(d[g]) * (1 + 1e-5))


def test_q2_hand_built_groups():
    # arithmetic progression on the 4 levels: lossless
    lv = np.array([-1.5, -1.0, -0.5, 0.0], np.float32)
    r = lv[RNG.integers(0, 4, 128)]
    r[:4] = lv
    codes, mn, d = oracle.q2_encode(r, 128)
    assert mn[0] == -1.5 and d[0] == 0.5
    c = oracle.q2_decode(codes, mn, d, 128, 128)
    assert np.array_equal(c, r)
    # ties round half to even: mn = 0, mx = 3 (d = 1): 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    r = np.zeros(128, np.float32)
    r[1], r[2], r[3], r[4], r[5] = 3.0, 0.5, 1.5, 2.5, 1.0
    codes, mn, d = oracle.q2_encode(r, 128)
    q = [(codes[k // 4] >> (2 * (k % 4))) & 3 for k in range(8)]
    assert q[:6] == [0, 3, 0, 2, 2, 1]
    # constant group: d = 0, every code 0, decodes exactly
    r = np.full(128, 0.7, np.float32)
    codes, mn, d = oracle.q2_encode(r, 128)
    assert d[0] == 0 and not codes.any()
    assert np.array_equal(oracle.q2_decode(codes, mn, d, 128, 128), r)
    # min maps to code 0, max to code 3
    r = RNG.standard_normal(128).astype(np.float32)
    codes, mn, d = oracle.q2_encode(r, 128)
    q = np.array([(codes[k // 4] >> (2 * (k % 4))) & 3 for k in range(128)])
    assert q[np.argmin(r)] == 0 and q[np.argmax(r)] == 3


def test_q2_packing_is_lsb_first():
    r = np.zeros(128, np.float32)
    r[1] = 3.0      # code 3 at element 1 -> bits 2..3 of byte 0
    r[6] = 1.0      # code 1 at element 6 -> bits 4..5 of byte 1
    codes, _, _ = oracle.q2_encode(r, 128)
    assert codes[0] == 0b1100 and codes[1] == 0b010000
