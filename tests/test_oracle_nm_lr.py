"""Pins of the CPU oracle's N:M sparsifier and low-rank (subspace iteration +
INT4) compressor.

N:M ("Accelerating Parallel Diffusion Model Serving with Residual Compression",
Key designs / System co-design): checked against a brute-force stable sort of
each 16-block, the textbook routine the selection replaces.
Low rank (same page, Key designs / Low-rank strategy for extreme compression):
checked against numpy's SVD (Eckart-Young lower bound and the optimum that the
iteration approaches), exact-rank inputs, orthonormality of the CholeskyQR2
output, the INT4 rounding bound, and the zero / rank-deficient degenerate cases.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(7)


# ------------------------------------------------------------------ N:M
def test_nm_matches_stable_sort_per_block():
    r = (RNG.standard_normal(16 * 3000) * np.exp(RNG.standard_normal(16 * 3000))).astype(np.float32)
    # plant exact ties in some blocks
    r[16 * 5:16 * 6] = np.float32(0.5) * np.where(RNG.random(16) < 0.5, 1, -1)
    r[16 * 7 + 3] = r[16 * 7 + 11] = np.float32(-9.0)
    r[16 * 7 + 8] = np.float32(9.0)
    r[16 * 9:16 * 10] = 0.0
    vals, idx = oracle.nm_encode(r)
    for b in range(3000):
        blk = r[16 * b:16 * (b + 1)]
        order = np.argsort(-np.abs(blk.astype(np.float64)), kind="stable")[:2]
        i0, i1 = sorted(order.tolist())
        assert idx[b] == (i0 | (i1 << 4)), b
        want = oracle.bf16_bits(blk[[i0, i1]])
        assert vals[2 * b] == want[0] and vals[2 * b + 1] == want[1]
    assert idx[5] == (0 | (1 << 4))            # all-equal block keeps 0 and 1
    assert idx[7] == (3 | (8 << 4))            # |-9| at 3, 8, 11: the two lowest indices
    assert idx[9] == (0 | (1 << 4))            # all-zero block keeps 0 and 1


def test_nm_properties_and_lossless_blocks():
    r = RNG.standard_normal(16 * 500).astype(np.float32)
    vals, idx = oracle.nm_encode(r)
    c = oracle.nm_decode(vals, idx, r.size)
    e, _ = oracle.ef_update(r, c, np.zeros_like(r))
    kept = c != 0
    for b in range(500):
        sl = slice(16 * b, 16 * (b + 1))
        k = kept[sl]
        assert k.sum() == 2
        assert np.abs(r[sl][k]).min() >= np.abs(r[sl][~k]).max()
    assert np.array_equal(e[~kept], r[~kept])                      # dropped: whole residual stays
    assert np.array_equal(e[kept], r[kept] - oracle.bf16_round(r[kept]))
    # blocks with at most two bf16-representable non-zeros are lossless
    z = np.zeros(16 * 100, np.float32)
    for b in range(100):
        pos = RNG.choice(16, size=RNG.integers(0, 3), replace=False)
        z[16 * b + pos] = oracle.bf16_round(RNG.standard_normal(pos.size).astype(np.float32))
    c = oracle.nm_decode(*oracle.nm_encode(z), z.size)
    assert np.array_equal(c, z)


# ------------------------------------------------------------------ low rank
def _tiny(n, m, k, spectrum, seed):
    rng = np.random.default_rng(seed)
    Ua, _ = np.linalg.qr(rng.standard_normal((n, min(n, m))))
    Va, _ = np.linalg.qr(rng.standard_normal((m, min(n, m))))
    r = (Ua * spectrum) @ Va.T
    return r.astype(np.float32), rng.standard_normal((m, k)).astype(np.float32)


def _opt(rb, k):
    s = np.linalg.svd(rb, compute_uv=False)
    return np.sqrt(np.sum(s[k:] ** 2)) / np.linalg.norm(rb)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_lr_never_beats_svd_and_approaches_it(k):
    spectrum = 2.0 ** -np.arange(10) * 3
    r, q0 = _tiny(12, 10, k, spectrum, seed=k)
    rb = oracle.bf16_round(r).astype(np.float64)
    opt = _opt(rb, k)
    proj_err = []
    for iters in (1, 2, 4, 8, 16, 32):
        U, V, nd = oracle.lr_factors(r, q0, k, iters)
        assert nd == 0
        err = np.linalg.norm(rb - U @ V.T) / np.linalg.norm(rb)
        assert err >= opt * (1 - 1e-12)                   # Eckart-Young: rank-k error >= optimum
        proj_err.append(np.linalg.norm(rb - U @ (U.T @ rb)) / np.linalg.norm(rb))
    assert proj_err[-1] <= opt * (1 + 1e-4)                 # the subspace converges to the SVD one
    # monotone until converged (the bf16 operands leave a ~1e-7 relative wobble at the fixed point)
    assert all(b <= a * (1 + 1e-9) or b <= opt * (1 + 1e-6) for a, b in zip(proj_err, proj_err[1:]))
    assert proj_err[0] > proj_err[-1]


def test_lr_orthonormal_panel_and_exact_rank():
    # integer outer products are exact in bf16, so R has exact rank 2
    A = RNG.integers(-2, 3, (40, 2)).astype(np.float64)
    B = RNG.integers(-2, 3, (30, 2)).astype(np.float64)
    r = (A @ B.T).astype(np.float32)
    q0 = RNG.standard_normal((30, 2)).astype(np.float32)
    U, V, nd = oracle.lr_factors(r, q0, 2, 1)
    assert nd == 0
    assert np.abs(U.T @ U - np.eye(2)).max() < 1e-12
    rb = r.astype(np.float64)
    # one iteration already spans range(R); the projection is exact to fp64
    assert np.linalg.norm(rb - U @ (U.T @ rb)) / np.linalg.norm(rb) < 1e-12
    # U V^T differs from R only through the bf16 rounding of the U operand
    assert np.linalg.norm(rb - U @ V.T) / np.linalg.norm(rb) < 2.0 ** -7


def test_lr_int4_bound_and_range():
    r = RNG.standard_normal((64, 48)).astype(np.float32)
    q0 = RNG.standard_normal((48, 8)).astype(np.float32)
    qu, qv, su, sv, U, V, nd = oracle.lr_encode(r, q0, 8, 2, return_factors=True)
    for q, s, X in ((qu, su, U), (qv, sv, V)):
        assert np.abs(q).max() <= 7
        assert np.all(np.abs(q).max(axis=0) == 7)                       # absmax hits +-7
        assert np.all(np.abs(X - q * s.astype(np.float64)) <= s.astype(np.float64) / 2 * (1 + 1e-6))
    c = oracle.lr_decode(qu, qv, su, sv)
    assert np.allclose(c, (qu * su.astype(np.float64)) @ (qv * sv.astype(np.float64)).T, rtol=1e-12,
                       atol=1e-300)


def test_lr_zero_and_rank_deficient_residuals():
    q0 = RNG.standard_normal((24, 4)).astype(np.float32)
    r = np.zeros((20, 24), np.float32)
    qu, qv, su, sv, nd = oracle.lr_encode(r, q0, 4, 2)
    assert nd == 4 and not qu.any() and not qv.any() and not su.any()
    c = oracle.lr_decode(qu, qv, su, sv)
    assert np.all(c == 0)
    A = RNG.integers(-3, 4, (20, 2)).astype(np.float64)
    B = RNG.integers(-3, 4, (24, 2)).astype(np.float64)
    r = (A @ B.T).astype(np.float32)
    qu, qv, su, sv, U, V, nd = oracle.lr_encode(r, q0, 4, 2, return_factors=True)
    assert nd == 2
    assert np.all(np.isfinite(U)) and np.all(np.isfinite(V))
    assert np.count_nonzero(np.abs(U).max(axis=0)) == 2


def test_lr_zero_start_columns_are_dead_and_change_nothing():
    # Rank k from a start matrix padded with zero columns to width k' > k gives
    # exactly the rank-k result: the zero columns stay zero through every
    # product, every CholeskyQR pass declares them dead, and the live columns
    # see the same arithmetic (the products only add exact zeros). A rank-8
    # request may therefore run 16 wide.
    n, m = 40, 48
    A = RNG.standard_normal((n, 10)) * np.linspace(3, 0.2, 10)
    r = (A @ RNG.standard_normal((10, m)) + 0.05 * RNG.standard_normal((n, m))).astype(np.float32)
    q0 = RNG.standard_normal((m, 8)).astype(np.float32)
    q0w = np.concatenate([q0, np.zeros((m, 8), np.float32)], axis=1)
    U8, V8, nd8 = oracle.lr_factors(r, q0, 8, 2)
    U16, V16, nd16 = oracle.lr_factors(r, q0w, 16, 2)
    assert nd8 == 0 and nd16 == 8
    assert np.array_equal(U16[:, :8], U8) and np.array_equal(V16[:, :8], V8)
    assert not U16[:, 8:].any() and not V16[:, 8:].any()
    qu8, qv8, su8, sv8, _ = oracle.lr_encode(r, q0, 8, 2)
    qu16, qv16, su16, sv16, _ = oracle.lr_encode(r, q0w, 16, 2)
    assert np.array_equal(qu16[:, :8], qu8) and np.array_equal(qv16[:, :8], qv8)
    assert np.array_equal(su16[:8], su8) and not su16[8:].any() and not qu16[:, 8:].any()
    c8 = oracle.lr_decode(qu8, qv8, su8, sv8)
    c16 = oracle.lr_decode(qu16, qv16, su16, sv16)
    assert np.array_equal(c16.view(np.uint32), c8.view(np.uint32))


def test_lr_bf16_factors_rounding_and_bound():
    # factor-precision alternative: the same factors, each element sent as bf16
    import torch
    r = RNG.standard_normal((96, 64)).astype(np.float32)
    q0 = RNG.standard_normal((64, 16)).astype(np.float32)
    U, V, _ = oracle.lr_factors(r, q0, 16, 2)
    ub, vb, _ = oracle.lr_encode_bf16(r, q0, 16, 2)
    for X, xb in ((U, ub), (V, vb)):
        want = torch.from_numpy(X.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(xb.view(np.int16), want)
    # each factor element within u = 2^-8 (+ the fp32 step) of the fp64 value,
    # so c = Ub Vb^T is within (2u + u^2) |U| |V|^T of U V^T elementwise
    u = 2.0 ** -8 + 2.0 ** -24
    c = oracle.lr_decode_bf16(ub, vb)
    bound = (2 * u + u * u) * (np.abs(U) @ np.abs(V).T)
    assert np.all(np.abs(c - U @ V.T) <= bound * (1 + 1e-12))


def test_lr_bf16_factor_layout_roundtrip():
    n, m, k = 40, 64, 16
    assert oracle.section_sizes("lr", n, m, rank=k, factors="bf16") == [2 * n * k, 2 * m * k]
    a = RNG.standard_normal((n, m)).astype(np.float32)
    ahat = RNG.standard_normal((n, m)).astype(np.float32)
    q0 = RNG.standard_normal((m, k)).astype(np.float32)
    o = oracle.compress_tensor("lr", a, ahat, rank=k, iters=2, q0=q0, factors="bf16")
    assert o["packed"].size == oracle.tensor_bytes("lr", n, m, rank=k, factors="bf16")
    c = oracle.decode_tensor("lr", o["packed"], n, m, rank=k, factors="bf16")
    assert np.array_equal(c.astype(np.float64), o["c"].astype(np.float64))
    f = oracle.unpack_fields("lr", o["packed"], n, m, rank=k, factors="bf16")
    assert f["ub"].shape == (n, k) and f["vb"].shape == (m, k)
    rec = oracle.decompress_tensor("lr", o["packed"], ahat, rank=k, factors="bf16")
    assert np.array_equal(rec.view(np.uint32), o["ahat"].view(np.uint32))
