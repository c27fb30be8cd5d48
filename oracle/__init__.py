"""CPU ORACLE -- test infrastructure only.

Plain, slow, obviously-correct CPU implementation of the residual-compression
path (the C functions in ``oracle.c``, driven from here). Only ``tests/``, the
smoke check and the benchmark's ``cpu_baseline`` leg may import it. It shares no
code with the GPU library: the packed byte layout below is written out here
independently of the library's own layout code.

Method source: the paper-notes page "Accelerating Parallel Diffusion Model
Serving with Residual Compression" (CompactFusion), sections Method / Overall
framework, Key designs (Residual compression, Error feedback, Low-rank strategy
for extreme compression, System co-design), Main experiment table and
Limitations (warm-up); block selection follows the page "Otil: Accelerating
Diffusion Model Inference via Communication-Efficient Multi-GPU Parallelism",
Key designs 1-3. See ``oracle.c`` for the per-function citations and the
readings taken where the pages are silent.

Parity status: every scheme is pinned by the CPU tests (closed forms, brute
force, library routines, invariants); the low-rank factors themselves are
compared by tolerance only (their bits are not fixed by any definition).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Compile flags: IEEE single/double semantics, no contraction into FMA.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


# AddressSanitizer + UndefinedBehaviorSanitizer build (a CPU check of the C
# code; the library is then loaded with the sanitizer runtimes preloaded and
# ORACLE_LIB naming it).
SAN_CFLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all"]


def build(force: bool = True, sanitize: bool = False, out: str = None) -> str:
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, *(SAN_CFLAGS if sanitize else []), _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.orc_bf16_bits.restype = ctypes.c_uint16
        lib.orc_bf16_bits.argtypes = [ctypes.c_float]
        lib.orc_bf16_round_array.argtypes = [i64, vp, vp]
        lib.orc_residual.argtypes = [i64, vp, vp, vp]
        lib.orc_ef_update.argtypes = [i64, vp, vp, vp, vp]
        lib.orc_accumulate.argtypes = [i64, vp, vp]
        lib.orc_ef_update_f64.argtypes = [i64, vp, vp, vp, vp]
        lib.orc_accumulate_f64.argtypes = [i64, vp, vp]
        lib.orc_q1_encode.argtypes = [i64, i32, vp, vp, vp]
        lib.orc_q1_decode.argtypes = [i64, i32, vp, vp, vp]
        lib.orc_q2_encode.argtypes = [i64, i32, vp, vp, vp, vp]
        lib.orc_q2_decode.argtypes = [i64, i32, vp, vp, vp, vp]
        lib.orc_nm_encode.argtypes = [i64, vp, vp, vp]
        lib.orc_nm_decode.argtypes = [i64, vp, vp, vp]
        lib.orc_lr_encode.restype = i32
        lib.orc_lr_encode.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_lr_decode.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        lib.orc_bs_scores.argtypes = [i32, i32, i32, vp, vp, vp]
        lib.orc_lr_factors.restype = i32
        lib.orc_lr_factors.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


# ------------------------------------------------------------ elementwise
def bf16_round(x) -> np.ndarray:
    x = _f32(x)
    out = np.empty_like(x)
    _load().orc_bf16_round_array(x.size, _p(x), _p(out))
    return out


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (oracle's own rounding)."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def residual(a, ahat) -> np.ndarray:
    a, ahat = _f32(a), _f32(ahat)
    r = np.empty_like(a)
    _load().orc_residual(a.size, _p(a), _p(ahat), _p(r))
    return r


def ef_update(r, c, ahat):
    """(e, ahat_new) with e = r - c, ahat_new = ahat + c (fp32, or fp64 c)."""
    r = _f32(r)
    e = np.empty_like(r)
    ahat = _f32(ahat).copy()
    if np.asarray(c).dtype == np.float64:
        c = np.ascontiguousarray(c, np.float64)
        _load().orc_ef_update_f64(r.size, _p(r), _p(c), _p(e), _p(ahat))
    else:
        c = _f32(c)
        _load().orc_ef_update(r.size, _p(r), _p(c), _p(e), _p(ahat))
    return e, ahat


def accumulate(c, ahat) -> np.ndarray:
    ahat = _f32(ahat).copy()
    if np.asarray(c).dtype == np.float64:
        c = np.ascontiguousarray(c, np.float64)
        _load().orc_accumulate_f64(ahat.size, _p(c), _p(ahat))
    else:
        c = _f32(c)
        _load().orc_accumulate(ahat.size, _p(c), _p(ahat))
    return ahat


# ------------------------------------------------------------ schemes
def q1_encode(r, group=64):
    r = _f32(r)
    assert r.size % group == 0 and group in (8, 16, 32, 64, 128, 256)
    bits = np.zeros(r.size // 8, np.uint8)
    scale = np.empty(r.size // group, np.float32)
    _load().orc_q1_encode(r.size, group, _p(r), _p(bits), _p(scale))
    return bits, scale


def q1_decode(bits, scale, count, group=64):
    c = np.empty(count, np.float32)
    _load().orc_q1_decode(count, group, _p(np.ascontiguousarray(bits, np.uint8)), _p(_f32(scale)),
                          _p(c))
    return c


def q2_encode(r, group=128):
    r = _f32(r)
    assert r.size % group == 0 and group % 4 == 0
    codes = np.zeros(r.size // 4, np.uint8)
    mn = np.empty(r.size // group, np.float32)
    d = np.empty(r.size // group, np.float32)
    _load().orc_q2_encode(r.size, group, _p(r), _p(codes), _p(mn), _p(d))
    return codes, mn, d


def q2_decode(codes, mn, d, count, group=128):
    c = np.empty(count, np.float32)
    _load().orc_q2_decode(count, group, _p(np.ascontiguousarray(codes, np.uint8)), _p(_f32(mn)),
                          _p(_f32(d)), _p(c))
    return c


def nm_encode(r):
    r = _f32(r)
    assert r.size % 16 == 0
    vals = np.empty(2 * (r.size // 16), np.uint16)
    idx = np.empty(r.size // 16, np.uint8)
    _load().orc_nm_encode(r.size, _p(r), _p(vals), _p(idx))
    return vals, idx


def nm_decode(vals, idx, count):
    c = np.empty(count, np.float32)
    _load().orc_nm_decode(count, _p(np.ascontiguousarray(vals, np.uint16)),
                          _p(np.ascontiguousarray(idx, np.uint8)), _p(c))
    return c


def lr_encode(r, q0, rank, iters, return_factors=False):
    """r: fp32 [n, m]; q0: fp32 [m, rank]. Returns (qu, qv, su, sv[, U, V], ndead)."""
    r = _f32(r)
    n, m = r.shape
    q0 = _f32(q0)
    assert q0.shape == (m, rank)
    qu = np.empty((n, rank), np.int8)
    qv = np.empty((m, rank), np.int8)
    su = np.empty(rank, np.float32)
    sv = np.empty(rank, np.float32)
    U = np.empty((n, rank), np.float64) if return_factors else None
    V = np.empty((m, rank), np.float64) if return_factors else None
    nd = _load().orc_lr_encode(n, m, rank, iters, _p(r), _p(q0), _p(qu), _p(qv), _p(su), _p(sv),
                               _p(U), _p(V))
    if return_factors:
        return qu, qv, su, sv, U, V, nd
    return qu, qv, su, sv, nd


def lr_decode(qu, qv, su, sv):
    n, k = qu.shape
    m = qv.shape[0]
    c = np.empty((n, m), np.float64)
    _load().orc_lr_decode(n, m, k, _p(np.ascontiguousarray(qu, np.int8)),
                          _p(np.ascontiguousarray(qv, np.int8)), _p(_f32(su)), _p(_f32(sv)), _p(c))
    return c


def lr_encode_bf16(r, q0, rank, iters):
    """Low-rank factors sent as bf16 instead of INT4 (the factor-precision
    alternative of the Low-rank strategy section: fewer, finer factors against
    more, coarser ones). U, V are the same subspace-iteration factors as in
    lr_encode; each element is rounded to fp32 and then to bf16 (RNE).
    Returns (ub, vb, ndead): bf16 bit patterns [n, rank], [m, rank]."""
    U, V, nd = lr_factors(r, q0, rank, iters)
    return bf16_bits(U.astype(np.float32)), bf16_bits(V.astype(np.float32)), nd


def lr_decode_bf16(ub, vb):
    """c = Ub Vb^T in fp64 from bf16 factor bit patterns."""
    U = bf16_value(np.asarray(ub, np.uint16)).astype(np.float64)
    V = bf16_value(np.asarray(vb, np.uint16)).astype(np.float64)
    return U @ V.T


def lr_factors(r, q0, rank, iters):
    """Unquantised factors (U [n,k], V [m,k]) of the subspace iteration."""
    r = _f32(r)
    n, m = r.shape
    U = np.empty((n, rank), np.float64)
    V = np.empty((m, rank), np.float64)
    nd = _load().orc_lr_factors(n, m, rank, iters, _p(r), _p(_f32(q0)), _p(U), _p(V))
    return U, V, nd


# ------------------------------------------------------------ block selection
def bs_scores(a, ahat, grid_w):
    """Cosine dissimilarity between a and ahat of every 8x8-token block
    (raster order), fp64."""
    a, ahat = _f32(a), _f32(ahat)
    n, m = a.shape
    K = (n // grid_w // 8) * (grid_w // 8)
    d = np.empty(K, np.float64)
    _load().orc_bs_scores(n, m, grid_w, _p(a), _p(ahat), _p(d))
    return d


def bs_select(d, visited, keep):
    """Top-`keep` blocks by dissimilarity among the blocks not yet visited in
    this round (ties to the lower index), then mark them visited (Otil page,
    Key design 3: dynamic round robin). Reading: when every block has been
    visited, the round restarts before selecting, and a round's last step sends
    only the blocks still unvisited. Returns (selected indices ascending,
    visited mask after the step)."""
    visited = np.array(visited, dtype=bool, copy=True)
    if visited.all():
        visited[:] = False
    cand = np.flatnonzero(~visited)
    order = cand[np.lexsort((cand, -np.asarray(d)[cand]))]
    sel = np.sort(order[:keep])
    visited[sel] = True
    return sel, visited


def bs_block_tokens(i, grid_w):
    """Token indices of block i (raster order inside the block)."""
    nbx = grid_w // 8
    by, bx = divmod(int(i), nbx)
    return np.array([(by * 8 + dy) * grid_w + bx * 8 + dx for dy in range(8) for dx in range(8)])


# ------------------------------------------------------------ packed layout
# Per tensor, sections in this order, each starting at a multiple of 256 bytes;
# tensors follow each other, each tensor's block a multiple of 256 bytes.
#   q1: sign bits [N/8]            | scales f32 [N/G]
#   q2: 2-bit codes [N/4]          | group minima mn f32 [N/G] | steps d f32 [N/G]
#   nm: (v_i0, v_i1) bf16 pairs [N/16] | index bytes i0 | i1<<4 [N/16]
#   lr: U nibbles [n*k/2] | V nibbles [m*k/2] | s_U f32 [k] | s_V f32 [k]
#       nibble t of a row-major [rows x k] INT4 matrix = element t; even t in
#       the low nibble; two's complement.
#   lr with bf16 factors: U bf16 [n*k] | V bf16 [m*k], row-major.
#   bs: u32 [1 + keep] (count, then the sent block indices ascending, unused
#       slots 0) | block values [keep][64 tokens][m] in the input dtype (bf16 bit
#       patterns or fp32), tokens of a block in raster order, unused slots 0.
ALIGN = 256


def _al(x):
    return (x + ALIGN - 1) // ALIGN * ALIGN


def section_sizes(scheme, n, m, group=None, rank=None, factors="int4", keep=None, in_bytes=2):
    N = n * m
    if scheme == "bs":
        return [4 * (1 + keep), keep * 64 * m * in_bytes]
    if scheme == "lr" and factors == "bf16":
        return [2 * n * rank, 2 * m * rank]
    if scheme == "q1":
        return [N // 8, 4 * (N // group)]
    if scheme == "q2":
        return [N // 4, 4 * (N // group), 4 * (N // group)]
    if scheme == "nm":
        return [4 * (N // 16), N // 16]
    if scheme == "lr":
        return [n * rank // 2, m * rank // 2, 4 * rank, 4 * rank]
    raise ValueError(scheme)


def tensor_bytes(scheme, n, m, group=None, rank=None, factors="int4", keep=None, in_bytes=2):
    return sum(_al(s) for s in section_sizes(scheme, n, m, group, rank, factors, keep, in_bytes))


def _place(sections, scheme, n, m, group, rank, factors="int4", keep=None, in_bytes=2):
    buf = np.zeros(tensor_bytes(scheme, n, m, group, rank, factors, keep, in_bytes), np.uint8)
    off = 0
    for raw, size in zip(sections, section_sizes(scheme, n, m, group, rank, factors, keep, in_bytes)):
        raw = np.ascontiguousarray(raw).view(np.uint8).ravel()
        assert raw.size == size, (raw.size, size)
        buf[off:off + size] = raw
        off += _al(size)
    return buf


def _split(buf, scheme, n, m, group, rank, factors="int4", keep=None, in_bytes=2):
    out, off = [], 0
    for size in section_sizes(scheme, n, m, group, rank, factors, keep, in_bytes):
        out.append(buf[off:off + size])
        off += _al(size)
    return out


def _pack_int4(q):
    q = np.asarray(q, np.int8).ravel()
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def _unpack_int4(b, count):
    b = np.asarray(b, np.uint8)
    lo = (b & 0xF).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    q = np.empty(2 * b.size, np.int16)
    q[0::2], q[1::2] = lo, hi
    q = np.where(q >= 8, q - 16, q)
    return q[:count].astype(np.int8)


# ------------------------------------------------------------ one tensor
def compress_tensor(scheme, a, ahat, *, group=None, rank=None, iters=None, q0=None,
                    factors="int4"):
    """One sender step on one tensor.

    a: library-view activations as fp32 values [n, m]; ahat: fp32 [n, m].
    Returns dict(packed, c, e, ahat, r) where ahat is the new sender state.
    """
    a = _f32(a)
    n, m = a.shape
    r = residual(a, ahat)
    flat = r.ravel()
    if scheme == "q1":
        bits, scale = q1_encode(flat, group)
        c = q1_decode(bits, scale, flat.size, group)
        packed = _place([bits, scale], scheme, n, m, group, rank)
    elif scheme == "q2":
        codes, mn, d = q2_encode(flat, group)
        c = q2_decode(codes, mn, d, flat.size, group)
        packed = _place([codes, mn, d], scheme, n, m, group, rank)
    elif scheme == "nm":
        vals, idx = nm_encode(flat)
        c = nm_decode(vals, idx, flat.size)
        packed = _place([vals, idx], scheme, n, m, group, rank)
    elif scheme == "lr" and factors == "bf16":
        ub, vb, _ = lr_encode_bf16(r, q0, rank, iters)
        c = lr_decode_bf16(ub, vb).ravel()
        packed = _place([ub, vb], scheme, n, m, group, rank, factors)
    elif scheme == "lr":
        qu, qv, su, sv, _ = lr_encode(r, q0, rank, iters)
        c = lr_decode(qu, qv, su, sv).ravel()
        packed = _place([_pack_int4(qu), _pack_int4(qv), su, sv], scheme, n, m, group, rank)
    elif scheme == "identity":
        c = flat.copy()
        packed = None
    else:
        raise ValueError(scheme)
    e, ahat_new = ef_update(flat, c, ahat.ravel())
    return dict(packed=packed, c=c.reshape(n, m), e=e.reshape(n, m), ahat=ahat_new.reshape(n, m),
                r=r)


def bs_compress_tensor(a, ahat, *, grid_w, keep, visited, prev=None, score="prev",
                       in_dtype="bf16", selected=None):
    """One sender step of Otil-style block selection on one tensor.

    Scores (Otil page, Key design 2): the cosine dissimilarity of each block
    between this step's activation `a` and the previous step's activation
    `prev` (the same block one denoising step apart). After the warm-up the
    sender's reconstruction equals the previous activation exactly, so
    prev=None means prev = ahat. score="last_sent" instead compares `a` with
    the receiver's copy `ahat` (the block as last sent): an alternative, not
    the page's rule.
    The selected blocks are sent as they are (values of a_t in the input dtype)
    and replace the receiver's copy, so after the step ahat = a_t there and
    e = 0; elsewhere ahat is unchanged and e = fl(a_t - ahat) (the whole
    residual stays on the sender). `selected` (ascending block indices) replaces
    the top-k choice, e.g. to follow another implementation's choice among
    near-equal scores. Returns dict(packed, e, ahat, visited, selected,
    scores)."""
    a = _f32(a)
    ahat = _f32(ahat)
    n, m = a.shape
    if score == "prev":
        ref = ahat if prev is None else _f32(prev)
    elif score == "last_sent":
        ref = ahat
    else:
        raise ValueError(score)
    d = bs_scores(a, ref, grid_w)
    sel, vis = bs_select(d, visited, keep)
    if selected is not None:
        vis = np.array(visited, dtype=bool, copy=True)
        if vis.all():
            vis[:] = False
        sel = np.sort(np.asarray(selected, np.int64))
        vis[sel] = True
    e = residual(a, ahat).reshape(n, m).copy()
    ahat_new = ahat.copy()
    in_bytes = 2 if in_dtype == "bf16" else 4
    head = np.zeros(1 + keep, np.uint32)
    head[0] = sel.size
    head[1:1 + sel.size] = sel
    vals = np.zeros((keep, 64, m), np.uint16 if in_bytes == 2 else np.float32)
    for j, i in enumerate(sel):
        tok = bs_block_tokens(i, grid_w)
        ahat_new[tok] = a[tok]
        e[tok] = 0.0
        vals[j] = bf16_bits(a[tok]) if in_bytes == 2 else a[tok]
    packed = _place([head, vals], "bs", n, m, None, None, keep=keep, in_bytes=in_bytes)
    return dict(packed=packed, e=e, ahat=ahat_new, visited=vis, selected=sel, scores=d)


def bs_decompress_tensor(packed, ahat_r, *, grid_w, keep, in_dtype="bf16"):
    """Receiver: put every sent block back at its place."""
    n, m = ahat_r.shape
    in_bytes = 2 if in_dtype == "bf16" else 4
    head, vals = _split(np.asarray(packed, np.uint8), "bs", n, m, None, None, keep=keep,
                        in_bytes=in_bytes)
    head = head.view(np.uint32)
    vals = (bf16_value(vals.view(np.uint16)) if in_bytes == 2 else vals.view(np.float32)).reshape(keep, 64, m)
    out = _f32(ahat_r).copy()
    for j in range(int(head[0])):
        out[bs_block_tokens(head[1 + j], grid_w)] = vals[j]
    return out


def decode_tensor(scheme, packed, n, m, *, group=None, rank=None, factors="int4"):
    """Decode one tensor's packed bytes to C(r) (fp32, or fp64 for lr)."""
    secs = _split(np.asarray(packed, np.uint8), scheme, n, m, group, rank, factors)
    N = n * m
    if scheme == "lr" and factors == "bf16":
        return lr_decode_bf16(secs[0].view(np.uint16).reshape(n, rank),
                              secs[1].view(np.uint16).reshape(m, rank))
    if scheme == "q1":
        return q1_decode(secs[0], secs[1].view(np.float32), N, group).reshape(n, m)
    if scheme == "q2":
        return q2_decode(secs[0], secs[1].view(np.float32), secs[2].view(np.float32), N,
                         group).reshape(n, m)
    if scheme == "nm":
        return nm_decode(secs[0].view(np.uint16), secs[1], N).reshape(n, m)
    if scheme == "lr":
        qu = _unpack_int4(secs[0], n * rank).reshape(n, rank)
        qv = _unpack_int4(secs[1], m * rank).reshape(m, rank)
        return lr_decode(qu, qv, secs[2].view(np.float32), secs[3].view(np.float32))
    raise ValueError(scheme)


def decompress_tensor(scheme, packed, ahat_r, *, group=None, rank=None, factors="int4"):
    n, m = ahat_r.shape
    c = decode_tensor(scheme, packed, n, m, group=group, rank=rank, factors=factors)
    return accumulate(c.ravel(), ahat_r.ravel()).reshape(n, m)


def unpack_fields(scheme, packed, n, m, *, group=None, rank=None, factors="int4"):
    """Named views of one tensor's packed sections (for exact comparisons)."""
    secs = _split(np.asarray(packed, np.uint8), scheme, n, m, group, rank, factors)
    if scheme == "lr" and factors == "bf16":
        return dict(ub=secs[0].view(np.uint16).reshape(n, rank),
                    vb=secs[1].view(np.uint16).reshape(m, rank))
    if scheme == "q1":
        return dict(bits=secs[0], scale=secs[1].view(np.float32))
    if scheme == "q2":
        return dict(codes=secs[0], mn=secs[1].view(np.float32), d=secs[2].view(np.float32))
    if scheme == "nm":
        return dict(vals=secs[0].view(np.uint16), idx=secs[1])
    if scheme == "lr":
        return dict(qu=_unpack_int4(secs[0], n * rank).reshape(n, rank),
                    qv=_unpack_int4(secs[1], m * rank).reshape(m, rank),
                    su=secs[2].view(np.float32), sv=secs[3].view(np.float32))
    raise ValueError(scheme)


# ------------------------------------------------------------ trajectories
def compress_values(scheme, x, *, group=None, rank=None, iters=None, q0=None, factors="int4"):
    """C(x) for a fp32 matrix x [n, m] (fp32, or fp64 for lr)."""
    x = _f32(x)
    flat = x.ravel()
    if scheme == "q1":
        return q1_decode(*q1_encode(flat, group), flat.size, group).reshape(x.shape)
    if scheme == "q2":
        return q2_decode(*q2_encode(flat, group), flat.size, group).reshape(x.shape)
    if scheme == "nm":
        return nm_decode(*nm_encode(flat), flat.size).reshape(x.shape)
    if scheme == "lr" and factors == "bf16":
        ub, vb, _ = lr_encode_bf16(x, q0, rank, iters)
        return lr_decode_bf16(ub, vb)
    if scheme == "lr":
        qu, qv, su, sv, _ = lr_encode(x, q0, rank, iters)
        return lr_decode(qu, qv, su, sv)
    if scheme == "identity":
        return x.copy()
    raise ValueError(scheme)


def run_schedule(frames, kinds):
    """Closed-loop sequence of one tensor with a scheme chosen per step.

    CompactFusion notes, Limitations: step 0 has no history and is sent in full,
    and the steps where the noise level changes sharply (the first few) may be
    sent in full or with a finer scheme before the cheap one takes over.
    kinds[t] is None for a step sent in full (both copies become a_t, the
    carried residual is dropped) or (scheme, params) for a compressed step of
    the closed loop (Overall framework / Error feedback), params as for
    compress_tensor. kinds[0] must be None. Returns ahat_t for every step.
    """
    if kinds[0] is not None:
        raise ValueError("step 0 is sent in full")
    out = []
    ahat = None
    for a, kind in zip(frames, kinds):
        a = _f32(a)
        if kind is None:
            ahat = a.copy()
        else:
            scheme, params = kind
            ahat = compress_tensor(scheme, a, ahat, **params)["ahat"]
        out.append(ahat.copy())
    return out


def run_trajectory(mode, scheme, frames, **kw):
    """Free-running sequence of one tensor through the scheme.

    frames: list of fp32 [n, m] activations a_0..a_{T-1} (a_0 is sent in full,
    the warm-up step in the Limitations section). Modes:
      closed  -- the normative loop: r = a_t - ahat_{t-1}; ahat += C(r); e = r - C(r)
      open    -- error feedback written against the previous activation:
                 r = (a_t - a_{t-1}) + e_{t-1}
      noef    -- r = a_t - a_{t-1}, the dropped part is discarded
      literal -- r = a_t - ahat_{t-1} + e_{t-1} (counts the carried error twice)
      direct  -- no residual: ahat_t = C(a_t)
    Returns a list of ahat_t (fp32 [n, m]) for t = 0..T-1.
    """
    a0 = _f32(frames[0])
    ahat = a0.copy()
    e = np.zeros_like(a0)
    out = [ahat.copy()]
    prev = a0
    for t in range(1, len(frames)):
        a = _f32(frames[t])
        if mode == "direct":
            c = compress_values(scheme, a, **kw)
            ahat = c.astype(np.float32) if c.dtype == np.float64 else c
            out.append(ahat.copy())
            continue
        if mode == "closed":
            r = residual(a, ahat)
        elif mode == "open":
            r = (residual(a, prev) + e).astype(np.float32)
        elif mode == "noef":
            r = residual(a, prev)
        elif mode == "literal":
            r = (residual(a, ahat) + e).astype(np.float32)
        else:
            raise ValueError(mode)
        c = compress_values(scheme, r, **kw)
        e_new, ahat = ef_update(r.ravel(), c.ravel(), ahat.ravel())
        ahat = ahat.reshape(a.shape)
        e = e_new.reshape(a.shape) if mode != "noef" else np.zeros_like(a)
        prev = a
        out.append(ahat.copy())
    return out
