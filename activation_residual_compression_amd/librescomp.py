"""ctypes binding of the librescomp C ABI (``include/librescomp.h``).

Argument marshalling only: every step of the compression path runs in the HIP
kernels of ``librescomp.so``. Functions keep the C names; a non-RC_OK status
raises :class:`RcError`. Tensor arguments may be torch tensors (their
``data_ptr()`` is passed) or raw integer device addresses; the low-rank start
matrices ``q0`` may also be a host numpy array, which ``Plan`` copies to the
device for the plan's set-up. Streams may be a ``torch.cuda.Stream``, a raw
``hipStream_t`` integer, or None for torch's current stream.

The library must be built first (``__graft_entry__.build()`` or
``python -m activation_residual_compression_amd.build``); importing this module
without it raises, so nothing can silently fall back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIBRESCOMP_LIB names another build of the library (the CPU sanitizer build
# of the host code); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("LIBRESCOMP_LIB") or os.path.join(_HERE, "lib", "librescomp.so")

RC_OK, RC_ERR_INVALID_ARG, RC_ERR_UNSUPPORTED, RC_ERR_ALIGNMENT, RC_ERR_HIP = 0, 1, 2, 3, 4
RC_ERR_NUMERIC, RC_ERR_NONFINITE = 5, 6
RC_BF16, RC_F32 = 0, 1
RC_Q1, RC_Q2, RC_NM, RC_LOWRANK, RC_BLOCKSEL = 0, 1, 2, 3, 4
RC_MAX_PEERS = 8
RC_LR_BF16_FACTORS = 1  # rc_params_t.flags, RC_LOWRANK only
RC_LR_ONE_STREAM = 2    # rc_params_t.flags, RC_LOWRANK only: no second stream in rc_compress
RC_BS_SCORE_LAST_SENT = 4  # rc_params_t.flags, RC_BLOCKSEL only: score against ahat
RC_CHECK_FINITE = 8        # rc_params_t.flags, any scheme: reject NaN / Inf inputs (syncs)
RC_LR_CHECK_NUMERIC = 16   # rc_params_t.flags, RC_LOWRANK only: report dead pivots (syncs)

SCHEMES = {"q1": RC_Q1, "q2": RC_Q2, "nm": RC_NM, "lr": RC_LOWRANK, "bs": RC_BLOCKSEL}
DTYPES = {"bf16": RC_BF16, "f32": RC_F32}


class rc_shape_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class rc_params_t(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("nm_keep", ctypes.c_int32),
                ("nm_block", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("seed", ctypes.c_uint64), ("q0", ctypes.c_void_p),
                ("flags", ctypes.c_uint32),
                ("grid_w", ctypes.c_int32), ("keep_blocks", ctypes.c_int32)]


class rc_state_t(ctypes.Structure):
    _fields_ = [("ahat", ctypes.c_void_p), ("e", ctypes.c_void_p)]


class RcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, rc_status_string(status)))


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "librescomp.so is not built (expected at %s); run __graft_entry__.build() "
            "or python -m activation_residual_compression_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    lib.rc_plan_create.restype = st
    lib.rc_plan_create.argtypes = [rc_shape_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(rc_params_t), ctypes.POINTER(vp)]
    lib.rc_compress.restype = st
    lib.rc_compress.argtypes = [vp, vp, vp, ctypes.POINTER(rc_state_t), vp]
    lib.rc_compress_lowrank_noalloc.restype = st
    lib.rc_compress_lowrank_noalloc.argtypes = [rc_shape_t, ctypes.c_int, ctypes.POINTER(rc_params_t),
                                                vp, vp, ctypes.POINTER(rc_state_t), vp]
    lib.rc_decompress.restype = st
    lib.rc_decompress.argtypes = [vp, vp, vp, vp]
    lib.rc_compress_send.restype = st
    lib.rc_compress_send.argtypes = [vp, vp, vp, vp, ctypes.POINTER(rc_state_t), vp, vp, ctypes.c_int]
    lib.rc_decompress_many.restype = st
    lib.rc_decompress_many.argtypes = [vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int]
    lib.rc_plan_destroy.restype = st
    lib.rc_plan_destroy.argtypes = [vp]
    lib.rc_plan_reset_state.restype = st
    lib.rc_plan_reset_state.argtypes = [vp, vp]
    for f in ("rc_packed_bytes", "rc_tensor_packed_bytes", "rc_workspace_bytes"):
        getattr(lib, f).restype = sz
        getattr(lib, f).argtypes = [vp]
    lib.rc_status_string.restype = ctypes.c_char_p
    lib.rc_status_string.argtypes = [ctypes.c_int]
    lib.rcx_lowrank_workspace.restype = ctypes.c_int
    lib.rcx_lowrank_r_probe.restype = ctypes.c_int
    lib.rcx_lowrank_r_probe.argtypes = [vp, ctypes.c_int, vp]
    lib.rcx_lowrank_workspace.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int]
    lib.rcx_device_to_host.restype = ctypes.c_int
    lib.rcx_device_to_host.argtypes = [vp, vp, sz]
    lib.rcx_hbm_probe.restype = ctypes.c_int
    lib.rcx_hbm_probe.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_int64, vp]
    return lib


_lib = _load()
lib = _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):  # numpy (host)
        return x.ctypes.data
    raise TypeError("cannot take a device pointer of %r" % type(x))


def _dev_buffer(x, nbytes, what):
    """Device pointer of x, checked when x is a tensor: on a GPU, contiguous and
    at least nbytes long (the kernels would otherwise read or write past it, or
    dereference host memory). Raw integers pass through unchecked."""
    if hasattr(x, "data_ptr") and hasattr(x, "is_cuda"):
        if not x.is_cuda:
            raise ValueError("%s must be a device tensor" % what)
        if not x.is_contiguous():
            raise ValueError("%s must be contiguous" % what)
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise ValueError("%s holds %d bytes, the call needs %d" % (what, have, nbytes))
    return _ptr(x)


def _sized(x, nbytes, what):
    """Pointer of x (device or pinned host), checked for size when x is a tensor."""
    if hasattr(x, "numel") and hasattr(x, "element_size"):
        have = x.numel() * x.element_size()
        if have < nbytes:
            raise ValueError("%s holds %d bytes, the call needs %d" % (what, have, nbytes))
    return _ptr(x)


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str):
    if status != RC_OK:
        raise RcError(status, where)


# ------------------------------------------------------------------ C names
def rc_status_string(status: int) -> str:
    return _lib.rc_status_string(int(status)).decode()


def rc_plan_create(shape, dtype, scheme, params: rc_params_t):
    """shape: rc_shape_t or (batch, rows, cols); dtype/scheme: enum ints or names."""
    if not isinstance(shape, rc_shape_t):
        shape = rc_shape_t(*shape)
    dtype = DTYPES.get(dtype, dtype)
    scheme = SCHEMES.get(scheme, scheme)
    plan = ctypes.c_void_p()
    _check(_lib.rc_plan_create(shape, int(dtype), int(scheme), ctypes.byref(params),
                               ctypes.byref(plan)), "rc_plan_create")
    return plan


def rc_compress(plan, stream, a_t, state: rc_state_t, packed_out):
    _check(_lib.rc_compress(plan, _stream(stream), _ptr(a_t), ctypes.byref(state), _ptr(packed_out)),
           "rc_compress")


RC_NOALLOC_SCRATCH_BYTES = 64 << 20


def rc_compress_lowrank_noalloc(shape, dtype, params: rc_params_t, stream, a_t, state: rc_state_t,
                                packed_out):
    """The plan-free, allocation-free low-rank sender step (librescomp.h)."""
    if not isinstance(shape, rc_shape_t):
        shape = rc_shape_t(*shape)
    _check(_lib.rc_compress_lowrank_noalloc(shape, int(DTYPES.get(dtype, dtype)), ctypes.byref(params),
                                            _stream(stream), _ptr(a_t), ctypes.byref(state),
                                            _ptr(packed_out)), "rc_compress_lowrank_noalloc")


def rc_decompress(plan, stream, packed_in, recon_state):
    _check(_lib.rc_decompress(plan, _stream(stream), _ptr(packed_in), _ptr(recon_state)),
           "rc_decompress")


def rc_compress_send(plan, stream, copy_stream, a_t, state: rc_state_t, packed_out, packed_dst,
                     chunk):
    _check(_lib.rc_compress_send(plan, _stream(stream), _stream(copy_stream), _ptr(a_t),
                                 ctypes.byref(state), _ptr(packed_out), _ptr(packed_dst), int(chunk)),
           "rc_compress_send")


def rc_decompress_many(plan, stream, packed_in, recon_states):
    """packed_in, recon_states: equal-length sequences (one entry per peer)."""
    n = len(packed_in)
    if n != len(recon_states):
        raise ValueError("one recon state per packed stream")
    pk = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in packed_in])
    rs = (ctypes.c_void_p * max(n, 1))(*[_ptr(x) for x in recon_states])
    _check(_lib.rc_decompress_many(plan, _stream(stream), pk, rs, n), "rc_decompress_many")


def rc_plan_reset_state(plan, stream):
    _check(_lib.rc_plan_reset_state(plan, _stream(stream)), "rc_plan_reset_state")


def rc_plan_destroy(plan):
    _check(_lib.rc_plan_destroy(plan), "rc_plan_destroy")


def rc_packed_bytes(plan) -> int:
    return int(_lib.rc_packed_bytes(plan))


def rc_tensor_packed_bytes(plan) -> int:
    return int(_lib.rc_tensor_packed_bytes(plan))


def rc_workspace_bytes(plan) -> int:
    return int(_lib.rc_workspace_bytes(plan))


def make_params(scheme, *, group=0, nm_keep=0, nm_block=0, rank=0, iters=0, seed=0, q0=None,
                flags=0, grid_w=0, keep_blocks=0):
    """rc_params_t for a scheme; q0 (device fp32 [batch][cols][rank], or None to
    draw the start matrices from `seed`) is referenced, not copied, so keep it
    alive until rc_plan_create returns."""
    p = rc_params_t(int(group), int(nm_keep), int(nm_block), int(rank), int(iters), int(seed),
                    _ptr(q0), int(flags), int(grid_w), int(keep_blocks))
    p._q0_ref = q0
    return p


RCX_PROBE_COPY, RCX_PROBE_READ, RCX_PROBE_WRITE, RCX_PROBE_SENDER_MIX, RCX_PROBE_RECEIVER_RMW = range(5)
RCX_R_PROBE_RQ, RCX_R_PROBE_RTP = 0, 1


def rcx_device_to_host(src, nbytes):
    """bytes at device address src, copied synchronously (librescomp_diag.h)."""
    import numpy as np
    out = np.empty(int(nbytes), np.uint8)
    err = _lib.rcx_device_to_host(out.ctypes.data, _ptr(src), int(nbytes))
    if err != 0:
        raise RuntimeError("rcx_device_to_host: hipError %d" % err)
    return out


def rcx_hbm_probe(kind, a, b, c, n, stream=None):
    """Launch one HBM reference kernel (librescomp_diag.h); raises on a HIP error."""
    err = _lib.rcx_hbm_probe(int(kind), _ptr(a), _ptr(b), _ptr(c), int(n), _stream(stream))
    if err != 0:
        raise RuntimeError("rcx_hbm_probe: hipError %d" % err)


# ------------------------------------------------------------------ convenience
class Plan:
    """Owns one rc_plan_t; a thin wrapper over the C calls above."""

    def __init__(self, shape, dtype, scheme, **params):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.scheme = scheme
        q0 = params.get("q0")
        if q0 is not None:
            want = self.shape[0] * self.shape[2] * int(params.get("rank", 0))
            size = q0.numel() if hasattr(q0, "numel") else int(getattr(q0, "size", -1))
            if SCHEMES.get(scheme, scheme) == RC_LOWRANK and size != want:
                # the library reads batch * cols * rank floats through the pointer
                raise ValueError("q0 holds %d floats; [batch][cols][rank] needs %d" % (size, want))
            if hasattr(q0, "data_ptr"):
                if not (q0.is_cuda and q0.is_contiguous()) or str(q0.dtype) != "torch.float32":
                    raise ValueError("q0 must be a contiguous fp32 device tensor")
            else:  # host array: a device copy for the plan's set-up
                import numpy as np
                import torch
                q0 = torch.from_numpy(np.ascontiguousarray(q0, dtype=np.float32)).to("cuda")
                torch.cuda.synchronize()
            params["q0"] = q0
        self._params = make_params(scheme, **params)
        self.handle = rc_plan_create(self.shape, dtype, scheme, self._params)
        self._params._q0_ref = None  # the plan has its own copy of the start matrices
        self.packed_bytes = rc_packed_bytes(self.handle)
        self.tensor_packed_bytes = rc_tensor_packed_bytes(self.handle)
        self.workspace_bytes = rc_workspace_bytes(self.handle)

    def _elems(self):
        return self.shape[0] * self.shape[1] * self.shape[2]

    def _in_bytes(self):
        return self._elems() * (2 if DTYPES.get(self.dtype, self.dtype) == RC_BF16 else 4)

    def _input(self, a_t):
        """a_t checked as _dev_buffer does, and for the plan's dtype (an fp32 tensor
        given to a bf16 plan would otherwise be read as pairs of bf16 values)."""
        if hasattr(a_t, "dtype") and hasattr(a_t, "data_ptr"):
            want = "torch.bfloat16" if DTYPES.get(self.dtype, self.dtype) == RC_BF16 else "torch.float32"
            if str(a_t.dtype) != want:
                raise ValueError("a_t is %s, the plan takes %s" % (a_t.dtype, want))
        return _dev_buffer(a_t, self._in_bytes(), "a_t")

    def compress(self, a_t, ahat, e, packed_out, stream=None):
        a = self._input(a_t)
        st = rc_state_t(_dev_buffer(ahat, 4 * self._elems(), "ahat"),
                        _dev_buffer(e, 4 * self._elems(), "e"))
        rc_compress(self.handle, stream, a, st,
                    _dev_buffer(packed_out, self.packed_bytes, "packed_out"))

    def decompress(self, packed_in, recon_state, stream=None):
        rc_decompress(self.handle, stream, _dev_buffer(packed_in, self.packed_bytes, "packed_in"),
                      _dev_buffer(recon_state, 4 * self._elems(), "recon_state"))

    def compress_send(self, a_t, ahat, e, packed_out, packed_dst, chunk, copy_stream, stream=None):
        a = self._input(a_t)
        st = rc_state_t(_dev_buffer(ahat, 4 * self._elems(), "ahat"),
                        _dev_buffer(e, 4 * self._elems(), "e"))
        rc_compress_send(self.handle, stream, copy_stream, a, st,
                         _dev_buffer(packed_out, self.packed_bytes, "packed_out"),
                         _sized(packed_dst, self.packed_bytes, "packed_dst"), chunk)

    def decompress_many(self, packed_in, recon_states, stream=None):
        rc_decompress_many(self.handle, stream,
                           [_dev_buffer(p, self.packed_bytes, "packed_in") for p in packed_in],
                           [_dev_buffer(r, 4 * self._elems(), "recon_state") for r in recon_states])

    def reset_state(self, stream=None):
        rc_plan_reset_state(self.handle, stream)

    def r_probe(self, pattern, stream=None):
        """Read this low-rank plan's R in the pattern of its R*Q (RCX_R_PROBE_RQ)
        or R^T*P (RCX_R_PROBE_RTP) pass and nothing else (librescomp_diag.h)."""
        err = _lib.rcx_lowrank_r_probe(self.handle, int(pattern), _stream(stream))
        if err != 0:
            raise RuntimeError("rcx_lowrank_r_probe: %d" % err)

    def lowrank_workspace(self):
        """Device pointers (R, P, Pbt, Qt, Q0t, Qtb, gsum, linv) and rows_pad (diagnostics)."""
        arr = (ctypes.c_void_p * 8)()
        rp = _lib.rcx_lowrank_workspace(self.handle, arr, 8)
        if rp < 0:
            raise ValueError("not a low-rank plan")
        return [int(v or 0) for v in arr], rp

    def close(self):
        if self.handle is not None:
            rc_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
