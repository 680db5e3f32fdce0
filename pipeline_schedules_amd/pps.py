"""Thin ctypes binding of libpps.so (C ABI in include/pps.h).

Argument marshalling only: every step of the stage runs in the library's HIP
kernels.  Device buffers are passed as raw addresses (``tensor.data_ptr()``);
PyTorch is used by callers for device memory and streams.  Loading fails
loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

# Import torch first so that libpps.so binds to the same HIP runtime instance
# that PyTorch uses (the two copies share a SONAME).
import torch  # noqa: F401

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpps.so")

OK, EINVAL, EFULL, EORDER, ENOENT, ESTATE, ENOMEM, EHIP, ETOOBIG = 0, -1, -2, -3, -4, -5, -6, -7, -8
NOALLOC_MAX_BYTES = 64 << 20
OP_F, OP_B, OP_W = 0, 1, 2
GPIPE, ONE_F_ONE_B, ZB1P, ZB2P = 0, 1, 2, 3
BLOCK_SWIGLU, BLOCK_TOY_GELU = 0, 1
DTYPE_BF16, DTYPE_FP32 = 0, 1
FLAG_BOOKKEEPING_ONLY, FLAG_PROFILE, FLAG_RECOMPUTE = 1, 2, 4

KIND_BY_NAME = {"gpipe": GPIPE, "1f1b": ONE_F_ONE_B, "zb1p": ZB1P, "zb2p": ZB2P}
DTYPE_BY_NAME = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}
BLOCK_BY_NAME = {"swiglu": BLOCK_SWIGLU, "toy": BLOCK_TOY_GELU}

EXPORTED = [
    "pps_make_schedule", "pps_stage_create", "pps_stage_create_noalloc", "pps_stage_forward", "pps_stage_backward",
    "pps_stage_backward_weight", "pps_stage_zero_grad", "pps_stage_get_grad", "pps_stage_sync",
    "pps_stage_get_stats", "pps_stage_get_oplog", "pps_stage_kernel_times", "pps_kernel_name",
    "pps_stage_destroy", "pps_strerror", "pps_scale", "pps_simulate_pipeline",
]


class PpsOp(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("mb", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("slot", ctypes.c_int32), ("inflight_after", ctypes.c_int32), ("t_start", ctypes.c_int32)]

    def as_tuple(self):
        return (self.op, self.mb, self.chunk, self.slot, self.inflight_after, self.t_start)


class PpsStageDesc(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("M", ctypes.c_int32), ("k", ctypes.c_int32), ("v", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("block_type", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("L", ctypes.c_int32), ("d", ctypes.c_int64), ("ffn", ctypes.c_int64), ("T", ctypes.c_int64),
                ("eps", ctypes.c_float), ("flags", ctypes.c_uint32), ("profile_capacity", ctypes.c_int32),
                ("profile_stride", ctypes.c_int32), ("stream", ctypes.c_void_p),
                ("weights", ctypes.POINTER(ctypes.c_void_p))]


class PpsStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_slots", "slot_bytes", "pool_bytes", "scratch_bytes", "grad_bytes", "live_entries", "live_bytes",
        "peak_live_entries", "peak_live_bytes", "n_forward", "n_backward", "n_backward_weight",
        "passes_completed")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class PpsKernelTime(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("reserved", ctypes.c_int32), ("launches", ctypes.c_int64),
                ("timed", ctypes.c_int64), ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class PpsError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {strerror(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if libpps.so is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libpps.so not built at {_LIB_PATH}; run `python -m pipeline_schedules_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.pps_make_schedule.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(PpsOp), i32, ctypes.POINTER(i32)]
        L.pps_stage_create.argtypes = [ctypes.POINTER(PpsStageDesc), ctypes.POINTER(vp)]
        L.pps_stage_create_noalloc.argtypes = [ctypes.POINTER(PpsStageDesc), ctypes.POINTER(vp)]
        L.pps_stage_forward.argtypes = [vp, i32, i32, vp, vp]
        L.pps_stage_backward.argtypes = [vp, i32, i32, vp, vp]
        L.pps_stage_backward_weight.argtypes = [vp, i32, i32]
        L.pps_stage_zero_grad.argtypes = [vp]
        L.pps_stage_get_grad.argtypes = [vp, i32, i32, i32, ctypes.POINTER(vp)]
        L.pps_stage_sync.argtypes = [vp]
        L.pps_stage_get_stats.argtypes = [vp, ctypes.POINTER(PpsStats)]
        L.pps_stage_get_oplog.argtypes = [vp, ctypes.POINTER(PpsOp), i32, ctypes.POINTER(i32)]
        L.pps_stage_kernel_times.argtypes = [vp, ctypes.POINTER(PpsKernelTime), i32, ctypes.POINTER(i32)]
        L.pps_kernel_name.argtypes = [i32]
        L.pps_kernel_name.restype = ctypes.c_char_p
        L.pps_stage_destroy.argtypes = [vp]
        L.pps_stage_destroy.restype = None
        L.pps_strerror.argtypes = [i32]
        L.pps_strerror.restype = ctypes.c_char_p
        L.pps_scale.argtypes = [vp, vp, i64, ctypes.c_float, i32, vp]
        dbl = ctypes.c_double
        L.pps_simulate_pipeline.argtypes = [i32, i32, i32, i32, dbl, dbl, dbl, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
        for name in EXPORTED:
            if name not in ("pps_kernel_name", "pps_stage_destroy", "pps_strerror"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(status):
    return lib().pps_strerror(int(status)).decode()


def kernel_name(k):
    return lib().pps_kernel_name(int(k)).decode()


def _check(status, what):
    if status != OK:
        raise PpsError(status, what)


def make_schedule(P, M, k, v=1, kind=ONE_F_ONE_B):
    """Op list of stage k: list of (op, mb, chunk, slot, inflight_after, t_start)."""
    n = ctypes.c_int(0)
    st = lib().pps_make_schedule(P, M, k, v, kind, None, 0, ctypes.byref(n))
    if st not in (OK, EFULL):
        raise PpsError(st, "pps_make_schedule")
    arr = (PpsOp * max(n.value, 1))()
    _check(lib().pps_make_schedule(P, M, k, v, kind, arr, n.value, ctypes.byref(n)), "pps_make_schedule")
    return [arr[i].as_tuple() for i in range(n.value)]


def simulate_pipeline(P, M, v, kind, t_f, t_b, t_w=0.0):
    """(makespan, bubble) of all P stages running ``kind`` with per-op
    durations t_f, t_b (and t_w for the ZB kinds)."""
    mk = ctypes.c_double(0.0)
    bu = ctypes.c_double(0.0)
    _check(lib().pps_simulate_pipeline(P, M, v, kind, float(t_f), float(t_b), float(t_w), ctypes.byref(mk),
                                       ctypes.byref(bu)), "pps_simulate_pipeline")
    return mk.value, bu.value


def scale(dst, src, n, factor, dtype, stream=None):
    """dst = src * factor on the device (n elements)."""
    st = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
    _check(lib().pps_scale(_ptr(dst), _ptr(src), int(n), float(factor), int(dtype), st), "pps_scale")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


class Stage:
    """One pipeline stage handle (pps_stage)."""

    def __init__(self, P, M, k, v=1, kind=ONE_F_ONE_B, block=BLOCK_SWIGLU, dtype=DTYPE_BF16, L=1,
                 d=64, ffn=64, T=8, eps=1e-6, weights=None, stream=None, flags=0, profile_capacity=0,
                 noalloc=False, profile_stride=0):
        self._h = None
        nw = 4 if block == BLOCK_SWIGLU else 2
        desc = PpsStageDesc()
        desc.P, desc.M, desc.k, desc.v, desc.kind = P, M, k, v, kind
        desc.block_type, desc.dtype, desc.L = block, dtype, L
        desc.d, desc.ffn, desc.T, desc.eps = d, ffn, T, eps
        desc.flags, desc.profile_capacity, desc.profile_stride = flags, profile_capacity, profile_stride
        desc.stream = stream if isinstance(stream, int) or stream is None else stream.cuda_stream
        self._keep = weights
        if weights is not None:
            flat = [_ptr(w) for w in weights]
            if len(flat) != v * L * nw:
                raise ValueError(f"expected {v * L * nw} weight pointers, got {len(flat)}")
            self._warr = (ctypes.c_void_p * len(flat))(*flat)
            desc.weights = ctypes.cast(self._warr, ctypes.POINTER(ctypes.c_void_p))
        else:
            desc.weights = None
        h = ctypes.c_void_p()
        fn = "pps_stage_create_noalloc" if noalloc else "pps_stage_create"
        _check(getattr(lib(), fn)(ctypes.byref(desc), ctypes.byref(h)), fn)
        self._h = h
        self.desc = desc

    def close(self):
        if self._h is not None:
            lib().pps_stage_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # raw calls (return the status code)
    def forward_status(self, mb, chunk, x, y):
        return lib().pps_stage_forward(self._h, mb, chunk, _ptr(x), _ptr(y))

    def backward_status(self, mb, chunk, dy, dx):
        return lib().pps_stage_backward(self._h, mb, chunk, _ptr(dy), _ptr(dx))

    def backward_weight_status(self, mb, chunk=0):
        return lib().pps_stage_backward_weight(self._h, mb, chunk)

    # checked calls
    def forward(self, mb, chunk, x, y):
        _check(self.forward_status(mb, chunk, x, y), "pps_stage_forward")

    def backward(self, mb, chunk, dy, dx):
        _check(self.backward_status(mb, chunk, dy, dx), "pps_stage_backward")

    def backward_weight(self, mb, chunk=0):
        _check(self.backward_weight_status(mb, chunk), "pps_stage_backward_weight")

    def zero_grad(self):
        _check(lib().pps_stage_zero_grad(self._h), "pps_stage_zero_grad")

    def sync(self):
        _check(lib().pps_stage_sync(self._h), "pps_stage_sync")

    def grad_ptr(self, chunk, block, which):
        p = ctypes.c_void_p()
        _check(lib().pps_stage_get_grad(self._h, chunk, block, which, ctypes.byref(p)), "pps_stage_get_grad")
        return p.value

    def grad(self, chunk, block, which, shape):
        """Copy a gradient buffer into a new fp32 torch tensor on the current device.  The copy
        runs on the caller's current stream once the stage's stream has finished, so later work on
        that stream sees it (a synchronous device-to-device hipMemcpy is not ordered with a
        non-default stream)."""
        import torch
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        self.sync()
        src = self.grad_ptr(chunk, block, which)
        rc = _hip().hipMemcpyAsync(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(src),
                                   ctypes.c_size_t(out.numel() * 4), 3,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync of a gradient failed (hipError {rc})")
        return out

    def stats(self):
        s = PpsStats()
        _check(lib().pps_stage_get_stats(self._h, ctypes.byref(s)), "pps_stage_get_stats")
        return s.as_dict()

    def oplog(self):
        n = ctypes.c_int(0)
        st = lib().pps_stage_get_oplog(self._h, None, 0, ctypes.byref(n))
        if st not in (OK, EFULL):
            raise PpsError(st, "pps_stage_get_oplog")
        arr = (PpsOp * max(n.value, 1))()
        _check(lib().pps_stage_get_oplog(self._h, arr, n.value, ctypes.byref(n)), "pps_stage_get_oplog")
        return [arr[i].as_tuple() for i in range(n.value)]

    def kernel_times(self):
        arr = (PpsKernelTime * 32)()
        n = ctypes.c_int(0)
        _check(lib().pps_stage_kernel_times(self._h, arr, 32, ctypes.byref(n)), "pps_stage_kernel_times")
        return [{"kernel": arr[i].kernel, "name": kernel_name(arr[i].kernel), "launches": arr[i].launches,
                 "timed": arr[i].timed, "total_ms": arr[i].total_ms, "flops": arr[i].flops, "bytes": arr[i].bytes}
                for i in range(n.value)]


_hiplib = None


def _hip():
    """The HIP runtime already loaded in this process (the one torch uses)."""
    global _hiplib
    if _hiplib is None:
        _hiplib = ctypes.CDLL("libamdhip64.so.7", mode=ctypes.RTLD_GLOBAL | os.RTLD_NOLOAD) \
            if hasattr(os, "RTLD_NOLOAD") else ctypes.CDLL("libamdhip64.so.7")
        _hiplib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                           ctypes.c_void_p]
        _hiplib.hipMemcpyAsync.restype = ctypes.c_int
    return _hiplib


def stage_from_config(cfg, weights=None, stream=None, flags=0, profile_capacity=0, k=None, T=None, M=None,
                      kind=None, noalloc=False, profile_stride=0):
    """Stage handle for a ``configs.StageConfig`` (optionally overriding k, T, M, kind)."""
    return Stage(P=cfg.P, M=cfg.M if M is None else M, k=cfg.k if k is None else k, v=cfg.v,
                 kind=KIND_BY_NAME[cfg.kind if kind is None else kind], block=BLOCK_BY_NAME[cfg.block],
                 dtype=DTYPE_BY_NAME[cfg.dtype], L=cfg.L, d=cfg.d, ffn=cfg.f, T=cfg.T if T is None else T,
                 eps=cfg.eps, weights=weights, stream=stream, flags=flags, profile_capacity=profile_capacity,
                 noalloc=noalloc, profile_stride=profile_stride)
