"""Thin Python binding of the C ABI in ``include/ssd.h`` (argument marshalling only).

The functions named like the C entry points (``ssd_fwd``, ``ssd_bwd``,
``ssd_state_moments``, ``ssd_state_moments_bwd``, ``ssd_workspace_size``,
``ssd_last_error``) take torch tensors (or ``None`` for nullable pointers),
check that each one is a contiguous tensor of the right dtype, device and
element count for ``dims`` -- so that a wrong buffer is refused on the host
instead of faulting on the GPU -- pass the raw pointers and return the C status
code.  ``forward``, ``backward``, ``state_moments`` and ``state_moments_bwd``
allocate outputs and workspace with torch and raise :class:`SsdError` on a
nonzero status.  Every step of the computation runs in the HIP library; there
is no Python or CPU fallback, and importing a function whose library is missing
raises immediately.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libmamba_ssd_hip.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_OP_FWD, SSD_OP_BWD, SSD_OP_MOMENTS, SSD_OP_MOMENTS_BWD = 0, 1, 2, 3
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
          4: "SSD_ERR_DTYPE", 5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_HIP", 7: "SSD_ERR_NONFINITE"}
EXPORTS = ("ssd_workspace_size", "ssd_fwd", "ssd_fwd_noalloc", "ssd_bwd", "ssd_state_moments",
           "ssd_state_moments_bwd", "ssd_moments_pr", "ssd_moments_pr_bwd", "ssd_y_diag",
           "ssd_y_diag_bwd", "ssd_quat_scan", "ssd_quat_scan_bwd", "ssd_quat_workspace_size",
           "ssd_step", "ssd_last_error", "ssd_debug_enable", "ssd_timing_enable",
           "ssd_timing_collect", "ssd_bwd_partial_region", "ssd_stream_probe")


class ssd_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nchunks", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("kernel_chunk_len", ctypes.c_int32)]

    def __repr__(self):
        return ("ssd_dims(b=%d, n=%d, l=%d, h=%d, p=%d, r=%d, io=%d, kernel_chunk_len=%d)" %
                (self.batch, self.nchunks, self.chunk_len, self.nheads, self.headdim,
                 self.dstate, self.io_dtype, self.kernel_chunk_len))


class SsdError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP library {path} is missing: build it with "
                          "`python -m mamba_ssd_chunked_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(ssd_dims)
    lib.ssd_workspace_size.argtypes = [D, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_fwd.argtypes = [D] + [P] * 10 + [ctypes.c_size_t, P]
    lib.ssd_fwd_noalloc.argtypes = [D] + [P] * 10
    lib.ssd_bwd.argtypes = [D] + [P] * 17 + [ctypes.c_size_t, P]
    lib.ssd_state_moments.argtypes = [D] + [P] * 14 + [ctypes.c_size_t, P]
    lib.ssd_state_moments_bwd.argtypes = [D] + [P] * 14 + [ctypes.c_size_t, P]
    I64 = ctypes.c_int64
    lib.ssd_moments_pr.argtypes = [I64, I64, I64, P, P, P, ctypes.c_int, P, P, P]
    lib.ssd_moments_pr_bwd.argtypes = [I64, I64, I64, P, P, P, P, ctypes.c_int, P, P, P]
    lib.ssd_y_diag.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 6
    lib.ssd_y_diag_bwd.argtypes = [I64] * 5 + [ctypes.c_int] + [P] * 10
    lib.ssd_quat_scan.argtypes = [I64] * 4 + [P] * 4 + [ctypes.c_size_t, P]
    lib.ssd_quat_scan_bwd.argtypes = [I64] * 4 + [P] * 6 + [ctypes.c_size_t, P]
    lib.ssd_quat_workspace_size.argtypes = [I64] * 4 + [ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_step.argtypes = [I64] * 4 + [ctypes.c_int] + [P] * 10
    for f in ("ssd_workspace_size", "ssd_fwd", "ssd_fwd_noalloc", "ssd_bwd", "ssd_state_moments",
              "ssd_state_moments_bwd", "ssd_moments_pr", "ssd_moments_pr_bwd", "ssd_y_diag",
              "ssd_y_diag_bwd", "ssd_quat_scan", "ssd_quat_scan_bwd", "ssd_quat_workspace_size", "ssd_step"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_debug_enable.argtypes = [ctypes.c_int]
    lib.ssd_debug_enable.restype = ctypes.c_int
    lib.ssd_timing_enable.argtypes = [ctypes.c_int]
    lib.ssd_timing_enable.restype = ctypes.c_int
    lib.ssd_timing_collect.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t,
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int)]
    lib.ssd_timing_collect.restype = ctypes.c_int
    lib.ssd_bwd_partial_region.argtypes = [D, ctypes.c_char_p, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_bwd_partial_region.restype = ctypes.c_int
    lib.ssd_stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int64, P]
    lib.ssd_stream_probe.restype = ctypes.c_int
    _lib = lib
    return lib


# ------------------------------------------------------------------ marshalling
def make_dims(batch, nchunks, chunk_len, nheads, headdim, dstate, io_dtype=SSD_F32,
              kernel_chunk_len=0) -> ssd_dims:
    return ssd_dims(int(batch), int(nchunks), int(chunk_len), int(nheads), int(headdim),
                    int(dstate), int(io_dtype), int(kernel_chunk_len))


def dims_of(x: torch.Tensor, B: torch.Tensor, kernel_chunk_len: int = 0) -> ssd_dims:
    """dims from x ``[b, n, l, h, p]`` and B ``[b, n, l, h, r]``."""
    b, n, l, h, p = x.shape
    io_dtype = SSD_BF16 if x.dtype == torch.bfloat16 else SSD_F32
    return make_dims(b, n, l, h, p, B.shape[-1], io_dtype, kernel_chunk_len)


def _io_dtype(d: ssd_dims):
    return torch.bfloat16 if d.io_dtype == SSD_BF16 else torch.float32


def _sizes(d: ssd_dims):
    b, n, l, h, p, r = d.batch, d.nchunks, d.chunk_len, d.nheads, d.headdim, d.dstate
    return dict(tok_p=b * n * l * h * p, tok_r=b * n * l * h * r, dt=b * h * n * l, head=h,
                state=b * h * p * r, m2=b * h * r * r, m1=b * h * r, batch=b)


def _ptr(t: Optional[torch.Tensor], name: str, dtype, numel: int, required: bool):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, dims need {numel}")
    if dtype == torch.int64:
        if t.device.type != "cpu":
            raise ValueError(f"{name} must be a host (CPU) tensor")
    elif t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr()) if numel > 0 else ctypes.c_void_p(t.data_ptr() or 0)


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


# ------------------------------------------------------------ C-named functions
def ssd_last_error() -> str:
    return load_library().ssd_last_error().decode()


def ssd_debug_enable(on: bool) -> int:
    """Debug mode: the SSD and moments entry points check their outputs for NaN / inf
    (synchronising) and return SSD_ERR_NONFINITE when they find one."""
    return load_library().ssd_debug_enable(1 if on else 0)


def ssd_timing_enable(on: bool) -> int:
    return load_library().ssd_timing_enable(1 if on else 0)


def ssd_timing_collect(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} of the launches timed since the last call."""
    stride = 64
    names = ctypes.create_string_buffer(max_kernels * stride)
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int64 * max_kernels)()
    n = ctypes.c_int(0)
    rc = load_library().ssd_timing_collect(max_kernels, names, stride, ms, cnt, ctypes.byref(n))
    if rc:
        raise SsdError(rc, "ssd_timing_collect", ssd_last_error())
    out = {}
    for k in range(min(n.value, max_kernels)):
        nm = names.raw[k * stride:(k + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (float(ms[k]), int(cnt[k]))
    return out


def ssd_stream_probe(reads: int, writes: int, nontemporal: bool, src: torch.Tensor,
                     dst: torch.Tensor, n16: int, stream=None) -> int:
    """Benchmark instrumentation: one streaming launch over `reads` source and `writes`
    destination arrays of n16 16-byte elements (src / dst: contiguous fp32 device tensors of
    exactly 4 * reads * n16 and 4 * max(writes, 1) * n16 elements; src may be None when
    reads = 0)."""
    ps = _ptr(src, "src", torch.float32, 4 * reads * n16, reads > 0)
    pd = _ptr(dst, "dst", torch.float32, 4 * max(writes, 1) * n16, True)
    return load_library().ssd_stream_probe(int(reads), int(writes), 1 if nontemporal else 0, ps, pd,
                                           int(n16), _stream(stream))


def ssd_workspace_size(dims: ssd_dims, op: int) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().ssd_workspace_size(ctypes.byref(dims), int(op), ctypes.byref(out))
    if rc:
        raise SsdError(rc, "ssd_workspace_size", ssd_last_error())
    return int(out.value)


def ssd_bwd_partial_region(dims: ssd_dims, name: str):
    """(byte offset, bytes) of one of ssd_bwd's per-token partials ("g1", "g2", "d_delta")
    in its workspace; bytes 0 where the backward does not write it for these dims."""
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = load_library().ssd_bwd_partial_region(ctypes.byref(dims), name.encode(), ctypes.byref(off),
                                               ctypes.byref(n))
    if rc:
        raise SsdError(rc, "ssd_bwd_partial_region", ssd_last_error())
    return int(off.value), int(n.value)


def ssd_fwd(dims, x, dt, A, B, C, D, init, y, final_state, ws, stream=None) -> int:
    s, io, f = _sizes(dims), _io_dtype(dims), torch.float32
    args = [_ptr(x, "x", io, s["tok_p"], True), _ptr(dt, "dt", f, s["dt"], True),
            _ptr(A, "A", f, s["head"], True), _ptr(B, "B", io, s["tok_r"], True),
            _ptr(C, "C", io, s["tok_r"], True), _ptr(D, "D", f, s["head"], True),
            _ptr(init, "init", f, s["state"], False), _ptr(y, "y", io, s["tok_p"], True),
            _ptr(final_state, "final_state", f, s["state"], False)]
    wp, wb = _ws(ws)
    return load_library().ssd_fwd(ctypes.byref(dims), *args, wp, wb, _stream(stream))


# bytes of the library's fixed scratch array (SSD_NOALLOC_SCRATCH_BYTES in include/ssd.h)
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def ssd_fwd_noalloc(dims, x, dt, A, B, C, D, init, y, final_state, stream=None) -> int:
    """ssd_fwd without a workspace: the library's fixed per-GPU scratch array stands in
    for it (problems needing more than NOALLOC_SCRATCH_BYTES return SSD_ERR_WORKSPACE)."""
    s, io, f = _sizes(dims), _io_dtype(dims), torch.float32
    args = [_ptr(x, "x", io, s["tok_p"], True), _ptr(dt, "dt", f, s["dt"], True),
            _ptr(A, "A", f, s["head"], True), _ptr(B, "B", io, s["tok_r"], True),
            _ptr(C, "C", io, s["tok_r"], True), _ptr(D, "D", f, s["head"], True),
            _ptr(init, "init", f, s["state"], False), _ptr(y, "y", io, s["tok_p"], True),
            _ptr(final_state, "final_state", f, s["state"], False)]
    return load_library().ssd_fwd_noalloc(ctypes.byref(dims), *args, _stream(stream))


def ssd_bwd(dims, dy, d_final, x, dt, A, B, C, D, init, d_x, d_dt, d_A, d_B, d_C, d_D, d_init,
            ws, stream=None) -> int:
    s, io, f = _sizes(dims), _io_dtype(dims), torch.float32
    args = [_ptr(dy, "dy", io, s["tok_p"], True), _ptr(d_final, "d_final", f, s["state"], False),
            _ptr(x, "x", io, s["tok_p"], True), _ptr(dt, "dt", f, s["dt"], True),
            _ptr(A, "A", f, s["head"], True), _ptr(B, "B", io, s["tok_r"], True),
            _ptr(C, "C", io, s["tok_r"], True), _ptr(D, "D", f, s["head"], True),
            _ptr(init, "init", f, s["state"], False), _ptr(d_x, "d_x", io, s["tok_p"], True),
            _ptr(d_dt, "d_dt", f, s["dt"], True), _ptr(d_A, "d_A", f, s["head"], True),
            _ptr(d_B, "d_B", io, s["tok_r"], True), _ptr(d_C, "d_C", io, s["tok_r"], True),
            _ptr(d_D, "d_D", f, s["head"], True), _ptr(d_init, "d_init", f, s["state"], False)]
    wp, wb = _ws(ws)
    return load_library().ssd_bwd(ctypes.byref(dims), *args, wp, wb, _stream(stream))


def ssd_state_moments(dims, x, dt, A, B, init, valid_len, m2, m1, count, y, C, D, final_state,
                      ws, stream=None) -> int:
    s, io, f = _sizes(dims), _io_dtype(dims), torch.float32
    args = [_ptr(x, "x", io, s["tok_p"], True), _ptr(dt, "dt", f, s["dt"], True),
            _ptr(A, "A", f, s["head"], True), _ptr(B, "B", io, s["tok_r"], True),
            _ptr(init, "init", f, s["state"], False),
            _ptr(valid_len, "valid_len", torch.int64, s["batch"], False),
            _ptr(m2, "m2", f, s["m2"], True), _ptr(m1, "m1", f, s["m1"], True),
            _ptr(count, "count", torch.int64, s["batch"], True),
            _ptr(y, "y", io, s["tok_p"], False), _ptr(C, "C", io, s["tok_r"], False),
            _ptr(D, "D", f, s["head"], False),
            _ptr(final_state, "final_state", f, s["state"], False)]
    wp, wb = _ws(ws)
    return load_library().ssd_state_moments(ctypes.byref(dims), *args, wp, wb, _stream(stream))


def ssd_state_moments_bwd(dims, d_m2, d_m1, x, dt, A, B, init, valid_len, d_x, d_dt, d_A, d_B,
                          d_init, ws, stream=None) -> int:
    s, io, f = _sizes(dims), _io_dtype(dims), torch.float32
    args = [_ptr(d_m2, "d_m2", f, s["m2"], True), _ptr(d_m1, "d_m1", f, s["m1"], False),
            _ptr(x, "x", io, s["tok_p"], True), _ptr(dt, "dt", f, s["dt"], True),
            _ptr(A, "A", f, s["head"], True), _ptr(B, "B", io, s["tok_r"], True),
            _ptr(init, "init", f, s["state"], False),
            _ptr(valid_len, "valid_len", torch.int64, s["batch"], False),
            _ptr(d_x, "d_x", io, s["tok_p"], True), _ptr(d_dt, "d_dt", f, s["dt"], True),
            _ptr(d_A, "d_A", f, s["head"], True), _ptr(d_B, "d_B", io, s["tok_r"], True),
            _ptr(d_init, "d_init", f, s["state"], False)]
    wp, wb = _ws(ws)
    return load_library().ssd_state_moments_bwd(ctypes.byref(dims), *args, wp, wb,
                                                _stream(stream))


def ssd_moments_pr(batch, nheads, dstate, m2, m1, count, center, pr, trace, stream=None) -> int:
    f, bh = torch.float32, batch * nheads
    args = [_ptr(m2, "m2", f, bh * dstate * dstate, True),
            _ptr(m1, "m1", f, bh * dstate, bool(center)),
            _ptr(count, "count", torch.int64, batch, True)]
    outs = [_ptr(pr, "pr", f, bh, True), _ptr(trace, "trace", f, bh, False)]
    return load_library().ssd_moments_pr(batch, nheads, dstate, *args, int(bool(center)), *outs,
                                         _stream(stream))


def ssd_moments_pr_bwd(batch, nheads, dstate, d_pr, m2, m1, count, center, d_m2, d_m1,
                       stream=None) -> int:
    f, bh = torch.float32, batch * nheads
    args = [_ptr(d_pr, "d_pr", f, bh, True), _ptr(m2, "m2", f, bh * dstate * dstate, True),
            _ptr(m1, "m1", f, bh * dstate, bool(center)),
            _ptr(count, "count", torch.int64, batch, True)]
    outs = [_ptr(d_m2, "d_m2", f, bh * dstate * dstate, True),
            _ptr(d_m1, "d_m1", f, bh * dstate, False)]
    return load_library().ssd_moments_pr_bwd(batch, nheads, dstate, *args, int(bool(center)),
                                             *outs, _stream(stream))


def _diag_sizes(v: torch.Tensor, B: torch.Tensor):
    """(tokens, m, h, p, r, io dtype) of v [..., m, h, p] and B [..., m, h, r]."""
    if v.dim() < 3 or B.dim() != v.dim() or B.shape[:-1] != v.shape[:-1]:
        raise ValueError("v must be [..., m, h, p] and B [..., m, h, r] over the same leading axes")
    m, h, p = v.shape[-3:]
    T = math.prod(v.shape[:-3])
    io = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}.get(v.dtype)
    if io is None:
        raise TypeError(f"v must be float32 or bfloat16 (got {v.dtype})")
    return T, m, h, p, B.shape[-1], io


def ssd_y_diag(v, B, C, gamma, y_diag, stream=None) -> int:
    T, m, h, p, r, io = _diag_sizes(v, B)
    dt = v.dtype
    args = [_ptr(v, "v", dt, T * m * h * p, True), _ptr(B, "B", dt, T * m * h * r, True),
            _ptr(C, "C", dt, T * m * h * r, True), _ptr(gamma, "gamma", torch.float32, T * h, True),
            _ptr(y_diag, "y_diag", dt, T * m * h * p, True)]
    return load_library().ssd_y_diag(T, m, h, p, r, io, *args, _stream(stream))


def ssd_y_diag_bwd(dy, v, B, C, gamma, d_v, d_B, d_C, d_gamma, stream=None) -> int:
    T, m, h, p, r, io = _diag_sizes(v, B)
    dt, f = v.dtype, torch.float32
    args = [_ptr(dy, "dy", dt, T * m * h * p, True), _ptr(v, "v", dt, T * m * h * p, True),
            _ptr(B, "B", dt, T * m * h * r, True), _ptr(C, "C", dt, T * m * h * r, True),
            _ptr(gamma, "gamma", f, T * h, True), _ptr(d_v, "d_v", dt, T * m * h * p, True),
            _ptr(d_B, "d_B", dt, T * m * h * r, True), _ptr(d_C, "d_C", dt, T * m * h * r, True),
            _ptr(d_gamma, "d_gamma", f, T * h, True)]
    return load_library().ssd_y_diag_bwd(T, m, h, p, r, io, *args, _stream(stream))


def _quat_sizes(q: torch.Tensor):
    """(b, s, h, j) of q ``[b, s, h, j, 4]``."""
    if q.dim() != 5 or q.shape[-1] != 4:
        raise ValueError("q must be [b, s, h, j, 4]")
    return tuple(int(v) for v in q.shape[:4])


def ssd_quat_workspace_size(batch, seq, nheads, nquat, bwd) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().ssd_quat_workspace_size(batch, seq, nheads, nquat, int(bool(bwd)),
                                                ctypes.byref(n))
    if rc != 0:
        raise SsdError(rc, "ssd_quat_workspace_size", ssd_last_error())
    return n.value


def ssd_quat_scan(q, init, cum, ws, stream=None) -> int:
    b, s, h, j = _quat_sizes(q)
    f = torch.float32
    w, nbytes = _ws(ws)
    args = [_ptr(q, "q", f, b * s * h * j * 4, True), _ptr(init, "init", f, b * h * j * 4, False),
            _ptr(cum, "cum", f, b * s * h * j * 4, True)]
    return load_library().ssd_quat_scan(b, s, h, j, *args, w, nbytes, _stream(stream))


def ssd_quat_scan_bwd(q, init, d_cum, d_q, d_init, ws, stream=None) -> int:
    b, s, h, j = _quat_sizes(q)
    f = torch.float32
    w, nbytes = _ws(ws)
    args = [_ptr(q, "q", f, b * s * h * j * 4, True), _ptr(init, "init", f, b * h * j * 4, False),
            _ptr(d_cum, "d_cum", f, b * s * h * j * 4, True),
            _ptr(d_q, "d_q", f, b * s * h * j * 4, True),
            _ptr(d_init, "d_init", f, b * h * j * 4, False)]
    return load_library().ssd_quat_scan_bwd(b, s, h, j, *args, w, nbytes, _stream(stream))


def ssd_step(x, dt, A, B, C, D, state, new_state, y, stream=None) -> int:
    """x ``[b, h, p]``, dt ``[b, h]``, B/C ``[b, h, r]``, state/new_state ``[b, h, p, r]``
    (new_state may be state itself), y like x."""
    if x.dim() != 3 or B.dim() != 3 or B.shape[:2] != x.shape[:2]:
        raise ValueError("x must be [b, h, p] and B [b, h, r]")
    b, h, p = x.shape
    r = B.shape[-1]
    io = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}.get(x.dtype)
    if io is None:
        raise TypeError(f"x must be float32 or bfloat16 (got {x.dtype})")
    dt_, f = x.dtype, torch.float32
    args = [_ptr(x, "x", dt_, b * h * p, True), _ptr(dt, "dt", f, b * h, True),
            _ptr(A, "A", f, h, True), _ptr(B, "B", dt_, b * h * r, True),
            _ptr(C, "C", dt_, b * h * r, True), _ptr(D, "D", f, h, True),
            _ptr(state, "state", f, b * h * p * r, True),
            _ptr(new_state, "new_state", f, b * h * p * r, True), _ptr(y, "y", dt_, b * h * p, True)]
    return load_library().ssd_step(b, h, p, r, io, *args, _stream(stream))


# ------------------------------------------------------------ allocating helpers
def _check(rc: int, where: str):
    if rc != 0:
        raise SsdError(rc, where, ssd_last_error())


def workspace(dims: ssd_dims, op: int, device="cuda") -> torch.Tensor:
    n = ssd_workspace_size(dims, op)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def forward(x, dt, A, B, C, D, init=None, want_final=True, ws=None, stream=None,
            kernel_chunk_len=0):
    """y, final_state = SSD(x, dt, A, B, C, D, init)."""
    d = dims_of(x, B, kernel_chunk_len)
    y = torch.empty_like(x)
    final = torch.empty((d.batch, d.nheads, d.headdim, d.dstate), device=x.device,
                        dtype=torch.float32) if want_final else None
    ws = workspace(d, SSD_OP_FWD, x.device) if ws is None else ws
    _check(ssd_fwd(d, x, dt, A, B, C, D, init, y, final, ws, stream), "ssd_fwd")
    return y, final


def backward(dy, x, dt, A, B, C, D, init=None, d_final=None, want_d_init=True, ws=None,
             stream=None, kernel_chunk_len=0):
    """Returns dict(d_x, d_dt, d_A, d_B, d_C, d_D, d_init)."""
    d = dims_of(x, B, kernel_chunk_len)
    out = dict(d_x=torch.empty_like(x), d_dt=torch.empty_like(dt), d_A=torch.empty_like(A),
               d_B=torch.empty_like(B), d_C=torch.empty_like(C), d_D=torch.empty_like(D),
               d_init=torch.empty((d.batch, d.nheads, d.headdim, d.dstate), device=x.device,
                                  dtype=torch.float32) if want_d_init else None)
    ws = workspace(d, SSD_OP_BWD, x.device) if ws is None else ws
    _check(ssd_bwd(d, dy, d_final, x, dt, A, B, C, D, init, out["d_x"], out["d_dt"], out["d_A"],
                   out["d_B"], out["d_C"], out["d_D"], out["d_init"], ws, stream), "ssd_bwd")
    return out


def state_moments(x, dt, A, B, init=None, valid_len=None, C=None, D=None, want_y=False,
                  want_final=False, ws=None, stream=None, kernel_chunk_len=0):
    """Returns dict(m2, m1, count[, y][, final_state])."""
    d = dims_of(x, B, kernel_chunk_len)
    dev = x.device
    out = dict(m2=torch.empty((d.batch, d.nheads, d.dstate, d.dstate), device=dev),
               m1=torch.empty((d.batch, d.nheads, d.dstate), device=dev),
               count=torch.empty((d.batch,), dtype=torch.int64))
    y = torch.empty_like(x) if want_y else None
    fin = torch.empty((d.batch, d.nheads, d.headdim, d.dstate), device=dev) if want_final else None
    if valid_len is not None and not isinstance(valid_len, torch.Tensor):
        valid_len = torch.tensor(list(valid_len), dtype=torch.int64)
    ws = workspace(d, SSD_OP_MOMENTS, dev) if ws is None else ws
    _check(ssd_state_moments(d, x, dt, A, B, init, valid_len, out["m2"], out["m1"], out["count"],
                             y, C, D, fin, ws, stream), "ssd_state_moments")
    if want_y:
        out["y"] = y
    if want_final:
        out["final_state"] = fin
    return out


def state_moments_bwd(d_m2, x, dt, A, B, init=None, valid_len=None, d_m1=None, want_d_init=True,
                      ws=None, stream=None, kernel_chunk_len=0):
    """Returns dict(d_x, d_dt, d_A, d_B, d_init)."""
    d = dims_of(x, B, kernel_chunk_len)
    dev = x.device
    out = dict(d_x=torch.empty_like(x), d_dt=torch.empty_like(dt), d_A=torch.empty_like(A),
               d_B=torch.empty_like(B),
               d_init=torch.empty((d.batch, d.nheads, d.headdim, d.dstate), device=dev)
               if want_d_init else None)
    if valid_len is not None and not isinstance(valid_len, torch.Tensor):
        valid_len = torch.tensor(list(valid_len), dtype=torch.int64)
    ws = workspace(d, SSD_OP_MOMENTS_BWD, dev) if ws is None else ws
    _check(ssd_state_moments_bwd(d, d_m2, d_m1, x, dt, A, B, init, valid_len, out["d_x"],
                                 out["d_dt"], out["d_A"], out["d_B"], out["d_init"], ws, stream),
           "ssd_state_moments_bwd")
    return out


def _count_tensor(count, batch):
    if not isinstance(count, torch.Tensor):
        count = torch.tensor(list(count) if hasattr(count, "__len__") else [count] * batch,
                             dtype=torch.int64)
    return count.to(torch.int64).contiguous()


def moments_pr(m2, m1, count, center=False, stream=None):
    """Participation ratio and raw trace of pooled moments: returns ``(pr, trace)``,
    each ``[b, h]`` fp32.  m2 ``[b, h, r, r]``, m1 ``[b, h, r]`` (device), count host
    int64 ``[b]`` (or one int for every row)."""
    b, h, r, _ = m2.shape
    count = _count_tensor(count, b)
    pr = torch.empty((b, h), device=m2.device)
    trace = torch.empty((b, h), device=m2.device)
    _check(ssd_moments_pr(b, h, r, m2, m1 if center else None, count, center, pr, trace, stream),
           "ssd_moments_pr")
    return pr, trace


def moments_pr_bwd(d_pr, m2, m1, count, center=False, want_d_m1=True, stream=None):
    """Gradient of ``<d_pr, PR>``: returns ``(d_m2, d_m1)`` (d_m1 None unless wanted)."""
    b, h, r, _ = m2.shape
    count = _count_tensor(count, b)
    d_m2 = torch.empty_like(m2)
    d_m1 = torch.empty((b, h, r), device=m2.device) if want_d_m1 else None
    _check(ssd_moments_pr_bwd(b, h, r, d_pr, m2, m1 if center else None, count, center, d_m2,
                              d_m1, stream), "ssd_moments_pr_bwd")
    return d_m2, d_m1


def y_diag(v, B, C, gamma, stream=None):
    """Same-step correction gamma (C B^T) v per token and head (see ssd_y_diag)."""
    y = torch.empty_like(v)
    _check(ssd_y_diag(v, B, C, gamma, y, stream), "ssd_y_diag")
    return y


def y_diag_bwd(dy, v, B, C, gamma, stream=None):
    """Returns dict(d_v, d_B, d_C, d_gamma)."""
    out = dict(d_v=torch.empty_like(v), d_B=torch.empty_like(B), d_C=torch.empty_like(C),
               d_gamma=torch.empty_like(gamma))
    _check(ssd_y_diag_bwd(dy, v, B, C, gamma, out["d_v"], out["d_B"], out["d_C"], out["d_gamma"],
                          stream), "ssd_y_diag_bwd")
    return out


def quat_workspace(q: torch.Tensor, bwd: bool) -> torch.Tensor:
    b, s, h, j = _quat_sizes(q)
    n = ssd_quat_workspace_size(b, s, h, j, bwd)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def quat_scan(q, init=None, ws=None, stream=None):
    """cum[t] = q_t (x) cum[t-1] over q ``[b, s, h, j, 4]`` (see ssd_quat_scan)."""
    cum = torch.empty_like(q)
    ws = quat_workspace(q, False) if ws is None else ws
    _check(ssd_quat_scan(q, init, cum, ws, stream), "ssd_quat_scan")
    return cum


def quat_scan_bwd(q, init, d_cum, want_d_init=True, ws=None, stream=None):
    """Returns ``(d_q, d_init)`` (d_init None unless wanted)."""
    b, s, h, j = _quat_sizes(q)
    d_q = torch.empty_like(q)
    d_init = torch.empty((b, h, j, 4), device=q.device) if want_d_init else None
    ws = quat_workspace(q, True) if ws is None else ws
    _check(ssd_quat_scan_bwd(q, init, d_cum, d_q, d_init, ws, stream), "ssd_quat_scan_bwd")
    return d_q, d_init


def step(x, dt, A, B, C, D, state, in_place=False, stream=None):
    """One decode step: returns ``(y, new_state)``; with ``in_place`` the state tensor is
    updated and returned as new_state."""
    y = torch.empty_like(x)
    new_state = state if in_place else torch.empty_like(state)
    _check(ssd_step(x, dt, A, B, C, D, state, new_state, y, stream), "ssd_step")
    return y, new_state
