"""CPU oracle for the Mamba-2 SSD chunked scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``mamba_ssd_chunked_amd``
and its HIP library) never imports, links or calls it, and the two share no code.

The computation lives in ``ssd_oracle.c`` (plain C, fp64, single-threaded): the
token-by-token recurrence ``h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t``,
``y_t = C_t . h_t + D x_t`` and its reverse-mode recurrence, plus the pooled
state moments of the burn-mamba ``state_moments.rs`` page and their gradient, and
that page's participation ratio of the moments with its gradient, and the
gamma-weighted same-step correction ``y_diag`` of the Mamba-3 SSD with its gradient,
and the Mamba-3 quaternion cumulative-product scan with its gradient; the
decode step is the forward over one token from a cached state.
This module only builds the shared library with gcc and marshals numpy arrays.

Every function takes and returns float64 numpy arrays in the pages' layouts:
x/y ``[b, n, l, h, p]``, B/C ``[b, n, l, h, r]``, dt ``[b, h, n, l]``,
A/D ``[h]``, states ``[b, h, p, r]``, m2 ``[b, h, r, r]``, m1 ``[b, h, r]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libssd_oracle.so")

_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in
                ("batch", "nchunks", "chunk_len", "nheads", "headdim", "dstate")]


def build(force: bool = True) -> str:
    """Compile ``ssd_oracle.c`` with gcc (-O2, no fast-math) into ``_build/``."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off",
                        "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    _lib = _open(_LIB_PATH)
    return _lib


def use_library(path):
    """Point this module at another build of ``ssd_oracle.c`` (the mutation tests
    use it to run the pins against deliberately broken copies).  Returns the
    previous library handle; ``use_library(None)`` restores the default build."""
    global _lib
    prev = _lib
    _lib = None if path is None else _open(path)
    return prev


def _open(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_ssd_fwd.argtypes = [ctypes.POINTER(_Dims)] + [P] * 9
    lib.oracle_ssd_bwd.argtypes = [ctypes.POINTER(_Dims)] + [P] * 16 + [ctypes.c_int64]
    lib.oracle_state_moments.argtypes = [ctypes.POINTER(_Dims)] + [P] * 9
    lib.oracle_state_moments_bwd.argtypes = [ctypes.POINTER(_Dims)] + [P] * 13 + [ctypes.c_int64]
    I64 = ctypes.c_int64
    lib.oracle_moments_pr.argtypes = [I64, I64, I64, P, P, P, ctypes.c_int, P, P]
    lib.oracle_moments_pr_bwd.argtypes = [I64, I64, I64, P, P, P, P, ctypes.c_int, P, P]
    lib.oracle_diag_fwd.argtypes = [I64] * 5 + [P] * 5
    lib.oracle_diag_bwd.argtypes = [I64] * 5 + [P] * 9
    lib.oracle_quat_scan.argtypes = [I64] * 4 + [P] * 3
    lib.oracle_quat_scan_bwd.argtypes = [I64] * 4 + [P] * 5
    for f in (lib.oracle_ssd_fwd, lib.oracle_ssd_bwd, lib.oracle_state_moments,
              lib.oracle_state_moments_bwd):
        f.restype = ctypes.c_int
    return lib


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor -> numpy (CPU copy)
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(x, B):
    b, n, l, h, p = x.shape
    r = B.shape[-1]
    return _Dims(b, n, l, h, p, r)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def ssd_fwd(x, dt, A, B, C, D, init=None):
    """Token-by-token forward.  Returns ``(y, final_state)``."""
    x, dt, A, B, C, D, init = map(_f64, (x, dt, A, B, C, D, init))
    d = _dims(x, B)
    y = np.empty_like(x)
    final = np.empty((d.batch, d.nheads, d.headdim, d.dstate))
    rc = _load().oracle_ssd_fwd(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                _ptr(D), _ptr(init), _ptr(y), _ptr(final))
    _check(rc, "ssd_fwd")
    return y, final


def ssd_step(x, dt, A, B, C, D, state):
    """One decode step of the recurrence from the cached state (the token-by-token
    ``step`` loop the state_moments.rs page refers to): the forward over a single
    token with ``init = state``.  x ``[b, h, p]``, dt ``[b, h]``, B/C ``[b, h, r]``,
    state ``[b, h, p, r]``.  Returns ``(y [b, h, p], new_state [b, h, p, r])``."""
    x, dt, B, C, state = map(_f64, (x, dt, B, C, state))
    b, h, p = x.shape
    r = B.shape[-1]
    y, new_state = ssd_fwd(x.reshape(b, 1, 1, h, p), dt.reshape(b, h, 1, 1), A,
                           B.reshape(b, 1, 1, h, r), C.reshape(b, 1, 1, h, r), D, state)
    return y.reshape(b, h, p), new_state


def ssd_bwd(dy, d_final, x, dt, A, B, C, D, init=None, seg: int = 256):
    """Reverse-mode recurrence.  Returns a dict with the seven gradients."""
    dy, d_final, x, dt, A, B, C, D, init = map(_f64, (dy, d_final, x, dt, A, B, C, D, init))
    d = _dims(x, B)
    out = dict(d_x=np.empty_like(x), d_dt=np.empty_like(dt), d_A=np.empty_like(A),
               d_B=np.empty_like(B), d_C=np.empty_like(C), d_D=np.empty_like(D),
               d_init=np.empty((d.batch, d.nheads, d.headdim, d.dstate)))
    rc = _load().oracle_ssd_bwd(ctypes.byref(d), _ptr(dy), _ptr(d_final), _ptr(x), _ptr(dt),
                                _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
                                _ptr(out["d_x"]), _ptr(out["d_dt"]), _ptr(out["d_A"]),
                                _ptr(out["d_B"]), _ptr(out["d_C"]), _ptr(out["d_D"]),
                                _ptr(out["d_init"]), int(seg))
    _check(rc, "ssd_bwd")
    return out


def _valid(valid_len, batch):
    if valid_len is None:
        return None
    v = np.ascontiguousarray(np.asarray(valid_len, dtype=np.int64).reshape(batch))
    return v


def state_moments(x, dt, A, B, init=None, valid_len=None):
    """Brute-force pooled moments.  Returns ``(m2, m1, count)``."""
    x, dt, A, B, init = map(_f64, (x, dt, A, B, init))
    d = _dims(x, B)
    v = _valid(valid_len, d.batch)
    m2 = np.empty((d.batch, d.nheads, d.dstate, d.dstate))
    m1 = np.empty((d.batch, d.nheads, d.dstate))
    count = np.empty((d.batch,), dtype=np.int64)
    rc = _load().oracle_state_moments(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                      _ptr(init), None if v is None else _ptr(v), _ptr(m2),
                                      _ptr(m1), _ptr(count))
    _check(rc, "state_moments")
    return m2, m1, count


def state_moments_bwd(d_m2, d_m1, x, dt, A, B, init=None, valid_len=None, seg: int = 256):
    """Gradient of ``<d_m2, m2> + <d_m1, m1>``.  Returns a dict of five gradients."""
    d_m2, d_m1, x, dt, A, B, init = map(_f64, (d_m2, d_m1, x, dt, A, B, init))
    d = _dims(x, B)
    v = _valid(valid_len, d.batch)
    out = dict(d_x=np.empty_like(x), d_dt=np.empty_like(dt), d_A=np.empty_like(A),
               d_B=np.empty_like(B), d_init=np.empty((d.batch, d.nheads, d.headdim, d.dstate)))
    rc = _load().oracle_state_moments_bwd(ctypes.byref(d), _ptr(d_m2), _ptr(d_m1), _ptr(x),
                                          _ptr(dt), _ptr(A), _ptr(B), _ptr(init),
                                          None if v is None else _ptr(v), _ptr(out["d_x"]),
                                          _ptr(out["d_dt"]), _ptr(out["d_A"]), _ptr(out["d_B"]),
                                          _ptr(out["d_init"]), int(seg))
    _check(rc, "state_moments_bwd")
    return out


def moments_pr(m2, m1, count, center=False):
    """Participation ratio of the pooled moments (StateMoments::pr) and the raw
    trace (StateMoments::trace).  m2 ``[b, h, r, r]``, m1 ``[b, h, r]``, count ``[b]``.
    Returns ``(pr, trace)``, each ``[b, h]``."""
    m2, m1 = _f64(m2), _f64(m1)
    b, h, r, _ = m2.shape
    cnt = np.ascontiguousarray(np.asarray(count, dtype=np.int64).reshape(b))
    pr = np.empty((b, h))
    tr = np.empty((b, h))
    rc = _load().oracle_moments_pr(b, h, r, _ptr(m2), _ptr(m1), _ptr(cnt), int(bool(center)),
                                   _ptr(pr), _ptr(tr))
    _check(rc, "moments_pr")
    return pr, tr


def moments_pr_bwd(d_pr, m2, m1, count, center=False):
    """Gradient of ``<d_pr, PR>`` w.r.t. m2 and m1 with the trace normaliser held
    fixed.  Returns ``(d_m2, d_m1)``."""
    d_pr, m2, m1 = _f64(d_pr), _f64(m2), _f64(m1)
    b, h, r, _ = m2.shape
    cnt = np.ascontiguousarray(np.asarray(count, dtype=np.int64).reshape(b))
    d_m2 = np.empty_like(m2)
    d_m1 = np.empty((b, h, r))
    rc = _load().oracle_moments_pr_bwd(b, h, r, _ptr(d_pr), _ptr(m2), _ptr(m1), _ptr(cnt),
                                       int(bool(center)), _ptr(d_m2), _ptr(d_m1))
    _check(rc, "moments_pr_bwd")
    return d_m2, d_m1


def _diag_dims(V, B):
    """V ``[..., m, h, p]`` and B ``[..., m, h, r]``: the leading axes ([b, n, l]) are tokens."""
    *lead, m, h, p = V.shape
    r = B.shape[-1]
    return int(np.prod(lead)) if lead else 1, m, h, p, r


def diag_fwd(V, B, C, gamma):
    """Same-step correction y_diag (mamba3 diag.rs page).  V ``[b, n, l, m, h, p]``,
    B / C ``[b, n, l, m, h, r]``, gamma ``[b, n, l, h]``; returns y_diag like V."""
    V, B, C, gamma = map(_f64, (V, B, C, gamma))
    T, m, h, p, r = _diag_dims(V, B)
    y = np.empty_like(V)
    _check(_load().oracle_diag_fwd(T, m, h, p, r, _ptr(V), _ptr(B), _ptr(C), _ptr(gamma), _ptr(y)),
           "diag_fwd")
    return y


def diag_bwd(dy, V, B, C, gamma):
    """Gradients of ``<dy, y_diag>``: dict(d_v, d_b, d_c, d_gamma)."""
    dy, V, B, C, gamma = map(_f64, (dy, V, B, C, gamma))
    T, m, h, p, r = _diag_dims(V, B)
    out = dict(d_v=np.empty_like(V), d_b=np.empty_like(B), d_c=np.empty_like(C),
               d_gamma=np.empty_like(gamma))
    _check(_load().oracle_diag_bwd(T, m, h, p, r, _ptr(dy), _ptr(V), _ptr(B), _ptr(C), _ptr(gamma),
                                   _ptr(out["d_v"]), _ptr(out["d_b"]), _ptr(out["d_c"]),
                                   _ptr(out["d_gamma"])), "diag_bwd")
    return out


def quat_scan(q, init=None):
    """Quaternion cumulative product cum[t] = q_t (x) cum[t-1] (mamba3 quat_scan page).
    q ``[b, s, h, j, 4]`` (w, x, y, z), init ``[b, h, j, 4]`` or None (identity)."""
    q, init = _f64(q), _f64(init)
    b, s, h, j, _ = q.shape
    cum = np.empty_like(q)
    _check(_load().oracle_quat_scan(b, s, h, j, _ptr(q), _ptr(init), _ptr(cum)), "quat_scan")
    return cum


def quat_scan_bwd(q, init, d_cum):
    """Exact reverse mode of quat_scan: returns ``(d_q, d_init)``."""
    q, init, d_cum = _f64(q), _f64(init), _f64(d_cum)
    b, s, h, j, _ = q.shape
    d_q = np.empty_like(q)
    d_init = np.empty((b, h, j, 4))
    _check(_load().oracle_quat_scan_bwd(b, s, h, j, _ptr(q), _ptr(init), _ptr(d_cum), _ptr(d_q),
                                        _ptr(d_init)), "quat_scan_bwd")
    return d_q, d_init
