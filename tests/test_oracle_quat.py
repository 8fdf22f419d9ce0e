"""Pins of the CPU oracle's quaternion cumulative-product scan and its gradient (no GPU).

The Mamba-3 rotation scan of the burn-mamba page "mamba3/quat_scan/backward.rs":
cum[t] = q_t (x) cum[t-1], cum[-1] = init, Hamilton product on (w, x, y, z).  The
oracle runs it token by token and back-propagates with the exact per-factor
VJPs.  It is checked against:

* the quaternion unit table (i j = k, j k = i, k i = j, i^2 = j^2 = k^2 = -1) and
  the identity as init;
* scipy's rotation composition: for unit quaternions, cum[t] as a rotation is
  R(q_t) ... R(q_0) R(init) (scipy stores quaternions scalar-last);
* the multiplicative norm |cum[t]| = prod |q_s| |init| for arbitrary quaternions;
* central finite differences of d_q and d_init for arbitrary (non-unit) quaternions;
* the page's parallel closed form for unit quaternions (prefix product P, suffix
  sum S = sum_{s>=t} conj(P_s) (x) d_cum[s], G = P (x) S, d_q = G (x) conj(cum[t-1]),
  d_init = S[0]), evaluated in numpy -- and that it differs for non-unit inputs.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import oracle


def hamilton(a, b):
    """Reference product for the closed-form pin (numpy, broadcast over leading axes)."""
    aw, ax, ay, az = np.moveaxis(a, -1, 0)
    bw, bx, by, bz = np.moveaxis(b, -1, 0)
    return np.stack([aw * bw - ax * bx - ay * by - az * bz,
                     aw * bx + ax * bw + ay * bz - az * by,
                     aw * by - ax * bz + ay * bw + az * bx,
                     aw * bz + ax * by - ay * bx + az * bw], -1)


def conj(a):
    return a * np.array([1.0, -1.0, -1.0, -1.0])


def unit(shape, seed):
    v = np.random.default_rng(seed).standard_normal(shape + (4,))
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def test_unit_table():
    one, i, j, k = np.eye(4)
    def prod(a, b):  # a (x) b as a one-step scan: cum[0] = q_0 (x) init
        return oracle.quat_scan(a.reshape(1, 1, 1, 1, 4), b.reshape(1, 1, 1, 4))[0, 0, 0, 0]
    np.testing.assert_array_equal(prod(i, j), k)
    np.testing.assert_array_equal(prod(j, k), i)
    np.testing.assert_array_equal(prod(k, i), j)
    np.testing.assert_array_equal(prod(j, i), -k)
    for u in (i, j, k):
        np.testing.assert_array_equal(prod(u, u), -one)
    q = np.random.default_rng(0).standard_normal((2, 5, 3, 2, 4))
    np.testing.assert_array_equal(oracle.quat_scan(q)[:, 0], q[:, 0])  # identity init


def test_matches_scipy_rotation_composition():
    q = unit((2, 7, 2, 3), 1)
    init = unit((2, 2, 3), 2)
    cum = oracle.quat_scan(q, init)
    xyzw = lambda a: np.concatenate([a[..., 1:], a[..., :1]], -1)  # noqa: E731
    for b in range(2):
        for h in range(2):
            for jj in range(3):
                r = Rotation.from_quat(xyzw(init[b, h, jj]))
                for t in range(7):
                    r = Rotation.from_quat(xyzw(q[b, t, h, jj])) * r
                    np.testing.assert_allclose(Rotation.from_quat(xyzw(cum[b, t, h, jj])).as_matrix(),
                                               r.as_matrix(), atol=1e-12)


def test_norm_is_multiplicative():
    q = np.random.default_rng(3).standard_normal((1, 9, 2, 2, 4))
    init = np.random.default_rng(4).standard_normal((1, 2, 2, 4))
    cum = oracle.quat_scan(q, init)
    expect = np.cumprod(np.linalg.norm(q, axis=-1), axis=1) * np.linalg.norm(init, axis=-1)[:, None]
    np.testing.assert_allclose(np.linalg.norm(cum, axis=-1), expect, rtol=1e-12)


def test_finite_differences_general_quaternions():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 1, 2, 4))
    init = rng.standard_normal((1, 1, 2, 4))
    dc = rng.standard_normal(q.shape)
    d_q, d_init = oracle.quat_scan_bwd(q, init, dc)
    f = lambda qq, ii: float((dc * oracle.quat_scan(qq, ii)).sum())  # noqa: E731
    for a, g, which in ((q, d_q, 0), (init, d_init, 1)):
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            e = np.zeros_like(a)
            e[idx] = 1e-6
            args_p = (q + e, init) if which == 0 else (q, init + e)
            args_m = (q - e, init) if which == 0 else (q, init - e)
            fd[idx] = (f(*args_p) - f(*args_m)) / 2e-6
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8 * np.abs(fd).max())


def closed_form(q, init, dc):
    """The page's parallel form, in numpy: valid for unit quaternions."""
    S = q.shape[1]
    P = np.empty_like(q)
    acc = np.broadcast_to(np.array([1.0, 0, 0, 0]), q[:, 0].shape)
    for t in range(S):
        acc = hamilton(q[:, t], acc)
        P[:, t] = acc
    cum = hamilton(P, init[:, None])
    terms = hamilton(conj(P), dc)
    Ssum = np.flip(np.cumsum(np.flip(terms, 1), 1), 1)
    G = hamilton(P, Ssum)
    prev = np.concatenate([init[:, None], cum[:, :-1]], 1)
    return hamilton(G, conj(prev)), Ssum[:, 0]


def test_page_closed_form_for_unit_quaternions():
    q = unit((2, 33, 3, 2), 6)
    init = unit((2, 3, 2), 7)
    dc = np.random.default_rng(8).standard_normal(q.shape)
    d_q, d_init = oracle.quat_scan_bwd(q, init, dc)
    cq, ci = closed_form(q, init, dc)
    np.testing.assert_allclose(d_q, cq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(d_init, ci, rtol=1e-10, atol=1e-11)
    # the closed form relies on conj(q) = q^-1: with non-unit steps it is not the gradient
    q2 = q * 1.3
    d_q2, _ = oracle.quat_scan_bwd(q2, init, dc)
    assert np.abs(closed_form(q2, init, dc)[0] - d_q2).max() > 1e-2


def test_empty_sequence_gradient_of_init_is_zero():
    q = np.zeros((2, 0, 3, 2, 4))
    d_q, d_init = oracle.quat_scan_bwd(q, unit((2, 3, 2), 9), q)
    assert d_q.size == 0 and np.all(d_init == 0)
