"""Pins of the CPU oracle's same-step correction y_diag and its gradient (no GPU).

The Mamba-3 SSD adds, per token and head, y_diag = gamma (C B^T) V over the mimo
axis (burn-mamba page "mamba3/single_ssd/ssd/serial_recalculated/diag.rs").  The
oracle evaluates the general (MIMO) definition and its reverse mode; it is
checked against:

* the page's SISO path (mimo rank 1: one reduction over r, then broadcast
  multiplies) for the value and all four gradients -- the page's own claim that
  the SISO fast path equals the general path;
* the Mamba-2 SSD oracle in the memoryless limit: with A = -1e4 every decay
  exp(dt A) is 0, the scan keeps only each token's own write, and its output is
  exactly the diagonal term dt (C.B) x, i.e. y_diag with V = x and gamma = dt
  (and its d_x, d_B, d_C, d_dt are the correction's gradients);
* central finite differences of all four gradients at mimo rank 3;
* linearity of y_diag in each of V, gamma, B and C separately:
  <dy, y> = <d_v, V> = <d_gamma, gamma> = <d_b, B> = <d_c, C>.
"""
import numpy as np
import pytest

import oracle


def draw(b=1, n=2, l=3, m=1, h=2, p=4, r=5, seed=0):
    rng = np.random.default_rng(seed)
    return dict(V=rng.standard_normal((b, n, l, m, h, p)), B=rng.standard_normal((b, n, l, m, h, r)),
                C=rng.standard_normal((b, n, l, m, h, r)), gamma=rng.standard_normal((b, n, l, h)),
                dy=rng.standard_normal((b, n, l, m, h, p)))


def test_siso_path_equals_general_path():
    i = draw(m=1, h=3, p=6, r=7, seed=1)
    V, B, C, dy = (i[k][:, :, :, 0] for k in ("V", "B", "C", "dy"))  # drop the mimo axis
    g = i["gamma"]
    qk = (C * B).sum(-1)                      # [b, n, l, h]
    dyv = (dy * V).sum(-1)
    y = oracle.diag_fwd(i["V"], i["B"], i["C"], i["gamma"])[:, :, :, 0]
    np.testing.assert_allclose(y, V * (qk * g)[..., None], rtol=1e-13, atol=1e-13)
    gr = oracle.diag_bwd(i["dy"], i["V"], i["B"], i["C"], i["gamma"])
    dqk = dyv * g
    np.testing.assert_allclose(gr["d_gamma"], qk * dyv, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gr["d_v"][:, :, :, 0], dy * (qk * g)[..., None], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gr["d_c"][:, :, :, 0], B * dqk[..., None], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gr["d_b"][:, :, :, 0], C * dqk[..., None], rtol=1e-13, atol=1e-13)


def test_memoryless_ssd_is_the_diagonal_term():
    """Mamba-2 SSD with every decay 0 and D = 0: y_t = dt_t (C_t . B_t) x_t."""
    rng = np.random.default_rng(2)
    b, n, l, h, p, r = 2, 2, 4, 3, 5, 6
    x = rng.standard_normal((b, n, l, h, p))
    B = rng.standard_normal((b, n, l, h, r))
    C = rng.standard_normal((b, n, l, h, r))
    dt = 0.1 + rng.random((b, h, n, l))
    A = np.full(h, -1e4)
    D = np.zeros(h)
    dy = rng.standard_normal((b, n, l, h, p))
    y, _ = oracle.ssd_fwd(x, dt, A, B, C, D)
    gamma = dt.transpose(0, 2, 3, 1)          # [b, h, n, l] -> [b, n, l, h]
    yd = oracle.diag_fwd(x[:, :, :, None], B[:, :, :, None], C[:, :, :, None], gamma)
    np.testing.assert_allclose(yd[:, :, :, 0], y, rtol=1e-12, atol=1e-14)
    g = oracle.ssd_bwd(dy, None, x, dt, A, B, C, D)
    gd = oracle.diag_bwd(dy[:, :, :, None], x[:, :, :, None], B[:, :, :, None], C[:, :, :, None], gamma)
    np.testing.assert_allclose(gd["d_v"][:, :, :, 0], g["d_x"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gd["d_b"][:, :, :, 0], g["d_B"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gd["d_c"][:, :, :, 0], g["d_C"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gd["d_gamma"], g["d_dt"].transpose(0, 2, 3, 1), rtol=1e-12, atol=1e-14)


def test_finite_differences_all_four_gradients():
    i = draw(m=3, h=2, p=3, r=4, seed=3)
    gr = oracle.diag_bwd(i["dy"], i["V"], i["B"], i["C"], i["gamma"])
    f = lambda **kw: float((i["dy"] * oracle.diag_fwd(**{**{k: i[k] for k in ("V", "B", "C", "gamma")}, **kw})).sum())  # noqa: E731
    for name, gname in (("V", "d_v"), ("B", "d_b"), ("C", "d_c"), ("gamma", "d_gamma")):
        a = i[name]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            e = np.zeros_like(a)
            step = 1e-6 * max(1.0, abs(a[idx]))
            e[idx] = step
            fd[idx] = (f(**{name: a + e}) - f(**{name: a - e})) / (2 * step)
        np.testing.assert_allclose(gr[gname], fd, rtol=1e-6, atol=1e-7 * np.abs(fd).max(), err_msg=name)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_linearity_in_each_input(m):
    i = draw(b=2, n=2, l=4, m=m, h=3, p=8, r=16, seed=10 + m)
    y = oracle.diag_fwd(i["V"], i["B"], i["C"], i["gamma"])
    gr = oracle.diag_bwd(i["dy"], i["V"], i["B"], i["C"], i["gamma"])
    ref = (i["dy"] * y).sum()
    for name, gname in (("V", "d_v"), ("B", "d_b"), ("C", "d_c"), ("gamma", "d_gamma")):
        assert (gr[gname] * i[name]).sum() == pytest.approx(ref, rel=1e-12), name


def test_empty_token_set():
    i = draw(n=0)
    assert oracle.diag_fwd(i["V"], i["B"], i["C"], i["gamma"]).size == 0
