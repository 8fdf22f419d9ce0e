"""Pins of the CPU oracle's participation ratio and its gradient (no GPU).

StateMoments::pr of the burn-mamba state_moments.rs page: Sigma = m2 / count
(centred: minus mu mu^T), PR = (tr Sigma)^2 / ||Sigma||_F^2, evaluated through the
trace-normalised Sigma_hat = Sigma / max(tr Sigma, min_positive) with the
normaliser detached and the denominator floored at div_eps; StateMoments::trace
= tr(m2) / count.  The oracle is checked against:

* the eigenvalue form (sum lambda)^2 / sum lambda^2 of the sample covariance,
  with numpy's ``cov`` for the centred case (a different route to the value);
* isotropic (PR = r), rank-k (PR = k) and 1 <= PR <= r;
* the trace as the mean squared sample norm;
* central finite differences of the plain formula, which has no normaliser, so
  this is the page's claim that detaching it leaves the gradient exact
  (``pr_gradient_matches_direct_formula``);
* Euler's identity for a degree-0 function (the gradient has no radial part);
* scaling the samples over 18 decades: PR unchanged, gradient finite and of
  degree -1 (``pr_gradient_finite_as_magnitude_shrinks``);
* an all-zero state: PR 0, trace 0, zero gradient, nothing non-finite.
"""
import numpy as np
import pytest

import oracle


def samples(batch=2, nheads=3, r=6, counts=(40, 25), seed=5, mean=0.0, rank=None):
    """Seeded sample rows per (batch, head): list of lists of [n_b, r] arrays."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(batch):
        row = []
        for _ in range(nheads):
            k = r if rank is None else rank
            z = rng.standard_normal((counts[b], k)) @ rng.standard_normal((k, r))
            row.append(z + mean * rng.standard_normal(r))
        out.append(row)
    return out


def pooled(hs):
    m2 = np.array([[h.T @ h for h in row] for row in hs])
    m1 = np.array([[h.sum(0) for h in row] for row in hs])
    count = np.array([row[0].shape[0] for row in hs], dtype=np.int64)
    return m2, m1, count


def eig_pr(S):
    lam = np.linalg.eigvalsh(S)
    return lam.sum() ** 2 / (lam ** 2).sum()


@pytest.mark.parametrize("center", [False, True])
def test_pr_equals_the_eigenvalue_form(center):
    hs = samples(mean=1.5)
    m2, m1, count = pooled(hs)
    pr, _ = oracle.moments_pr(m2, m1, count, center)
    for b, row in enumerate(hs):
        for h, x in enumerate(row):
            S = np.cov(x.T, bias=True) if center else x.T @ x / x.shape[0]
            assert pr[b, h] == pytest.approx(eig_pr(S), rel=1e-12)


def test_pr_isotropic_rank_k_and_bounds():
    r = 8
    # isotropic: an orthonormal frame of r samples, repeated
    q, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((r, r)))
    iso = np.tile(q, (3, 1))
    m2, m1, count = pooled([[iso]])
    assert oracle.moments_pr(m2, m1, count)[0][0, 0] == pytest.approx(r, rel=1e-12)
    # rank k with equal spectrum: k orthonormal directions
    for k in (1, 3, 5):
        m2, m1, count = pooled([[np.tile(q[:k], (2, 1))]])
        assert oracle.moments_pr(m2, m1, count)[0][0, 0] == pytest.approx(k, rel=1e-12)
    # random low-rank and full-rank samples stay within [1, rank]
    for rank in (1, 2, r):
        hs = samples(r=r, rank=rank, seed=rank)
        pr, _ = oracle.moments_pr(*pooled(hs))
        assert np.all(pr >= 1 - 1e-12) and np.all(pr <= rank + 1e-9)
        if rank == 1:
            assert np.allclose(pr, 1.0, atol=1e-12)


def test_trace_is_the_mean_squared_sample_norm():
    hs = samples(mean=0.7)
    m2, m1, count = pooled(hs)
    for center in (False, True):
        _, tr = oracle.moments_pr(m2, m1, count, center)
        for b, row in enumerate(hs):
            for h, x in enumerate(row):
                assert tr[b, h] == pytest.approx((x ** 2).sum(1).mean(), rel=1e-13)


def direct(m2, m1, n, center):
    """The plain ratio (tr S)^2 / ||S||_F^2 with no normaliser and no floors."""
    mu = m1 / n
    S = m2 / n - (np.outer(mu, mu) if center else 0.0)
    return np.trace(S) ** 2 / (S * S).sum()


@pytest.mark.parametrize("center", [False, True])
def test_pr_gradient_matches_direct_formula(center):
    hs = samples(batch=2, nheads=2, r=4, counts=(9, 14), mean=0.8, seed=11)
    m2, m1, count = pooled(hs)
    # a non-symmetric perturbation of m2 as well: the gradient is taken entry by entry
    m2 = m2 + 0.05 * np.random.default_rng(2).standard_normal(m2.shape)
    d_pr = np.random.default_rng(3).standard_normal((2, 2))
    d_m2, d_m1 = oracle.moments_pr_bwd(d_pr, m2, m1, count, center)
    for b in range(2):
        for h in range(2):
            n = float(count[b])
            fd2 = np.zeros((4, 4))
            for i in range(4):
                for j in range(4):
                    e = np.zeros((4, 4))
                    step = 1e-6 * max(1.0, abs(m2[b, h, i, j]))
                    e[i, j] = step
                    fd2[i, j] = (direct(m2[b, h] + e, m1[b, h], n, center)
                                 - direct(m2[b, h] - e, m1[b, h], n, center)) / (2 * step)
            fd1 = np.zeros(4)
            for i in range(4):
                e = np.zeros(4)
                step = 1e-6 * max(1.0, abs(m1[b, h, i]))
                e[i] = step
                fd1[i] = (direct(m2[b, h], m1[b, h] + e, n, center)
                          - direct(m2[b, h], m1[b, h] - e, n, center)) / (2 * step)
            np.testing.assert_allclose(d_m2[b, h], d_pr[b, h] * fd2, rtol=1e-6,
                                       atol=1e-7 * np.abs(fd2).max() * abs(d_pr[b, h]))
            np.testing.assert_allclose(d_m1[b, h], d_pr[b, h] * fd1, rtol=1e-6,
                                       atol=1e-7 * max(np.abs(fd1).max(), 1e-300) * abs(d_pr[b, h]))


def test_pr_gradient_has_no_radial_part():
    """PR is of degree 0 in (m2, m1) scaled as (c^2, c): <d_m2, 2 m2> + <d_m1, m1> = 0.
    Dropping the numerator's gradient (the rewrite the page warns about) breaks this."""
    hs = samples(mean=1.1)
    m2, m1, count = pooled(hs)
    d_pr = np.ones((2, 3))
    for center in (False, True):
        d_m2, d_m1 = oracle.moments_pr_bwd(d_pr, m2, m1, count, center)
        euler = 2 * np.einsum("bhij,bhij->bh", d_m2, m2) + np.einsum("bhi,bhi->bh", d_m1, m1)
        scale = np.einsum("bhij,bhij->bh", np.abs(d_m2), np.abs(m2))
        assert np.all(np.abs(euler) <= 1e-12 * scale)
        assert np.all(np.abs(d_m2).max(axis=(2, 3)) > 0)


def test_pr_gradient_finite_as_magnitude_shrinks():
    """Samples scaled by c = 10^-k, k = 0..18 (tr Sigma down to ~1e-36, above the
    min_positive floor): PR is unchanged and c^2 d_m2(c) = d_m2(1), c d_m1(c) = d_m1(1)."""
    hs = samples(mean=0.5, seed=8)
    m2, m1, count = pooled(hs)
    d_pr = np.random.default_rng(4).standard_normal((2, 3))
    for center in (False, True):
        pr1, _ = oracle.moments_pr(m2, m1, count, center)
        g2, g1 = oracle.moments_pr_bwd(d_pr, m2, m1, count, center)
        for k in range(19):
            c = 10.0 ** -k
            prc, _ = oracle.moments_pr(m2 * c * c, m1 * c, count, center)
            h2, h1 = oracle.moments_pr_bwd(d_pr, m2 * c * c, m1 * c, count, center)
            assert np.all(np.isfinite(h2)) and np.all(np.isfinite(h1))
            np.testing.assert_allclose(prc, pr1, rtol=1e-12)
            np.testing.assert_allclose(h2 * c * c, g2, rtol=1e-10, atol=1e-12 * np.abs(g2).max())
            np.testing.assert_allclose(h1 * c, g1, rtol=1e-10, atol=1e-12 * np.abs(g1).max())


def test_all_zero_state():
    m2 = np.zeros((2, 3, 6, 6))
    m1 = np.zeros((2, 3, 6))
    count = np.array([7, 3])
    for center in (False, True):
        pr, tr = oracle.moments_pr(m2, m1, count, center)
        assert np.all(pr == 0) and np.all(tr == 0)
        d_m2, d_m1 = oracle.moments_pr_bwd(np.ones((2, 3)), m2, m1, count, center)
        assert np.all(d_m2 == 0) and np.all(d_m1 == 0)


def test_collapsing_state_reads_below_one():
    """A state far below fp32's smallest normal: the trace floor fires, the
    denominator clamp drags PR under its true floor of 1 (StateMoments::trace
    documentation), and everything stays finite."""
    m2 = np.eye(4)[None, None] * 1e-45
    m1 = np.zeros((1, 1, 4))
    pr, tr = oracle.moments_pr(m2, m1, [1])
    assert 0 <= pr[0, 0] < 1 and tr[0, 0] == pytest.approx(4e-45)
    d_m2, _ = oracle.moments_pr_bwd(np.ones((1, 1)), m2, m1, [1])
    assert np.all(np.isfinite(d_m2))


def test_bad_count_is_rejected():
    with pytest.raises(RuntimeError):
        oracle.moments_pr(np.eye(2)[None, None], np.zeros((1, 1, 2)), [0])
