"""Pins of the CPU oracle's pooled state moments and their gradient (no GPU).

The oracle accumulates m2 = sum_t h_t^T h_t and m1 = sum_t sum_p h_t[p,:] while
it runs the recurrence (burn-mamba state_moments.rs page, StateMoments).  It is
checked against:

* an explicit-sum brute force: every h_t written as a sum over earlier tokens
  (no recursion), then pooled (I6);
* the per-chunk closed form the GPU path uses, evaluated in numpy (I7);
* symmetry, positive semi-definiteness and tr(m2) = sum_t ||h_t||_F^2 (I8);
* merge additivity across a split at a chunk boundary (StateMoments::merge) (I9);
* 1 <= PR <= dstate and PR = 1 for a rank-one state (StateMoments::pr) (I10);
* valid_len truncation (I11);
* finite differences of the gradient, zero gradients past valid_len, Euler
  identities and the hand-worked example in ``golden/``.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import chunked_scan
from mamba_ssd_chunked_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(batch=2, seq=16, nheads=2, headdim=3, dstate=4, chunk_len=4, init_std=0.5, seed=21):
    w = inputs.custom(batch=batch, seq=seq, nheads=nheads, headdim=headdim, dstate=dstate,
                      chunk_len=chunk_len, init_std=init_std, seed=seed, dt_shift=1.0)
    t = inputs.make_inputs(w)
    return {k: v.double().numpy() for k, v in t.items()}


def rel(a, b):
    den = np.linalg.norm(np.ravel(b))
    return np.linalg.norm(np.ravel(a) - np.ravel(b)) / (den if den > 0 else 1.0)


def explicit_states(i):
    """h_t = exp(c_t) init + sum_{s<=t} exp(c_t - c_s) dt_s x_s (outer) B_s, c = global
    inclusive cumsum of dt*A.  Returns [b, seq, h, p, r]."""
    b, n, l, h, p = i["x"].shape
    r = i["B"].shape[-1]
    seq = n * l
    x = i["x"].reshape(b, seq, h, p)
    B = i["B"].reshape(b, seq, h, r)
    dt = i["dt"].reshape(b, h, seq)
    c = np.cumsum(dt * i["A"][None, :, None], axis=2)
    out = np.zeros((b, seq, h, p, r))
    for t in range(seq):
        acc = np.exp(c[:, :, t])[:, :, None, None] * i["init"]
        for s in range(t + 1):
            wgt = np.exp(c[:, :, t] - c[:, :, s]) * dt[:, :, s]
            acc = acc + wgt[:, :, None, None] * np.einsum("bhp,bhr->bhpr", x[:, s], B[:, s])
        out[:, t] = acc
    return out


def moments(i, valid=None):
    return oracle.state_moments(i["x"], i["dt"], i["A"], i["B"], i["init"], valid)


def test_I6_explicit_sum_brute_force():
    i = tiny()
    hs = explicit_states(i)
    m2, m1, count = moments(i)
    assert rel(m2, np.einsum("bthpr,bthps->bhrs", hs, hs)) < 1e-12
    assert rel(m1, hs.sum(axis=(1, 3))) < 1e-12
    assert list(count) == [16 * 3, 16 * 3]


def closed_form(i, valid):
    """Per-chunk closed form: with entry state H, e_t = exp(cum_t),
    L[t,s] = exp(cum_t - cum_s) dt_s (s <= t), M = diag(mask):
      m2 += Bm^T (K o G) Bm + H^T X^T diag(v) Bm + (.)^T + (sum M e^2) H^T H,
            K = L^T M L, G = X X^T, v = L^T M e
      m1 += (sum M e) 1^T H + sum_s u_s (1^T x_s) B_s,  u = L^T M 1."""
    b, n, l, h, p = i["x"].shape
    r = i["B"].shape[-1]
    cum = chunked_scan.within_chunk_cumsum(i["dt"], i["A"])
    s_in = chunked_scan.chunk_entry_states(i["x"], i["dt"], i["A"], i["B"], i["init"])
    m2 = np.zeros((b, h, r, r))
    m1 = np.zeros((b, h, r))
    tril = np.tril(np.ones((l, l)))
    for bb in range(b):
        for hh in range(h):
            for k in range(n):
                t_glob = k * l + np.arange(l)
                M = (t_glob < valid[bb]).astype(float)
                c = cum[bb, hh, k]
                e = np.exp(c)
                L = tril * np.exp(np.minimum(c[:, None] - c[None, :], 0.0)) * i["dt"][bb, hh, k][None, :]
                X = i["x"][bb, k, :, hh, :]
                Bm = i["B"][bb, k, :, hh, :]
                H = s_in[bb, k, hh]
                K = L.T @ (M[:, None] * L)
                G = X @ X.T
                v = L.T @ (M * e)
                u = L.T @ M
                cross = H.T @ (X.T @ (v[:, None] * Bm))
                m2[bb, hh] += Bm.T @ ((K * G) @ Bm) + cross + cross.T + np.sum(M * e * e) * (H.T @ H)
                m1[bb, hh] += np.sum(M * e) * H.sum(axis=0) + ((u * X.sum(axis=1))[:, None] * Bm).sum(axis=0)
    return m2, m1


def test_I7_closed_form_matches():
    i = tiny(seq=24, chunk_len=8)
    valid = [24, 13]
    m2, m1, _ = moments(i, valid)
    c2, c1 = closed_form(i, valid)
    assert rel(m2, c2) < 1e-12
    assert rel(m1, c1) < 1e-12


def test_I8_symmetric_psd_and_trace():
    i = tiny()
    m2, _, _ = moments(i)
    assert np.max(np.abs(m2 - np.swapaxes(m2, 2, 3))) < 1e-12 * np.max(np.abs(m2))
    ev = np.linalg.eigvalsh(0.5 * (m2 + np.swapaxes(m2, 2, 3)))
    assert np.min(ev) > -1e-10 * np.max(ev)
    hs = explicit_states(i)
    tr = np.einsum("bhrr->bh", m2)
    assert rel(tr, (hs ** 2).sum(axis=(1, 3, 4))) < 1e-12


def test_I9_merge_additivity_at_a_chunk_boundary():
    i = tiny(seq=16, chunk_len=4)
    m2, m1, count = moments(i)
    a = dict(i)
    for k in ("x", "B", "C", "dy"):
        a[k] = i[k][:, :2]
    a["dt"] = i["dt"][:, :, :2]
    m2a, m1a, ca = moments(a)
    _, fa = oracle.ssd_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"])
    bpart = dict(a)
    for k in ("x", "B", "C", "dy"):
        bpart[k] = i[k][:, 2:]
    bpart["dt"] = i["dt"][:, :, 2:]
    bpart["init"] = fa
    m2b, m1b, cb = moments(bpart)
    assert rel(m2a + m2b, m2) < 1e-13
    assert rel(m1a + m1b, m1) < 1e-13
    assert list(ca + cb) == list(count)


def pr_uncentred(m2, count):
    """(tr S)^2 / tr(S^2), S = m2 / count (StateMoments::pr with center = false)."""
    S = m2 / count[:, None, None, None]
    tr = np.einsum("bhrr->bh", S)
    return tr ** 2 / np.einsum("bhrs,bhrs->bh", S, S)


def test_I10_participation_ratio_bounds_and_rank_one():
    i = tiny(dstate=6)
    m2, _, count = moments(i)
    pr = pr_uncentred(m2, count)
    assert np.all(pr >= 1 - 1e-12) and np.all(pr <= 6 + 1e-12)
    # rank one: every B_t is the same direction and the state starts at 0
    one = dict(i)
    one["init"] = np.zeros_like(i["init"])
    one["B"] = np.broadcast_to(i["B"][:, :1, :1], i["B"].shape).copy()
    m2r, _, cr = moments(one)
    assert np.allclose(pr_uncentred(m2r, cr), 1.0, atol=1e-12)


def test_I11_valid_len_equals_truncated_sequence():
    i = tiny(seq=16, chunk_len=4)
    valid = [11, 6]
    m2, m1, count = moments(i, valid)
    for bb, v in enumerate(valid):
        t = {k: i[k][bb:bb + 1] for k in ("x", "B", "init")}
        # rewrite with chunk_len 1 so that any prefix length is representable
        t["x"] = i["x"][bb:bb + 1].reshape(1, 16, 1, 2, 3)[:, :v]
        t["B"] = i["B"][bb:bb + 1].reshape(1, 16, 1, 2, 4)[:, :v]
        t["dt"] = i["dt"][bb:bb + 1].reshape(1, 2, 16, 1)[:, :, :v]
        t["A"] = i["A"]
        m2t, m1t, ct = moments(t)
        assert rel(m2[bb], m2t[0]) < 1e-13
        assert rel(m1[bb], m1t[0]) < 1e-13
        assert count[bb] == ct[0] == v * 3


# ---------------------------------------------------------------- backward pins
def mbwd(i, valid=None, dm1=True):
    return oracle.state_moments_bwd(i["d_m2"], i["d_m1"] if dm1 else None, i["x"], i["dt"],
                                    i["A"], i["B"], i["init"], valid)


def test_moments_finite_differences():
    i = tiny(batch=2, seq=8, nheads=1, headdim=2, dstate=3, chunk_len=4, seed=9)
    valid = [8, 5]
    g = mbwd(i, valid)

    def loss(inp):
        m2, m1, _ = moments(inp, valid)
        return float(np.sum(m2 * inp["d_m2"]) + np.sum(m1 * inp["d_m1"]))

    names = dict(x="d_x", dt="d_dt", A="d_A", B="d_B", init="d_init")
    for src, gname in names.items():
        base = i[src]
        fd = np.empty_like(base)
        for j in range(base.size):
            v = base.reshape(-1)[j]
            eps = 1e-6 * max(1.0, abs(v))
            plus, minus = dict(i), dict(i)
            plus[src], minus[src] = base.copy(), base.copy()
            plus[src].reshape(-1)[j] = v + eps
            minus[src].reshape(-1)[j] = v - eps
            fd.reshape(-1)[j] = (loss(plus) - loss(minus)) / (2 * eps)
        err = np.max(np.abs(fd - g[gname])) / max(1e-30, np.max(np.abs(g[gname])))
        assert err < 1e-6, (gname, err)


def test_moments_gradients_vanish_past_valid_len():
    i = tiny(seq=16, chunk_len=4)
    valid = [16, 6]
    g = mbwd(i, valid)
    assert np.all(g["d_x"][1].reshape(16, 2, 3)[6:] == 0)
    assert np.all(g["d_B"][1].reshape(16, 2, 4)[6:] == 0)
    assert np.all(g["d_dt"][1].reshape(2, 16)[:, 6:] == 0)
    assert np.any(g["d_x"][1].reshape(16, 2, 3)[:6] != 0)


def test_moments_euler_identities():
    i = tiny(seq=16, chunk_len=4)
    m2, m1, _ = moments(i)
    g = mbwd(i)
    L2 = float(np.sum(m2 * i["d_m2"]))
    L1 = float(np.sum(m1 * i["d_m1"]))
    # m2 is homogeneous of degree 2 and m1 of degree 1 in (x, init)
    lhs = float(np.sum(g["d_x"] * i["x"]) + np.sum(g["d_init"] * i["init"]))
    assert abs(lhs - (2 * L2 + L1)) < 1e-11 * (abs(2 * L2) + abs(L1))
    # with init = 0 the same degrees hold in B and under dt -> s dt, A -> A / s
    z = dict(i)
    z["init"] = np.zeros_like(i["init"])
    m2z, m1z, _ = moments(z)
    gz = mbwd(z)
    rhs = 2 * float(np.sum(m2z * z["d_m2"])) + float(np.sum(m1z * z["d_m1"]))
    assert abs(float(np.sum(gz["d_B"] * z["B"])) - rhs) < 1e-11 * abs(rhs)
    lhs = float(np.sum(gz["d_dt"] * z["dt"]) - np.sum(gz["d_A"] * z["A"]))
    assert abs(lhs - rhs) < 1e-11 * abs(rhs)


def test_null_d_m1_means_zero():
    i = tiny()
    z = dict(i)
    z["d_m1"] = np.zeros_like(i["d_m1"])
    a = mbwd(i, dm1=False)
    b = mbwd(z)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_golden_hand_worked_moments():
    with open(os.path.join(GOLDEN, "hand_worked_p1r1_seq3.json")) as f:
        gold = json.load(f)
    tol = gold["tolerance_abs"]
    inp = {k: np.asarray(v, dtype=np.float64) for k, v in gold["inputs"].items()}
    x = inp["x"].reshape(1, 3, 1, 1, 1)
    B = inp["B"].reshape(1, 3, 1, 1, 1)
    dt = inp["dt"].reshape(1, 1, 3, 1)
    init = inp["init"].reshape(1, 1, 1, 1)
    e = gold["expected"]
    m2, m1, count = oracle.state_moments(x, dt, inp["A"], B, init)
    assert np.allclose(m2.ravel(), e["m2"], atol=tol, rtol=0)
    assert np.allclose(m1.ravel(), e["m1"], atol=tol, rtol=0)
    assert list(count) == e["count"]
    g = oracle.state_moments_bwd(inp["d_m2"].reshape(1, 1, 1, 1), inp["d_m1"].reshape(1, 1, 1),
                                 x, dt, inp["A"], B, init)
    ln2 = math.log(2.0)
    d_dt = np.asarray(e["moments_d_dt"]["const"]) + ln2 * np.asarray(e["moments_d_dt"]["ln2_coeff"])
    assert np.allclose(g["d_dt"].ravel(), d_dt, atol=tol, rtol=0)
    for k in ("d_x", "d_A", "d_B", "d_init"):
        assert np.allclose(g[k].ravel(), e["moments_" + k], atol=tol, rtol=0), k
