"""Pins of the CPU oracle's SSD forward and backward (no GPU).

The oracle is the token-by-token recurrence and its reverse-mode recurrence.
Nothing here retypes its loops: every check compares it with something else
that fixes the answer --

* a chunked evaluation of the scan (``chunked_scan``: per-chunk affine state maps
  and causal kernel matrices, chunks combined by a prefix-doubling scan; plain
  PyTorch fp64) at several chunk lengths (invariant I1), and its reverse-mode
  automatic differentiation for the seven gradients;
* chaining two calls through the final state (I1b);
* ``scipy.signal.lfilter`` on the scalar special case (I2);
* central finite differences of the forward for all seven gradients (I3);
* the local d_da identity of the combined_backward.rs page's CombinedGrads docs
  (gradient w.r.t. the within-chunk cumsum through the chunk's own terms equals
  out_x . dout - ddt . dt), on the chunked evaluation, with out_x from the oracle (I4);
* Euler / linearity identities that hold exactly for this scan (I5);
* closed forms for dt = 0, for a memoryless decay and for an empty sequence;
* a hand-worked three-token example (``golden/hand_worked_p1r1_seq3.json``).

Shapes use headdim != dstate so a transposed operand cannot pass unnoticed.
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


def tiny(batch=2, seq=16, nheads=2, headdim=3, dstate=5, chunk_len=4, init_std=0.5, seed=11,
         dt_shift=1.0):
    w = inputs.custom(batch=batch, seq=seq, nheads=nheads, headdim=headdim, dstate=dstate,
                      chunk_len=chunk_len, init_std=init_std, seed=seed, dt_shift=dt_shift)
    t = inputs.make_inputs(w)
    return {k: v.double().numpy() for k, v in t.items()}


def rechunk(inp, l):
    """The same tokens laid out with chunk length ``l``."""
    out = dict(inp)
    b, n, L, h, p = inp["x"].shape
    seq = n * L
    assert seq % l == 0
    for k in ("x", "dy", "B", "C"):
        a = inp[k]
        out[k] = a.reshape(b, seq // l, l, h, a.shape[-1])
    out["dt"] = inp["dt"].reshape(b, h, seq // l, l)
    return out


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0)


def fwd(i):
    return oracle.ssd_fwd(i["x"], i["dt"], i["A"], i["B"], i["C"], i["D"], i["init"])


def bwd(i, d_final=True, seg=256):
    return oracle.ssd_bwd(i["dy"], i["d_final"] if d_final else None, i["x"], i["dt"], i["A"],
                          i["B"], i["C"], i["D"], i["init"], seg=seg)


GRADS = ("d_x", "d_dt", "d_A", "d_B", "d_C", "d_D", "d_init")


# ----------------------------------------------------------------- forward pins
@pytest.mark.parametrize("l", [1, 2, 4, 8, 16])
def test_I1_chunked_forward_matches_recurrence(l):
    i = rechunk(tiny(), l)
    y, fin = fwd(i)
    y2, fin2 = chunked_scan.forward(i["x"], i["dt"], i["A"], i["B"], i["C"], i["D"], i["init"])
    assert rel(y, y2) < 1e-12
    assert rel(fin, fin2) < 1e-12


def test_I1b_two_chained_calls_equal_one():
    i = tiny(seq=16, chunk_len=4)
    y, fin = fwd(i)
    first = {k: v for k, v in i.items()}
    first["x"], first["B"], first["C"] = (i[k][:, :2] for k in ("x", "B", "C"))
    first["dt"] = i["dt"][:, :, :2]
    ya, fa = fwd(first)
    second = dict(first)
    second["x"], second["B"], second["C"] = (i[k][:, 2:] for k in ("x", "B", "C"))
    second["dt"] = i["dt"][:, :, 2:]
    second["init"] = fa
    yb, fb = fwd(second)
    assert rel(np.concatenate([ya, yb], axis=1), y) < 1e-13
    assert rel(fb, fin) < 1e-13


def test_I2_scalar_case_is_a_first_order_iir_filter():
    scipy_signal = pytest.importorskip("scipy.signal")
    rng = np.random.default_rng(3)
    seq = 64
    x = rng.standard_normal(seq)
    Bv = rng.standard_normal(seq)
    Cv = rng.standard_normal(seq)
    dt = 0.3
    A = -1.7
    D = 0.25
    a = math.exp(dt * A)
    h = scipy_signal.lfilter([1.0], [1.0, -a], dt * x * Bv)
    y_ref = Cv * h + D * x
    y, fin = oracle.ssd_fwd(x.reshape(1, 1, seq, 1, 1), np.full((1, 1, 1, seq), dt),
                            np.array([A]), Bv.reshape(1, 1, seq, 1, 1),
                            Cv.reshape(1, 1, seq, 1, 1), np.array([D]), None)
    assert np.max(np.abs(y.ravel() - y_ref)) < 1e-12
    assert abs(fin.ravel()[0] - h[-1]) < 1e-12


def test_dt_zero_keeps_the_initial_state():
    i = tiny()
    i["dt"] = np.zeros_like(i["dt"])
    y, fin = fwd(i)
    # a = 1 and no input: h_t = init for all t
    y_ref = np.einsum("bnlhr,bhpr->bnlhp", i["C"], i["init"]) + i["D"][None, None, None, :, None] * i["x"]
    assert rel(y, y_ref) < 1e-14
    assert rel(fin, i["init"]) == 0.0
    g = bwd(i)
    assert rel(g["d_x"], i["dy"] * i["D"][None, None, None, :, None]) < 1e-14


def test_memoryless_decay_closed_form():
    i = tiny()
    i["A"] = np.full_like(i["A"], -1.0e4)
    i["dt"] = 0.5 + 0.5 * np.abs(i["dt"])  # dt*A < -5000: exp underflows to exactly 0
    y, fin = fwd(i)
    b, n, l, h, p = i["x"].shape
    dt_tok = np.transpose(i["dt"], (0, 2, 3, 1))  # [b,n,l,h]
    bc = np.einsum("bnlhr,bnlhr->bnlh", i["B"], i["C"])
    y_ref = (dt_tok * bc)[..., None] * i["x"] + i["D"][None, None, None, :, None] * i["x"]
    assert rel(y, y_ref) < 1e-14
    fin_ref = np.einsum("bhp,bhr->bhpr", dt_tok[:, -1, -1][..., None] * i["x"][:, -1, -1],
                        i["B"][:, -1, -1])
    assert rel(fin, fin_ref) < 1e-14


def test_empty_sequence():
    i = tiny()
    e = dict(i)
    for k in ("x", "dy", "B", "C"):
        e[k] = i[k][:, :0]
    e["dt"] = i["dt"][:, :, :0]
    y, fin = fwd(e)
    assert y.size == 0
    assert np.array_equal(fin, i["init"])
    g = bwd(e)
    assert np.array_equal(g["d_init"], i["d_final"])
    assert np.all(g["d_A"] == 0) and np.all(g["d_D"] == 0)


def test_golden_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_p1r1_seq3.json")) as f:
        gold = json.load(f)
    tol = gold["tolerance_abs"]
    inp = {k: np.asarray(v, dtype=np.float64) for k, v in gold["inputs"].items()}
    x = inp["x"].reshape(1, 3, 1, 1, 1)
    B = inp["B"].reshape(1, 3, 1, 1, 1)
    C = inp["C"].reshape(1, 3, 1, 1, 1)
    dt = inp["dt"].reshape(1, 1, 3, 1)
    init = inp["init"].reshape(1, 1, 1, 1)
    y, fin = oracle.ssd_fwd(x, dt, inp["A"], B, C, inp["D"], init)
    e = gold["expected"]
    ln2 = math.log(2.0)
    assert np.allclose(y.ravel(), e["y"], atol=tol, rtol=0)
    assert np.allclose(fin.ravel(), e["final"], atol=tol, rtol=0)
    g = oracle.ssd_bwd(inp["dy"].reshape(1, 3, 1, 1, 1), inp["d_final"].reshape(1, 1, 1, 1), x, dt,
                       inp["A"], B, C, inp["D"], init)
    d_dt = np.asarray(e["d_dt"]["const"]) + ln2 * np.asarray(e["d_dt"]["ln2_coeff"])
    assert np.allclose(g["d_dt"].ravel(), d_dt, atol=tol, rtol=0)
    for k in ("d_x", "d_A", "d_B", "d_C", "d_D", "d_init"):
        assert np.allclose(g[k].ravel(), e[k], atol=tol, rtol=0), k


# ---------------------------------------------------------------- backward pins
@pytest.mark.parametrize("l", [1, 4, 16])
def test_chunked_backward_matches_reverse_recurrence(l):
    """The oracle's reverse recurrence == autodiff of the chunked evaluation."""
    i = rechunk(tiny(), l)
    g = bwd(i)
    ref = chunked_scan.backward(i["dy"], i["d_final"], i["x"], i["dt"], i["A"], i["B"], i["C"],
                                i["D"], i["init"])
    for k in GRADS:
        assert rel(g[k], ref[k]) < 1e-11, k


def test_I3_finite_differences_all_seven_gradients():
    i = tiny(batch=1, seq=8, nheads=2, headdim=3, dstate=2, chunk_len=4, seed=5)
    g = bwd(i)

    def loss(inp):
        y, fin = fwd(inp)
        return float(np.sum(y * inp["dy"]) + np.sum(fin * inp["d_final"]))

    names = dict(x="d_x", dt="d_dt", A="d_A", B="d_B", C="d_C", D="d_D", init="d_init")
    for src, gname in names.items():
        base = i[src]
        fd = np.empty_like(base)
        flat = base.reshape(-1)
        for j in range(flat.size):
            v = flat[j]
            eps = 1e-6 * max(1.0, abs(v))
            plus = dict(i)
            minus = dict(i)
            plus[src] = base.copy()
            minus[src] = base.copy()
            plus[src].reshape(-1)[j] = v + eps
            minus[src].reshape(-1)[j] = v - eps
            fd.reshape(-1)[j] = (loss(plus) - loss(minus)) / (2 * eps)
        err = np.max(np.abs(fd - g[gname])) / max(1e-30, np.max(np.abs(g[gname])))
        assert err < 1e-6, (gname, err)


def test_I4_local_dda_identity_of_the_page():
    """d_da_local[t] = sum_p dy[t,p] out_x[t,p] - d_dt_orange[t] dt[t], out_x = y - D x:
    the gradient w.r.t. the within-chunk cumsum through the chunk's own terms (entry-state
    read-out and causal kernel) against the one w.r.t. dt through the kernel's source
    weight, both by autodiff of the chunked evaluation; out_x from the oracle."""
    i = tiny(seq=32, chunk_len=8)
    d_local, d_dt_kernel = chunked_scan.local_gradients(i["dy"], i["x"], i["dt"], i["A"], i["B"],
                                                        i["C"], i["init"])
    y, _ = fwd(i)  # the oracle's y: ties the identity to the recurrence
    out_x = y - i["D"][None, None, None, :, None] * i["x"]
    rhs = np.transpose(np.einsum("bnlhp,bnlhp->bnlh", i["dy"], out_x), (0, 3, 1, 2)) \
        - d_dt_kernel * i["dt"]
    assert np.max(np.abs(d_local - rhs)) < 1e-12 * max(1.0, np.max(np.abs(d_local)))


def _dot(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


def test_I5_euler_identities():
    i = tiny(seq=32, chunk_len=8)
    y, fin = fwd(i)
    g = bwd(i)
    Dx = i["D"][None, None, None, :, None] * i["x"]
    L = _dot(i["dy"], y) + _dot(i["d_final"], fin)
    # (i) linear in (x, init)
    assert abs(_dot(g["d_x"], i["x"]) + _dot(g["d_init"], i["init"]) - L) < 1e-12 * abs(L)
    # (ii) linear in C
    yc = _dot(i["dy"], y - Dx)
    assert abs(_dot(g["d_C"], i["C"]) - yc) < 1e-12 * abs(yc)
    # (iii) linear in D
    assert abs(_dot(i["D"], g["d_D"]) - _dot(i["dy"], Dx)) < 1e-12 * abs(_dot(i["dy"], Dx))
    # (iv), (v) need a zero initial state
    z = dict(i)
    z["init"] = np.zeros_like(i["init"])
    y0, f0 = fwd(z)
    g0 = bwd(z)
    rhs = _dot(z["dy"], y0 - Dx) + _dot(z["d_final"], f0)
    assert abs(_dot(g0["d_B"], z["B"]) - rhs) < 1e-12 * abs(rhs)
    lhs = _dot(z["dt"], g0["d_dt"]) - _dot(z["A"], g0["d_A"])
    assert abs(lhs - rhs) < 1e-12 * abs(rhs)


@pytest.mark.parametrize("seg", [1, 3, 7, 1000])
def test_checkpoint_segment_length_does_not_change_the_gradients(seg):
    i = tiny(seq=32, chunk_len=8)
    ref = bwd(i, seg=32)
    g = bwd(i, seg=seg)
    for k in GRADS:
        assert rel(g[k], ref[k]) < 1e-14, k


def test_null_d_final_means_zero():
    i = tiny()
    z = dict(i)
    z["d_final"] = np.zeros_like(i["d_final"])
    a = bwd(i, d_final=False)
    b = bwd(z)
    for k in GRADS:
        assert np.array_equal(a[k], b[k]), k
