"""Pins of the oracle's decode step (no GPU).

One decode step from the cached state is the recurrence's per-token body
h <- exp(dt A) h + dt x (outer) B, y = C . h + D x (the token-by-token ``step``
loop the burn-mamba state_moments.rs page refers to); the oracle takes it as
the forward over one token with init = the state.  Checked against:

* the hand-worked three-token example (tests/golden/hand_worked_p1r1_seq3.json),
  stepped token by token from a zero state;
* the oracle forward over S tokens: S chained steps give its y and final state
  (this pins the layout changes between [b, h, ...] and [b, n, l, h, ...]);
* closed forms: dt = 0 leaves the state unchanged; a memoryless decay
  (A = -1e4) replaces it by dt x (outer) B.
"""
import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_example_step_by_step():
    g = json.load(open(os.path.join(HERE, "golden", "hand_worked_p1r1_seq3.json")))
    i, e = g["inputs"], g["expected"]
    state = np.zeros((1, 1, 1, 1))
    ys = []
    for t in range(3):
        y, state = oracle.ssd_step(np.full((1, 1, 1), i["x"][t]), np.full((1, 1), i["dt"][t]),
                                   np.array(i["A"]), np.full((1, 1, 1), i["B"][t]),
                                   np.full((1, 1, 1), i["C"][t]), np.array(i["D"]), state)
        ys.append(float(y[0, 0, 0]))
    np.testing.assert_allclose(ys, e["y"], rtol=1e-15)
    np.testing.assert_allclose(state.ravel(), e["final"], rtol=1e-15)


def test_chained_steps_equal_the_forward():
    rng = np.random.default_rng(0)
    b, S, h, p, r = 2, 9, 3, 4, 5
    x = rng.standard_normal((b, S, 1, h, p))
    dt = np.log1p(np.exp(rng.standard_normal((b, h, S, 1)) - 2))
    A = -np.exp(rng.uniform(0, np.log(16), h))
    B = rng.standard_normal((b, S, 1, h, r)) / np.sqrt(r)
    C = rng.standard_normal((b, S, 1, h, r)) / np.sqrt(r)
    D = rng.standard_normal(h)
    init = 0.3 * rng.standard_normal((b, h, p, r))
    y_ref, fin_ref = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    state = init.copy()
    for t in range(S):
        y, state = oracle.ssd_step(x[:, t, 0], dt[:, :, t, 0], A, B[:, t, 0], C[:, t, 0], D, state)
        np.testing.assert_allclose(y, y_ref[:, t, 0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(state, fin_ref, rtol=1e-13, atol=1e-15)


def test_closed_forms():
    rng = np.random.default_rng(1)
    b, h, p, r = 2, 2, 3, 4
    x = rng.standard_normal((b, h, p))
    B = rng.standard_normal((b, h, r))
    C = rng.standard_normal((b, h, r))
    D = rng.standard_normal(h)
    state = rng.standard_normal((b, h, p, r))
    A = -np.ones(h)
    # dt = 0: nothing is written or forgotten
    y, s2 = oracle.ssd_step(x, np.zeros((b, h)), A, B, C, D, state)
    np.testing.assert_array_equal(s2, state)
    np.testing.assert_allclose(y, np.einsum("bhpr,bhr->bhp", state, C) + D[None, :, None] * x,
                               rtol=1e-14)
    # memoryless decay: the state is replaced by the write dt x (outer) B
    dt = np.full((b, h), 0.5)
    _, s3 = oracle.ssd_step(x, dt, np.full(h, -1e4), B, C, D, state)
    np.testing.assert_allclose(s3, 0.5 * x[..., :, None] * B[..., None, :], rtol=1e-14)
