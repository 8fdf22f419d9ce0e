"""The GPU parity checkers themselves, on the CPU: the per-block error bound and the
all-heads identity check of ``gpu_common`` accept the oracle's own outputs and reject
a mistake confined to one chunk or one head (no GPU needed; the oracle's results stand
in for the device's)."""
import numpy as np
import pytest

import oracle
from gpu_common import TOL, check_identities_all_heads, compare
from mamba_ssd_chunked_amd import inputs


def _oracle_outputs(w, use_init, use_d_final):
    t = inputs.make_inputs(w)
    n = lambda k: t[k].double().numpy()  # noqa: E731
    init = n("init") if use_init else None
    df = n("d_final") if use_d_final else None
    y, fin = oracle.ssd_fwd(n("x"), n("dt"), n("A"), n("B"), n("C"), n("D"), init)
    g = oracle.ssd_bwd(n("dy"), df, n("x"), n("dt"), n("A"), n("B"), n("C"), n("D"), init)
    out = dict(y=y, final=fin)
    out.update(g)
    return t, {k: v.astype(np.float32) for k, v in out.items()}, out


W = inputs.custom(batch=2, seq=256, nheads=3, headdim=16, dstate=32, chunk_len=64, seed=31)


@pytest.mark.parametrize("use_init,use_d_final", [(False, False), (False, True), (True, False)])
def test_identities_hold_on_the_oracle_outputs(use_init, use_d_final):
    w = inputs.Workload(**{**W.__dict__, "init_std": 0.3 if use_init else 0.0})
    t, f32, _ = _oracle_outputs(w, use_init, use_d_final)
    worst = check_identities_all_heads(t, f32, TOL["f32"], use_init, use_d_final, "oracle")
    assert max(worst.values()) < 1e-6
    assert ("v" in worst) == (not use_init)


@pytest.mark.parametrize("kind", ["wrong_head", "scaled"])
@pytest.mark.parametrize("key", ["d_x", "d_C", "d_B", "d_dt", "d_A", "d_D", "y"])
def test_identities_catch_one_wrong_head(key, kind):
    """One head's output taken from another head (an indexing mistake), or off by 10 %.
    The residuals are scaled by Cauchy-Schwarz bounds, which outputs within the per-tensor
    tolerance can never exceed; small per-head errors are left to the per-block comparison
    with the oracle on the sampled heads."""
    t, f32, _ = _oracle_outputs(W, False, False)
    bad = dict(f32)
    v = f32[key].copy()
    if key in ("d_A", "d_D"):
        v[1] = v[0] if kind == "wrong_head" else 1.1 * v[1]
    elif key == "d_dt":
        v[:, 1] = v[:, 0] if kind == "wrong_head" else 1.1 * v[:, 1]
    else:
        v[:, :, :, 1] = v[:, :, :, 0] if kind == "wrong_head" else 1.1 * v[:, :, :, 1]
    bad[key] = v
    with pytest.raises(AssertionError):
        check_identities_all_heads(t, bad, TOL["f32"], False, False, "planted")


def test_block_bound_catches_an_error_in_one_chunk():
    _, f32, ref = _oracle_outputs(W, False, False)
    compare(f32, ref, TOL["f32"], ("y", "d_x", "d_dt", "final"), "clean")
    bad = dict(f32)
    bad["d_x"] = f32["d_x"].copy()
    bad["d_x"][1, 2, :, 0] *= 1.0005  # one (batch, chunk, head) block of 24: 5e-4 there
    from gpu_common import rel_l2
    assert rel_l2(bad["d_x"], ref["d_x"]) < 2e-4  # ... diluted to about 1e-4 per tensor
    compare(bad, ref, 2e-4, ("d_x",), "planted", block_tol=1e-3)
    with pytest.raises(AssertionError, match="block"):
        compare(bad, ref, 2e-4, ("d_x",), "planted", block_tol=4e-4)
