"""Debug mode of the C ABI (needs an MI355X): with ssd_debug_enable(1) the SSD and
moments entry points scan their outputs and return SSD_ERR_NONFINITE when one holds a
NaN or an infinity; finite results are unchanged bit for bit, and with the mode off the
same calls return 0."""
import pytest
import torch

from gpu_common import say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

NONFINITE = 7


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


@pytest.fixture()
def debug_on():
    assert ssd.ssd_debug_enable(True) == 0
    try:
        yield
    finally:
        ssd.ssd_debug_enable(False)


def _case(seed=71, valid=None):
    w = inputs.custom(batch=2, seq=256, nheads=2, headdim=32, dstate=64, chunk_len=128,
                      init_std=0.3, valid_len=valid, seed=seed)
    inp = inputs.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "valid_len"}
    return w, inp, d


def _fwd_bwd(d):
    dims = ssd.dims_of(d["x"], d["B"])
    y, fin = torch.empty_like(d["x"]), torch.empty_like(d["d_final"])
    g = [torch.empty_like(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "d_final")]
    rf = ssd.ssd_fwd(dims, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init"], y, fin,
                     ssd.workspace(dims, ssd.SSD_OP_FWD))
    mf = ssd.ssd_last_error()
    rb = ssd.ssd_bwd(dims, d["dy"], d["d_final"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                     d["init"], *g, ssd.workspace(dims, ssd.SSD_OP_BWD))
    mb = ssd.ssd_last_error()
    torch.cuda.synchronize()
    return (rf, mf, rb, mb), [y, fin] + g


def test_finite_results_pass_and_are_unchanged(debug_on):
    say("case debug mode, finite inputs")
    _, _, d = _case()
    (rf, _, rb, _), outs = _fwd_bwd(d)
    assert rf == 0 and rb == 0
    ssd.ssd_debug_enable(False)
    (rf2, _, rb2, _), ref = _fwd_bwd(d)
    assert rf2 == 0 and rb2 == 0
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)


def test_nan_input_is_reported_and_only_in_debug_mode(debug_on):
    say("case debug mode, NaN in x and in dy")
    _, _, d = _case()
    d["x"][1, 0, 5, 1, 3] = float("nan")
    (rf, mf, rb, mb), _ = _fwd_bwd(d)
    assert rf == NONFINITE and "ssd_fwd" in mf and " y " in mf, mf
    assert rb == NONFINITE and "ssd_bwd" in mb, mb
    _, _, d2 = _case()
    d2["dy"][0, 1, 7, 0, 2] = float("inf")
    (rf, _, rb, mb), _ = _fwd_bwd(d2)
    assert rf == 0 and rb == NONFINITE and "d_x" in mb, mb
    ssd.ssd_debug_enable(False)
    (rf, _, rb, _), _ = _fwd_bwd(d)
    assert rf == 0 and rb == 0


def test_moments_outputs_are_checked(debug_on):
    say("case debug mode, moments with a NaN step")
    w, inp, d = _case(valid=(256, 200))
    valid = inp["valid_len"].clone()
    d["dt"][0, 1, 0, 4] = float("nan")
    mo_rc = None
    try:
        ssd.state_moments(d["x"], d["dt"], d["A"], d["B"], d["init"], valid_len=valid)
    except ssd.SsdError as e:
        mo_rc = e.code
    assert mo_rc == NONFINITE
    ssd.ssd_debug_enable(False)
    out = ssd.state_moments(d["x"], d["dt"], d["A"], d["B"], d["init"], valid_len=valid)
    torch.cuda.synchronize()
    assert not torch.isfinite(out["m2"]).all()
