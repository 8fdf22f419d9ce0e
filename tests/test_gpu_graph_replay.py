"""HIP-graph capture of the moments, participation-ratio, same-step-correction and decode
entry points (needs an MI355X).

The library neither allocates nor synchronises and launches nothing but its own kernels,
so each call sequence below can be captured into a graph.  Every replay, with eager work
of the program and a device synchronisation in between, must reproduce the eager
outputs bit for bit (the outputs are overwritten with NaN before each replay).  The
fwd + bwd SSD step and the quaternion scan have their own replay tests beside their
parity tests.
"""
import numpy as np
import pytest
import torch

from gpu_common import say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


def replay_matches_eager(step, outs, label):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(REPLAYS):
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"{label}: output {k} differs on replay {it}"
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_moments_and_pr_loop_graph_replay():
    """ssd_state_moments (with y and the final state) -> ssd_moments_pr (centred) ->
    ssd_moments_pr_bwd -> ssd_state_moments_bwd fed the PR gradient, one captured graph."""
    w = inputs.custom(batch=2, seq=512, nheads=3, headdim=32, dstate=64, chunk_len=128,
                      init_std=0.3, valid_len=(512, 300), seed=61)
    inp = inputs.make_inputs(w)
    say("case graph capture of the moments / PR loop")
    d = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "valid_len"}
    valid = inp["valid_len"].clone()
    dims = ssd.dims_of(d["x"], d["B"])
    b, h, r = w.batch, w.nheads, w.dstate
    m2 = torch.empty((b, h, r, r), device="cuda")
    m1 = torch.empty((b, h, r), device="cuda")
    count = torch.empty((b,), dtype=torch.int64)
    y = torch.empty_like(d["x"])
    fin = torch.empty_like(d["init"])
    pr = torch.empty((b, h), device="cuda")
    trace = torch.empty((b, h), device="cuda")
    d_pr = torch.ones((b, h), device="cuda")
    d_m2 = torch.empty_like(m2)
    d_m1 = torch.empty_like(m1)
    gx, gB = torch.empty_like(d["x"]), torch.empty_like(d["B"])
    gdt, gA = torch.empty_like(d["dt"]), torch.empty_like(d["A"])
    ginit = torch.empty_like(d["init"])
    wf = ssd.workspace(dims, ssd.SSD_OP_MOMENTS)
    wb = ssd.workspace(dims, ssd.SSD_OP_MOMENTS_BWD)
    # the count is a host output; the PR calls read the eager call's value
    assert ssd.ssd_state_moments(dims, d["x"], d["dt"], d["A"], d["B"], d["init"], valid, m2, m1,
                                 count, y, d["C"], d["D"], fin, wf) == 0
    torch.cuda.synchronize()
    cnt = count.clone()

    def step():
        st = torch.cuda.current_stream()
        assert ssd.ssd_state_moments(dims, d["x"], d["dt"], d["A"], d["B"], d["init"], valid, m2,
                                     m1, count, y, d["C"], d["D"], fin, wf, st) == 0
        assert ssd.ssd_moments_pr(b, h, r, m2, m1, cnt, True, pr, trace, st) == 0
        assert ssd.ssd_moments_pr_bwd(b, h, r, d_pr, m2, m1, cnt, True, d_m2, d_m1, st) == 0
        assert ssd.ssd_state_moments_bwd(dims, d_m2, d_m1, d["x"], d["dt"], d["A"], d["B"],
                                         d["init"], valid, gx, gdt, gA, gB, ginit, wb, st) == 0

    outs = [m2, m1, y, fin, pr, trace, d_m2, d_m1, gx, gdt, gA, gB, ginit]
    replay_matches_eager(step, outs, "moments / PR loop")
    assert np.all(np.isfinite(gx.cpu().numpy())) and torch.equal(count, cnt)


@pytest.mark.parametrize("mimo", [1, 4])
def test_y_diag_graph_replay(mimo):
    w = inputs.DiagWorkload("graph", 2, 256, 64, mimo, 3, 64, 128, seed=62 + mimo)
    say(f"case graph capture of ssd_y_diag + ssd_y_diag_bwd, mimo rank {mimo}")
    d = {k: v.cuda() for k, v in inputs.make_diag_inputs(w).items()}
    y = torch.empty_like(d["v"])
    dv, dB, dC = torch.empty_like(d["v"]), torch.empty_like(d["B"]), torch.empty_like(d["C"])
    dg = torch.empty_like(d["gamma"])

    def step():
        st = torch.cuda.current_stream()
        assert ssd.ssd_y_diag(d["v"], d["B"], d["C"], d["gamma"], y, st) == 0
        assert ssd.ssd_y_diag_bwd(d["dy"], d["v"], d["B"], d["C"], d["gamma"], dv, dB, dC, dg,
                                  st) == 0

    replay_matches_eager(step, [y, dv, dB, dC, dg], f"y_diag m={mimo}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_step_graph_replay(io):
    """Out of place, so every replay starts from the same cached state."""
    w = inputs.StepWorkload("graph", 16, 5, 64, 128, io=io, seed=64)
    say(f"case graph capture of ssd_step, {io}")
    d = {k: v.cuda() for k, v in inputs.make_step_inputs(w).items()}
    y = torch.empty_like(d["x"])
    new_state = torch.empty_like(d["state"])

    def step():
        st = torch.cuda.current_stream()
        assert ssd.ssd_step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["state"], new_state,
                            y, st) == 0

    replay_matches_eager(step, [y, new_state], f"decode step {io}")
