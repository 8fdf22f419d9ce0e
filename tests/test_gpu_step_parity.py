"""GPU parity of ssd_step (the decode step) against the CPU oracle.

One token of the recurrence from a cached state, through the C ABI, on seeded
inputs: every p / r width class, fp32 and bf16 (the oracle sees the same
bf16-rounded values), odd head counts, out of place and in place (bitwise
equal); the two decode workloads in full (the oracle step is cheap); 48 chained
steps against the oracle forward over those 48 tokens and against the device's
own chunked forward; an empty batch.  Bar: per-tensor relative L2 <= 1e-5
(fp32 inputs) and <= 2e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL, compare, rel_l2, say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

KEYS = ("y", "new_state")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


def gpu_step(i, in_place=False):
    d = {k: v.cuda() for k, v in i.items()}
    y, ns = ssd.step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["state"], in_place=in_place)
    torch.cuda.synchronize()
    return dict(y=y.float().cpu().numpy(), new_state=ns.cpu().numpy())


def oracle_step(i):
    y, ns = oracle.ssd_step(*(i[k].double().numpy() for k in ("x", "dt", "A", "B", "C", "D", "state")))
    return dict(y=y, new_state=ns)


SHAPES = [
    # batch, nheads, headdim, dstate, io
    (1, 2, 16, 16, "f32"),
    (3, 5, 32, 64, "f32"),
    (2, 3, 64, 128, "f32"),
    (4, 7, 128, 32, "f32"),
    (2, 1, 16, 128, "f32"),
    (3, 4, 64, 128, "bf16"),
    (2, 3, 128, 16, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{s[0]}_h{s[1]}_p{s[2]}_r{s[3]}_{s[4]}" for s in SHAPES])
def test_step_shapes(shape):
    b, h, p, r, io = shape
    w = inputs.StepWorkload("t", b, h, p, r, io=io, seed=40 + p + r)
    say(f"step parity {shape}")
    i = inputs.make_step_inputs(w)
    out = gpu_step(i)
    compare(out, oracle_step(i), TOL[io], KEYS, f"step {shape}")
    inp = gpu_step(i, in_place=True)
    for k in KEYS:
        assert np.array_equal(out[k], inp[k]), f"in-place {k} differs from out-of-place"


@pytest.mark.parametrize("name", list(inputs.STEP_WORKLOADS))
def test_step_full_workloads(name):
    w = inputs.STEP_WORKLOADS[name]
    say(f"step parity {w.describe()}")
    i = inputs.make_step_inputs(w)
    compare(gpu_step(i), oracle_step(i), TOL[w.io], KEYS, name)


def test_chained_steps_match_the_chunked_forward():
    # 48 decode steps from a cached state == one forward over the 48 tokens (oracle and device)
    w = inputs.custom(name="chain", batch=2, seq=64, nheads=3, headdim=32, dstate=64, chunk_len=64,
                      init_std=0.5, seed=77)
    t = inputs.make_inputs(w)
    S = 48
    x, dt, B, C = t["x"][:, 0, :S], t["dt"][:, :, 0, :S], t["B"][:, 0, :S], t["C"][:, 0, :S]
    d = {k: v.cuda() for k, v in dict(x=x, dt=dt, B=B, C=C, A=t["A"], D=t["D"], init=t["init"]).items()}
    state = d["init"].clone()
    ys = []
    for s in range(S):
        y, state = ssd.step(d["x"][:, s].contiguous(), d["dt"][:, :, s].contiguous(), d["A"],
                            d["B"][:, s].contiguous(), d["C"][:, s].contiguous(), d["D"], state,
                            in_place=True)
        ys.append(y)
    torch.cuda.synchronize()
    y_steps = torch.stack(ys, 1).cpu().numpy()  # [b, S, h, p]
    fin_steps = state.cpu().numpy()
    # the oracle forward over the same 48 tokens (one chunk of 48)
    ry, rfin = oracle.ssd_fwd(x[:, None].numpy(), dt[:, :, None].numpy(), t["A"].numpy(),
                              B[:, None].numpy(), C[:, None].numpy(), t["D"].numpy(), t["init"].numpy())
    compare(dict(y=y_steps, final=fin_steps), dict(y=ry[:, 0], final=rfin), TOL["f32"], ("y", "final"),
            "48 steps vs oracle forward")
    # the device's chunked forward over the full 64-token chunk: its first 48 outputs
    fy, _ = ssd.forward(*(t[k].cuda() for k in ("x", "dt", "A", "B", "C", "D", "init")))
    torch.cuda.synchronize()
    e = rel_l2(y_steps, fy.cpu().numpy()[:, 0, :S])
    say(f"  48 steps vs ssd_fwd: y rel-L2 {e:.2e}")
    assert e <= TOL["f32"]


def test_step_empty_batch():
    x = torch.zeros((0, 3, 16), device="cuda")
    B = torch.zeros((0, 3, 16), device="cuda")
    st = torch.zeros((0, 3, 16, 16), device="cuda")
    y, ns = ssd.step(x, torch.zeros((0, 3), device="cuda"), torch.zeros(3, device="cuda"), B, B,
                     torch.zeros(3, device="cuda"), st)
    assert y.numel() == 0 and ns.numel() == 0


def draw_step_cases(seed=20261205, n=16):
    """Random decode steps from one fixed seed: batch and head counts, every headdim /
    dstate, io type, and a cached state of scale 0, 0.5 or 2."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        p, r = (int(v) for v in rng.choice([16, 32, 64, 128], 2))
        cases.append((int(rng.integers(1, 7)), int(rng.integers(1, 9)), p, r,
                      ["f32", "bf16"][rng.integers(2)], float(rng.choice([0.0, 0.5, 2.0])),
                      int(rng.integers(1 << 30))))
    return cases


STEP_CASES = draw_step_cases()


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"b{c[0]}_h{c[1]}_p{c[2]}_r{c[3]}_{c[4]}_s{c[5]:g}"
                                                  for c in STEP_CASES])
def test_step_random_case(case):
    b, h, p, r, io, state_std, seed = case
    w = inputs.StepWorkload("sweep", b, h, p, r, io=io, state_std=state_std, seed=seed)
    say(f"step sweep case {case}")
    i = inputs.make_step_inputs(w)
    out = gpu_step(i)
    compare(out, oracle_step(i), TOL[io], KEYS, f"step sweep {case}")
    inp = gpu_step(i, in_place=True)
    for k in KEYS:
        assert np.array_equal(out[k], inp[k]), f"in-place {k} differs from out-of-place"
