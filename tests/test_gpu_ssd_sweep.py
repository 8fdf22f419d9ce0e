"""A seeded sweep of random SSD problems: ssd_fwd / ssd_bwd against the CPU oracle.

The hand-picked cases of test_gpu_ssd_parity cover each kernel variant on purpose;
this sweep draws its cases from one fixed seed over every combination the C ABI
accepts -- io type, headdim and dstate in {16, 32, 64, 128}, chunk_len in {64, 128,
256} with a kernel chunk length that divides it (or the automatic one), one to three
chunks, batch and head counts, a random or zero initial state, a d_final or none,
and the step distribution (dt = softplus(z - shift) with shift 1, 2 or 4) -- so that
combinations nobody listed still meet the oracle.  Sizes are capped so the oracle
finishes each case in well under a second.  Bar: the parity tolerance of the
hand-picked cases (per-tensor relative L2 1e-5 fp32, 2e-2 bf16, plus the per-block
bounds of gpu_common.compare).
"""
import numpy as np
import pytest
import torch

from gpu_common import GRADS, TOL, compare, gpu_fwd_bwd, oracle_fwd_bwd, say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

KEYS = ("y", "final") + GRADS
N_CASES = 48
MAX_WORK = 1 << 24  # batch * seq * nheads * headdim * dstate


def draw_cases(seed=20261202, n=N_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        io = ["f32", "bf16"][rng.integers(2)]
        p, r = (int(v) for v in rng.choice([16, 32, 64, 128], 2))
        l = int(rng.choice([64, 128, 256]))
        kcl = int(rng.choice([0] + [k for k in (64, 128, 256) if k <= l and l % k == 0]))
        b, h, nch = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
        shift = float(rng.choice([1.0, 2.0, 4.0]))
        use_init, use_d_final = bool(rng.integers(2)), bool(rng.integers(2))
        if b * nch * l * h * p * r > MAX_WORK:
            continue
        cases.append((io, b, nch * l, h, p, r, l, kcl, shift, use_init, use_d_final,
                      int(rng.integers(1 << 30))))
    return cases


CASES = draw_cases()


def case_id(c):
    io, b, seq, h, p, r, l, kcl, shift, ui, ud, _ = c
    return f"{io}_b{b}_s{seq}_h{h}_p{p}_r{r}_l{l}_k{kcl}_sh{shift:g}_i{int(ui)}_f{int(ud)}"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_random_case(case):
    io, b, seq, h, p, r, l, kcl, shift, use_init, use_d_final, seed = case
    say(f"sweep case {case_id(case)} seed {seed}")
    w = inputs.custom(batch=b, seq=seq, nheads=h, headdim=p, dstate=r, chunk_len=l, io=io,
                      dt_shift=shift, init_std=0.5 if use_init else 0.0, seed=seed)
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp, use_init=use_init, use_d_final=use_d_final, kernel_chunk_len=kcl)
    ref = oracle_fwd_bwd(inp, use_init=use_init, use_d_final=use_d_final)
    compare(gpu, ref, TOL[io], KEYS, case_id(case))
