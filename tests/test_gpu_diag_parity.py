"""GPU parity of ssd_y_diag / ssd_y_diag_bwd against the CPU oracle.

The Mamba-3 same-step correction y_diag = gamma (C B^T) v per token and head
(burn-mamba mamba3 diag.rs page) and its four gradients, through the C ABI, on
seeded inputs: mimo ranks 1 (the SISO path), 2 and 4, every p / r width class,
fp32 and bf16 (the oracle sees the same bf16-rounded values), the two full-size
workloads on sampled tokens (the term is token-local, so the oracle computes
exactly those rows), linearity in each input on the device outputs, bitwise
determinism and an empty token set.  Bar: per-tensor relative L2 <= 1e-5 (fp32)
and <= 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL, compare, say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


def gpu_diag(i):
    d = {k: v.cuda() for k, v in i.items()}
    y = ssd.y_diag(d["v"], d["B"], d["C"], d["gamma"])
    g = ssd.y_diag_bwd(d["dy"], d["v"], d["B"], d["C"], d["gamma"])
    torch.cuda.synchronize()
    out = dict(y=y.float().cpu().numpy())
    out.update({k: t.float().cpu().numpy() for k, t in g.items()})
    return out


def oracle_diag(i):
    f = {k: v.double().numpy() for k, v in i.items()}
    y = oracle.diag_fwd(f["v"], f["B"], f["C"], f["gamma"])
    g = oracle.diag_bwd(f["dy"], f["v"], f["B"], f["C"], f["gamma"])
    return dict(y=y, d_v=g["d_v"], d_B=g["d_b"], d_C=g["d_c"], d_gamma=g["d_gamma"])


KEYS = ("y", "d_v", "d_B", "d_C", "d_gamma")
SHAPES = [
    # batch, seq, chunk_len, mimo_rank, nheads, headdim, dstate, io
    (1, 128, 64, 1, 2, 16, 16, "f32"),
    (2, 64, 64, 2, 3, 32, 64, "f32"),
    (1, 128, 64, 4, 5, 64, 128, "f32"),
    (2, 128, 128, 4, 2, 128, 32, "f32"),
    (1, 64, 64, 1, 3, 128, 128, "f32"),
    (1, 64, 64, 2, 7, 16, 128, "f32"),
    (2, 64, 64, 2, 3, 64, 128, "bf16"),
    (1, 64, 64, 4, 2, 64, 64, "bf16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_s%d_l%d_m%d_h%d_p%d_r%d_%s" % s)
def test_y_diag_matches_oracle(shape):
    b, seq, l, m, h, p, r, io = shape
    w = inputs.DiagWorkload("case", b, seq, l, m, h, p, r, io=io, seed=2000 + m * 7 + p + r)
    say(f"case y_diag {shape}")
    i = inputs.make_diag_inputs(w)
    compare(gpu_diag(i), oracle_diag(i), TOL[io], KEYS, f"y_diag {shape}")


@pytest.mark.parametrize("name", sorted(inputs.DIAG_WORKLOADS))
def test_y_diag_workload_sampled_tokens(name):
    w = inputs.DIAG_WORKLOADS[name]
    say(f"case y_diag workload {name}")
    i = inputs.make_diag_inputs(w)
    gpu = gpu_diag(i)
    # token-local: the first chunk of batch 0 and the last chunk of the last batch
    picks = [(0, 0), (w.batch - 1, w.seq // w.chunk_len - 1)]
    for bb, nn in picks:
        sub = {k: v[bb:bb + 1, nn:nn + 1] for k, v in i.items()}
        ref = oracle_diag(sub)
        got = {k: v[bb:bb + 1, nn:nn + 1] for k, v in gpu.items()}
        compare(got, ref, TOL[w.io], KEYS, f"{name} tokens of batch {bb} chunk {nn}")
    # linearity in each input, on the whole device output (fp64 sums on the host)
    f = {k: v.double().numpy() for k, v in i.items()}
    ref = float((f["dy"] * gpu["y"]).sum())
    for name_in, gname in (("v", "d_v"), ("B", "d_B"), ("C", "d_C"), ("gamma", "d_gamma")):
        got = float((f[name_in] * gpu[gname]).sum())
        assert abs(got - ref) <= 1e-5 * abs(ref), (name_in, got, ref)


def test_y_diag_determinism_and_empty():
    w = inputs.DiagWorkload("det", 2, 128, 64, 4, 3, 64, 128, seed=2100)
    say("case y_diag determinism / empty")
    i = inputs.make_diag_inputs(w)
    a, b = gpu_diag(i), gpu_diag(i)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k
    e = {k: v[:, :0].contiguous() for k, v in i.items()}
    out = gpu_diag(e)
    assert all(v.size == 0 for v in out.values())


def draw_diag_cases(seed=20261204, n=16):
    """Random same-step-correction problems from one fixed seed: mimo rank 1, 2 or 4, every
    headdim / dstate, io type, one or two chunks of 64 or 128 tokens, batch and head counts."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        l = int(rng.choice([64, 128]))
        p, r = (int(v) for v in rng.choice([16, 32, 64, 128], 2))
        cases.append((int(rng.integers(1, 4)), l * int(rng.integers(1, 3)), l,
                      int(rng.choice([1, 2, 4])), int(rng.integers(1, 7)), p, r,
                      ["f32", "bf16"][rng.integers(2)], int(rng.integers(1 << 30))))
    return cases


DIAG_CASES = draw_diag_cases()


@pytest.mark.parametrize("case", DIAG_CASES, ids=lambda c: "b%d_s%d_l%d_m%d_h%d_p%d_r%d_%s" % c[:8])
def test_y_diag_random_case(case):
    b, seq, l, m, h, p, r, io, seed = case
    w = inputs.DiagWorkload("sweep", b, seq, l, m, h, p, r, io=io, seed=seed)
    say(f"y_diag sweep case {case}")
    i = inputs.make_diag_inputs(w)
    compare(gpu_diag(i), oracle_diag(i), TOL[io], KEYS, f"y_diag sweep {case}")
