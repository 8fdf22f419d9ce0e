"""GPU parity of ssd_quat_scan / ssd_quat_scan_bwd against the CPU oracle.

The Mamba-3 quaternion cumulative-product scan cum[t] = q_t (x) cum[t-1]
(burn-mamba mamba3/quat_scan backward.rs page) and its exact reverse mode,
through the C ABI, on seeded inputs: one step; partial 64-lane groups and
ragged last segments; identity and random init; non-unit step quaternions;
chains of 32 to 1024 segments; the full-size workload on sampled heads
(lanes are independent, so the oracle computes exactly those outputs) plus the
unit-norm property on every output; workspace reuse across calls of different
sizes; empty sequence and batch; bitwise equality of repeated calls.  Bar:
per-tensor relative L2 <= 1e-5 (fp32 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL, compare, say
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

KEYS = ("cum", "d_q", "d_init")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


def gpu_quat(i, ws_fwd=None, ws_bwd=None):
    q = i["q"].cuda()
    init = i["init"].cuda() if i["init"] is not None else None
    dc = i["d_cum"].cuda()
    cum = ssd.quat_scan(q, init, ws=ws_fwd)
    d_q, d_init = ssd.quat_scan_bwd(q, init, dc, ws=ws_bwd)
    torch.cuda.synchronize()
    return dict(cum=cum.cpu().numpy(), d_q=d_q.cpu().numpy(), d_init=d_init.cpu().numpy())


def oracle_quat(i, heads=None):
    def sel(t, axis):
        if t is None:
            return None
        t = t.double().numpy()
        return t if heads is None else np.take(t, heads, axis=axis)
    q, init, dc = sel(i["q"], 2), sel(i["init"], 1), sel(i["d_cum"], 2)
    cum = oracle.quat_scan(q, init)
    d_q, d_init = oracle.quat_scan_bwd(q, init, dc)
    return dict(cum=cum, d_q=d_q, d_init=d_init)


SHAPES = [
    # batch, seq, nheads, nquat, norm_std, random_init
    (1, 1, 1, 1, 0.0, True),       # a single step
    (2, 37, 3, 5, 0.0, True),      # 15 lanes (part of one 64-lane group), ragged last segment
    (1, 32, 1, 64, 0.0, False),    # exactly one segment and one full group, identity init
    (2, 300, 2, 40, 0.0, True),    # 80 lanes: a full and a partial group, 10 segments
    (1, 1000, 4, 32, 0.0, True),   # 2 groups, 32 segments
    (3, 129, 5, 3, 0.05, True),    # non-unit steps (norms exp(0.05 z)), ragged
    (2, 64, 3, 7, 0.3, False),     # strongly non-unit steps, identity init
    (1, 4096, 1, 16, 0.0, False),  # 128-segment chains
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{s[0]}_s{s[1]}_h{s[2]}_j{s[3]}_n{s[4]}" for s in SHAPES])
def test_quat_small_shapes(shape):
    b, s, h, j, nstd, rinit = shape
    w = inputs.QuatWorkload("t", b, s, h, j, norm_std=nstd, random_init=rinit, seed=17 + s + j)
    say(f"quat parity {shape}")
    i = inputs.make_quat_inputs(w)
    compare(gpu_quat(i), oracle_quat(i), TOL["f32"], KEYS, f"quat {shape}")


def test_quat_full_workload_sampled_heads():
    w = inputs.QUAT_WORKLOADS["mamba3_quat_scan_fp32"]
    say(f"quat parity {w.describe()}")
    i = inputs.make_quat_inputs(w)
    g = gpu_quat(i)
    heads = [0, 11, 23]
    ref = oracle_quat(i, heads)
    sub = dict(cum=g["cum"][:, :, heads], d_q=g["d_q"][:, :, heads], d_init=g["d_init"][:, heads])
    compare(sub, ref, TOL["f32"], KEYS, "quat full workload, heads 0, 11, 23")
    # every output: the norm is multiplicative, |cum[t]| = prod_{s<=t} |q_s| |init|
    # (fp64 from the fp32 inputs, whose own norms are 1 only to fp32 rounding)
    qn = np.linalg.norm(i["q"].double().numpy(), axis=-1)
    expect = np.cumprod(qn, axis=1) * np.linalg.norm(i["init"].double().numpy(), axis=-1)[:, None]
    norms = np.linalg.norm(g["cum"].astype(np.float64), axis=-1)
    dev = np.abs(norms / expect - 1).max()
    say(f"  max | |cum| / (prod |q| |init|) - 1 | = {dev:.2e}")
    assert dev < 1e-6


def test_quat_long_chains():
    # one 64-lane group, 65536 steps: 1024 segments of 64 steps in 64 blocks
    w = inputs.QuatWorkload("long", 1, 65536, 2, 32, seed=1009)
    say("quat parity long chains (1, 65536, 2, 32)")
    i = inputs.make_quat_inputs(w)
    compare(gpu_quat(i), oracle_quat(i), TOL["f32"], KEYS, "quat 64k steps")


def test_quat_workspace_reused_across_sizes():
    big = inputs.make_quat_inputs(inputs.QuatWorkload("a", 2, 700, 3, 24, seed=31))
    small = inputs.make_quat_inputs(inputs.QuatWorkload("b", 1, 200, 2, 40, seed=32))
    qb = big["q"].cuda()
    ws_f = ssd.quat_workspace(qb, False)
    ws_b = ssd.quat_workspace(qb, True)
    for name, i in (("big", big), ("small", small), ("big again", big)):
        say(f"quat workspace reuse: {name}")
        compare(gpu_quat(i, ws_f, ws_b), oracle_quat(i), TOL["f32"], KEYS, f"reuse {name}")


def test_quat_empty_sequence_and_batch():
    q = torch.zeros((2, 0, 3, 4, 4), device="cuda")
    init = torch.randn((2, 3, 4, 4), device="cuda")
    cum = ssd.quat_scan(q, init)
    d_q, d_init = ssd.quat_scan_bwd(q, init, q)
    torch.cuda.synchronize()
    assert cum.numel() == 0 and d_q.numel() == 0
    assert torch.all(d_init == 0)
    q0 = torch.zeros((0, 5, 3, 4, 4), device="cuda")
    assert ssd.quat_scan(q0).numel() == 0
    d_q0, d_i0 = ssd.quat_scan_bwd(q0, None, q0)
    assert d_q0.numel() == 0 and d_i0.numel() == 0


def test_quat_runs_are_bitwise_reproducible():
    # every carry is a fold of published records in a fixed order (the block's earlier
    # aggregates, then the earlier blocks'), and a record is read with its tag bits cleared,
    # so repeated calls -- each with a new tag, on a workspace the previous call left full
    # of records -- give the same bits; also over 34 blocks of 16 segments (the last one
    # ragged), whose block aggregates carry every segment past the first block
    for w in (inputs.QUAT_WORKLOADS["mamba3_quat_scan_fp32"],
              inputs.QuatWorkload("long", 1, 64 * 16 * 33 + 5, 1, 40, norm_std=0.05, seed=61)):
        i = inputs.make_quat_inputs(w)
        qd = i["q"].cuda()
        ws_f, ws_b = ssd.quat_workspace(qd, False), ssd.quat_workspace(qd, True)
        a, b, c = (gpu_quat(i, ws_f, ws_b) for _ in range(3))
        for k in KEYS:
            say(f"  {w.name} {k}: {int(np.count_nonzero(a[k] != b[k]))} and "
                f"{int(np.count_nonzero(a[k] != c[k]))} of {a[k].size} elements differ between runs")
            assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


def test_quat_graph_replay_matches_eager():
    # every call advances the tag kept in the workspace from a kernel of its own, so
    # a call replayed from a captured graph uses a fresh tag; each replay (with eager
    # calls on the same workspaces in between) must match the eager result and the oracle
    w = inputs.QuatWorkload("graph", 2, 1500, 3, 24, norm_std=0.05, seed=58)
    i = inputs.make_quat_inputs(w)
    say("case graph capture of ssd_quat_scan + ssd_quat_scan_bwd")
    q, init, dc = i["q"].cuda(), i["init"].cuda(), i["d_cum"].cuda()
    cum, d_q = torch.empty_like(q), torch.empty_like(q)
    d_init = torch.empty_like(init)
    ws_f, ws_b = ssd.quat_workspace(q, False), ssd.quat_workspace(q, True)

    def step():
        st = torch.cuda.current_stream()
        assert ssd.ssd_quat_scan(q, init, cum, ws_f, st) == 0
        assert ssd.ssd_quat_scan_bwd(q, init, dc, d_q, d_init, ws_b, st) == 0

    step()
    torch.cuda.synchronize()
    ref = {k: t.clone().cpu().numpy() for k, t in dict(cum=cum, d_q=d_q, d_init=d_init).items()}
    compare(ref, oracle_quat(i), TOL["f32"], KEYS, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(3):
        for t in (cum, d_q, d_init):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dict(cum=cum.cpu().numpy(), d_q=d_q.cpu().numpy(), d_init=d_init.cpu().numpy())
        for k in KEYS:
            diff = np.abs(got[k].astype(np.float64) - ref[k]).max(axis=-1)
            bound = 2 * np.spacing(np.linalg.norm(ref[k], axis=-1).astype(np.float32)).astype(np.float64)
            assert np.all(diff <= bound), f"replay {it}: {k}"
        step()  # eager calls on the same workspaces between replays
        torch.cuda.synchronize()


def draw_quat_cases(seed=20261207, n=12):
    """Random quaternion-scan problems from one fixed seed: batch, lengths from 1 to 3000
    steps (ragged last segments in both directions' segmentations), 1 to 200 lanes per row
    (partial 64-lane groups), unit or non-unit steps, random or identity init."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 4)), int(rng.integers(1, 3001)), int(rng.integers(1, 5)),
             int(rng.integers(1, 51)), float(rng.choice([0.0, 0.05, 0.2])), bool(rng.integers(2)),
             int(rng.integers(1 << 30))) for _ in range(n)]


QUAT_CASES = draw_quat_cases()


@pytest.mark.parametrize("case", QUAT_CASES, ids=[f"b{c[0]}_s{c[1]}_h{c[2]}_j{c[3]}_n{c[4]}_i{int(c[5])}"
                                                  for c in QUAT_CASES])
def test_quat_random_case(case):
    b, s, h, j, nstd, rinit, seed = case
    w = inputs.QuatWorkload("sweep", b, s, h, j, norm_std=nstd, random_init=rinit, seed=seed)
    say(f"quat sweep case {case}")
    i = inputs.make_quat_inputs(w)
    compare(gpu_quat(i), oracle_quat(i), TOL["f32"], KEYS, f"quat sweep {case}")
