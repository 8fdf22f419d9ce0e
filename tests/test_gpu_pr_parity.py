"""GPU parity of ssd_moments_pr / ssd_moments_pr_bwd against the CPU oracle.

PR = (tr Sigma)^2 / ||Sigma||_F^2 of the (optionally centred) sample covariance
of pooled moments, through the page's detached trace normaliser and floors
(StateMoments::pr, burn-mamba state_moments.rs page), and its gradient with
respect to m2 and m1.  The moments here are built from seeded sample rows in
fp64 and rounded to fp32; the oracle and the kernels see the same fp32 values.
Bar: per-tensor relative L2 <= 1e-5 (the kernels form every sum in fp64, so the
observed error is the final fp32 rounding).  Also: the two gradient properties
the page names (matches the gradient of the plain formula; stays finite as the
state shrinks), the all-zero and collapsed states, more than 64 batch rows, and
the whole PR-penalty loop moments -> PR -> dPR -> moments backward.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL, compare, rel_l2, say, to_dev
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


def sample_moments(batch, nheads, r, counts, seed, mean=0.5, scale=1.0):
    """m2 = sum of h h^T and m1 = sum of h over seeded sample rows h (fp64 -> fp32)."""
    g = torch.Generator().manual_seed(seed)
    m2 = torch.zeros(batch, nheads, r, r, dtype=torch.float64)
    m1 = torch.zeros(batch, nheads, r, dtype=torch.float64)
    for b in range(batch):
        rows = min(int(counts[b]), 4 * r)
        mix = torch.randn(nheads, r, r, generator=g, dtype=torch.float64) / r ** 0.5
        h = torch.randn(nheads, rows, r, generator=g, dtype=torch.float64) @ mix
        h = scale * (h + mean * torch.randn(nheads, 1, r, generator=g, dtype=torch.float64))
        m2[b] = h.transpose(1, 2) @ h
        m1[b] = h.sum(1)
    return m2.float(), m1.float(), torch.tensor(counts, dtype=torch.int64)


def gpu_pr(m2, m1, count, center, d_pr):
    m2d, m1d, dprd = m2.cuda(), m1.cuda(), d_pr.cuda()
    pr, tr = ssd.moments_pr(m2d, m1d, count, center)
    d_m2, d_m1 = ssd.moments_pr_bwd(dprd, m2d, m1d, count, center)
    torch.cuda.synchronize()
    return dict(pr=pr.cpu().numpy(), trace=tr.cpu().numpy(), d_m2=d_m2.cpu().numpy(),
                d_m1=d_m1.cpu().numpy())


def oracle_pr(m2, m1, count, center, d_pr):
    pr, tr = oracle.moments_pr(m2.double().numpy(), m1.double().numpy(), count.numpy(), center)
    d_m2, d_m1 = oracle.moments_pr_bwd(d_pr.double().numpy(), m2.double().numpy(),
                                       m1.double().numpy(), count.numpy(), center)
    return dict(pr=pr, trace=tr, d_m2=d_m2, d_m1=d_m1)


CASES = [
    # batch, nheads, dstate, counts
    (1, 1, 16, (40,)),
    (3, 5, 32, (64, 96, 33)),
    (2, 24, 64, (4096 * 64, 3000 * 64)),
    (4, 3, 128, (2048 * 64, 100, 5000, 1)),
]


@pytest.mark.parametrize("center", [False, True], ids=["raw", "centred"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_h%d_r%d" % c[:3])
def test_pr_matches_oracle(case, center):
    b, h, r, counts = case
    say(f"case pr {case} center={center}")
    m2, m1, count = sample_moments(b, h, r, counts, seed=900 + r + b)
    d_pr = torch.randn(b, h, generator=torch.Generator().manual_seed(7))
    gpu = gpu_pr(m2, m1, count, center, d_pr)
    ref = oracle_pr(m2, m1, count, center, d_pr)
    keys = ("pr", "trace", "d_m2") + (("d_m1",) if center else ())
    compare(gpu, ref, TOL["f32"], keys, f"pr {case}")
    if not center:
        assert np.all(gpu["d_m1"] == 0)


def direct_grad(m2, m1, count, center, d_pr):
    """Autograd (fp64, CPU) of sum d_pr (tr S)^2 / ||S||_F^2: no normaliser, no floors."""
    m2 = m2.double().clone().requires_grad_(True)
    m1 = m1.double().clone().requires_grad_(True)
    n = count.double()[:, None, None, None]
    S = m2 / n
    if center:
        mu = m1 / n[..., 0]
        S = S - mu[..., :, None] * mu[..., None, :]
    tr = torch.diagonal(S, dim1=-2, dim2=-1).sum(-1)
    pr = tr ** 2 / (S * S).sum((-2, -1))
    (pr * d_pr.double()).sum().backward()
    return m2.grad.numpy(), (m1.grad.numpy() if m1.grad is not None else np.zeros(m1.shape))


@pytest.mark.parametrize("center", [False, True], ids=["raw", "centred"])
def test_pr_gradient_matches_direct_formula(center):
    """The detached-normaliser gradient equals the plain ratio's gradient, including
    its trace-tangential (rank-reducing) part."""
    say(f"case pr gradient vs direct formula center={center}")
    m2, m1, count = sample_moments(2, 6, 64, (300, 1000), seed=31, mean=0.8)
    d_pr = torch.randn(2, 6, generator=torch.Generator().manual_seed(8))
    gpu = gpu_pr(m2, m1, count, center, d_pr)
    g2, g1 = direct_grad(m2, m1, count, center, d_pr)
    assert rel_l2(gpu["d_m2"], g2) < TOL["f32"]
    if center:
        assert rel_l2(gpu["d_m1"], g1) < TOL["f32"]
    # no radial part: <d_m2, 2 m2> + <d_m1, m1> = 0 per slice (degree 0 in (m2, m1))
    m2n, m1n = m2.double().numpy(), m1.double().numpy()
    euler = 2 * np.einsum("bhij,bhij->bh", gpu["d_m2"], m2n) + np.einsum("bhi,bhi->bh", gpu["d_m1"], m1n)
    scale = np.einsum("bhij,bhij->bh", np.abs(gpu["d_m2"]), np.abs(m2n))
    assert np.all(np.abs(euler) <= 1e-5 * scale)


def test_pr_gradient_finite_as_magnitude_shrinks():
    """Samples scaled by 10^-k, k = 0..18 (tr Sigma down to ~1e-36): PR unchanged,
    gradient finite, of degree -1 in m2, and equal to the oracle at every scale."""
    m2, m1, count = sample_moments(2, 4, 32, (128, 512), seed=33, mean=0.4)
    d_pr = torch.ones(2, 4)
    for center in (False, True):
        base = gpu_pr(m2, m1, count, center, d_pr)
        for k in range(19):
            c = 10.0 ** -k
            say(f"case pr magnitude 1e-{k} center={center}")
            m2c = (m2.double() * c * c).float()
            m1c = (m1.double() * c).float()
            gpu = gpu_pr(m2c, m1c, count, center, d_pr)
            for v in gpu.values():
                assert np.all(np.isfinite(v))
            assert rel_l2(gpu["pr"], base["pr"]) < 1e-5
            assert rel_l2(gpu["d_m2"] * c * c, base["d_m2"]) < 1e-5
            ref = oracle_pr(m2c, m1c, count, center, d_pr)
            compare(gpu, ref, TOL["f32"], ("pr", "d_m2") + (("d_m1",) if center else ()),
                    f"pr magnitude 1e-{k}")


def test_pr_all_zero_and_collapsed_states():
    say("case pr zero / collapsed state")
    z2, z1 = torch.zeros(1, 2, 16, 16), torch.zeros(1, 2, 16)
    for center in (False, True):
        gpu = gpu_pr(z2, z1, torch.tensor([9]), center, torch.ones(1, 2))
        assert np.all(gpu["pr"] == 0) and np.all(gpu["trace"] == 0)
        assert np.all(gpu["d_m2"] == 0) and np.all(gpu["d_m1"] == 0)
    # Sigma = 1e-47 I: the trace floor and the 1e-12 clamp both act (PR, 16 for any
    # larger multiple of I, drops below 1); m2 itself stays a normal fp32 number
    # through a large sample count.
    m2 = (torch.eye(16) * 1e-35).expand(1, 2, 16, 16).contiguous()
    count = torch.tensor([10 ** 12])
    gpu = gpu_pr(m2, z1, count, False, torch.ones(1, 2))
    ref = oracle_pr(m2, z1, count, False, torch.ones(1, 2))
    assert np.all(gpu["pr"] < 1) and np.all(np.isfinite(gpu["d_m2"]))
    compare(gpu, ref, TOL["f32"], ("pr", "d_m2"), "pr collapsed")
    # the raw trace, 1.6e-46, is below fp32's range: the output is its fp32 rounding (0)
    assert np.array_equal(gpu["trace"], ref["trace"].astype(np.float32))


def test_pr_more_than_64_batch_rows_and_determinism():
    say("case pr batch 70")
    counts = tuple(10 + 3 * b for b in range(70))
    m2, m1, count = sample_moments(70, 2, 16, counts, seed=35)
    d_pr = torch.randn(70, 2, generator=torch.Generator().manual_seed(9))
    gpu = gpu_pr(m2, m1, count, True, d_pr)
    ref = oracle_pr(m2, m1, count, True, d_pr)
    compare(gpu, ref, TOL["f32"], ("pr", "trace", "d_m2", "d_m1"), "pr batch 70")
    again = gpu_pr(m2, m1, count, True, d_pr)
    for k in gpu:
        assert np.array_equal(gpu[k], again[k]), k


@pytest.mark.parametrize("center", [False, True], ids=["raw", "centred"])
def test_pr_penalty_loop_on_the_moments_workload(center):
    """moments -> PR -> dPR/d(m2, m1) -> moments backward, on the valid_len moments
    workload (2 x 4096 tokens, 24 heads, p = r = 64), against the oracle's own chain
    on two sampled heads."""
    w = inputs.WORKLOADS["moments_valid_len_fp32"]
    heads = [5, 17]
    say(f"case pr penalty loop {w.name} heads {heads} center={center}")
    inp = inputs.make_inputs(w)
    valid = list(w.valid_len)
    d = to_dev(inp)
    mo = ssd.state_moments(d["x"], d["dt"], d["A"], d["B"], None, valid_len=valid)
    pr, _ = ssd.moments_pr(mo["m2"], mo["m1"], mo["count"], center)
    d_pr = torch.ones_like(pr)
    d_m2, d_m1 = ssd.moments_pr_bwd(d_pr, mo["m2"], mo["m1"], mo["count"], center)
    g = ssd.state_moments_bwd(d_m2, d["x"], d["dt"], d["A"], d["B"], None, valid_len=valid,
                              d_m1=d_m1)
    torch.cuda.synchronize()
    gpu = dict(pr=pr.cpu().numpy()[:, heads], d_m2=d_m2.cpu().numpy()[:, heads],
               d_x=g["d_x"].cpu().numpy()[:, :, :, heads], d_B=g["d_B"].cpu().numpy()[:, :, :, heads],
               d_dt=g["d_dt"].cpu().numpy()[:, heads], d_A=g["d_A"].cpu().numpy()[heads])
    if center:
        gpu["d_m1"] = d_m1.cpu().numpy()[:, heads]

    sel = lambda k, ax: np.take(inp[k].double().numpy(), heads, axis=ax)  # noqa: E731
    x, dt, A, B = sel("x", 3), sel("dt", 1), sel("A", 0), sel("B", 3)
    m2, m1, count = oracle.state_moments(x, dt, A, B, None, valid)
    opr, _ = oracle.moments_pr(m2, m1, count, center)
    od_m2, od_m1 = oracle.moments_pr_bwd(np.ones_like(opr), m2, m1, count, center)
    og = oracle.state_moments_bwd(od_m2, od_m1, x, dt, A, B, None, valid)
    ref = dict(pr=opr, d_m2=od_m2, d_m1=od_m1, **{k: og[k] for k in ("d_x", "d_B", "d_dt", "d_A")})
    compare(gpu, ref, TOL["f32"], tuple(gpu), f"pr loop center={center}")


def draw_pr_cases(seed=20261206, n=16):
    """Random participation-ratio problems from one fixed seed: batch and head counts, every
    dstate, counts from 1 to 2^18 per row (so the sample can be rank-deficient), mean offset
    and magnitude, raw or centred."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        b = int(rng.integers(1, 6))
        counts = tuple(int(c) for c in np.exp(rng.uniform(0, np.log(1 << 18), size=b)).astype(int) + 1)
        cases.append((b, int(rng.integers(1, 9)), int(rng.choice([16, 32, 64, 128])), counts,
                      float(rng.choice([0.0, 0.5, 3.0])), float(10.0 ** rng.uniform(-3, 3)),
                      bool(rng.integers(2)), int(rng.integers(1 << 30))))
    return cases


PR_CASES = draw_pr_cases()


@pytest.mark.parametrize("case", PR_CASES, ids=lambda c: "b%d_h%d_r%d_mean%g_%s" % (
    c[0], c[1], c[2], c[4], "centred" if c[6] else "raw"))
def test_pr_random_case(case):
    b, h, r, counts, mean, scale, center, seed = case
    say(f"pr sweep case {case}")
    m2, m1, count = sample_moments(b, h, r, counts, seed=seed, mean=mean, scale=scale)
    d_pr = torch.randn(b, h, generator=torch.Generator().manual_seed(seed + 1))
    gpu = gpu_pr(m2, m1, count, center, d_pr)
    ref = oracle_pr(m2, m1, count, center, d_pr)
    keys = ("pr", "trace", "d_m2") + (("d_m1",) if center else ())
    compare(gpu, ref, TOL["f32"], keys, f"pr sweep {case[:3]}")
    if not center:
        assert np.all(gpu["d_m1"] == 0)
