"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from mamba_ssd_chunked_amd import inputs, ssd

# Tolerances: per-tensor relative L2 error against the fp64 oracle.  fp32 inputs:
# 1e-5; bf16 inputs (the oracle sees the same bf16-rounded values), fp32
# accumulation and bf16 outputs: 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}

GRADS = ("d_x", "d_dt", "d_A", "d_B", "d_C", "d_D", "d_init")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    return float(num / den) if den > 0 else float(num)


def to_dev(t: dict) -> dict:
    out = {}
    for k, v in t.items():
        if isinstance(v, torch.Tensor) and k != "valid_len":
            out[k] = v.cuda().contiguous()
        else:
            out[k] = v
    return out


def gpu_fwd_bwd(inp: dict, use_init=True, use_d_final=True, kernel_chunk_len=0):
    d = to_dev(inp)
    init = d["init"] if use_init else None
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], init,
                         kernel_chunk_len=kernel_chunk_len)
    g = ssd.backward(d["dy"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], init,
                     d_final=d["d_final"] if use_d_final else None,
                     kernel_chunk_len=kernel_chunk_len)
    torch.cuda.synchronize()
    out = dict(y=y.float().cpu().numpy(), final=fin.cpu().numpy())
    for k, v in g.items():
        out[k] = v.float().cpu().numpy()
    return out


def oracle_fwd_bwd(inp: dict, heads=None, use_init=True, use_d_final=True):
    """Oracle on all batches and the given heads (all when None)."""
    def sel(k):
        v = inp[k].double()
        if heads is None:
            return v.numpy()
        if k in ("x", "dy", "B", "C"):
            return v[:, :, :, heads, :].numpy()
        if k in ("dt", "init", "d_final"):
            return v[:, heads].numpy()
        return v[heads].numpy()  # A, D
    x, dt, A, B, C, D, init, dy, df = (sel(k) for k in
                                       ("x", "dt", "A", "B", "C", "D", "init", "dy", "d_final"))
    init = init if use_init else None
    df = df if use_d_final else None
    y, fin = oracle.ssd_fwd(x, dt, A, B, C, D, init)
    g = oracle.ssd_bwd(dy, df, x, dt, A, B, C, D, init)
    out = dict(y=y, final=fin)
    out.update(g)
    return out


def select_heads(gpu: dict, heads):
    out = {}
    for k, v in gpu.items():
        if k in ("y", "d_x", "d_B", "d_C"):
            out[k] = v[:, :, :, heads, :]
        elif k in ("final", "d_init", "d_dt"):
            out[k] = v[:, heads]
        else:  # d_A, d_D
            out[k] = v[heads]
    return out


# Worst relative L2 error of one (batch, head, chunk) block of a token tensor, or one
# (batch, head) state: a mistake confined to one chunk or one head is diluted in the
# per-tensor figure, so every block is also held to a bound (ten times the per-tensor
# tolerance for fp32 inputs, 5e-2 for bf16 ones).
BLOCK_TOL = {TOL["f32"]: 1e-4, TOL["bf16"]: 5e-2}
# (axes summed over inside one block, rank of the tensor), by output: token rows
# [b, n, l, h, f] (f = p or r), the step gradient [b, h, n, l], states [b, h, p, r]
BLOCK_AXES = {"y": ((2, 4), 5), "d_x": ((2, 4), 5), "d_B": ((2, 4), 5), "d_C": ((2, 4), 5),
              "d_dt": ((3,), 4), "final": ((2, 3), 4), "d_init": ((2, 3), 4)}


def worst_block_rel(a, b, axes) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.size == 0:
        return 0.0
    num = np.sqrt(np.sum((a - b) ** 2, axis=axes))
    den = np.sqrt(np.sum(b ** 2, axis=axes))
    # blocks whose reference is exactly zero compare absolutely
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def compare(gpu: dict, ref: dict, tol: float, keys, label="", block_tol=None):
    errs = {k: rel_l2(gpu[k], ref[k]) for k in keys}
    say(f"  {label} rel-L2: " + ", ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    assert not bad, f"{label}: rel-L2 above {tol}: {bad}"
    btol = block_tol if block_tol is not None else BLOCK_TOL.get(tol, 10 * tol)
    blk = {k: worst_block_rel(gpu[k], ref[k], BLOCK_AXES[k][0]) for k in keys
           if k in BLOCK_AXES and np.ndim(ref[k]) == BLOCK_AXES[k][1]}
    if blk:
        say(f"  {label} worst block rel-L2: " + ", ".join(f"{k}={e:.2e}" for k, e in blk.items()))
    bad = {k: e for k, e in blk.items() if not (e <= btol)}
    assert not bad, f"{label}: a (batch, head, chunk) block's rel-L2 is above {btol}: {bad}"
    return errs


def per_head_dot(a, b, head_axis=3, step=8):
    """fp64 sum over every axis but the head axis of a * b, for [b, n, l, h, f] token
    tensors (head_axis 3), [b, h, n, l] step tensors or [b, h, p, r] states (head_axis 1);
    accumulated in slices of the second axis to bound host memory."""
    if head_axis != 3:  # step tensors and states are small: in one piece
        ax = tuple(i for i in range(np.ndim(a)) if i != head_axis)
        return np.sum(np.asarray(a, dtype=np.float64) * np.asarray(b, dtype=np.float64), axis=ax)
    out = None
    for k0 in range(0, max(a.shape[1], 1), step):
        aa = np.asarray(a[:, k0:k0 + step], dtype=np.float64)
        bb = np.asarray(b[:, k0:k0 + step], dtype=np.float64)
        ax = tuple(i for i in range(aa.ndim) if i != head_axis)
        part = np.sum(aa * bb, axis=ax)
        out = part if out is None else out + part
    return out


def check_identities_all_heads(inp: dict, gpu: dict, tol: float, use_init: bool,
                               use_d_final: bool, label=""):
    """The exact linearity (Euler) identities of the SSD, evaluated per head over ALL heads
    of the device's outputs, in fp64 on the host (the oracle pins them to 1e-12):
      (i)   <dy, y> + <d_final, final> = <d_x, x> + <d_init, init>
      (ii)  <d_C, C> = <dy, y - D x>
      (iii) d_D = <dy, x>
    and, with a zero initial state,
      (iv)  <d_B, B> = <dy, y - D x> + <d_final, final>
      (v)   <dt, d_dt> - A d_A = <dy, y - D x> + <d_final, final>
    each residual scaled by the Cauchy-Schwarz size of its terms (sums of norm products),
    so rounding of the outputs gives about the outputs' relative error."""
    f = lambda k: np.asarray(inp[k].float().numpy() if hasattr(inp[k], "numpy") else inp[k])  # noqa: E731
    x, dy, Bm, Cm, dt = f("x"), f("dy"), f("B"), f("C"), f("dt")
    A, D = f("A").astype(np.float64), f("D").astype(np.float64)
    nrm = lambda a, ax=3: np.sqrt(per_head_dot(a, a, ax))  # noqa: E731
    dy_y, dy_x = per_head_dot(dy, gpu["y"]), per_head_dot(dy, x)
    dy_skip = dy_y - D * dy_x                       # <dy, y - D x>
    s_dy, s_y, s_x = nrm(dy), nrm(gpu["y"]), nrm(x)
    lhs1, rhs1, sc1 = dy_y.copy(), per_head_dot(gpu["d_x"], x), s_dy * s_y + nrm(gpu["d_x"]) * s_x
    fin_term = np.zeros_like(dy_y)
    if use_d_final:
        dfin = f("d_final")
        fin_term = per_head_dot(dfin, gpu["final"], 1)
        lhs1 += fin_term
        sc1 += nrm(dfin, 1) * nrm(gpu["final"], 1)
    if use_init:
        ini = f("init")
        rhs1 += per_head_dot(gpu["d_init"], ini, 1)
        sc1 += nrm(gpu["d_init"], 1) * nrm(ini, 1)
    sc_skip = s_dy * (s_y + np.abs(D) * s_x)
    res = {"i": np.abs(lhs1 - rhs1) / sc1,
           "ii": np.abs(per_head_dot(gpu["d_C"], Cm) - dy_skip) / (nrm(gpu["d_C"]) * nrm(Cm) + sc_skip),
           "iii": np.abs(gpu["d_D"].astype(np.float64) - dy_x) / (s_dy * s_x)}
    if not use_init:
        sc_fin = nrm(f("d_final"), 1) * nrm(gpu["final"], 1) if use_d_final else 0.0
        res["iv"] = (np.abs(per_head_dot(gpu["d_B"], Bm) - dy_skip - fin_term)
                     / (nrm(gpu["d_B"]) * nrm(Bm) + sc_skip + sc_fin))
        t_dt = per_head_dot(dt, gpu["d_dt"], 1)
        t_A = A * gpu["d_A"].astype(np.float64)
        res["v"] = (np.abs(t_dt - t_A - dy_skip - fin_term)
                    / (nrm(dt, 1) * nrm(gpu["d_dt"], 1) + np.abs(t_A) + sc_skip + sc_fin))
    worst = {k: float(np.max(v)) for k, v in res.items()}
    say(f"  {label} identities over all {len(D)} heads, worst scaled residual: "
        + ", ".join(f"({k})={e:.1e}" for k, e in worst.items()))
    bad = {k: e for k, e in worst.items() if not (e <= tol)}
    assert not bad, f"{label}: identities violated beyond {tol}: {bad}"
    return worst


def workload_inputs(w: inputs.Workload):
    return inputs.make_inputs(w)
