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


def compare(gpu: dict, ref: dict, tol: float, keys, label=""):
    errs = {k: rel_l2(gpu[k], ref[k]) for k in keys}
    say(f"  {label} rel-L2: " + ", ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    bad = {k: e for k, e in errs.items() if not (e <= tol)}
    assert not bad, f"{label}: rel-L2 above {tol}: {bad}"
    return errs


def workload_inputs(w: inputs.Workload):
    return inputs.make_inputs(w)
