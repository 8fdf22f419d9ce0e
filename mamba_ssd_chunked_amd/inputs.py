"""Seeded synthetic inputs for the SSD scan (shared by the tests and the benchmark).

This module draws random tensors and nothing else: it holds none of the scan's
arithmetic.  The distributions are the workload recipe of the project (the pages
publish no data set):

* x, D, dy, d_final ~ N(0, 1)
* B, C ~ N(0, 1) / sqrt(dstate), iid per element and head (no group sharing)
* dt = softplus(z - dt_shift), z ~ N(0, 1)   (the discretised step is the input)
* A_h = -exp(u * ln 16), u ~ U(0, 1), so A lies in [-16, -1]
* initial_state = init_std * N(0, 1)  (init_std = 0 gives zeros)
* d_m2 ~ N(0, 1) [b, h, r, r], d_m1 ~ N(0, 1) [b, h, r]

Draw order is fixed (x, B, C, z, u, D, init, dy, d_final, d_m2, d_m1) from one
CPU ``torch.Generator`` seeded with ``seed``.  For bf16 workloads x, B, C and dy
are rounded to bfloat16 (round-to-nearest-even) after the fp32 draw; every other
tensor stays fp32.

Layouts follow the pages' tensor naming: x/dy ``[b, n, l, h, p]``, B/C
``[b, n, l, h, r]``, dt ``[b, h, n, l]``, A/D ``[h]``, states ``[b, h, p, r]``.

The Mamba-3 same-step correction (``DiagWorkload``) draws, in this order, v and
dy ~ N(0, 1) ``[b, n, l, m, h, p]``, B and C ~ N(0, 1) / sqrt(dstate)
``[b, n, l, m, h, r]`` and gamma = softplus(z - 2) ``[b, n, l, h]`` (a
step-sized positive weight, like dt), after which bf16 workloads round v, B, C
and dy to bfloat16.

The Mamba-3 quaternion rotation scan (``QuatWorkload``) draws, in this order,
g ~ N(0, 1) ``[b, s, h, j, 4]``, z ~ N(0, 1) ``[b, s, h, j]``, g0 ~ N(0, 1)
``[b, h, j, 4]`` and d_cum ~ N(0, 1) ``[b, s, h, j, 4]``.  The step quaternions
are q = g / |g| (uniform on the unit 3-sphere: Haar-random rotations, the
largest per-step rotations a rotation can produce), times exp(norm_std * z)
when norm_std > 0 (non-unit steps); init = g0 / |g0| or None (the identity).

The decode step (``StepWorkload``) draws, in this order, x ~ N(0, 1) ``[b, h, p]``,
B and C ~ N(0, 1) / sqrt(dstate) ``[b, h, r]``, z ~ N(0, 1) ``[b, h]`` (dt =
softplus(z - 2)), u ~ U(0, 1) ``[h]`` (A = -exp(u ln 16)), D ~ N(0, 1) ``[h]`` and
the cached state = state_std * N(0, 1) ``[b, h, p, r]``; bf16 workloads round x,
B and C to bfloat16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    nheads: int
    headdim: int
    dstate: int
    chunk_len: int
    io: str = "f32"            # "f32" or "bf16" (x, B, C, dy, y and their gradients)
    dt_shift: float = 2.0
    init_std: float = 0.0
    valid_len: Optional[Sequence[int]] = None
    seed: int = 1000

    @property
    def nchunks(self) -> int:
        return self.seq // self.chunk_len

    def describe(self) -> dict:
        d = dict(workload=self.name, batch=self.batch, seq_len=self.seq, nheads=self.nheads,
                 headdim=self.headdim, dstate=self.dstate, chunk_len=self.chunk_len,
                 io_dtype=self.io)
        if self.valid_len is not None:
            d["valid_len"] = list(self.valid_len)
        return d


# The five named workloads (shapes only; "130M"/"2.7B" borrow model shapes, no weights).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 16, 16, 64, seed=1000),
    "mamba2_130m_fp32": Workload("mamba2_130m_fp32", 4, 2048, 24, 64, 128, 256, seed=1001),
    "mamba2_2p7b_bf16": Workload("mamba2_2p7b_bf16", 2, 4096, 80, 64, 128, 256, io="bf16",
                                 seed=1002),
    "long_context_64k_fp32": Workload("long_context_64k_fp32", 1, 65536, 32, 64, 128, 256,
                                      dt_shift=4.0, init_std=0.1, seed=1003),
    "moments_valid_len_fp32": Workload("moments_valid_len_fp32", 2, 4096, 24, 64, 64, 128,
                                       valid_len=(4096, 3000), seed=1004),
}
WORKLOAD_ORDER = list(WORKLOADS)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw every input of workload ``w`` on the CPU (see module docstring)."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    b, n, l, h, p, r = w.batch, w.nchunks, w.chunk_len, w.nheads, w.headdim, w.dstate
    if n * l != w.seq:
        raise ValueError("seq must be a multiple of chunk_len")

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32)

    x = randn(b, n, l, h, p)
    B = randn(b, n, l, h, r) / math.sqrt(r)
    C = randn(b, n, l, h, r) / math.sqrt(r)
    z = randn(b, h, n, l)
    u = torch.rand(h, generator=g, dtype=torch.float32)
    D = randn(h)
    init = randn(b, h, p, r) * w.init_std
    dy = randn(b, n, l, h, p)
    d_final = randn(b, h, p, r)
    d_m2 = randn(b, h, r, r)
    d_m1 = randn(b, h, r)
    dt = torch.nn.functional.softplus(z - w.dt_shift)
    A = -torch.exp(u * math.log(16.0))
    if w.io == "bf16":
        x, B, C, dy = (t.to(torch.bfloat16) for t in (x, B, C, dy))
    elif w.io != "f32":
        raise ValueError(f"unknown io dtype {w.io!r}")
    out = dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init=init, dy=dy, d_final=d_final,
               d_m2=d_m2, d_m1=d_m1)
    if w.valid_len is not None:
        out["valid_len"] = torch.tensor(list(w.valid_len), dtype=torch.int64)
    return out


def custom(name="custom", batch=1, seq=256, nheads=2, headdim=16, dstate=16, chunk_len=64,
           io="f32", dt_shift=2.0, init_std=0.0, valid_len=None, seed=7) -> Workload:
    """A workload with the standard distributions and arbitrary shapes (for tests)."""
    return Workload(name, batch, seq, nheads, headdim, dstate, chunk_len, io=io,
                    dt_shift=dt_shift, init_std=init_std, valid_len=valid_len, seed=seed)


@dataclasses.dataclass(frozen=True)
class DiagWorkload:
    """Shapes of the Mamba-3 same-step correction: tokens [b, n, l], mimo rank m."""
    name: str
    batch: int
    seq: int
    chunk_len: int
    mimo_rank: int
    nheads: int
    headdim: int
    dstate: int
    io: str = "f32"
    seed: int = 1005

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def describe(self) -> dict:
        return dict(workload=self.name, batch=self.batch, seq_len=self.seq, chunk_len=self.chunk_len,
                    mimo_rank=self.mimo_rank, nheads=self.nheads, headdim=self.headdim,
                    dstate=self.dstate, io_dtype=self.io)


# The SSD benchmark's shapes (4 x 2048 tokens, 24 heads, p = 64, r = 128) at mimo rank 1
# (the SISO path) and 4.
DIAG_WORKLOADS = {
    "mamba3_diag_siso_fp32": DiagWorkload("mamba3_diag_siso_fp32", 4, 2048, 256, 1, 24, 64, 128,
                                          seed=1005),
    "mamba3_diag_mimo4_fp32": DiagWorkload("mamba3_diag_mimo4_fp32", 4, 2048, 256, 4, 24, 64, 128,
                                           seed=1006),
}


def make_diag_inputs(w: DiagWorkload) -> dict:
    """Draw v, dy, B, C, gamma for the same-step correction (see module docstring)."""
    g = torch.Generator().manual_seed(w.seed)
    b, l, m, h, p, r = w.batch, w.chunk_len, w.mimo_rank, w.nheads, w.headdim, w.dstate
    n = w.seq // l
    if n * l != w.seq:
        raise ValueError("seq must be a multiple of chunk_len")

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32)

    v = randn(b, n, l, m, h, p)
    dy = randn(b, n, l, m, h, p)
    B = randn(b, n, l, m, h, r) / math.sqrt(r)
    C = randn(b, n, l, m, h, r) / math.sqrt(r)
    gamma = torch.nn.functional.softplus(randn(b, n, l, h) - 2.0)
    if w.io == "bf16":
        v, dy, B, C = (t.to(torch.bfloat16) for t in (v, dy, B, C))
    elif w.io != "f32":
        raise ValueError(f"unknown io dtype {w.io!r}")
    return dict(v=v, dy=dy, B=B, C=C, gamma=gamma)


@dataclasses.dataclass(frozen=True)
class QuatWorkload:
    """Shapes of the quaternion cumulative-product scan: q [b, s, h, j, 4]."""
    name: str
    batch: int
    seq: int
    nheads: int
    nquat: int                 # quaternion blocks per head (state_rank / 4 when fully rotated)
    norm_std: float = 0.0      # 0: unit step quaternions
    random_init: bool = True   # False: init = None (the identity)
    seed: int = 1007

    def describe(self) -> dict:
        return dict(workload=self.name, batch=self.batch, seq_len=self.seq, nheads=self.nheads,
                    nquat=self.nquat, unit=self.norm_std == 0.0,
                    init="random unit" if self.random_init else "identity")


# The SSD benchmark's shapes with its 128-wide state rotated as 32 quaternion blocks.
QUAT_WORKLOADS = {
    "mamba3_quat_scan_fp32": QuatWorkload("mamba3_quat_scan_fp32", 4, 2048, 24, 32, seed=1007),
}


def make_quat_inputs(w: QuatWorkload) -> dict:
    """Draw q, init, d_cum for the quaternion scan (see module docstring)."""
    g = torch.Generator().manual_seed(w.seed)
    b, s, h, j = w.batch, w.seq, w.nheads, w.nquat
    raw = torch.randn(b, s, h, j, 4, generator=g, dtype=torch.float32)
    z = torch.randn(b, s, h, j, generator=g, dtype=torch.float32)
    raw0 = torch.randn(b, h, j, 4, generator=g, dtype=torch.float32)
    d_cum = torch.randn(b, s, h, j, 4, generator=g, dtype=torch.float32)
    q = raw / raw.norm(dim=-1, keepdim=True)
    if w.norm_std > 0:
        q = q * torch.exp(w.norm_std * z)[..., None]
    init = raw0 / raw0.norm(dim=-1, keepdim=True) if w.random_init else None
    return dict(q=q.contiguous(), init=init, d_cum=d_cum)


@dataclasses.dataclass(frozen=True)
class StepWorkload:
    """Shapes of the decode step: one token for each of `batch` sequences."""
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    io: str = "f32"
    state_std: float = 0.5
    seed: int = 1010

    def describe(self) -> dict:
        return dict(workload=self.name, batch=self.batch, nheads=self.nheads, headdim=self.headdim,
                    dstate=self.dstate, io_dtype=self.io)


# Decode batches of 128 (130M shapes, fp32) and 64 (2.7B shapes, bf16 x/B/C/y) sequences.
STEP_WORKLOADS = {
    "mamba2_130m_decode_fp32": StepWorkload("mamba2_130m_decode_fp32", 128, 24, 64, 128, seed=1010),
    "mamba2_2p7b_decode_bf16": StepWorkload("mamba2_2p7b_decode_bf16", 64, 80, 64, 128, io="bf16",
                                            seed=1011),
}


def make_step_inputs(w: StepWorkload) -> dict:
    """Draw x, B, C, dt, A, D and the cached state for one decode step (see module docstring)."""
    g = torch.Generator().manual_seed(w.seed)
    b, h, p, r = w.batch, w.nheads, w.headdim, w.dstate

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32)

    x = randn(b, h, p)
    B = randn(b, h, r) / math.sqrt(r)
    C = randn(b, h, r) / math.sqrt(r)
    z = randn(b, h)
    u = torch.rand(h, generator=g, dtype=torch.float32)
    D = randn(h)
    state = randn(b, h, p, r) * w.state_std
    dt = torch.nn.functional.softplus(z - 2.0)
    A = -torch.exp(u * math.log(16.0))
    if w.io == "bf16":
        x, B, C = (t.to(torch.bfloat16) for t in (x, B, C))
    elif w.io != "f32":
        raise ValueError(f"unknown io dtype {w.io!r}")
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, state=state)
