"""A chunked evaluation of the SSD scan in plain PyTorch fp64 on the CPU -- test-only.

It exists to pin the oracle (a token-by-token recurrence and its hand-written
reverse-mode recurrence) against a structurally different computation.  The
state after token t of a chunk entered with state S is

    h_t = exp(c_t) S + sum_{s<=t} exp(c_t - c_s) dt_s x_s (outer) B_s,

with c the inclusive cumsum of dt*A inside the chunk.  So each chunk, taken on
its own from a zero entry state, is

  * an affine map of the state, S -> alpha S + U, with alpha = exp(c_last) and
    U = sum_s exp(c_last - c_s) dt_s x_s (outer) B_s;
  * its tokens' own outputs, a causal kernel matrix applied to the chunk's
    inputs: y0_t = sum_{s<=t} exp(c_t - c_s) dt_s (C_t . B_s) x_s;
  * a read-out of the entry state: exp(c_t) C_t . S.

The entry states of all chunks then come from an inclusive prefix-doubling
(Hillis-Steele) scan of the chunks' affine maps, composed as
(a2, U2) o (a1, U1) = (a2 a1, a2 U1 + U2), applied to the initial state: no
serial loop over chunks.  Gradients are those of reverse-mode automatic
differentiation of this evaluation (torch.autograd), not a hand-derived adjoint.

Layouts are the pages': x/dy [b, n, l, h, p], B/C [b, n, l, h, r],
dt [b, h, n, l], A/D [h], init/final [b, h, p, r]; numpy in, numpy out.
"""
from __future__ import annotations

import numpy as np
import torch

F64 = torch.float64


def _t(a, grad=False):
    t = torch.as_tensor(np.asarray(a, dtype=np.float64), dtype=F64)
    return t.requires_grad_(grad)


def chunk_pieces(x, dt, A, B, C, cum=None, dt_kernel=None):
    """Per chunk (torch, fp64): the cumsum c [b,h,n,l] (or the given one), the chunk's
    affine map (alpha [b,h,n], U [b,h,n,p,r]), its own outputs from a zero entry state
    y0 [b,h,n,l,p] and the read-out weights exp(c_t) C_t [b,h,n,l,r].  `dt_kernel`, when
    given, is the dt used as the kernel matrix's source weight (for separating the
    gradient that reaches dt through that weight alone)."""
    if cum is None:
        cum = torch.cumsum(dt * A[None, :, None, None], dim=3)
    dtk = dt if dt_kernel is None else dt_kernel
    xs = x.permute(0, 3, 1, 2, 4)                    # [b,h,n,l,p]
    Bs = B.permute(0, 3, 1, 2, 4)                    # [b,h,n,l,r]
    Cs = C.permute(0, 3, 1, 2, 4)
    l = cum.shape[-1]
    gap = cum[..., :, None] - cum[..., None, :]      # c_t - c_s  [b,h,n,t,s]
    causal = torch.tril(torch.ones(l, l, dtype=torch.bool))
    kern = torch.where(causal, torch.exp(torch.where(causal, gap, torch.zeros_like(gap))),
                       torch.zeros_like(gap))
    cb = torch.einsum("bhntr,bhnsr->bhnts", Cs, Bs)
    y0 = torch.einsum("bhnts,bhnsp->bhntp", kern * cb * dtk[..., None, :], xs)
    to_end = torch.exp(cum[..., -1:] - cum) * dt      # exp(c_last - c_s) dt_s
    U = torch.einsum("bhns,bhnsp,bhnsr->bhnpr", to_end, xs, Bs)
    alpha = torch.exp(cum[..., -1])
    readout = torch.exp(cum)[..., None] * Cs
    return cum, alpha, U, y0, readout


def entry_states(alpha, U, init):
    """Entry state of every chunk and the final state, from an inclusive prefix-doubling
    scan of the chunks' affine maps applied to init (zeros when None)."""
    b, h, n = alpha.shape
    p, r = U.shape[-2:]
    a, u = alpha, U
    d = 1
    while d < n:  # after the step with offset d, (a, u)[k] composes chunks k-2d+1 .. k
        a_prev = torch.cat([torch.ones_like(a[:, :, :d]), a[:, :, :-d]], dim=2)
        u_prev = torch.cat([torch.zeros_like(u[:, :, :d]), u[:, :, :-d]], dim=2)
        u = a[..., None, None] * u_prev + u
        a = a * a_prev
        d *= 2
    s0 = torch.zeros(b, h, p, r, dtype=F64) if init is None else init
    through = a[..., None, None] * s0[:, :, None] + u      # state after chunk k
    s_in = torch.cat([s0[:, :, None], through[:, :, :-1]], dim=2)
    return s_in, through[:, :, -1] if n > 0 else s0


def forward_t(x, dt, A, B, C, D, init):
    """y [b,n,l,h,p], final [b,h,p,r] (torch fp64, differentiable)."""
    _, alpha, U, y0, readout = chunk_pieces(x, dt, A, B, C)
    s_in, final = entry_states(alpha, U, init)
    y = y0 + torch.einsum("bhnlr,bhnpr->bhnlp", readout, s_in)
    y = y.permute(0, 2, 3, 1, 4) + D[None, None, None, :, None] * x
    return y, final


def forward(x, dt, A, B, C, D, init=None):
    with torch.no_grad():
        y, fin = forward_t(_t(x), _t(dt), _t(A), _t(B), _t(C), _t(D),
                           None if init is None else _t(init))
    return y.numpy(), fin.numpy()


def backward(dy, d_final, x, dt, A, B, C, D, init=None):
    """The seven gradients of <dy, y> + <d_final, final> by reverse-mode autodiff."""
    leaves = dict(x=_t(x, True), dt=_t(dt, True), A=_t(A, True), B=_t(B, True), C=_t(C, True),
                  D=_t(D, True), init=_t(np.zeros(np.shape(d_final)) if init is None else init, True))
    y, fin = forward_t(leaves["x"], leaves["dt"], leaves["A"], leaves["B"], leaves["C"],
                       leaves["D"], leaves["init"])
    loss = torch.sum(y * _t(dy))
    if d_final is not None:
        loss = loss + torch.sum(fin * _t(d_final))
    names = ("x", "dt", "A", "B", "C", "D", "init")
    grads = torch.autograd.grad(loss, [leaves[k] for k in names])
    return {"d_" + k: g.numpy() for k, g in zip(names, grads)}


def local_gradients(dy, x, dt, A, B, C, init=None):
    """Gradients of <dy, y - D x> through the chunks' own terms only -- the read-out of the
    entry state and the causal kernel matrix, with the entry states held fixed:
      d_cum_local [b,h,n,l]: w.r.t. the within-chunk cumsum c as those terms use it;
      d_dt_kernel [b,h,n,l]: w.r.t. dt as the kernel matrix's source weight alone."""
    xt, dtt, At, Bt, Ct = _t(x), _t(dt), _t(A), _t(B), _t(C)
    with torch.no_grad():
        _, alpha, U, _, _ = chunk_pieces(xt, dtt, At, Bt, Ct)
        s_in, _ = entry_states(alpha, U, None if init is None else _t(init))
        cum0 = torch.cumsum(dtt * At[None, :, None, None], dim=3)
    cum = cum0.clone().requires_grad_(True)
    dtk = dtt.clone().requires_grad_(True)
    _, _, _, y0, readout = chunk_pieces(xt, dtt, At, Bt, Ct, cum=cum, dt_kernel=dtk)
    out_x = y0 + torch.einsum("bhnlr,bhnpr->bhnlp", readout, s_in)
    loss = torch.sum(out_x.permute(0, 2, 3, 1, 4) * _t(dy))
    g_cum, g_dt = torch.autograd.grad(loss, [cum, dtk])
    return g_cum.numpy(), g_dt.numpy()


def chunk_entry_states(x, dt, A, B, init=None):
    """Entry state of every chunk, [b, n, h, p, r] (numpy)."""
    with torch.no_grad():
        xt, Bt = _t(x), _t(B)
        _, alpha, U, _, _ = chunk_pieces(xt, _t(dt), _t(A), Bt, Bt)
        s_in, _ = entry_states(alpha, U, None if init is None else _t(init))
    return s_in.permute(0, 2, 1, 3, 4).numpy()


def within_chunk_cumsum(dt, A):
    """c [b, h, n, l]: the inclusive cumsum of dt * A inside each chunk (numpy)."""
    return np.cumsum(np.asarray(dt) * np.asarray(A)[None, :, None, None], axis=3)
