"""fp64 numpy restatement of the pages' chunked SSD (K1-K5 and the recompute backward).

Test-only.  It exists to pin the oracle (a token-by-token recurrence) against a
second, structurally different algorithm: the chunked form of the burn-mamba
"combined_backward.rs" page.  Each function names the part of that page it
restates; the code is written from the math, vectorised over chunks, and is not
the GPU path (which never imports it).

Layouts: x/dy ``[b, n, l, h, p]``, B/C ``[b, n, l, h, r]``, dt ``[b, h, n, l]``,
states ``[b, n, h, p, r]``, initial/final state ``[b, h, p, r]``.
"""
from __future__ import annotations

import numpy as np


def k1_cumsum(dt, A):
    """K1: inclusive within-chunk cumsum of dt*A (RECOMPUTE section, K1).

    Returns ``cum [b,h,n,l]`` and the chunk totals ``end [b,h,n]``."""
    cum = np.cumsum(dt * A[None, :, None, None], axis=3)
    return cum, cum[..., -1]


def k2_cb(C, B):
    """K2: ``CB[b,n,h,t,s] = sum_r C[t,r] B[s,r]`` (RECOMPUTE section, K2)."""
    return np.einsum("bnthr,bnshr->bnhts", C, B)


def k3_states(x, B, cum, dt):
    """K3 extended (``k3_ssd_chunk_state_extended`` doc).

    Returns the chunk-end states from a zero entry state ``[b,n,h,p,r]``, the
    scale ``dt * exp(end - cum)``, the decay ``exp(end - cum)`` (``[b,h,n,l]``) and
    B scaled per token ``[b,n,h,l,r]``."""
    decay_end = np.exp(cum[..., -1:] - cum)
    scale = decay_end * dt
    b_scaled = np.einsum("bnlhr,bhnl->bnhlr", B, scale)
    intra = np.einsum("bnlhp,bnhlr->bnhpr", x, b_scaled)
    return intra, scale, decay_end, b_scaled


def k4_pass(intra, end, init):
    """K4: serial carry ``s_{i+1} = exp(end_i) s_i + intra_i``; returns the
    chunk-entry states ``[b,n,h,p,r]`` and the final state."""
    b, n, h, p, r = intra.shape
    s = np.zeros((b, h, p, r)) if init is None else init.copy()
    s_in = np.empty_like(intra)
    for i in range(n):
        s_in[:, i] = s
        s = np.exp(end[:, :, i])[:, :, None, None] * s + intra[:, i]
    return s_in, s


def causal_decay(cum):
    """``exp(cum[t] - cum[s])`` for s <= t and 0 above the diagonal, ``[b,h,n,t,s]``."""
    l = cum.shape[-1]
    diff = cum[..., :, None] - cum[..., None, :]
    keep = np.tril(np.ones((l, l), dtype=bool))
    return np.where(keep, np.exp(np.where(keep, diff, 0.0)), 0.0)


def forward(x, dt, A, B, C, D, init=None):
    """Chunked forward: K1, K2, K3, K4 then K5 = BLUE + ORANGE + D*x."""
    cum, end = k1_cumsum(dt, A)
    cb = k2_cb(C, B)
    intra, _, _, _ = k3_states(x, B, cum, dt)
    s_in, final = k4_pass(intra, end, init)
    e = np.exp(cum)                                        # [b,h,n,l]
    blue = np.einsum("bnlhr,bnhpr,bhnl->bnlhp", C, s_in, e)
    w = cb * np.transpose(causal_decay(cum), (0, 2, 1, 3, 4)) \
        * np.transpose(dt, (0, 2, 1, 3))[:, :, :, None, :]  # [b,n,h,t,s]
    orange = np.einsum("bnhts,bnshp->bnthp", w, x)
    y = blue + orange + D[None, None, None, :, None] * x
    return y, final


def backward(dy, d_final, x, dt, A, B, C, D, init=None):
    """Chunked recompute backward in the order of the page's ``combined_backward``.

    Returns the seven gradients plus the two test-only exports the page's
    ``CombinedGrads`` documents: ``d_da_local`` (BLUE + ORANGE part of the
    gradient w.r.t. the cumsum) and ``d_dt_orange``."""
    b, n, l, h, p = x.shape
    r = B.shape[-1]
    # recompute K1-K4
    cum, end = k1_cumsum(dt, A)
    cb = k2_cb(C, B)                                          # [b,n,h,t,s]
    intra, scale, decay_end, b_scaled = k3_states(x, B, cum, dt)
    s_in, _ = k4_pass(intra, end, init)
    # SKIP backward
    d_D = np.einsum("bnlhp,bnlhp->h", dy, x)
    d_x = dy * D[None, None, None, :, None]
    # BLUE backward (all chunks at once: nothing here depends on the carry)
    e = np.exp(cum)                                           # [b,h,n,l]
    d_ch = np.einsum("bnlhp,bhnl->bnhlp", dy, e)
    d_state_local = np.einsum("bnlhr,bnhlp->bnhpr", C, d_ch)  # C^T d_ch
    d_C_blue = np.einsum("bnhlp,bnhpr->bnlhr", d_ch, s_in)
    ch = np.einsum("bnlhr,bnhpr->bnhlp", C, s_in)
    d_da_blue = np.einsum("bnlhp,bnhlp,bhnl->bhnl", dy, ch, e)
    # ORANGE backward
    decay = np.transpose(causal_decay(cum), (0, 2, 1, 3, 4))   # [b,n,h,t,s]
    dt_s = np.transpose(dt, (0, 2, 1, 3))[:, :, :, None, :]     # [b,n,h,1,s]
    w = cb * decay * dt_s
    d_w = np.einsum("bnthp,bnshp->bnhts", dy, x)
    d_x = d_x + np.einsum("bnhts,bnthp->bnshp", w, dy)
    keep = np.tril(np.ones((l, l), dtype=bool))
    d_w = np.where(keep, d_w, 0.0)
    d_cb_decay = d_w * dt_s
    d_dt_orange = np.transpose((d_w * cb * decay).sum(axis=3), (0, 2, 1, 3))  # colsum -> [b,h,n,s]
    d_cb = d_cb_decay * decay
    d_diff = d_cb_decay * cb * decay
    d_da_orange = np.transpose(d_diff.sum(axis=4) - d_diff.sum(axis=3), (0, 2, 1, 3))
    # K4 backward: reverse carry over chunks
    d_run = np.zeros((b, h, p, r)) if d_final is None else d_final.copy()
    d_intra = np.empty_like(intra)
    d_end = np.empty((b, h, n))
    for i in reversed(range(n)):
        d_intra[:, i] = d_run
        dec = np.exp(end[:, :, i])[:, :, None, None]
        d_end[:, :, i] = (d_run * s_in[:, i] * dec).sum(axis=(2, 3))
        d_run = dec * d_run + d_state_local[:, i]
    d_init = d_run
    d_cum_k4 = np.zeros((b, h, n, l))
    d_cum_k4[..., -1] = d_end
    # K3 backward
    d_x = d_x + np.einsum("bnhpr,bnhlr->bnlhp", d_intra, b_scaled)
    d_b_scaled = np.einsum("bnlhp,bnhpr->bnhlr", x, d_intra)
    d_B = np.einsum("bnhlr,bhnl->bnlhr", d_b_scaled, scale)
    d_scale = np.einsum("bnhlr,bnlhr->bhnl", d_b_scaled, B)
    d_dt_k3 = d_scale * decay_end
    d_delta = d_scale * dt * decay_end
    d_cum_k3 = -d_delta
    d_cum_k3[..., -1] += d_delta.sum(axis=3)
    # K2 backward
    d_C = np.einsum("bnhts,bnshr->bnthr", d_cb, B) + d_C_blue
    d_B = d_B + np.einsum("bnhts,bnthr->bnshr", d_cb, C)
    # sum + K1 backward: suffix sum within each chunk
    d_cum = d_da_blue + d_da_orange + d_cum_k3 + d_cum_k4
    d_da = np.flip(np.cumsum(np.flip(d_cum, axis=3), axis=3), axis=3)
    d_dt = d_dt_orange + d_dt_k3 + d_da * A[None, :, None, None]
    d_A = (d_da * dt).sum(axis=(0, 2, 3))
    return dict(d_x=d_x, d_dt=d_dt, d_A=d_A, d_B=d_B, d_C=d_C, d_D=d_D, d_init=d_init,
                d_da_local=d_da_blue + d_da_orange, d_dt_orange=d_dt_orange)
