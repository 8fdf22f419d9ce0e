"""The forward entry point that allocates nothing (``ssd_fwd_noalloc``), through the C ABI.

Its workspace is the library's fixed per-GPU scratch array.  Two calls in a row on one
GPU -- the Mamba-2-130M-shaped workload (51.9 MB of scratch, near the 64 MiB limit), then a
smaller problem with an initial state -- each give exactly the outputs of ``ssd_fwd`` with
a workspace of its own (the same kernels), and match the oracle within the fp32 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from gpu_common import TOL, rel_l2, say, to_dev
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _both(w: inputs.Workload):
    t = inputs.make_inputs(w)
    d = to_dev(t)
    init = d["init"] if w.init_std > 0 else None
    dims = ssd.dims_of(d["x"], d["B"])
    need = ssd.ssd_workspace_size(dims, ssd.SSD_OP_FWD)
    assert need <= ssd.NOALLOC_SCRATCH_BYTES
    y0, f0 = torch.empty_like(d["x"]), torch.empty_like(d["d_final"])
    y1, f1 = torch.full_like(d["x"], float("nan")), torch.full_like(d["d_final"], float("nan"))
    ws = ssd.workspace(dims, ssd.SSD_OP_FWD, d["x"].device)
    st = torch.cuda.current_stream()
    rc = ssd.ssd_fwd(dims, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], init, y0, f0, ws, st)
    assert rc == 0, ssd.ssd_last_error()
    rc = ssd.ssd_fwd_noalloc(dims, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], init, y1, f1, st)
    assert rc == 0, ssd.ssd_last_error()
    torch.cuda.synchronize()
    return t, (y0, f0), (y1, f1), need


def _oracle_heads(t, w, heads):
    sel = lambda k: t[k].double()  # noqa: E731
    x, B, C = (sel(k)[:, :, :, heads].numpy() for k in ("x", "B", "C"))
    dt, init = sel("dt")[:, heads].numpy(), sel("init")[:, heads].numpy()
    A, D = sel("A")[heads].numpy(), sel("D")[heads].numpy()
    return oracle.ssd_fwd(x, dt, A, B, C, D, init if w.init_std > 0 else None)


def test_noalloc_forward_matches_ssd_fwd_on_two_calls_in_a_row():
    cases = [inputs.WORKLOADS["mamba2_130m_fp32"],
             inputs.custom(name="noalloc_small", batch=1, seq=512, nheads=3, headdim=32,
                           dstate=64, chunk_len=128, init_std=0.5, seed=4321)]
    needs = []
    for w in cases:
        say(f"ssd_fwd_noalloc vs ssd_fwd on {w.name}")
        t, (y0, f0), (y1, f1), need = _both(w)
        needs.append(need)
        assert torch.equal(y0, y1) and torch.equal(f0, f1), "outputs differ from ssd_fwd"
        heads = [0, w.nheads - 1] if w.nheads > 3 else list(range(w.nheads))
        ry, rf = _oracle_heads(t, w, heads)
        ey = rel_l2(y1[:, :, :, heads].cpu().numpy(), ry)
        ef = rel_l2(f1[:, heads].cpu().numpy(), rf)
        say(f"  scratch {need / 2**20:.1f} MiB; oracle rel-L2 y={ey:.2e} final={ef:.2e}")
        assert ey <= TOL["f32"] and ef <= TOL["f32"]
        assert np.isfinite(y1.cpu().numpy()).all()
    assert needs[1] < needs[0]


def test_noalloc_rejects_problems_beyond_the_scratch():
    w = inputs.WORKLOADS["long_context_64k_fp32"]
    dims = ssd.make_dims(w.batch, w.nchunks, w.chunk_len, w.nheads, w.headdim, w.dstate)
    assert ssd.ssd_workspace_size(dims, ssd.SSD_OP_FWD) > ssd.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda", 0)
    small = torch.empty(16, device=dev)  # never touched: the size check comes first
    import ctypes
    p = ctypes.c_void_p(small.data_ptr())
    rc = ssd.load_library().ssd_fwd_noalloc(ctypes.byref(dims), *([p] * 9), None)
    assert rc == 5 and "scratch" in ssd.ssd_last_error()
