"""GPU parity of ssd_fwd / ssd_bwd against the CPU oracle (needs an MI355X).

Every case draws seeded inputs, runs the HIP library through the C ABI
(``mamba_ssd_chunked_amd.ssd`` marshals torch tensors into ``include/ssd.h``)
and compares each output tensor with the fp64 oracle by relative L2 error:
<= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs (the oracle is fed the same
bf16-rounded values).  Small shapes are compared in full; the five named
workloads run at full size in the benchmark's launch configuration and are
compared on all batches of sampled heads (heads are independent, so the oracle
computes exactly those outputs); on those, every head of the device's outputs is
also held to the exact linearity identities of the scan.  Besides the per-tensor
error, every (batch, head, chunk) block is held to its own bound (gpu_common).
"""
import numpy as np
import pytest
import torch

from gpu_common import (GRADS, TOL, check_identities_all_heads, compare, gpu_fwd_bwd,
                        oracle_fwd_bwd, rel_l2, say, select_heads)
from mamba_ssd_chunked_amd import inputs, ssd

pytestmark = pytest.mark.gpu

KEYS = ("y", "final") + GRADS


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.load_library()


@pytest.mark.parametrize("use_init,use_d_final", [(False, False), (True, True)])
def test_tiny_workload_full(use_init, use_d_final):
    w = inputs.WORKLOADS["tiny_fp32"]
    w = inputs.Workload(**{**w.__dict__, "init_std": 0.5 if use_init else 0.0})
    say(f"case tiny_fp32 init={use_init} d_final={use_d_final}")
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp, use_init=use_init, use_d_final=use_d_final)
    ref = oracle_fwd_bwd(inp, use_init=use_init, use_d_final=use_d_final)
    compare(gpu, ref, TOL["f32"], KEYS, "tiny_fp32")


SHAPES = [
    # batch, seq, nheads, headdim, dstate, chunk_len, io
    (2, 768, 3, 64, 128, 256, "f32"),
    (1, 384, 2, 32, 64, 128, "f32"),
    (2, 320, 3, 16, 32, 64, "f32"),
    (1, 256, 2, 128, 16, 64, "f32"),
    (1, 512, 1, 16, 128, 128, "f32"),
    (1, 256, 2, 128, 128, 128, "f32"),
    (1, 64, 1, 64, 64, 64, "f32"),
    (2, 512, 2, 64, 128, 256, "bf16"),
    (1, 384, 3, 32, 16, 128, "bf16"),
    (1, 256, 2, 128, 64, 128, "bf16"),
    (2, 384, 2, 16, 128, 128, "bf16"),
    (1, 256, 2, 128, 128, 128, "bf16"),  # p * r above the whole-chunk kernels': block kernels
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%d_s%d_h%d_p%d_r%d_l%d_%s" % s)
def test_shapes_full(shape):
    b, seq, h, p, r, l, io = shape
    w = inputs.custom(batch=b, seq=seq, nheads=h, headdim=p, dstate=r, chunk_len=l, io=io,
                      init_std=0.3, seed=100 + seq + p + r)
    say(f"case {shape}")
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp)
    ref = oracle_fwd_bwd(inp)
    compare(gpu, ref, TOL[io], KEYS, str(shape))


# (workload, sampled heads, kernel_chunk_len): 0 is the automatic choice the benchmark
# times (128); 64 and 256 run the other kernel chunk lengths (256: the workloads' chunks unsplit).
FULL = [("mamba2_130m_fp32", [0, 13], 0), ("mamba2_130m_fp32", [5], 256),
        ("mamba2_130m_fp32", [22], 64),
        ("mamba2_2p7b_bf16", [41], 0), ("mamba2_2p7b_bf16", [12], 64), ("mamba2_2p7b_bf16", [63], 256),
        ("long_context_64k_fp32", [7], 0), ("long_context_64k_fp32", [30], 256),
        ("long_context_64k_fp32", [19], 64), ("moments_valid_len_fp32", [3], 0)]


@pytest.mark.parametrize("name,heads,kcl", FULL, ids=[f"{f[0]}-k{f[2]}" for f in FULL])
def test_full_size_sampled_heads(name, heads, kcl):
    w = inputs.WORKLOADS[name]
    say(f"case {name} full size, heads {heads}, kernel_chunk_len {kcl}")
    inp = inputs.make_inputs(w)
    use_init = w.init_std > 0
    gpu = gpu_fwd_bwd(inp, use_init=use_init, use_d_final=False, kernel_chunk_len=kcl)
    ref = oracle_fwd_bwd(inp, heads=heads, use_init=use_init, use_d_final=False)
    compare(select_heads(gpu, heads), ref, TOL[w.io], KEYS, name)
    for k in KEYS:
        assert np.all(np.isfinite(gpu[k])), k
    # every head of the device's outputs, through the exact linearity identities
    check_identities_all_heads(inp, gpu, TOL[w.io], use_init, False, name)


KCL = [(256, 64, "f32"), (256, 128, "f32"), (256, 256, "f32"), (128, 64, "f32"),
       (256, 64, "bf16"), (256, 256, "bf16")]


@pytest.mark.parametrize("l,kcl,io", KCL, ids=[f"l{k[0]}_k{k[1]}_{k[2]}" for k in KCL])
def test_kernel_chunk_len_matches_oracle(l, kcl, io):
    """Every kernel chunk length gives the recurrence's outputs (to the same bar)."""
    w = inputs.custom(batch=2, seq=768 if l == 256 else 384, nheads=3, headdim=64, dstate=128,
                      chunk_len=l, io=io, init_std=0.3, seed=700 + kcl)
    say(f"case chunk_len {l} kernel_chunk_len {kcl} {io}")
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp, kernel_chunk_len=kcl)
    ref = oracle_fwd_bwd(inp)
    compare(gpu, ref, TOL[io], KEYS, f"l={l} k={kcl} {io}")


# The limits of the decay, head by head: memoryless (A dt about -5e3: every decay between
# distinct tokens underflows to exactly 0 in fp32 and fp64 alike), no step (dt = 0: a = 1
# and nothing enters the state, d_A = 0), tiny steps, and an ordinary head; at the
# whole-chunk (128) and block (64) kernel chunk lengths, fp32 and bf16 inputs.  d_dt gets
# A d_da, and d_da's pair terms are a difference of the target- and source-side sums of
# d_diff; the diagonal pair t = s, whose terms cancel exactly and dominate a memoryless
# head, is held out of both sums, so A d_da carries no |A|-scaled rounding and every head,
# A = -1e4 included, is held to the plain tolerance.
# Also at the benchmarks' (headdim, dstate) = (64, 128), where the fp32 source-row kernel
# hands a tile over between waves on the diagonal block and bf16 runs the whole-chunk kernels.
EXTREME = [("f32", 128, 32, 32), ("f32", 64, 32, 32), ("bf16", 128, 32, 32), ("bf16", 64, 32, 32),
           ("f32", 128, 64, 128), ("f32", 64, 64, 128), ("bf16", 128, 64, 128)]


@pytest.mark.parametrize("io,kcl,p,r", EXTREME, ids=[f"{e[0]}_k{e[1]}_p{e[2]}_r{e[3]}" for e in EXTREME])
def test_extreme_decay_regimes(io, kcl, p, r):
    w = inputs.custom(batch=2, seq=256, nheads=4, headdim=p, dstate=r, chunk_len=128, io=io,
                      init_std=0.3, seed=901)
    inp = inputs.make_inputs(w)
    A, dt = inp["A"].clone(), inp["dt"].clone()
    A[0] = -1.0e4
    dt[:, 0] = 0.5 + 0.5 * dt[:, 0].abs()
    dt[:, 1] = 0.0
    dt[:, 2] = dt[:, 2] * 1e-6
    inp["A"], inp["dt"] = A, dt
    say(f"case extreme decay {io} kernel_chunk_len {kcl} p {p} r {r}")
    gpu = gpu_fwd_bwd(inp, kernel_chunk_len=kcl)
    ref = oracle_fwd_bwd(inp)
    for k in KEYS:
        assert np.all(np.isfinite(gpu[k])), k
    # the memoryless and no-step heads have no gradient w.r.t. A at all
    assert np.all(gpu["d_A"][:2] == 0.0) and np.all(ref["d_A"][:2] == 0.0)
    compare(gpu, ref, TOL[io], [k for k in KEYS if k != "d_dt"], f"extreme decay {io} k={kcl}")
    for h in range(w.nheads):
        e = rel_l2(gpu["d_dt"][:, h], ref["d_dt"][:, h])
        say(f"  head {h} (A = {float(A[h]):.3g}) d_dt rel-L2 {e:.2e} (bound {TOL[io]:.1e})")
        assert e <= TOL[io], (h, e)


# The backward's local gradient w.r.t. the within-chunk cumsum before its suffix sums
# (combined_backward.rs page, CombinedGrads: the local d_da of BLUE and ORANGE): g1 + g2,
# read from the workspace after ssd_bwd, against autodiff of the chunked evaluation through
# the chunk's own terms with the entry states held fixed (chunked_scan.local_gradients,
# which the page's identity d_da_local = dy . out_x - d_dt_orange dt ties to the oracle on
# the CPU).  At the layout's own chunk length, where the kernels' chunks are the layout's;
# the block kernels at 64 and 256, and at 128 with p * r above the whole-chunk kernels'.
LOCAL = [(64, 32, 64, "f32"), (256, 64, 128, "f32"), (128, 128, 128, "f32"), (64, 64, 32, "bf16")]


@pytest.mark.parametrize("l,p,r,io", LOCAL, ids=[f"l{c[0]}_p{c[1]}_r{c[2]}_{c[3]}" for c in LOCAL])
def test_local_dda_before_the_suffix_sums(l, p, r, io):
    import chunked_scan
    w = inputs.custom(batch=2, seq=3 * l, nheads=3, headdim=p, dstate=r, chunk_len=l, io=io,
                      init_std=0.3, seed=1300 + l + p)
    inp = inputs.make_inputs(w)
    say(f"case local d_da l={l} p={p} r={r} {io}")
    d = {k: v.cuda().contiguous() for k, v in inp.items() if isinstance(v, torch.Tensor)}
    dims = ssd.dims_of(d["x"], d["B"], l)
    ws = ssd.workspace(dims, ssd.SSD_OP_BWD, d["x"].device)
    ssd.backward(d["dy"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init"],
                 d_final=d["d_final"], ws=ws, kernel_chunk_len=l)
    torch.cuda.synchronize()

    def region(name):
        off, n = ssd.ssd_bwd_partial_region(dims, name)
        assert n > 0, name
        return ws[off:off + n].view(torch.float32).cpu().numpy().astype(np.float64)

    local_dev = region("g1") + region("g2")
    h = {k: inp[k].double().numpy() for k in ("dy", "x", "dt", "A", "B", "C", "init")}
    ref, _ = chunked_scan.local_gradients(h["dy"], h["x"], h["dt"], h["A"], h["B"], h["C"],
                                          h["init"])
    e = rel_l2(local_dev, ref.reshape(-1))
    say(f"  local d_da rel-L2 {e:.2e}")
    assert e <= TOL[io], e


# Many short slices: 8192 and 16384 chunks (batch x heads x chunks) at each kernel
# chunk length (the cumsum's lane widths 1, 2, 4), small headdim and dstate.
# (batch, seq, nheads, chunk_len, kernel_chunk_len, heads compared or None for all);
# headdim = dstate = 16.
MANY = [(2, 4096, 64, 64, 64, None), (2, 4096, 128, 64, 64, None),
        (2, 4096, 128, 128, 128, None), (2, 16384, 128, 256, 256, [0, 77, 127])]


@pytest.mark.parametrize("b,seq,h,l,kcl,heads", MANY,
                         ids=[f"b{m[0]}_s{m[1]}_h{m[2]}_k{m[4]}" for m in MANY])
def test_many_chunks(b, seq, h, l, kcl, heads):
    w = inputs.custom(batch=b, seq=seq, nheads=h, headdim=16, dstate=16, chunk_len=l, io="f32",
                      init_std=0.3, seed=800 + h + kcl)
    say(f"case many chunks b={b} seq={seq} h={h} kernel_chunk_len {kcl}")
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp, kernel_chunk_len=kcl)
    ref = oracle_fwd_bwd(inp, heads=heads)
    if heads is not None:
        gpu = select_heads(gpu, heads)
    compare(gpu, ref, TOL["f32"], KEYS, f"many chunks h={h} k={kcl}")


def test_bitwise_deterministic():
    w = inputs.custom(batch=2, seq=1024, nheads=4, headdim=64, dstate=128, chunk_len=256,
                      init_std=0.2, seed=77)
    say("case determinism")
    inp = inputs.make_inputs(w)
    a = gpu_fwd_bwd(inp)
    b = gpu_fwd_bwd(inp)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_null_init_and_d_final_mean_zero():
    w = inputs.custom(batch=1, seq=256, nheads=2, headdim=32, dstate=32, chunk_len=64,
                      init_std=0.0, seed=5)
    inp = inputs.make_inputs(w)
    inp["d_final"] = torch.zeros_like(inp["d_final"])
    say("case null init/d_final")
    a = gpu_fwd_bwd(inp, use_init=False, use_d_final=False)
    b = gpu_fwd_bwd(inp, use_init=True, use_d_final=True)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_empty_sequence_and_batch():
    say("case empty")
    w = inputs.custom(batch=2, seq=0, nheads=3, headdim=16, dstate=32, chunk_len=64,
                      init_std=1.0, seed=9)
    inp = inputs.make_inputs(w)
    gpu = gpu_fwd_bwd(inp)
    assert np.array_equal(gpu["final"], inp["init"].numpy())
    assert np.array_equal(gpu["d_init"], inp["d_final"].numpy())
    assert np.all(gpu["d_A"] == 0) and np.all(gpu["d_D"] == 0)
    w0 = inputs.custom(batch=0, seq=128, nheads=3, headdim=16, dstate=32, chunk_len=64, seed=9)
    inp0 = inputs.make_inputs(w0)
    gpu0 = gpu_fwd_bwd(inp0)
    assert gpu0["y"].size == 0 and np.all(gpu0["d_A"] == 0) and np.all(gpu0["d_D"] == 0)


def test_graph_replay_matches_eager():
    """The library neither allocates nor synchronises, so a fwd + bwd step can be captured
    into a HIP graph; every replay (with eager work of the program in between) must give
    the eager outputs bit for bit."""
    w = inputs.custom(batch=2, seq=512, nheads=3, headdim=64, dstate=128, chunk_len=256,
                      init_std=0.3, seed=57)
    inp = inputs.make_inputs(w)
    say("case graph capture of ssd_fwd + ssd_bwd")
    d = {k: v.cuda() for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "valid_len"}
    dims = ssd.dims_of(d["x"], d["B"])
    y, fin = torch.empty_like(d["x"]), torch.empty_like(d["d_final"])
    outs = [torch.empty_like(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "d_final")]
    wf, wb = ssd.workspace(dims, ssd.SSD_OP_FWD), ssd.workspace(dims, ssd.SSD_OP_BWD)

    def step():
        st = torch.cuda.current_stream()
        assert ssd.ssd_fwd(dims, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init"], y,
                           fin, wf, st) == 0
        assert ssd.ssd_bwd(dims, d["dy"], d["d_final"], d["x"], d["dt"], d["A"], d["B"], d["C"],
                           d["D"], d["init"], *outs, wb, st) == 0

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in [y, fin] + outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for it in range(3):
        for t in [y, fin] + outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip([y, fin] + outs, ref):
            assert torch.equal(a, b), f"replay {it}"
        step()  # eager work between replays
        torch.cuda.synchronize()
