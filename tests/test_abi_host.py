"""Host-side checks of the C ABI (no GPU needed; no kernel is ever launched here).

* the HIP library loads and exports every function ``include/ssd.h`` declares;
* ``ssd_workspace_size`` follows the documented plan;
* every entry point rejects bad arguments with its documented status code
  before it touches HIP (fake, aligned device addresses are never dereferenced
  because validation fails first);
* the Python binding refuses buffers of the wrong device, dtype or size, and
  fails loudly when the library is missing.
"""
import ctypes
import os
import re

import pytest
import torch

from mamba_ssd_chunked_amd import build as hipbuild
from mamba_ssd_chunked_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

FAKE = 1 << 20  # an aligned non-null address: only validation ever sees it


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        hipbuild.build()
    return ssd.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert header_functions() == sorted(ssd.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def dims(b=2, n=3, l=64, h=2, p=16, r=32, io=0):
    return ssd.make_dims(b, n, l, h, p, r, io)


@pytest.mark.parametrize("kcl,k", [(256, 256), (128, 128), (64, 64), (0, 128)])
def test_workspace_plan(lib, kcl, k):
    """The plan at kernel chunk length k: the 8 x 256-token chunks become 8 * 256 / k."""
    d = dims(b=4, n=8, l=256, h=24, p=64, r=128)
    d.kernel_chunk_len = kcl
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    tok, chunks = 4 * 24 * 8 * 256, 4 * 24 * 8 * 256 // k
    states = chunks * 64 * 128
    assert ssd.ssd_workspace_size(d, ssd.SSD_OP_FWD) == up(8 * tok) + up(4 * states)
    pair_tiles = (k // 16) * (k // 16 + 1) // 2  # causal 16 x 16 tiles per chunk (d_CB hand-off)
    bwd = up(8 * tok) + 2 * up(4 * states) + 3 * up(4 * tok) + up(4 * chunks) \
        + 3 * up(8 * chunks * (k // 64)) + up(4 * 256 * chunks * pair_tiles) \
        + up(4 * tok)  # the diagonal d_CB[t, t], handed over beside the pair tiles
    assert ssd.ssd_workspace_size(d, ssd.SSD_OP_BWD) == bwd


@pytest.mark.parametrize("kcl,p,r,g1_written", [(64, 64, 128, True), (256, 64, 128, True),
                                                 (128, 64, 128, False), (128, 128, 128, True)])
def test_bwd_partial_regions(lib, kcl, p, r, g1_written):
    """g1, g2, d_delta sit where the backward's plan puts them (after the cumsums and the
    two state buffers, one fp32 per token-head each); g1 is reported unwritten where the
    whole-chunk kernels run (kernel chunk 128, p * r <= 8192)."""
    d = dims(b=2, n=4, l=256, h=3, p=p, r=r)
    d.kernel_chunk_len = kcl
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    k = kcl
    tok, chunks = 2 * 3 * 4 * 256, 2 * 3 * 4 * 256 // k
    states = chunks * p * r
    base = up(8 * tok) + 2 * up(4 * states)
    assert ssd.ssd_bwd_partial_region(d, "g1") == (base, 4 * tok if g1_written else 0)
    assert ssd.ssd_bwd_partial_region(d, "g2") == (base + up(4 * tok), 4 * tok)
    assert ssd.ssd_bwd_partial_region(d, "d_delta") == (base + 2 * up(4 * tok), 4 * tok)
    total = ssd.ssd_workspace_size(d, ssd.SSD_OP_BWD)
    for name in ("g1", "g2", "d_delta"):
        off, n = ssd.ssd_bwd_partial_region(d, name)
        assert off + n <= total and off % 256 == 0


def test_bwd_partial_region_rejects_bad_arguments(lib):
    d = dims()
    with pytest.raises(ssd.SsdError, match="unknown region"):
        ssd.ssd_bwd_partial_region(d, "g3")
    off = ctypes.c_size_t(0)
    assert lib.ssd_bwd_partial_region(ctypes.byref(d), b"g1", ctypes.byref(off), None) == 1
    assert lib.ssd_bwd_partial_region(ctypes.byref(d), None, ctypes.byref(off), ctypes.byref(off)) == 1
    for name in ("g1", "g2", "d_delta"):  # an empty sequence writes none of them
        assert ssd.ssd_bwd_partial_region(dims(n=0), name)[1] == 0


@pytest.mark.parametrize("l,kcl", [(256, 96), (256, 512), (128, 256), (64, 128), (256, -64),
                                   (128, 32)])
def test_bad_kernel_chunk_len_is_rejected(lib, l, kcl):
    d = dims(l=l)
    d.kernel_chunk_len = kcl
    out = ctypes.c_size_t(0)
    assert lib.ssd_workspace_size(ctypes.byref(d), 0, ctypes.byref(out)) == 3
    assert "kernel_chunk_len" in ssd.ssd_last_error()
    assert lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 10), 1 << 30, FAKE) == 3


@pytest.mark.parametrize("bad,code", [
    (dict(l=32), 3), (dict(l=96), 3), (dict(l=512), 3), (dict(p=8), 3), (dict(p=48), 3),
    (dict(r=256), 3), (dict(b=-1), 2), (dict(n=-1), 2), (dict(h=0), 2), (dict(p=0), 2),
    (dict(io=2), 4),
])
def test_bad_dims_are_rejected(lib, bad, code):
    d = dims(**bad)
    out = ctypes.c_size_t(0)
    assert lib.ssd_workspace_size(ctypes.byref(d), 0, ctypes.byref(out)) == code
    assert ssd.ssd_last_error() != ""
    rc = lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 10), 1 << 30, FAKE)
    assert rc == code


def test_null_dims_and_null_pointers(lib):
    out = ctypes.c_size_t(0)
    assert lib.ssd_workspace_size(None, 0, ctypes.byref(out)) == 1
    d = dims()
    args = [FAKE] * 10
    for i in (0, 1, 2, 3, 4, 5, 7):  # x, dt, A, B, C, D, y (init and final are nullable)
        a = list(args)
        a[i] = None
        assert lib.ssd_fwd(ctypes.byref(d), *a, 1 << 30, None) == 1, i
    bargs = [FAKE] * 17
    for i, name in enumerate(["dy", "d_final", "x", "dt", "A", "B", "C", "D", "init", "d_x",
                              "d_dt", "d_A", "d_B", "d_C", "d_D", "d_init"]):
        if name in ("d_final", "init", "d_init"):
            continue
        a = list(bargs)
        a[i] = None
        assert lib.ssd_bwd(ctypes.byref(d), *a, 1 << 30, None) == 1, name


def test_workspace_too_small_and_misaligned(lib):
    d = dims()
    need = ssd.ssd_workspace_size(d, ssd.SSD_OP_FWD)
    assert lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 9), FAKE, need - 1, None) == 5
    assert lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 9), None, need, None) == 5
    assert lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 9), FAKE + 4, need, None) == 3
    # misaligned tensor pointers
    a = [FAKE] * 10
    a[0] = FAKE + 4
    assert lib.ssd_fwd(ctypes.byref(d), *a, need, None) == 3
    bf = dims(io=1)
    a[0] = FAKE + 8  # 8-byte alignment is enough for bf16 tensors ...
    need_bf = ssd.ssd_workspace_size(bf, ssd.SSD_OP_FWD)
    assert lib.ssd_fwd(ctypes.byref(bf), *a[:9], FAKE + 4, need_bf, None) == 3  # ... not for ws


def test_noalloc_forward_validation(lib):
    """ssd_fwd_noalloc checks what ssd_fwd checks and rejects problems whose workspace
    exceeds its fixed scratch with SSD_ERR_WORKSPACE, all before any HIP call."""
    d = dims()
    args = [FAKE] * 9
    for i in (0, 1, 2, 3, 4, 5, 7):  # x, dt, A, B, C, D, y
        a = list(args)
        a[i] = None
        assert lib.ssd_fwd_noalloc(ctypes.byref(d), *a, None) == 1, i
    assert lib.ssd_fwd_noalloc(ctypes.byref(dims(l=96)), *args, None) == 3
    a = list(args)
    a[0] = FAKE + 4
    assert lib.ssd_fwd_noalloc(ctypes.byref(d), *a, None) == 3
    big = dims(b=1, n=256, l=256, h=32, p=64, r=128)  # the 64k-token workload: 0.55 GB
    assert ssd.ssd_workspace_size(big, ssd.SSD_OP_FWD) > ssd.NOALLOC_SCRATCH_BYTES
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), *args, None) == 5
    assert "scratch" in ssd.ssd_last_error()
    fits = dims(b=4, n=8, l=256, h=24, p=64, r=128)  # the 130M-shaped workload: 51.9 MB
    assert ssd.ssd_workspace_size(fits, ssd.SSD_OP_FWD) <= ssd.NOALLOC_SCRATCH_BYTES
    header = open(HEADER).read()
    assert "#define SSD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)" in header
    assert ssd.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024


def test_moments_validation(lib):
    d = dims()
    assert lib.ssd_state_moments(None, *([FAKE] * 14), 1 << 30, None) == 1
    assert lib.ssd_state_moments_bwd(ctypes.byref(dims(l=100)), *([FAKE] * 14), 1 << 30,
                                     None) == 3
    del d


def test_binding_refuses_wrong_buffers(lib):
    d = dims(b=1, n=1, l=64, h=1, p=16, r=16)
    x = torch.zeros(1, 1, 64, 1, 16)
    with pytest.raises(ValueError, match="device tensor"):
        ssd.ssd_fwd(d, x, x, x, x, x, x, None, x, None, None)
    with pytest.raises(ValueError, match="elements"):
        ssd.ssd_fwd(d, torch.zeros(5), x, x, x, x, x, None, x, None, None)
    with pytest.raises(TypeError, match="float32"):
        ssd.ssd_fwd(d, x.double(), x, x, x, x, x, None, x, None, None)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(ssd, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        ssd.load_library("/nonexistent/libmamba_ssd_hip.so")


def counts(*v):
    return (ctypes.c_int64 * len(v))(*v)


@pytest.mark.parametrize("case,code", [
    (dict(b=-1), 2), (dict(h=0), 2), (dict(r=8), 3), (dict(r=48), 3), (dict(r=256), 3),
    (dict(count=(4, 0)), 2), (dict(count=(-3, 4)), 2), (dict(m2=0), 1), (dict(out=0), 1),
    (dict(center=1, m1=0), 1), (dict(m2=FAKE + 4), 3), (dict(out=FAKE + 8), 3),
])
def test_pr_entry_points_reject_bad_arguments(lib, case, code):
    a = dict(b=2, h=3, r=32, m2=FAKE, m1=FAKE, count=(5, 7), center=0, out=FAKE)
    a.update(case)
    cnt = counts(*a["count"])
    if "out" not in case or case["out"] == 0:  # pr itself needs no 16-byte alignment
        rc = lib.ssd_moments_pr(a["b"], a["h"], a["r"], a["m2"], a["m1"], cnt, a["center"],
                                a["out"], None, None)
        assert rc == code, ssd.ssd_last_error()
    rc = lib.ssd_moments_pr_bwd(a["b"], a["h"], a["r"], FAKE, a["m2"], a["m1"], cnt, a["center"],
                                a["out"], None, None)
    assert rc == code, ssd.ssd_last_error()


def test_pr_of_an_empty_batch_is_a_no_op(lib):
    assert lib.ssd_moments_pr(0, 3, 32, None, None, None, 1, None, None, None) == 0
    assert lib.ssd_moments_pr_bwd(0, 3, 32, None, None, None, None, 1, None, None, None) == 0


@pytest.mark.parametrize("case,code", [
    (dict(T=-1), 2), (dict(m=0), 2), (dict(h=0), 2), (dict(p=0), 2), (dict(m=3), 3), (dict(m=8), 3),
    (dict(p=48), 3), (dict(r=256), 3), (dict(io=2), 4), (dict(v=0), 1), (dict(gamma=0), 1),
    (dict(out=0), 1), (dict(v=FAKE + 4), 3), (dict(out=FAKE + 8), 3), (dict(io=1, v=FAKE + 4), 3),
])
def test_y_diag_entry_points_reject_bad_arguments(lib, case, code):
    a = dict(T=10, m=2, h=3, p=32, r=64, io=0, v=FAKE, gamma=FAKE, out=FAKE)
    a.update(case)
    rc = lib.ssd_y_diag(a["T"], a["m"], a["h"], a["p"], a["r"], a["io"], a["v"], FAKE, FAKE,
                        a["gamma"], a["out"], None)
    assert rc == code, ssd.ssd_last_error()
    rc = lib.ssd_y_diag_bwd(a["T"], a["m"], a["h"], a["p"], a["r"], a["io"], FAKE, a["v"], FAKE, FAKE,
                            a["gamma"], a["out"], FAKE, FAKE, FAKE, None)
    assert rc == code, ssd.ssd_last_error()


def test_y_diag_of_no_tokens_is_a_no_op(lib):
    assert lib.ssd_y_diag(0, 4, 3, 64, 128, 0, None, None, None, None, None, None) == 0
    assert lib.ssd_y_diag_bwd(0, 4, 3, 64, 128, 0, *([None] * 10)) == 0


@pytest.mark.parametrize("case,code", [
    (dict(b=-1), 2), (dict(s=-1), 2), (dict(h=0), 2), (dict(j=0), 2), (dict(h=1 << 13, j=1 << 12), 3),
    (dict(q=0), 1), (dict(out=0), 1), (dict(q=FAKE + 4), 3), (dict(out=FAKE + 8), 3),
    (dict(init=FAKE + 4), 3), (dict(ws=0), 5), (dict(ws_bytes=16), 5), (dict(ws=FAKE + 64), 3),
])
def test_quat_entry_points_reject_bad_arguments(lib, case, code):
    a = dict(b=2, s=50, h=3, j=5, q=FAKE, init=None, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(case)
    rc = lib.ssd_quat_scan(a["b"], a["s"], a["h"], a["j"], a["q"], a["init"], a["out"], a["ws"],
                           a["ws_bytes"], None)
    assert rc == code, ssd.ssd_last_error()
    rc = lib.ssd_quat_scan_bwd(a["b"], a["s"], a["h"], a["j"], a["q"], a["init"], FAKE, a["out"],
                               None, a["ws"], a["ws_bytes"], None)
    assert rc == code, ssd.ssd_last_error()


def test_quat_workspace_plan(lib):
    # a ticket per (batch, 64-lane group) chain (64 words each) and pass, and fp64
    # quaternion records of 64 lanes x 4 words per segment (2 KiB each): forward the
    # aggregates; backward also the forward-carry pass's inclusive values and the reverse
    # pass's two aggregate arrays (M and v); plus per block of 8 segments the block
    # aggregates (1 array forward, 3 backward).  Segments are 64 steps in the forward and the
    # backward's carry pass (its aggregates and block aggregates) and 32 steps in the reverse
    # pass (the inclusive values, one per reverse segment, and the reverse pass's arrays).
    b, s, h, j = 4, 2048, 24, 32
    chains = b * (h * j // 64)
    segs_f, segs_b = chains * (s // 64), chains * (s // 32)
    blocks_f, blocks_b = chains * -(-(s // 64) // 8), chains * -(-(s // 32) // 8)
    rec = 64 * 32
    fwd = ssd.ssd_quat_workspace_size(b, s, h, j, False)
    bwd = ssd.ssd_quat_workspace_size(b, s, h, j, True)
    # (plus 256 bytes for the call tag kept across calls)
    assert fwd == 256 + 4 * 64 * chains + rec * (segs_f + blocks_f)
    assert bwd == 256 + 8 * 64 * chains + rec * (segs_f + blocks_f + 3 * segs_b + 2 * blocks_b)
    # ragged: 15 lanes still take a whole group; 97 steps are two 64-step segments and four
    # 32-step ones (one block each)
    assert ssd.ssd_quat_workspace_size(2, 97, 3, 5, False) == 256 + 4 * 64 * 2 + rec * (2 * 2 + 2)
    assert ssd.ssd_quat_workspace_size(2, 97, 3, 5, True) == (
        256 + 8 * 64 * 2 + rec * (2 * 2 + 2 + 3 * 2 * 4 + 2 * 2))
    for args in ((0, 10, 2, 2), (3, 0, 2, 2)):
        assert ssd.ssd_quat_workspace_size(*args, False) == 0
        assert ssd.ssd_quat_workspace_size(*args, True) == 0


def test_quat_of_nothing_is_a_no_op(lib):
    assert lib.ssd_quat_scan(0, 10, 2, 2, None, None, None, None, 0, None) == 0
    assert lib.ssd_quat_scan(3, 0, 2, 2, None, None, None, None, 0, None) == 0
    assert lib.ssd_quat_scan_bwd(0, 10, 2, 2, None, None, None, None, None, None, 0, None) == 0
    # an empty sequence with no d_init requested enqueues nothing
    assert lib.ssd_quat_scan_bwd(3, 0, 2, 2, None, None, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("case,code", [
    (dict(b=-1), 2), (dict(h=0), 2), (dict(p=0), 2), (dict(p=48), 3), (dict(r=8), 3), (dict(r=256), 3),
    (dict(io=2), 4), (dict(x=0), 1), (dict(state=0), 1), (dict(y=0), 1), (dict(B=FAKE + 4), 3),
    (dict(state=FAKE + 8), 3), (dict(io=1, B=FAKE + 4), 3),
    # new_state overlapping state without being it
    (dict(new=FAKE + 4096), 3),
])
def test_step_rejects_bad_arguments(lib, case, code):
    a = dict(b=2, h=3, p=32, r=64, io=0, x=FAKE, B=FAKE, state=FAKE + (1 << 24), new=None, y=FAKE)
    a.update(case)
    new = a["new"] if a["new"] is not None else a["state"]
    if "new" in case:
        a["state"] = FAKE
    rc = lib.ssd_step(a["b"], a["h"], a["p"], a["r"], a["io"], a["x"], FAKE, FAKE, a["B"], FAKE,
                      FAKE, a["state"], new, a["y"], None)
    assert rc == code, ssd.ssd_last_error()


def test_step_of_an_empty_batch_is_a_no_op(lib):
    assert lib.ssd_step(0, 3, 64, 128, 0, *([None] * 10)) == 0


def test_debug_switch_is_host_only(lib):
    """ssd_debug_enable only flips a host flag (no device call): it works without a GPU."""
    assert lib.ssd_debug_enable(1) == 0
    assert lib.ssd_debug_enable(0) == 0
    assert ssd.STATUS[7] == "SSD_ERR_NONFINITE"


# Every launch's grid must fit the 32-bit work-item count of a dispatch: each entry point
# rejects, before any device call, a problem whose largest launch would not.
@pytest.mark.parametrize("b,n,l,h,p,r,ok", [
    (1, 1 << 12, 256, 1024, 16, 16, False),   # per-token-block kernels: 4 b h n l = 2^32
    (1, 1 << 11, 256, 1024, 16, 16, True),    # 2^31
    (1, 1, 64, 1 << 18, 128, 128, False),     # state copies: b h p r = 2^32
    (1, 1, 64, 1 << 17, 128, 128, True),
])
def test_ssd_grid_size_limit(lib, b, n, l, h, p, r, ok):
    d = dims(b=b, n=n, l=l, h=h, p=p, r=r)
    out = ctypes.c_size_t(0)
    for op in range(4):
        rc = lib.ssd_workspace_size(ctypes.byref(d), op, ctypes.byref(out))
        if ok:
            assert rc == 0, ssd.ssd_last_error()
        else:
            assert rc == 3 and "2^32 work-items" in ssd.ssd_last_error()
    if not ok:
        assert lib.ssd_fwd(ctypes.byref(d), *([FAKE] * 10), 1 << 62, FAKE) == 3


def test_other_entry_points_grid_size_limit(lib):
    def rejected(rc):
        return rc == 3 and "2^32 work-items" in ssd.ssd_last_error()
    # y_diag: 16 work-items per (token, head)
    assert rejected(lib.ssd_y_diag(1 << 28, 1, 1, 16, 16, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None))
    assert rejected(lib.ssd_y_diag_bwd(1 << 28, 1, 1, 16, 16, 0, *([FAKE] * 9), None))
    # quaternion scan: 256 per (batch, 64-lane group, segment), segments of 64 steps in the
    # forward and 32 in the backward, so 2^9 groups of 2^20 steps fit the forward (2^31
    # work-items) but not the backward (2^32)
    assert rejected(lib.ssd_quat_scan(1, 1 << 20, 1 << 13, 8, FAKE, None, FAKE, FAKE, 1 << 62, None))
    size = ctypes.c_size_t(0)
    assert lib.ssd_quat_workspace_size(1, 1 << 20, 1 << 12, 8, 0, ctypes.byref(size)) == 0
    assert rejected(lib.ssd_quat_workspace_size(1, 1 << 20, 1 << 12, 8, 1, ctypes.byref(size)))
    assert rejected(lib.ssd_quat_scan_bwd(1, 1 << 20, 1 << 12, 8, FAKE, None, FAKE, FAKE, None,
                                          FAKE, 1 << 62, None))
    # decode step and participation ratio: 256 per (batch, head)
    assert rejected(lib.ssd_step(1 << 12, 1 << 12, 16, 16, 0, *([FAKE] * 10)))
    cnt = counts(1)
    assert rejected(lib.ssd_moments_pr(1 << 12, 1 << 12, 16, FAKE, FAKE, cnt, 0, FAKE, None, None))


def test_stream_probe_validates_before_any_launch(lib):
    """The benchmark's streaming probe refuses an unknown mix, a missing buffer and a negative
    size on the host."""
    buf = ctypes.c_void_p(0x1000)
    assert lib.ssd_stream_probe(5, 1, 0, buf, buf, 16, None) == 3      # SSD_ERR_UNSUPPORTED
    assert lib.ssd_stream_probe(2, 2, 0, buf, buf, 16, None) == 3
    assert lib.ssd_stream_probe(3, 1, 0, None, buf, 16, None) == 1     # SSD_ERR_NULL
    assert lib.ssd_stream_probe(0, 1, 0, None, None, 16, None) == 1
    assert lib.ssd_stream_probe(1, 1, 1, buf, buf, -1, None) == 2      # SSD_ERR_SHAPE
    assert lib.ssd_stream_probe(1, 0, 0, buf, buf, 0, None) == 0       # nothing to move: no launch
