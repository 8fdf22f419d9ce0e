"""Benchmark: SSD forward + recompute backward on one MI355X.

One step = ``ssd_fwd`` + ``ssd_bwd`` (K1-K5 forward, then the recompute
backward) over one batch of the workload, inputs already resident in HBM.
The headline workload is the largest one that fits one GPU: 65536 tokens x 32
heads (p = 64, r = 128, fp32).  Prints ONE JSON line with tokens/s, the roofline
of the dominant kernel (algorithmic work per launch / its mean duration,
measured with HIP events on the launch stream during the timed region) and the
CPU oracle timed on a bounded sample of the same workload, single-threaded and
over all host cores.

Warm-up: the --warmup steps, then more steps until at least --warmup-ms of GPU
time has passed (the clocks take tens of milliseconds to settle); both counts
are reported.  The kernels run the chunked algorithm at the library's automatic
kernel chunk length (min(chunk_len, 128); the workload's chunk_len fixes the
buffer layout); the same step with the kernels at the layout's chunk length is
timed as well and reported under "at_layout_chunk_len".  The Mamba-2-130M- and
2.7B-shaped workloads are timed the same way under "other_workloads".

    python bench.py [--gpus 1] [--steps 30] [--warmup 10] [--warmup-ms 300]
                    [--workload long_context_64k_fp32] [--graph]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd+bwd tokens/s on 1 MI355X; % MFMA peak (GEMMs), % HBM BW (K1/K4)"
PEAK_FP32_MFMA = 157.3e12   # FLOP/s, MI355X dense fp32 matrix
PEAK_BF16_MFMA = 2.5e15     # FLOP/s, MI355X dense bf16 matrix
PEAK_HBM = 8.0e12           # B/s
HEADLINE = "long_context_64k_fp32"


# HBM bytes per launch (read, write) of a kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
# WRITE_SIZE; scaled x2.0 / x1.0 by the same counters on a 256 MiB device copy), keyed by
# (kernel, workload, kernel chunk length), valid only while the hash of the kernel's code (its
# source files without comments) is the one they were taken on (profiles/ssd_kernels_*.md
# have the runs).
TRAFFIC = {
    ("k_bwd_source", "long_context_64k_fp32", 128): (5_383_494_528, 2_250_249_587, "73e7055f476ac366"),
    ("k_bwd_source", "mamba2_130m_fp32", 128): (501_964_390, 210_973_709, "73e7055f476ac366"),
    ("k_bwd_source", "mamba2_2p7b_bf16", 128): (744_073_728, 451_298_918, "c3af78ca06b3b471"),
}
# the files a kernel's code comes from, by io type: with bf16 io the source-row kernel at
# 128-token chunks is the whole-chunk one
TRAFFIC_SOURCES = {("k_bwd_source", "f32"): ("k_chunk_bwd.hip", "ssd_device.hpp"),
                   ("k_bwd_source", "bf16"): ("k_chunk_wide.hip", "ssd_device.hpp"),
                   ("k_bwd_target", "f32"): ("k_chunk_wide.hip", "ssd_device.hpp"),
                   ("k_bwd_target", "bf16"): ("k_chunk_wide.hip", "ssd_device.hpp")}


def code_of(src: str) -> str:
    """C++ source without its comments and with runs of white space made one space: what the
    compiler sees, so that an edited comment does not count as a changed kernel."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"' or c == "'":  # a string or character literal, escapes included
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def traffic_hash(kernel: str, io: str) -> str:
    """First 16 hex digits of the sha256 of the code (comments dropped) of the kernel's source
    files (TRAFFIC_SOURCES)."""
    import hashlib
    m = hashlib.sha256()
    for f in TRAFFIC_SOURCES[(kernel, io)]:
        with open(os.path.join(ROOT, "mamba_ssd_chunked_amd", "csrc", f), encoding="utf-8") as fh:
            m.update(code_of(fh.read()).encode())
    return m.hexdigest()[:16]


def measured_traffic(kernel: str, w, k: int):
    """HBM bytes per launch of `kernel` from the counter runs, or None when none were taken for
    this workload or the kernel's sources changed since."""
    ent = TRAFFIC.get((kernel, w.name, k))
    if ent is None:
        return None
    return ent[0] + ent[1] if traffic_hash(kernel, w.io) == ent[2] else None


def kernel_chunk_len(w, requested: int = 0) -> int:
    """The chunk length the kernels run at (the library's rule for 0: min(l, 128))."""
    return requested or min(w.chunk_len, 128)


def _shape(w, k):
    """(b, n, l, h, p, r) of workload w run at kernel chunk length k."""
    return w.batch, w.seq // k, k, w.nheads, w.headdim, w.dstate


def matrix_flops(w, kernel: str, k: int):
    """Algorithmic flops of ONE launch of a matrix kernel for workload w run at kernel chunk
    length k, by the matrix-core form that performs them: (fp32 MFMA, bf16 MFMA with two bf16
    operands, bf16 MFMA on the three exact bf16 parts of an fp32 operand), or None for a kernel
    without products.  Only the causal triangle counts (pairs s <= t of a chunk), each product
    once.  With bf16 io the products whose two operands are both bf16 inputs -- C B^T and
    dy x^T -- run on bf16 MFMAs; every other product has one exact-bf16 operand and one
    fp32 operand (the decay-weighted tile W, d_CB, S_in in BLUE, d_intra in K3, the
    token-weighted rows of the state kernel) and runs split: three bf16 MFMAs on the fp32
    operand's exact bf16 parts.  None runs on fp32 MFMAs."""
    b, n, l, h, p, r = _shape(w, k)
    ch = b * n * h                      # chunk-heads
    pairs = l * (l + 1) // 2            # (t, s) pairs with s <= t per chunk
    cb, dw = 2 * pairs * r, 2 * pairs * p          # C B^T and dy x^T tiles
    if kernel == "k_chunk_states":      # fwd: 1 job; bwd: 2 jobs (timed per launch: see jobs)
        both, split = 0, 2 * l * p * r
    elif kernel == "k5_chunk_scan":     # BLUE C S_in, C B^T, W x
        both, split = cb, 2 * l * p * r + 2 * pairs * p
    elif kernel == "k_bwd_target":      # BLUE dy S_in, d_CB B (d_CB handed over by k_bwd_source)
        both, split = 0, 2 * l * p * r + 2 * pairs * r
    elif kernel == "k_bwd_source":      # K3 (two products), C B^T, dy x^T, W^T dy, d_CB^T C
        both, split = cb + dw, 4 * l * p * r + 2 * pairs * p + 2 * pairs * r
    else:
        return None
    if w.io != "bf16":
        return (both + split) * ch, 0, 0
    return 0, both * ch, split * ch


def mfma_roof_s(w, kernel: str, k: int, launches: float = 1.0):
    """Seconds the matrix cores need at their dense peaks for `launches` launches of a
    matrix kernel: fp32 flops at the fp32 peak, bf16 flops at the bf16 peak, split products
    three times at the bf16 peak."""
    f32, both, split = matrix_flops(w, kernel, k)
    return launches * (f32 / PEAK_FP32_MFMA + (both + 3 * split) / PEAK_BF16_MFMA)


def kernel_work(w, kernel: str, k: int):
    """Algorithmic work of ONE launch of `kernel` for workload w run at kernel chunk
    length k: (amount, kind).

    kind "flop": the products the kernel performs, causal triangle only
    (pairs s <= t of a chunk); kind "byte": the HBM bytes the kernel must move."""
    b, n, l, h, p, r = _shape(w, k)
    ch = b * n * h                      # chunk-heads
    tok = ch * l                        # token-heads
    mf = matrix_flops(w, kernel, k)
    if mf is not None:
        return sum(mf), "flop"
    if kernel == "k1_cumsum":
        return 12 * tok + 4 * h, "byte"
    if kernel == "k4_state_pass":
        return 8 * p * r * ch + 8 * ch + 8 * b * h * p * r, "byte"
    if kernel == "k4_state_pass_bwd":
        return 16 * p * r * ch + 8 * ch + 8 * b * h * p * r, "byte"
    if kernel == "k1t_revcumsum":       # with the per-head d_A / d_D sums in the same launch
        return 24 * tok + 8 * ch + 24 * ch * (l // 64) + 8 * h, "byte"
    return None, None


RIDGE_FP32 = PEAK_FP32_MFMA / PEAK_HBM  # flop/B where the fp32 matrix and HBM roofs meet


def chunk_kernel_bytes(w, kernel: str, k: int):
    """Algorithmic HBM bytes of one launch of a chunk (matrix) kernel: every input it needs read
    once and every output written once (io-dtype token rows, fp32 dt and chunk states, fp64
    cumsums), for the roofline it is not bound by.  None for the other kernels."""
    b, n, l, h, p, r = _shape(w, k)
    ch = b * n * h
    tok = ch * l
    io = 2 if w.io == "bf16" else 4
    st = 4 * p * r * ch                 # one fp32 [p, r] state per chunk-head
    if kernel == "k_chunk_states":      # mean of the fwd launch (job 0) and the bwd one (jobs 0, 1)
        job0 = tok * (io * (p + r) + 12) + st     # x, B, dt, cdt -> S
        job1 = tok * (io * (p + r) + 8) + st      # dy, C, cdt -> dS
        return (2 * job0 + job1) / 2
    if kernel == "k5_chunk_scan":       # x, B, C, dt, cdt, S_in -> y
        return tok * (io * (2 * p + 2 * r) + 12) + st
    tiles = 1024 * (l // 16) * (l // 16 + 1) // 2 * ch   # the causal d_CB pair tiles (fp32)
    if kernel == "k_bwd_target":        # dy, C, B, cdt, S_in, d_intra, d_CB tiles and diagonal,
        return tok * (io * (p + 3 * r) + 28) + 2 * st + tiles   # g2, d_delta, d_dt -> d_C, d_dt
    if kernel == "k_bwd_source":        # dy, x, B, C, dt, cdt, d_intra -> d_x, d_B, d_dt, g2,
        return tok * (io * (3 * p + 3 * r) + 28) + st + tiles   # d_delta, d_CB tiles and diagonal
    return None


def kernel_rw(w, kernel: str, k: int):
    """(read, write) split of the algorithmic HBM bytes of one launch (the totals of kernel_work
    and chunk_kernel_bytes), for the comparison with the streaming rate of the same mix; None for
    kernels without a byte count."""
    b, n, l, h, p, r = _shape(w, k)
    ch = b * n * h
    tok = ch * l
    io = 2 if w.io == "bf16" else 4
    st = 4 * p * r * ch
    tiles = 1024 * (l // 16) * (l // 16 + 1) // 2 * ch
    if kernel == "k1_cumsum":
        return 4 * tok + 4 * h, 8 * tok
    if kernel == "k4_state_pass":
        return 4 * p * r * ch + 8 * ch + 4 * b * h * p * r, 4 * p * r * ch + 4 * b * h * p * r
    if kernel == "k4_state_pass_bwd":
        return 8 * p * r * ch + 8 * ch + 4 * b * h * p * r, 8 * p * r * ch + 4 * b * h * p * r
    if kernel == "k_chunk_states":      # mean of the fwd launch (job 0) and the bwd one (jobs 0, 1)
        r0, r1 = tok * (io * (p + r) + 12), tok * (io * (p + r) + 8)
        return (2 * r0 + r1) / 2, 1.5 * st
    if kernel == "k5_chunk_scan":
        return tok * (io * (p + 2 * r) + 12) + st, tok * io * p
    if kernel == "k_bwd_target":
        return tok * (io * (p + 2 * r) + 24) + 2 * st + tiles, tok * (io * r + 4)
    if kernel == "k_bwd_source":
        return tok * (io * (2 * p + 2 * r) + 12) + st, tok * (io * (p + r) + 16) + tiles
    return None


STREAM_MIXES = [(1, 0), (6, 1), (4, 1), (3, 1), (2, 1), (1, 1), (0, 1)]


def stream_roofs(mib: int = 256, reps: int = 10) -> dict:
    """HBM rate (bytes/s) of the library's streaming probe (ssd_stream_probe) for each
    read:write mix, the better of cached and non-temporal accesses, over arrays of `mib` MiB:
    what a kernel that only moves bytes in that mix reaches on this GPU."""
    import torch
    from mamba_ssd_chunked_amd import ssd
    n16 = mib * (1 << 20) // 16
    src = torch.zeros(6 * 4 * n16, device="cuda")
    dst = torch.zeros(4 * n16, device="cuda")
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for nr, nw in STREAM_MIXES:
        best = 0.0
        for nt in (False, True):
            sv = src[:4 * nr * n16] if nr else None
            dv = dst[:4 * max(nw, 1) * n16]
            for it in range(3 + reps):
                if it == 3:
                    e0.record(st)
                rc = ssd.ssd_stream_probe(nr, nw, nt, sv, dv, n16, st)
                if rc:
                    raise ssd.SsdError(rc, "ssd_stream_probe", ssd.ssd_last_error())
            e1.record(st)
            e1.synchronize()
            sec = e0.elapsed_time(e1) / 1e3 / reps
            best = max(best, (nr + nw) * 16 * n16 / sec)
        out[f"{nr}:{nw}"] = best
    del src, dst
    return out


def annotate_stream(kernels: dict, w, k: int, roofs: dict):
    """Each kernel with a byte rate gets its read:write split and the streaming rate of the
    nearest mix (by read share): stream_roof_gbps, and stream_frac = its algorithmic bytes per
    second over that rate."""
    for name, ent in kernels.items():
        rw = kernel_rw(w, name, k)
        if rw is None or "gbps" not in ent:
            continue
        rd, wr = rw
        share = rd / (rd + wr)
        mix = min(STREAM_MIXES, key=lambda m: abs(m[0] / (m[0] + m[1]) - share))
        roof = roofs[f"{mix[0]}:{mix[1]}"]
        ent.update(read_share=round(share, 3), stream_mix=f"{mix[0]}:{mix[1]}",
                   stream_roof_gbps=round(roof / 1e9, 1),
                   stream_frac=round(ent["gbps"] * 1e9 / roof, 4))


def moments_kernel_work(w, kernel: str, k: int):
    """Algorithmic flops of one launch of a moments kernel (pairs over the whole chunk)."""
    b, n, l, h, p, r = _shape(w, k)
    ch = b * n * h
    if kernel == "km_fwd_rows":    # G tiles (l^2 p) + Z = Q B (l^2 r) + U = B^T Z (l r^2)
        return (2 * l * l * p + 2 * l * l * r + 2 * l * r * r) * ch
    if kernel == "km_bwd_rows":    # G, Qb tiles + two pair products + four per-row products
        return (2 * l * l * p + 2 * l * l * r + 2 * l * l * p + 2 * l * l * r + 8 * l * p * r) * ch
    if kernel == "km_chunk":       # fwd: H^T V (2 p r^2); bwd: HS, (c2H+T)S (4 p r^2) + BS (2 l r^2)
        return None
    return None


def method_flops(w, k):
    """Algorithmic fwd + bwd flops of the method per step at chunk length k (causal
    triangle only)."""
    b, n, l, h, p, r = _shape(w, k)
    per_tok_fwd = (l + 1) * r + 4 * p * r + (l + 1) * p
    per_tok_bwd = 3 * (l + 1) * r + 12 * p * r + 2 * (l + 1) * p
    return (per_tok_fwd + per_tok_bwd) * b * n * l * h


def host_cpu() -> dict:
    """The host the oracle runs on: CPU model and the logical CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": n}


def _oracle_slice(inp, b: int, h: int):
    """fp64 numpy arrays of the (batch b, head h) slice of the workload's inputs."""
    sl = lambda k: inp[k][b:b + 1, :, :, h:h + 1].double().numpy()  # noqa: E731
    return dict(x=sl("x"), dy=sl("dy"), B=sl("B"), C=sl("C"),
                dt=inp["dt"][b:b + 1, h:h + 1].double().numpy(),
                A=inp["A"][h:h + 1].double().numpy(), D=inp["D"][h:h + 1].double().numpy(),
                init=inp["init"][b:b + 1, h:h + 1].double().numpy())


def _oracle_fwd_bwd(a):
    import oracle
    oracle.ssd_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"])
    oracle.ssd_bwd(a["dy"], None, a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"])


def cpu_baseline(w, inp, budget_s: float = 10.0):
    """The oracle (plain fp64 C, one (batch, head) slice per call) on the workload's own
    slices, scaled to whole-workload tokens/s (token-heads/s / heads):
      * single-threaded: slices in order until about `budget_s` of CPU time (the baseline);
      * all host cores: one thread per logical CPU (ctypes releases the GIL during the
        oracle's C calls), two slices per thread, wall time of the whole pool."""
    import concurrent.futures
    host = host_cpu()
    nslices = w.batch * w.nheads
    order = [(k // w.nheads, k % w.nheads) for k in range(nslices)]
    done, t_tot = 0, 0.0
    for b, h in order:
        a = _oracle_slice(inp, b, h)
        t0 = time.perf_counter()
        _oracle_fwd_bwd(a)
        t_tot += time.perf_counter() - t0
        done += 1
        if t_tot >= budget_s:
            break
    one = done * w.seq / t_tot / w.nheads
    res = {"value": round(one, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle", "host": host,
           "sample": f"fwd+bwd of {done} (batch, head) slice(s) x {w.seq} tokens of {w.name}, one "
                     f"thread, in {t_tot:.1f} s; tokens/s = token-heads/s / {w.nheads} heads"}
    threads = max(1, min(host["logical_cpus"] or 1, nslices))
    m = min(nslices, 2 * threads)
    sl = [_oracle_slice(inp, b, h) for b, h in order[:m]]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(_oracle_fwd_bwd, sl))
    el = time.perf_counter() - t0
    del sl
    res["all_cores"] = {
        "value": round(m * w.seq / el / w.nheads, 2), "unit": "tokens/s", "cores": threads,
        "kind": "oracle", "nproc": host["logical_cpus"],
        "sample": f"fwd+bwd of {m} (batch, head) slices x {w.seq} tokens of {w.name} on "
                  f"{threads} threads in {el:.1f} s wall; tokens/s = token-heads/s / {w.nheads} heads"}
    return res


WARMUP_DONE: dict = {}  # warm-up of the last timed_regions call: steps run, wall ms


def timed_regions(step, args, stream):
    """W warm-up steps (then more until --warmup-ms of GPU time has passed), then K steps
    timed with torch events on the launch stream,
    bracketed by device synchronisations -> ms per step (with --graph: K replays of the
    step captured once into a HIP graph; the library neither allocates nor
    synchronises, so capture needs nothing else); then K steps with the library's
    per-kernel HIP events -> (ms per step, {kernel: (total ms, launches)}).  The
    per-kernel events sit between launches, so they are kept out of the first region."""
    import torch
    from mamba_ssd_chunked_amd import ssd
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_warm = args.warmup
    # keep warming until the GPU has run at least --warmup-ms (whole batches of steps
    # between synchronisations, sized from the rate so far)
    min_ms = getattr(args, "warmup_ms", 0.0)
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        el = (time.perf_counter() - t0) * 1e3
        per = el / max(n_warm, 1)
        more = max(1, min(1000, int((min_ms - el) / max(per, 1e-3)) + 1))
        for _ in range(more):
            step()
        torch.cuda.synchronize()
        n_warm += more
    WARMUP_DONE.update(steps=n_warm, ms=round((time.perf_counter() - t0) * 1e3, 1))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def region(run):
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps

    run = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()  # one untimed replay
        run = graph.replay
    ms = region(run)
    ssd.ssd_timing_enable(True)
    ms_ev = region(step)
    ssd.ssd_timing_enable(False)
    return ms, ms_ev, ssd.ssd_timing_collect()


def pr_bytes(w, kernel: str):
    """Algorithmic HBM bytes of one launch of a PR kernel over all (b, h) slices (centred):
    fwd reads m2, m1 and writes pr, trace; bwd reads d_pr, m2, m1 and writes d_m2, d_m1."""
    bh, r = w.batch * w.nheads, w.dstate
    if kernel == "k_pr_fwd":
        return bh * (4 * (r * r + r) + 8)
    if kernel == "k_pr_bwd":
        return bh * (8 * (r * r + r) + 4)
    return None


def bench_pr(args, w, dims, m2, m1, count, stream):
    """ssd_moments_pr + ssd_moments_pr_bwd (centred) on the moments of the workload."""
    import torch
    from mamba_ssd_chunked_amd import ssd
    dev = m2.device
    bh = (w.batch, w.nheads, w.dstate)
    pr = torch.empty(w.batch, w.nheads, device=dev)
    tr = torch.empty_like(pr)
    dpr = torch.ones_like(pr)
    gm2, gm1 = torch.empty_like(m2), torch.empty_like(m1)

    def step():
        st = torch.cuda.current_stream()
        rc = ssd.ssd_moments_pr(*bh, m2, m1, count, 1, pr, tr, st)
        if rc:
            raise ssd.SsdError(rc, "ssd_moments_pr", ssd.ssd_last_error())
        rc = ssd.ssd_moments_pr_bwd(*bh, dpr, m2, m1, count, 1, gm2, gm1, st)
        if rc:
            raise ssd.SsdError(rc, "ssd_moments_pr_bwd", ssd.ssd_last_error())

    ms, _, kt = timed_regions(step, args, stream)
    kernels = {}
    for name, (tot, cnt) in kt.items():
        avg = tot / cnt
        ent = {"avg_us": round(avg * 1e3, 2), "launches_per_step": cnt / args.steps}
        nbytes = pr_bytes(w, name)
        if nbytes is not None:
            rate = nbytes / (avg / 1e3)
            ent.update(bytes=nbytes, gbps=round(rate / 1e9, 1), hbm_frac=round(rate / PEAK_HBM, 4))
        kernels[name] = ent
    return {"step": "ssd_moments_pr + ssd_moments_pr_bwd, centred, on the workload's m2 / m1",
            "us_per_step": round(ms * 1e3, 2), "kernels": kernels}


def diag_bytes(w, kernel: str):
    """Algorithmic HBM bytes of one launch of the same-step correction over all (token, head)
    pairs: fwd reads v, B, C, gamma and writes y; bwd reads dy, v, B, C, gamma and writes
    d_v, d_B, d_C, d_gamma."""
    e = 2 if w.io == "bf16" else 4
    m, p, r = w.mimo_rank, w.headdim, w.dstate
    pairs = w.tokens * w.nheads
    if kernel == "k_diag_fwd":
        return pairs * (e * (2 * m * p + 2 * m * r) + 4)
    if kernel == "k_diag_bwd":
        return pairs * (e * (3 * m * p + 4 * m * r) + 8)
    return None


def bench_diag(args):
    """ssd_y_diag + ssd_y_diag_bwd on each same-step-correction workload."""
    import torch
    from mamba_ssd_chunked_amd import inputs, ssd
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    res = {}
    for name, w in inputs.DIAG_WORKLOADS.items():
        d = {k: v.to(dev) for k, v in inputs.make_diag_inputs(w).items()}
        y = torch.empty_like(d["v"])
        g = dict(d_v=torch.empty_like(d["v"]), d_B=torch.empty_like(d["B"]),
                 d_C=torch.empty_like(d["C"]), d_gamma=torch.empty_like(d["gamma"]))

        def step():
            st = torch.cuda.current_stream()
            rc = ssd.ssd_y_diag(d["v"], d["B"], d["C"], d["gamma"], y, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_y_diag", ssd.ssd_last_error())
            rc = ssd.ssd_y_diag_bwd(d["dy"], d["v"], d["B"], d["C"], d["gamma"], g["d_v"], g["d_B"],
                                    g["d_C"], g["d_gamma"], st)
            if rc:
                raise ssd.SsdError(rc, "ssd_y_diag_bwd", ssd.ssd_last_error())

        ms, _, kt = timed_regions(step, args, stream)
        kernels = {}
        for kname, (tot, cnt) in kt.items():
            avg = tot / cnt
            nbytes = diag_bytes(w, kname)
            rate = nbytes / (avg / 1e3)
            kernels[kname] = {"avg_us": round(avg * 1e3, 2), "bytes": nbytes,
                              "gbps": round(rate / 1e9, 1), "hbm_frac": round(rate / PEAK_HBM, 4)}
        res[name] = {"workload": w.describe(), "ms_per_step": round(ms, 4),
                     "value": round(w.tokens / (ms / 1e3), 1), "unit": "tokens/s",
                     "step": "ssd_y_diag + ssd_y_diag_bwd", "kernels": kernels}
        del d, y, g
    return res


def quat_bytes(w, kernel: str):
    """HBM bytes one launch of a quaternion-scan kernel must move (16 B per quaternion):
    fwd reads q and writes cum (plus init); the carry pass reads q; the reverse pass reads q
    and d_cum and writes d_q (plus init, d_init).  The carry pass's read of q is a re-read of
    the backward's input: the backward's algorithmic bytes are those of the reverse pass."""
    n = w.batch * w.seq * w.nheads * w.nquat
    lanes = w.batch * w.nheads * w.nquat
    if kernel == "k_quat_fwd":
        return 32 * n + 16 * lanes
    if kernel == "k_quat_carry":
        return 16 * n + 16 * lanes
    if kernel == "k_quat_bwd":
        return 48 * n + 32 * lanes
    return None


def bench_quat(args):
    """ssd_quat_scan + ssd_quat_scan_bwd on the quaternion-scan workload."""
    import torch
    from mamba_ssd_chunked_amd import inputs, ssd
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    res = {}
    for name, w in inputs.QUAT_WORKLOADS.items():
        i = inputs.make_quat_inputs(w)
        q, dc = i["q"].to(dev), i["d_cum"].to(dev)
        init = i["init"].to(dev) if i["init"] is not None else None
        cum, d_q = torch.empty_like(q), torch.empty_like(q)
        d_init = torch.empty((w.batch, w.nheads, w.nquat, 4), device=dev)
        ws_f, ws_b = ssd.quat_workspace(q, False), ssd.quat_workspace(q, True)

        def step():
            st = torch.cuda.current_stream()
            rc = ssd.ssd_quat_scan(q, init, cum, ws_f, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_quat_scan", ssd.ssd_last_error())
            rc = ssd.ssd_quat_scan_bwd(q, init, dc, d_q, d_init, ws_b, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_quat_scan_bwd", ssd.ssd_last_error())

        ms, _, kt = timed_regions(step, args, stream)
        kernels = {}
        for kname, (tot, cnt) in kt.items():
            avg = tot / cnt
            ent = {"avg_us": round(avg * 1e3, 2), "launches_per_step": cnt / args.steps}
            nbytes = quat_bytes(w, kname)
            if nbytes is not None:
                rate = nbytes / (avg / 1e3)
                ent.update(bytes=nbytes, gbps=round(rate / 1e9, 1), hbm_frac=round(rate / PEAK_HBM, 4))
            kernels[kname] = ent
        algo = quat_bytes(w, "k_quat_fwd") + quat_bytes(w, "k_quat_bwd")
        tokens = w.batch * w.seq
        res[name] = {"workload": w.describe(), "ms_per_step": round(ms, 4),
                     "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s",
                     "step": "ssd_quat_scan + ssd_quat_scan_bwd",
                     "step_algorithmic_gbps": round(algo / (ms / 1e3) / 1e9, 1),
                     "kernels": kernels}
        del q, dc, init, cum, d_q, d_init, ws_f, ws_b
    return res


def step_bytes(w):
    """Algorithmic HBM bytes of one decode step over the batch: the state read and written
    (4 B each per element), x, B, C read and y written (io dtype), dt read (fp32)."""
    e = 2 if w.io == "bf16" else 4
    bh = w.batch * w.nheads
    return bh * (8 * w.headdim * w.dstate + e * (2 * w.headdim + 2 * w.dstate) + 4)


def bench_step(args):
    """ssd_step (in place) on each decode workload: tokens/s = sequences per step."""
    import torch
    from mamba_ssd_chunked_amd import inputs, ssd
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    res = {}
    for name, w in inputs.STEP_WORKLOADS.items():
        d = {k: v.to(dev) for k, v in inputs.make_step_inputs(w).items()}
        y = torch.empty_like(d["x"])

        def step():
            st = torch.cuda.current_stream()
            rc = ssd.ssd_step(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["state"],
                              d["state"], y, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_step", ssd.ssd_last_error())

        ms, _, kt = timed_regions(step, args, stream)
        kernels = {}
        nbytes = step_bytes(w)
        for kname, (tot, cnt) in kt.items():
            avg = tot / cnt
            rate = nbytes / (avg / 1e3)
            kernels[kname] = {"avg_us": round(avg * 1e3, 2), "bytes": nbytes,
                              "gbps": round(rate / 1e9, 1), "hbm_frac": round(rate / PEAK_HBM, 4)}
        res[name] = {"workload": w.describe(), "us_per_step": round(ms * 1e3, 2),
                     "value": round(w.batch / (ms / 1e3), 1), "unit": "tokens/s",
                     "step": "ssd_step (in place)", "kernels": kernels}
        del d, y
    return res


def bench_ssd(w, inp, args, layout=True, steps=None, warmup=None):
    """ssd_fwd + ssd_bwd on workload w (inputs already drawn): step time, per-kernel rates and the
    roofline of the dominant kernel; with `layout`, also the step at the layout's chunk length."""
    import argparse as _ap
    import torch
    from mamba_ssd_chunked_amd import ssd
    dev = torch.device("cuda", 0)
    targs = _ap.Namespace(steps=steps or args.steps, warmup=warmup or args.warmup, graph=args.graph,
                          warmup_ms=args.warmup_ms)
    d = {k: v.to(dev) for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "valid_len"}
    init = d["init"] if w.init_std > 0 else None
    y = torch.empty_like(d["x"])
    final = torch.empty_like(d["d_final"])
    gx, gB, gC = torch.empty_like(d["x"]), torch.empty_like(d["B"]), torch.empty_like(d["C"])
    gdt, gA, gD = torch.empty_like(d["dt"]), torch.empty_like(d["A"]), torch.empty_like(d["D"])
    ginit = torch.empty_like(d["d_final"])
    stream = torch.cuda.current_stream()

    def make_step(kcl):
        dims = ssd.dims_of(d["x"], d["B"], kcl)
        ws_f = ssd.workspace(dims, ssd.SSD_OP_FWD, dev)
        ws_b = ssd.workspace(dims, ssd.SSD_OP_BWD, dev)

        def step():
            st = torch.cuda.current_stream()
            rc = ssd.ssd_fwd(dims, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], init, y,
                             final, ws_f, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_fwd", ssd.ssd_last_error())
            rc = ssd.ssd_bwd(dims, d["dy"], None, d["x"], d["dt"], d["A"], d["B"], d["C"],
                             d["D"], init, gx, gdt, gA, gB, gC, gD, ginit, ws_b, st)
            if rc:
                raise ssd.SsdError(rc, "ssd_bwd", ssd.ssd_last_error())
        return step

    k = kernel_chunk_len(w, args.kernel_chunk_len)
    ms, ms_ev, kt = timed_regions(make_step(args.kernel_chunk_len), targs, stream)
    tokens = w.batch * w.seq

    warm = dict(WARMUP_DONE)
    kernels = {}
    for name, (tot, cnt) in kt.items():
        avg = tot / cnt
        work, kind = kernel_work(w, name, k)
        ent = {"avg_ms": round(avg, 5), "launches_per_step": cnt / targs.steps}
        jobs = 1.5 if name == "k_chunk_states" else 1.0
        if name == "k_chunk_states":
            # launched once in ssd_fwd (1 job) and once in ssd_bwd (2 jobs): average work
            work = work * jobs
        if work is not None:
            if kind == "flop":
                # matrix roof: fp32 flops at the fp32 peak + bf16 flops at the bf16 peak;
                # HBM roof: each input read once, each output written once
                roof_s = mfma_roof_s(w, name, k, jobs)
                nbytes = chunk_kernel_bytes(w, name, k)
                ent.update(tflops=round(work / (avg / 1e3) / 1e12, 2),
                           mfma_frac=round(roof_s / (avg / 1e3), 4))
                if nbytes:
                    hbm_s = nbytes / PEAK_HBM
                    ent.update(gbps=round(nbytes / (avg / 1e3) / 1e9, 1),
                               hbm_frac=round(hbm_s / (avg / 1e3), 4),
                               bound="mfma" if roof_s >= hbm_s else "hbm")
                if w.io == "bf16":
                    f32, both, split = matrix_flops(w, name, k)
                    ent.update(fp32_mfma_gflop=round(jobs * f32 / 1e9, 2),
                               bf16_mfma_gflop=round(jobs * both / 1e9, 2),
                               split_bf16_mfma_gflop=round(jobs * split / 1e9, 2))
            else:
                rate = work / (avg / 1e3)
                ent.update(gbps=round(rate / 1e9, 1), hbm_frac=round(rate / PEAK_HBM, 4), bound="hbm")
        kernels[name] = ent
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_step"])
    work, kind = kernel_work(w, dom, k)
    davg = kernels[dom]["avg_ms"]
    if kind == "flop" and kernels[dom].get("bound", "mfma") == "mfma":
        roof_s = mfma_roof_s(w, dom, k)
        ach = work / (davg / 1e3) / 1e12
        peak = work / roof_s / 1e12   # the fp32 peak; with bf16 io the flop mix's peak
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom, w, k)}
    else:
        nbytes = work if kind == "byte" else chunk_kernel_bytes(w, dom, k)
        ach = nbytes / (davg / 1e3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": 8000.0,
                "unit": "GB/s", "frac": round(ach / 8000.0, 4),
                "traffic": measured_traffic(dom, w, k)}
    res = {"value": round(tokens / (ms / 1e3), 1), "ms_per_step": round(ms, 4),
           "ms_per_step_with_kernel_events": round(ms_ev, 4), "kernel_chunk_len": k,
           "warmup_steps_run": warm.get("steps"), "warmup_ms_run": warm.get("ms"),
           "roofline": roof, "method_tflops": round(method_flops(w, k) / (ms / 1e3) / 1e12, 3),
           "kernels": kernels}
    if layout and k != w.chunk_len:
        # the same step with the kernels run at the layout's chunk length
        ms_l, _, _ = timed_regions(make_step(w.chunk_len), targs, stream)
        res["at_layout_chunk_len"] = {"kernel_chunk_len": w.chunk_len, "ms_per_step": round(ms_l, 4),
                                      "value": round(tokens / (ms_l / 1e3), 1)}
    del d, y, final, gx, gB, gC, gdt, gA, gD, ginit
    return res


def bench_other_workloads(args):
    """The SSD step on the other full-size SSD workloads (the Mamba-2-130M- and 2.7B-shaped
    ones, or the 64k-token one when another workload is the headline), same step counts."""
    from mamba_ssd_chunked_amd import inputs
    res = {}
    for name in ("mamba2_130m_fp32", "mamba2_2p7b_bf16", "long_context_64k_fp32"):
        if name == args.workload:
            continue
        w = inputs.WORKLOADS[name]
        r = bench_ssd(w, inputs.make_inputs(w), args, layout=False)
        res[name] = {"workload": w.describe(), "kernel_chunk_len": r["kernel_chunk_len"],
                     "steps": args.steps, "warmup_steps_run": r["warmup_steps_run"],
                     "warmup_ms_run": r["warmup_ms_run"],
                     "ms_per_step": r["ms_per_step"], "value": r["value"], "unit": "tokens/s",
                     "roofline": r["roofline"], "method_tflops": r["method_tflops"],
                     "kernels": r["kernels"]}
    return res


def bench_moments(args):
    """ssd_state_moments (with y) + ssd_state_moments_bwd on the moments workload."""
    import torch
    from mamba_ssd_chunked_amd import inputs, ssd
    w = inputs.WORKLOADS["moments_valid_len_fp32"]
    inp = inputs.make_inputs(w)
    dev = torch.device("cuda", 0)
    d = {k: v.to(dev) for k, v in inp.items() if isinstance(v, torch.Tensor) and k != "valid_len"}
    valid = inp["valid_len"].clone()
    k = kernel_chunk_len(w)
    dims = ssd.dims_of(d["x"], d["B"])
    m2 = torch.empty_like(d["d_m2"])
    m1 = torch.empty_like(d["d_m1"])
    count = torch.empty(w.batch, dtype=torch.int64)
    y = torch.empty_like(d["x"])
    gx, gB = torch.empty_like(d["x"]), torch.empty_like(d["B"])
    gdt, gA = torch.empty_like(d["dt"]), torch.empty_like(d["A"])
    ginit = torch.empty_like(d["d_final"])
    ws_f = ssd.workspace(dims, ssd.SSD_OP_MOMENTS, dev)
    ws_b = ssd.workspace(dims, ssd.SSD_OP_MOMENTS_BWD, dev)
    stream = torch.cuda.current_stream()

    def step():
        st = torch.cuda.current_stream()
        rc = ssd.ssd_state_moments(dims, d["x"], d["dt"], d["A"], d["B"], None, valid, m2, m1, count,
                                   y, d["C"], d["D"], None, ws_f, st)
        if rc:
            raise ssd.SsdError(rc, "ssd_state_moments", ssd.ssd_last_error())
        rc = ssd.ssd_state_moments_bwd(dims, d["d_m2"], d["d_m1"], d["x"], d["dt"], d["A"], d["B"],
                                       None, valid, gx, gdt, gA, gB, ginit, ws_b, st)
        if rc:
            raise ssd.SsdError(rc, "ssd_state_moments_bwd", ssd.ssd_last_error())

    ms, ms_ev, kt = timed_regions(step, args, stream)
    kernels = {}
    for name, (tot, cnt) in kt.items():
        avg = tot / cnt
        ent = {"avg_ms": round(avg, 5), "launches_per_step": cnt / args.steps}
        work = moments_kernel_work(w, name, k)
        if work is None and name in ("k_chunk_states", "k5_chunk_scan", "k1_cumsum", "k4_state_pass",
                                     "k4_state_pass_bwd"):
            work, kind = kernel_work(w, name, k)
            if kind == "byte":
                ent.update(gbps=round(work / (avg / 1e3) / 1e9, 1))
                work = None
        if work is not None:
            rate = work / (avg / 1e3)
            ent.update(tflops=round(rate / 1e12, 2), mfma_frac=round(rate / PEAK_FP32_MFMA, 4))
        kernels[name] = ent
    res = {"workload": {**w.describe(), "kernel_chunk_len": k}, "ms_per_step": round(ms, 4),
           "ms_per_step_with_kernel_events": round(ms_ev, 4),
           "value": round(w.batch * w.seq / (ms / 1e3), 1), "unit": "tokens/s",
           "valid_tokens_per_s": round(sum(min(v, w.seq) for v in w.valid_len) / (ms / 1e3), 1),
           "step": "ssd_state_moments (with y) + ssd_state_moments_bwd", "kernels": kernels}
    res["pr"] = bench_pr(args, w, dims, m2, m1, count, stream)

    # The PR-penalty loop: moments (with y) -> PR -> dPR/d(m2, m1) -> moments backward.
    prv = torch.empty(w.batch, w.nheads, device=dev)
    dpr = torch.ones_like(prv)
    gm2, gm1 = torch.empty_like(m2), torch.empty_like(m1)
    bh = (w.batch, w.nheads, w.dstate)

    def loop_step():
        st = torch.cuda.current_stream()
        for rc, what in (
                (ssd.ssd_state_moments(dims, d["x"], d["dt"], d["A"], d["B"], None, valid, m2, m1,
                                       count, y, d["C"], d["D"], None, ws_f, st), "ssd_state_moments"),
                (ssd.ssd_moments_pr(*bh, m2, m1, count, 1, prv, None, st), "ssd_moments_pr"),
                (ssd.ssd_moments_pr_bwd(*bh, dpr, m2, m1, count, 1, gm2, gm1, st), "ssd_moments_pr_bwd"),
                (ssd.ssd_state_moments_bwd(dims, gm2, gm1, d["x"], d["dt"], d["A"], d["B"], None, valid,
                                           gx, gdt, gA, gB, ginit, ws_b, st), "ssd_state_moments_bwd")):
            if rc:
                raise ssd.SsdError(rc, what, ssd.ssd_last_error())

    ms_loop, _, _ = timed_regions(loop_step, args, stream)
    res["pr_penalty_loop"] = {
        "step": "ssd_state_moments (with y) + ssd_moments_pr + ssd_moments_pr_bwd (centred) + "
                "ssd_state_moments_bwd fed the PR gradient",
        "ms_per_step": round(ms_loop, 4), "value": round(w.batch * w.seq / (ms_loop / 1e3), 1),
        "unit": "tokens/s"}
    if not args.no_cpu_baseline:
        import oracle
        hs = [0]
        t0 = time.perf_counter()
        sl = {k: inp[k][:, :, :, hs].double().numpy() for k in ("x", "B")}
        dt = inp["dt"][:, hs].double().numpy()
        A = inp["A"][hs].double().numpy()
        oracle.state_moments(sl["x"], dt, A, sl["B"], None, list(w.valid_len))
        oracle.state_moments_bwd(inp["d_m2"][:, hs].double().numpy(), inp["d_m1"][:, hs].double().numpy(),
                                 sl["x"], dt, A, sl["B"], None, list(w.valid_len))
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(w.batch * w.seq / w.nheads / el, 2), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle", "host": host_cpu(),
                               "sample": f"moments fwd+bwd of head 0, all {w.batch} batches x {w.seq} "
                                         f"tokens in {el:.1f} s; tokens/s = token-heads/s / {w.nheads} heads"}
    return res


def copy_probe(mib: int) -> int:
    """Copy a device buffer of `mib` MiB three times (a plain copy kernel of known size, to
    calibrate HBM byte counters); returns the bytes copied per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return 4 * n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps first")
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="after the --warmup steps, keep running untimed steps until this much "
                         "GPU time has passed (the clocks take tens of ms to settle)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-moments", action="store_true",
                    help="skip the state-moments leg (moments_valid_len_fp32 workload)")
    ap.add_argument("--kernel-chunk-len", type=int, default=0,
                    help="chunk length the kernels run at (0: the library's automatic choice)")
    ap.add_argument("--no-layout-chunk", action="store_true",
                    help="skip the second timing with the kernels at the layout's chunk length")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured into a HIP graph (on this ROCm about "
                         "1 %% slower than eager launches)")
    ap.add_argument("--moments-only", action="store_true",
                    help="run only the state-moments leg and print its JSON object")
    ap.add_argument("--no-diag", action="store_true",
                    help="skip the same-step-correction leg (Mamba-3 y_diag workloads)")
    ap.add_argument("--diag-only", action="store_true",
                    help="run only the same-step-correction leg and print its JSON object")
    ap.add_argument("--no-quat", action="store_true",
                    help="skip the quaternion-scan leg (Mamba-3 rotation workload)")
    ap.add_argument("--quat-only", action="store_true",
                    help="run only the quaternion-scan leg and print its JSON object")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the SSD step on the other full-size SSD workloads")
    ap.add_argument("--no-step", action="store_true",
                    help="skip the decode-step leg")
    ap.add_argument("--step-only", action="store_true",
                    help="run only the decode-step leg and print its JSON object")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="skip the streaming probe (the HBM rate of a plain kernel per read:write "
                         "mix, against which each kernel's byte rate is also reported)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 3 times (a plain copy "
                         "kernel of known size, to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the sequence/head sharding across GPUs is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_ssd_chunked_amd import inputs, ssd

    if args.moments_only:
        torch.cuda.set_device(0)
        res = bench_moments(args)
        if args.copy_probe_mib > 0:
            res["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
        print(json.dumps(res), flush=True)
        return
    if args.diag_only:
        torch.cuda.set_device(0)
        print(json.dumps(bench_diag(args)), flush=True)
        return
    if args.step_only:
        torch.cuda.set_device(0)
        res = bench_step(args)
        if args.copy_probe_mib > 0:
            res["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
        print(json.dumps(res), flush=True)
        return
    if args.quat_only:
        torch.cuda.set_device(0)
        res = bench_quat(args)
        if args.copy_probe_mib > 0:
            res["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
        print(json.dumps(res), flush=True)
        return

    w = inputs.WORKLOADS[args.workload]
    inp = inputs.make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    r = bench_ssd(w, inp, args, layout=not args.no_layout_chunk)
    out = {
        "metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_min_ms": args.warmup_ms,
        "warmup_steps_run": r["warmup_steps_run"], "warmup_ms_run": r["warmup_ms_run"],
        "ms_per_step": r["ms_per_step"],
        "ms_per_step_with_kernel_events": r["ms_per_step_with_kernel_events"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.io == "f32" else "f32+bf16", "io_dtype": w.io,
        "data": "synthetic (seeded draws of the workload recipe; no dataset)",
        "config": {**w.describe(), "kernel_chunk_len": r["kernel_chunk_len"]},
        "roofline": r["roofline"],
        "method_tflops": r["method_tflops"],
        "kernels": r["kernels"],
    }
    if "at_layout_chunk_len" in r:
        out["at_layout_chunk_len"] = r["at_layout_chunk_len"]
    roofs = None
    if not args.no_stream_probe:
        roofs = stream_roofs()
        out["hbm_stream_roofs"] = {"unit": "GB/s", "probe": "ssd_stream_probe, 256 MiB arrays, best "
                                   "of cached and non-temporal", **{m: round(v / 1e9, 1) for m, v in roofs.items()}}
        annotate_stream(out["kernels"], w, r["kernel_chunk_len"], roofs)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    if not args.no_moments:
        out["moments"] = bench_moments(args)
    if not args.no_diag:
        out["y_diag"] = bench_diag(args)
    if not args.no_quat:
        out["quat_scan"] = bench_quat(args)
    if not args.no_step:
        out["decode_step"] = bench_step(args)
    if not args.no_other_workloads:
        out["other_workloads"] = bench_other_workloads(args)
        if roofs:
            for name, res in out["other_workloads"].items():
                annotate_stream(res["kernels"], inputs.WORKLOADS[name], res["kernel_chunk_len"], roofs)
    if args.copy_probe_mib > 0:
        out["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
