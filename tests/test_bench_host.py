"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic work
model behind the roofline, and the source-hash gate on the measured HBM traffic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mamba_ssd_chunked_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_chunk_len_rule():
    w = inputs.WORKLOADS["mamba2_130m_fp32"]
    assert bench.kernel_chunk_len(w) == 128
    assert bench.kernel_chunk_len(w, 256) == 256
    assert bench.kernel_chunk_len(inputs.WORKLOADS["tiny_fp32"]) == 64


def test_work_model_counts_the_causal_products():
    """k5 at k = 128 on c1: 1536 chunk-heads x (2 k p r + 2 pairs (r + p)), by hand."""
    w = inputs.WORKLOADS["mamba2_130m_fp32"]
    pairs = 128 * 129 // 2
    ch = 4 * (2048 // 128) * 24
    assert bench.kernel_work(w, "k5_chunk_scan", 128) == ((2 * 128 * 64 * 128 + 2 * pairs * 192) * ch,
                                                          "flop")
    # the same step at k = 256 has half the chunk-heads and (k + 1) / 2 pairs per token
    f128 = bench.kernel_work(w, "k_bwd_source", 128)[0]
    f256 = bench.kernel_work(w, "k_bwd_source", 256)[0]
    assert f256 > f128
    assert bench.kernel_work(w, "k4_state_pass", 128)[1] == "byte"
    # the method total is per token-head, independent of how the kernels split it
    assert bench.method_flops(w, 128) < bench.method_flops(w, 256)


def test_traffic_is_reported_only_for_the_profiled_sources(monkeypatch):
    w = inputs.WORKLOADS["mamba2_130m_fp32"]
    key = ("k_bwd_source", w.name, 128)
    rd, wr, h = bench.TRAFFIC[key]
    monkeypatch.setitem(bench.TRAFFIC, key, (rd, wr, "0" * 16))
    assert bench.measured_traffic("k_bwd_source", w, 128) is None
    assert bench.measured_traffic("k_bwd_source", w, 256) is None  # never profiled at 256
    assert bench.measured_traffic("k5_chunk_scan", w, 128) is None


def test_diag_bytes_count_every_tensor_once():
    w = inputs.DIAG_WORKLOADS["mamba3_diag_mimo4_fp32"]
    pairs = 4 * 2048 * 24
    # fwd: v, B, C, y (4 B each) + gamma; bwd: dy, v, B, C, d_v, d_B, d_C + gamma, d_gamma
    assert bench.diag_bytes(w, "k_diag_fwd") == pairs * (4 * (4 * 64 + 2 * 4 * 128 + 4 * 64) + 4)
    assert bench.diag_bytes(w, "k_diag_bwd") == pairs * (4 * (3 * 4 * 64 + 4 * 4 * 128) + 8)
    assert bench.diag_bytes(w, "other") is None


def test_quat_bytes_count_every_tensor_once():
    w = inputs.QUAT_WORKLOADS["mamba3_quat_scan_fp32"]
    n, lanes = 4 * 2048 * 24 * 32, 4 * 24 * 32
    # fwd: q in, cum out (16 B per quaternion each) + init; reverse pass: q, d_cum, d_q + init, d_init
    assert bench.quat_bytes(w, "k_quat_fwd") == 32 * n + 16 * lanes
    assert bench.quat_bytes(w, "k_quat_bwd") == 48 * n + 32 * lanes
    assert bench.quat_bytes(w, "k_quat_carry") == 16 * n + 16 * lanes
    assert bench.quat_bytes(w, "k_quat_clear") is None


def test_step_bytes_count_every_tensor_once():
    w = inputs.STEP_WORKLOADS["mamba2_2p7b_decode_bf16"]
    bh = 64 * 80
    # state read + written in fp32; x, y (p each) and B, C (r each) in bf16; dt fp32
    assert bench.step_bytes(w) == bh * (8 * 64 * 128 + 2 * (2 * 64 + 2 * 128) + 4)


def test_chunk_kernel_bytes_count_every_tensor_once():
    """The matrix kernels' HBM bytes on the 130M-shaped workload at k = 128 (1536 chunk-heads,
    196608 token-heads): each token row, dt, cumsum and chunk state once."""
    w = inputs.WORKLOADS["mamba2_130m_fp32"]
    tok, st = 196608, 4 * 64 * 128 * 1536
    assert bench.chunk_kernel_bytes(w, "k5_chunk_scan", 128) == tok * (4 * (64 + 2 * 128) + 4 * 64 + 12) + st
    tiles = 1024 * 36 * 1536  # 36 causal 16 x 16 d_CB tiles per 128-token chunk-head
    # per token-head besides the rows: source dt, cdt (fp64) in; d_dt, g2, d_delta, diagonal
    # d_CB out; target cdt, g2, d_delta, diagonal d_CB in, d_dt in and out
    assert bench.chunk_kernel_bytes(w, "k_bwd_source", 128) == tok * (4 * (2 * 64 + 2 * 128) + 4 * (64 + 128) + 12 + 16) + st + tiles
    assert bench.chunk_kernel_bytes(w, "k_bwd_target", 128) == tok * (4 * (64 + 3 * 128) + 8 + 12 + 8) + 2 * st + tiles
    job0 = tok * (4 * 192 + 12) + st
    job1 = tok * (4 * 192 + 8) + st
    assert bench.chunk_kernel_bytes(w, "k_chunk_states", 128) == (2 * job0 + job1) / 2
    assert bench.chunk_kernel_bytes(w, "k4_state_pass", 128) is None
    # bf16 io halves the token rows only
    wb = inputs.Workload("b", 4, 2048, 24, 64, 128, 256, io="bf16")
    assert bench.chunk_kernel_bytes(wb, "k5_chunk_scan", 128) == tok * (2 * (2 * 64 + 2 * 128) + 12) + st


def test_matrix_flops_split_by_matrix_core_type():
    """bf16 io: C B^T and dy x^T run on bf16 MFMAs, every product with an fp32 operand on
    the bf16 ones split in three (nothing on fp32 ones); fp32 io: everything on fp32 ones.
    The total is the same either way."""
    pairs = 128 * 129 // 2
    wb = inputs.WORKLOADS["mamba2_2p7b_bf16"]
    ch = 2 * (4096 // 128) * 80
    f32, both, split = bench.matrix_flops(wb, "k_bwd_source", 128)
    assert f32 == 0
    assert both == (2 * pairs * 128 + 2 * pairs * 64) * ch      # C B^T, dy x^T
    # K3 (d_intra's parts), W^T dy, d_CB^T C
    assert split == (4 * 128 * 64 * 128 + 2 * pairs * 64 + 2 * pairs * 128) * ch
    assert f32 + both + split == bench.kernel_work(wb, "k_bwd_source", 128)[0]
    k5 = bench.matrix_flops(wb, "k5_chunk_scan", 128)
    assert k5[0] == 0 and k5[1] == 2 * pairs * 128 * ch            # C B^T
    assert k5[2] == (2 * 128 * 64 * 128 + 2 * pairs * 64) * ch     # BLUE (S_in's parts), W x
    assert bench.mfma_roof_s(wb, "k_bwd_source", 128) == pytest.approx(
        f32 / 157.3e12 + (both + 3 * split) / 2.5e15)
    # the state kernel's products run split on the bf16 cores: each costs three bf16 products
    f32, both, split = bench.matrix_flops(wb, "k_chunk_states", 128)
    assert f32 == 0 and both == 0 and split == 2 * 128 * 64 * 128 * ch
    assert bench.mfma_roof_s(wb, "k_chunk_states", 128) == pytest.approx(3 * split / 2.5e15)
    wf = inputs.WORKLOADS["long_context_64k_fp32"]
    f32, both, split = bench.matrix_flops(wf, "k_bwd_target", 128)
    assert both == 0 and split == 0 and f32 == bench.kernel_work(wf, "k_bwd_target", 128)[0]
    # the target-row kernel takes d_CB from the source-row kernel: BLUE and d_CB B only
    assert f32 == (2 * 128 * 64 * 128 + 2 * pairs * 128) * (65536 // 128) * 32
    assert bench.matrix_flops(wf, "k4_state_pass", 128) is None


def test_cpu_baseline_has_a_single_thread_and_an_all_cores_leg():
    w = inputs.WORKLOADS["tiny_fp32"]
    res = bench.cpu_baseline(w, inputs.make_inputs(w), budget_s=0.01)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["value"] > 0
    allc = res["all_cores"]
    assert allc["kind"] == "oracle" and allc["value"] > 0
    assert 1 <= allc["cores"] <= w.batch * w.nheads
    assert allc["nproc"] == bench.host_cpu()["logical_cpus"]


def test_headline_is_the_largest_single_gpu_workload():
    big = max(("mamba2_130m_fp32", "mamba2_2p7b_bf16", "long_context_64k_fp32"),
              key=lambda n: bench.method_flops(inputs.WORKLOADS[n], 128))
    assert bench.HEADLINE == big == "long_context_64k_fp32"


def test_traffic_hash_ignores_comments_not_code():
    """The counters stay valid across comment edits and lapse on any change of code."""
    a = 'int f(int x) { return x + 1; }  // one\n/* two */ const char* s = "// kept";\n'
    b = '/* other */ int f(int x)\n{ return x + 1; }\nconst char* s = "// kept";  // three\n'
    assert bench.code_of(a) == bench.code_of(b)
    assert bench.code_of(a) != bench.code_of(a.replace("x + 1", "x + 2"))
    assert bench.code_of(a) != bench.code_of(a.replace('"// kept"', '"// gone"'))
    assert bench.code_of("char c = '\\'';  // q\nint y;") == "char c = '\\''; int y;"
    for key in bench.TRAFFIC_SOURCES:
        assert len(bench.traffic_hash(*key)) == 16


@pytest.mark.parametrize("name", ["mamba2_130m_fp32", "mamba2_2p7b_bf16", "long_context_64k_fp32"])
def test_read_write_split_adds_up_to_the_byte_counts(name):
    """kernel_rw splits each kernel's algorithmic bytes into reads and writes without changing
    the total that the byte rates use."""
    w = inputs.WORKLOADS[name]
    for k in (64, 128, 256):
        for kern in ("k_chunk_states", "k5_chunk_scan", "k_bwd_target", "k_bwd_source"):
            rd, wr = bench.kernel_rw(w, kern, k)
            assert rd > 0 and wr > 0
            assert rd + wr == pytest.approx(bench.chunk_kernel_bytes(w, kern, k), rel=1e-12), (kern, k)
        for kern in ("k1_cumsum", "k4_state_pass", "k4_state_pass_bwd"):
            rd, wr = bench.kernel_rw(w, kern, k)
            total, kind = bench.kernel_work(w, kern, k)
            assert kind == "byte" and rd + wr == total, (kern, k)
    assert bench.kernel_rw(w, "reduce_heads", 128) is None


def test_stream_annotation_takes_the_nearest_mix():
    """A kernel's byte rate is set against the probe's rate for the mix nearest its read share."""
    w = inputs.WORKLOADS["long_context_64k_fp32"]
    roofs = {f"{r}:{wr}": 5e12 + 1e11 * i for i, (r, wr) in enumerate(bench.STREAM_MIXES)}
    kernels = {"k4_state_pass": {"gbps": 6000.0}, "k_chunk_states": {"gbps": 5600.0},
               "reduce_heads": {"avg_ms": 0.01}}
    bench.annotate_stream(kernels, w, 128, roofs)
    assert kernels["k4_state_pass"]["stream_mix"] == "1:1"
    assert kernels["k4_state_pass"]["stream_frac"] == pytest.approx(6e12 / roofs["1:1"], rel=1e-3)
    rd, wr = bench.kernel_rw(w, "k_chunk_states", 128)
    assert 0.7 < rd / (rd + wr) < 0.8 and kernels["k_chunk_states"]["stream_mix"] == "3:1"
    assert "stream_frac" not in kernels["reduce_heads"]
