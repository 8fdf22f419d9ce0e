// C ABI of the SSD scan: argument validation, workspace plan and the launch
// sequence of each entry point (declared and documented in include/ssd.h).
//
// Every entry point validates all of its arguments before it enqueues anything,
// then enqueues its kernels on the caller's stream and returns without
// synchronising.  The workspace is caller-owned; the library allocates nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <utility>
#include <vector>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return SSD_OK;
}

bool pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

int validate_dims(const ssd_dims* d, ssd::Shape* s) {
    if (!d) return fail(SSD_ERR_NULL, "dims is NULL");
    if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "io_dtype must be SSD_F32 (0) or SSD_BF16 (1) (got %d)", d->io_dtype);
    if (d->batch < 0 || d->nchunks < 0 || d->chunk_len <= 0 || d->nheads <= 0 || d->headdim <= 0 ||
        d->dstate <= 0)
        return fail(SSD_ERR_SHAPE,
                    "need batch >= 0, nchunks >= 0 and chunk_len, nheads, headdim, dstate > 0 "
                    "(got b=%lld n=%lld l=%lld h=%lld p=%lld r=%lld)",
                    (long long)d->batch, (long long)d->nchunks, (long long)d->chunk_len,
                    (long long)d->nheads, (long long)d->headdim, (long long)d->dstate);
    if (!pow2_in(d->chunk_len, 64, 256))
        return fail(SSD_ERR_UNSUPPORTED, "chunk_len must be 64, 128 or 256 (got %lld)", (long long)d->chunk_len);
    if (!pow2_in(d->headdim, 16, 128) || !pow2_in(d->dstate, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "headdim and dstate must be 16, 32, 64 or 128 (got %lld, %lld)",
                    (long long)d->headdim, (long long)d->dstate);
    // index arithmetic and grid limits.  The largest grids: the per-64-token-block kernels
    // (256 work-items per block, 4 per token-head), the state copies (one per state
    // element, p r or r r per (b, h)) and the carry passes (a quarter or half of that).
    const double bh = (double)d->batch * (double)d->nheads;
    const double per_bh = std::max({4.0 * (double)d->nchunks * (double)d->chunk_len,
                                    (double)d->headdim * d->dstate, (double)d->dstate * d->dstate});
    const double elems = (double)d->batch * d->nchunks * d->chunk_len * d->nheads * 128.0;
    if (bh * per_bh > ssd::kMaxGridItems || elems > 4.0e18 || d->nchunks > (1 << 30) ||
        d->nheads > (1 << 30) || d->batch > (1 << 30))
        return fail(SSD_ERR_UNSUPPORTED,
                    "problem too large for one call: a launch would exceed 2^32 work-items "
                    "(split the batch or the heads)");
    // The kernels run the chunked algorithm at chunk length k (a divisor of chunk_len):
    // the caller's [b, n, l, ...] buffers are the same memory as [b, n l / k, k, ...].
    const int64_t k = d->kernel_chunk_len == 0 ? (d->chunk_len < 128 ? d->chunk_len : 128)
                                               : d->kernel_chunk_len;
    if (!pow2_in(k, 64, 256) || k > d->chunk_len || d->chunk_len % k != 0)
        return fail(SSD_ERR_UNSUPPORTED,
                    "kernel_chunk_len must be 0 or one of 64, 128, 256 dividing chunk_len "
                    "(got %d for chunk_len %lld)", d->kernel_chunk_len, (long long)d->chunk_len);
    if (d->nchunks * (d->chunk_len / k) > (1 << 30))
        return fail(SSD_ERR_UNSUPPORTED, "problem too large for one call (split the batch)");
    s->B = (int)d->batch;
    s->N = (int)(d->nchunks * (d->chunk_len / k));
    s->L = (int)k;
    s->H = (int)d->nheads;
    s->P = (int)d->headdim;
    s->R = (int)d->dstate;
    s->io = d->io_dtype;
    return SSD_OK;
}

int check_align(const void* p, const char* name, size_t a) {
    if (p && (reinterpret_cast<uintptr_t>(p) % a) != 0)
        return fail(SSD_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", name, a);
    return SSD_OK;
}

size_t round_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace plan (256-byte aligned regions):
//   cdt    fp64 [b,h,n,l]  cumsum of dt inside each chunk (K1)
//   S      fp32 [b,n,h,p,r] chunk states (K3, then chunk-entry states after K4)
//   bwd:   dS fp32 [b,n,h,p,r] (BLUE state gradient, then the carried d_intra),
//          g1, g2, dlt fp32 [b,h,n,l], dend fp32 [b,h,n],
//          dAT, dAS, dD fp64 [b,n,h,l/64] (per-block d_A / d_D partials),
//          dcbt fp32 [b,n,h,pairs,256]: the d_CB tiles of the causal 16 x 16 pair tiles
//          (pairs = pair_tiles_of(l); the diagonal elements t = s held out as zeros),
//          ddg fp32 [b,h,n,l]: those diagonal elements d_CB[t, t]
//   moments: valid int64 [b]; phi, psi, phit, psit fp64 [b,h,n,l]; T fp32 [b,n,h,p,r];
//          fwd: U [b,n,h,l/64,r,r], W [b,n,h,r,r], m1b [b,n,h,l/64,r], m1c [b,n,h,r] fp32
//          bwd: HS, dS fp32 [b,n,h,p,r]; BS fp32 [b,n,h,l,r]; fin fp32 [b,h,p,r];
//               hsh, hdm fp64 [b,n,h]; dend2 fp64 [b,h,n]; ddtW, rho, eta, zeta fp32
//               [b,h,n,l]; dA fp64 [b,n,h,l/64]
struct Ws {
    size_t cdt = 0, S = 0, dS = 0, g1 = 0, g2 = 0, dlt = 0, dend = 0, dAT = 0, dAS = 0, dD = 0,
           dcbt = 0, ddg = 0;
    size_t valid = 0, phi = 0, psi = 0, phit = 0, psit = 0, T = 0, U = 0, W = 0, m1b = 0, m1c = 0, HS = 0, BS = 0,
           fin = 0, hsh = 0, hdm = 0, dend2 = 0, ddtW = 0, rho = 0, eta = 0, zeta = 0, dA = 0;
    size_t total = 0;
};

Ws plan(const ssd::Shape& s, int op) {
    Ws w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    const size_t tok = static_cast<size_t>(s.B) * s.H * s.N * s.L;  // (b, h, token)
    const size_t chunks = static_cast<size_t>(s.B) * s.H * s.N;
    const size_t states = chunks * s.P * s.R;
    const size_t nb = static_cast<size_t>(s.nblk());
    w.cdt = take(8 * tok);
    w.S = take(4 * states);
    if (op == SSD_OP_BWD) {
        w.dS = take(4 * states);
        w.g1 = take(4 * tok);
        w.g2 = take(4 * tok);
        w.dlt = take(4 * tok);
        w.dend = take(4 * chunks);
        w.dAT = take(8 * chunks * nb);
        w.dAS = take(8 * chunks * nb);
        w.dD = take(8 * chunks * nb);
        const size_t tiles = chunks * static_cast<size_t>(ssd::pair_tiles_of(s.L));
        w.dcbt = take(4 * 256 * tiles);
        w.ddg = take(4 * tok);
    }
    if (op == SSD_OP_MOMENTS || op == SSD_OP_MOMENTS_BWD) {
        w.valid = take(8 * static_cast<size_t>(s.B));
        w.phi = take(8 * tok);
        w.psi = take(8 * tok);
        w.phit = take(8 * tok);
        w.psit = take(8 * tok);
        w.T = take(4 * states);
    }
    if (op == SSD_OP_MOMENTS) {
        const size_t rr = static_cast<size_t>(s.R) * s.R;
        w.U = take(4 * chunks * nb * rr);
        w.W = take(4 * chunks * rr);
        w.m1b = take(4 * chunks * nb * s.R);
        w.m1c = take(4 * chunks * s.R);
    }
    if (op == SSD_OP_MOMENTS_BWD) {
        w.HS = take(4 * states);
        w.dS = take(4 * states);
        w.BS = take(4 * tok * s.R);
        w.fin = take(4 * static_cast<size_t>(s.B) * s.H * s.P * s.R);
        w.hsh = take(8 * chunks);
        w.hdm = take(8 * chunks);
        w.dend2 = take(8 * chunks);
        w.ddtW = take(4 * tok);
        w.rho = take(4 * tok);
        w.eta = take(4 * tok);
        w.zeta = take(4 * tok);
        w.dA = take(8 * chunks * nb);
    }
    w.total = off;
    return w;
}

template <class T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------- timing
// Optional per-kernel timing: when enabled, every launch below is bracketed by
// a pair of HIP events recorded on the caller's stream; ssd_timing_collect()
// waits for them and sums the elapsed times per kernel name.
struct TimingRec {
    const char* name;
    hipEvent_t a, b;
};
std::mutex g_tm;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    // timing-only events: no system-scope fence (cache write-back) at each record
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
    bool on;
    {
        std::lock_guard<std::mutex> lk(g_tm);
        on = g_timing;
    }
    if (!on) return launch();
    hipEvent_t a, b;
    {
        std::lock_guard<std::mutex> lk(g_tm);
        a = pool_event();
        b = pool_event();
    }
    if (!a || !b) return launch();
    hipEventRecord(a, st);
    const hipError_t e = launch();
    hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_tm);
    g_recs.push_back({name, a, b});
    return e;
}

#define SSD_HIP(call, what)                                                         \
    do {                                                                            \
        hipError_t e_ = timed(what, st, [&]() { return (call); });                  \
        if (e_ != hipSuccess)                                                       \
            return fail(SSD_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e_)); \
    } while (0)

// Debug mode (ssd_debug_enable): after an entry point's work, scan its outputs for NaN or
// infinity (a stream synchronisation).
std::atomic<bool> g_debug{false};

struct Checked {
    const void* p;
    int64_t n;
    bool bf16;
    const char* name;
};

// The flag words are one device array per GPU shared by every caller, so a check holds
// this lock from clearing them until its results are back on the host: overlapping
// checks (other threads, other streams) wait instead of clearing each other's flags.
std::mutex g_check_mu;

int check_outputs(hipStream_t st, const char* where, std::initializer_list<Checked> outs) {
    std::lock_guard<std::mutex> lk(g_check_mu);
    int* flags = nullptr;
    hipError_t e = ssd::nonfinite_flags(&flags);
    const char* names[16];
    int n = 0;
    if (e == hipSuccess) e = ssd::launch_clear_flags(flags, 16, st);
    for (const Checked& o : outs) {
        if (e != hipSuccess || n == 16) break;
        if (!o.p || o.n <= 0) continue;
        e = ssd::launch_nonfinite(o.p, o.n, o.bf16, flags + n, st);
        names[n++] = o.name;
    }
    int host[16] = {0};
    if (e == hipSuccess && n > 0) e = hipMemcpyAsync(host, flags, sizeof(int) * n, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return fail(SSD_ERR_HIP, "%s: output check failed: %s", where, hipGetErrorString(e));
    for (int k = 0; k < n; ++k)
        if (host[k]) return fail(SSD_ERR_NONFINITE, "%s: %s holds a NaN or an infinity", where, names[k]);
    return SSD_OK;
}

int check_ws(const ssd::Shape& s, int op, void* ws, size_t ws_bytes) {
    const size_t need = plan(s, op).total;
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(SSD_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                    ws ? "" : ", NULL pointer");
    if (need > 0 && (reinterpret_cast<uintptr_t>(ws) % 256) != 0)
        return fail(SSD_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
    return SSD_OK;
}

int check_io_ptrs(const ssd::Shape& s, std::initializer_list<std::pair<const void*, const char*>> io,
                  std::initializer_list<std::pair<const void*, const char*>> f32) {
    const size_t ia = s.io == SSD_BF16 ? 8 : 16;
    for (auto& p : io)
        if (int rc = check_align(p.first, p.second, ia)) return rc;
    for (auto& p : f32)
        if (int rc = check_align(p.first, p.second, 16)) return rc;
    return SSD_OK;
}

// Shared checks of the two PR entry points (sizes, counts, pointers, alignment).
int validate_pr(const char* who, int64_t batch, int64_t nheads, int64_t dstate, const float* m2,
                const float* m1, const int64_t* count, int center, const void* out,
                const void* out16) {
    if (batch < 0 || nheads <= 0)
        return fail(SSD_ERR_SHAPE, "%s: need 0 <= batch and 0 < nheads (got %lld, %lld)", who,
                    (long long)batch, (long long)nheads);
    // one workgroup of at most 256 work-items per (b, h)
    if (batch > (1 << 30) || nheads > (1 << 30) ||
        (double)batch * nheads * 256.0 > ssd::kMaxGridItems)
        return fail(SSD_ERR_UNSUPPORTED, "%s: problem too large for one call: a launch would exceed "
                    "2^32 work-items (split the batch)", who);
    if (!pow2_in(dstate, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "%s: dstate must be 16, 32, 64 or 128 (got %lld)", who,
                    (long long)dstate);
    if (batch == 0) return SSD_OK;
    if (!m2 || !count || !out || (center && !m1))
        return fail(SSD_ERR_NULL, "%s: m2, count, the outputs%s are required", who,
                    center ? " and m1 (center)" : "");
    for (int64_t b = 0; b < batch; ++b)
        if (count[b] <= 0)
            return fail(SSD_ERR_SHAPE, "%s: count[%lld] = %lld holds no samples", who, (long long)b,
                        (long long)count[b]);
    if (int rc = check_align(m2, "m2", 16)) return rc;
    if (int rc = check_align(out16, "d_m2", 16)) return rc;
    return SSD_OK;
}

// Shared checks of the two y_diag entry points; fills *d.
int validate_diag(const char* who, int64_t ntokens, int64_t mimo_rank, int64_t nheads,
                  int64_t headdim, int64_t dstate, int io_dtype, ssd::DiagShape* d) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "%s: io_dtype must be SSD_F32 (0) or SSD_BF16 (1) (got %d)", who,
                    io_dtype);
    if (ntokens < 0 || mimo_rank <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0)
        return fail(SSD_ERR_SHAPE,
                    "%s: need ntokens >= 0 and mimo_rank, nheads, headdim, dstate > 0 "
                    "(got %lld, %lld, %lld, %lld, %lld)", who, (long long)ntokens,
                    (long long)mimo_rank, (long long)nheads, (long long)headdim, (long long)dstate);
    if (mimo_rank != 1 && mimo_rank != 2 && mimo_rank != 4)
        return fail(SSD_ERR_UNSUPPORTED, "%s: mimo_rank must be 1, 2 or 4 (got %lld)", who,
                    (long long)mimo_rank);
    if (!pow2_in(headdim, 16, 128) || !pow2_in(dstate, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "%s: headdim and dstate must be 16, 32, 64 or 128 "
                    "(got %lld, %lld)", who, (long long)headdim, (long long)dstate);
    // the backward launches 16 work-items per (token, head)
    if (nheads > (1 << 30) || (double)ntokens * (double)nheads * 16.0 > ssd::kMaxGridItems ||
        (double)ntokens * mimo_rank * nheads * 128.0 > 4.0e18)
        return fail(SSD_ERR_UNSUPPORTED, "%s: problem too large for one call: a launch would "
                    "exceed 2^32 work-items (split the tokens)", who);
    d->T = ntokens;
    d->M = (int)mimo_rank;
    d->H = (int)nheads;
    d->P = (int)headdim;
    d->R = (int)dstate;
    d->io = io_dtype;
    return SSD_OK;
}

int check_diag_ptrs(const ssd::DiagShape& d,
                    std::initializer_list<std::pair<const void*, const char*>> io) {
    const size_t ia = d.io == SSD_BF16 ? 8 : 16;
    for (auto& p : io)
        if (int rc = check_align(p.first, p.second, ia)) return rc;
    return SSD_OK;
}

// Shared checks of the quaternion-scan entry points; fills *s.
int validate_quat(const char* who, int64_t batch, int64_t seq, int64_t nheads, int64_t nquat,
                  bool bwd, ssd::QuatShape* s) {
    if (batch < 0 || seq < 0 || nheads <= 0 || nquat <= 0)
        return fail(SSD_ERR_SHAPE,
                    "%s: need batch >= 0, seq >= 0 and nheads, nquat > 0 (got %lld, %lld, %lld, %lld)",
                    who, (long long)batch, (long long)seq, (long long)nheads, (long long)nquat);
    const double lanes = (double)nheads * (double)nquat;
    if (lanes > (double)(1 << 24) || batch > (1 << 30) || seq > (int64_t(1) << 40) ||
        (double)batch * seq * lanes * 4.0 > 4.0e18)
        return fail(SSD_ERR_UNSUPPORTED, "%s: problem too large for one call", who);
    *s = ssd::quat_shape(batch, seq, nheads, nquat, bwd);
    // one workgroup of 256 work-items per (b, 64-lane group, segment)
    if ((double)s->B * s->G * s->nseg * 256.0 > ssd::kMaxGridItems)
        return fail(SSD_ERR_UNSUPPORTED, "%s: problem too large for one call: a launch would "
                    "exceed 2^32 work-items (split the batch)", who);
    return SSD_OK;
}

int check_valid_len(const ssd::Shape& s, const int64_t* valid_len) {
    if (!valid_len) return SSD_OK;
    const int64_t seq = static_cast<int64_t>(s.N) * s.L;
    for (int b = 0; b < s.B; ++b)
        if (valid_len[b] < 0 || valid_len[b] > seq)
            return fail(SSD_ERR_SHAPE, "valid_len[%d] = %lld is outside [0, %lld]", b,
                        (long long)valid_len[b], (long long)seq);
    return SSD_OK;
}

// The forward of ssd_fwd and ssd_fwd_noalloc.  With `fixed_scratch` the workspace is
// the library's fixed device array (ws / ws_bytes are ignored): problems that need
// more are rejected before anything is enqueued, and nothing is allocated.
int fwd_impl(const char* who, const ssd_dims* dims, const void* x, const float* dt, const float* A,
             const void* B, const void* C, const float* D, const float* init, void* y,
             float* final_state, void* ws, size_t ws_bytes, bool fixed_scratch, void* stream) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    const bool tok = s.B > 0 && s.N > 0;  // token tensors are non-empty
    if (!A || !D || (tok && (!x || !dt || !B || !C || !y)))
        return fail(SSD_ERR_NULL, "%s: x, dt, A, B, C, D and y are required", who);
    if (int rc = check_io_ptrs(s, {{x, "x"}, {B, "B"}, {C, "C"}, {y, "y"}},
                               {{dt, "dt"}, {init, "init"}, {final_state, "final_state"}}))
        return rc;
    if (fixed_scratch) {
        const size_t need = plan(s, SSD_OP_FWD).total;
        if (need > SSD_NOALLOC_SCRATCH_BYTES)
            return fail(SSD_ERR_WORKSPACE,
                        "%s: the problem needs %zu bytes of scratch, more than the %u bytes the "
                        "library holds per GPU (call ssd_fwd with a workspace of %zu bytes)",
                        who, need, SSD_NOALLOC_SCRATCH_BYTES, need);
        if (need > 0) {
            const hipError_t e = ssd::noalloc_scratch(&ws);
            if (e != hipSuccess)
                return fail(SSD_ERR_HIP, "%s: scratch lookup failed: %s", who, hipGetErrorString(e));
            ws_bytes = SSD_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (int rc = check_ws(s, SSD_OP_FWD, ws, ws_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t nstate = static_cast<int64_t>(s.B) * s.H * s.P * s.R;
    if (s.B == 0 || s.N == 0) {
        if (final_state) SSD_HIP(ssd::launch_copy_or_zero(final_state, init, nstate, st), "copy init");
        return ok();
    }
    const Ws w = plan(s, SSD_OP_FWD);
    double* cdt = at<double>(ws, w.cdt);
    float* S = at<float>(ws, w.S);
    SSD_HIP(ssd::launch_k1_cumsum(s, dt, cdt, st), "k1_cumsum");
    SSD_HIP(ssd::launch_chunk_states(s, true, false, x, B, nullptr, nullptr, dt, A, cdt, S, nullptr, st),
            "k_chunk_states");
    SSD_HIP(ssd::launch_k4_pass(s, S, cdt, A, init, final_state, st), "k4_state_pass");
    SSD_HIP(ssd::launch_k5_scan(s, x, dt, B, C, A, D, cdt, S, y, st), "k5_chunk_scan");
    if (g_debug) {
        const bool bf = s.io == SSD_BF16;
        const int64_t tp = static_cast<int64_t>(s.B) * s.N * s.L * s.H * s.P;
        if (int rc = check_outputs(st, who, {{y, tp, bf, "y"}, {final_state, nstate, false, "final_state"}}))
            return rc;
    }
    return ok();
}

}  // namespace

extern "C" {

const char* ssd_last_error(void) { return g_err; }

int ssd_debug_enable(int on) {
    g_debug = on != 0;
    return ok();
}

int ssd_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_tm);
    g_timing = on != 0;
    return ok();
}

int ssd_timing_collect(int max_kernels, char* names, size_t name_stride, double* total_ms,
                       int64_t* launches, int* n_kernels) {
    if (!n_kernels || (max_kernels > 0 && (!names || !total_ms || !launches)) || name_stride < 2)
        return fail(SSD_ERR_NULL, "ssd_timing_collect: output arrays are required");
    std::vector<TimingRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_tm);
        recs.swap(g_recs);
    }
    std::vector<const char*> seen;
    std::vector<double> ms;
    std::vector<int64_t> cnt;
    int rc = SSD_OK;
    for (const TimingRec& r : recs) {
        float el = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&el, r.a, r.b) != hipSuccess)
            rc = fail(SSD_ERR_HIP, "ssd_timing_collect: event query failed");
        size_t k = 0;
        while (k < seen.size() && std::strcmp(seen[k], r.name) != 0) ++k;
        if (k == seen.size()) {
            seen.push_back(r.name);
            ms.push_back(0.0);
            cnt.push_back(0);
        }
        ms[k] += el;
        cnt[k] += 1;
    }
    {
        std::lock_guard<std::mutex> lk(g_tm);
        for (const TimingRec& r : recs) {
            g_pool.push_back(r.a);
            g_pool.push_back(r.b);
        }
    }
    const int n = static_cast<int>(seen.size());
    *n_kernels = n;
    for (int k = 0; k < n && k < max_kernels; ++k) {
        std::snprintf(names + static_cast<size_t>(k) * name_stride, name_stride, "%s", seen[k]);
        total_ms[k] = ms[k];
        launches[k] = cnt[k];
    }
    return rc == SSD_OK ? ok() : rc;
}

int ssd_stream_probe(int reads, int writes, int nontemporal, const void* src, void* dst,
                     int64_t n16, void* stream) {
    static const int kMixes[][2] = {{1, 0}, {6, 1}, {4, 1}, {3, 1}, {2, 1}, {1, 1}, {0, 1}};
    bool known = false;
    for (const auto& m : kMixes) known = known || (m[0] == reads && m[1] == writes);
    if (!known) return fail(SSD_ERR_UNSUPPORTED, "ssd_stream_probe: no (%d reads, %d writes) mix", reads, writes);
    if (n16 < 0) return fail(SSD_ERR_SHAPE, "ssd_stream_probe: n16 = %lld", static_cast<long long>(n16));
    if ((reads > 0 && !src) || !dst) return fail(SSD_ERR_NULL, "ssd_stream_probe: a buffer is NULL");
    if (hipError_t e = ssd::launch_stream_probe(reads, writes, nontemporal != 0, src, dst, n16,
                                                static_cast<hipStream_t>(stream)))
        return fail(SSD_ERR_HIP, "ssd_stream_probe: %s", hipGetErrorString(e));
    return ok();
}

int ssd_workspace_size(const ssd_dims* dims, int op, size_t* bytes) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    if (!bytes) return fail(SSD_ERR_NULL, "bytes is NULL");
    if (op < SSD_OP_FWD || op > SSD_OP_MOMENTS_BWD)
        return fail(SSD_ERR_SHAPE, "unknown op %d", op);
    *bytes = plan(s, op).total;
    return ok();
}

int ssd_bwd_partial_region(const ssd_dims* dims, const char* name, size_t* offset, size_t* bytes) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    if (!name || !offset || !bytes)
        return fail(SSD_ERR_NULL, "ssd_bwd_partial_region: name, offset and bytes are required");
    const Ws w = plan(s, SSD_OP_BWD);
    const size_t tok = static_cast<size_t>(s.B) * s.H * s.N * s.L;
    if (std::strcmp(name, "g1") == 0) {
        *offset = w.g1;
        *bytes = ssd::wide_supported(s) ? 0 : 4 * tok;  // the whole-chunk kernel keeps it in registers
    } else if (std::strcmp(name, "g2") == 0) {
        *offset = w.g2;
        *bytes = 4 * tok;
    } else if (std::strcmp(name, "d_delta") == 0) {
        *offset = w.dlt;
        *bytes = 4 * tok;
    } else {
        return fail(SSD_ERR_SHAPE, "ssd_bwd_partial_region: unknown region '%s' (g1, g2, d_delta)",
                    name);
    }
    return ok();
}

int ssd_fwd(const ssd_dims* dims, const void* x, const float* dt, const float* A, const void* B,
            const void* C, const float* D, const float* init, void* y, float* final_state, void* ws,
            size_t ws_bytes, void* stream) {
    return fwd_impl("ssd_fwd", dims, x, dt, A, B, C, D, init, y, final_state, ws, ws_bytes, false,
                    stream);
}

int ssd_fwd_noalloc(const ssd_dims* dims, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* init, void* y,
                    float* final_state, void* stream) {
    return fwd_impl("ssd_fwd_noalloc", dims, x, dt, A, B, C, D, init, y, final_state, nullptr, 0,
                    true, stream);
}

int ssd_bwd(const ssd_dims* dims, const void* dy, const float* d_final, const void* x,
            const float* dt, const float* A, const void* B, const void* C, const float* D,
            const float* init, void* d_x, float* d_dt, float* d_A, void* d_B, void* d_C,
            float* d_D, float* d_init, void* ws, size_t ws_bytes, void* stream) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    const bool tok = s.B > 0 && s.N > 0;
    if (!A || !D || !d_A || !d_D ||
        (tok && (!dy || !x || !dt || !B || !C || !d_x || !d_dt || !d_B || !d_C)))
        return fail(SSD_ERR_NULL,
                    "ssd_bwd: dy, x, dt, A, B, C, D, d_x, d_dt, d_A, d_B, d_C and d_D are required");
    if (int rc = check_io_ptrs(s, {{dy, "dy"}, {x, "x"}, {B, "B"}, {C, "C"}, {d_x, "d_x"}, {d_B, "d_B"}, {d_C, "d_C"}},
                               {{dt, "dt"}, {d_dt, "d_dt"}, {init, "init"}, {d_final, "d_final"}, {d_init, "d_init"}}))
        return rc;
    if (int rc = check_ws(s, SSD_OP_BWD, ws, ws_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t nstate = static_cast<int64_t>(s.B) * s.H * s.P * s.R;
    if (s.B == 0 || s.N == 0) {
        SSD_HIP(ssd::launch_copy_or_zero(d_A, nullptr, s.H, st), "zero d_A");
        SSD_HIP(ssd::launch_copy_or_zero(d_D, nullptr, s.H, st), "zero d_D");
        if (d_init) SSD_HIP(ssd::launch_copy_or_zero(d_init, d_final, nstate, st), "copy d_final");
        return ok();
    }
    const Ws w = plan(s, SSD_OP_BWD);
    double* cdt = at<double>(ws, w.cdt);
    float* S = at<float>(ws, w.S);
    float* dS = at<float>(ws, w.dS);
    float* g1 = at<float>(ws, w.g1);
    float* g2 = at<float>(ws, w.g2);
    float* dlt = at<float>(ws, w.dlt);
    float* dend = at<float>(ws, w.dend);
    double* dAT = at<double>(ws, w.dAT);
    double* dAS = at<double>(ws, w.dAS);
    double* dDp = at<double>(ws, w.dD);
    SSD_HIP(ssd::launch_k1_cumsum(s, dt, cdt, st), "k1_cumsum");
    SSD_HIP(ssd::launch_chunk_states(s, true, true, x, B, dy, C, dt, A, cdt, S, dS, st), "k_chunk_states");
    SSD_HIP(ssd::launch_k4_pass_bwd(s, S, dS, cdt, A, init, d_final, d_init, st), "k4_state_pass_bwd");
    float* dcbt = at<float>(ws, w.dcbt);
    float* ddg = at<float>(ws, w.ddg);
    // rows s first: they hand every causal pair tile's d_CB to rows t.  The whole-chunk
    // source kernel (one workgroup per CU) pays off where the kernel is bound by its vector
    // work (bf16 io); with fp32 io the two 64-row block workgroups per CU overlap one
    // another's loads and are faster.
    const bool wide = ssd::wide_supported(s);
    if (wide && s.io == SSD_BF16)
        SSD_HIP(ssd::launch_bwd_source_wide(s, dy, x, dt, B, C, A, D, cdt, dS, d_x, d_B, d_dt, g2,
                                            dlt, dAS, dDp, dcbt, ddg, st),
                "k_bwd_source");
    else
        SSD_HIP(ssd::launch_bwd_source(s, dy, x, dt, B, C, A, D, cdt, dS, d_x, d_B, d_dt, g2, dlt,
                                       dAS, dDp, dcbt, ddg, st),
                "k_bwd_source");
    if (wide) {
        // whole chunks: K1's backward runs inside the target-row kernel
        SSD_HIP(ssd::launch_bwd_target_wide(s, dy, B, C, A, cdt, S, dS, dcbt, ddg, g2, dlt, d_C,
                                            d_dt, dAT, st),
                "k_bwd_target");
        SSD_HIP(ssd::launch_reduce_heads(s, dAT, dAS, dDp, s.nblk(), d_A, d_D, st), "reduce_heads");
    } else {
        SSD_HIP(ssd::launch_bwd_target(s, dy, B, C, A, cdt, S, dS, dcbt, ddg, d_C, g1, dend, dAT, st),
                "k_bwd_target");
        SSD_HIP(ssd::launch_k1t_heads(s, g1, g2, dlt, dend, A, d_dt, dAT, dAS, dDp, s.nblk(), d_A,
                                      d_D, st),
                "k1t_revcumsum");
    }
    if (g_debug) {
        const bool bf = s.io == SSD_BF16;
        const int64_t tk = static_cast<int64_t>(s.B) * s.N * s.L * s.H;
        if (int rc = check_outputs(st, "ssd_bwd",
                                   {{d_x, tk * s.P, bf, "d_x"}, {d_dt, tk, false, "d_dt"}, {d_A, s.H, false, "d_A"},
                                    {d_B, tk * s.R, bf, "d_B"}, {d_C, tk * s.R, bf, "d_C"}, {d_D, s.H, false, "d_D"},
                                    {d_init, nstate, false, "d_init"}}))
            return rc;
    }
    return ok();
}

int ssd_state_moments(const ssd_dims* dims, const void* x, const float* dt, const float* A,
                      const void* B, const float* init, const int64_t* valid_len, float* m2,
                      float* m1, int64_t* count, void* y, const void* C, const float* D,
                      float* final_state, void* ws, size_t ws_bytes, void* stream) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    const bool tok = s.B > 0 && s.N > 0;
    if (!A || (s.B > 0 && (!m2 || !m1 || !count)) || (tok && (!x || !dt || !B)))
        return fail(SSD_ERR_NULL, "ssd_state_moments: x, dt, A, B, m2, m1 and count are required");
    if (y && (!C || !D)) return fail(SSD_ERR_NULL, "ssd_state_moments: y needs C and D");
    if (int rc = check_io_ptrs(s, {{x, "x"}, {B, "B"}, {C, "C"}, {y, "y"}},
                               {{dt, "dt"}, {init, "init"}, {m2, "m2"}, {m1, "m1"},
                                {final_state, "final_state"}}))
        return rc;
    if (int rc = check_valid_len(s, valid_len)) return rc;
    if (int rc = check_ws(s, SSD_OP_MOMENTS, ws, ws_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t seq = static_cast<int64_t>(s.N) * s.L;
    for (int b = 0; b < s.B; ++b) count[b] = (valid_len ? valid_len[b] : seq) * s.P;
    const int64_t nstate = static_cast<int64_t>(s.B) * s.H * s.P * s.R;
    if (!tok) {
        SSD_HIP(ssd::launch_copy_or_zero(m2, nullptr, static_cast<int64_t>(s.B) * s.H * s.R * s.R, st), "zero m2");
        SSD_HIP(ssd::launch_copy_or_zero(m1, nullptr, static_cast<int64_t>(s.B) * s.H * s.R, st), "zero m1");
        if (final_state) SSD_HIP(ssd::launch_copy_or_zero(final_state, init, nstate, st), "copy init");
        return ok();
    }
    const Ws w = plan(s, SSD_OP_MOMENTS);
    double* cdt = at<double>(ws, w.cdt);
    float* S = at<float>(ws, w.S);
    int64_t* vd = at<int64_t>(ws, w.valid);
    double* phi = at<double>(ws, w.phi);
    double* psi = at<double>(ws, w.psi);
    float* T = at<float>(ws, w.T);
    SSD_HIP(ssd::launch_set_i64(vd, valid_len, seq, s.B, st), "set_i64");
    SSD_HIP(ssd::launch_k1_cumsum(s, dt, cdt, st), "k1_cumsum");
    SSD_HIP(ssd::launch_chunk_states(s, true, false, x, B, nullptr, nullptr, dt, A, cdt, S, nullptr, st),
            "k_chunk_states");
    SSD_HIP(ssd::launch_k4_pass(s, S, cdt, A, init, final_state, st), "k4_state_pass");
    SSD_HIP(ssd::launch_km_phi(s, cdt, A, vd, phi, psi, at<double>(ws, w.phit), at<double>(ws, w.psit), st),
            "km_phi");
    SSD_HIP(ssd::launch_chunk_states(s, false, false, x, B, nullptr, nullptr, dt, A, cdt, nullptr,
                                     nullptr, st, phi, T),
            "k_chunk_states");
    SSD_HIP(ssd::launch_km_fwd_rows(s, x, B, dt, A, cdt, phi, psi, at<float>(ws, w.U),
                                    at<float>(ws, w.m1b), st),
            "km_fwd_rows");
    SSD_HIP(ssd::launch_km_chunk(s, S, T, cdt, A, phi, psi, at<float>(ws, w.W), at<float>(ws, w.m1c),
                                 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, st),
            "km_chunk");
    SSD_HIP(ssd::launch_km_reduce(s, at<float>(ws, w.U), at<float>(ws, w.W), at<float>(ws, w.m1b),
                                  at<float>(ws, w.m1c), m2, m1, st),
            "km_reduce");
    if (y) SSD_HIP(ssd::launch_k5_scan(s, x, dt, B, C, A, D, cdt, S, y, st), "k5_chunk_scan");
    if (g_debug) {
        const int64_t bh = static_cast<int64_t>(s.B) * s.H;
        const int64_t tp = static_cast<int64_t>(s.B) * s.N * s.L * s.H * s.P;
        if (int rc = check_outputs(st, "ssd_state_moments",
                                   {{m2, bh * s.R * s.R, false, "m2"}, {m1, bh * s.R, false, "m1"},
                                    {y, tp, s.io == SSD_BF16, "y"}, {final_state, nstate, false, "final_state"}}))
            return rc;
    }
    return ok();
}

int ssd_state_moments_bwd(const ssd_dims* dims, const float* d_m2, const float* d_m1,
                          const void* x, const float* dt, const float* A, const void* B,
                          const float* init, const int64_t* valid_len, void* d_x, float* d_dt,
                          float* d_A, void* d_B, float* d_init, void* ws, size_t ws_bytes,
                          void* stream) {
    ssd::Shape s;
    if (int rc = validate_dims(dims, &s)) return rc;
    const bool tok = s.B > 0 && s.N > 0;
    if (!A || !d_A || (s.B > 0 && !d_m2) || (tok && (!x || !dt || !B || !d_x || !d_dt || !d_B)))
        return fail(SSD_ERR_NULL,
                    "ssd_state_moments_bwd: d_m2, x, dt, A, B, d_x, d_dt, d_A and d_B are required");
    if (int rc = check_io_ptrs(s, {{x, "x"}, {B, "B"}, {d_x, "d_x"}, {d_B, "d_B"}},
                               {{dt, "dt"}, {d_dt, "d_dt"}, {init, "init"}, {d_m2, "d_m2"},
                                {d_m1, "d_m1"}, {d_init, "d_init"}}))
        return rc;
    if (int rc = check_valid_len(s, valid_len)) return rc;
    if (int rc = check_ws(s, SSD_OP_MOMENTS_BWD, ws, ws_bytes)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t seq = static_cast<int64_t>(s.N) * s.L;
    const int64_t nstate = static_cast<int64_t>(s.B) * s.H * s.P * s.R;
    if (!tok) {
        SSD_HIP(ssd::launch_copy_or_zero(d_A, nullptr, s.H, st), "zero d_A");
        if (d_init) SSD_HIP(ssd::launch_copy_or_zero(d_init, nullptr, nstate, st), "zero d_init");
        return ok();
    }
    const Ws w = plan(s, SSD_OP_MOMENTS_BWD);
    double* cdt = at<double>(ws, w.cdt);
    float* S = at<float>(ws, w.S);
    int64_t* vd = at<int64_t>(ws, w.valid);
    double* phi = at<double>(ws, w.phi);
    double* psi = at<double>(ws, w.psi);
    float* T = at<float>(ws, w.T);
    float* HS = at<float>(ws, w.HS);
    float* dS = at<float>(ws, w.dS);
    float* BS = at<float>(ws, w.BS);
    float* fin = at<float>(ws, w.fin);
    double* hsh = at<double>(ws, w.hsh);
    double* hdm = at<double>(ws, w.hdm);
    double* dend2 = at<double>(ws, w.dend2);
    float* ddtW = at<float>(ws, w.ddtW);
    float* rho = at<float>(ws, w.rho);
    float* eta = at<float>(ws, w.eta);
    float* zeta = at<float>(ws, w.zeta);
    double* dA = at<double>(ws, w.dA);
    SSD_HIP(ssd::launch_set_i64(vd, valid_len, seq, s.B, st), "set_i64");
    SSD_HIP(ssd::launch_k1_cumsum(s, dt, cdt, st), "k1_cumsum");
    SSD_HIP(ssd::launch_chunk_states(s, true, false, x, B, nullptr, nullptr, dt, A, cdt, S, nullptr, st),
            "k_chunk_states");
    SSD_HIP(ssd::launch_k4_pass(s, S, cdt, A, init, fin, st), "k4_state_pass");
    SSD_HIP(ssd::launch_km_phi(s, cdt, A, vd, phi, psi, at<double>(ws, w.phit), at<double>(ws, w.psit), st),
            "km_phi");
    SSD_HIP(ssd::launch_chunk_states(s, false, false, x, B, nullptr, nullptr, dt, A, cdt, nullptr,
                                     nullptr, st, phi, T),
            "k_chunk_states");
    SSD_HIP(ssd::launch_km_chunk(s, S, T, cdt, A, phi, psi, nullptr, nullptr, d_m2, d_m1, B, HS, dS,
                                 BS, hsh, hdm, st),
            "km_chunk");
    SSD_HIP(ssd::launch_k4_pass_bwd(s, S, dS, cdt, A, init, nullptr, d_init, st, false),
            "k4_state_pass_bwd");
    SSD_HIP(ssd::launch_km_bwd_rows(s, x, B, dt, A, cdt, phi, psi, at<double>(ws, w.phit),
                                    at<double>(ws, w.psit), HS, BS, dS, S, fin, d_m1, hsh, hdm, d_x,
                                    d_B, ddtW, rho, eta, zeta, dend2, dA, st),
            "km_bwd_rows");
    SSD_HIP(ssd::launch_km_scan_bwd(s, cdt, dt, A, vd, ddtW, rho, eta, zeta, hsh, hdm, dend2, d_dt, st),
            "km_scan_bwd");
    SSD_HIP(ssd::launch_reduce_heads(s, dA, nullptr, nullptr, s.nblk(), d_A, nullptr, st), "reduce_heads");
    if (g_debug) {
        const bool bf = s.io == SSD_BF16;
        const int64_t tk = static_cast<int64_t>(s.B) * s.N * s.L * s.H;
        if (int rc = check_outputs(st, "ssd_state_moments_bwd",
                                   {{d_x, tk * s.P, bf, "d_x"}, {d_dt, tk, false, "d_dt"}, {d_A, s.H, false, "d_A"},
                                    {d_B, tk * s.R, bf, "d_B"}, {d_init, nstate, false, "d_init"}}))
            return rc;
    }
    return ok();
}

int ssd_moments_pr(int64_t batch, int64_t nheads, int64_t dstate, const float* m2,
                   const float* m1, const int64_t* count, int center, float* pr, float* trace,
                   void* stream) {
    if (int rc = validate_pr("ssd_moments_pr", batch, nheads, dstate, m2, m1, count, center, pr,
                             nullptr))
        return rc;
    if (batch == 0) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    SSD_HIP(ssd::launch_pr_fwd((int)batch, (int)nheads, (int)dstate, m2, center ? m1 : nullptr,
                               count, center != 0, pr, trace, st),
            "k_pr_fwd");
    return ok();
}

int ssd_moments_pr_bwd(int64_t batch, int64_t nheads, int64_t dstate, const float* d_pr,
                       const float* m2, const float* m1, const int64_t* count, int center,
                       float* d_m2, float* d_m1, void* stream) {
    if (int rc = validate_pr("ssd_moments_pr_bwd", batch, nheads, dstate, m2, m1, count, center,
                             d_m2, d_m2))
        return rc;
    if (batch == 0) return ok();
    if (!d_pr) return fail(SSD_ERR_NULL, "ssd_moments_pr_bwd: d_pr is required");
    hipStream_t st = static_cast<hipStream_t>(stream);
    SSD_HIP(ssd::launch_pr_bwd((int)batch, (int)nheads, (int)dstate, d_pr, m2,
                               center ? m1 : nullptr, count, center != 0, d_m2, d_m1, st),
            "k_pr_bwd");
    return ok();
}

int ssd_y_diag(int64_t ntokens, int64_t mimo_rank, int64_t nheads, int64_t headdim,
               int64_t dstate, int io_dtype, const void* v, const void* B, const void* C,
               const float* gamma, void* y_diag, void* stream) {
    ssd::DiagShape d;
    if (int rc = validate_diag("ssd_y_diag", ntokens, mimo_rank, nheads, headdim, dstate, io_dtype, &d))
        return rc;
    if (ntokens > 0 && (!v || !B || !C || !gamma || !y_diag))
        return fail(SSD_ERR_NULL, "ssd_y_diag: v, B, C, gamma and y_diag are required");
    if (int rc = check_diag_ptrs(d, {{v, "v"}, {B, "B"}, {C, "C"}, {y_diag, "y_diag"}})) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ntokens > 0) SSD_HIP(ssd::launch_diag_fwd(d, v, B, C, gamma, y_diag, st), "k_diag_fwd");
    return ok();
}

int ssd_y_diag_bwd(int64_t ntokens, int64_t mimo_rank, int64_t nheads, int64_t headdim,
                   int64_t dstate, int io_dtype, const void* dy, const void* v, const void* B,
                   const void* C, const float* gamma, void* d_v, void* d_B, void* d_C,
                   float* d_gamma, void* stream) {
    ssd::DiagShape d;
    if (int rc = validate_diag("ssd_y_diag_bwd", ntokens, mimo_rank, nheads, headdim, dstate,
                               io_dtype, &d))
        return rc;
    if (ntokens > 0 && (!dy || !v || !B || !C || !gamma || !d_v || !d_B || !d_C || !d_gamma))
        return fail(SSD_ERR_NULL,
                    "ssd_y_diag_bwd: dy, v, B, C, gamma, d_v, d_B, d_C and d_gamma are required");
    if (int rc = check_diag_ptrs(d, {{dy, "dy"}, {v, "v"}, {B, "B"}, {C, "C"}, {d_v, "d_v"},
                                     {d_B, "d_B"}, {d_C, "d_C"}}))
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ntokens > 0)
        SSD_HIP(ssd::launch_diag_bwd(d, dy, v, B, C, gamma, d_v, d_B, d_C, d_gamma, st), "k_diag_bwd");
    return ok();
}

int ssd_quat_workspace_size(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, int bwd,
                            size_t* bytes) {
    ssd::QuatShape s;
    if (int rc = validate_quat("ssd_quat_workspace_size", batch, seq, nheads, nquat, bwd != 0, &s)) return rc;
    if (!bytes) return fail(SSD_ERR_NULL, "ssd_quat_workspace_size: bytes is NULL");
    *bytes = ssd::quat_plan(s, bwd != 0).total;
    return ok();
}

int ssd_quat_scan(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, const float* q,
                  const float* init, float* cum, void* ws, size_t ws_bytes, void* stream) {
    ssd::QuatShape s;
    if (int rc = validate_quat("ssd_quat_scan", batch, seq, nheads, nquat, false, &s)) return rc;
    const bool work = batch > 0 && seq > 0;
    if (work && (!q || !cum)) return fail(SSD_ERR_NULL, "ssd_quat_scan: q and cum are required");
    for (auto p : {std::make_pair((const void*)q, "q"), std::make_pair((const void*)init, "init"),
                   std::make_pair((const void*)cum, "cum")})
        if (int rc = check_align(p.first, p.second, 16)) return rc;
    const ssd::QuatPlan plan = ssd::quat_plan(s, false);
    if (plan.total > 0 && (!ws || ws_bytes < plan.total))
        return fail(SSD_ERR_WORKSPACE, "ssd_quat_scan: workspace needs %zu bytes (got %zu%s)",
                    plan.total, ws_bytes, ws ? "" : ", NULL pointer");
    if (int rc = check_align(ws, "workspace", 256)) return rc;
    if (!work) return ok();
    hipStream_t st = static_cast<hipStream_t>(stream);
    SSD_HIP(ssd::launch_quat_clear(s, false, ws, st), "k_quat_clear");
    SSD_HIP(ssd::launch_quat_fwd(s, q, init, cum, ws, st), "k_quat_fwd");
    return ok();
}

int ssd_quat_scan_bwd(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, const float* q,
                      const float* init, const float* d_cum, float* d_q, float* d_init, void* ws,
                      size_t ws_bytes, void* stream) {
    ssd::QuatShape s;
    if (int rc = validate_quat("ssd_quat_scan_bwd", batch, seq, nheads, nquat, true, &s)) return rc;
    const bool work = batch > 0 && seq > 0;
    if (work && (!q || !d_cum || !d_q))
        return fail(SSD_ERR_NULL, "ssd_quat_scan_bwd: q, d_cum and d_q are required");
    for (auto p : {std::make_pair((const void*)q, "q"), std::make_pair((const void*)init, "init"),
                   std::make_pair((const void*)d_cum, "d_cum"), std::make_pair((const void*)d_q, "d_q"),
                   std::make_pair((const void*)d_init, "d_init")})
        if (int rc = check_align(p.first, p.second, 16)) return rc;
    const ssd::QuatPlan plan = ssd::quat_plan(s, true);
    if (plan.total > 0 && (!ws || ws_bytes < plan.total))
        return fail(SSD_ERR_WORKSPACE, "ssd_quat_scan_bwd: workspace needs %zu bytes (got %zu%s)",
                    plan.total, ws_bytes, ws ? "" : ", NULL pointer");
    if (int rc = check_align(ws, "workspace", 256)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!work) {  // nothing flows back: d_init = 0
        if (batch > 0 && d_init)
            SSD_HIP(ssd::launch_quat_zero(d_init, batch * nheads * nquat * 4, st), "k_fill_u32");
        return ok();
    }
    SSD_HIP(ssd::launch_quat_clear(s, true, ws, st), "k_quat_clear");
    SSD_HIP(ssd::launch_quat_bwd(s, q, init, d_cum, d_q, d_init, ws, st, 0), "k_quat_carry");
    SSD_HIP(ssd::launch_quat_bwd(s, q, init, d_cum, d_q, d_init, ws, st, 1), "k_quat_bwd");
    return ok();
}

int ssd_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype,
             const void* x, const float* dt, const float* A, const void* B, const void* C,
             const float* D, const float* state, float* new_state, void* y, void* stream) {
    if (io_dtype != SSD_F32 && io_dtype != SSD_BF16)
        return fail(SSD_ERR_DTYPE, "ssd_step: io_dtype must be SSD_F32 (0) or SSD_BF16 (1) (got %d)",
                    io_dtype);
    if (batch < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0)
        return fail(SSD_ERR_SHAPE, "ssd_step: need batch >= 0 and nheads, headdim, dstate > 0 "
                    "(got %lld, %lld, %lld, %lld)", (long long)batch, (long long)nheads,
                    (long long)headdim, (long long)dstate);
    if (!pow2_in(headdim, 16, 128) || !pow2_in(dstate, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "ssd_step: headdim and dstate must be 16, 32, 64 or 128 "
                    "(got %lld, %lld)", (long long)headdim, (long long)dstate);
    // one workgroup of 256 work-items per (b, h)
    if (batch > (1 << 30) || nheads > (1 << 30) ||
        (double)batch * nheads * 256.0 > ssd::kMaxGridItems)
        return fail(SSD_ERR_UNSUPPORTED, "ssd_step: problem too large for one call: a launch would "
                    "exceed 2^32 work-items (split the batch)");
    if (batch == 0) return ok();
    if (!x || !dt || !A || !B || !C || !D || !state || !new_state || !y)
        return fail(SSD_ERR_NULL, "ssd_step: every pointer is required");
    const size_t ia = io_dtype == SSD_BF16 ? 8 : 16;
    if (int rc = check_align(B, "B", ia)) return rc;
    if (int rc = check_align(C, "C", ia)) return rc;
    if (int rc = check_align(state, "state", 16)) return rc;
    if (int rc = check_align(new_state, "new_state", 16)) return rc;
    const size_t sbytes = (size_t)batch * nheads * headdim * dstate * sizeof(float);
    const char* a = reinterpret_cast<const char*>(state);
    const char* b = reinterpret_cast<const char*>(new_state);
    if (a != b && a < b + sbytes && b < a + sbytes)
        return fail(SSD_ERR_UNSUPPORTED, "ssd_step: state and new_state overlap without being equal");
    ssd::StepShape s{(int)batch, (int)nheads, (int)headdim, (int)dstate, io_dtype};
    hipStream_t st = static_cast<hipStream_t>(stream);
    SSD_HIP(ssd::launch_step(s, x, dt, A, B, C, D, state, new_state, y, st), "k_step");
    return ok();
}

}  // extern "C"
