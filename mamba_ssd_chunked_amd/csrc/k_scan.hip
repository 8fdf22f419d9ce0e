// Bandwidth-bound passes of the SSD scan: K1 (within-chunk cumsum), the K4
// serial carry across chunks and its reverse, K1's backward (suffix sums), the
// per-head reductions of d_A / d_D, and a small fill kernel.
//
// Page: burn-mamba "mamba2/ssd/serial_recalculated/combined_backward.rs".
//  - K1 is the inclusive cumsum of dt * a_decay inside each chunk (RECOMPUTE
//    section); its backward is the suffix sum of the gradient w.r.t. the
//    cumsum ("SUM GRADIENT CONTRIBUTIONS + K1 BACKWARD").
//  - K4 passes s_{i+1} = exp(end_i) s_i + intra_i across chunks; its reverse
//    ("K4 backward step") keeps d_s_i = exp(end_i) d_s_{i+1} + d_chunk_input_i
//    and hands d_s_{i+1} to chunk i as the gradient of its intra-chunk state.
//
// Precision: A is constant per head, so the cumsum of dt * A equals A times the
// cumsum of dt.  K1 stores cdt = cumsum(dt) in fp64 and every consumer forms a
// decay exponent as A * (cdt[t] - cdt[s]) in fp64 before one fp32 exp.  At
// |cumsum| of several hundred an fp32 cumsum would put relative errors of
// 1e-5..1e-4 on the decays; cdt also gives d_A its exact per-pair weights
// (see k_chunk_bwd.hip).
#include <mutex>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// One wave64 per chunk; lane j owns positions [j*E, j*E + E), E = L / 64, read
// as one vector and written as E / 2 pairs of doubles.  (Packing 2 or 4 chunks
// into a wave, their loads issued together and their scans interleaved, was no
// faster on 16384 chunks.)
template <int E>
__device__ __forceinline__ void load_e(const float* p, float (&v)[E]) {
    if constexpr (E == 4) {
        const v4f u = *reinterpret_cast<const v4f*>(p);
        v[0] = u[0]; v[1] = u[1]; v[2] = u[2]; v[3] = u[3];
    } else if constexpr (E == 2) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        v[0] = u.x; v[1] = u.y;
    } else {
        v[0] = *p;
    }
}

template <int E>
__global__ __launch_bounds__(NT) void k1_cumsum(const float* __restrict__ dt,
                                                double* __restrict__ cdt, int64_t nchunks_total) {
    constexpr int L = 64 * E;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (c >= nchunks_total) return;
    float v[E];
    load_e<E>(dt + c * L + lane * E, v);
    double run[E];
    double incl = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        incl += static_cast<double>(v[e]);
        run[e] = incl;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    double* dst = cdt + c * L + lane * E;
    if constexpr (E == 1) {
        dst[0] = run[0] + excl;
    } else {
#pragma unroll
        for (int e = 0; e < E; e += 2)
            *reinterpret_cast<v2d*>(dst + e) = v2d{run[e] + excl, run[e + 1] + excl};
    }
}

hipError_t launch_k1_cumsum(const Shape& s, const float* dt, double* cdt, hipStream_t st) {
    const int64_t nc = s.chunks();
    if (nc == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((nc + 3) / 4));
    switch (s.L) {
        case 64: hipLaunchKernelGGL(k1_cumsum<1>, grid, dim3(NT), 0, st, dt, cdt, nc); break;
        case 128: hipLaunchKernelGGL(k1_cumsum<2>, grid, dim3(NT), 0, st, dt, cdt, nc); break;
        case 256: hipLaunchKernelGGL(k1_cumsum<4>, grid, dim3(NT), 0, st, dt, cdt, nc); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------- K4
// One thread per (b, h, 4 consecutive state elements); a serial loop over the
// chunks.
__device__ __forceinline__ float chunk_decay(const double* cdt_bh, double a, int i, int L) {
    return static_cast<float>(exp(a * cdt_bh[static_cast<int64_t>(i) * L + (L - 1)]));
}

// The serial carry s <- dec_i s + in_i over the chunks of one (b, h, 4 state
// elements), visited forward (i = 0 .. N-1) or in reverse; each chunk's input
// at p0 + i * stride is overwritten in place by the carry entering it.  KF
// chunks (input and chunk-end cumsum) are loaded ahead of the FMA chain -- with
// one chunk ahead the long-sequence passes (512 chunks, 65536 threads) waited a
// memory latency per chunk (2.7 TB/s; 8 ahead: 6.3 TB/s).  Every chunk's input
// is loaded before its slot is overwritten.
template <int KF>
__device__ __forceinline__ v4f carry_pass(float* p0, int64_t stride, int N, bool reverse,
                                          const double* cdt_bh, double a, int L, v4f s) {
    // visit order as a start and a signed step; the ring holds raw inputs (a decay
    // computed at load time would wait for its load, and the in-order load counter
    // would drain every load behind it), and the steady-state loop is straight-line
    // code so that each use waits only for its own load
    float* const q0 = reverse ? p0 + static_cast<int64_t>(N - 1) * stride : p0;
    const int64_t qs = reverse ? -stride : stride;
    const double* const c0 = cdt_bh + (reverse ? static_cast<int64_t>(N - 1) * L : 0) + (L - 1);
    const int64_t cs = reverse ? -static_cast<int64_t>(L) : static_cast<int64_t>(L);
    v4f buf[KF];
    double cend[KF];
#pragma unroll
    for (int k = 0; k < KF; ++k)
        if (k < N) {
            buf[k] = *reinterpret_cast<const v4f*>(q0 + k * qs);
            cend[k] = c0[k * cs];
        }
    int kk = 0;
    for (; kk + 2 * KF <= N; kk += KF) {  // every step loads the chunk KF ahead
#pragma unroll
        for (int k = 0; k < KF; ++k) {
            const v4f cur = buf[k];
            const float d = static_cast<float>(exp(a * cend[k]));
            buf[k] = *reinterpret_cast<const v4f*>(q0 + (kk + k + KF) * qs);
            cend[k] = c0[(kk + k + KF) * cs];
            *reinterpret_cast<v4f*>(q0 + (kk + k) * qs) = s;
            s = d * s + cur;
        }
    }
    for (; kk < N; kk += KF) {  // the last chunks
#pragma unroll
        for (int k = 0; k < KF; ++k)
            if (kk + k < N) {
                const v4f cur = buf[k];
                const float d = static_cast<float>(exp(a * cend[k]));
                if (kk + k + KF < N) {
                    buf[k] = *reinterpret_cast<const v4f*>(q0 + (kk + k + KF) * qs);
                    cend[k] = c0[(kk + k + KF) * cs];
                }
                *reinterpret_cast<v4f*>(q0 + (kk + k) * qs) = s;
                s = d * s + cur;
            }
    }
    return s;
}

template <int KF>
__global__ __launch_bounds__(NT) void k4_state_pass(float* __restrict__ S,
                                                     const double* __restrict__ cdt,
                                                     const float* __restrict__ A,
                                                     const float* __restrict__ init,
                                                     float* __restrict__ final_state, int N,
                                                     int H, int L, int PR, int64_t total4) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (idx >= total4) return;
    const int PR4 = PR >> 2;
    const int64_t bh = idx / PR4;
    const int e = static_cast<int>(idx - bh * PR4) * 4;
    const int h = static_cast<int>(bh % H);
    const int64_t b = bh / H;
    const double* cdt_bh = cdt + bh * N * L;
    const double a = static_cast<double>(A[h]);
    const int64_t stride = static_cast<int64_t>(H) * PR;
    v4f s = init ? *reinterpret_cast<const v4f*>(init + bh * PR + e) : zero4();
    s = carry_pass<KF>(S + (b * N * H + h) * PR + e, stride, N, false, cdt_bh, a, L, s);
    if (final_state) *reinterpret_cast<v4f*>(final_state + bh * PR + e) = s;
}

// The two carries of the backward are independent (the forward carry of the chunk
// states S -> S_in, the reverse carry of the chunk gradients dS -> d_intra), so they run
// in separate threads: with `forward` the first nb blocks take the forward carry and the
// next nb the reverse one (nb = blocks of one pass), which doubles the loads in flight
// of a launch whose threads each walk a whole chain (the 64k-token workload's 65536
// threads: 404 -> 379 us; equal on the 130M-shaped one).
template <int KF>
__global__ __launch_bounds__(NT) void k4_state_pass_bwd(
    float* __restrict__ S, float* __restrict__ dS, const double* __restrict__ cdt,
    const float* __restrict__ A, const float* __restrict__ init, const float* __restrict__ d_final,
    float* __restrict__ d_init, int N, int H, int L, int PR, int64_t total4, int forward,
    int64_t nb) {
    const bool fwd_role = forward && static_cast<int64_t>(blockIdx.x) < nb;
    const int64_t blk = forward && !fwd_role ? blockIdx.x - nb : blockIdx.x;
    const int64_t idx = blk * NT + threadIdx.x;
    if (idx >= total4) return;
    const int PR4 = PR >> 2;
    const int64_t bh = idx / PR4;
    const int e = static_cast<int>(idx - bh * PR4) * 4;
    const int h = static_cast<int>(bh % H);
    const int64_t b = bh / H;
    const double* cdt_bh = cdt + bh * N * L;
    const double a = static_cast<double>(A[h]);
    const int64_t stride = static_cast<int64_t>(H) * PR;
    if (fwd_role) {  // chunk-entry states
        const v4f s0 = init ? *reinterpret_cast<const v4f*>(init + bh * PR + e) : zero4();
        carry_pass<KF>(S + (b * N * H + h) * PR + e, stride, N, false, cdt_bh, a, L, s0);
        return;
    }
    // reverse: gradient of the state leaving each chunk
    v4f gacc = d_final ? *reinterpret_cast<const v4f*>(d_final + bh * PR + e) : zero4();
    gacc = carry_pass<KF>(dS + (b * N * H + h) * PR + e, stride, N, true, cdt_bh, a, L, gacc);
    if (d_init) *reinterpret_cast<v4f*>(d_init + bh * PR + e) = gacc;
}

// Chunks loaded ahead by the carry passes: 8 for chains of 64 chunks or more
// (the 64k-token workload: 512 serial steps, 65536 threads), else 4 (measured on
// gfx950: as fast as 1 with 196608 threads, 1.4x faster with 49152).
int k4_depth(const Shape& s) { return s.N >= 64 ? 8 : 4; }

hipError_t launch_k4_pass(const Shape& s, float* S, const double* cdt, const float* A,
                          const float* init, float* final_state, hipStream_t st) {
    const int PR = s.P * s.R;
    const int64_t total4 = static_cast<int64_t>(s.B) * s.H * (PR / 4);
    if (total4 == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((total4 + NT - 1) / NT));
    if (k4_depth(s) == 8)
        hipLaunchKernelGGL(k4_state_pass<8>, grid, dim3(NT), 0, st, S, cdt, A, init, final_state,
                           s.N, s.H, s.L, PR, total4);
    else
        hipLaunchKernelGGL(k4_state_pass<4>, grid, dim3(NT), 0, st, S, cdt, A, init,
                           final_state, s.N, s.H, s.L, PR, total4);
    return hipGetLastError();
}

hipError_t launch_k4_pass_bwd(const Shape& s, float* S, float* dS, const double* cdt,
                              const float* A, const float* init, const float* d_final,
                              float* d_init, hipStream_t st, bool forward) {
    const int PR = s.P * s.R;
    const int64_t total4 = static_cast<int64_t>(s.B) * s.H * (PR / 4);
    if (total4 == 0) return hipSuccess;
    const int64_t nb = (total4 + NT - 1) / NT;
    const dim3 grid(static_cast<unsigned>(forward ? 2 * nb : nb));
    if (k4_depth(s) == 8)
        hipLaunchKernelGGL(k4_state_pass_bwd<8>, grid, dim3(NT), 0, st, S, dS, cdt, A, init,
                           d_final, d_init, s.N, s.H, s.L, PR, total4, forward ? 1 : 0, nb);
    else
        hipLaunchKernelGGL(k4_state_pass_bwd<4>, grid, dim3(NT), 0, st, S, dS, cdt, A,
                           init, d_final, d_init, s.N, s.H, s.L, PR, total4, forward ? 1 : 0, nb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------- K1^T
// Per chunk (one wave64): with g[k] = g1[k] + g2[k] the gradient w.r.t. the
// cumsum at k from BLUE/ORANGE, d_delta[k] the K3 gradient w.r.t. the decay
// exponent (end - cumsum[k]) and d_end the K4 gradient w.r.t. end = cumsum[L-1],
// the gradient w.r.t. dA_t = dt_t * A is
//   d_da[t] = sum_{k>=t} g[k] + sum_{k<t} d_delta[k] + d_end
// (end - cumsum[k] sums dA over positions k+1..L-1, so d_delta[k] reaches every
// t > k), and d_dt[t] += A d_da[t].  (d_A is assembled from per-pair weights in
// the chunk kernels instead of sum_t d_da[t] dt[t], which cancels badly.)
__device__ __forceinline__ void k1t_block(const float* __restrict__ g1, const float* __restrict__ g2,
                                          const float* __restrict__ d_delta,
                                          const float* __restrict__ d_end,
                                          const float* __restrict__ A, float* __restrict__ d_dt,
                                          int64_t nchunks_total, int H, int N, int L, int64_t blk) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c = blk * 4 + wave;
    if (c >= nchunks_total) return;
    const int h = static_cast<int>((c / N) % H);
    const double a = static_cast<double>(A[h]);
    const int E = L >> 6;
    const int64_t base = c * L + lane * E;
    double gv[4], dl[4];
    double gtot = 0.0, dtot = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) {
            gv[e] = static_cast<double>(g1[base + e]) + static_cast<double>(g2[base + e]);
            dl[e] = static_cast<double>(d_delta[base + e]);
            gtot += gv[e];
            dtot += dl[e];
        }
    // sum of g over the lanes after this one; sum of d_delta over the lanes before it
    double suf = gtot, pre = dtot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o1 = __shfl_down(suf, off);
        const double o2 = __shfl_up(pre, off);
        if (lane + off < 64) suf += o1;
        if (lane >= off) pre += o2;
    }
    double after = __shfl_down(suf, 1);
    if (lane == 63) after = 0.0;
    double before = __shfl_up(pre, 1);
    if (lane == 0) before = 0.0;
    const double dend = static_cast<double>(d_end[c]);
    double sfx[4];
    double run = after;
#pragma unroll
    for (int e = 3; e >= 0; --e)
        if (e < E) {
            run += gv[e];
            sfx[e] = run;
        }
    double pfx = before;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) {
            const double dda = sfx[e] + pfx + dend;
            pfx += dl[e];
            d_dt[base + e] = static_cast<float>(static_cast<double>(d_dt[base + e]) + a * dda);
        }
}


// ------------------------------------------------------------- head reductions
// One workgroup per head sums partials stored in [b, n, h, k] order (k < nk) in
// a fixed order: thread j takes a fixed strided subset, then a fixed tree, so
// the result does not depend on scheduling.  Up to two arrays are summed per
// output (d_A gets the target- and source-side partials).
__device__ __forceinline__ void reduce_head(const double* __restrict__ a0,
                                            const double* __restrict__ a1,
                                            const double* __restrict__ d0, float* __restrict__ d_A,
                                            float* __restrict__ d_D, int B, int H, int N, int nk,
                                            int h) {
    __shared__ double ra[NT], rd[NT];
    const int tid = threadIdx.x;
    double a = 0.0, d = 0.0;
    const int64_t total = static_cast<int64_t>(B) * N * nk;
    for (int64_t j = tid; j < total; j += NT) {
        const int64_t bn = j / nk, k = j - (j / nk) * nk;
        const int64_t o = (bn * H + h) * nk + k;
        if (a0) a += a0[o];
        if (a1) a += a1[o];
        if (d0) d += d0[o];
    }
    ra[tid] = a;
    rd[tid] = d;
    __syncthreads();
    for (int w = NT / 2; w > 0; w >>= 1) {
        if (tid < w) {
            ra[tid] += ra[tid + w];
            rd[tid] += rd[tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        if (d_A) d_A[h] = static_cast<float>(ra[0]);
        if (d_D) d_D[h] = static_cast<float>(rd[0]);
    }
}

__global__ __launch_bounds__(NT) void reduce_heads(const double* __restrict__ a0,
                                                   const double* __restrict__ a1,
                                                   const double* __restrict__ d0,
                                                   float* __restrict__ d_A,
                                                   float* __restrict__ d_D, int B, int H, int N,
                                                   int nk) {
    reduce_head(a0, a1, d0, d_A, d_D, B, H, N, nk, blockIdx.x);
}

// K1^T and the per-head d_A / d_D sums of the SSD backward in one launch (both read
// only what the chunk kernels wrote): blocks [0, nk1t) take four chunks each, block
// nk1t + h sums head h.  One launch instead of two: the two small grids run side by side.
__global__ __launch_bounds__(NT) void k1t_and_heads(
    const float* __restrict__ g1, const float* __restrict__ g2,
    const float* __restrict__ d_delta, const float* __restrict__ d_end,
    const float* __restrict__ A, float* __restrict__ d_dt, int64_t nchunks_total, int H, int N,
    int L, int64_t nk1t, const double* __restrict__ a0, const double* __restrict__ a1,
    const double* __restrict__ d0, float* __restrict__ d_A, float* __restrict__ d_D, int B,
    int nk) {
    const int64_t blk = blockIdx.x;
    if (blk < nk1t)
        k1t_block(g1, g2, d_delta, d_end, A, d_dt, nchunks_total, H, N, L, blk);
    else
        reduce_head(a0, a1, d0, d_A, d_D, B, H, N, nk, static_cast<int>(blk - nk1t));
}

hipError_t launch_k1t_heads(const Shape& s, const float* g1, const float* g2, const float* d_delta,
                            const float* d_end, const float* A, float* d_dt,
                            const double* dA_part0, const double* dA_part1, const double* dD_part,
                            int nk, float* d_A, float* d_D, hipStream_t st) {
    const int64_t nc = s.chunks();
    const int64_t nk1t = (nc + 3) / 4;
    const int64_t blocks = nk1t + s.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k1t_and_heads, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, st, g1, g2,
                       d_delta, d_end, A, d_dt, nc, s.H, s.N, s.L, nk1t, dA_part0, dA_part1,
                       dD_part, d_A, d_D, s.B, nk);
    return hipGetLastError();
}

hipError_t launch_reduce_heads(const Shape& s, const double* dA_part0, const double* dA_part1,
                               const double* dD_part, int nk, float* d_A, float* d_D,
                               hipStream_t st) {
    if (s.H == 0) return hipSuccess;
    hipLaunchKernelGGL(reduce_heads, dim3(s.H), dim3(NT), 0, st, dA_part0, dA_part1, dD_part, d_A,
                       d_D, s.B, s.H, s.N, nk);
    return hipGetLastError();
}

__global__ __launch_bounds__(NT) void copy_or_zero(float* __restrict__ dst,
                                                  const float* __restrict__ src, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

struct I64Pack {
    int64_t v[64];
};

__global__ void set_i64(int64_t* __restrict__ dst, I64Pack vals, int n) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = vals.v[i];
}

hipError_t launch_set_i64(int64_t* dst, const int64_t* vals, int64_t fill, int64_t n, hipStream_t st) {
    for (int64_t o = 0; o < n; o += 64) {
        I64Pack pk;
        const int m = static_cast<int>(n - o < 64 ? n - o : 64);
        for (int k = 0; k < 64; ++k) pk.v[k] = k < m ? (vals ? vals[o + k] : fill) : 0;
        hipLaunchKernelGGL(set_i64, dim3(1), dim3(64), 0, st, dst + o, pk, m);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t st) {
    if (n <= 0 || !dst) return hipSuccess;
    hipLaunchKernelGGL(copy_or_zero, dim3(static_cast<unsigned>((n + NT - 1) / NT)), dim3(NT), 0,
                       st, dst, src, n);
    return hipGetLastError();
}

// ------------------------------------------------------------ debug checks
// One flag word per checked tensor (a file-scope device array; each GPU has its own
// copy, found with hipGetSymbolAddress).  The scan stores 1 into its word when it meets
// a NaN or an infinity: plain stores of one value, so concurrent finds need no atomics.
constexpr int kMaxChecked = 16;
static __device__ int g_nonfinite[kMaxChecked];

__global__ void k_clear_flags(int* __restrict__ f, int n) {
    if (static_cast<int>(threadIdx.x) < n) f[threadIdx.x] = 0;
}

__global__ __launch_bounds__(NT) void k_nonfinite(const void* __restrict__ p, int64_t n, int bf16,
                                                  int* __restrict__ flag) {
    bool bad = false;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * NT) {
        const uint32_t e = bf16 ? (static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16)
                                : static_cast<const uint32_t*>(p)[i];
        bad |= (e & 0x7f800000u) == 0x7f800000u;  // exponent all ones: infinity or NaN
    }
    if (bad) *flag = 1;
}

hipError_t nonfinite_flags(int** flags) {
    static std::mutex mu;
    static int* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(g_nonfinite));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<int*>(a);
    }
    *flags = addr[dev];
    return hipSuccess;
}

hipError_t launch_clear_flags(int* flags, int n, hipStream_t st) {
    hipLaunchKernelGGL(k_clear_flags, dim3(1), dim3(64), 0, st, flags, n);
    return hipGetLastError();
}

hipError_t launch_nonfinite(const void* p, int64_t n, bool bf16, int* flag, hipStream_t st) {
    if (n <= 0 || !p) return hipSuccess;
    const int64_t want = (n + NT - 1) / NT;
    const unsigned grid = static_cast<unsigned>(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(k_nonfinite, dim3(grid), dim3(NT), 0, st, p, n, bf16 ? 1 : 0, flag);
    return hipGetLastError();
}

}  // namespace ssd
