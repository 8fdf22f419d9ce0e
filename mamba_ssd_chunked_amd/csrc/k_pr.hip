// Participation ratio of the pooled state moments and its gradient.
//
// Page: burn-mamba "modules/state_moments.rs", StateMoments::pr and ::trace.
// Per (batch, head) slice, with n = count[b] and mu = m1 / n:
//   Sigma     = m2 / n                 (centred: minus mu mu^T)
//   s         = max(tr Sigma, 2^-126)  fp32's smallest normal; the page detaches s
//   PR        = tr(Sigma/s)^2 / max(||Sigma/s||_F^2, 1e-12)
//   trace     = tr(m2) / n
// Because s is held fixed, dPR/dSigma = G = alpha I - beta Sigma with
//   alpha = 2 tr1 / (tr2 s),  beta = 2 tr1^2 / (tr2^2 s^2)   (tr1 = tr(Sigma)/s,
//   tr2 = ||Sigma||_F^2 / s^2; beta = 0 while the 1e-12 floor is active), so
//   d_m2 = d_pr G / n  and, centred,  d_m1 = -d_pr (G + G^T) mu / n
//        = -d_pr (2 alpha mu - beta (Sigma + Sigma^T) mu) / n.
// The page computes in the moments' fp32; here every sum and every Sigma entry
// is formed in fp64 from the fp32 inputs (the kernels read each slice once and
// are bound by HBM, so the wider arithmetic is free), and the results are
// rounded to fp32 once.
//
// Layout and work split: one workgroup per slice.  The r x r slice is read as
// float4 column quads: thread t takes quad cq = t % (r/4) of the rows
// rg + G k (rg = t / (r/4), G = threads / (r/4) row groups), so a wave reads
// 64/(r/4) whole consecutive rows -- contiguous 1 KB per wave instruction.  The
// backward keeps its quads in registers between the reductions and the writes,
// so each slice crosses HBM once in and once out.  Reductions are fixed-order
// (butterflies inside a wave, then the waves in index order): bitwise
// reproducible, no atomics.
#include <float.h>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr double kMinPositive = 1.1754943508222875e-38;  // 2^-126
constexpr double kDivEps = 1e-12;

template <int R>
struct PrTile {
    static constexpr int Q = R / 4;                           // column quads per row
    static constexpr int NTH = R * R / 4 < NT ? R * R / 4 : NT;  // threads per slice
    static constexpr int G = NTH / Q;                         // row groups
    static constexpr int KR = R / G;                          // rows per thread
    static constexpr int NW = NTH / 64;                       // waves
    static_assert(Q <= 64 && 64 % Q == 0 && R % G == 0 && NTH % 64 == 0, "tile shape");
};

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// Sum of three per-thread values over the workgroup; every thread gets the totals.
template <int NW>
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c, double (*red)[3]) {
    a = wave_sum(a);
    b = wave_sum(b);
    c = wave_sum(c);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[wave][0] = a;
        red[wave][1] = b;
        red[wave][2] = c;
    }
    __syncthreads();
    a = b = c = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        a += red[w][0];
        b += red[w][1];
        c += red[w][2];
    }
}

// Loads this thread's quads of slice m2 and forms the sums tr Sigma, ||Sigma||_F^2
// and tr m2 (every thread returns the slice totals).
template <int R>
__device__ __forceinline__ void slice_sums(const float* __restrict__ m2, const double* mu,
                                           double inv_n, v4f (&v)[PrTile<R>::KR], double& tr,
                                           double& sq, double& raw, double (*red)[3]) {
    using T = PrTile<R>;
    const int cq = threadIdx.x % T::Q, rg = threadIdx.x / T::Q;
#pragma unroll
    for (int k = 0; k < T::KR; ++k)
        v[k] = *reinterpret_cast<const v4f*>(m2 + (rg + T::G * k) * R + 4 * cq);
    tr = sq = raw = 0.0;
#pragma unroll
    for (int k = 0; k < T::KR; ++k) {
        const int i = rg + T::G * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * cq + e;
            const double S = static_cast<double>(v[k][e]) * inv_n - mu[i] * mu[j];
            sq += S * S;
            if (i == j) {
                tr += S;
                raw += static_cast<double>(v[k][e]);
            }
        }
    }
    block_sum3<T::NW>(tr, sq, raw, red);
}

// mu = m1 / n of slice bh when centring, else 0 (m1 may then be NULL).
template <int R>
__device__ __forceinline__ void load_mu(const float* __restrict__ m1, int64_t bh, int center,
                                        double inv_n, double* mu) {
    for (int i = threadIdx.x; i < R; i += PrTile<R>::NTH)
        mu[i] = center ? static_cast<double>(m1[bh * R + i]) * inv_n : 0.0;
    __syncthreads();
}

}  // namespace

template <int R>
__global__ __launch_bounds__(PrTile<R>::NTH) void k_pr_fwd(const float* __restrict__ m2,
                                                          const float* __restrict__ m1,
                                                          PrCounts cnt, int H, int center,
                                                          float* __restrict__ pr,
                                                          float* __restrict__ trace) {
    using T = PrTile<R>;
    __shared__ double mu[R];
    __shared__ double red[T::NW][3];
    const int64_t bh = blockIdx.x;  // slice within this launch's batch group
    const double inv_n = cnt.inv_n[bh / H];
    load_mu<R>(m1, bh, center, inv_n, mu);
    v4f v[T::KR];
    double tr, sq, raw;
    slice_sums<R>(m2 + bh * R * R, mu, inv_n, v, tr, sq, raw, red);
    if (threadIdx.x == 0) {
        const double s = tr > kMinPositive ? tr : kMinPositive;
        const double tr1 = tr / s;
        double tr2 = sq / (s * s);
        tr2 = tr2 > kDivEps ? tr2 : kDivEps;
        pr[bh] = static_cast<float>(tr1 * tr1 / tr2);
        if (trace) trace[bh] = static_cast<float>(raw * inv_n);
    }
}

template <int R>
__global__ __launch_bounds__(PrTile<R>::NTH) void k_pr_bwd(const float* __restrict__ d_pr,
                                                          const float* __restrict__ m2,
                                                          const float* __restrict__ m1,
                                                          PrCounts cnt, int H, int center,
                                                          float* __restrict__ d_m2,
                                                          float* __restrict__ d_m1) {
    using T = PrTile<R>;
    __shared__ double mu[R];
    __shared__ double red[T::NW][3];
    __shared__ double colbuf[T::NW][R];
    __shared__ double rowbuf[R];
    const int64_t bh = blockIdx.x;
    const double inv_n = cnt.inv_n[bh / H];
    load_mu<R>(m1, bh, center, inv_n, mu);
    v4f v[T::KR];
    double tr, sq, raw;
    slice_sums<R>(m2 + bh * R * R, mu, inv_n, v, tr, sq, raw, red);

    const double s = tr > kMinPositive ? tr : kMinPositive;
    const double tr1 = tr / s;
    const double t2 = sq / (s * s);
    const bool live = t2 > kDivEps;
    const double tr2 = live ? t2 : kDivEps;
    const double g = static_cast<double>(d_pr[bh]);
    const double alpha = g * 2.0 * tr1 / (tr2 * s);
    const double beta = live ? g * 2.0 * tr1 * tr1 / (tr2 * tr2 * s * s) : 0.0;

    const int cq = threadIdx.x % T::Q, rg = threadIdx.x / T::Q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double colp[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < T::KR; ++k) {
        const int i = rg + T::G * k;
        v4f out;
        double rowp = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * cq + e;
            const double S = static_cast<double>(v[k][e]) * inv_n - mu[i] * mu[j];
            out[e] = static_cast<float>(((i == j ? alpha : 0.0) - beta * S) * inv_n);
            rowp += S * mu[j];
            colp[e] += S * mu[i];
        }
        *reinterpret_cast<v4f*>(d_m2 + bh * R * R + i * R + 4 * cq) = out;
        if (d_m1 && center) {
            // row i's sum over its Q quads: lanes rg*Q .. rg*Q + Q - 1 of this wave
#pragma unroll
            for (int o = 1; o < T::Q; o <<= 1) rowp += __shfl_xor(rowp, o);
            if (cq == 0) rowbuf[i] = rowp;
        }
    }
    if (!d_m1) return;
    if (center) {
        // column sums: fold the row groups of this wave (lanes cq + Q m), then the waves
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int o = T::Q; o < 64; o <<= 1) colp[e] += __shfl_xor(colp[e], o);
        if (lane < T::Q)
#pragma unroll
            for (int e = 0; e < 4; ++e) colbuf[wave][4 * cq + e] = colp[e];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R; i += T::NTH) {
        double r = 0.0;
        if (center) {
            double col = 0.0;
#pragma unroll
            for (int w = 0; w < T::NW; ++w) col += colbuf[w][i];
            r = -(2.0 * alpha * mu[i] - beta * (rowbuf[i] + col)) * inv_n;
        }
        d_m1[bh * R + i] = static_cast<float>(r);
    }
}

namespace {

template <class F>
hipError_t per_batch_group(int B, const int64_t* count, F&& launch) {
    for (int b0 = 0; b0 < B; b0 += PrCounts::kMax) {
        PrCounts c;
        const int m = B - b0 < PrCounts::kMax ? B - b0 : PrCounts::kMax;
        for (int k = 0; k < PrCounts::kMax; ++k)
            c.inv_n[k] = k < m ? 1.0 / static_cast<double>(count[b0 + k]) : 0.0;
        const hipError_t e = launch(b0, m, c);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_pr_fwd(int B, int H, int R, const float* m2, const float* m1,
                         const int64_t* count, int center, float* pr, float* trace,
                         hipStream_t st) {
    return per_batch_group(B, count, [&](int b0, int m, const PrCounts& c) {
        const int64_t o = static_cast<int64_t>(b0) * H;
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(m) * H));
        const float* m1o = m1 ? m1 + o * R : nullptr;
        float* tro = trace ? trace + o : nullptr;
#define X(RR)                                                                                   \
    if (R == RR) {                                                                              \
        hipLaunchKernelGGL(k_pr_fwd<RR>, grid, dim3(PrTile<RR>::NTH), 0, st, m2 + o * RR * RR,  \
                           m1o, c, H, center, pr + o, tro);                                      \
        return hipGetLastError();                                                               \
    }
        X(16) X(32) X(64) X(128)
#undef X
        return hipErrorInvalidValue;
    });
}

hipError_t launch_pr_bwd(int B, int H, int R, const float* d_pr, const float* m2, const float* m1,
                         const int64_t* count, int center, float* d_m2, float* d_m1,
                         hipStream_t st) {
    return per_batch_group(B, count, [&](int b0, int m, const PrCounts& c) {
        const int64_t o = static_cast<int64_t>(b0) * H;
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(m) * H));
        const float* m1o = m1 ? m1 + o * R : nullptr;
        float* dm1o = d_m1 ? d_m1 + o * R : nullptr;
#define X(RR)                                                                                     \
    if (R == RR) {                                                                                \
        hipLaunchKernelGGL(k_pr_bwd<RR>, grid, dim3(PrTile<RR>::NTH), 0, st, d_pr + o,            \
                           m2 + o * RR * RR, m1o, c, H, center, d_m2 + o * RR * RR, dm1o);         \
        return hipGetLastError();                                                                 \
    }
        X(16) X(32) X(64) X(128)
#undef X
        return hipErrorInvalidValue;
    });
}

}  // namespace ssd
