// Gamma-weighted same-step correction y_diag of the Mamba-3 SSD, and its gradient.
//
// Page: burn-mamba "mamba3/single_ssd/ssd/serial_recalculated/diag.rs" (module
// doc, the general MIMO path and its analytic backward).  Per token t (the
// [b, n, l] axes flattened) and head h, over the mimo axis m:
//   qk[mo][mi] = sum_r C[t,mo,h,r] B[t,mi,h,r]
//   y[t,mo,h,p] = gamma[t,h] sum_mi qk[mo][mi] V[t,mi,h,p]
// and, for an upstream gradient dy,
//   DV[mo][mi] = sum_p dy[mo,p] V[mi,p],      d_gamma = sum qk o DV,
//   d_V[mi,p]  = gamma sum_mo qk[mo][mi] dy[mo,p],
//   d_C[mo,r]  = gamma sum_mi DV[mo][mi] B[mi,r],
//   d_B[mi,r]  = gamma sum_mo DV[mo][mi] C[mo,r].
// At mimo rank 1 this is the page's SISO path (one reduction over r, broadcast
// multiplies); the same code covers it with M = 1.
//
// The term has no recurrence and about one flop per byte even at mimo rank 4,
// so it is bound by HBM: no matrix cores, just coalesced vector loads.  A group
// of 16 lanes owns one (token, head): lane j holds the float4s j, j + 16 of every
// p- and r-row it needs, the m x m dot products are reduced across the group with
// butterflies (the group is 16 aligned lanes of one wave), and every output is
// written once.  The four groups of a wave are consecutive heads of one token,
// whose rows are adjacent in memory ([T, M, H, W] layout).  fp32 accumulation;
// bf16 tensors are widened on load and rounded to nearest even on store.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kGroup = 16;  // lanes per (token, head)


template <int M>
__device__ __forceinline__ void group_sum(float (&a)[M][M]) {
#pragma unroll
    for (int o = 1; o < kGroup; o <<= 1)
#pragma unroll
        for (int x = 0; x < M; ++x)
#pragma unroll
            for (int y = 0; y < M; ++y) a[x][y] += __shfl_xor(a[x][y], o);
}

__device__ __forceinline__ float dot4(v4f a, v4f b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// Outputs are written once and not read again by this kernel: non-temporal
// stores (measured: the mimo-rank-4 forward 246 -> 215 us; no change elsewhere).
template <class IO>
__device__ __forceinline__ void st4_out(typename IO::T* p, int64_t i, v4f v) {
    if constexpr (sizeof(typename IO::T) == 4) {
        __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p + i));
    } else {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 w{f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(w, reinterpret_cast<u2*>(p + i));
    }
}

// Every input element is read once per launch: non-temporal loads (the fwd + bwd step on
// the rank-1 workload 0.163 -> 0.151 ms, rank 4 0.611 -> 0.571 ms; with cached loads the
// 250 MB rank-1 working set partly stayed in the last-level cache between the two
// launches, a reuse a model with other work between them would not see).
template <class IO>
__device__ __forceinline__ v4f ld4_nt(const typename IO::T* p, int64_t i) {
    if constexpr (sizeof(typename IO::T) == 4) {
        return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p + i));
    } else {
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 w = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p + i));
        return v4f{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                   __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
    }
}

// Row (t, m, h) of a [T, M, H, W] tensor.
__device__ __forceinline__ int64_t row_of(int64_t t, int m, int h, int M, int H, int W) {
    return ((t * M + m) * H + h) * static_cast<int64_t>(W);
}

}  // namespace

// KP / KR: float4 slots per lane along p / r (1 for widths up to 64, 2 for 128).
// U: consecutive (token, head) pairs per group; all of their loads are issued
// before the first reduction, so a wave keeps U times more bytes in flight and
// the grid has U times fewer workgroups to dispatch.
template <class IO, int M, int KP, int KR, int U>
__global__ __launch_bounds__(NT) void k_diag_fwd(const typename IO::T* __restrict__ V,
                                                  const typename IO::T* __restrict__ Bm,
                                                  const typename IO::T* __restrict__ Cm,
                                                  const float* __restrict__ gamma,
                                                  typename IO::T* __restrict__ y, int64_t pairs,
                                                  int H, int P, int R) {
    const int64_t g0 = (static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x) / kGroup * U;
    const int j = threadIdx.x % kGroup;
    if (g0 >= pairs) return;  // whole groups leave together
    v4f cb[U][KR][M], bb[U][KR][M], vv[U][KP][M];
    float gm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t g = g0 + u < pairs ? g0 + u : pairs - 1;  // a ragged tail recomputes the last pair
        const int64_t t = g / H;
        const int h = static_cast<int>(g - t * H);
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            const int c4 = 4 * (j + kGroup * k);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                cb[u][k][m] = c4 < R ? ld4_nt<IO>(Cm, row_of(t, m, h, M, H, R) + c4) : zero4();
                bb[u][k][m] = c4 < R ? ld4_nt<IO>(Bm, row_of(t, m, h, M, H, R) + c4) : zero4();
            }
        }
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int c4 = 4 * (j + kGroup * k);
#pragma unroll
            for (int m = 0; m < M; ++m)
                vv[u][k][m] = c4 < P ? ld4_nt<IO>(V, row_of(t, m, h, M, H, P) + c4) : zero4();
        }
        gm[u] = gamma[g];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (g0 + u >= pairs) break;
        const int64_t g = g0 + u;
        const int64_t t = g / H;
        const int h = static_cast<int>(g - t * H);
        float qk[M][M];
#pragma unroll
        for (int a = 0; a < M; ++a)
#pragma unroll
            for (int b = 0; b < M; ++b) {
                qk[a][b] = 0.f;
#pragma unroll
                for (int k = 0; k < KR; ++k) qk[a][b] += dot4(cb[u][k][a], bb[u][k][b]);
            }
        group_sum<M>(qk);
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int c4 = 4 * (j + kGroup * k);
            if (c4 < P) {
#pragma unroll
                for (int a = 0; a < M; ++a) {
                    v4f acc = zero4();
#pragma unroll
                    for (int b = 0; b < M; ++b) acc += qk[a][b] * vv[u][k][b];
                    st4_out<IO>(y, row_of(t, a, h, M, H, P) + c4, gm[u] * acc);
                }
            }
        }
    }
}

template <class IO, int M, int KP, int KR>
__global__ __launch_bounds__(NT) void k_diag_bwd(const typename IO::T* __restrict__ dy,
                                                  const typename IO::T* __restrict__ V,
                                                  const typename IO::T* __restrict__ Bm,
                                                  const typename IO::T* __restrict__ Cm,
                                                  const float* __restrict__ gamma,
                                                  typename IO::T* __restrict__ d_v,
                                                  typename IO::T* __restrict__ d_b,
                                                  typename IO::T* __restrict__ d_c,
                                                  float* __restrict__ d_gamma, int64_t pairs,
                                                  int H, int P, int R) {
    const int64_t g = (static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x) / kGroup;
    const int j = threadIdx.x % kGroup;
    if (g >= pairs) return;
    const int64_t t = g / H;
    const int h = static_cast<int>(g - t * H);
    v4f cb[KR][M], bb[KR][M], vv[KP][M], dd[KP][M];
    float qk[M][M], dv[M][M];
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
        for (int b = 0; b < M; ++b) qk[a][b] = dv[a][b] = 0.f;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int c4 = 4 * (j + kGroup * k);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            cb[k][m] = c4 < R ? ld4_nt<IO>(Cm, row_of(t, m, h, M, H, R) + c4) : zero4();
            bb[k][m] = c4 < R ? ld4_nt<IO>(Bm, row_of(t, m, h, M, H, R) + c4) : zero4();
        }
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int c4 = 4 * (j + kGroup * k);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            vv[k][m] = c4 < P ? ld4_nt<IO>(V, row_of(t, m, h, M, H, P) + c4) : zero4();
            dd[k][m] = c4 < P ? ld4_nt<IO>(dy, row_of(t, m, h, M, H, P) + c4) : zero4();
        }
    }
#pragma unroll
    for (int a = 0; a < M; ++a)
#pragma unroll
        for (int b = 0; b < M; ++b) {
#pragma unroll
            for (int k = 0; k < KR; ++k) qk[a][b] += dot4(cb[k][a], bb[k][b]);
#pragma unroll
            for (int k = 0; k < KP; ++k) dv[a][b] += dot4(dd[k][a], vv[k][b]);
        }
    group_sum<M>(qk);
    group_sum<M>(dv);
    const float gm = gamma[g];
    if (j == 0) {
        float s = 0.f;
#pragma unroll
        for (int a = 0; a < M; ++a)
#pragma unroll
            for (int b = 0; b < M; ++b) s += qk[a][b] * dv[a][b];
        d_gamma[g] = s;
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int c4 = 4 * (j + kGroup * k);
        if (c4 < P) {
#pragma unroll
            for (int b = 0; b < M; ++b) {
                v4f acc = zero4();
#pragma unroll
                for (int a = 0; a < M; ++a) acc += qk[a][b] * dd[k][a];
                st4_out<IO>(d_v, row_of(t, b, h, M, H, P) + c4, gm * acc);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
        const int c4 = 4 * (j + kGroup * k);
        if (c4 < R) {
#pragma unroll
            for (int a = 0; a < M; ++a) {
                v4f acc = zero4();
#pragma unroll
                for (int b = 0; b < M; ++b) acc += dv[a][b] * bb[k][b];
                st4_out<IO>(d_c, row_of(t, a, h, M, H, R) + c4, gm * acc);
            }
#pragma unroll
            for (int b = 0; b < M; ++b) {
                v4f acc = zero4();
#pragma unroll
                for (int a = 0; a < M; ++a) acc += dv[a][b] * cb[k][a];
                st4_out<IO>(d_b, row_of(t, b, h, M, H, R) + c4, gm * acc);
            }
        }
    }
}

namespace {

template <class IO, int M, int KP, int KR>
hipError_t diag_go(const DiagShape& d, const void* dy, const void* V, const void* B, const void* C,
                   const float* gamma, void* y, void* d_v, void* d_b, void* d_c, float* d_gamma,
                   hipStream_t st) {
    using T = typename IO::T;
    const int64_t pairs = d.T * d.H;
    const dim3 grid(static_cast<unsigned>((pairs * kGroup + NT - 1) / NT));
    if (!dy) {
        constexpr int U = M == 4 ? 1 : 2;  // 1, 2 and 4 measured alike; 2 halves the grid
        const int64_t groups = (pairs + U - 1) / U;
        const dim3 gridf(static_cast<unsigned>((groups * kGroup + NT - 1) / NT));
        hipLaunchKernelGGL((k_diag_fwd<IO, M, KP, KR, U>), gridf, dim3(NT), 0, st,
                           static_cast<const T*>(V), static_cast<const T*>(B),
                           static_cast<const T*>(C), gamma, static_cast<T*>(y), pairs, d.H, d.P,
                           d.R);
    } else {
        hipLaunchKernelGGL((k_diag_bwd<IO, M, KP, KR>), grid, dim3(NT), 0, st,
                           static_cast<const T*>(dy), static_cast<const T*>(V),
                           static_cast<const T*>(B), static_cast<const T*>(C), gamma,
                           static_cast<T*>(d_v), static_cast<T*>(d_b), static_cast<T*>(d_c),
                           d_gamma, pairs, d.H, d.P, d.R);
    }
    return hipGetLastError();
}

template <class IO, int M>
hipError_t diag_k(const DiagShape& d, const void* dy, const void* V, const void* B, const void* C,
                  const float* gamma, void* y, void* d_v, void* d_b, void* d_c, float* d_gamma,
                  hipStream_t st) {
    const bool wp = d.P > 64, wr = d.R > 64;
#define X(KP, KR)                                                                          \
    if (wp == (KP == 2) && wr == (KR == 2))                                                \
        return diag_go<IO, M, KP, KR>(d, dy, V, B, C, gamma, y, d_v, d_b, d_c, d_gamma, st);
    X(1, 1) X(1, 2) X(2, 1) X(2, 2)
#undef X
    return hipErrorInvalidValue;
}

template <class IO>
hipError_t diag_io(const DiagShape& d, const void* dy, const void* V, const void* B, const void* C,
                   const float* gamma, void* y, void* d_v, void* d_b, void* d_c, float* d_gamma,
                   hipStream_t st) {
    switch (d.M) {
        case 1: return diag_k<IO, 1>(d, dy, V, B, C, gamma, y, d_v, d_b, d_c, d_gamma, st);
        case 2: return diag_k<IO, 2>(d, dy, V, B, C, gamma, y, d_v, d_b, d_c, d_gamma, st);
        case 4: return diag_k<IO, 4>(d, dy, V, B, C, gamma, y, d_v, d_b, d_c, d_gamma, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_diag_fwd(const DiagShape& d, const void* V, const void* B, const void* C,
                           const float* gamma, void* y, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    return d.io == 1 ? diag_io<BF16>(d, nullptr, V, B, C, gamma, y, nullptr, nullptr, nullptr, nullptr, st)
                     : diag_io<F32>(d, nullptr, V, B, C, gamma, y, nullptr, nullptr, nullptr, nullptr, st);
}

hipError_t launch_diag_bwd(const DiagShape& d, const void* dy, const void* V, const void* B,
                           const void* C, const float* gamma, void* d_v, void* d_b, void* d_c,
                           float* d_gamma, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    return d.io == 1 ? diag_io<BF16>(d, dy, V, B, C, gamma, nullptr, d_v, d_b, d_c, d_gamma, st)
                     : diag_io<F32>(d, dy, V, B, C, gamma, nullptr, d_v, d_b, d_c, d_gamma, st);
}

}  // namespace ssd
