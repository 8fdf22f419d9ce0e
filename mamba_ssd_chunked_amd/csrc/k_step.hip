// Decode step of the Mamba-2 SSD: one token of the recurrence from a cached state.
//
// The chunked scan (burn-mamba "mamba2/ssd/serial_recalculated/
// combined_backward.rs") computes the recurrence h_t = exp(dt_t A) h_{t-1} +
// dt_t x_t (outer) B_t, y_t = C_t . h_t + D x_t for a whole sequence; a decoder
// runs it one token at a time, reading and writing the state it caches (the
// token-by-token `step` loop the burn-mamba "modules/state_moments.rs" page
// refers to).  Per (b, h) slice with state S [p, r]:
//   S' = exp(dt A) S + dt x (outer) B,    y = S' C + D x.
//
// Two flops per state element against 8 bytes of state traffic (read + write):
// bound by HBM, no matrix cores.  One workgroup per (b, h) slice: thread t owns
// column group c4 = t % (r / 4) of the rows t / (r / 4) + k * (256 / (r / 4)), so
// a wave reads contiguous state, a state row (r / 4 float4s) is held by r / 4
// consecutive lanes of one wave, which reduce their partial dot products with C
// by butterflies (the row's first lane writes y), and each thread loads its
// slices of B and C once (reloading them per row cost 1.23x the algorithmic
// HBM reads).  All of a thread's state loads are issued before the first use.
// The decay exponent is formed in fp64 and raised once in fp32; the state stays
// fp32, x, B, C, y are the io dtype.  The state may be updated in place: each
// element is read and written by the same thread.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

__device__ __forceinline__ float dot4(v4f a, v4f b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

}  // namespace

// R4 = dstate / 4: lanes per state row; P = headdim.
template <class IO, int R4, int P>
__global__ __launch_bounds__(NT) void k_step(const typename IO::T* __restrict__ x,
                                             const float* __restrict__ dt,
                                             const float* __restrict__ A,
                                             const typename IO::T* __restrict__ Bm,
                                             const typename IO::T* __restrict__ Cm,
                                             const float* __restrict__ D, const float* state,
                                             float* new_state, typename IO::T* __restrict__ y,
                                             int H) {
    constexpr int ROWS = NT / R4;                         // rows per pass of the workgroup
    constexpr int K = P > ROWS ? P / ROWS : 1;            // passes
    const int64_t slice = blockIdx.x;                     // (b, h)
    const int c4 = threadIdx.x % R4;
    const int r0 = threadIdx.x / R4;
    const int h = static_cast<int>(slice % H);
    const float dtv = dt[slice];
    const float a = exp2_of(static_cast<double>(dtv) * static_cast<double>(A[h]) * kLog2e);
    const float dh = D[h];
    const v4f bv = io<IO>::ld4(Bm, slice * (4 * R4) + 4 * c4);
    const v4f cv = io<IO>::ld4(Cm, slice * (4 * R4) + 4 * c4);
    const v4f* src = reinterpret_cast<const v4f*>(state) + slice * P * R4;
    v4f* dst = reinterpret_cast<v4f*>(new_state) + slice * P * R4;
    v4f s[K];
    float xv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int pp = r0 + k * ROWS;
        if (pp < P) {
            s[k] = __builtin_nontemporal_load(src + pp * R4 + c4);
            xv[k] = io<IO>::ld(x, slice * P + pp);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int pp = r0 + k * ROWS;
        if (pp < P) {  // whole rows are in or out together
            const v4f n = a * s[k] + (dtv * xv[k]) * bv;
            __builtin_nontemporal_store(n, dst + pp * R4 + c4);
            float part = dot4(cv, n);
#pragma unroll
            for (int o = R4 / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
            if (c4 == 0) io<IO>::st(y, slice * P + pp, part + dh * xv[k]);
        }
    }
}

namespace {

template <class IO, int R4>
hipError_t step_r(const StepShape& s, const void* x, const float* dt, const float* A, const void* B,
                  const void* C, const float* D, const float* state, float* new_state, void* y,
                  hipStream_t st) {
    using T = typename IO::T;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(s.B) * s.H)), block(NT);
    const T* xx = static_cast<const T*>(x);
    const T* bb = static_cast<const T*>(B);
    const T* cc = static_cast<const T*>(C);
    T* yy = static_cast<T*>(y);
    switch (s.P) {
        case 16: k_step<IO, R4, 16><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, s.H); break;
        case 32: k_step<IO, R4, 32><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, s.H); break;
        case 64: k_step<IO, R4, 64><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, s.H); break;
        case 128: k_step<IO, R4, 128><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, s.H); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class IO>
hipError_t step_io(const StepShape& s, const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* state,
                   float* new_state, void* y, hipStream_t st) {
    switch (s.R) {
        case 16: return step_r<IO, 4>(s, x, dt, A, B, C, D, state, new_state, y, st);
        case 32: return step_r<IO, 8>(s, x, dt, A, B, C, D, state, new_state, y, st);
        case 64: return step_r<IO, 16>(s, x, dt, A, B, C, D, state, new_state, y, st);
        case 128: return step_r<IO, 32>(s, x, dt, A, B, C, D, state, new_state, y, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_step(const StepShape& s, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* state,
                       float* new_state, void* y, hipStream_t st) {
    return s.io == 1 ? step_io<BF16>(s, x, dt, A, B, C, D, state, new_state, y, st)
                     : step_io<F32>(s, x, dt, A, B, C, D, state, new_state, y, st);
}

}  // namespace ssd
