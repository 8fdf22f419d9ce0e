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
// bound by HBM, no matrix cores.  The state of every slice is one stream of
// float4s; thread f takes float4 f, so a wave reads 1 KB of contiguous state,
// and a state row (r / 4 float4s) is held by r / 4 consecutive lanes of one wave,
// which reduce their partial dot products with C by butterflies; the row's first
// lane writes y.  The decay exponent is formed in fp64 and raised once in fp32;
// the state stays fp32, x, B, C, y are the io dtype.  The state may be updated in
// place: each element is read and written by the same thread.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

__device__ __forceinline__ float dot4(v4f a, v4f b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

}  // namespace

// R4 = dstate / 4: lanes per state row.
template <class IO, int R4>
__global__ __launch_bounds__(NT) void k_step(const typename IO::T* __restrict__ x,
                                             const float* __restrict__ dt,
                                             const float* __restrict__ A,
                                             const typename IO::T* __restrict__ Bm,
                                             const typename IO::T* __restrict__ Cm,
                                             const float* __restrict__ D, const float* state,
                                             float* new_state, typename IO::T* __restrict__ y,
                                             int64_t total4, int H, int P) {
    const int64_t f = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (f >= total4) return;  // whole rows leave together (total4 and NT are multiples of R4)
    const int64_t row = f / R4;    // (b, h, p)
    const int c4 = static_cast<int>(f % R4);
    const int64_t slice = row / P;  // (b, h)
    const int pp = static_cast<int>(row % P);
    const int h = static_cast<int>(slice % H);
    const float dtv = dt[slice];
    const float a = exp2_of(static_cast<double>(dtv) * static_cast<double>(A[h]) * kLog2e);
    const float xv = io<IO>::ld(x, slice * P + pp);
    const v4f bv = io<IO>::ld4(Bm, slice * (4 * R4) + 4 * c4);
    const v4f cv = io<IO>::ld4(Cm, slice * (4 * R4) + 4 * c4);
    v4f s = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(state) + f);
    s = a * s + (dtv * xv) * bv;
    __builtin_nontemporal_store(s, reinterpret_cast<v4f*>(new_state) + f);
    float part = dot4(cv, s);
#pragma unroll
    for (int o = R4 / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (c4 == 0) io<IO>::st(y, slice * P + pp, part + D[h] * xv);
}

namespace {

template <class IO>
hipError_t step_io(const StepShape& s, const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* state,
                   float* new_state, void* y, hipStream_t st) {
    using T = typename IO::T;
    const int64_t total4 = static_cast<int64_t>(s.B) * s.H * s.P * (s.R / 4);
    const dim3 grid(static_cast<unsigned>((total4 + NT - 1) / NT)), block(NT);
    const T* xx = static_cast<const T*>(x);
    const T* bb = static_cast<const T*>(B);
    const T* cc = static_cast<const T*>(C);
    T* yy = static_cast<T*>(y);
    switch (s.R) {
        case 16: k_step<IO, 4><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, total4, s.H, s.P); break;
        case 32: k_step<IO, 8><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, total4, s.H, s.P); break;
        case 64: k_step<IO, 16><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, total4, s.H, s.P); break;
        case 128: k_step<IO, 32><<<grid, block, 0, st>>>(xx, dt, A, bb, cc, D, state, new_state, yy, total4, s.H, s.P); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepShape& s, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* state,
                       float* new_state, void* y, hipStream_t st) {
    return s.io == 1 ? step_io<BF16>(s, x, dt, A, B, C, D, state, new_state, y, st)
                     : step_io<F32>(s, x, dt, A, B, C, D, state, new_state, y, st);
}

}  // namespace ssd
