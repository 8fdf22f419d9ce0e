// Chunk-parallel MFMA kernels of the forward: K3 (chunk states) and K5 (chunk
// scan with K2 fused in, plus the D skip).  The backward reuses the K3 kernel
// for its BLUE state gradient (the same contraction with dy, C and exp(cum)).
//
// Page: burn-mamba "mamba2/ssd/serial_recalculated/combined_backward.rs".
//  - K3 (k3_ssd_chunk_state_extended): intra[p,r] = sum_t x[t,p] * b_scaled[t,r]
//    with b_scaled = B * dt * exp(cumA_last - cumA).
//  cumA is formed as A * cdt with cdt the fp64 cumsum of dt (K1).
//  - K5 is defined there by its backward: y = BLUE + ORANGE + D x with
//    BLUE[t,p]   = exp(cumA[t]) sum_r C[t,r] state[p,r]   (the chunk-entry state)
//    ORANGE[t,p] = sum_{s<=t} CB[t,s] exp(cumA[t] - cumA[s]) dt[s] x[s,p],
//    CB = C B^T (K2), the mask keeping s <= t (diagonal included).
//  - The backward's "d_chunk_input_state = C^T d_ch" with d_ch = dy * exp(cumA)
//    (BLUE backward) is job 1 of the state kernel.
//  - Job 2 is the same contraction for the state moments: T = X^T diag(v) B with
//    v_t = dt_t exp(cumA_t) phi_t (see k_moments.hip).
// The [l, l] CB and decay matrices never leave the chip: K5 builds each 16x16
// tile of CB^T with MFMA, scales it in registers and feeds it straight back to
// the next MFMA as its A operand.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ------------------------------------------------------------------ K3 / dS
// One workgroup per (chunk-head, job).  K (tokens) runs over 64-token blocks
// staged through LDS TRANSPOSED ([feature][token], the V rows pre-scaled by the
// token weight), so both MFMA operands are float4 reads along the contraction.
// Output [P, R] in 16x16 tiles: each wave owns whole 16-row p strips (its A
// operand is read once per k group and reused over all r tiles); with fewer than
// four p strips the r tiles of a strip are split between waves.
template <class IO, int P, int R>
__global__ __launch_bounds__(NT) void k_chunk_states(
    const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ Bm,
    const typename IO::T* __restrict__ dy, const typename IO::T* __restrict__ Cm,
    const float* __restrict__ dt, const float* __restrict__ Av, const double* __restrict__ cdt,
    float* __restrict__ S, float* __restrict__ dS, const double* __restrict__ phi,
    float* __restrict__ T, int N, int H, int L, int job0) {
    constexpr int TS = TB + 4;  // token stride of the transposed tiles
    __shared__ float sU[P * TS];
    __shared__ float sV[R * TS];
    __shared__ float sw[256];  // token weights of the chunk (L <= 256)
    const int job = job0 + static_cast<int>(blockIdx.y);
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const typename IO::T* U = job == 1 ? dy : x;
    const typename IO::T* V = job == 1 ? Cm : Bm;
    float* out = (job == 0 ? S : job == 1 ? dS : T) + c.ch * (P * R);
    const int64_t urow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t ustride = static_cast<int64_t>(H) * P;
    const int64_t vrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t vstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double end = cc[L - 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    constexpr int NPT = P / 16, NRT = R / 16;
    constexpr int PPW = NPT >= 4 ? NPT / 4 : 1;          // p strips per wave
    constexpr int WPS = NPT >= 4 ? 1 : 4 / NPT;          // waves per p strip
    constexpr int RPW = NRT >= WPS ? NRT / WPS : 1;      // r tiles per wave
    const int pt0 = NPT >= 4 ? wave : wave / WPS;
    const int rt0 = (NPT >= 4 ? 0 : wave % WPS) * RPW;
    const bool active = rt0 < NRT;
    v4f acc[PPW][RPW];
#pragma unroll
    for (int q = 0; q < PPW; ++q)
#pragma unroll
        for (int k = 0; k < RPW; ++k) acc[q][k] = zero4();

    // The chunk's token weights and block 0's rows first; then every block's
    // matrix work runs while the next block's rows load into registers.
    v4f tu[RowsT<IO, P>::IT], tv[RowsT<IO, R>::IT];
    load_rows_t<IO, P>(tu, U + urow0, ustride);
    load_rows_t<IO, R>(tv, V + vrow0, vstride);
    for (int t = tid; t < L; t += NT)
        sw[t] = job == 0   ? dtc[t] * expf(static_cast<float>(a * (end - cc[t])))
                : job == 1 ? expf(static_cast<float>(a * cc[t]))
                           : static_cast<float>(static_cast<double>(dtc[t]) * exp(a * cc[t]) *
                                                phi[c.c_bhn * L + t]);
    __syncthreads();
    for (int t0 = 0; t0 < L; t0 += TB) {
        store_rows_t<IO, P>(sU, tu, nullptr);
        store_rows_t<IO, R>(sV, tv, sw + t0);
        __syncthreads();
        if (t0 + TB < L) {
            load_rows_t<IO, P>(tu, U + urow0 + (t0 + TB) * ustride, ustride);
            load_rows_t<IO, R>(tv, V + vrow0 + (t0 + TB) * vstride, vstride);
        }
        if (active) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                v4f av[PPW];
#pragma unroll
                for (int q = 0; q < PPW; ++q)
                    av[q] = *reinterpret_cast<const v4f*>(sU + ((pt0 + 4 * q) * 16 + i) * TS + 16 * kk + 4 * g);
#pragma unroll
                for (int k = 0; k < RPW; ++k) {
                    const v4f bv = *reinterpret_cast<const v4f*>(sV + ((rt0 + k) * 16 + i) * TS + 16 * kk + 4 * g);
#pragma unroll
                    for (int q = 0; q < PPW; ++q)
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[q][k] = mfma16(av[q][v], bv[v], acc[q][k]);
                }
            }
        }
        __syncthreads();
    }
    if (active) {
#pragma unroll
        for (int q = 0; q < PPW; ++q)
#pragma unroll
            for (int k = 0; k < RPW; ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    out[((pt0 + 4 * q) * 16 + 4 * g + v) * R + (rt0 + k) * 16 + i] = acc[q][k][v];
    }
}

// The same contraction for bf16 io on the bf16 matrix cores.  The token weight goes on
// the U side, S = sum_t (w_t U_t)^T V_t: V (B or C) holds exact bf16 values and is staged
// transposed as bf16; w U (U = x or dy, the narrower operand) is an fp32 operand, staged
// as its three exact bf16 parts (split3).  Each 32-token slice is three 16x16x32 bf16
// MFMAs per output tile instead of eight fp32 ones; a wave reads its U parts once per
// slice and reuses them over its r tiles.  The token stride of the bf16 tiles is 72
// (144-byte rows: the 16-byte reads of 16 consecutive rows fall on distinct banks).
template <int P, int R>
__global__ __launch_bounds__(NT) void k_chunk_states_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ Cm,
    const float* __restrict__ dt, const float* __restrict__ Av, const double* __restrict__ cdt,
    float* __restrict__ S, float* __restrict__ dS, const double* __restrict__ phi,
    float* __restrict__ T, int N, int H, int L, int job0) {
    constexpr int TS = TB + 8;
    __shared__ __align__(16) uint16_t sU[3][P * TS];
    __shared__ __align__(16) uint16_t sV[R * TS];
    __shared__ float sw[256];  // token weights of the chunk (L <= 256)
    const int job = job0 + static_cast<int>(blockIdx.y);
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const uint16_t* U = job == 1 ? dy : x;
    const uint16_t* V = job == 1 ? Cm : Bm;
    float* out = (job == 0 ? S : job == 1 ? dS : T) + c.ch * (P * R);
    const int64_t urow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t ustride = static_cast<int64_t>(H) * P;
    const int64_t vrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t vstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double end = cc[L - 1];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    constexpr int NPT = P / 16, NRT = R / 16;
    constexpr int PPW = NPT >= 4 ? NPT / 4 : 1;
    constexpr int WPS = NPT >= 4 ? 1 : 4 / NPT;
    constexpr int RPW = NRT >= WPS ? NRT / WPS : 1;
    const int pt0 = NPT >= 4 ? wave : wave / WPS;
    const int rt0 = (NPT >= 4 ? 0 : wave % WPS) * RPW;
    const bool active = rt0 < NRT;
    v4f acc[PPW][RPW];
#pragma unroll
    for (int q = 0; q < PPW; ++q)
#pragma unroll
        for (int k = 0; k < RPW; ++k) acc[q][k] = zero4();

    using RU = RowsT<BF16, P>;
    using RV = RowsT<BF16, R>;
    v4f tu[RU::IT], tv[RV::IT];
    load_rows_t<BF16, P>(tu, U + urow0, ustride);
    load_rows_t<BF16, R>(tv, V + vrow0, vstride);
    for (int t = tid; t < L; t += NT)
        sw[t] = job == 0   ? dtc[t] * expf(static_cast<float>(a * (end - cc[t])))
                : job == 1 ? expf(static_cast<float>(a * cc[t]))
                           : static_cast<float>(static_cast<double>(dtc[t]) * exp(a * cc[t]) *
                                                phi[c.c_bhn * L + t]);
    __syncthreads();
    for (int t0 = 0; t0 < L; t0 += TB) {
#pragma unroll
        for (int it = 0; it < RU::IT; ++it) {
            const int idx = tid + it * NT;
            if (RU::TOTAL % NT == 0 || idx < RU::TOTAL) {
                const int row = RU::row(idx), c4 = RU::col4(idx);
                const float w = sw[t0 + row];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const Split3 sp = split3(tu[it][e] * w);
                    sU[0][(c4 * 4 + e) * TS + row] = sp.hi;
                    sU[1][(c4 * 4 + e) * TS + row] = sp.mid;
                    sU[2][(c4 * 4 + e) * TS + row] = sp.lo;
                }
            }
        }
#pragma unroll
        for (int it = 0; it < RV::IT; ++it) {
            const int idx = tid + it * NT;
            if (RV::TOTAL % NT == 0 || idx < RV::TOTAL) {
                const int row = RV::row(idx), c4 = RV::col4(idx);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sV[(c4 * 4 + e) * TS + row] = static_cast<uint16_t>(__float_as_uint(tv[it][e]) >> 16);
            }
        }
        __syncthreads();
        if (t0 + TB < L) {
            load_rows_t<BF16, P>(tu, U + urow0 + (t0 + TB) * ustride, ustride);
            load_rows_t<BF16, R>(tv, V + vrow0 + (t0 + TB) * vstride, vstride);
        }
        if (active) {
#pragma unroll
            for (int kk = 0; kk < TB / 32; ++kk) {
                b8v ah[PPW], am[PPW], al[PPW];
#pragma unroll
                for (int q = 0; q < PPW; ++q) {
                    const int o = ((pt0 + 4 * q) * 16 + i) * TS + 32 * kk + 8 * g;
                    ah[q] = *reinterpret_cast<const b8v*>(sU[0] + o);
                    am[q] = *reinterpret_cast<const b8v*>(sU[1] + o);
                    al[q] = *reinterpret_cast<const b8v*>(sU[2] + o);
                }
#pragma unroll
                for (int k = 0; k < RPW; ++k) {
                    const b8v bv = *reinterpret_cast<const b8v*>(sV + ((rt0 + k) * 16 + i) * TS + 32 * kk + 8 * g);
#pragma unroll
                    for (int q = 0; q < PPW; ++q) {
                        // the smallest part first into the fp32 accumulator
                        acc[q][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[q], bv, acc[q][k], 0, 0, 0);
                        acc[q][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[q], bv, acc[q][k], 0, 0, 0);
                        acc[q][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[q], bv, acc[q][k], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
    }
    if (active) {
#pragma unroll
        for (int q = 0; q < PPW; ++q)
#pragma unroll
            for (int k = 0; k < RPW; ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    out[((pt0 + 4 * q) * 16 + 4 * g + v) * R + (rt0 + k) * 16 + i] = acc[q][k][v];
    }
}

// ------------------------------------------------------------------------- K5
// One workgroup per (chunk-head, 64-token target block tb); wave w owns target
// rows t = 16w .. 16w+15 of the block and keeps its C rows in registers.
//   BLUE:   acc[t, p] = exp(cum[t]) sum_r C[t,r] S_in[p,r]
//   ORANGE: for every source block sb <= tb and 16-token source tile j,
//           CB^T[s, t] = sum_r B[s,r] C[t,r]  (MFMA; lane holds t = i, s = 4g+v),
//           W[t, s] = CB * exp(cum[t] - cum[s]) * dt[s]  (s <= t),
//           acc[t, p] += sum_s W[t,s] x[s,p]  (the W registers are the A operand).
//   y = acc + D x.
template <class IO, int P, int R>
__global__ __launch_bounds__(NT, 2) void k5_chunk_scan(
    const typename IO::T* __restrict__ x, const float* __restrict__ dt,
    const typename IO::T* __restrict__ Bm, const typename IO::T* __restrict__ Cm,
    const float* __restrict__ Av, const float* __restrict__ Dv, const double* __restrict__ cdt,
    const float* __restrict__ S, typename IO::T* __restrict__ y, int N, int H, int L, int64_t CH) {
    constexpr int RS = R + 4, PS = P + 4;
    constexpr int ROWS = P > TB ? P : TB;
    __shared__ float sBS[ROWS * RS];  // S_in [P, R] for BLUE, then B of the source block
    __shared__ float sX[TB * PS];
    __shared__ double sCumT[TB];
    __shared__ __align__(16) double sCumS[TB];
    __shared__ __align__(16) float sDt[TB];
    const int nblk = L / TB;
    const int tb = nblk - 1 - static_cast<int>(blockIdx.x / CH);  // heaviest blocks first
    const ChunkHead c = decode_ch(blockIdx.x % CH, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const int tl = 16 * wave + i;  // this lane's target row inside the block (operand layout)

    v4f creg[R / 16];
    {
        const int64_t row = brow0 + static_cast<int64_t>(tb * TB + tl) * bstride;
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) creg[kk] = io<IO>::ld4(Cm, row + 16 * kk + 4 * g);
    }
    stage_mat<R, P>(sBS, S + c.ch * (P * R));
    if (tid < TB) sCumT[tid] = cc[tb * TB + tid];
    __syncthreads();

    v4f acc[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) acc[pt] = zero4();
    // BLUE: A = C rows (k = r), B operand = S_in[p, r] read along r
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const v4f bop = *reinterpret_cast<const v4f*>(sBS + (pt * 16 + i) * RS + 16 * kk + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[pt] = mfma16(creg[kk][v], bop[v], acc[pt]);
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float e = expf(static_cast<float>(a * sCumT[16 * wave + 4 * g + v]));
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[pt][v] *= e;
    }

    const double ct = sCumT[tl];
    const double la2 = a * kLog2e;
    for (int sb = 0; sb <= tb; ++sb) {
        __syncthreads();
        double cnext = 0.0;
        float dnext = 0.0f;
        if (tid < TB) {
            cnext = cc[sb * TB + tid];
            dnext = dtc[sb * TB + tid];
        }
        stage_rows2<IO, R, P>(sBS, Bm + brow0 + static_cast<int64_t>(sb * TB) * bstride, bstride,
                              sX, x + xrow0 + static_cast<int64_t>(sb * TB) * xstride, xstride);
        if (tid < TB) {
            sCumS[tid] = cnext;
            sDt[tid] = dnext;
        }
        __syncthreads();
        const int jmax = (sb == tb) ? wave : 3;  // diagonal block: s-tiles up to this wave's
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > jmax) break;
            v4f cbt = zero4();
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) {
                const v4f aop = *reinterpret_cast<const v4f*>(sBS + (16 * j + i) * RS + 16 * kk + 4 * g);
                cbt = mfma_k16<IO>(aop, creg[kk], cbt);
            }
            // this lane's four source rows: cumsums and dt as 16-byte LDS reads
            const v2d cs01 = *reinterpret_cast<const v2d*>(sCumS + 16 * j + 4 * g);
            const v2d cs23 = *reinterpret_cast<const v2d*>(sCumS + 16 * j + 4 * g + 2);
            const v4f dts = *reinterpret_cast<const v4f*>(sDt + 16 * j + 4 * g);
            const double csv[4] = {cs01.x, cs01.y, cs23.x, cs23.y};
            float wv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool keep = (sb < tb) || (16 * j + 4 * g + v <= tl);
                // masked pairs (s > t) take gap 0 and weight 0: arithmetic, not a branch
                const double gap = keep ? ct - csv[v] : 0.0;
                wv[v] = cbt[v] * exp2_of(la2 * gap) * dts[v] * (keep ? 1.0f : 0.0f);
            }
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[pt] = mfma16(wv[v], sX[(16 * j + 4 * g + v) * PS + pt * 16 + i], acc[pt]);
            }
        }
    }
    // sX now holds x of the target block (the last source block is tb itself).
    const float Dh = Dv[c.h];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int t = 16 * wave + 4 * g + v;
        const int64_t row = xrow0 + static_cast<int64_t>(tb * TB + t) * xstride;
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const float val = acc[pt][v] + Dh * sX[t * PS + pt * 16 + i];
            io<IO>::st(y, row + pt * 16 + i, val);
        }
    }
}

// ------------------------------------------------------------------ dispatch
#define SSD_FOR_EACH_PR(X) \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) \
    X(128, 16) X(128, 32) X(128, 64) X(128, 128)

template <class IO>
static hipError_t states_io(const Shape& s, bool js, bool jd, const void* x, const void* Bm,
                            const void* dy, const void* Cm, const float* dt, const float* A,
                            const double* cdt, float* S, float* dS, const double* phi,
                            float* Tm, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    const bool jm = phi && Tm;
    if (CH == 0 || (!js && !jd && !jm)) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH), jm ? 1u : (js && jd) ? 2u : 1u);
    const int job0 = jm ? 2 : js ? 0 : 1;
#define X(PP, RR)                                                                                \
    if (s.P == PP && s.R == RR) {                                                                \
        if constexpr (sizeof(T) == 2)                                                            \
            hipLaunchKernelGGL((k_chunk_states_bf16<PP, RR>), grid, dim3(NT), 0, st,             \
                               static_cast<const T*>(x), static_cast<const T*>(Bm),              \
                               static_cast<const T*>(dy), static_cast<const T*>(Cm), dt, A, cdt, \
                               S, dS, phi, Tm, s.N, s.H, s.L, job0);                             \
        else                                                                                     \
            hipLaunchKernelGGL((k_chunk_states<IO, PP, RR>), grid, dim3(NT), 0, st,             \
                               static_cast<const T*>(x), static_cast<const T*>(Bm),              \
                               static_cast<const T*>(dy), static_cast<const T*>(Cm), dt, A, cdt, \
                               S, dS, phi, Tm, s.N, s.H, s.L, job0);                             \
        return hipGetLastError();                                                                \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_states(const Shape& s, bool job_state, bool job_dstate, const void* x,
                               const void* Bm, const void* dy, const void* Cm, const float* dt,
                               const float* A, const double* cdt, float* S, float* dS,
                               hipStream_t st, const double* phi, float* T) {
    return s.io == 1
               ? states_io<BF16>(s, job_state, job_dstate, x, Bm, dy, Cm, dt, A, cdt, S, dS, phi, T, st)
               : states_io<F32>(s, job_state, job_dstate, x, Bm, dy, Cm, dt, A, cdt, S, dS, phi, T, st);
}

template <class IO>
static hipError_t k5_io(const Shape& s, const void* x, const float* dt, const void* Bm,
                        const void* Cm, const float* A, const float* D, const double* cdt,
                        const float* S, void* y, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH * s.nblk()));
#define X(PP, RR)                                                                              \
    if (s.P == PP && s.R == RR) {                                                              \
        hipLaunchKernelGGL((k5_chunk_scan<IO, PP, RR>), grid, dim3(NT), 0, st,                \
                           static_cast<const T*>(x), dt, static_cast<const T*>(Bm),            \
                           static_cast<const T*>(Cm), A, D, cdt, S, static_cast<T*>(y), s.N, s.H, \
                           s.L, CH);                                                           \
        return hipGetLastError();                                                              \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_k5_scan(const Shape& s, const void* x, const float* dt, const void* Bm,
                          const void* Cm, const float* A, const float* D, const double* cdt,
                          const float* S, void* y, hipStream_t st) {
    if (wide_supported(s)) return launch_k5_scan_wide(s, x, dt, Bm, Cm, A, D, cdt, S, y, st);
    return s.io == 1 ? k5_io<BF16>(s, x, dt, Bm, Cm, A, D, cdt, S, y, st)
                     : k5_io<F32>(s, x, dt, Bm, Cm, A, D, cdt, S, y, st);
}

}  // namespace ssd
