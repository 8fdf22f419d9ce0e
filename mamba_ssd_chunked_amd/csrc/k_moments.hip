// Pooled state moments (forward) and their gradient, chunk-parallel and without
// materialising any per-token state.
//
// Pages: burn-mamba "modules/state_moments.rs" (StateMoments: m2 = sum_t h_t^T h_t,
// m1 = sum_t sum_p h_t[p,:], count = valid tokens * per_head_dim) and the
// "mamba3/moments/backward" module page (Gradient math: per-token cotangent
// d_c[t] = mask_t (c_t (d_m2 + d_m2^T) + d_m1), the carry d_h+ into the chunk's
// last state, d_W_j = sum_t L[t,j] G[t], and the decay gradient), here with the
// rotation equal to the identity; "state_moments.rs" notes the Mamba-2 moments
// have a closed form with no state materialisation.  The closed form used:
//
// Per chunk with entry state H (K4 output), positions t, s in [0, l), c = cdt
// (fp64 cumsum of dt), a = A, mask M_t = (chunk start + t < valid_len):
//   e_t = exp(a c_t),  Lp[t,s] = exp(a (c_t - c_s)) (s <= t),  L = Lp diag(dt)
//   h_t = e_t H + sum_{s<=t} L[t,s] x_s B_s^T
//   phi_m = sum_{t>=m} M_t exp(2a (c_t - c_m)),  psi_m = sum_{t>=m} M_t exp(a (c_t - c_m))
//   K[s,s'] = sum_t M_t L[t,s] L[t,s'] = dt_s dt_s' exp(a |c_s - c_s'|) phi_max(s,s')
//   v_s = sum_t M_t e_t L[t,s] = dt_s e_s phi_s,  u_s = sum_t M_t L[t,s] = dt_s psi_s
//   c2 = sum_t M_t e_t^2 = e_0^2 phi_0,  c1 = sum_t M_t e_t = e_0 psi_0
//   G = X X^T,  T = X^T diag(v) B
//   m2 += B^T (K o G) B + H^T T + T^T H + c2 H^T H
//   m1 += c1 colsum(H) + sum_s u_s (1^T x_s) B_s
// Backward of <d_m2, m2> + <d_m1, m1>, S = d_m2 + d_m2^T, d_h+ = gradient of the
// chunk's last state from later chunks (the K4 reverse carry), Qb = B S B^T,
// N = G o Qb, eta_s = x_s^T H S B_s, zeta_s = (1^T x_s)(d_m1 . B_s):
//   d_H (chunk-local, into the K4 carry) = (c2 H + T) S + c1 1 d_m1^T
//   d_x_s  = v_s (H S) B_s + sum_s' K[s,s'] Qb[s,s'] x_s' + u_s (d_m1.B_s) 1 + bbar_s d_h+ B_s
//   d_B_s  = v_s S H^T x_s + sum_s' K[s,s'] G[s,s'] S B_s' + u_s (1^T x_s) d_m1 + bbar_s d_h+^T x_s
//   d_dt_s = ddtW_s + a sum_{k>=s} dac_k, with
//   ddtW_s = e_s phi_s eta_s + sum_s' (K[s,s']/dt_s) N[s,s'] + psi_s zeta_s + de_s x_s^T d_h+ B_s
//   dac_k  = M_k (<S, h_k^T h_k> + d_m1 . colsum(h_k)) - dt_k ddtW_k (+ <d_h+, h_{l-1}> at k = l-1)
//   <S, h_k^T h_k> = e_k^2 <H, HS> + 2 e_k lambda_k + tau_k, where
//     lambda_k = sum_{s<=k} L[k,s] eta_s  and  tau_k = sum_{s,s'<=k} L[k,s] L[k,s'] N[s,s']
//   follow first-order recurrences (tau_k = exp(2a dt_k) tau_{k-1} + 2 dt_k rho_k with
//   rho_k = sum_{s<k} L[k,s] N[k,s] + dt_k N[k,k] / 2).
//   d_A equals sum_k c_k dac_k, but that sum cancels badly in fp32, so it is taken
//   term by term against the dt span each exponent covers (with the scans
//   phit_m = sum_{t>=m} M_t (c_t - c_m) exp(2a (c_t - c_m)) and psit likewise):
//     d_A = <H,HS> e_0^2 (phit_0 + c_0 phi_0) + sum_s eta_s dt_s e_s (2 phit_s + c_s phi_s)
//         + sum_{s,s'} N dt_s dt_s' exp(a |c_s - c_s'|) (phit_max + |c_s - c_s'| phi_max / 2)
//         + hdm e_0 (psit_0 + c_0 psi_0) + sum_s zeta_s dt_s psit_s
//         + c_{l-1} e_{l-1} <d_h+, H> + sum_s (c_{l-1} - c_s) bbar_s x_s^T d_h+ B_s.
// (de_s = exp(a (c_{l-1} - c_s)), bbar_s = dt_s de_s.)  Every sum over time has
// collapsed into per-chunk pair weights and O(l) scans, so the work is O(l^2 (p + r))
// per chunk instead of O(l p r^2) for the per-token states.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Valid tokens of chunk n of batch b.
__device__ __forceinline__ int chunk_valid(const int64_t* valid, int64_t b, int n, int L) {
    const int64_t v = valid[b] - static_cast<int64_t>(n) * L;
    return v <= 0 ? 0 : (v >= L ? L : static_cast<int>(v));
}

// Wave-level scans over one chunk.  Lane j owns positions j*E .. j*E+E-1 (E <= 4)
// and passes its c values.  Reverse: y_t = m_t + exp(ka (c_{t+1} - c_t)) y_{t+1},
// y_L = 0.  Forward: y_t = exp(ka (c_t - c_{t-1})) y_{t-1} + q_t, y_{-1} = 0.
// Both combine per-lane affine maps with a Hillis-Steele scan.
__device__ void wave_rev_scan(const double* c, const double* m, double ka, int E, int lane,
                              double* out) {
    double yl[4];
    double y = 0.0;
#pragma unroll
    for (int e = 3; e >= 0; --e)
        if (e < E) {
            if (e < E - 1) y *= exp(ka * (c[e + 1] - c[e]));
            y += m[e];
            yl[e] = y;
        }
    const double cnext = __shfl_down(c[0], 1);
    double mu = (lane < 63) ? exp(ka * (cnext - c[0])) : 0.0;
    double b = yl[0];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double mu2 = __shfl_down(mu, off), b2 = __shfl_down(b, off);
        if (lane + off < 64) {
            b = b + mu * b2;
            mu = mu * mu2;
        }
    }
    double ynext = __shfl_down(b, 1);
    if (lane == 63) ynext = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) out[e] = yl[e] + (lane < 63 ? exp(ka * (cnext - c[e])) * ynext : 0.0);
}

__device__ void wave_fwd_scan(const double* c, const double* q, double ka, int E, int lane,
                              double* out) {
    double yl[4];
    double y = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) {
            if (e > 0) y *= exp(ka * (c[e] - c[e - 1]));
            y += q[e];
            yl[e] = y;
        }
    const double cprev = __shfl_up(c[E - 1], 1);
    double nu = (lane > 0) ? exp(ka * (c[E - 1] - cprev)) : 0.0;
    double b = yl[E - 1];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double nu2 = __shfl_up(nu, off), b2 = __shfl_up(b, off);
        if (lane >= off) {
            b = b + nu * b2;
            nu = nu * nu2;
        }
    }
    double yprev = __shfl_up(b, 1);
    if (lane == 0) yprev = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) out[e] = yl[e] + (lane > 0 ? exp(ka * (c[e] - cprev)) * yprev : 0.0);
}

// ------------------------------------------------------------------ phi, psi
__global__ __launch_bounds__(NT) void km_phi(const double* __restrict__ cdt,
                                              const float* __restrict__ A,
                                              const int64_t* __restrict__ valid,
                                              double* __restrict__ phi, double* __restrict__ psi,
                                              double* __restrict__ phit, double* __restrict__ psit,
                                              int64_t nchunks_total, int H, int N, int L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (c >= nchunks_total) return;
    const int n = static_cast<int>(c % N);
    const int h = static_cast<int>((c / N) % H);
    const int64_t b = c / (static_cast<int64_t>(N) * H);
    const double a = static_cast<double>(A[h]);
    const int vl = chunk_valid(valid, b, n, L);
    const int E = L >> 6;
    double cv[4], m[4], mc[4], o1[4], o2[4], o3[4], o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = lane * E + e;
        cv[e] = e < E ? cdt[c * L + t] : 0.0;
        m[e] = (e < E && t < vl) ? 1.0 : 0.0;
        mc[e] = m[e] * cv[e];
    }
    wave_rev_scan(cv, m, 2.0 * a, E, lane, o1);
    wave_rev_scan(cv, m, a, E, lane, o2);
    wave_rev_scan(cv, mc, 2.0 * a, E, lane, o3);
    wave_rev_scan(cv, mc, a, E, lane, o4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < E) {
            const int64_t o = c * L + lane * E + e;
            phi[o] = o1[e];
            psi[o] = o2[e];
            phit[o] = o3[e] - cv[e] * o1[e];  // fp64: c <= a few hundred, no harmful cancellation
            psit[o] = o4[e] - cv[e] * o2[e];
        }
}

hipError_t launch_km_phi(const Shape& s, const double* cdt, const float* A, const int64_t* valid,
                         double* phi, double* psi, double* phit, double* psit, hipStream_t st) {
    const int64_t nc = s.chunks();
    if (nc == 0) return hipSuccess;
    hipLaunchKernelGGL(km_phi, dim3(static_cast<unsigned>((nc + 3) / 4)), dim3(NT), 0, st, cdt, A,
                       valid, phi, psi, phit, psit, nc, s.H, s.N, s.L);
    return hipGetLastError();
}

// ------------------------------------------------------------- forward rows
// One workgroup per (chunk-head, 64-row block sb); wave w owns rows s = 16w + i.
//   Z[s, :] = sum_{s'} K[s,s'] G[s,s'] B_s'   over all s' of the chunk
//   U_blk   = sum_{s in block} B_s Z_s^T      (r x r, written as a partial)
//   m1_blk  = sum_{s in block} u_s (1^T x_s) B_s
template <class IO, int P, int R>
__global__ __launch_bounds__(NT, 2) void km_fwd_rows(
    const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ Bm,
    const float* __restrict__ dt, const float* __restrict__ Av, const double* __restrict__ cdt,
    const double* __restrict__ phi, const double* __restrict__ psi, float* __restrict__ U,
    float* __restrict__ m1b, int N, int H, int L, int64_t CH) {
    constexpr int RS = R + 4, PS = P + 4;
    __shared__ float sX[TB * PS];  // X of the partner block
    __shared__ float sB[TB * RS];  // B of the partner block, then B of the own block
    __shared__ float sZ[TB * RS];  // Z rows of the own block
    __shared__ double sC[TB], sPhi[TB];
    __shared__ float sDt[TB], sUx[TB];
    const int nblk = L / TB;
    const int sb = static_cast<int>(blockIdx.x / CH);
    const ChunkHead c = decode_ch(blockIdx.x % CH, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double* ph = phi + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double la2 = a * kLog2e;
    const int sl = 16 * wave + i, spos = sb * TB + sl;

    v4f xreg[P / 16];
    {
        const int64_t row = xrow0 + static_cast<int64_t>(spos) * xstride;
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) xreg[kk] = io<IO>::ld4(x, row + 16 * kk + 4 * g);
    }
    const double cs = cc[spos], phs = ph[spos];
    const float dts = dtc[spos];

    v4f z[R / 16];
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) z[rt] = zero4();
    // Partner blocks in the order sb + 1, ..., nblk - 1, 0, ..., sb: the last one
    // staged is the own block, whose B rows the U product below reads from sB.
    // Each block's rows load into registers while the previous block's tiles run.
    v4f preX[RowTiles<P, TB>::IT], preB[RowTiles<R, TB>::IT];
    double pc = 0.0, pp = 0.0;
    float pd = 0.0f;
    auto load_block = [&](int b2) {
        load_rows<IO, P, TB>(preX, x + xrow0 + static_cast<int64_t>(b2 * TB) * xstride, xstride);
        load_rows<IO, R, TB>(preB, Bm + brow0 + static_cast<int64_t>(b2 * TB) * bstride, bstride);
        if (tid < TB) {
            pc = cc[b2 * TB + tid];
            pp = ph[b2 * TB + tid];
            pd = dtc[b2 * TB + tid];
        }
    };
    auto block_at = [&](int k) { return sb + 1 + k < nblk ? sb + 1 + k : sb + 1 + k - nblk; };
    load_block(block_at(0));
    for (int k = 0; k < nblk; ++k) {
        const int b2 = block_at(k);
        __syncthreads();
        store_rows<P, TB>(sX, preX);
        store_rows<R, TB>(sB, preB);
        if (tid < TB) {
            sC[tid] = pc;
            sPhi[tid] = pp;
            sDt[tid] = pd;
        }
        __syncthreads();
        if (k + 1 < nblk) load_block(block_at(k + 1));
        for (int j = 0; j < 4; ++j) {
            // G^T tile: M = s' (16j + 4g + v), N = s
            v4f gt = zero4();
#pragma unroll
            for (int kk = 0; kk < P / 16; ++kk) {
                const v4f u = *reinterpret_cast<const v4f*>(sX + (16 * j + i) * PS + 16 * kk + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) gt = mfma16(u[v], xreg[kk][v], gt);
            }
            float q[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int sp = 16 * j + 4 * g + v;          // partner row in its block
                const int ppos = b2 * TB + sp;              // ... in the chunk
                const double cp = sC[sp];
                const bool pm = ppos >= spos;               // partner is the later one
                const double gap = pm ? cp - cs : cs - cp;
                const double phm = pm ? sPhi[sp] : phs;
                const float kv = dts * sDt[sp] * exp2_of(la2 * gap) * static_cast<float>(phm);
                q[v] = kv * gt[v];
            }
            // Z[s, r] += sum_{s'} Q[s, s'] B[s', r]
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    z[rt] = mfma16(q[v], sB[(16 * j + 4 * g + v) * RS + rt * 16 + i], z[rt]);
            }
        }
    }
    __syncthreads();
    // own block: its B rows are in sB already; Z rows into sZ, u_s (1^T x_s) into sUx
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sZ[(16 * wave + 4 * g + v) * RS + rt * 16 + i] = z[rt][v];
    {
        float xs = 0.f;
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) xs += xreg[kk][0] + xreg[kk][1] + xreg[kk][2] + xreg[kk][3];
        xs = sum_over_g(xs);
        if (g == 0) sUx[sl] = static_cast<float>(static_cast<double>(dts) * psi[c.c_bhn * L + spos]) * xs;
    }
    __syncthreads();
    // U[r1, r2] = sum_s B[s, r1] Z[s, r2]; wave w takes the 16-row strips r1t = w, w + 4, ...
    // with all their column tiles at once (independent accumulator chains; one tile at a
    // time made every MFMA wait for the one before it)
    constexpr int NTR = R / 16;
    float* Uo = U + (c.ch * nblk + sb) * static_cast<int64_t>(R * R);
    for (int r1t = wave; r1t < NTR; r1t += 4) {
        v4f acc[NTR];
#pragma unroll
        for (int r2t = 0; r2t < NTR; ++r2t) acc[r2t] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int s_ = 16 * kk + 4 * g + v;
                const float av = sB[s_ * RS + r1t * 16 + i];
#pragma unroll
                for (int r2t = 0; r2t < NTR; ++r2t)
                    acc[r2t] = mfma16(av, sZ[s_ * RS + r2t * 16 + i], acc[r2t]);
            }
#pragma unroll
        for (int r2t = 0; r2t < NTR; ++r2t)
#pragma unroll
            for (int v = 0; v < 4; ++v) Uo[(r1t * 16 + 4 * g + v) * R + r2t * 16 + i] = acc[r2t][v];
    }
    float* mo = m1b + (c.ch * nblk + sb) * static_cast<int64_t>(R);
    for (int r = tid; r < R; r += NT) {
        float acc = 0.f;
        for (int s_ = 0; s_ < TB; ++s_) acc += sUx[s_] * sB[s_ * RS + r];
        mo[r] = acc;
    }
}

// ---------------------------------------------------------------- per chunk
// Rows of a [rows, K] fp32 matrix (16 per wave) times a SYMMETRIC LDS matrix [K, NC] (stride
// lds_ld): out tiles in the MFMA result layout.  The B operand S[k][col] for k = 16 kk + 4 g + v
// is read as S[col][16 kk + 4 g .. + 3], one float4 per k group instead of four scalars.
template <int K, int NC>
__device__ __forceinline__ void rows_x_sym_lds(const v4f* areg, const float* lds, int lds_ld, v4f* acc,
                                               int i, int g) {
#pragma unroll
    for (int kk = 0; kk < K / 16; ++kk)
#pragma unroll
        for (int nt = 0; nt < NC / 16; ++nt) {
            const v4f b = *reinterpret_cast<const v4f*>(lds + (nt * 16 + i) * lds_ld + 16 * kk + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[nt] = mfma16(areg[kk][v], b[v], acc[nt]);
        }
}

// FWD selects the forward (dm2 == nullptr) or the backward instance: separate kernels, so that
// each allocates only its own LDS (the backward's 17 KB at r = 64 instead of the forward's 35 KB
// lets every chunk-head of the moments workload run in one round of the machine).
template <class IO, int P, int R, bool FWD>
__global__ __launch_bounds__(NT, (FWD || R > 64) ? 1 : 3) void km_chunk(
    const float* __restrict__ Sin, const float* __restrict__ Tm, const double* __restrict__ cdt,
    const float* __restrict__ Av, const double* __restrict__ phi, const double* __restrict__ psi,
    float* __restrict__ W, float* __restrict__ m1c, const float* __restrict__ dm2,
    const float* __restrict__ dm1, const typename IO::T* __restrict__ Bm, float* __restrict__ HS,
    float* __restrict__ dSl, float* __restrict__ BS, double* __restrict__ hsh,
    double* __restrict__ hdm, int N, int H, int L) {
    constexpr int RS = R + 4;
    __shared__ __align__(16) float sA[(FWD ? P : R) * RS];  // fwd: H ; bwd: S = dm2 + dm2^T
    __shared__ double sRed[2 * (NT / 64)];
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const double a = static_cast<double>(Av[c.h]);
    const double c0 = cdt[c.c_bhn * L];
    const double c2 = exp(2.0 * a * c0) * phi[c.c_bhn * L];
    const double c1 = exp(a * c0) * psi[c.c_bhn * L];
    const float* Hm = Sin + c.ch * (P * R);
    const float* Tc = Tm + c.ch * (P * R);
    const int64_t bh = static_cast<int64_t>(c.b) * H + c.h;
    if constexpr (FWD) {
        // forward: W = H^T (2T + c2 H), m1c = c1 colsum(H).  Every load of H and T is
        // issued before the first LDS write (one memory latency, not one per row batch).
        __shared__ float sV[P * RS];  // 2T + c2 H
        {
            constexpr int V = R / 4, TOT = P * V, IT = (TOT + NT - 1) / NT;
            v4f hv[IT], tv[IT];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int idx = tid + it * NT;
                if (TOT % NT == 0 || idx < TOT) {
                    hv[it] = *reinterpret_cast<const v4f*>(Hm + idx * 4);
                    tv[it] = *reinterpret_cast<const v4f*>(Tc + idx * 4);
                }
            }
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int idx = tid + it * NT;
                if (TOT % NT == 0 || idx < TOT) {
                    const int row = idx / V, c4 = idx % V;
                    *reinterpret_cast<v4f*>(sA + row * RS + c4 * 4) = hv[it];
                    *reinterpret_cast<v4f*>(sV + row * RS + c4 * 4) =
                        2.0f * tv[it] + static_cast<float>(c2) * hv[it];
                }
            }
        }
        __syncthreads();
        // wave w takes the 16-row strips r1t = w, w + 4, ... with all their column tiles at
        // once (independent accumulator chains)
        constexpr int NTR = R / 16;
        float* Wo = W + c.ch * static_cast<int64_t>(R * R);
        for (int r1t = wave; r1t < NTR; r1t += 4) {
            v4f acc[NTR];
#pragma unroll
            for (int r2t = 0; r2t < NTR; ++r2t) acc[r2t] = zero4();
            for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int p_ = 16 * kk + 4 * g + v;
                    const float av = sA[p_ * RS + r1t * 16 + i];
#pragma unroll
                    for (int r2t = 0; r2t < NTR; ++r2t)
                        acc[r2t] = mfma16(av, sV[p_ * RS + r2t * 16 + i], acc[r2t]);
                }
#pragma unroll
            for (int r2t = 0; r2t < NTR; ++r2t)
#pragma unroll
                for (int v = 0; v < 4; ++v) Wo[(r1t * 16 + 4 * g + v) * R + r2t * 16 + i] = acc[r2t][v];
        }
        // m1c: NT / R threads per column r, each summing a fixed slice of the P rows, then
        // combined in a fixed order across lanes (the NT / R threads of r are R lanes apart)
        {
            constexpr int TPC = NT / R;  // threads per column (R <= 128 divides 256)
            const int r = tid % R, part = tid / R;
            float acc = 0.f;
#pragma unroll 4
            for (int p_ = part; p_ < P; p_ += TPC) acc += sA[p_ * RS + r];
            __shared__ float sPart[NT];
            sPart[tid] = acc;
            __syncthreads();
            if (part == 0) {
                float tot = 0.f;
#pragma unroll
                for (int k = 0; k < TPC; ++k) tot += sPart[k * R + r];
                m1c[c.ch * R + r] = static_cast<float>(c1) * tot;
            }
        }
    } else {
    // backward.  The first pass's H and T rows and the first B rows load into registers
    // ahead of the S staging, so their latency overlaps it.
    const float* d1 = dm1 ? dm1 + bh * R : nullptr;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    v4f ah[R / 16], at[R / 16], ab[R / 16];
    {
        const int row = 16 * wave + i;
        if (row < P) {
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) {
                ah[kk] = *reinterpret_cast<const v4f*>(Hm + row * R + 16 * kk + 4 * g);
                at[kk] = *reinterpret_cast<const v4f*>(Tc + row * R + 16 * kk + 4 * g);
            }
        }
        if (row < L) {
            const int64_t brow = brow0 + static_cast<int64_t>(row) * bstride;
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) ab[kk] = io<IO>::ld4(Bm, brow + 16 * kk + 4 * g);
        }
    }
    // S = dm2 + dm2^T into LDS: coalesced loads of dm2, then each unordered pair {r1, r2}
    // is summed and written to both places by one thread (the sum is symmetric exactly)
    {
        const float* d2 = dm2 + bh * (R * R);
        constexpr int V = R / 4, TOT = R * V, IT = (TOT + NT - 1) / NT;
        v4f dv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT) dv[it] = *reinterpret_cast<const v4f*>(d2 + idx * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT)
                *reinterpret_cast<v4f*>(sA + (idx / V) * RS + (idx % V) * 4) = dv[it];
        }
        __syncthreads();
        for (int idx = tid; idx < R * R; idx += NT) {
            const int r1 = idx / R, r2 = idx - (idx / R) * R;
            if (r1 < r2) {
                const float v = sA[r1 * RS + r2] + sA[r2 * RS + r1];
                sA[r1 * RS + r2] = v;
                sA[r2 * RS + r1] = v;
            } else if (r1 == r2) {
                sA[r1 * RS + r1] = sA[r1 * RS + r1] + sA[r1 * RS + r1];
            }
        }
        __syncthreads();
    }
    double part_hsh = 0.0, part_hdm = 0.0;
    // HS = H S and dS_local = (c2 H + T) S + c1 1 dm1^T, 16 rows per wave per pass
    for (int r0 = 16 * wave; r0 < P; r0 += 64) {
        const int row = r0 + i;
        if (r0 != 16 * wave) {
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) {
                ah[kk] = *reinterpret_cast<const v4f*>(Hm + row * R + 16 * kk + 4 * g);
                at[kk] = *reinterpret_cast<const v4f*>(Tc + row * R + 16 * kk + 4 * g);
            }
        }
        v4f av[R / 16];
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            av[kk] = static_cast<float>(c2) * ah[kk] + at[kk];
            if (d1) {
                const v4f dv = *reinterpret_cast<const v4f*>(d1 + 16 * kk + 4 * g);
                part_hdm += static_cast<double>(ah[kk][0] * dv[0] + ah[kk][1] * dv[1]) +
                            static_cast<double>(ah[kk][2] * dv[2] + ah[kk][3] * dv[3]);
            }
        }
        // H and dm1 in the result tiles' layout load during the products
        float hq[R / 16][4], d1q[R / 16];
#pragma unroll
        for (int nt = 0; nt < R / 16; ++nt) {
            d1q[nt] = d1 ? static_cast<float>(c1) * d1[nt * 16 + i] : 0.f;
#pragma unroll
            for (int v = 0; v < 4; ++v) hq[nt][v] = Hm[(r0 + 4 * g + v) * R + nt * 16 + i];
        }
        v4f o1[R / 16], o2[R / 16];
#pragma unroll
        for (int nt = 0; nt < R / 16; ++nt) o1[nt] = o2[nt] = zero4();
        rows_x_sym_lds<R, R>(ah, sA, RS, o1, i, g);
        rows_x_sym_lds<R, R>(av, sA, RS, o2, i, g);
#pragma unroll
        for (int nt = 0; nt < R / 16; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int p_ = r0 + 4 * g + v, r_ = nt * 16 + i;
                HS[c.ch * (P * R) + p_ * R + r_] = o1[nt][v];
                part_hsh += static_cast<double>(o1[nt][v]) * hq[nt][v];
                dSl[c.ch * (P * R) + p_ * R + r_] = o2[nt][v] + d1q[nt];
            }
    }
    // BS = B S for the chunk's tokens
    for (int r0 = 16 * wave; r0 < L; r0 += 64) {
        if (r0 != 16 * wave) {
            const int64_t brow = brow0 + static_cast<int64_t>(r0 + i) * bstride;
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) ab[kk] = io<IO>::ld4(Bm, brow + 16 * kk + 4 * g);
        }
        v4f o[R / 16];
#pragma unroll
        for (int nt = 0; nt < R / 16; ++nt) o[nt] = zero4();
        rows_x_sym_lds<R, R>(ab, sA, RS, o, i, g);
#pragma unroll
        for (int nt = 0; nt < R / 16; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                BS[(c.ch * L + r0 + 4 * g + v) * static_cast<int64_t>(R) + nt * 16 + i] = o[nt][v];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        part_hsh += __shfl_xor(part_hsh, off);
        part_hdm += __shfl_xor(part_hdm, off);
    }
    if (lane == 0) {
        sRed[wave] = part_hsh;
        sRed[4 + wave] = part_hdm;
    }
    __syncthreads();
    if (tid == 0) {
        hsh[c.ch] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
        hdm[c.ch] = sRed[4] + sRed[5] + sRed[6] + sRed[7];
    }
    }
}

// ------------------------------------------------------------------- reduce
// m2[b,h] = (Z + Z^T)/2 with Z = sum over chunks (and blocks) of U and W;
// m1[b,h] = sum of the m1 parts.  First a coalesced sum (one thread per output
// element, fixed order over the partials) written into m2/m1, then an in-place
// symmetrisation (one thread per pair r1 < r2).
__global__ __launch_bounds__(NT) void km_reduce_sum(const float* __restrict__ U,
                                                     const float* __restrict__ W,
                                                     const float* __restrict__ m1b,
                                                     const float* __restrict__ m1c,
                                                     float* __restrict__ m2, float* __restrict__ m1,
                                                     int N, int H, int R, int nblk) {
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H, h = bh - (bh / H) * H;
    const int RR = R * R;
    const int idx = blockIdx.y * NT + threadIdx.x;
    // the partials of CU chunks are loaded before they are added (in the fixed order
    // chunk by chunk, blocks then the chunk term): one load in flight per thread made
    // the sum latency-bound (2.4 TB/s); nblk <= 4
    constexpr int CU = 4;
    const bool is_m2 = idx < RR;
    if (idx >= RR + R) return;
    const int r = idx - RR;
    const float* part = is_m2 ? U : m1b;
    const float* term = is_m2 ? W : m1c;
    const int width = is_m2 ? RR : R;
    const int col = is_m2 ? idx : r;
    double acc = 0.0;
    for (int n0 = 0; n0 < N; n0 += CU) {
        float v[CU][5];
#pragma unroll
        for (int u = 0; u < CU; ++u)
            if (n0 + u < N) {
                const int64_t ch = (b * N + n0 + u) * H + h;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (k < nblk) v[u][k] = part[(ch * nblk + k) * width + col];
                v[u][4] = term[ch * width + col];
            }
#pragma unroll
        for (int u = 0; u < CU; ++u)
            if (n0 + u < N) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (k < nblk) acc += static_cast<double>(v[u][k]);
                acc += static_cast<double>(v[u][4]);
            }
    }
    if (is_m2)
        m2[bh * RR + idx] = static_cast<float>(acc);
    else
        m1[bh * R + r] = static_cast<float>(acc);
}

__global__ __launch_bounds__(NT) void km_symmetrise(float* __restrict__ m2, int R) {
    const int64_t bh = blockIdx.x;
    const int idx = blockIdx.y * NT + threadIdx.x;
    if (idx >= R * R) return;
    const int r1 = idx / R, r2 = idx - (idx / R) * R;
    if (r1 >= r2) return;
    float* m = m2 + bh * R * R;
    const float avg = 0.5f * (m[r1 * R + r2] + m[r2 * R + r1]);
    m[r1 * R + r2] = avg;
    m[r2 * R + r1] = avg;
}

// ----------------------------------------------------------- backward rows
template <class IO, int P, int R>
__global__ __launch_bounds__(NT, (P * R <= 64 * 64 && P <= 64) ? 2 : 1) void km_bwd_rows(
    const typename IO::T* __restrict__ x, const typename IO::T* __restrict__ Bm,
    const float* __restrict__ dt, const float* __restrict__ Av, const double* __restrict__ cdt,
    const double* __restrict__ phi, const double* __restrict__ psi,
    const double* __restrict__ phit, const double* __restrict__ psit, const float* __restrict__ HS,
    const float* __restrict__ BS, const float* __restrict__ dI, const float* __restrict__ Sin,
    const float* __restrict__ final_state, const float* __restrict__ dm1,
    const double* __restrict__ hsh, const double* __restrict__ hdm,
    typename IO::T* __restrict__ dx, typename IO::T* __restrict__ dB, float* __restrict__ ddtW,
    float* __restrict__ rho, float* __restrict__ eta, float* __restrict__ zeta,
    double* __restrict__ dend2, double* __restrict__ dA_part, int N, int H, int L, int64_t CH) {
    constexpr int RS = R + 4, PS = P + 4;
    constexpr int MAINF = P * RS > TB * (PS + RS) ? P * RS : TB * (PS + RS);
    __shared__ float sM[MAINF];  // phase 1: HS, then d_intra [P, R]; phase 2: X | BS blocks
    __shared__ double sC[TB], sPhi[TB], sPhit[TB];
    __shared__ float sDt[TB];
    __shared__ double sRed[2 * (NT / 64)];
    float* sX = sM;
    float* sQ = sM + TB * PS;
    const int nblk = L / TB;
    const int sb = static_cast<int>(blockIdx.x / CH);
    const ChunkHead c = decode_ch(blockIdx.x % CH, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double* ph = phi + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double la2 = a * kLog2e;
    const int sl = 16 * wave + i, spos = sb * TB + sl;
    const int64_t bh = static_cast<int64_t>(c.b) * H + c.h;

    v4f xreg[P / 16], breg[R / 16];
    const int64_t xrow = xrow0 + static_cast<int64_t>(spos) * xstride;
    const int64_t brow = brow0 + static_cast<int64_t>(spos) * bstride;
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) xreg[kk] = io<IO>::ld4(x, xrow + 16 * kk + 4 * g);
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) breg[kk] = io<IO>::ld4(Bm, brow + 16 * kk + 4 * g);
    const double cs = cc[spos], phs = ph[spos], pss = psi[c.c_bhn * L + spos];
    const double phts = phit[c.c_bhn * L + spos], psts = psit[c.c_bhn * L + spos];
    const double cend = cc[L - 1];
    double dAacc = 0.0;  // this thread's part of the chunk's d_A (pair form, see the header)
    const float dts = dtc[spos];
    const double es = exp(a * cs);
    const float de = expf(static_cast<float>(a * (cc[L - 1] - cs)));
    const float bbar = dts * de;
    const float vs = static_cast<float>(static_cast<double>(dts) * es * phs);
    const float us = static_cast<float>(static_cast<double>(dts) * pss);

    // per-row scalars: xsum = 1^T x_s, dmb = d_m1 . B_s
    float xsum = 0.f, dmb = 0.f;
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) xsum += xreg[kk][0] + xreg[kk][1] + xreg[kk][2] + xreg[kk][3];
    const float* d1 = dm1 ? dm1 + bh * R : nullptr;
    if (d1) {
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            const v4f dv = *reinterpret_cast<const v4f*>(d1 + 16 * kk + 4 * g);
            dmb += dv[0] * breg[kk][0] + dv[1] * breg[kk][1] + dv[2] * breg[kk][2] + dv[3] * breg[kk][3];
        }
    }
    xsum = sum_over_g(xsum);
    dmb = sum_over_g(dmb);

    v4f accX[P / 16], accB[R / 16];
    float eta_s = 0.f, xdb = 0.f;
    // phase 1a: HS terms; d_intra loads into registers meanwhile
    stage_mat<R, P>(sM, HS + c.ch * (P * R));
    __syncthreads();
    constexpr int MV = R / 4, MTOT = P * MV, MIT = (MTOT + NT - 1) / NT;
    v4f pre_dI[MIT];
    {
        const float* g = dI + c.ch * (P * R);
#pragma unroll
        for (int it = 0; it < MIT; ++it) {
            const int idx = tid + it * NT;
            if (MTOT % NT == 0 || idx < MTOT) pre_dI[it] = *reinterpret_cast<const v4f*>(g + idx * 4);
        }
    }
    {
        v4f t[P / 16];
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) t[pt] = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk)
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                const v4f u = *reinterpret_cast<const v4f*>(sM + (pt * 16 + i) * RS + 16 * kk + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) t[pt] = mfma16(u[v], breg[kk][v], t[pt]);
            }
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) eta_s += t[pt][v] * xreg[pt][v];
            accX[pt] = vs * t[pt] + us * dmb;
        }
        v4f tb_[R / 16];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) tb_[rt] = zero4();
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    tb_[rt] = mfma16(sM[(16 * kk + 4 * g + v) * RS + rt * 16 + i], xreg[kk][v], tb_[rt]);
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
            v4f dv = zero4();
            if (d1) dv = *reinterpret_cast<const v4f*>(d1 + rt * 16 + 4 * g);
            accB[rt] = vs * tb_[rt] + (us * xsum) * dv;
        }
    }
    __syncthreads();
    // phase 1b: d_intra (the carried gradient of the chunk's last state) terms; the first
    // partner block's rows load into registers meanwhile
#pragma unroll
    for (int it = 0; it < MIT; ++it) {
        const int idx = tid + it * NT;
        if (MTOT % NT == 0 || idx < MTOT)
            *reinterpret_cast<v4f*>(sM + (idx / MV) * RS + (idx % MV) * 4) = pre_dI[it];
    }
    __syncthreads();
    v4f preX[RowTiles<P, TB>::IT], preQ[RowTiles<R, TB>::IT];
    load_rows<IO, P, TB>(preX, x + xrow0, xstride);
    load_rows<F32, R, TB>(preQ, BS + c.ch * L * static_cast<int64_t>(R), R);
    double pc = 0.0, pph = 0.0, ppt = 0.0;
    float pdt = 0.0f;
    if (tid < TB) {
        pc = cc[tid];
        pph = ph[tid];
        ppt = phit[c.c_bhn * L + tid];
        pdt = dtc[tid];
    }
    {
        v4f t[P / 16];
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) t[pt] = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk)
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                const v4f u = *reinterpret_cast<const v4f*>(sM + (pt * 16 + i) * RS + 16 * kk + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) t[pt] = mfma16(u[v], breg[kk][v], t[pt]);
            }
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) xdb += t[pt][v] * xreg[pt][v];
            accX[pt] += bbar * t[pt];
        }
        v4f tb_[R / 16];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) tb_[rt] = zero4();
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    tb_[rt] = mfma16(sM[(16 * kk + 4 * g + v) * RS + rt * 16 + i], xreg[kk][v], tb_[rt]);
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) accB[rt] += bbar * tb_[rt];
    }
    if (sb == 0) {
        // <d_intra, h_end> (h_end: the next chunk's entry state or the final state) and
        // <d_intra, H>, plus the chunk-level d_A terms
        const float* he = (c.n + 1 < N) ? Sin + (c.ch + H) * (P * R) : final_state + bh * (P * R);
        const float* hm = Sin + c.ch * (P * R);
        double part = 0.0, part2 = 0.0;
#pragma unroll
        for (int it = 0; it < MIT; ++it) {
            const int idx = tid + it * NT;
            if (MTOT % NT == 0 || idx < MTOT) {
                const v4f u = *reinterpret_cast<const v4f*>(he + idx * 4);
                const v4f u2 = *reinterpret_cast<const v4f*>(hm + idx * 4);
                const v4f w = *reinterpret_cast<const v4f*>(sM + (idx / MV) * RS + (idx % MV) * 4);
                part += static_cast<double>(u[0] * w[0] + u[1] * w[1]) + static_cast<double>(u[2] * w[2] + u[3] * w[3]);
                part2 += static_cast<double>(u2[0] * w[0] + u2[1] * w[1]) + static_cast<double>(u2[2] * w[2] + u2[3] * w[3]);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            part += __shfl_xor(part, off);
            part2 += __shfl_xor(part2, off);
        }
        if (lane == 0) {
            sRed[wave] = part;
            sRed[4 + wave] = part2;
        }
        __syncthreads();
        if (tid == 0) {
            dend2[c.c_bhn] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
            const double dhH = sRed[4] + sRed[5] + sRed[6] + sRed[7];
            const double c0 = cc[0], e0 = exp(a * c0);
            const int64_t o0 = c.c_bhn * L;
            dAacc += hsh[c.ch] * e0 * e0 * (phit[o0] + c0 * ph[0]) +
                     hdm[c.ch] * e0 * (psit[o0] + c0 * psi[o0]) + cend * exp(a * cend) * dhH;
        }
        __syncthreads();
    }

    // phase 2: pairs (s, s') over the whole chunk
    float kpn = 0.f, rh = 0.f;
    for (int b2 = 0; b2 < nblk; ++b2) {
        __syncthreads();
        if (b2 == 0) {
            store_rows<P, TB>(sX, preX);
            store_rows<R, TB>(sQ, preQ);
            if (tid < TB) {
                sC[tid] = pc;
                sPhi[tid] = pph;
                sPhit[tid] = ppt;
                sDt[tid] = pdt;
            }
        } else {
            stage_rows<IO, P>(sX, x + xrow0 + static_cast<int64_t>(b2 * TB) * xstride, xstride);
            stage_mat<R, TB>(sQ, BS + (c.ch * L + b2 * TB) * static_cast<int64_t>(R));
            if (tid < TB) {
                sC[tid] = cc[b2 * TB + tid];
                sPhi[tid] = ph[b2 * TB + tid];
                sPhit[tid] = phit[c.c_bhn * L + b2 * TB + tid];
                sDt[tid] = dtc[b2 * TB + tid];
            }
        }
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
            v4f gt = zero4(), qt = zero4();
#pragma unroll
            for (int kk = 0; kk < P / 16; ++kk) {
                const v4f u = *reinterpret_cast<const v4f*>(sX + (16 * j + i) * PS + 16 * kk + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) gt = mfma16(u[v], xreg[kk][v], gt);
            }
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk) {
                const v4f u = *reinterpret_cast<const v4f*>(sQ + (16 * j + i) * RS + 16 * kk + 4 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) qt = mfma16(u[v], breg[kk][v], qt);
            }
            float kq[4], kg[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int sp = 16 * j + 4 * g + v;
                const int ppos = b2 * TB + sp;
                const double cp = sC[sp];
                const bool pm = ppos >= spos;
                const double gap = pm ? cp - cs : cs - cp;
                const double phm = pm ? sPhi[sp] : phs;
                const double phtm = pm ? sPhit[sp] : phts;
                const float dex = sDt[sp] * exp2_of(la2 * gap);
                const float kp = dex * static_cast<float>(phm);  // K / dt_s
                const float kv = dts * kp;
                const float nv = gt[v] * qt[v];
                kq[v] = kv * qt[v];
                kg[v] = kv * gt[v];
                kpn += kp * nv;
                // pair term of d_A: weight formed in fp64, product in fp32, sum in fp64
                const float wA = static_cast<float>(phtm + 0.5 * gap * phm);
                dAacc += static_cast<double>(nv * dts * dex * wA);
                rh += ppos < spos ? dex * nv : (ppos == spos ? 0.5f * dts * nv : 0.0f);
            }
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    accX[pt] = mfma16(sX[(16 * j + 4 * g + v) * PS + pt * 16 + i], kq[v], accX[pt]);
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    accB[rt] = mfma16(sQ[(16 * j + 4 * g + v) * RS + rt * 16 + i], kg[v], accB[rt]);
        }
    }
    if constexpr (sizeof(typename IO::T) != 4) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) io<IO>::st4(dx, xrow + pt * 16 + 4 * g, accX[pt]);
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) io<IO>::st4(dB, brow + rt * 16 + 4 * g, accB[rt]);
    } else {
        // fp32 io: the rows leave through LDS so that each non-temporal store instruction
        // writes whole rows (scattered 64-byte row pieces wrote 20 % more bytes)
        __syncthreads();  // every wave is done with the partner rows
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
            *reinterpret_cast<v4f*>(sX + sl * PS + pt * 16 + 4 * g) = accX[pt];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
            *reinterpret_cast<v4f*>(sQ + sl * RS + rt * 16 + 4 * g) = accB[rt];
        __syncthreads();
        const int64_t row0 = static_cast<int64_t>(sb * TB + 16 * wave);
#pragma unroll
        for (int k = lane; k < 16 * (P / 4); k += 64) {
            const int r_ = k / (P / 4), c4 = k % (P / 4);
            st4_nt<IO>(dx, xrow0 + (row0 + r_) * xstride + c4 * 4,
                       *reinterpret_cast<const v4f*>(sX + (16 * wave + r_) * PS + c4 * 4));
        }
#pragma unroll
        for (int k = lane; k < 16 * (R / 4); k += 64) {
            const int r_ = k / (R / 4), c4 = k % (R / 4);
            st4_nt<IO>(dB, brow0 + (row0 + r_) * bstride + c4 * 4,
                       *reinterpret_cast<const v4f*>(sQ + (16 * wave + r_) * RS + c4 * 4));
        }
    }
    eta_s = sum_over_g(eta_s);
    xdb = sum_over_g(xdb);
    kpn = sum_over_g(kpn);
    rh = sum_over_g(rh);
    if (g == 0) {
        const int64_t o = c.c_bhn * L + spos;
        const float zs = xsum * dmb;
        ddtW[o] = static_cast<float>(es * phs) * eta_s + kpn + static_cast<float>(pss) * zs + de * xdb;
        rho[o] = rh;
        eta[o] = eta_s;
        zeta[o] = zs;
        dAacc += static_cast<double>(eta_s) * dts * es * (2.0 * phts + cs * phs) +
                 static_cast<double>(zs) * dts * psts +
                 (cend - cs) * static_cast<double>(bbar) * static_cast<double>(xdb);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dAacc += __shfl_xor(dAacc, off);
    __syncthreads();
    if (lane == 0) sRed[wave] = dAacc;
    __syncthreads();
    if (tid == 0) dA_part[c.ch * nblk + sb] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
}

// --------------------------------------------------------------- bwd scans
__global__ __launch_bounds__(NT) void km_scan_bwd(
    const double* __restrict__ cdt, const float* __restrict__ dt, const float* __restrict__ A,
    const int64_t* __restrict__ valid, const float* __restrict__ ddtW,
    const float* __restrict__ rho, const float* __restrict__ eta, const float* __restrict__ zeta,
    const double* __restrict__ hsh, const double* __restrict__ hdm,
    const double* __restrict__ dend2, float* __restrict__ d_dt, int64_t nchunks_total, int H,
    int N, int L) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (c >= nchunks_total) return;
    const int n = static_cast<int>(c % N);
    const int h = static_cast<int>((c / N) % H);
    const int64_t b = c / (static_cast<int64_t>(N) * H);
    const int64_t ch = (b * N + n) * H + h;
    const double a = static_cast<double>(A[h]);
    const int vl = chunk_valid(valid, b, n, L);
    const int E = L >> 6;
    double cv[4], dtv[4], q1[4], q2[4], q3[4], tau[4], lam[4], mu[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = lane * E + e;
        const bool in = e < E;
        cv[e] = in ? cdt[c * L + t] : 0.0;
        dtv[e] = in ? static_cast<double>(dt[c * L + t]) : 0.0;
        q1[e] = in ? 2.0 * dtv[e] * rho[c * L + t] : 0.0;
        q2[e] = in ? dtv[e] * eta[c * L + t] : 0.0;
        q3[e] = in ? dtv[e] * zeta[c * L + t] : 0.0;
    }
    wave_fwd_scan(cv, q1, 2.0 * a, E, lane, tau);
    wave_fwd_scan(cv, q2, a, E, lane, lam);
    wave_fwd_scan(cv, q3, a, E, lane, mu);
    const double hs = hsh[ch], hd = hdm[ch], d2 = dend2[c];
    double dac[4], ddw[4];
    double tot = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = lane * E + e;
        if (e < E) {
            const double et = exp(a * cv[e]);
            const double sig = et * et * hs + 2.0 * et * lam[e] + tau[e];
            const double lin = et * hd + mu[e];
            ddw[e] = static_cast<double>(ddtW[c * L + t]);
            dac[e] = (t < vl ? sig + lin : 0.0) - dtv[e] * ddw[e];
            if (t == L - 1) dac[e] += d2;
            tot += dac[e];
        } else {
            dac[e] = 0.0;
            ddw[e] = 0.0;
        }
    }
    // suffix sums of dac over the chunk
    double suf = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_down(suf, off);
        if (lane + off < 64) suf += o;
    }
    double after = __shfl_down(suf, 1);
    if (lane == 63) after = 0.0;
    double run = after;
#pragma unroll
    for (int e = 3; e >= 0; --e)
        if (e < E) {
            run += dac[e];
            d_dt[c * L + lane * E + e] = static_cast<float>(ddw[e] + a * run);
        }
}

// ------------------------------------------------------------------ dispatch
#define SSD_FOR_EACH_PR(X) \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) \
    X(128, 16) X(128, 32) X(128, 64) X(128, 128)

template <class IO>
static hipError_t fwd_rows_io(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, float* U, float* m1b, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH * s.nblk()));
#define X(PP, RR)                                                                               \
    if (s.P == PP && s.R == RR) {                                                               \
        hipLaunchKernelGGL((km_fwd_rows<IO, PP, RR>), grid, dim3(NT), 0, st,                   \
                           static_cast<const T*>(x), static_cast<const T*>(Bm), dt, A, cdt, phi, \
                           psi, U, m1b, s.N, s.H, s.L, CH);                                     \
        return hipGetLastError();                                                               \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_km_fwd_rows(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, float* U, float* m1b, hipStream_t st) {
    return s.io == 1 ? fwd_rows_io<BF16>(s, x, Bm, dt, A, cdt, phi, psi, U, m1b, st)
                     : fwd_rows_io<F32>(s, x, Bm, dt, A, cdt, phi, psi, U, m1b, st);
}

template <class IO>
static hipError_t chunk_io(const Shape& s, const float* Sin, const float* T, const double* cdt,
                           const float* A, const double* phi, const double* psi, float* W,
                           float* m1c, const float* dm2, const float* dm1, const void* Bm,
                           float* HS, float* dSl, float* BS, double* hsh, double* hdm,
                           hipStream_t st) {
    using TT = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH));
#define X(PP, RR)                                                                                  \
    if (s.P == PP && s.R == RR) {                                                                  \
        if (dm2)                                                                                   \
            hipLaunchKernelGGL((km_chunk<IO, PP, RR, false>), grid, dim3(NT), 0, st, Sin, T, cdt, A, \
                               phi, psi, W, m1c, dm2, dm1, static_cast<const TT*>(Bm), HS, dSl, BS, \
                               hsh, hdm, s.N, s.H, s.L);                                           \
        else                                                                                       \
            hipLaunchKernelGGL((km_chunk<IO, PP, RR, true>), grid, dim3(NT), 0, st, Sin, T, cdt, A,  \
                               phi, psi, W, m1c, dm2, dm1, static_cast<const TT*>(Bm), HS, dSl, BS, \
                               hsh, hdm, s.N, s.H, s.L);                                           \
        return hipGetLastError();                                                                  \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_km_chunk(const Shape& s, const float* Sin, const float* T, const double* cdt,
                           const float* A, const double* phi, const double* psi, float* W,
                           float* m1c, const float* dm2, const float* dm1, const void* Bm,
                           float* HS, float* dSl, float* BS, double* hsh, double* hdm,
                           hipStream_t st) {
    return s.io == 1 ? chunk_io<BF16>(s, Sin, T, cdt, A, phi, psi, W, m1c, dm2, dm1, Bm, HS, dSl, BS,
                                      hsh, hdm, st)
                     : chunk_io<F32>(s, Sin, T, cdt, A, phi, psi, W, m1c, dm2, dm1, Bm, HS, dSl, BS,
                                     hsh, hdm, st);
}

hipError_t launch_km_reduce(const Shape& s, const float* U, const float* W, const float* m1b,
                            const float* m1c, float* m2, float* m1, hipStream_t st) {
    const int64_t BH = static_cast<int64_t>(s.B) * s.H;
    if (BH == 0) return hipSuccess;
    const int RR = s.R * s.R;
    hipLaunchKernelGGL(km_reduce_sum, dim3(static_cast<unsigned>(BH),
                                           static_cast<unsigned>((RR + s.R + NT - 1) / NT)),
                       dim3(NT), 0, st, U, W, m1b, m1c, m2, m1, s.N, s.H, s.R, s.nblk());
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(km_symmetrise, dim3(static_cast<unsigned>(BH), static_cast<unsigned>((RR + NT - 1) / NT)),
                       dim3(NT), 0, st, m2, s.R);
    return hipGetLastError();
}

template <class IO>
static hipError_t bwd_rows_io(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, const double* phit, const double* psit,
                              const float* HS, const float* BS, const float* dI, const float* Sin,
                              const float* fin, const float* dm1, const double* hsh,
                              const double* hdm, void* dx, void* dB, float* ddtW, float* rho,
                              float* eta, float* zeta, double* dend2, double* dA_part,
                              hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH * s.nblk()));
#define X(PP, RR)                                                                                 \
    if (s.P == PP && s.R == RR) {                                                                 \
        hipLaunchKernelGGL((km_bwd_rows<IO, PP, RR>), grid, dim3(NT), 0, st,                     \
                           static_cast<const T*>(x), static_cast<const T*>(Bm), dt, A, cdt, phi,   \
                           psi, phit, psit, HS, BS, dI, Sin, fin, dm1, hsh, hdm,                 \
                           static_cast<T*>(dx), static_cast<T*>(dB), ddtW, rho, eta, zeta, dend2, \
                           dA_part, s.N, s.H, s.L, CH);                                           \
        return hipGetLastError();                                                                 \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_km_bwd_rows(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, const double* phit, const double* psit,
                              const float* HS, const float* BS, const float* dI, const float* Sin,
                              const float* final_state, const float* dm1, const double* hsh,
                              const double* hdm, void* dx, void* dB, float* ddtW, float* rho,
                              float* eta, float* zeta, double* dend2, double* dA_part,
                              hipStream_t st) {
    return s.io == 1 ? bwd_rows_io<BF16>(s, x, Bm, dt, A, cdt, phi, psi, phit, psit, HS, BS, dI, Sin,
                                         final_state, dm1, hsh, hdm, dx, dB, ddtW, rho, eta, zeta,
                                         dend2, dA_part, st)
                     : bwd_rows_io<F32>(s, x, Bm, dt, A, cdt, phi, psi, phit, psit, HS, BS, dI, Sin,
                                        final_state, dm1, hsh, hdm, dx, dB, ddtW, rho, eta, zeta,
                                        dend2, dA_part, st);
}

hipError_t launch_km_scan_bwd(const Shape& s, const double* cdt, const float* dt, const float* A,
                              const int64_t* valid, const float* ddtW, const float* rho,
                              const float* eta, const float* zeta, const double* hsh,
                              const double* hdm, const double* dend2, float* d_dt,
                              hipStream_t st) {
    const int64_t nc = s.chunks();
    if (nc == 0) return hipSuccess;
    hipLaunchKernelGGL(km_scan_bwd, dim3(static_cast<unsigned>((nc + 3) / 4)), dim3(NT), 0, st, cdt,
                       dt, A, valid, ddtW, rho, eta, zeta, hsh, hdm, dend2, d_dt, nc, s.H, s.N, s.L);
    return hipGetLastError();
}

}  // namespace ssd
