// Chunk-parallel MFMA kernels of the recompute backward.
//
// Page: burn-mamba "mamba2/ssd/serial_recalculated/combined_backward.rs".  The
// page runs one reverse loop over chunks that mixes the K5 backward (BLUE and
// ORANGE) with the K4 backward step, then batched K3/K2/K1 backwards.  Only the
// K4 carry is serial, and the quantity it consumes from each chunk (the BLUE
// "d_chunk_input_state = C^T d_ch") is chunk-local, so here the work is split
// into: a chunk-parallel pass for d_chunk_input_state (k_chunk_states, job 1),
// the serial carry (k4_state_pass_bwd), and the two chunk-parallel kernels of
// this file, which consume the carried gradient d_intra of every chunk.
//
// With e_t = exp(cum[t]), decay(t,s) = exp(cum[t] - cum[s]) for s <= t,
// CB = C B^T, W = CB * decay * dt[s], d_w = dy x^T (kept for s <= t),
// d_CB = d_w * dt[s] * decay and d_diff = d_CB * CB (ORANGE backward), and
// b_scaled = B * bbar with bbar = dt * exp(end - cum) (K3):
//
//   source side, rows s (bwd_source, runs first):
//     d_x[s]     = D dy[s]                                   (SKIP backward)
//                + sum_{t>=s} W[t,s] dy[t]                    (ORANGE, d_x = w^T d_orange)
//                + bbar[s] d_intra B[s]^T                     (K3, d_x = d_intra b_scaled^T)
//     d_B[s]     = sum_{t>=s} d_CB[t,s] C[t]                  (K2, d_b = d_cb^T c)
//                + bbar[s] x[s] d_intra                       (K3, d_b = d_b_scaled bbar)
//     d_dt[s]    = sum_{t>=s} d_w CB decay                    (ORANGE d_dt)
//                + d_bbar[s] exp(end - cum[s])                (K3 d_dt), d_bbar = <x[s] d_intra, B[s]>
//     g2[s]      = -sum_{t>s} d_diff[t,s]                     (ORANGE d_da, source side)
//     d_delta[s] = d_bbar[s] dt[s] exp(end - cum[s])          (K3: gradient of end - cum[s])
//     dD_part    = sum dy x                                   (SKIP, d_D)
//   and it hands d_CB of every causal 16 x 16 pair tile to the target side, so C B^T and
//   dy x^T are formed once per pair: the tiles hold the diagonal elements d_CB[t,t] as 0
//   and ddg[t] holds them;
//   target side, rows t (bwd_target, from those tiles):
//     d_C[t]     = e_t dy[t] S_in              (BLUE backward, d_C_blue)
//                + sum_{s<t} d_CB[t,s] B[s]     (K2 backward, d_c = d_cb B)
//                + ddg[t] B[t]                  (its s = t term, added after g1 is taken)
//     g1[t]      = sum_r C[t,r] (d_C[t,r] - ddg[t] B[t,r])   (BLUE d_da + ORANGE d_da, target
//                  side: sum_{s<t} d_diff[t,s] = C_t . sum_{s<t} d_CB[t,s] B_s)
//     d_end      = exp(end) <d_intra, S_in>      (K4 backward, d_da_chunk_end)
//   The diagonal pair's d_diff[t,t] is in neither g1 nor g2: in exact arithmetic it
//   cancels between them, in fp32 each side would round it its own way, and d_dt gets
//   A (g1 + g2 + ...), which would carry |A| times that difference (a memoryless head,
//   A dt ~ -1e4, is nothing but diagonal pairs).
// K1^T then turns g1 + g2, d_delta and d_end into d_cum's suffix sum (for d_dt):
// k1t_and_heads, or the epilogue of the whole-chunk target kernel (k_chunk_wide.hip).
//
// d_A is NOT formed as sum_t d_da[t] dt[t]: the suffix sums of rowsum - colsum
// cancel the large near-diagonal ORANGE terms, which costs d_A ~1e-5 relative
// accuracy in fp32.  Summing each term against the dt it depends on gives the
// same value exactly (cumA = A cdt with cdt the cumsum of dt):
//   d_A = sum_pairs d_diff[t,s] (cdt[t] - cdt[s]) + sum_t blue[t] cdt[t]
//       + sum_s d_delta[s] (cdt[L-1] - cdt[s]) + d_end cdt[L-1]
// per chunk, where near-diagonal pairs get small weights instead of cancelling.
// The source side writes the first and third sums, the target side the second
// (plus the d_end term); reduce_heads adds them per head.
//
// Layout trick (no LDS transposes): every 16x16 product tile is computed with
// its M index along the rows the NEXT product contracts over, so the four MFMA
// result registers of a lane (M = 4g+v, N = i) are exactly the B operand the
// next MFMA needs.  The target side therefore accumulates d_C^T tiles
// (M = r, N = t) and the source side d_x^T / d_B^T tiles (M = p or r, N = s);
// each lane finally stores four consecutive features of one token.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <class IO, int P, int R>
__global__ __launch_bounds__(NT, 2) void k_bwd_target(
    const typename IO::T* __restrict__ dy, const typename IO::T* __restrict__ Bm,
    const typename IO::T* __restrict__ Cm, const float* __restrict__ Av,
    const double* __restrict__ cdt, const float* __restrict__ S, const float* __restrict__ dS,
    const float* __restrict__ dcbt, const float* __restrict__ ddg,
    typename IO::T* __restrict__ dC, float* __restrict__ g1, float* __restrict__ d_end,
    double* __restrict__ dA_T, int N, int H, int L, int64_t CH) {
    constexpr int RS = R + 4;
    constexpr int ROWS = P > TB ? P : TB;
    __shared__ float sBS[ROWS * RS];  // S_in [P, R], then B of the source block
    __shared__ __align__(16) double sCdtT[TB];
    __shared__ double sRed[NT / 64];
    const int nblk = L / TB;
    const int tb = nblk - 1 - static_cast<int>(blockIdx.x / CH);  // heaviest first
    const ChunkHead c = decode_ch(blockIdx.x % CH, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const int tl = 16 * wave + i;  // target row of this lane inside the block
    const int it = 4 * tb + wave;  // this wave's target tile inside the chunk
    const int64_t tiles0 = c.ch * pair_tiles_of(L);

    v4f creg[R / 16], dyreg[P / 16];
    {
        const int64_t crow = brow0 + static_cast<int64_t>(tb * TB + tl) * bstride;
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) creg[kk] = io<IO>::ld4(Cm, crow + 16 * kk + 4 * g);
        const int64_t yrow = xrow0 + static_cast<int64_t>(tb * TB + tl) * xstride;
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) dyreg[kk] = io<IO>::ld4(dy, yrow + 16 * kk + 4 * g);
    }
    stage_mat<R, P>(sBS, S + c.ch * (P * R));
    if (tid < TB) sCdtT[tid] = cc[tb * TB + tid];
    __syncthreads();

    double dA = 0.0;  // this thread's part of the chunk's d_A (see the file header)
    // K4 backward: d_end = exp(A cdt[L-1]) <d_intra, S_in>, once per chunk (block 0).
    if (tb == 0) {
        const float* dsp = dS + c.ch * (P * R);
        double part = 0.0;
        for (int idx = tid; idx < P * (R / 4); idx += NT) {
            const int row = idx / (R / 4), c4 = idx - (idx / (R / 4)) * (R / 4);
            const v4f u = *reinterpret_cast<const v4f*>(dsp + row * R + c4 * 4);
            const v4f w = *reinterpret_cast<const v4f*>(sBS + row * RS + c4 * 4);
            part += static_cast<double>(u[0] * w[0] + u[1] * w[1]) +
                    static_cast<double>(u[2] * w[2] + u[3] * w[3]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) sRed[wave] = part;
        __syncthreads();
        if (tid == 0) {
            const double end = cc[L - 1];
            const double de = (sRed[0] + sRed[1] + sRed[2] + sRed[3]) * exp(a * end);
            const float def = static_cast<float>(de);
            d_end[c.c_bhn] = def;
            dA += static_cast<double>(def) * end;
        }
    }

    // BLUE: d_C^T[r, t] = e_t sum_p S_in[p, r] dy[t, p]
    v4f acc[R / 16];
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) acc[rt] = zero4();
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) {
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[rt] = mfma16(sBS[(16 * kk + 4 * g + v) * RS + rt * 16 + i], dyreg[kk][v], acc[rt]);
        }
    }
    const double ct = sCdtT[tl];
    const float et = expf(static_cast<float>(a * ct));
    float gblue = 0.0f;  // this lane's part of the BLUE gradient w.r.t. the cumsum at t = tl
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) {
        acc[rt] *= et;
#pragma unroll
        for (int v = 0; v < 4; ++v) gblue += creg[rt][v] * acc[rt][v];
    }
    dA += static_cast<double>(gblue) * ct;

    // K2 backward from the source-row kernel's d_CB tiles: d_C^T[r, t] += sum_s B[s, r] d_CB[t, s].
    // The tiles hold the diagonal elements d_CB[t, t] as zeros (they come in ddg), so g1
    // below leaves out the diagonal pair's d_diff, as g2 does in the source-row kernel: in
    // exact arithmetic the two cancel, in fp32 each side rounds its own way and
    // d_dt = ... + A d_da would carry |A| times the difference.  They join d_C after g1.
    for (int sb = 0; sb <= tb; ++sb) {
        const int jmax = (sb == tb) ? wave : 3;  // diagonal block: s-tiles up to this wave's
        v4f dct[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > jmax) break;
            const int64_t tat = tiles0 + pair_index(it, 4 * sb + j);
            dct[j] = *reinterpret_cast<const v4f*>(dcbt + tat * 256 + i * 16 + 4 * g);
        }
        __syncthreads();
        stage_rows<IO, R>(sBS, Bm + brow0 + static_cast<int64_t>(sb * TB) * bstride, bstride);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j > jmax) break;
            if constexpr (sizeof(typename IO::T) == 2) {
                const S4x3 ds = split4(dct[j]);  // bf16 io: B exact, d_CB split (ssd_device.hpp)
#pragma unroll
                for (int rt = 0; rt < R / 16; ++rt) {
                    v4f a;
#pragma unroll
                    for (int v = 0; v < 4; ++v) a[v] = sBS[(16 * j + 4 * g + v) * RS + rt * 16 + i];
                    acc[rt] = mfma16_split(pack_bf16x4(a), ds, acc[rt]);
                }
            } else {
#pragma unroll
                for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[rt] = mfma16(sBS[(16 * j + 4 * g + v) * RS + rt * 16 + i], dct[j][v], acc[rt]);
                }
            }
        }
    }
    // g1[t] = sum_r C[t, r] d_C[t, r]: the BLUE term plus ORANGE's target side, since
    // sum_s d_diff[t, s] = sum_s d_CB[t, s] (C_t . B_s) = C_t . (sum_s d_CB[t, s] B_s)
    // (s = t held out, above)
    float gsum = 0.0f;
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
        for (int v = 0; v < 4; ++v) gsum += creg[rt][v] * acc[rt][v];
    gsum = sum_over_g(gsum);
    if (g == 0) g1[c.c_bhn * L + tb * TB + tl] = gsum;
    // the diagonal element: d_C[t] += d_CB[t, t] B_t (B of this block is still in LDS); store
    // d_C[t = tl][r = 16 rt + 4g .. +3]
    const float dgd = ddg[c.c_bhn * L + tb * TB + tl];
    {
        const int64_t row = brow0 + static_cast<int64_t>(tb * TB + tl) * bstride;
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
            acc[rt] += dgd * *reinterpret_cast<const v4f*>(sBS + tl * RS + rt * 16 + 4 * g);
            io<IO>::st4(dC, row + rt * 16 + 4 * g, acc[rt]);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dA += __shfl_xor(dA, off);
    __syncthreads();
    if (lane == 0) sRed[wave] = dA;
    __syncthreads();
    if (tid == 0) dA_T[c.ch * nblk + tb] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
}

template <class IO, int P, int R>
__global__ __launch_bounds__(NT, 2) void k_bwd_source(
    const typename IO::T* __restrict__ dy, const typename IO::T* __restrict__ x,
    const float* __restrict__ dt, const typename IO::T* __restrict__ Bm,
    const typename IO::T* __restrict__ Cm, const float* __restrict__ Av,
    const float* __restrict__ Dv, const double* __restrict__ cdt, const float* __restrict__ dS,
    typename IO::T* __restrict__ dx, typename IO::T* __restrict__ dB, float* __restrict__ d_dt,
    float* __restrict__ g2, float* __restrict__ d_delta, double* __restrict__ dA_S,
    double* __restrict__ dD_part, float* __restrict__ dcbt, float* __restrict__ ddg, int N, int H,
    int L, int64_t CH) {
    constexpr int RS = R + 4, PS = P + 4;
    constexpr int ROWS = P > TB ? P : TB;
    __shared__ float sCT[ROWS * RS];  // d_intra [P, R], then C of the target block
    __shared__ float sDY[TB * PS];
    __shared__ __align__(16) double sCdtT[TB];
    __shared__ double sRed[2 * (NT / 64)];
    constexpr int NEX = 4 * (P / 16 + R / 16) + 2;  // floats per lane handed from wave 3 to wave 0
    __shared__ float sEx[NEX * 64];
    const int nblk = L / TB;
    const int sb = static_cast<int>(blockIdx.x / CH);  // block 0 has the most targets
    const ChunkHead c = decode_ch(blockIdx.x % CH, N, H);
    // the wave index as a scalar (it is the same in every lane of a wave): the row-tile
    // offsets built from it stay in scalar registers (249 against 256 VGPRs, 1 % faster)
    const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double la2 = a * kLog2e;
    const int sl = 16 * wave + i;   // source row of this lane inside the block
    const int spos = sb * TB + sl;  // ... inside the chunk

    v4f xreg[P / 16], breg[R / 16];
    const int64_t xrow = xrow0 + static_cast<int64_t>(spos) * xstride;
    const int64_t brow = brow0 + static_cast<int64_t>(spos) * bstride;
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) xreg[kk] = io<IO>::ld4(x, xrow + 16 * kk + 4 * g);
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) breg[kk] = io<IO>::ld4(Bm, brow + 16 * kk + 4 * g);
    stage_mat<R, P>(sCT, dS + c.ch * (P * R));
    const double end = cc[L - 1];
    const double cs = cc[spos];
    const float dts = dtc[spos];
    const float dec_end = expf(static_cast<float>(a * (end - cs)));
    const float bbar = dts * dec_end;
    __syncthreads();
    // the first partner block (the farthest, nblk - 1) loads into registers during K3
    v4f preC[RowTiles<R, TB>::IT], preD[RowTiles<P, TB>::IT];
    load_rows<IO, R, TB>(preC, Cm + brow0 + static_cast<int64_t>((nblk - 1) * TB) * bstride, bstride);
    load_rows<IO, P, TB>(preD, dy + xrow0 + static_cast<int64_t>((nblk - 1) * TB) * xstride, xstride);
    const double cpre = tid < TB ? cc[(nblk - 1) * TB + tid] : 0.0;

    // K3 backward.  d_b_scaled^T[r, s] = sum_p d_intra[p, r] x[s, p]
    v4f accB[R / 16];
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) accB[rt] = zero4();
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) {
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                accB[rt] = mfma16(sCT[(16 * kk + 4 * g + v) * RS + rt * 16 + i], xreg[kk][v], accB[rt]);
        }
    }
    float dbb = 0.0f;  // d_bbar[s] = sum_r d_b_scaled[s, r] B[s, r] (this lane's part)
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) dbb += accB[rt][v] * breg[rt][v];
        accB[rt] *= bbar;
    }
    // d_x^T[p, s] = bbar[s] sum_r d_intra[p, r] B[s, r]
    v4f accX[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) accX[pt] = zero4();
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const v4f u = *reinterpret_cast<const v4f*>(sCT + (pt * 16 + i) * RS + 16 * kk + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) accX[pt] = mfma16(u[v], breg[kk][v], accX[pt]);
        }
    }
    // SKIP backward: d_x += D dy; d_D partial sum dy x
    const float Dh = Dv[c.h];
    double dD = 0.0;
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) {
        const v4f dyv = io<IO>::ld4(dy, xrow + pt * 16 + 4 * g);
        accX[pt] = accX[pt] * bbar + Dh * dyv;
        dD += static_cast<double>(dyv[0] * xreg[pt][0] + dyv[1] * xreg[pt][1]) +
              static_cast<double>(dyv[2] * xreg[pt][2] + dyv[3] * xreg[pt][3]);
    }

    float ddt_or = 0.0f, dsrc = 0.0f;
    // d_CB[s, s] of this lane's source row, on the lane of the diagonal tile that holds it:
    // the one whose element v = i - 4 g lies in 0..3
    float dgk = 0.0f;
    const int dvl = i - 4 * g;
    double dA = 0.0;  // this lane's part of the chunk's d_A (the pair terms and K3; file header)
    const int64_t tiles0 = c.ch * pair_tiles_of(L);  // this chunk-head's first pair tile
    // One (16-row target tile j of block tb, 16-row source tile) pair: the source tile's
    // operands xr / br, cumsum csr, dt dtr and row srow inside the block, its accumulators.
    // The pair's d_CB tile goes to the target-row kernel.
    auto tile = [&](int j, int tb, const v4f (&xr)[P / 16], const v4f (&br)[R / 16], double csr,
                    float dtr, int srow, v4f (&aX)[P / 16], v4f (&aB)[R / 16], float& ddt,
                    float& dsr) __attribute__((always_inline)) {
        // tiles with M = t (16j + 4g + v), N = s
        v4f cb = zero4(), dw = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            const v4f u = *reinterpret_cast<const v4f*>(sCT + (16 * j + i) * RS + 16 * kk + 4 * g);
            cb = mfma_k16<IO>(u, br[kk], cb);
        }
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) {
            const v4f u = *reinterpret_cast<const v4f*>(sDY + (16 * j + i) * PS + 16 * kk + 4 * g);
            dw = mfma_k16<IO>(u, xr[kk], dw);
        }
        // this lane's four target rows: cumsums as two 16-byte LDS reads
        const v2d ct01 = *reinterpret_cast<const v2d*>(sCdtT + 16 * j + 4 * g);
        const v2d ct23 = *reinterpret_cast<const v2d*>(sCdtT + 16 * j + 4 * g + 2);
        const double ctv[4] = {ct01.x, ct01.y, ct23.x, ct23.y};
        // hand-off: d_CB[t][s] of the pair tile, t-major, as the target-row kernel reads it
        const int64_t tile_at =
            tiles0 + pair_index(4 * tb + j, 4 * sb + __builtin_amdgcn_readfirstlane(srow >> 4));
        float* const tdst = dcbt + tile_at * 256;
        float wv[4], dcb[4];
        const bool dtile = tb == sb && 16 * j == (srow & ~15);  // the diagonal pair tile
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const bool keep = (tb > sb) || (16 * j + 4 * g + v >= srow);
            // masked pairs (t < s) take gap 0 and weight 0: arithmetic, not a branch
            const double gap = keep ? ctv[v] - csr : 0.0;
            const float dec = exp2_of(la2 * gap) * (keep ? 1.0f : 0.0f);
            const float cbd = cb[v] * dec;
            wv[v] = cbd * dtr;
            dcb[v] = dw[v] * dtr * dec;
            ddt += dw[v] * cbd;
            const float dd = dcb[v] * cb[v];  // d_diff[t, s]
            // the diagonal pair t = s: left out of g2 (the target side leaves it out of g1),
            // its d_CB handed over in ddg, not in the tile
            const bool diag = dtile && dvl == v;
            dsr += diag ? 0.0f : dd;
            dA += static_cast<double>(dd) * gap;
            tdst[(4 * g + v) * 16 + i] = diag ? 0.0f : dcb[v];
            dgk = diag ? dcb[v] : dgk;
        }
        if constexpr (sizeof(typename IO::T) == 2) {
            // bf16 io: dy and C are exact bf16, W and d_CB fp32 tiles split once into
            // three exact bf16 parts; one 16x16x16 bf16 MFMA per part (ssd_device.hpp)
            const S4x3 ws = split4(v4f{wv[0], wv[1], wv[2], wv[3]});
            const S4x3 ds = split4(v4f{dcb[0], dcb[1], dcb[2], dcb[3]});
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
                v4f a;
#pragma unroll
                for (int v = 0; v < 4; ++v) a[v] = sDY[(16 * j + 4 * g + v) * PS + pt * 16 + i];
                aX[pt] = mfma16_split(pack_bf16x4(a), ws, aX[pt]);
            }
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt) {
                v4f a;
#pragma unroll
                for (int v = 0; v < 4; ++v) a[v] = sCT[(16 * j + 4 * g + v) * RS + rt * 16 + i];
                aB[rt] = mfma16_split(pack_bf16x4(a), ds, aB[rt]);
            }
        } else {
            // ORANGE: d_x^T[p, s] += sum_t dy[t, p] W[t, s]
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    aX[pt] = mfma16(sDY[(16 * j + 4 * g + v) * PS + pt * 16 + i], wv[v], aX[pt]);
            }
            // K2 backward: d_B^T[r, s] += sum_t C[t, r] d_CB[t, s]
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    aB[rt] = mfma16(sCT[(16 * j + 4 * g + v) * RS + rt * 16 + i], dcb[v], aB[rt]);
            }
        }
    };
    // Partner blocks from the farthest to the diagonal one.  On the diagonal block wave w
    // owns the t-tiles j >= w (4, 3, 2, 1 tiles); with fp32 io wave 0's last one (j = 3)
    // goes to wave 3, which is idle there otherwise, so no wave carries more than 3 and
    // the block's barrier-to-end time drops by one tile.  (With bf16 io the hand-over's
    // registers spill and the kernel is 5 % slower, so there wave 0 keeps all four.)
    constexpr bool kSplit = sizeof(typename IO::T) == 4;
    auto partner_block = [&](int tb) __attribute__((always_inline)) {
        const bool diag = tb == sb;
        const int jmin = diag ? wave : 0;
        const int jmax = (kSplit && diag && wave == 0) ? 3 : 4;
        for (int j = jmin; j < jmax; ++j) tile(j, tb, xreg, breg, cs, dts, sl, accX, accB, ddt_or, dsrc);
    };
    // wave 0 hands its source tile's operands (lane for lane) and dt to wave 3 through sEx
    // before the barrier that opens the diagonal block
    auto handoff = [&]() __attribute__((always_inline)) {
        if (kSplit && wave == 0) {
#pragma unroll
            for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
                for (int v = 0; v < 4; ++v) sEx[(4 * kk + v) * 64 + lane] = xreg[kk][v];
#pragma unroll
            for (int kk = 0; kk < R / 16; ++kk)
#pragma unroll
                for (int v = 0; v < 4; ++v) sEx[(4 * (P / 16) + 4 * kk + v) * 64 + lane] = breg[kk][v];
            sEx[(NEX - 2) * 64 + lane] = dts;
        }
    };
    __syncthreads();  // K3 is done with d_intra
    store_rows<R, TB>(sCT, preC);
    store_rows<P, TB>(sDY, preD);
    if (tid < TB) sCdtT[tid] = cpre;
    if (nblk - 1 == sb) handoff();
    __syncthreads();
    partner_block(nblk - 1);
    for (int tb = nblk - 2; tb >= sb; --tb) {
        __syncthreads();
        const double cnext = tid < TB ? cc[tb * TB + tid] : 0.0;
        stage_rows<IO, R>(sCT, Cm + brow0 + static_cast<int64_t>(tb * TB) * bstride, bstride);
        stage_rows<IO, P>(sDY, dy + xrow0 + static_cast<int64_t>(tb * TB) * xstride, xstride);
        if (tid < TB) sCdtT[tid] = cnext;
        if (tb == sb) handoff();
        __syncthreads();
        partner_block(tb);
    }
    // wave 3: the pair (t-tile 3, source tile 0) of the diagonal block, still in LDS; the
    // source tile's cumsums are the diagonal block's own (sCdtT).  Its partial sums go
    // back to wave 0 through sEx, lane for lane
    if (kSplit && wave == 3) {
        v4f x0[P / 16], b0[R / 16], aX0[P / 16], aB0[R / 16];
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) {
#pragma unroll
            for (int v = 0; v < 4; ++v) x0[kk][v] = sEx[(4 * kk + v) * 64 + lane];
            aX0[kk] = zero4();
        }
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
#pragma unroll
            for (int v = 0; v < 4; ++v) b0[kk][v] = sEx[(4 * (P / 16) + 4 * kk + v) * 64 + lane];
            aB0[kk] = zero4();
        }
        const float dts0 = sEx[(NEX - 2) * 64 + lane];
        float ddt0 = 0.0f, dsr0 = 0.0f;
        tile(3, sb, x0, b0, sCdtT[i], dts0, i, aX0, aB0, ddt0, dsr0);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v) sEx[(4 * pt + v) * 64 + lane] = aX0[pt][v];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) sEx[(4 * (P / 16) + 4 * rt + v) * 64 + lane] = aB0[rt][v];
        sEx[(NEX - 2) * 64 + lane] = ddt0;
        sEx[(NEX - 1) * 64 + lane] = dsr0;
    }
    if (kSplit) __syncthreads();
    if (kSplit && wave == 0) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v) accX[pt][v] += sEx[(4 * pt + v) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) accB[rt][v] += sEx[(4 * (P / 16) + 4 * rt + v) * 64 + lane];
        ddt_or += sEx[(NEX - 2) * 64 + lane];
        dsrc += sEx[(NEX - 1) * 64 + lane];
    }
    // fp32 io: d_x and d_B leave through LDS so that each non-temporal store instruction
    // writes whole rows (16 B per lane scattered over 64-byte row pieces wrote 20 % more
    // bytes than the outputs hold): wave w's 16 rows go to sDY / sCT, then back out
    // row-major.  bf16 io stores straight from the accumulators (ordinary stores; the
    // detour through LDS made that kernel 4 % slower).
    if constexpr (sizeof(typename IO::T) != 4) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) io<IO>::st4(dx, xrow + pt * 16 + 4 * g, accX[pt]);
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) io<IO>::st4(dB, brow + rt * 16 + 4 * g, accB[rt]);
    } else {
        __syncthreads();  // every wave is done with the partner rows
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
            *reinterpret_cast<v4f*>(sDY + sl * PS + pt * 16 + 4 * g) = accX[pt];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
            *reinterpret_cast<v4f*>(sCT + sl * RS + rt * 16 + 4 * g) = accB[rt];
        __syncthreads();
        const int64_t row0 = static_cast<int64_t>(sb * TB + 16 * wave);
#pragma unroll
        for (int k = lane; k < 16 * (P / 4); k += 64) {
            const int r_ = k / (P / 4), c4 = k % (P / 4);
            st4_nt<IO>(dx, xrow0 + (row0 + r_) * xstride + c4 * 4,
                       *reinterpret_cast<const v4f*>(sDY + (16 * wave + r_) * PS + c4 * 4));
        }
#pragma unroll
        for (int k = lane; k < 16 * (R / 4); k += 64) {
            const int r_ = k / (R / 4), c4 = k % (R / 4);
            st4_nt<IO>(dB, brow0 + (row0 + r_) * bstride + c4 * 4,
                       *reinterpret_cast<const v4f*>(sCT + (16 * wave + r_) * RS + c4 * 4));
        }
    }

    dbb = sum_over_g(dbb);
    ddt_or = sum_over_g(ddt_or);
    dsrc = sum_over_g(dsrc);
    dgk = sum_over_g(dgk);  // one lane of the four holds it, the others 0
    if (g == 0) {
        const int64_t o = c.c_bhn * L + spos;
        ddg[o] = dgk;
        const float dl = dbb * dts * dec_end;
        d_dt[o] = ddt_or + dbb * dec_end;
        g2[o] = -dsrc;
        d_delta[o] = dl;
        dA += static_cast<double>(dl) * (end - cs);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        dD += __shfl_xor(dD, off);
        dA += __shfl_xor(dA, off);
    }
    if (lane == 0) {
        sRed[wave] = dD;
        sRed[4 + wave] = dA;
    }
    __syncthreads();
    if (tid == 0) {
        dD_part[c.ch * nblk + sb] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
        dA_S[c.ch * nblk + sb] = sRed[4] + sRed[5] + sRed[6] + sRed[7];
    }
}

// ------------------------------------------------------------------ dispatch
#define SSD_FOR_EACH_PR(X) \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) \
    X(128, 16) X(128, 32) X(128, 64) X(128, 128)

template <class IO>
static hipError_t target_io(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                            const float* A, const double* cdt, const float* S, const float* dS,
                            const float* dcbt, const float* ddg, void* dC, float* g1,
                            float* d_end, double* dA_T, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH * s.nblk()));
#define X(PP, RR)                                                                                \
    if (s.P == PP && s.R == RR) {                                                                \
        hipLaunchKernelGGL((k_bwd_target<IO, PP, RR>), grid, dim3(NT), 0, st,                   \
                           static_cast<const T*>(dy), static_cast<const T*>(Bm),                 \
                           static_cast<const T*>(Cm), A, cdt, S, dS, dcbt, ddg,                  \
                           static_cast<T*>(dC), g1, d_end, dA_T, s.N, s.H, s.L, CH);             \
        return hipGetLastError();                                                                \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_target(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                             const float* A, const double* cdt, const float* S, const float* dS,
                             const float* dcbt, const float* ddg, void* dC, float* g1,
                             float* d_end, double* dA_T, hipStream_t st) {
    return s.io == 1 ? target_io<BF16>(s, dy, Bm, Cm, A, cdt, S, dS, dcbt, ddg, dC, g1, d_end, dA_T, st)
                     : target_io<F32>(s, dy, Bm, Cm, A, cdt, S, dS, dcbt, ddg, dC, g1, d_end, dA_T, st);
}

template <class IO>
static hipError_t source_io(const Shape& s, const void* dy, const void* x, const float* dt,
                            const void* Bm, const void* Cm, const float* A, const float* D,
                            const double* cdt, const float* dS, void* dx, void* dB, float* d_dt,
                            float* g2, float* d_delta, double* dA_S, double* dD_part,
                            float* dcbt, float* ddg, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(CH * s.nblk()));
#define X(PP, RR)                                                                                 \
    if (s.P == PP && s.R == RR) {                                                                 \
        hipLaunchKernelGGL((k_bwd_source<IO, PP, RR>), grid, dim3(NT), 0, st,                    \
                           static_cast<const T*>(dy), static_cast<const T*>(x), dt,               \
                           static_cast<const T*>(Bm), static_cast<const T*>(Cm), A, D, cdt, dS,   \
                           static_cast<T*>(dx), static_cast<T*>(dB), d_dt, g2, d_delta, dA_S,     \
                           dD_part, dcbt, ddg, s.N, s.H, s.L, CH);                                \
        return hipGetLastError();                                                                 \
    }
    SSD_FOR_EACH_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_source(const Shape& s, const void* dy, const void* x, const float* dt,
                             const void* Bm, const void* Cm, const float* A, const float* D,
                             const double* cdt, const float* dS, void* dx, void* dB, float* d_dt,
                             float* g2, float* d_delta, double* dA_S, double* dD_part,
                             float* dcbt, float* ddg, hipStream_t st) {
    return s.io == 1 ? source_io<BF16>(s, dy, x, dt, Bm, Cm, A, D, cdt, dS, dx, dB, d_dt, g2,
                                       d_delta, dA_S, dD_part, dcbt, ddg, st)
                     : source_io<F32>(s, dy, x, dt, Bm, Cm, A, D, cdt, dS, dx, dB, d_dt, g2,
                                      d_delta, dA_S, dD_part, dcbt, ddg, st);
}

}  // namespace ssd
