// Whole-chunk variants of two ORANGE kernels (K5 forward output and the
// backward's target rows) for 128-token chunks: one workgroup per chunk-head
// instead of one per (chunk-head, 64-token block).
//
// Page: burn-mamba "mamba2/ssd/serial_recalculated/combined_backward.rs"; the
// per-element formulas are those of k_chunk_fwd.hip (K5: BLUE + ORANGE + D x)
// and of k_bwd_target in k_chunk_bwd.hip (BLUE, ORANGE and K2 backward, K4
// backward's d_end, pair-form d_A).
//
// Why a second shape.  In a causal chunk, row tile k of 8 has k + 1 partner
// tiles as a target and 8 - k as a source.  The block kernels give each wave one
// row tile, so the waves of a workgroup carry 1..4 tiles on the diagonal block
// and wait for each other at every block change; each workgroup also re-stages
// the partner blocks it shares with the other blocks of its chunk.  Here wave w
// owns the two row tiles w and 7 - w, which as targets pair with
// (w + 1) + (8 - w) = 9 partner tiles for every wave (the fp32 K5 gives the two tiles
// to the two waves of one SIMD instead, below).  The partner rows are
// staged in two halves of 64 rows: the even 16-row tiles, then the odd ones.
// With that split every wave has 5 pair tiles in the even half and 4 in the
// odd one, so the barrier between the halves costs no waiting, and the LDS of
// one half (about 52 KB at
// (p, r) = (64, 128), shared with the chunk's p x r state of the prologue)
// leaves room for two workgroups per CU.  The source-row side keeps its block
// kernel: two row tiles of B and x operands plus the d_x and d_B accumulators
// are 192 registers per lane at (64, 128), which does not leave room for the
// rest within the 256 registers of two waves per SIMD.
//
// Layouts and the MFMA operand convention are those of ssd_device.hpp; every
// 16x16 product tile is formed with its M index along the rows the next
// product contracts over, so its registers are the next MFMA's operand.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int KC = 128;       // the chunk length these kernels take
constexpr int NRT = KC / 16;  // row tiles per chunk

// Shapes that take the whole-chunk kernels: two row tiles of operands and
// accumulators per wave must fit the 256 registers of two waves per SIMD.
template <int P, int R>
constexpr bool wide_fits() {
    return P * R <= 64 * 128;
}

// LDS floats of the main buffer: the [P, R] state, or one half of the partner rows.
template <int P, int R>
constexpr int wide_main() {
    return P * (R + 4) > TB * (R + 4) + TB * (P + 4) ? P * (R + 4) : TB * (R + 4) + TB * (P + 4);
}

template <int N>
struct Q {
    static constexpr int value = N;
};

// bf16 rows staged in four-row groups ([t / 4][feature][t % 4]): r holds rows 4q .. 4q + 3
// at features 4 f4 .. 4 f4 + 3 (raw bf16, two per word); the group entry of feature
// 4 f4 + f is those four rows' values, one 8-byte LDS word.
__device__ __forceinline__ uint2 group4(const uint2 (&r)[4], int f) {
    const int sh = (f & 1) * 16;
    const uint32_t w0 = (f < 2 ? r[0].x : r[0].y) >> sh, w1 = (f < 2 ? r[1].x : r[1].y) >> sh;
    const uint32_t w2 = (f < 2 ? r[2].x : r[2].y) >> sh, w3 = (f < 2 ? r[3].x : r[3].y) >> sh;
    return uint2{(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
}

}  // namespace

// ------------------------------------------------------------------------- K5
// fp32 io (bf16 io: k5_chunk_scan_wb below).  Eight waves, one target row tile each:
// wave w < 4 owns tile w, wave w >= 4 tile 11 - w, so the two waves that share a SIMD
// (w and w + 4) own tiles w and 7 - w, (w + 1) + (8 - w) = 9 pair tiles per SIMD.  One
// row tile's operands and accumulators fit 128 registers at (p, r) = (64, 128), so the two
// workgroups of a CU are four waves per SIMD, which hide more of each other's vector,
// LDS and barrier phases than two waves holding two tiles each (929 -> 894 us on the
// 64k-token workload, 96.9 -> 91.3 us on the 130M-shaped one).  acc[pt][v] is y[t][p]
// with t = 16 tt + 4g + v, p = 16 pt + i (BLUE e_t C_t S_in, then ORANGE, then D x).
constexpr int NT8 = 2 * NT;  // threads of the fp32 K5 workgroup
template <int P, int R>
__global__ __launch_bounds__(NT8, 2) void k5_chunk_scan_w(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ Av, const float* __restrict__ Dv,
    const double* __restrict__ cdt, const float* __restrict__ S, float* __restrict__ y, int N,
    int H) {
    constexpr int RS = R + 4, PS = P + 4, L = KC;
    __shared__ __align__(16) float sM[wide_main<P, R>()];  // S_in [P, R], then one half of B | x
    float* sB = sM;
    float* sX = sM + TB * RS;
    __shared__ __align__(16) double sCdt[KC];
    __shared__ __align__(16) float sDt[KC];
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    // the wave index as a scalar (the same in every lane of a wave): its row-tile offsets stay
    // in scalar registers (1 % faster)
    const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double la2 = static_cast<double>(Av[c.h]) * kLog2e;
    const int tt = wave < 4 ? wave : 11 - wave;
    const int tl = 16 * tt + i;

    v4f creg[R / 16];
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk)
        creg[kk] = *reinterpret_cast<const v4f*>(Cm + brow0 + static_cast<int64_t>(tl) * bstride + 16 * kk + 4 * g);
    {
        // S_in [P, R] into LDS, every load issued before the first store
        constexpr int V = R / 4, TOT = P * V, IT = (TOT + NT8 - 1) / NT8;
        const float* sp = S + c.ch * (P * R);
        v4f sv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT8;
            if (TOT % NT8 == 0 || idx < TOT) sv[it] = *reinterpret_cast<const v4f*>(sp + idx * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT8;
            if (TOT % NT8 == 0 || idx < TOT)
                *reinterpret_cast<v4f*>(sM + (idx / V) * RS + (idx % V) * 4) = sv[it];
        }
    }
    if (tid < KC) {
        sCdt[tid] = cc[tid];
        sDt[tid] = dt[c.c_bhn * L + tid];
    }
    __syncthreads();

    // One half of the source rows (LDS row 16u + e is chunk row 16 (2u + half) + e) in
    // registers, loaded while the matrix cores work, then stored after a barrier.
    constexpr int VB = R / 4, TOTB = TB * VB, ITB = (TOTB + NT8 - 1) / NT8;
    constexpr int VX = P / 4, TOTX = TB * VX, ITX = (TOTX + NT8 - 1) / NT8;
    v4f preB[ITB], preX[ITX];
    auto load_half = [&](int half) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
            const int idx = tid + it * NT8, lr = idx / VB;
            const int crow = 16 * (2 * (lr >> 4) + half) + (lr & 15);
            if (TOTB % NT8 == 0 || idx < TOTB)
                preB[it] = *reinterpret_cast<const v4f*>(Bm + brow0 + static_cast<int64_t>(crow) * bstride + (idx % VB) * 4);
        }
#pragma unroll
        for (int it = 0; it < ITX; ++it) {
            const int idx = tid + it * NT8, lr = idx / VX;
            const int crow = 16 * (2 * (lr >> 4) + half) + (lr & 15);
            if (TOTX % NT8 == 0 || idx < TOTX)
                preX[it] = *reinterpret_cast<const v4f*>(x + xrow0 + static_cast<int64_t>(crow) * xstride + (idx % VX) * 4);
        }
    };
    auto store_half = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
            const int idx = tid + it * NT8;
            if (TOTB % NT8 == 0 || idx < TOTB)
                *reinterpret_cast<v4f*>(sB + (idx / VB) * RS + (idx % VB) * 4) = preB[it];
        }
#pragma unroll
        for (int it = 0; it < ITX; ++it) {
            const int idx = tid + it * NT8;
            if (TOTX % NT8 == 0 || idx < TOTX)
                *reinterpret_cast<v4f*>(sX + (idx / VX) * PS + (idx % VX) * 4) = preX[it];
        }
    };
    // the even half of the source rows loads into registers during BLUE
    load_half(0);
    v4f acc[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) acc[pt] = zero4();
    // BLUE: A = C rows (k = r), B operand = S_in[p, r] read along r
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const v4f bop = *reinterpret_cast<const v4f*>(sM + (pt * 16 + i) * RS + 16 * kk + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[pt] = mfma16(creg[kk][v], bop[v], acc[pt]);
        }
    }
    const double ct = sCdt[tl];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float e = exp2_of(la2 * sCdt[16 * tt + 4 * g + v]);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[pt][v] *= e;
    }

    // ORANGE over source tiles j <= tt: CB^T[s, t] (lane: t = tl, s = 16j + 4g + v), its
    // decay-weighted W, then y += W x.
    auto tile = [&](int j, int u) __attribute__((always_inline)) {
        v4f cbt = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            const v4f aop = *reinterpret_cast<const v4f*>(sB + (16 * u + i) * RS + 16 * kk + 4 * g);
            cbt = mfma_k16<F32>(aop, creg[kk], cbt);
        }
        const v2d cs01 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g);
        const v2d cs23 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g + 2);
        const v4f dts = *reinterpret_cast<const v4f*>(sDt + 16 * j + 4 * g);
        const double csv[4] = {cs01.x, cs01.y, cs23.x, cs23.y};
        // the update's x operands, read before the decay math so their LDS latency overlaps it
        float xs[4][P / 16];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) xs[v][pt] = sX[(16 * u + 4 * g + v) * PS + pt * 16 + i];
        float wv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // masked pairs (s > t) take gap 0 and weight 0: arithmetic, not a branch
            const bool keep = (j < tt) || (16 * j + 4 * g + v <= tl);
            const double gap = keep ? ct - csv[v] : 0.0;
            wv[v] = cbt[v] * exp2_of(la2 * gap) * dts[v] * (keep ? 1.0f : 0.0f);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) acc[pt] = mfma16(wv[v], xs[v][pt], acc[pt]);
    };
    const float Dh = Dv[c.h];
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // the previous contents of sM are consumed
        store_half();
        __syncthreads();
        if (half == 0) load_half(1);
        // SKIP: D x of this wave's target rows if they sit in this half
        if ((tt & 1) == half)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int pt = 0; pt < P / 16; ++pt)
                    acc[pt][v] += Dh * sX[(16 * (tt >> 1) + 4 * g + v) * PS + pt * 16 + i];
        for (int u = 0; u < 4; ++u) {
            const int j = 2 * u + half;
            if (j <= tt) tile(j, u);
        }
    }

#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int64_t row = xrow0 + static_cast<int64_t>(16 * tt + 4 * g + v) * xstride;
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) st_nt<F32>(y, row + pt * 16 + i, acc[pt][v]);
    }
}

// K5 with bf16 io.  The halves' B rows are staged as bf16 row-major (stride R + 16): the
// A operand of C B^T, four features of one row.  Their x rows go in four-row groups
// (stride P + 16): the operand of W x, one feature of four rows.  The own C rows are
// packed once after BLUE.  Every MFMA operand is one 8-byte read with no conversion
// (the fp32 staging read scalars and repacked them for every MFMA).  S_in, the fp32
// operand of BLUE, is split once into its three exact bf16 parts as it is staged, so
// BLUE runs on the bf16 matrix cores too (three 16x16x16 MFMAs per 16-wide k slice
// instead of four fp32 ones at twice their time); the LDS of a half fits within that of
// the parts.  Three workgroups per CU (at most 168 registers) hide the loads of the
// halves, which fp32 io hides with a register prefetch.
template <int P, int R>
__global__ __launch_bounds__(NT, 3) void k5_chunk_scan_wb(
    const BF16::T* __restrict__ x, const float* __restrict__ dt, const BF16::T* __restrict__ Bm,
    const BF16::T* __restrict__ Cm, const float* __restrict__ Av, const float* __restrict__ Dv,
    const double* __restrict__ cdt, const float* __restrict__ S, BF16::T* __restrict__ y, int N,
    int H) {
    using IO = BF16;
    constexpr int L = KC, RB = R + 16, PB = P + 16, SB = R + 8;
    constexpr int HB = TB * RB, HX = (TB / 4) * PB * 4;  // uint16 of a half: B rows, x groups
    constexpr int SP = P * SB;                           // uint16 of one S_in part
    constexpr int MAINH = 3 * SP > HB + HX ? 3 * SP : HB + HX;
    // S_in [P, R] as its three exact bf16 parts (row stride R + 8), then one half of B | x
    __shared__ __align__(16) uint16_t sMh[MAINH];
    uint16_t* const sBr = sMh;
    uint16_t* const sXq = sBr + HB;
    __shared__ __align__(16) double sCdt[KC];
    __shared__ __align__(16) float sDt[KC];
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double la2 = static_cast<double>(Av[c.h]) * kLog2e;
    const int tt[2] = {wave, NRT - 1 - wave};
    const int tl[2] = {16 * tt[0] + i, 16 * tt[1] + i};
    auto ld_s4 = [](const uint16_t* p) __attribute__((always_inline)) {
        return *reinterpret_cast<const s4*>(p);
    };

    v4f creg[2][R / 16];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk)
            creg[q][kk] = io<IO>::ld4(Cm, brow0 + static_cast<int64_t>(tl[q]) * bstride + 16 * kk + 4 * g);
    {
        // S_in split once: each part as four-feature words, one 8-byte write per part
        constexpr int V = R / 4, TOT = P * V, IT = (TOT + NT - 1) / NT;
        const float* src = S + c.ch * (P * R);
        v4f tmp[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT) tmp[it] = *reinterpret_cast<const v4f*>(src + idx * 4);
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT) {
                const S4x3 sp = split4(tmp[it]);
                const int o = (idx / V) * SB + (idx % V) * 4;
                *reinterpret_cast<s4*>(sMh + o) = sp.hi;
                *reinterpret_cast<s4*>(sMh + SP + o) = sp.mid;
                *reinterpret_cast<s4*>(sMh + 2 * SP + o) = sp.lo;
            }
        }
    }
    if (tid < KC) {
        sCdt[tid] = cc[tid];
        sDt[tid] = dt[c.c_bhn * L + tid];
    }
    __syncthreads();

    v4f acc[2][P / 16];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) acc[q][pt] = zero4();
    s4 cpk[2][R / 16];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) cpk[q][kk] = pack_bf16x4(creg[q][kk]);
    // BLUE: A = C rows (k = r, exact), B operand = S_in[p, r] read along r (its parts)
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) {
            const int o = (pt * 16 + i) * SB + 16 * kk + 4 * g;
            const S4x3 bop{ld_s4(sMh + o), ld_s4(sMh + SP + o), ld_s4(sMh + 2 * SP + o)};
#pragma unroll
            for (int q = 0; q < 2; ++q) acc[q][pt] = mfma16_split(cpk[q][kk], bop, acc[q][pt]);
        }
    }
    double ct[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        ct[q] = sCdt[tl[q]];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float e = exp2_of(la2 * sCdt[16 * tt[q] + 4 * g + v]);
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) acc[q][pt][v] *= e;
        }
    }
    // ORANGE over source tiles j <= tt[q] (u: the tile's place in its half)
    auto tile = [&](int j, int u, auto qlo) {
        constexpr int QLO = decltype(qlo)::value;
        v4f cbt[2];
#pragma unroll
        for (int q = QLO; q < 2; ++q) cbt[q] = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            const s4 aop = ld_s4(sBr + (16 * u + i) * RB + 16 * kk + 4 * g);
#pragma unroll
            for (int q = QLO; q < 2; ++q)
                cbt[q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, cpk[q][kk], cbt[q], 0, 0, 0);
        }
        const v2d cs01 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g);
        const v2d cs23 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g + 2);
        const v4f dts = *reinterpret_cast<const v4f*>(sDt + 16 * j + 4 * g);
        const double csv[4] = {cs01.x, cs01.y, cs23.x, cs23.y};
        // the update's x operands (rows 16 j + 4g .. + 3 at p = 16 pt + i), read before the
        // decay math so their LDS latency overlaps it
        s4 xb[P / 16];
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) xb[pt] = ld_s4(sXq + ((4 * u + g) * PB + 16 * pt + i) * 4);
        float wv[2][4];
#pragma unroll
        for (int q = QLO; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // masked pairs (s > t) take gap 0 and weight 0: arithmetic, not a branch
                const bool keep = (j < tt[q]) || (16 * j + 4 * g + v <= tl[q]);
                const double gap = keep ? ct[q] - csv[v] : 0.0;
                wv[q][v] = cbt[q][v] * exp2_of(la2 * gap) * dts[v] * (keep ? 1.0f : 0.0f);
            }
        // x exact, W split once per own tile (ssd_device.hpp)
        S4x3 ws[2];
#pragma unroll
        for (int q = QLO; q < 2; ++q) ws[q] = split4(v4f{wv[q][0], wv[q][1], wv[q][2], wv[q][3]});
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int q = QLO; q < 2; ++q) acc[q][pt] = mfma16_split(ws[q], xb[pt], acc[q][pt]);
    };
    const float Dh = Dv[c.h];
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        __syncthreads();  // the previous contents of sM are consumed
        {
            // LDS row 16 u + e of the half is chunk row 16 (2u + half) + e
            auto crow = [&](int lr) { return 16 * (2 * (lr >> 4) + half) + (lr & 15); };
            constexpr int NB = TB * (R / 4), ITB = (NB + NT - 1) / NT;
            constexpr int NX = (TB / 4) * (P / 4), ITX = (NX + NT - 1) / NT;
            uint2 rb[ITB], rx[ITX][4];
#pragma unroll
            for (int it = 0; it < ITB; ++it) {
                const int idx = tid + it * NT;
                if (NB % NT == 0 || idx < NB)
                    rb[it] = *reinterpret_cast<const uint2*>(
                        Bm + brow0 + static_cast<int64_t>(crow(idx / (R / 4))) * bstride + 4 * (idx % (R / 4)));
            }
#pragma unroll
            for (int it = 0; it < ITX; ++it) {
                const int idx = tid + it * NT;
                if (NX % NT == 0 || idx < NX) {
                    const int q4 = idx / (P / 4), f4 = idx % (P / 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rx[it][e] = *reinterpret_cast<const uint2*>(
                            x + xrow0 + static_cast<int64_t>(crow(4 * q4 + e)) * xstride + 4 * f4);
                }
            }
#pragma unroll
            for (int it = 0; it < ITB; ++it) {
                const int idx = tid + it * NT;
                if (NB % NT == 0 || idx < NB)
                    *reinterpret_cast<uint2*>(sBr + (idx / (R / 4)) * RB + 4 * (idx % (R / 4))) = rb[it];
            }
#pragma unroll
            for (int it = 0; it < ITX; ++it) {
                const int idx = tid + it * NT;
                if (NX % NT == 0 || idx < NX) {
                    const int q4 = idx / (P / 4), f4 = idx % (P / 4);
#pragma unroll
                    for (int f = 0; f < 4; ++f)
                        *reinterpret_cast<uint2*>(sXq + (q4 * PB + 4 * f4 + f) * 4) = group4(rx[it], f);
                }
            }
        }
        __syncthreads();
        // SKIP: D x of this wave's target rows that sit in this half
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if ((tt[q] & 1) == half)
#pragma unroll
                for (int pt = 0; pt < P / 16; ++pt) {
                    const s4 xv = ld_s4(sXq + ((4 * (tt[q] >> 1) + g) * PB + 16 * pt + i) * 4);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[q][pt][v] += Dh * bf16_to_f32(static_cast<uint16_t>(xv[v]));
                }
        for (int u = 0; u < 4; ++u) {
            const int j = 2 * u + half;
            if (j <= tt[0]) tile(j, u, Q<0>{});
            else if (j <= tt[1]) tile(j, u, Q<1>{});
        }
    }

#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = xrow0 + static_cast<int64_t>(16 * tt[q] + 4 * g + v) * xstride;
#pragma unroll
            for (int pt = 0; pt < P / 16; ++pt) st_nt<IO>(y, row + pt * 16 + i, acc[q][pt][v]);
        }
}

// ---------------------------------------------------------- backward, rows t
// Runs after the source-row kernel, which leaves the d_CB tile of every causal pair tile
// of the chunk (pair_index order).  Wave w owns
// target tiles tt = {w, 7 - w} (9 pair tiles each); acc[q][rt][v] is d_C[t][r] with
// t = 16 tt[q] + i, r = 16 rt + 4g + v.  The whole chunk is in this workgroup, so K1's
// backward (the suffix sums of the gradient w.r.t. the within-chunk cumsum, and
// d_dt += A d_da) runs in its epilogue, on the source-row kernel's g2, d_delta and d_dt.
// LDS floats: S_in [P, R] (stride R + 4), then the chunk's B rows -- fp32 rows of stride
// R + 4, or with bf16 io four-row groups of bf16 (group stride R + 16), the layout of
// their one use, the A operand of d_C += d_CB B (one feature of four consecutive rows:
// one 8-byte read, no conversion).
// With bf16 io S_in is staged as its three exact bf16 parts in four-row groups (group
// stride R + 16), the layout of BLUE's A operand (S_in^T: one r, four consecutive p), so
// BLUE runs on the bf16 matrix cores.
template <class IO, int P, int R>
constexpr int wide_target_lds() {
    constexpr bool b16 = sizeof(typename IO::T) == 2;
    constexpr int sin = b16 ? 3 * (P / 4) * (R + 16) * 2 : P * (R + 4);
    constexpr int rows = b16 ? (KC / 4) * (R + 16) * 2 : KC * (R + 4);
    return sin > rows ? sin : rows;
}

template <class IO, int P, int R>
__global__ __launch_bounds__(NT, 2) void k_bwd_target_w(
    const typename IO::T* __restrict__ dy, const typename IO::T* __restrict__ Bm,
    const typename IO::T* __restrict__ Cm, const float* __restrict__ Av,
    const double* __restrict__ cdt, const float* __restrict__ S, const float* __restrict__ dS,
    const float* __restrict__ dcbt, const float* __restrict__ ddg, const float* __restrict__ g2,
    const float* __restrict__ d_delta, typename IO::T* __restrict__ dC, float* __restrict__ d_dt,
    double* __restrict__ dA_T, int N, int H) {
    constexpr int RS = R + 4, L = KC, NBLK = KC / TB;
    __shared__ __align__(16) float sM[wide_target_lds<IO, P, R>()];
    __shared__ __align__(16) double sCdt[KC];
    __shared__ double sG[KC];  // g1 per token: BLUE + ORANGE target side (gradient w.r.t. the cumsum)
    __shared__ double sRed[NT / 64];
    __shared__ double sDend;
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double la2 = a * kLog2e;
    const int tt[2] = {wave, NRT - 1 - wave};
    const int tl[2] = {16 * tt[0] + i, 16 * tt[1] + i};
    const int64_t tiles0 = c.ch * pair_tiles_of(L);

    v4f creg[2][R / 16], dyreg[2][P / 16];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk)
            creg[q][kk] = io<IO>::ld4(Cm, brow0 + static_cast<int64_t>(tl[q]) * bstride + 16 * kk + 4 * g);
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
            dyreg[q][kk] = io<IO>::ld4(dy, xrow0 + static_cast<int64_t>(tl[q]) * xstride + 16 * kk + 4 * g);
    }
    // S_in into LDS, and K4 backward's d_end = exp(A cdt[L-1]) <d_intra, S_in> from the
    // same registers: both matrices' loads are in flight together with the operand rows'
    double dA = 0.0;  // this thread's part of the chunk's d_A (pair form)
    constexpr bool kB16 = sizeof(typename IO::T) == 2;
    constexpr int RB = R + 16;                // bf16 group stride
    constexpr int SPG = (P / 4) * RB * 4;     // uint16 of one S_in part (bf16 io)
    uint16_t* const sMh = reinterpret_cast<uint16_t*>(sM);
    if constexpr (kB16) {
        // item (p4, r4): rows 4 p4 .. + 3 at r = 4 r4 .. + 3; each r's four p values split
        // into three parts, one 8-byte group entry per part
        constexpr int NI = (P / 4) * (R / 4), IT = (NI + NT - 1) / NT;
        const float* sp = S + c.ch * (P * R);
        const float* dsp = dS + c.ch * (P * R);
        v4f sv[IT][4], dv[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (NI % NT == 0 || idx < NI) {
                const int p4 = idx / (R / 4), r4 = idx % (R / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[it][e] = *reinterpret_cast<const v4f*>(sp + (4 * p4 + e) * R + 4 * r4);
                    dv[it][e] = *reinterpret_cast<const v4f*>(dsp + (4 * p4 + e) * R + 4 * r4);
                }
            }
        }
        double part = 0.0;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (NI % NT == 0 || idx < NI) {
                const int p4 = idx / (R / 4), r4 = idx % (R / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part += static_cast<double>(dv[it][e][0] * sv[it][e][0] + dv[it][e][1] * sv[it][e][1]) +
                            static_cast<double>(dv[it][e][2] * sv[it][e][2] + dv[it][e][3] * sv[it][e][3]);
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const S4x3 pz = split4(v4f{sv[it][0][f], sv[it][1][f], sv[it][2][f], sv[it][3][f]});
                    const int o = (p4 * RB + 4 * r4 + f) * 4;
                    *reinterpret_cast<s4*>(sMh + o) = pz.hi;
                    *reinterpret_cast<s4*>(sMh + SPG + o) = pz.mid;
                    *reinterpret_cast<s4*>(sMh + 2 * SPG + o) = pz.lo;
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) sRed[wave] = part;
    } else {
        constexpr int V = R / 4, TOT = P * V, IT = (TOT + NT - 1) / NT;
        const float* sp = S + c.ch * (P * R);
        const float* dsp = dS + c.ch * (P * R);
        v4f sv[IT], dv[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT) {
                sv[it] = *reinterpret_cast<const v4f*>(sp + idx * 4);
                dv[it] = *reinterpret_cast<const v4f*>(dsp + idx * 4);
            }
        }
        double part = 0.0;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (TOT % NT == 0 || idx < TOT) {
                *reinterpret_cast<v4f*>(sM + (idx / V) * RS + (idx % V) * 4) = sv[it];
                part += static_cast<double>(dv[it][0] * sv[it][0] + dv[it][1] * sv[it][1]) +
                        static_cast<double>(dv[it][2] * sv[it][2] + dv[it][3] * sv[it][3]);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) sRed[wave] = part;
    }
    if (tid < KC) sCdt[tid] = cc[tid];
    __syncthreads();
    if (tid == 0) {
        const double end = sCdt[L - 1];
        const double de = (sRed[0] + sRed[1] + sRed[2] + sRed[3]) * exp(a * end);
        const float def = static_cast<float>(de);
        sDend = static_cast<double>(def);
        dA += static_cast<double>(def) * end;
    }

    // BLUE: d_C^T[r, t] = e_t sum_p S_in[p, r] dy[t, p]
    v4f acc[2][R / 16];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) acc[q][rt] = zero4();
    if constexpr (kB16) {
        // dy exact, S_in as its parts: one group entry (p = 16 kk + 4g .. + 3 at r) per part
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) {
            s4 dyp[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) dyp[q] = pack_bf16x4(dyreg[q][kk]);
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt) {
                const int o = ((4 * kk + g) * RB + 16 * rt + i) * 4;
                const S4x3 sa{*reinterpret_cast<const s4*>(sMh + o), *reinterpret_cast<const s4*>(sMh + SPG + o),
                              *reinterpret_cast<const s4*>(sMh + 2 * SPG + o)};
#pragma unroll
                for (int q = 0; q < 2; ++q) acc[q][rt] = mfma16_split(sa, dyp[q], acc[q][rt]);
            }
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float sv = sM[(16 * kk + 4 * g + v) * RS + rt * 16 + i];
#pragma unroll
                    for (int q = 0; q < 2; ++q) acc[q][rt] = mfma16(sv, dyreg[q][kk][v], acc[q][rt]);
                }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const double ct = sCdt[tl[q]];
        const float et = exp2_of(la2 * ct);
        float gblue = 0.0f;  // this lane's part of the BLUE gradient w.r.t. the cumsum at t
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
            acc[q][rt] *= et;
#pragma unroll
            for (int v = 0; v < 4; ++v) gblue += creg[q][rt][v] * acc[q][rt][v];
        }
        dA += static_cast<double>(gblue) * ct;
    }

    // the wave's pair tiles in order k = 0 .. 8: (own tile tt[0], source tile k) for k <= w,
    // then (tt[1], k - w - 1); each tile's d_CB (this lane's four s of row t = 16 tt + i)
    // loads DQ tiles ahead of its products: two with bf16 io (256 -> 242 us on the
    // 2.7B-shaped workload), one with fp32 io (two spill registers there: 1074 -> 1091 us
    // on the 64k-token workload)
    auto tile_at = [&](int k) -> int64_t {
        return k <= wave ? tiles0 + pair_index(tt[0], k) : tiles0 + pair_index(tt[1], k - wave - 1);
    };
    constexpr int DQ = sizeof(typename IO::T) == 2 ? 2 : 1;
    v4f dq[DQ];
#pragma unroll
    for (int d = 0; d < DQ; ++d) dq[d] = *reinterpret_cast<const v4f*>(dcbt + tile_at(d) * 256 + i * 16 + 4 * g);
    // the chunk's B rows into LDS once S_in is consumed, every load of a thread in flight
    // before its first LDS write (one memory latency: 1105 -> 1067 us on the 64k-token
    // workload against four batches of four)
    __syncthreads();
    uint16_t* const sBq = sMh;
    if constexpr (kB16) {
        constexpr int NI = (KC / 4) * (R / 4), IT = (NI + NT - 1) / NT;
        uint2 rq[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (NI % NT == 0 || idx < NI) {
                const int q4 = idx / (R / 4), f4 = idx % (R / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rq[it][e] = *reinterpret_cast<const uint2*>(Bm + brow0 + static_cast<int64_t>(4 * q4 + e) * bstride + 4 * f4);
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NT;
            if (NI % NT == 0 || idx < NI) {
                const int q4 = idx / (R / 4), f4 = idx % (R / 4);
#pragma unroll
                for (int f = 0; f < 4; ++f) *reinterpret_cast<uint2*>(sBq + (q4 * RB + 4 * f4 + f) * 4) = group4(rq[it], f);
            }
        }
    } else {
        stage_rows<IO, R, KC, 16>(sM, Bm + brow0, bstride);
    }
    __syncthreads();
    // K2 backward: d_C^T[r, t] += sum_s B[s, r] d_CB[t, s].  The tiles hold the diagonal
    // elements d_CB[t, t] as zeros (they come in ddg), so g1 below leaves out the diagonal
    // pair's d_diff, as g2 does in the source-row kernel: in exact arithmetic the two
    // cancel, in fp32 each side rounds its own way and d_dt = ... + A d_da would carry |A|
    // times the difference.  They join d_C after g1 is taken.
    auto pair = [&](int j, v4f dcb, auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        if constexpr (sizeof(typename IO::T) == 2) {
            const S4x3 ds = split4(dcb);  // bf16 io: B exact, d_CB split (ssd_device.hpp)
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
                acc[q][rt] = mfma16_split(*reinterpret_cast<const s4*>(sBq + ((4 * j + g) * RB + 16 * rt + i) * 4),
                                          ds, acc[q][rt]);
        } else {
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[q][rt] = mfma16(sM[(16 * j + 4 * g + v) * RS + rt * 16 + i], dcb[v], acc[q][rt]);
        }
    };
    auto step = [&](int k, v4f& slot) __attribute__((always_inline)) {
        const v4f dcur = slot;
        if (k + DQ < NRT + 1) slot = *reinterpret_cast<const v4f*>(dcbt + tile_at(k + DQ) * 256 + i * 16 + 4 * g);
        if (k <= wave)
            pair(k, dcur, Q<0>{});
        else
            pair(k - wave - 1, dcur, Q<1>{});
    };
    if constexpr (DQ == 1) {
        for (int k = 0; k < NRT + 1; ++k) step(k, dq[0]);
    } else {
#pragma unroll
        for (int k = 0; k < NRT + 1; ++k) step(k, dq[k % DQ]);
    }

#pragma unroll
    for (int q = 0; q < 2; ++q) {
        // g1[t] = sum_r C[t, r] d_C[t, r]: the BLUE term plus ORANGE's target side, since
        // sum_s d_diff[t, s] = sum_s d_CB[t, s] (C_t . B_s) = C_t . (sum_s d_CB[t, s] B_s)
        // (s = t held out, above; the own C rows stay in registers: read again at this
        // point they came from HBM)
        float gsum = 0.0f;
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) gsum += creg[q][rt][v] * acc[q][rt][v];
        // then the diagonal element joins d_C: d_C[t] += d_CB[t, t] B_t, B_t from LDS (row t
        // of the chunk's B rows; with fp32 io the d_C staging below overwrites rows 0 .. 63
        // only, after tile tt[0] (< 4) has read its row, so tile tt[1]'s row is intact)
        const float dg = ddg[c.c_bhn * L + tl[q]];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) {
            if constexpr (sizeof(typename IO::T) != 4) {
                v4f bt;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    bt[v] = bf16_to_f32(sBq[((tl[q] >> 2) * RB + 16 * rt + 4 * g + v) * 4 + (tl[q] & 3)]);
                acc[q][rt] += dg * bt;
            } else {
                acc[q][rt] += dg * *reinterpret_cast<const v4f*>(sM + tl[q] * RS + rt * 16 + 4 * g);
            }
        }
        if constexpr (sizeof(typename IO::T) != 4) {
            const int64_t row = brow0 + static_cast<int64_t>(tl[q]) * bstride;
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt) io<IO>::st4(dC, row + rt * 16 + 4 * g, acc[q][rt]);
        } else {
            // fp32 io: the tile's d_C rows leave through LDS so that each non-temporal
            // store instruction writes whole rows (scattered 64-byte row pieces wrote 20 %
            // more bytes than the output holds)
            __syncthreads();  // sM's previous contents are consumed
#pragma unroll
            for (int rt = 0; rt < R / 16; ++rt)
                *reinterpret_cast<v4f*>(sM + (16 * wave + i) * RS + rt * 16 + 4 * g) = acc[q][rt];
            __syncthreads();
            const int64_t row0 = brow0 + static_cast<int64_t>(16 * tt[q]) * bstride;
#pragma unroll
            for (int k = lane; k < 16 * (R / 4); k += 64) {
                const int r_ = k / (R / 4), c4 = k % (R / 4);
                st4_nt<IO>(dC, row0 + r_ * bstride + c4 * 4,
                           *reinterpret_cast<const v4f*>(sM + (16 * wave + r_) * RS + c4 * 4));
            }
        }
        const float gs = sum_over_g(gsum);
        if (g == 0) sG[tl[q]] = static_cast<double>(gs);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dA += __shfl_xor(dA, off);
    __syncthreads();  // sG complete
    if (lane == 0) sRed[wave] = dA;
    if (wave == 0) {
        // K1 backward over the chunk (lane j owns tokens 2j, 2j + 1): with g = g1 + g2 the
        // gradient w.r.t. the cumsum and d_delta that w.r.t. the decay exponents end - cumsum,
        //   d_da[t] = sum_{k>=t} g[k] + sum_{k<t} d_delta[k] + d_end,   d_dt[t] += A d_da[t]
        const int64_t base = c.c_bhn * L + 2 * lane;
        const float2 g2v = *reinterpret_cast<const float2*>(g2 + base);
        const float2 dlv = *reinterpret_cast<const float2*>(d_delta + base);
        const float2 ddt = *reinterpret_cast<const float2*>(d_dt + base);
        const double gv0 = sG[2 * lane] + static_cast<double>(g2v.x);
        const double gv1 = sG[2 * lane + 1] + static_cast<double>(g2v.y);
        const double dl0 = static_cast<double>(dlv.x), dl1 = static_cast<double>(dlv.y);
        double suf = gv0 + gv1, pre = dl0 + dl1;  // this lane's totals, then scans over lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double o1 = __shfl_down(suf, off);
            const double o2 = __shfl_up(pre, off);
            if (lane + off < 64) suf += o1;
            if (lane >= off) pre += o2;
        }
        double after = __shfl_down(suf, 1);  // sum of g over the later lanes
        if (lane == 63) after = 0.0;
        double before = __shfl_up(pre, 1);   // sum of d_delta over the earlier lanes
        if (lane == 0) before = 0.0;
        const double dend = sDend;
        const double dda1 = after + gv1 + before + dl0 + dend;
        const double dda0 = after + gv1 + gv0 + before + dend;
        *reinterpret_cast<float2*>(d_dt + base) =
            float2{static_cast<float>(static_cast<double>(ddt.x) + a * dda0),
                   static_cast<float>(static_cast<double>(ddt.y) + a * dda1)};
    }
    __syncthreads();
    if (tid == 0) {
        // one partial per 64-token block slot: the chunk's total in the first, zeros after
        dA_T[c.ch * NBLK] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
        for (int b = 1; b < NBLK; ++b) dA_T[c.ch * NBLK + b] = 0.0;
    }
}

// ---------------------------------------------------------- backward, rows s
// Whole-chunk source-row kernel: one 8-wave workgroup per chunk-head.  The chunk's
// d_intra, then its C and dy rows, are staged into LDS once (the block kernel's second
// 64-row block read d_intra and the partner rows again), and the pair tiles are spread
// so that the two waves sharing a SIMD carry 9 tiles together.  Source tile s has
// 8 - s target tiles.  Wave w < 4 owns source tile w and its first five target tiles;
// wave w >= 4 owns source tile 11 - w (7, 6, 5, 4: w - 3 tiles) and, for w < 7, forms the
// remaining targets of source tile w - 4 (tiles w + 1 .. 7) as a partial that it hands
// to wave w - 4 through LDS.  Waves w and w + 4 (one SIMD, as the dispatcher places a
// workgroup's waves round-robin) then carry 5 + 4 tiles.  Per-element formulas: those
// of k_bwd_source (k_chunk_bwd.hip).
//
// bf16 io only.  The LDS of a whole chunk leaves one workgroup per CU, so nothing
// overlaps its loads at the start of a chunk-head with matrix work.  With bf16 io the
// block kernel is bound by its vector work (decays, splits, operand packing), which the
// balance here cuts (2.7B-shaped workload: 589 -> 538 us); with fp32 io the block kernel's
// two workgroups per CU overlap one another's loads, and this shape was slower there
// (64k-token workload: 1.95 -> 2.26 ms).
constexpr int NTS = 512;      // threads of the whole-chunk source kernel
constexpr int NWS = NTS / 64; // its waves

// The chunk's C and dy rows are staged as bf16 twice: row-major (row stride w + 16) for
// the C B^T and dy x^T tiles, whose A operand is four consecutive features of one row,
// and in four-row groups ([t / 4][feature][t % 4], group stride w + 16) for the output
// products, whose A operand is one feature of four consecutive rows: every MFMA operand
// is then one 8-byte LDS read with no conversion (the fp32 staging read four scalars
// and repacked them for every MFMA).  The paddings spread a wave's 8-byte reads over
// the banks evenly.
template <int P, int R>
struct SrcWLds {
    static constexpr int RB = R + 16, PB = P + 16;                // bf16 row / group strides
    static constexpr int CR = KC * RB, DR = KC * PB;              // row-major C, dy (uint16)
    static constexpr int CQ = (KC / 4) * RB * 4, DQ = (KC / 4) * PB * 4;  // grouped C, dy
    // K3's d_intra [P, R] as its three exact bf16 parts, row-major (row stride R + 8) and in
    // four-row groups (group stride R + 16), where the rows go later
    static constexpr int IR = P * (R + 8), IQ = (P / 4) * RB * 4;
    static constexpr int ROWS = CR + DR + CQ + DQ, PARTS = 3 * (IR + IQ);
    static constexpr int TOTAL = ROWS > PARTS ? ROWS : PARTS;
};

template <int P, int R>
__global__ __launch_bounds__(NTS, 1) void k_bwd_source_w(
    const BF16::T* __restrict__ dy, const BF16::T* __restrict__ x,
    const float* __restrict__ dt, const BF16::T* __restrict__ Bm,
    const BF16::T* __restrict__ Cm, const float* __restrict__ Av,
    const float* __restrict__ Dv, const double* __restrict__ cdt, const float* __restrict__ dS,
    BF16::T* __restrict__ dx, BF16::T* __restrict__ dB, float* __restrict__ d_dt,
    float* __restrict__ g2, float* __restrict__ d_delta, double* __restrict__ dA_S,
    double* __restrict__ dD_part, float* __restrict__ dcbt, float* __restrict__ ddg, int N, int H) {
    using IO = BF16;
    using LY = SrcWLds<P, R>;
    constexpr int RB = LY::RB, PB = LY::PB, IRS = R + 8, L = KC, NBLK = KC / TB;
    constexpr int NEX = 4 * (P / 16 + R / 16) + 2;  // floats per lane of one handed-over partial
    __shared__ __align__(16) uint16_t sMb[LY::TOTAL];
    uint16_t* const sCr = sMb;
    uint16_t* const sDr = sCr + LY::CR;
    uint16_t* const sCq = sDr + LY::DR;
    uint16_t* const sDq = sCq + LY::CQ;
    uint16_t* const sIr = sMb;                // d_intra's parts during K3: row-major ...
    uint16_t* const sIq = sMb + 3 * LY::IR;   // ... and in four-row groups
    __shared__ float sPart[3 * NEX * 64];
    __shared__ __align__(16) double sCdt[KC];
    __shared__ double sRed[2 * NWS];
    const ChunkHead c = decode_ch(blockIdx.x, N, H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(P);
    const int64_t xstride = static_cast<int64_t>(H) * P;
    const int64_t brow0 = (c.bn * L * H + c.h) * static_cast<int64_t>(R);
    const int64_t bstride = static_cast<int64_t>(H) * R;
    const double* cc = cdt + c.c_bhn * L;
    const float* dtc = dt + c.c_bhn * L;
    const double a = static_cast<double>(Av[c.h]);
    const double la2 = a * kLog2e;
    const int so = wave < 4 ? wave : 11 - wave;  // own source tile
    const int spos = 16 * so + i;                // this lane's source row in the chunk
    const int64_t tiles0 = c.ch * pair_tiles_of(L);
    // 8-byte LDS operand: four bf16
    auto ld_s4 = [](const uint16_t* p) __attribute__((always_inline)) {
        return *reinterpret_cast<const s4*>(p);
    };

    v4f xreg[P / 16], breg[R / 16];
    const int64_t xrow = xrow0 + static_cast<int64_t>(spos) * xstride;
    const int64_t brow = brow0 + static_cast<int64_t>(spos) * bstride;
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) xreg[kk] = io<IO>::ld4(x, xrow + 16 * kk + 4 * g);
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) breg[kk] = io<IO>::ld4(Bm, brow + 16 * kk + 4 * g);
    {
        // d_intra split once into its three exact bf16 parts: item (p4, r4) is rows
        // 4 p4 .. + 3 at r = 4 r4 .. + 3; its rows go to the row-major parts, its columns
        // to the grouped ones
        constexpr int NI = (P / 4) * (R / 4), IT = (NI + NTS - 1) / NTS;
        const float* src = dS + c.ch * (P * R);
        v4f tmp[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NTS;
            if (NI % NTS == 0 || idx < NI) {
                const int p4 = idx / (R / 4), r4 = idx % (R / 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) tmp[it][e] = *reinterpret_cast<const v4f*>(src + (4 * p4 + e) * R + 4 * r4);
            }
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int idx = tid + it * NTS;
            if (NI % NTS == 0 || idx < NI) {
                const int p4 = idx / (R / 4), r4 = idx % (R / 4);
                Split3 sp[4][4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int f = 0; f < 4; ++f) sp[e][f] = split3(tmp[it][e][f]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int o = (4 * p4 + e) * IRS + 4 * r4;
                    *reinterpret_cast<s4*>(sIr + o) = s4{short(sp[e][0].hi), short(sp[e][1].hi), short(sp[e][2].hi), short(sp[e][3].hi)};
                    *reinterpret_cast<s4*>(sIr + LY::IR + o) = s4{short(sp[e][0].mid), short(sp[e][1].mid), short(sp[e][2].mid), short(sp[e][3].mid)};
                    *reinterpret_cast<s4*>(sIr + 2 * LY::IR + o) = s4{short(sp[e][0].lo), short(sp[e][1].lo), short(sp[e][2].lo), short(sp[e][3].lo)};
                }
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int o = (p4 * RB + 4 * r4 + f) * 4;
                    *reinterpret_cast<s4*>(sIq + o) = s4{short(sp[0][f].hi), short(sp[1][f].hi), short(sp[2][f].hi), short(sp[3][f].hi)};
                    *reinterpret_cast<s4*>(sIq + LY::IQ + o) = s4{short(sp[0][f].mid), short(sp[1][f].mid), short(sp[2][f].mid), short(sp[3][f].mid)};
                    *reinterpret_cast<s4*>(sIq + 2 * LY::IQ + o) = s4{short(sp[0][f].lo), short(sp[1][f].lo), short(sp[2][f].lo), short(sp[3][f].lo)};
                }
            }
        }
    }
    if (tid < KC) sCdt[tid] = cc[tid];
    const double end = cc[L - 1];
    const double cs = cc[spos];
    const float dts = dtc[spos];
    const float dec_end = expf(static_cast<float>(a * (end - cs)));
    const float bbar = dts * dec_end;
    __syncthreads();
    // the chunk's C and dy rows load during K3, as raw bf16: item (row group q4, feature
    // group f4) is rows 4 q4 .. 4 q4 + 3 at features 4 f4 .. 4 f4 + 3
    constexpr int NIC = (KC / 4) * (R / 4), ITC = (NIC + NTS - 1) / NTS;
    constexpr int NID = (KC / 4) * (P / 4), ITD = (NID + NTS - 1) / NTS;
    uint2 pc[ITC][4], pd[ITD][4];
#pragma unroll
    for (int it = 0; it < ITC; ++it) {
        const int idx = tid + it * NTS;
        if (NIC % NTS == 0 || idx < NIC) {
            const int q4 = idx / (R / 4), f4 = idx % (R / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pc[it][e] = *reinterpret_cast<const uint2*>(Cm + brow0 + static_cast<int64_t>(4 * q4 + e) * bstride + 4 * f4);
        }
    }
#pragma unroll
    for (int it = 0; it < ITD; ++it) {
        const int idx = tid + it * NTS;
        if (NID % NTS == 0 || idx < NID) {
            const int q4 = idx / (P / 4), f4 = idx % (P / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pd[it][e] = *reinterpret_cast<const uint2*>(dy + xrow0 + static_cast<int64_t>(4 * q4 + e) * xstride + 4 * f4);
        }
    }

    // the own rows feed only bf16 MFMAs: packed once
    s4 xpk[P / 16], bpk[R / 16];
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) xpk[kk] = pack_bf16x4(xreg[kk]);
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk) bpk[kk] = pack_bf16x4(breg[kk]);
    auto parts = [&](const uint16_t* p0, int stride_parts, int o) __attribute__((always_inline)) {
        return S4x3{ld_s4(p0 + o), ld_s4(p0 + stride_parts + o), ld_s4(p0 + 2 * stride_parts + o)};
    };
    // K3 backward.  d_b_scaled^T[r, s] = sum_p d_intra[p, r] x[s, p]: A = d_intra^T (one r,
    // four consecutive p: a group entry), x exact
    v4f accB[R / 16];
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) accB[rt] = zero4();
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
            accB[rt] = mfma16_split(parts(sIq, LY::IQ, ((4 * kk + g) * RB + 16 * rt + i) * 4), xpk[kk], accB[rt]);
    float dbb = 0.0f;  // d_bbar[s] = sum_r d_b_scaled[s, r] B[s, r] (this lane's part)
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) dbb += accB[rt][v] * breg[rt][v];
        accB[rt] *= bbar;
    }
    // d_x^T[p, s] = bbar[s] sum_r d_intra[p, r] B[s, r]: A = d_intra (one p, four
    // consecutive r: a row-major word), B exact
    v4f accX[P / 16];
#pragma unroll
    for (int pt = 0; pt < P / 16; ++pt) accX[pt] = zero4();
#pragma unroll
    for (int kk = 0; kk < R / 16; ++kk)
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
            accX[pt] = mfma16_split(parts(sIr, LY::IR, (pt * 16 + i) * IRS + 16 * kk + 4 * g), bpk[kk], accX[pt]);
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
    __syncthreads();  // K3 is done with d_intra
#pragma unroll
    for (int it = 0; it < ITC; ++it) {
        const int idx = tid + it * NTS;
        if (NIC % NTS == 0 || idx < NIC) {
            const int q4 = idx / (R / 4), f4 = idx % (R / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<uint2*>(sCr + (4 * q4 + e) * RB + 4 * f4) = pc[it][e];
#pragma unroll
            for (int f = 0; f < 4; ++f) *reinterpret_cast<uint2*>(sCq + (q4 * RB + 4 * f4 + f) * 4) = group4(pc[it], f);
        }
    }
#pragma unroll
    for (int it = 0; it < ITD; ++it) {
        const int idx = tid + it * NTS;
        if (NID % NTS == 0 || idx < NID) {
            const int q4 = idx / (P / 4), f4 = idx % (P / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) *reinterpret_cast<uint2*>(sDr + (4 * q4 + e) * PB + 4 * f4) = pd[it][e];
#pragma unroll
            for (int f = 0; f < 4; ++f) *reinterpret_cast<uint2*>(sDq + (q4 * PB + 4 * f4 + f) * 4) = group4(pd[it], f);
        }
    }
    __syncthreads();

    double dA = 0.0;  // this lane's part of the chunk's d_A (the pair terms and K3)
    float dgk = 0.0f;  // d_CB[s, s] of this lane's source row, on the lane whose tile holds it
    // One (target tile j, source tile s) pair, j >= s: the source tile's packed operands
    // xr / br, cumsum csr and dt dtr of this lane's source row 16 s + i, its accumulators.
    // The pair's d_CB tile goes to the target-row kernel.
    auto tile = [&](int j, int s, const s4 (&xr)[P / 16], const s4 (&br)[R / 16], double csr,
                    float dtr, v4f (&aX)[P / 16], v4f (&aB)[R / 16], float& ddt,
                    float& dsr) __attribute__((always_inline)) {
        // tiles with M = t (16j + 4g + v), N = s: exact bf16 products
        v4f cb = zero4(), dw = zero4();
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk)
            cb = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ld_s4(sCr + (16 * j + i) * RB + 16 * kk + 4 * g),
                                                          br[kk], cb, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
            dw = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ld_s4(sDr + (16 * j + i) * PB + 16 * kk + 4 * g),
                                                          xr[kk], dw, 0, 0, 0);
        const v2d ct01 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g);
        const v2d ct23 = *reinterpret_cast<const v2d*>(sCdt + 16 * j + 4 * g + 2);
        const double ctv[4] = {ct01.x, ct01.y, ct23.x, ct23.y};
        float* const tdst = dcbt + (tiles0 + pair_index(j, s)) * 256;
        float wv[4], dcb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const bool keep = 16 * j + 4 * g + v >= 16 * s + i;
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
            const bool diag = 16 * j + 4 * g + v == 16 * s + i;
            dsr += diag ? 0.0f : dd;
            dA += static_cast<double>(dd) * gap;
            tdst[(4 * g + v) * 16 + i] = diag ? 0.0f : dcb[v];
            dgk = diag ? dcb[v] : dgk;
        }
        // W and d_CB split once into three exact bf16 parts; dy and C exact
        const S4x3 ws = split4(v4f{wv[0], wv[1], wv[2], wv[3]});
        const S4x3 ds = split4(v4f{dcb[0], dcb[1], dcb[2], dcb[3]});
        // ORANGE: d_x^T[p, s] += sum_t dy[t, p] W[t, s]
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
            aX[pt] = mfma16_split(ld_s4(sDq + ((4 * j + g) * PB + 16 * pt + i) * 4), ws, aX[pt]);
        // K2 backward: d_B^T[r, s] += sum_t C[t, r] d_CB[t, s]
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
            aB[rt] = mfma16_split(ld_s4(sCq + ((4 * j + g) * RB + 16 * rt + i) * 4), ds, aB[rt]);
    };
    float ddt_or = 0.0f, dsrc = 0.0f;
    const int jend = wave < 4 ? so + 4 : NRT - 1;
    for (int j = so; j <= jend; ++j) tile(j, so, xpk, bpk, cs, dts, accX, accB, ddt_or, dsrc);

    // The own tile's outputs: d_x and d_B rows (stored from the accumulators: staging them
    // through LDS for whole-row stores was 4 % slower), and per row d_dt (ORANGE + K3), g2,
    // d_delta and the K3 term of d_A.
    auto finalize = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt) io<IO>::st4(dx, xrow + pt * 16 + 4 * g, accX[pt]);
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt) io<IO>::st4(dB, brow + rt * 16 + 4 * g, accB[rt]);
        const float db = sum_over_g(dbb);
        const float dto = sum_over_g(ddt_or);
        const float dsc = sum_over_g(dsrc);
        const float dgs = sum_over_g(dgk);  // one lane of the four holds it, the others 0
        if (g == 0) {
            const int64_t o = c.c_bhn * L + spos;
            const float dl = db * dts * dec_end;
            d_dt[o] = dto + db * dec_end;
            g2[o] = -dsc;
            ddg[o] = dgs;
            d_delta[o] = dl;
            dA += static_cast<double>(dl) * (end - cs);
        }
    };
    if (wave >= 4 && wave < 7) {
        // source tiles 7, 6, 5 are complete: their outputs leave before this wave forms
        // the partial of source tile s2 = w - 4 (its targets s2 + 5 .. 7) for wave s2
        finalize();
        const int s2 = wave - 4, sp2 = 16 * s2 + i;
        s4 x2[P / 16], b2[R / 16];
        v4f aX2[P / 16], aB2[R / 16];
        const int64_t xr2 = xrow0 + static_cast<int64_t>(sp2) * xstride;
        const int64_t br2 = brow0 + static_cast<int64_t>(sp2) * bstride;
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk) {
            x2[kk] = *reinterpret_cast<const s4*>(x + xr2 + 16 * kk + 4 * g);
            aX2[kk] = zero4();
        }
#pragma unroll
        for (int kk = 0; kk < R / 16; ++kk) {
            b2[kk] = *reinterpret_cast<const s4*>(Bm + br2 + 16 * kk + 4 * g);
            aB2[kk] = zero4();
        }
        const double cs2 = sCdt[sp2];
        const float dt2 = dtc[sp2];
        float ddt2 = 0.0f, dsr2 = 0.0f;
        for (int j = s2 + 5; j < NRT; ++j) tile(j, s2, x2, b2, cs2, dt2, aX2, aB2, ddt2, dsr2);
        float* const pp = sPart + s2 * (NEX * 64);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v) pp[(4 * pt + v) * 64 + lane] = aX2[pt][v];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) pp[(4 * (P / 16) + 4 * rt + v) * 64 + lane] = aB2[rt][v];
        pp[(NEX - 2) * 64 + lane] = ddt2;
        pp[(NEX - 1) * 64 + lane] = dsr2;
    }
    __syncthreads();  // every pair tile is done, the partials are in
    if (wave < 3) {
        const float* pp = sPart + wave * (NEX * 64);
#pragma unroll
        for (int pt = 0; pt < P / 16; ++pt)
#pragma unroll
            for (int v = 0; v < 4; ++v) accX[pt][v] += pp[(4 * pt + v) * 64 + lane];
#pragma unroll
        for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) accB[rt][v] += pp[(4 * (P / 16) + 4 * rt + v) * 64 + lane];
        ddt_or += pp[(NEX - 2) * 64 + lane];
        dsrc += pp[(NEX - 1) * 64 + lane];
    }
    if (wave < 4 || wave == 7) finalize();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        dD += __shfl_xor(dD, off);
        dA += __shfl_xor(dA, off);
    }
    if (lane == 0) {
        sRed[wave] = dD;
        sRed[NWS + wave] = dA;
    }
    __syncthreads();
    if (tid == 0) {
        // one partial per 64-token block slot: the chunk's total in the first, zeros after
        double sd = 0.0, sa = 0.0;
        for (int w = 0; w < NWS; ++w) {
            sd += sRed[w];
            sa += sRed[NWS + w];
        }
        dD_part[c.ch * NBLK] = sd;
        dA_S[c.ch * NBLK] = sa;
        for (int b = 1; b < NBLK; ++b) {
            dD_part[c.ch * NBLK + b] = 0.0;
            dA_S[c.ch * NBLK + b] = 0.0;
        }
    }
}

// ------------------------------------------------------------------ dispatch
#define SSD_WIDE_PR(X) \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) \
    X(32, 16) X(32, 32) X(32, 64) X(32, 128) \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) \
    X(128, 16) X(128, 32) X(128, 64) X(128, 128)

bool wide_supported(const Shape& s) {
    if (s.L != KC) return false;
#define X(PP, RR) \
    if (s.P == PP && s.R == RR) return wide_fits<PP, RR>();
    SSD_WIDE_PR(X)
#undef X
    return false;
}

template <class IO>
static hipError_t k5_wide_io(const Shape& s, const void* x, const float* dt, const void* Bm,
                             const void* Cm, const float* A, const float* D, const double* cdt,
                             const float* S, void* y, hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
#define X(PP, RR)                                                                                 \
    if (s.P == PP && s.R == RR) {                                                                 \
        if constexpr (wide_fits<PP, RR>()) {                                                      \
            if constexpr (sizeof(T) == 2)                                                         \
                hipLaunchKernelGGL((k5_chunk_scan_wb<PP, RR>), dim3(static_cast<unsigned>(CH)),   \
                                   dim3(NT), 0, st, static_cast<const T*>(x), dt,                 \
                                   static_cast<const T*>(Bm), static_cast<const T*>(Cm), A, D,    \
                                   cdt, S, static_cast<T*>(y), s.N, s.H);                         \
            else                                                                                  \
                hipLaunchKernelGGL((k5_chunk_scan_w<PP, RR>), dim3(static_cast<unsigned>(CH)),     \
                                   dim3(NT8), 0, st, static_cast<const float*>(x), dt,            \
                                   static_cast<const float*>(Bm), static_cast<const float*>(Cm),  \
                                   A, D, cdt, S, static_cast<float*>(y), s.N, s.H);               \
            return hipGetLastError();                                                             \
        }                                                                                         \
        return hipErrorInvalidValue;                                                              \
    }
    SSD_WIDE_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_k5_scan_wide(const Shape& s, const void* x, const float* dt, const void* Bm,
                               const void* Cm, const float* A, const float* D, const double* cdt,
                               const float* S, void* y, hipStream_t st) {
    return s.io == 1 ? k5_wide_io<BF16>(s, x, dt, Bm, Cm, A, D, cdt, S, y, st)
                     : k5_wide_io<F32>(s, x, dt, Bm, Cm, A, D, cdt, S, y, st);
}

template <class IO>
static hipError_t target_wide_io(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                                 const float* A, const double* cdt, const float* S, const float* dS,
                                 const float* dcbt, const float* ddg, const float* g2,
                                 const float* d_delta, void* dC, float* d_dt, double* dA_T,
                                 hipStream_t st) {
    using T = typename IO::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
#define X(PP, RR)                                                                                  \
    if (s.P == PP && s.R == RR) {                                                                  \
        if constexpr (wide_fits<PP, RR>()) {                                                       \
            hipLaunchKernelGGL((k_bwd_target_w<IO, PP, RR>), dim3(static_cast<unsigned>(CH)),      \
                               dim3(NT), 0, st, static_cast<const T*>(dy),                         \
                               static_cast<const T*>(Bm), static_cast<const T*>(Cm), A, cdt, S,    \
                               dS, dcbt, ddg, g2, d_delta, static_cast<T*>(dC), d_dt, dA_T, s.N,   \
                               s.H);                                                               \
            return hipGetLastError();                                                              \
        }                                                                                          \
        return hipErrorInvalidValue;                                                               \
    }
    SSD_WIDE_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_target_wide(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                                  const float* A, const double* cdt, const float* S,
                                  const float* dS, const float* dcbt, const float* ddg,
                                  const float* g2, const float* d_delta, void* dC, float* d_dt,
                                  double* dA_T, hipStream_t st) {
    return s.io == 1 ? target_wide_io<BF16>(s, dy, Bm, Cm, A, cdt, S, dS, dcbt, ddg, g2, d_delta,
                                            dC, d_dt, dA_T, st)
                     : target_wide_io<F32>(s, dy, Bm, Cm, A, cdt, S, dS, dcbt, ddg, g2, d_delta,
                                           dC, d_dt, dA_T, st);
}


static hipError_t source_wide_bf16(const Shape& s, const void* dy, const void* x, const float* dt,
                                 const void* Bm, const void* Cm, const float* A, const float* D,
                                 const double* cdt, const float* dS, void* dx, void* dB,
                                 float* d_dt, float* g2, float* d_delta, double* dA_S,
                                 double* dD_part, float* dcbt, float* ddg, hipStream_t st) {
    using T = BF16::T;
    const int64_t CH = static_cast<int64_t>(s.B) * s.N * s.H;
    if (CH == 0) return hipSuccess;
#define X(PP, RR)                                                                                 \
    if (s.P == PP && s.R == RR) {                                                                 \
        if constexpr (wide_fits<PP, RR>()) {                                                      \
            hipLaunchKernelGGL((k_bwd_source_w<PP, RR>), dim3(static_cast<unsigned>(CH)),     \
                               dim3(NTS), 0, st, static_cast<const T*>(dy),                       \
                               static_cast<const T*>(x), dt, static_cast<const T*>(Bm),           \
                               static_cast<const T*>(Cm), A, D, cdt, dS, static_cast<T*>(dx),     \
                               static_cast<T*>(dB), d_dt, g2, d_delta, dA_S, dD_part, dcbt, ddg,  \
                               s.N, s.H);                                                         \
            return hipGetLastError();                                                             \
        }                                                                                         \
        return hipErrorInvalidValue;                                                              \
    }
    SSD_WIDE_PR(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_source_wide(const Shape& s, const void* dy, const void* x, const float* dt,
                                  const void* Bm, const void* Cm, const float* A, const float* D,
                                  const double* cdt, const float* dS, void* dx, void* dB,
                                  float* d_dt, float* g2, float* d_delta, double* dA_S,
                                  double* dD_part, float* dcbt, float* ddg, hipStream_t st) {
    if (s.io != 1) return hipErrorInvalidValue;  // bf16 io only (see the kernel)
    return source_wide_bf16(s, dy, x, dt, Bm, Cm, A, D, cdt, dS, dx, dB, d_dt, g2, d_delta, dA_S,
                            dD_part, dcbt, ddg, st);
}

}  // namespace ssd
