// Device-side building blocks shared by the SSD kernels (gfx950, wave64).
//
// Tiling convention used by every chunk kernel: a chunk of l tokens is split
// into blocks of TB = 64 tokens; a workgroup has 4 wave64s and wave w owns the
// 16 token rows [16w, 16w+16) of its block.  Matrix products use the fp32
// MFMA v_mfma_f32_16x16x4_f32: for lane L (i = L % 16, g = L / 16) the
// A operand is A[i][k = g], the B operand B[k = g][i], and the four result
// registers hold D[4g + v][i], v = 0..3.  Four MFMAs that take element v of a
// float4 read at k = 4g .. 4g+3 cover 16 consecutive k exactly once (the k
// order inside the group is permuted identically on both operands, which a
// sum does not see).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int TB = 64;   // tokens per block
constexpr int NT = 256;  // threads per workgroup

__device__ __forceinline__ v4f mfma16(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f zero4() { return v4f{0.f, 0.f, 0.f, 0.f}; }

typedef double v2d __attribute__((ext_vector_type(2)));

// Decay factors exp(a * gap), gap an fp64 difference of cumulative sums of dt:
// the caller forms the base-2 exponent (a log2 e) * gap in fp64; it is rounded
// once to fp32 and raised with the hardware base-2 exponential (v_exp_f32,
// about 1 ulp).  Results below the fp32 range flush to 0.
constexpr double kLog2e = 1.4426950408889634;
__device__ __forceinline__ float exp2_of(double e2) {
    return __builtin_amdgcn_exp2f(static_cast<float>(e2));
}

// ------------------------------------------------------------------ io types
struct F32;
struct BF16;
typedef short s4 __attribute__((ext_vector_type(4)));

// fp32 values exact in bf16 (widened bf16 inputs) -> four packed bf16 (exact).
__device__ __forceinline__ s4 pack_bf16x4(v4f a) {
    return s4{static_cast<short>(__float_as_uint(a[0]) >> 16),
              static_cast<short>(__float_as_uint(a[1]) >> 16),
              static_cast<short>(__float_as_uint(a[2]) >> 16),
              static_cast<short>(__float_as_uint(a[3]) >> 16)};
}

// One 16-wide k slice of a 16x16 product whose two operands are float4s of this
// lane (k = 4g + v, v = 0..3, on both sides): four fp32 16x16x4 MFMAs -- or, for
// a bf16 workload when both operands are (widened) bf16 inputs, one bf16
// 16x16x16 MFMA, whose lane holds exactly those four k values of each operand
// and whose result layout is the same: exact products, fp32 accumulation, a
// sixteenth of the fp32 matrix-core time on gfx950.
template <class IO>
__device__ __forceinline__ v4f mfma_k16(v4f a, v4f b, v4f c) {
    if constexpr (__is_same(IO, BF16)) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pack_bf16x4(a), pack_bf16x4(b), c, 0, 0, 0);
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) c = mfma16(a[v], b[v], c);
        return c;
    }
}

// ------------------------------------------------- bf16 matrix cores, fp32 operands
// A product with one operand of exact bf16 values (the bf16 workloads' x, B, C, dy)
// and one fp32 operand (a state, a decay-weighted tile, a gradient) runs on the bf16
// matrix cores without narrowing anything: the fp32 operand is split exactly into
// three bf16 parts, x = hi + mid + lo, each bf16 x bf16 product is exact in fp32, and
// the three products accumulate in fp32.  hi keeps the sign, the exponent and the top
// 7 fraction bits (a truncation, so x - hi is exact in fp32 with at most 16
// significant bits); the same step on that remainder leaves at most 8 significant
// bits, which bf16 holds exactly.  Only parts below bf16's normal range (|x| < about
// 2^-110) are lost.  On gfx950 a 16x16x32 bf16 MFMA issues in about the time of two
// thirds of one fp32 16x16x4 MFMA's (measured 7.2 against 14 ns per SIMD), so a 32-wide
// k slice takes three of them instead of eight fp32 ones.
typedef __bf16 b8v __attribute__((ext_vector_type(8)));

struct Split3 {
    uint16_t hi, mid, lo;
};
__device__ __forceinline__ Split3 split3(float x) {
    const uint32_t h = __float_as_uint(x) & 0xffff0000u;
    const float r1 = x - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(m);
    return Split3{static_cast<uint16_t>(h >> 16), static_cast<uint16_t>(m >> 16),
                  static_cast<uint16_t>(__float_as_uint(r2) >> 16)};
}

// The same on the 16x16x16 bf16 MFMA (k slices of 16, four k values per lane, the layout
// of four fp32 16x16x4 MFMAs): an fp32 operand tile split once into three packed parts,
// reused against every exact-bf16 operand it meets.
struct S4x3 {
    s4 hi, mid, lo;
};
__device__ __forceinline__ S4x3 split4(v4f b) {
    S4x3 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const Split3 sp = split3(b[e]);
        o.hi[e] = static_cast<short>(sp.hi);
        o.mid[e] = static_cast<short>(sp.mid);
        o.lo[e] = static_cast<short>(sp.lo);
    }
    return o;
}
// a (exact bf16) x b (fp32, split) and a (fp32, split) x b (exact bf16)
__device__ __forceinline__ v4f mfma16_split(s4 a, const S4x3& b, v4f c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b.mid, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b.hi, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma16_split(const S4x3& a, s4 b, v4f c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.mid, b, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b, c, 0, 0, 0);
}

struct F32 {
    using T = float;
};
struct BF16 {
    using T = uint16_t;  // raw bfloat16 bits
};

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Two fp32 -> two bf16 packed in one word (a in the low half), round to nearest even,
// NaN stays NaN: one v_cvt_pk_bf16_f32 on gfx950.  (Over every non-NaN fp32 bit pattern
// it gives the same bits as the rounding written out -- add 0x7fff plus the kept lsb,
// keep the high half -- which compiled to about 12 branchy instructions per value.)
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(f32x2_to_bf16x2(f, 0.0f) & 0xffffu);
}

template <class IO>
struct io;

template <>
struct io<F32> {
    using T = float;
    static __device__ __forceinline__ float ld(const T* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ v4f ld4(const T* p, size_t i) {
        return *reinterpret_cast<const v4f*>(p + i);
    }
    static __device__ __forceinline__ void st4(T* p, size_t i, v4f v) {
        *reinterpret_cast<v4f*>(p + i) = v;
    }
    static __device__ __forceinline__ void st(T* p, size_t i, float v) { p[i] = v; }
};

template <>
struct io<BF16> {
    using T = uint16_t;
    static __device__ __forceinline__ float ld(const T* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ v4f ld4(const T* p, size_t i) {
        uint2 w = *reinterpret_cast<const uint2*>(p + i);
        return v4f{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ void st4(T* p, size_t i, v4f v) {
        uint2 w;
        w.x = f32x2_to_bf16x2(v[0], v[1]);
        w.y = f32x2_to_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(p + i) = w;
    }
    static __device__ __forceinline__ void st(T* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ------------------------------------------------------------------ geometry
// Index helpers for one chunk-head (b, n, h).  Token row t of x sits at
// xrow(t) = ((b*n_chunks + n) * l + t) * h_heads * width + h * width.
struct ChunkHead {
    int b, n, h;
    int64_t bn;     // b * nchunks + n
    int64_t c_bhn;  // (b * nheads + h) * nchunks + n   (index of the chunk in dt / cumA order)
    int64_t ch;     // (b * nchunks + n) * nheads + h   (index in the [b, n, h, ...] state order)
};

__device__ __forceinline__ ChunkHead decode_ch(int64_t ch, int N, int H) {
    ChunkHead c;
    c.ch = ch;
    c.h = static_cast<int>(ch % H);
    c.bn = ch / H;
    c.n = static_cast<int>(c.bn % N);
    c.b = static_cast<int>(c.bn / N);
    c.c_bhn = (static_cast<int64_t>(c.b) * H + c.h) * N + c.n;
    return c;
}

// Stage ROWS rows of width W (io dtype in global, row stride gstride elements)
// into LDS as fp32 rows of stride W + 4, in batches of at most MAXB float4 loads
// per thread, each batch's loads issued before its LDS writes (one memory latency
// per batch; MAXB bounds the registers the staging takes).
template <class IO, int W, int ROWS = TB, int MAXB = 4>
__device__ __forceinline__ void stage_rows(float* lds, const typename IO::T* g, int64_t gstride) {
    constexpr int V = W / 4, TOTAL = ROWS * V, IT = (TOTAL + NT - 1) / NT;
    constexpr int BATCH = IT < MAXB ? IT : MAXB;  // at most MAXB float4 in flight per thread
#pragma unroll
    for (int b0 = 0; b0 < IT; b0 += BATCH) {
        v4f tmp[BATCH];
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int idx = static_cast<int>(threadIdx.x) + (b0 + it) * NT;
            if (b0 + it < IT && (TOTAL % NT == 0 || idx < TOTAL))
                tmp[it] = io<IO>::ld4(g, static_cast<int64_t>(idx / V) * gstride + (idx % V) * 4);
        }
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int idx = static_cast<int>(threadIdx.x) + (b0 + it) * NT;
            if (b0 + it < IT && (TOTAL % NT == 0 || idx < TOTAL))
                *reinterpret_cast<v4f*>(lds + (idx / V) * (W + 4) + (idx % V) * 4) = tmp[it];
        }
    }
}

// Stage two TB-row blocks (widths W1, W2; LDS row strides W + 4) with every
// global load of both in flight before the first LDS write: one memory latency
// per call instead of one per batch.  For use where the caller's other
// temporaries are dead (between the barriers around a block change).
template <class IO, int W1, int W2>
__device__ __forceinline__ void stage_rows2(float* l1, const typename IO::T* g1, int64_t s1,
                                            float* l2, const typename IO::T* g2, int64_t s2) {
    constexpr int V1 = W1 / 4, T1 = TB * V1, I1 = (T1 + NT - 1) / NT;
    constexpr int V2 = W2 / 4, T2 = TB * V2, I2 = (T2 + NT - 1) / NT;
    const int tid = static_cast<int>(threadIdx.x);
    v4f a[I1], b[I2];
#pragma unroll
    for (int it = 0; it < I1; ++it) {
        const int idx = tid + it * NT;
        if (T1 % NT == 0 || idx < T1) a[it] = io<IO>::ld4(g1, static_cast<int64_t>(idx / V1) * s1 + (idx % V1) * 4);
    }
#pragma unroll
    for (int it = 0; it < I2; ++it) {
        const int idx = tid + it * NT;
        if (T2 % NT == 0 || idx < T2) b[it] = io<IO>::ld4(g2, static_cast<int64_t>(idx / V2) * s2 + (idx % V2) * 4);
    }
#pragma unroll
    for (int it = 0; it < I1; ++it) {
        const int idx = tid + it * NT;
        if (T1 % NT == 0 || idx < T1) *reinterpret_cast<v4f*>(l1 + (idx / V1) * (W1 + 4) + (idx % V1) * 4) = a[it];
    }
#pragma unroll
    for (int it = 0; it < I2; ++it) {
        const int idx = tid + it * NT;
        if (T2 % NT == 0 || idx < T2) *reinterpret_cast<v4f*>(l2 + (idx / V2) * (W2 + 4) + (idx % V2) * 4) = b[it];
    }
}

// Row staging split in two so the loads can be issued long before the LDS
// writes: one float4 per (thread, step), element idx = tid + it * NT is row
// idx / (W / 4), float4 column idx % (W / 4); store_rows writes ROWS rows to LDS
// rows of stride W + 4.
template <int W, int ROWS>
struct RowTiles {
    static constexpr int V = W / 4, TOTAL = ROWS * V, IT = (TOTAL + NT - 1) / NT;
};
// Load ROWS consecutive rows (global row stride gstride) for store_rows.
template <class IO, int W, int ROWS>
__device__ __forceinline__ void load_rows(v4f* r, const typename IO::T* g, int64_t gstride) {
    using RT = RowTiles<W, ROWS>;
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        if (RT::TOTAL % NT == 0 || idx < RT::TOTAL)
            r[it] = io<IO>::ld4(g, static_cast<int64_t>(idx / RT::V) * gstride + (idx % RT::V) * 4);
    }
}
// Load the 64 rows of one half of a 128-row chunk that holds its even (half 0)
// or odd (half 1) 16-row tiles: LDS row 16u + e is chunk row 16 (2u + half) + e.
template <class IO, int W>
__device__ __forceinline__ void load_half_rows(v4f* r, const typename IO::T* g, int64_t gstride,
                                               int half) {
    using RT = RowTiles<W, 64>;
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        const int lr = idx / RT::V;
        const int crow = 16 * (2 * (lr >> 4) + half) + (lr & 15);
        if (RT::TOTAL % NT == 0 || idx < RT::TOTAL)
            r[it] = io<IO>::ld4(g, static_cast<int64_t>(crow) * gstride + (idx % RT::V) * 4);
    }
}
// Load and store one half (as load_half_rows) in batches of at most 4 float4
// per thread, for callers with few registers to spare.
template <class IO, int W>
__device__ __forceinline__ void stage_half_rows(float* lds, const typename IO::T* g, int64_t gstride,
                                                int half) {
    using RT = RowTiles<W, 64>;
    constexpr int BATCH = RT::IT < 4 ? RT::IT : 4;
#pragma unroll
    for (int b0 = 0; b0 < RT::IT; b0 += BATCH) {
        v4f tmp[BATCH];
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int idx = static_cast<int>(threadIdx.x) + (b0 + it) * NT;
            const int lr = idx / RT::V;
            const int crow = 16 * (2 * (lr >> 4) + half) + (lr & 15);
            if (b0 + it < RT::IT && (RT::TOTAL % NT == 0 || idx < RT::TOTAL))
                tmp[it] = io<IO>::ld4(g, static_cast<int64_t>(crow) * gstride + (idx % RT::V) * 4);
        }
#pragma unroll
        for (int it = 0; it < BATCH; ++it) {
            const int idx = static_cast<int>(threadIdx.x) + (b0 + it) * NT;
            if (b0 + it < RT::IT && (RT::TOTAL % NT == 0 || idx < RT::TOTAL))
                *reinterpret_cast<v4f*>(lds + (idx / RT::V) * (W + 4) + (idx % RT::V) * 4) = tmp[it];
        }
    }
}
template <int W, int ROWS>
__device__ __forceinline__ void store_rows(float* lds, const v4f* r) {
    using RT = RowTiles<W, ROWS>;
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        if (RT::TOTAL % NT == 0 || idx < RT::TOTAL)
            *reinterpret_cast<v4f*>(lds + (idx / RT::V) * (W + 4) + (idx % RT::V) * 4) = r[it];
    }
}

// Stage a contiguous fp32 [ROWS, W] matrix into LDS rows of stride W + 4.
template <int W, int ROWS>
__device__ __forceinline__ void stage_mat(float* lds, const float* g) {
    stage_rows<F32, W, ROWS>(lds, g, W);
}

// Stage TB token rows of width W transposed: lds[f * (TB + 4) + t] = scale[t] * g[t, f]
// (scale may be null).  Element (row t, float4 column c4) is handled by linear
// index idx with t % 16 = idx % 16, c4 % 4 = (idx / 16) % 4, t / 16 = (idx / 64) % 4,
// c4 / 4 = idx / 256: one 64-lane store then covers 16 rows x 4 columns, i.e.
// 64 distinct LDS banks (the token stride TB + 4 shifts each column by 4 banks),
// and every row is still read as a 64-byte segment.  The load half (into
// registers) and the store half (into LDS) are separate so that a kernel can
// issue the next block's loads before its matrix work on the current one.
template <class IO, int W>
struct RowsT {
    static constexpr int V = W / 4, TOTAL = TB * V, IT = (TOTAL + NT - 1) / NT;
    static constexpr int CL = V < 4 ? V : 4;  // float4 columns per 64-lane group
    __device__ static int row(int idx) { return (idx & 15) + 16 * ((idx / (16 * CL)) & 3); }
    __device__ static int col4(int idx) { return (idx / 16) % CL + CL * (idx / (64 * CL)); }
};

template <class IO, int W, int IT>
__device__ __forceinline__ void load_rows_t(v4f (&tmp)[IT], const typename IO::T* g, int64_t gstride) {
    using RT = RowsT<IO, W>;
    static_assert(IT == RT::IT, "register tile size");
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        if (RT::TOTAL % NT == 0 || idx < RT::TOTAL)
            tmp[it] = io<IO>::ld4(g, static_cast<int64_t>(RT::row(idx)) * gstride + RT::col4(idx) * 4);
    }
}

template <class IO, int W, int IT>
__device__ __forceinline__ void store_rows_t(float* lds, const v4f (&tmp)[IT], const float* scale) {
    using RT = RowsT<IO, W>;
    static_assert(IT == RT::IT, "register tile size");
#pragma unroll
    for (int it = 0; it < RT::IT; ++it) {
        const int idx = static_cast<int>(threadIdx.x) + it * NT;
        if (RT::TOTAL % NT == 0 || idx < RT::TOTAL) {
            const int row = RT::row(idx), c4 = RT::col4(idx);
            const v4f v = scale ? tmp[it] * scale[row] : tmp[it];
#pragma unroll
            for (int e = 0; e < 4; ++e) lds[(c4 * 4 + e) * (TB + 4) + row] = v[e];
        }
    }
}

template <class IO, int W>
__device__ __forceinline__ void stage_rows_t(float* lds, const typename IO::T* g, int64_t gstride,
                                             const float* scale) {
    v4f tmp[RowsT<IO, W>::IT];
    load_rows_t<IO, W>(tmp, g, gstride);
    store_rows_t<IO, W>(lds, tmp, scale);
}

// Stores of final outputs that nothing in the same call reads again: non-temporal for
// fp32 io (the fp32 130M-shaped step 0.668 -> 0.656 ms: K5 -3 %, the two backward chunk
// kernels -1 to -2 %); bf16 io keeps ordinary stores (non-temporal 8-byte stores made the
// bf16 backward kernels 4-10 % slower).
template <class IO>
__device__ __forceinline__ void st4_nt(typename IO::T* p, size_t i, v4f v) {
    if constexpr (sizeof(typename IO::T) == 4)
        __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p + i));
    else
        io<IO>::st4(p, i, v);
}
template <class IO>
__device__ __forceinline__ void st_nt(typename IO::T* p, size_t i, float v) {
    if constexpr (sizeof(typename IO::T) == 4)
        __builtin_nontemporal_store(v, p + i);
    else
        io<IO>::st(p, i, v);
}

// The causal (target tile, source tile) pairs of a chunk in 16-row tiles, it >= jt,
// numbered row by row (pair_tiles_of(L) of them): the backward's source-row kernel hands
// each pair's d_CB tile (256 floats, t-major) to the target-row kernel in this order.
__device__ __forceinline__ int pair_index(int it, int jt) { return it * (it + 1) / 2 + jt; }

// Sum over the four lane groups g = 0..3 that share i = lane % 16.
__device__ __forceinline__ float sum_over_g(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ double sum_over_g(double v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

}  // namespace ssd
