// Quaternion cumulative-product scan of the Mamba-3 rotation, and its gradient.
//
// Page: burn-mamba "mamba3/quat_scan/backward.rs" (module doc, "Gradient math").
// For every lane (b, h, j) of q [B, S, H, J, 4] (components w, x, y, z):
//   cum[t] = q_t (x) cum[t-1],   cum[-1] = init   (Hamilton product)
// and, for an upstream gradient d_cum, the exact reverse mode (valid for every
// quaternion, not only unit ones): with the per-factor VJPs of o = a (x) b,
// grad_a = g (x) conj(b) and grad_b = conj(a) (x) g, the cotangent G_t reaching
// cum[t] obeys G_t = d_cum[t] + conj(q_{t+1}) (x) G_{t+1}, and
//   d_q[t] = G_t (x) conj(cum[t-1]),    d_init = conj(q_0) (x) G_0.
// The page's parallel closed form of that recurrence (prefix product, suffix
// sum) assumes unit quaternions; the carries below need no such assumption.
//
// The scan moves 32 bytes per quaternion (q in, cum out) for about 28 flops, so
// it is bound by HBM.  Both directions are first-order recurrences along t whose
// step is associative, so the sequence is cut into segments of SEG = 4 * TS
// steps handled by one workgroup each, and the segments are chained in one pass:
//  * a workgroup covers 64 consecutive lanes (h, j) of one batch row -- one
//    lane per thread of a wave, 16 contiguous bytes each, so a wave reads 1 KB
//    of a row per step -- and its 4 waves take 4 consecutive sub-segments of TS
//    steps, holding their q (and d_cum) in registers, so HBM is read once;
//  * each wave reduces its sub-segment to one map (a product for the forward,
//    an affine map M (x) H + v for the reverse), the workgroup combines the 4
//    through LDS and publishes that aggregate;
//  * the segments of a chain are grouped in blocks of kQuatBlock; a segment's
//    carry is its block's earlier aggregates folded in order, then the earlier
//    blocks' aggregates in order, applied to the chain's start value; the last
//    segment of a block publishes the block's aggregate (its own aggregate
//    combined with the fold it takes for its carry).  The order of every fold
//    is fixed, so results are bitwise reproducible, and a segment waits only
//    for aggregates, which are published before any wait: no serial chain
//    through the segments.  A segment folds fewer than kQuatBlock + nseg /
//    kQuatBlock records, loaded 4 (forward) or 2 (reverse) at a time;
//  * a workgroup's chain (b, lane group) follows from its index; its segment is
//    the ticket it draws from its chain's atomic counter when it starts, taken
//    in dependency order (forward: from the first segment; reverse: from the
//    last), so a workgroup only ever waits for workgroups of its chain that have
//    already started and publish their aggregates without waiting.  Every wait
//    is bounded: past kMaxSpins polls the carry becomes NaN and is published,
//    so the grid always drains (a wrong result, never a hang);
//  * no memory fences: on gfx950 an agent-scope release writes back the whole
//    L2 of the XCD, and one per workgroup serialised the scan (6x slower).
//    Instead every record word is an fp64 value whose 16 lowest mantissa bits
//    carry the call's tag, written and read with agent-scope relaxed 64-bit
//    atomics (coherent across the XCDs' L2s without fences).  A reader accepts
//    a record once all four of its words carry the current tag, and retries
//    otherwise; it uses the value with the tag bits cleared, so a record
//    carries its value truncated to 36 significant bits (2^-36 relative), the
//    same in every call.  Before every call one small kernel zeroes the tickets
//    and advances the tag word kept in the workspace (never 0 in its low 16
//    bits); the scan kernels read the tag from there, so a call replayed from a
//    captured graph still gets a new tag.
// Products and carries are fp64 (the fp32 inputs are exact in fp64), so the
// result is within a few fp32 roundings of the exact scan at any length; cum
// and d_q are rounded to fp32 once.
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kLanes = 64;     // lanes (quaternions of a row) per workgroup
constexpr int kWaves = 4;      // sub-segments per workgroup
constexpr int kThreads = kLanes * kWaves;
constexpr int kMaxSpins = 1 << 20;
constexpr uint64_t kTagMask = 0xffffull;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef double d4 __attribute__((ext_vector_type(4)));

// Hamilton product a (x) b on (w, x, y, z).
__device__ __forceinline__ d4 qmul(d4 a, d4 b) {
    return d4{a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3],
              a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2],
              a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1],
              a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0]};
}

__device__ __forceinline__ d4 qconj(d4 a) { return d4{a[0], -a[1], -a[2], -a[3]}; }
__device__ __forceinline__ d4 to_d(f4 a) { return d4{a[0], a[1], a[2], a[3]}; }
__device__ __forceinline__ f4 to_f(d4 a) {
    return f4{static_cast<float>(a[0]), static_cast<float>(a[1]), static_cast<float>(a[2]),
              static_cast<float>(a[3])};
}
// The fp32 values pass through an empty asm statement, so the compiler cannot keep their fp64
// conversions from an earlier phase alive across the barriers (8 registers per quaternion
// instead of 4) and converts them again where they are used.
__device__ __forceinline__ void reconvert(f4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ d4 qone() { return d4{1.0, 0.0, 0.0, 0.0}; }
__device__ __forceinline__ d4 qzero() { return d4{0.0, 0.0, 0.0, 0.0}; }
__device__ __forceinline__ d4 qnan() {
    const double n = __builtin_nan("");
    return d4{n, n, n, n};
}

// ------------------------------------------------------------ tagged records
// Component c of record r of lane `lane` in a pass's array sits at word
// (r * 4 + c) * 64 + lane: one store or load instruction of a wave covers 512
// contiguous bytes (lane-interleaved records made every 8-byte write-through
// store a partial-line write: 4x the record bytes in HBM writes).
__device__ __forceinline__ int64_t word_of(int64_t r, int c, int lane) {
    return (r * 4 + c) * kLanes + lane;
}

__device__ __forceinline__ void store_record(uint64_t* rec, int64_t r, int lane, d4 v,
                                             uint32_t tag) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint64_t w = (static_cast<uint64_t>(__double_as_longlong(v[c])) & ~kTagMask) | tag;
        __hip_atomic_store(rec + word_of(r, c, lane), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Loads the record and reports whether every word carries `tag`.
__device__ __forceinline__ bool load_record(const uint64_t* rec, int64_t r, int lane, uint32_t tag,
                                            d4& v) {
    uint64_t* p = const_cast<uint64_t*>(rec);
    bool ok = true;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint64_t w = __hip_atomic_load(p + word_of(r, c, lane), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        ok = ok && (w & kTagMask) == tag;
        v[c] = __longlong_as_double(static_cast<long long>(w & ~kTagMask));
    }
    return ok;
}

// acc <- acc (x) rec[r0] (x) rec[r0 - 1] (x) ... over n records (latest first), loaded 4
// at a time, each waited for (bounded); false when a record never arrives.
__device__ __forceinline__ bool fold_prod(const uint64_t* rec, int64_t r0, int n, int lane,
                                          uint32_t tag, d4& acc) {
    for (int base = 0; base < n; base += 4) {
        d4 r[4];
        bool ok = false;
        for (int spin = 0; spin < kMaxSpins && !ok; ++spin) {
            bool all = true;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (base + u < n) all = load_record(rec, r0 - base - u, lane, tag, r[u]) && all;
            ok = __all(all);
            if (!ok) __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) return false;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (base + u < n) acc = qmul(acc, r[u]);
    }
    return true;
}

// (aM, av) <- (aM, av) o map[r0] o map[r0 + dir] o ... over n affine maps H -> M (x) H + v
// (records recm / recv), loaded 2 at a time, each waited for (bounded): two maps in flight
// are 32 registers per lane, which keeps the reverse pass at three waves per SIMD (four in
// flight took it to 189 VGPRs and two waves: 73 against 66 us on the quaternion workload).
__device__ __forceinline__ bool fold_affine(const uint64_t* recm, const uint64_t* recv, int64_t r0,
                                            int dir, int n, int lane, uint32_t tag, d4& aM, d4& av) {
    for (int base = 0; base < n; base += 2) {
        d4 rm[2], rv[2];
        bool ok = false;
        for (int spin = 0; spin < kMaxSpins && !ok; ++spin) {
            bool all = true;
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (base + u < n) {
                    all = load_record(recm, r0 + dir * (base + u), lane, tag, rm[u]) && all;
                    all = load_record(recv, r0 + dir * (base + u), lane, tag, rv[u]) && all;
                }
            ok = __all(all);
            if (!ok) __builtin_amdgcn_s_sleep(1);
        }
        if (!ok) return false;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (base + u < n) {
                av = qmul(aM, rv[u]) + av;
                aM = qmul(aM, rm[u]);
            }
    }
    return true;
}

// The chain (b, group) is the workgroup's blockIdx.x % BG; its position in the
// chain is the ticket it draws from the chain's own counter (one 256-byte line
// per chain, so chains do not queue on one address).
__device__ __forceinline__ uint32_t take_ticket(uint32_t* tickets, int bg, uint32_t* s_vid) {
    if (threadIdx.x == 0) *s_vid = atomicAdd(tickets + 64 * bg, 1u);
    __syncthreads();
    return *s_vid;
}

}  // namespace

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = v;
}

// Zero n ticket words and advance the call's tag (one thread).
__global__ void k_quat_clear(uint32_t* __restrict__ p, int64_t n, uint32_t* __restrict__ tag) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        uint32_t t = *tag + 1u;
        if ((t & 0xffffu) == 0u) t += 1u;
        *tag = t;
    }
}

// Forward scan.  WRITE: store cum; otherwise only the segment records (the backward's
// forward carries: inc[j] = cum at the end of the j-th half of a segment, one per segment
// of the reverse pass, nseg_inc of them per chain).
template <int TS, bool WRITE>
__global__ __launch_bounds__(kThreads) void k_quat_fwd(const float* __restrict__ q,
                                                        const float* __restrict__ init,
                                                        float* __restrict__ cum, QuatRecords rec,
                                                        int nb, int64_t S, int W, int G, int nseg,
                                                        int nseg_inc,
                                                        const uint32_t* __restrict__ tag_word) {
    constexpr int SEG = kWaves * TS;
    const uint32_t tag = *tag_word & 0xffffu;
    __shared__ uint32_t s_vid;
    __shared__ d4 s_part[kWaves][kLanes];
    __shared__ d4 s_carry[kLanes];
    // the wave index and the workgroup's segment are the same in every lane of a wave: taken
    // as scalars, the per-step row offsets below are scalar too (no 64-bit address per step
    // held in vector registers)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int BG = nb * G;
    const int bg = static_cast<int>(blockIdx.x % BG);
    const int seg =
        __builtin_amdgcn_readfirstlane(static_cast<int>(take_ticket(rec.ticket, bg, &s_vid)));
    const int b = bg / G, g = bg % G;
    const int col = g * kLanes + lane;
    const bool act = col < W;
    const int64_t t0 = static_cast<int64_t>(seg) * SEG + wave * TS;
    const int64_t row = static_cast<int64_t>(W) * 4;
    const float* qb = q + (static_cast<int64_t>(b) * S * W + col) * 4;

    f4 x[TS];
#pragma unroll
    for (int i = 0; i < TS; ++i) {
        const int64_t t = t0 + i;
        x[i] = act && t < S ? *reinterpret_cast<const f4*>(qb + t * row) : f4{1.f, 0.f, 0.f, 0.f};
    }
    d4 P = to_d(x[0]);
#pragma unroll
    for (int i = 1; i < TS; ++i) P = qmul(to_d(x[i]), P);
    s_part[wave][lane] = P;
    __syncthreads();

    if (wave == 0) {
        const int64_t row0 = static_cast<int64_t>(bg) * nseg;
        const int nblk = (nseg + kQuatBlock - 1) / kQuatBlock;
        const int64_t brow0 = static_cast<int64_t>(bg) * nblk;
        const int64_t k = row0 + seg;
        d4 a = s_part[0][lane], half = a;
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            a = qmul(s_part[w][lane], a);
            if (w == kWaves / 2 - 1) half = a;  // the first half's product
        }
        const int m = seg / kQuatBlock, first = m * kQuatBlock;
        store_record(rec.agg, k, lane, a, tag);  // for the block's later segments
        d4 carry = qone();  // the chain's start value
        if (init && act)
            carry = to_d(*reinterpret_cast<const f4*>(init + (static_cast<int64_t>(b) * W + col) * 4));
        // the product of every earlier segment, latest first: this block's, then earlier blocks'
        d4 acc = qone();
        bool ok = fold_prod(rec.agg, k - 1, seg - first, lane, tag, acc);
        if (seg - first == kQuatBlock - 1)  // the block's last segment publishes its aggregate
            store_record(rec.bagg, brow0 + m, lane, ok ? qmul(a, acc) : qnan(), tag);
        ok = fold_prod(rec.bagg, brow0 + m - 1, m, lane, tag, acc) && ok;
        carry = ok ? qmul(acc, carry) : qnan();  // NaN: a record never arrived
        if constexpr (!WRITE) {  // cum at the end of each half of the segment
            const int64_t j = static_cast<int64_t>(bg) * nseg_inc + 2 * seg;
            store_record(rec.inc, j, lane, qmul(half, carry), tag);
            if (2 * seg + 1 < nseg_inc) store_record(rec.inc, j + 1, lane, qmul(a, carry), tag);
        }
        s_carry[lane] = carry;
    }
    if constexpr (WRITE) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TS; ++i) reconvert(x[i]);
        d4 c = s_carry[lane];
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w)
            if (w < wave) c = qmul(s_part[w][lane], c);
        float* cb = cum + (static_cast<int64_t>(b) * S * W + col) * 4;
#pragma unroll
        for (int i = 0; i < TS; ++i) {
            const int64_t t = t0 + i;
            c = qmul(to_d(x[i]), c);
            if (act && t < S) __builtin_nontemporal_store(to_f(c), reinterpret_cast<f4*>(cb + t * row));
        }
    }
}

// Reverse pass of the backward.  With H_t = conj(q_t) (x) G_t (the cotangent that
// cum[t] hands to cum[t-1]; H_S = 0), a sub-segment [t0, t0 + TS) maps the H
// entering its end to the H leaving its start affinely: H_t0 = M (x) H_end + v.
// fwd_inc: the forward-carry pass's inclusive records (cum at the end of each
// segment; written by the previous kernel, so read as plain memory).
template <int TS>
__global__ __launch_bounds__(kThreads) void k_quat_bwd(const float* __restrict__ q,
                                                        const float* __restrict__ init,
                                                        const float* __restrict__ d_cum,
                                                        float* __restrict__ d_q,
                                                        float* __restrict__ d_init,
                                                        const uint64_t* __restrict__ fwd_inc,
                                                        QuatRecords rec, int nb, int64_t S, int W,
                                                        int G, int nseg,
                                                        const uint32_t* __restrict__ tag_word) {
    constexpr int SEG = kWaves * TS;
    const uint32_t tag = *tag_word & 0xffffu;
    __shared__ uint32_t s_vid;
    __shared__ d4 s_P[kWaves][kLanes], s_M[kWaves][kLanes], s_V[kWaves][kLanes];
    __shared__ d4 s_H[kLanes], s_C[kLanes];
    // the wave index and the workgroup's segment are the same in every lane of a wave: taken
    // as scalars, the per-step row offsets below are scalar too (no 64-bit address per step
    // held in vector registers)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int BG = nb * G;
    const int bg = static_cast<int>(blockIdx.x % BG);
    const int seg =
        __builtin_amdgcn_readfirstlane(nseg - 1 - static_cast<int>(take_ticket(rec.ticket, bg, &s_vid)));
    const int b = bg / G, g = bg % G;
    const int col = g * kLanes + lane;
    const bool act = col < W;
    const int64_t t0 = static_cast<int64_t>(seg) * SEG + wave * TS;
    const int64_t row = static_cast<int64_t>(W) * 4;
    const int64_t base = (static_cast<int64_t>(b) * S * W + col) * 4;

    f4 x[TS], dc[TS];
#pragma unroll
    for (int i = 0; i < TS; ++i) {
        const int64_t t = t0 + i;
        const bool in = act && t < S;
        x[i] = in ? *reinterpret_cast<const f4*>(q + base + t * row) : f4{1.f, 0.f, 0.f, 0.f};
        dc[i] = in ? *reinterpret_cast<const f4*>(d_cum + base + t * row) : f4{0.f, 0.f, 0.f, 0.f};
    }
    {
        d4 P = to_d(x[0]);
#pragma unroll
        for (int i = 1; i < TS; ++i) P = qmul(to_d(x[i]), P);
        d4 M = qone(), v = qzero();
#pragma unroll
        for (int i = TS - 1; i >= 0; --i) {
            const d4 cq = qconj(to_d(x[i]));
            v = qmul(cq, to_d(dc[i]) + v);
            M = qmul(cq, M);
        }
        s_P[wave][lane] = P;
        s_M[wave][lane] = M;
        s_V[wave][lane] = v;
    }
    __syncthreads();

    if (wave == 0) {
        const int64_t row0 = static_cast<int64_t>(bg) * nseg;
        const int64_t k = row0 + seg;
        // the workgroup's map f_0 o f_1 o f_2 o f_3 (sub-segment 0 is the earliest)
        d4 M = s_M[kWaves - 1][lane], v = s_V[kWaves - 1][lane];
#pragma unroll
        for (int w = kWaves - 2; w >= 0; --w) {
            v = qmul(s_M[w][lane], v) + s_V[w][lane];
            M = qmul(s_M[w][lane], M);
        }
        // H entering the end of this segment: the maps of every later segment composed in
        // order (this block's, then later blocks') applied to H past the end, 0
        const int nblk = (nseg + kQuatBlock - 1) / kQuatBlock;
        const int64_t brow0 = static_cast<int64_t>(bg) * nblk;
        const int pos = nseg - 1 - seg;  // place in the reverse order
        const int m = pos / kQuatBlock, last = nseg - 1 - m * kQuatBlock;  // block, its highest segment
        store_record(rec.agg, k, lane, M, tag);  // for the block's earlier segments
        store_record(rec.agg2, k, lane, v, tag);
        d4 aM = qone(), av = qzero();
        bool ok = fold_affine(rec.agg, rec.agg2, k + 1, 1, last - seg, lane, tag, aM, av);
        if (pos - m * kQuatBlock == kQuatBlock - 1) {  // the block's last segment: its map
            store_record(rec.bagg, brow0 + m, lane, ok ? qmul(M, aM) : qnan(), tag);
            store_record(rec.bagg2, brow0 + m, lane, ok ? qmul(M, av) + v : qnan(), tag);
        }
        ok = fold_affine(rec.bagg, rec.bagg2, brow0 + m - 1, -1, m, lane, tag, aM, av) && ok;
        const d4 carry = ok ? av : qnan();  // NaN: a record never arrived
        const d4 h_start = qmul(M, carry) + v;
        if (seg == 0 && d_init && act)
            *reinterpret_cast<f4*>(d_init + (static_cast<int64_t>(b) * W + col) * 4) = to_f(h_start);
        s_H[lane] = carry;
        d4 c0 = qone();
        if (seg == 0) {
            if (init && act)
                c0 = to_d(*reinterpret_cast<const f4*>(init + (static_cast<int64_t>(b) * W + col) * 4));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                c0[c] = __longlong_as_double(static_cast<long long>(fwd_inc[word_of(k - 1, c, lane)] & ~kTagMask));
        }
        s_C[lane] = c0;
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < TS; ++i) {
        reconvert(x[i]);
        reconvert(dc[i]);
    }
    d4 h = s_H[lane];  // H entering the end of this wave's sub-segment
#pragma unroll
    for (int w = kWaves - 1; w > 0; --w)
        if (w > wave) h = qmul(s_M[w][lane], h) + s_V[w][lane];
    d4 c = s_C[lane];  // cum[t0 - 1]
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w)
        if (w < wave) c = qmul(s_P[w][lane], c);
    f4 prev[TS];  // cum[t - 1] for the sub-segment's steps (rounded: it only scales d_q)
#pragma unroll
    for (int i = 0; i < TS; ++i) {
        prev[i] = to_f(c);
        c = qmul(to_d(x[i]), c);
    }
#pragma unroll
    for (int i = TS - 1; i >= 0; --i) {
        const d4 G = to_d(dc[i]) + h;
        const int64_t t = t0 + i;
        if (act && t < S)
            __builtin_nontemporal_store(to_f(qmul(G, qconj(to_d(prev[i])))),
                                        reinterpret_cast<f4*>(d_q + base + t * row));
        h = qmul(qconj(to_d(x[i])), G);
    }
}

// ------------------------------------------------------------------ host side
QuatPlan quat_plan(const QuatShape& s, bool bwd) {
    QuatPlan p;
    if (s.B <= 0 || s.S <= 0) return p;
    const int64_t chains = static_cast<int64_t>(s.B) * s.G;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~static_cast<size_t>(255);
        return at;
    };
    p.tag = take(256);  // the call tag (kept across calls)
    // per pass one ticket per chain, each in its own 256 bytes
    p.words_per_pass = 64 * chains;
    p.flag_words = p.words_per_pass * (bwd ? 2 : 1);
    p.flags = take(4 * static_cast<size_t>(p.flag_words));
    // one record per lane and segment (rec) or block of segments (brec) of a chain
    constexpr size_t kRec = static_cast<size_t>(kLanes) * 4 * sizeof(uint64_t);
    auto rec = [&](int nseg) { return static_cast<size_t>(chains) * nseg * kRec; };
    auto brec = [&](int nseg) {
        return static_cast<size_t>(chains) * ((nseg + kQuatBlock - 1) / kQuatBlock) * kRec;
    };
    p.agg = take(rec(s.nseg_c));  // the forward's, or the carry pass's
    p.bagg = take(brec(s.nseg_c));
    if (bwd) {
        p.inc = take(rec(s.nseg));  // one per reverse-pass segment
        p.agg_b = take(rec(s.nseg));
        p.agg2_b = take(rec(s.nseg));
        p.bagg_b = take(brec(s.nseg));
        p.bagg2_b = take(brec(s.nseg));
    }
    p.total = off;
    return p;
}

QuatShape quat_shape(int64_t B, int64_t S, int64_t H, int64_t J, bool bwd) {
    QuatShape s;
    s.B = static_cast<int>(B);
    s.S = S;
    s.W = static_cast<int>(H * J);
    s.G = static_cast<int>((s.W + kLanes - 1) / kLanes);
    s.nseg_c = static_cast<int>((S + quat_seg(false) - 1) / quat_seg(false));
    s.nseg = bwd ? static_cast<int>((S + quat_seg(true) - 1) / quat_seg(true)) : s.nseg_c;
    return s;
}

namespace {

QuatRecords records(const QuatShape& s, const QuatPlan& p, void* ws, int pass) {
    char* w = static_cast<char*>(ws);
    uint32_t* flags = reinterpret_cast<uint32_t*>(w + p.flags) + pass * p.words_per_pass;
    QuatRecords r;
    r.ticket = flags;
    if (pass == 0) {
        r.agg = reinterpret_cast<uint64_t*>(w + p.agg);
        r.agg2 = nullptr;
        r.bagg = reinterpret_cast<uint64_t*>(w + p.bagg);
        r.bagg2 = nullptr;
        r.inc = p.inc ? reinterpret_cast<uint64_t*>(w + p.inc) : nullptr;
    } else {
        r.agg = reinterpret_cast<uint64_t*>(w + p.agg_b);
        r.agg2 = reinterpret_cast<uint64_t*>(w + p.agg2_b);
        r.bagg = reinterpret_cast<uint64_t*>(w + p.bagg_b);
        r.bagg2 = reinterpret_cast<uint64_t*>(w + p.bagg2_b);
        r.inc = nullptr;
    }
    return r;
}

hipError_t fill_u32(uint32_t* p, int64_t n, hipStream_t st) {
    const int64_t blocks = (n + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
    k_fill_u32<<<dim3(grid), dim3(256), 0, st>>>(p, n, 0u);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quat_clear(const QuatShape& s, bool bwd, void* ws, hipStream_t st) {
    const QuatPlan p = quat_plan(s, bwd);
    char* w = static_cast<char*>(ws);
    const int64_t blocks = (p.flag_words + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks));
    k_quat_clear<<<dim3(grid), dim3(256), 0, st>>>(reinterpret_cast<uint32_t*>(w + p.flags),
                                                   p.flag_words, reinterpret_cast<uint32_t*>(w + p.tag));
    return hipGetLastError();
}

hipError_t launch_quat_fwd(const QuatShape& s, const float* q, const float* init, float* cum,
                           void* ws, hipStream_t st) {
    const QuatPlan p = quat_plan(s, false);
    const int64_t blocks = static_cast<int64_t>(s.B) * s.G * s.nseg;
    const uint32_t* tag = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + p.tag);
    k_quat_fwd<kQuatTSFwd, true><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
        q, init, cum, records(s, p, ws, 0), s.B, s.S, s.W, s.G, s.nseg, 0, tag);
    return hipGetLastError();
}

hipError_t launch_quat_bwd(const QuatShape& s, const float* q, const float* init,
                           const float* d_cum, float* d_q, float* d_init, void* ws, hipStream_t st,
                           int stage) {
    const QuatPlan p = quat_plan(s, true);
    const int64_t blocks = static_cast<int64_t>(s.B) * s.G * s.nseg;
    const QuatRecords r0 = records(s, p, ws, 0);
    const uint32_t* tag = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + p.tag);
    if (stage == 0) {
        const int64_t cblocks = static_cast<int64_t>(s.B) * s.G * s.nseg_c;
        k_quat_fwd<kQuatTSFwd, false><<<dim3(static_cast<unsigned>(cblocks)), dim3(kThreads), 0, st>>>(
            q, init, nullptr, r0, s.B, s.S, s.W, s.G, s.nseg_c, s.nseg, tag);
    } else {
        k_quat_bwd<kQuatTSBwd><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st>>>(
            q, init, d_cum, d_q, d_init, r0.inc, records(s, p, ws, 1), s.B, s.S, s.W, s.G, s.nseg,
            tag);
    }
    return hipGetLastError();
}

hipError_t launch_quat_zero(float* p, int64_t n, hipStream_t st) {
    return fill_u32(reinterpret_cast<uint32_t*>(p), n, st);
}

}  // namespace ssd
