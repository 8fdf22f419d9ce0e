// Host-side launchers of the SSD kernels (all enqueue on `stream`, never sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Work-items one launch may have along x: the AQL dispatch packet stores the grid
// size in 32 bits.  No workgroup of the library has more than 256 work-items, so
// an entry point that bounds its largest grid by this (less one workgroup for the
// rounding up of block counts) never asks for a grid the packet cannot hold.
constexpr double kMaxGridItems = 4294967295.0 - 256.0;

struct Shape {
    int B, N, L, H, P, R;  // batch, nchunks, chunk_len, nheads, headdim, dstate
    int io;                // 0 = fp32, 1 = bf16
    int64_t chunks() const { return static_cast<int64_t>(B) * H * N; }  // (b, h, n) chunks
    int64_t tokens() const { return static_cast<int64_t>(B) * N * L; }
    int nblk() const { return L / 64; }
};

// Causal 16 x 16 (target tile, source tile) pairs of a chunk of L tokens.
constexpr int pair_tiles_of(int L) { return (L / 16) * (L / 16 + 1) / 2; }

// K1: cdt[b,h,n,t] = sum_{k<=t} dt[b,h,n,k]  (fp64; the cumsum of dt*A is A[h] * cdt)
hipError_t launch_k1_cumsum(const Shape& s, const float* dt, double* cdt, hipStream_t st);

// Chunk-local token contractions (states order [b,n,h,p,r]):
//   job 0 (K3): S[p,r]  = sum_t x[t,p] * dt[t] * exp(A (cdt[L-1] - cdt[t])) * B[t,r]
//   job 1:      dS[p,r] = sum_t dy[t,p] * exp(A cdt[t]) * C[t,r]
//   job 2:      T[p,r]  = sum_t x[t,p] * dt[t] * exp(A cdt[t]) * phi[t] * B[t,r]   (moments)
hipError_t launch_chunk_states(const Shape& s, bool job_state, bool job_dstate, const void* x,
                               const void* Bm, const void* dy, const void* Cm, const float* dt,
                               const float* A, const double* cdt, float* S, float* dS,
                               hipStream_t st, const double* phi = nullptr, float* T = nullptr);

// Benchmark instrumentation (k_stream.hip): one streaming launch that reads `reads` and
// writes `writes` arrays of n float4 (src / dst, array a at offset a * n).
hipError_t launch_stream_probe(int reads, int writes, bool nontemporal, const void* src, void* dst,
                               int64_t n, hipStream_t st);

// ---------------------------------------------------------------- moments
// Per chunk (one wave each): phi[t] = sum_{u>=t} mask_u exp(2A(cdt_u - cdt_t)),
// psi[t] = sum_{u>=t} mask_u exp(A(cdt_u - cdt_t)), mask_u = (chunk start + u < valid[b]).
// phit[t] = sum_{u>=t} mask_u (cdt_u - cdt_t) exp(2A(cdt_u - cdt_t)), psit likewise with A.
hipError_t launch_km_phi(const Shape& s, const double* cdt, const float* A, const int64_t* valid,
                         double* phi, double* psi, double* phit, double* psit, hipStream_t st);

// Forward, per (chunk-head, 64-row block): U = sum_{s in block} B_s Z_s^T with
// Z = (K o G) B over the whole chunk; m1 block part sum_s u_s (1^T x_s) B_s.
hipError_t launch_km_fwd_rows(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, float* U, float* m1b, hipStream_t st);

// Per chunk-head.  Forward (dm2 == nullptr): W = H^T (2T + c2 H), m1c = c1 colsum(H).
// Backward: HS = H S, dS_local = (c2 H + T) S + c1 1 dm1^T, BS = B S, and the chunk
// scalars hsh = <H, HS>, hdm = dm1 . colsum(H); S = dm2 + dm2^T.
hipError_t launch_km_chunk(const Shape& s, const float* Sin, const float* T, const double* cdt,
                           const float* A, const double* phi, const double* psi, float* W,
                           float* m1c, const float* dm2, const float* dm1, const void* Bm,
                           float* HS, float* dSl, float* BS, double* hsh, double* hdm,
                           hipStream_t st);

// m2[b,h] = sym(sum U + sum W), m1[b,h] = sum m1b + sum m1c.
hipError_t launch_km_reduce(const Shape& s, const float* U, const float* W, const float* m1b,
                            const float* m1c, float* m2, float* m1, hipStream_t st);

// Backward, per (chunk-head, 64-row block): d_x, d_B, the per-token scalars
// ddtW, rho, eta, zeta, the d_A partials [b,n,h,block]; block 0 also <d_intra, h_end>.
hipError_t launch_km_bwd_rows(const Shape& s, const void* x, const void* Bm, const float* dt,
                              const float* A, const double* cdt, const double* phi,
                              const double* psi, const double* phit, const double* psit,
                              const float* HS, const float* BS, const float* dI, const float* Sin,
                              const float* final_state, const float* dm1, const double* hsh,
                              const double* hdm, void* dx, void* dB, float* ddtW, float* rho,
                              float* eta, float* zeta, double* dend2, double* dA_part,
                              hipStream_t st);

// Backward, per chunk (one wave): the per-token recurrences and d_dt.
hipError_t launch_km_scan_bwd(const Shape& s, const double* cdt, const float* dt, const float* A,
                              const int64_t* valid, const float* ddtW, const float* rho,
                              const float* eta, const float* zeta, const double* hsh,
                              const double* hdm, const double* dend2, float* d_dt,
                              hipStream_t st);

// K4: in place over S: S[i] <- state entering chunk i; final <- state after the last chunk.
hipError_t launch_k4_pass(const Shape& s, float* S, const double* cdt, const float* A,
                          const float* init, float* final_state, hipStream_t st);

// K4 recompute and its reverse in one pass: S as in launch_k4_pass; in place over dS:
// dS[i] <- gradient reaching the state that leaves chunk i; d_init <- gradient of init.
// With forward == false only the reverse carry runs (S untouched).
hipError_t launch_k4_pass_bwd(const Shape& s, float* S, float* dS, const double* cdt,
                              const float* A, const float* init, const float* d_final,
                              float* d_init, hipStream_t st, bool forward = true);

// K5: y = BLUE + ORANGE + D x.
hipError_t launch_k5_scan(const Shape& s, const void* x, const float* dt, const void* Bm,
                          const void* Cm, const float* A, const float* D, const double* cdt,
                          const float* S, void* y, hipStream_t st);

// Whole-chunk variants (k_chunk_wide.hip) of K5 and the backward target-row
// kernel for 128-token chunks: one workgroup per chunk-head.  wide_supported(s)
// says whether s takes them (chunk length 128, p * r <= 8192); launch_k5_scan
// routes to the K5 one then, and the backward calls launch_bwd_target_wide.
bool wide_supported(const Shape& s);
hipError_t launch_k5_scan_wide(const Shape& s, const void* x, const float* dt, const void* Bm,
                               const void* Cm, const float* A, const float* D, const double* cdt,
                               const float* S, void* y, hipStream_t st);

// The backward's chunk kernels.  The source-row kernel runs first: rows s get d_x, d_B,
// the ORANGE + K3 part of d_dt, g2 (-ORANGE d_da, source side), d_delta (K3) and the
// d_A / d_D partials dA_S, dD_part [b,n,h,block] (with every pair's d_diff (cdt_t - cdt_s));
// every causal pair tile of 16 x 16 (t, s) hands its d_CB tile to
// dcbt [chunk-heads, pair_tiles_of(l), 256] (t-major), the diagonal elements t = s as zeros:
// those go to ddg [b,h,n,l] (d_CB[t, t]), so that the target side can take g1 without
// them (g2 leaves them out too) and add them to d_C afterwards.
hipError_t launch_bwd_source(const Shape& s, const void* dy, const void* x, const float* dt,
                             const void* Bm, const void* Cm, const float* A, const float* D,
                             const double* cdt, const float* dS, void* dx, void* dB, float* d_dt,
                             float* g2, float* d_delta, double* dA_S, double* dD_part,
                             float* dcbt, float* ddg, hipStream_t st);

// The same per whole 128-token chunk (wide_supported shapes, bf16 io only): one 8-wave
// workgroup per chunk-head; the d_A / d_D partials go to the chunk-head's first block
// slot, zeros after.
hipError_t launch_bwd_source_wide(const Shape& s, const void* dy, const void* x, const float* dt,
                                  const void* Bm, const void* Cm, const float* A, const float* D,
                                  const double* cdt, const float* dS, void* dx, void* dB,
                                  float* d_dt, float* g2, float* d_delta, double* dA_S,
                                  double* dD_part, float* dcbt, float* ddg, hipStream_t st);

// Target side (rows t) from those tiles, per (chunk-head, 64-row block): d_C, g1 (BLUE +
// ORANGE-target gradient w.r.t. the cumsum), d_end, and the d_A partials dA_T.
hipError_t launch_bwd_target(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                             const float* A, const double* cdt, const float* S, const float* dS,
                             const float* dcbt, const float* ddg, void* dC, float* g1,
                             float* d_end, double* dA_T, hipStream_t st);

// The same per whole 128-token chunk (wide_supported shapes), with K1's backward folded
// in: d_C, d_dt (the source kernel's part plus A d_da, in place) and dA_T.
hipError_t launch_bwd_target_wide(const Shape& s, const void* dy, const void* Bm, const void* Cm,
                                  const float* A, const double* cdt, const float* S,
                                  const float* dS, const float* dcbt, const float* ddg,
                                  const float* g2, const float* d_delta, void* dC, float* d_dt,
                                  double* dA_T, hipStream_t st);

// K1 backward (suffix sums inside each chunk, d_dt += A d_da) and, in the same launch,
// the per-head sums of launch_reduce_heads below.
hipError_t launch_k1t_heads(const Shape& s, const float* g1, const float* g2, const float* d_delta,
                            const float* d_end, const float* A, float* d_dt,
                            const double* dA_part0, const double* dA_part1, const double* dD_part,
                            int nk, float* d_A, float* d_D, hipStream_t st);

// Deterministic per-head sums of partials in [b, n, h, k] order (k < nk):
// d_A[h] = sum of dA_part0 + dA_part1, d_D[h] = sum of dD_part.  NULL parts/outputs are skipped.
hipError_t launch_reduce_heads(const Shape& s, const double* dA_part0, const double* dA_part1,
                               const double* dD_part, int nk, float* d_A, float* d_D,
                               hipStream_t st);

// dst[i] = src ? src[i] : 0   (i < n)
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t st);

// dst[i] = (vals ? vals[i] : fill) for i < n; the values travel as kernel arguments.
// Debug checks: the device's flag words (kMaxChecked of them), clearing them, and a
// scan that sets *flag when n floats (or bf16 values) at p hold a NaN or an infinity.
hipError_t nonfinite_flags(int** flags);
hipError_t launch_clear_flags(int* flags, int n, hipStream_t st);
hipError_t launch_nonfinite(const void* p, int64_t n, bool bf16, int* flag, hipStream_t st);

// Device address of the fixed scratch array of ssd_fwd_noalloc on the current
// device (SSD_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_set_i64(int64_t* dst, const int64_t* vals, int64_t fill, int64_t n, hipStream_t st);

// ------------------------------------------------------ participation ratio
// 1 / count[b] for up to kMax batch rows, passed by value to the PR kernels.
struct PrCounts {
    static constexpr int kMax = 64;
    double inv_n[kMax];
};

// Per (b, h) slice of m2 [B,H,R,R] (m1 [B,H,R], read only when center != 0):
// pr[b,h] and, if trace != NULL, trace[b,h] = tr(m2) / count[b].  count is host.
hipError_t launch_pr_fwd(int B, int H, int R, const float* m2, const float* m1,
                         const int64_t* count, int center, float* pr, float* trace,
                         hipStream_t st);

// Gradient of sum d_pr * pr: d_m2 [B,H,R,R] and, if d_m1 != NULL, d_m1 [B,H,R]
// (zero unless center != 0).
hipError_t launch_pr_bwd(int B, int H, int R, const float* d_pr, const float* m2, const float* m1,
                         const int64_t* count, int center, float* d_m2, float* d_m1,
                         hipStream_t st);

// ------------------------------------------------- same-step correction y_diag
struct DiagShape {
    int64_t T;     // tokens (the [b, n, l] axes flattened)
    int M, H, P, R;  // mimo rank, heads, headdim, dstate
    int io;        // 0 = fp32, 1 = bf16
};

// y [T,M,H,P] = gamma [T,H] * (C B^T) V per (token, head); V [T,M,H,P], B/C [T,M,H,R].
hipError_t launch_diag_fwd(const DiagShape& d, const void* V, const void* B, const void* C,
                           const float* gamma, void* y, hipStream_t st);

// Gradients of <dy, y>: d_v like V, d_b / d_c like B, d_gamma [T,H].
hipError_t launch_diag_bwd(const DiagShape& d, const void* dy, const void* V, const void* B,
                           const void* C, const float* gamma, void* d_v, void* d_b, void* d_c,
                           float* d_gamma, hipStream_t st);

// ------------------------------------------------- quaternion cumulative-product scan
// Steps per wave (sub-segment); a workgroup's 4 waves take a segment of 4x as many.  The
// forward and the backward's forward-carry pass hold 16 steps per lane (64-step segments);
// the reverse pass holds 8 (32-step segments), since it keeps q and the upstream gradient
// and fits three waves per SIMD only at that length.  The carry pass publishes cum at the
// end of each half of its segments: one record per reverse-pass segment.
constexpr int kQuatTSFwd = 16;
constexpr int kQuatTSBwd = 8;
constexpr int quat_seg(bool reverse) { return 4 * (reverse ? kQuatTSBwd : kQuatTSFwd); }
static_assert(2 * quat_seg(true) == quat_seg(false), "a carry segment is two reverse segments");

struct QuatShape {
    int B;       // batch
    int64_t S;   // sequence length
    int W;       // quaternions per (b, t) row: nheads * nquat
    int G;       // 64-lane groups per row
    int nseg;    // segments: of quat_seg(false) steps for the forward, quat_seg(true) for the
                 // backward's reverse pass
    int nseg_c;  // segments of quat_seg(false) steps (the forward and the carry pass)
};

// Segments per block of a chain: a segment's carry folds the aggregates of its block's
// earlier segments and then the aggregates of the earlier blocks (k_quat.hip).
constexpr int kQuatBlock = 8;

// Records of one pass: a ticket counter per (b, group) chain (64 words apart), and per lane
// one quaternion record of 4 tagged fp64 words per workgroup (its aggregate; the forward
// carry pass also its inclusive value) and per block of kQuatBlock segments (the block's
// aggregate), see k_quat.hip.
struct QuatRecords {
    uint32_t* ticket;
    uint64_t* agg;    // aggregate (forward: product; reverse: M of the affine map)
    uint64_t* agg2;   // reverse only: v of the affine map
    uint64_t* bagg;   // block aggregates, same meaning
    uint64_t* bagg2;  // reverse only
    uint64_t* inc;    // forward: cum at the segment end (read by the reverse pass)
};

// Workspace layout (byte offsets, 256-byte aligned): the call tag word at `tag`
// (kept across calls), then the ticket words of all passes together at `flags`
// (flag_words 32-bit words) so one kernel clears them, then the records.
struct QuatPlan {
    size_t tag = 0, flags = 0, agg = 0, bagg = 0, inc = 0, agg_b = 0, agg2_b = 0, bagg_b = 0,
           bagg2_b = 0, total = 0;
    int64_t flag_words = 0, words_per_pass = 0;
};

QuatShape quat_shape(int64_t B, int64_t S, int64_t H, int64_t J, bool bwd);
QuatPlan quat_plan(const QuatShape& s, bool bwd);

// Zero the ticket words and advance the call tag (must precede every
// forward / backward: the scan kernels read the tag from the workspace).
hipError_t launch_quat_clear(const QuatShape& s, bool bwd, void* ws, hipStream_t st);
// cum [B,S,H,J,4] = scan of q (init [B,H,J,4], NULL = identity).
hipError_t launch_quat_fwd(const QuatShape& s, const float* q, const float* init, float* cum,
                           void* ws, hipStream_t st);
// stage 0: forward-carry records; stage 1: reverse pass writing d_q (and d_init).
hipError_t launch_quat_bwd(const QuatShape& s, const float* q, const float* init,
                           const float* d_cum, float* d_q, float* d_init, void* ws, hipStream_t st,
                           int stage);
// n floats of p set to 0.
hipError_t launch_quat_zero(float* p, int64_t n, hipStream_t st);

// ------------------------------------------------- decode step
struct StepShape {
    int B, H, P, R;  // batch, heads, headdim, dstate (16..128)
    int io;          // 0 = fp32, 1 = bf16
};

// One token from the cached state: new_state = exp(dt A) state + dt x (outer) B,
// y = new_state C + D x.  x/y [B,H,P], dt [B,H], B/C [B,H,R], state [B,H,P,R]
// (state may equal new_state).
hipError_t launch_step(const StepShape& s, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* state,
                       float* new_state, void* y, hipStream_t st);

}  // namespace ssd
