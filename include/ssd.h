/*
 * mamba_ssd_chunked_amd -- C ABI of the Mamba-2 SSD chunked scan for MI355X (gfx950).
 *
 * The operation is the selective state-space scan of Mamba-2, computed chunk by
 * chunk as in the burn-mamba page "mamba2/ssd/serial_recalculated/
 * combined_backward.rs":
 *
 *   h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t,
 *   y_t = C_t . h_t + D_h * x_t,          h_{-1} = initial_state,
 *
 * where the chunked form runs K1 (inclusive per-chunk cumsum of dt*A),
 * K2 (C B^T inside a chunk), K3 (chunk-end states), K4 (serial state passing
 * across chunks) and K5 (chunk-scan output plus the D skip).  The backward is
 * that page's recompute backward: it takes the seven leaf inputs again,
 * recomputes K1-K4 and returns the gradients of every input (the page's
 * CombinedGrads).  The state moments are the StateMoments of the burn-mamba
 * page "modules/state_moments.rs"; their backward follows the per-token
 * cotangent of the burn-mamba "mamba3/moments/backward" module page with no
 * rotation.
 *
 * Tensor layouts (row-major, contiguous; b batch, n nchunks, l chunk_len,
 * h nheads, p headdim, r dstate; the pages' naming):
 *   x, dy, y, d_x          [b, n, l, h, p]   io dtype
 *   B, C, d_B, d_C         [b, n, l, h, r]   io dtype (one B/C per head, no groups)
 *   dt, d_dt               [b, h, n, l]      fp32 (the discretised step; no softplus here)
 *   A, D, d_A, d_D         [h]               fp32 (A is used as is: dA = dt * A)
 *   init, final, d_final,
 *   d_init                 [b, h, p, r]      fp32
 *   m2 / m1                [b, h, r, r] / [b, h, r]   fp32
 *   valid_len, count       [b]               int64, HOST memory
 * io dtype SSD_F32: everything fp32.  SSD_BF16: x, B, C, dy, y, d_x, d_B, d_C
 * are bfloat16 (results rounded to nearest even); everything else stays fp32.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, except
 *    valid_len and count (host).  The caller owns every buffer, including the
 *    workspace sized by ssd_workspace_size(); the library never allocates,
 *    frees or synchronises, and enqueues all work on `stream` (a hipStream_t;
 *    NULL = the default stream).
 *  - Outputs are overwritten, never accumulated.  Inputs are not modified.
 *  - Supported shapes: chunk_len in {64, 128, 256}; headdim and dstate in
 *    {16, 32, 64, 128}; batch >= 0, nchunks >= 0 (an empty sequence is valid:
 *    final = init, d_init = d_final, d_A = d_D = 0).  Tensor pointers must be
 *    16-byte aligned (8-byte for bf16 tensors).
 *  - Size limit: one launch holds at most 2^32 - 1 work-items along x (the
 *    dispatch packet's grid size is 32 bits).  Every entry point rejects with
 *    SSD_ERR_UNSUPPORTED a problem whose largest launch would exceed that: for
 *    the chunked entry points batch * nheads * max(4 * nchunks * chunk_len,
 *    headdim * dstate, dstate^2) < 2^32; for ssd_y_diag 16 * ntokens * nheads;
 *    for ssd_step and ssd_moments_pr 256 * batch * nheads; for the quaternion
 *    scan 256 per (batch, 64 quaternions of a row, 64 steps of ssd_quat_scan or
 *    32 steps of ssd_quat_scan_bwd).  Larger problems
 *    are split by the caller (over batch or heads, which are independent).
 *  - kernel_chunk_len: the chunked algorithm is an exact re-association of the
 *    recurrence above for every chunk length, so the kernels may run it at a
 *    shorter chunk than the caller's layout: the [b, n, l, ...] buffers are the
 *    same memory as [b, n * l / k, k, ...] for any k dividing l.  0 picks
 *    min(chunk_len, 128) (on gfx950 the intra-chunk pair work per token grows
 *    with k on the fp32 matrix cores and the inter-chunk state traffic per
 *    token falls with 1/k; 128 balances them for the shapes measured).  Any
 *    other value must be 64, 128 or 256 and divide chunk_len
 *    (SSD_ERR_UNSUPPORTED otherwise).  Results for different kernel_chunk_len
 *    agree up to floating-point rounding; ssd_workspace_size() depends on it.
 *  - Results are bitwise reproducible for equal inputs and kernel_chunk_len
 *    (no float atomics).
 *  - Every call validates all arguments before it enqueues anything.  Return 0
 *    on success or one of the ssd_status codes; ssd_last_error() then gives a
 *    message (thread-local, valid until the next call on the thread).
 */
#ifndef MAMBA_SSD_CHUNKED_AMD_SSD_H
#define MAMBA_SSD_CHUNKED_AMD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssd_dims {
    int64_t batch;     /* b */
    int64_t nchunks;   /* n: sequence length = nchunks * chunk_len */
    int64_t chunk_len; /* l */
    int64_t nheads;    /* h */
    int64_t headdim;   /* p (per_head_dim) */
    int64_t dstate;    /* r (state_rank) */
    int32_t io_dtype;  /* SSD_F32 or SSD_BF16 */
    int32_t kernel_chunk_len; /* chunk length the kernels run at; 0 = automatic (see below) */
} ssd_dims;

enum ssd_io_dtype { SSD_F32 = 0, SSD_BF16 = 1 };

enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a dimension is negative / zero where not allowed, or valid_len out of range */
    SSD_ERR_UNSUPPORTED = 3, /* shape or alignment outside the supported set above */
    SSD_ERR_DTYPE = 4,       /* io_dtype not SSD_F32 / SSD_BF16 */
    SSD_ERR_WORKSPACE = 5,   /* ws_bytes smaller than ssd_workspace_size(), or ws NULL */
    SSD_ERR_HIP = 6,         /* a HIP launch failed (message names the kernel) */
    SSD_ERR_NONFINITE = 7    /* debug mode only: an output holds a NaN or an infinity */
};

enum ssd_op { SSD_OP_FWD = 0, SSD_OP_BWD = 1, SSD_OP_MOMENTS = 2, SSD_OP_MOMENTS_BWD = 3 };

/*
 * Workspace bytes that entry point `op` needs for `dims` (written to *bytes,
 * host).  The value depends only on dims and op.  0 is a valid answer.
 */
int ssd_workspace_size(const ssd_dims* dims, int op, size_t* bytes);

/*
 * Forward (combined_backward.rs page: K1, K2, K3, K4, K5 with the SKIP term).
 *   y           [b,n,l,h,p] out, io dtype
 *   final_state [b,h,p,r]   out, fp32, nullable (not written when NULL)
 *   init        [b,h,p,r]   in, nullable (NULL = zero initial state)
 * Nothing is saved for the backward: ssd_bwd recomputes from the leaves.
 */
int ssd_fwd(const ssd_dims* dims, const void* x, const float* dt, const float* A,
            const void* B, const void* C, const float* D, const float* init,
            void* y, float* final_state, void* ws, size_t ws_bytes, void* stream);

/*
 * The forward with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and kernels as ssd_fwd; the
 * workspace ssd_fwd would take (ssd_workspace_size(dims, SSD_OP_FWD) bytes) is
 * a fixed device array of SSD_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends.  Problems that need more return
 * SSD_ERR_WORKSPACE (use ssd_fwd with a workspace of their own) before anything
 * is enqueued.  The call allocates and frees nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams or
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs clearing between calls (the forward overwrites all of what it reads).
 */
#define SSD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int ssd_fwd_noalloc(const ssd_dims* dims, const void* x, const float* dt, const float* A,
                    const void* B, const void* C, const float* D, const float* init,
                    void* y, float* final_state, void* stream);

/*
 * Recompute backward (combined_backward.rs page: recompute K1-K4, SKIP
 * backward, BLUE/ORANGE and K4 backward, K3/K2/K1 backward, combine).
 *   dy       [b,n,l,h,p] in, io dtype: gradient of y
 *   d_final  [b,h,p,r]   in, nullable (NULL = zero): gradient of final_state
 *   x, dt, A, B, C, D, init: the forward's leaves (init nullable = zero)
 *   d_x, d_B, d_C (io dtype), d_dt, d_A, d_D (fp32): out, all required
 *   d_init   [b,h,p,r]   out, nullable (not written when NULL)
 * d_A and d_D are summed over batch (their parameters are shared by batch).
 */
int ssd_bwd(const ssd_dims* dims, const void* dy, const float* d_final, const void* x,
            const float* dt, const float* A, const void* B, const void* C, const float* D,
            const float* init, void* d_x, float* d_dt, float* d_A, void* d_B, void* d_C,
            float* d_D, float* d_init, void* ws, size_t ws_bytes, void* stream);

/*
 * Pooled state moments (state_moments.rs page, StateMoments): over the tokens
 * t < valid_len[b] of each (b, h), with h_t the state after token t,
 *   m2[b,h] = sum_t h_t^T h_t   [r,r]     m1[b,h] = sum_t sum_p h_t[p,:]   [r]
 *   count[b] = valid_len[b] * headdim  (host, int64)
 * valid_len (host int64 [b]) is nullable (NULL = full sequence); each entry
 * must lie in [0, nchunks * chunk_len].  valid_len masks only the moments.
 * Optionally also runs the forward: y (with C and D) and final_state are
 * nullable; y requires C and D.
 */
int ssd_state_moments(const ssd_dims* dims, const void* x, const float* dt, const float* A,
                      const void* B, const float* init, const int64_t* valid_len,
                      float* m2, float* m1, int64_t* count, void* y, const void* C,
                      const float* D, float* final_state, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Backward of <d_m2, m2> + <d_m1, m1> (moments/backward module page with the
 * rotation equal to the identity): per token t < valid_len[b] the state
 * receives the cotangent h_t (d_m2 + d_m2^T) + 1_p (outer) d_m1.
 *   d_m2 [b,h,r,r] in (need not be symmetric); d_m1 [b,h,r] in, nullable (= 0)
 *   d_x, d_B (io dtype), d_dt, d_A (fp32): out; d_init out, nullable
 * Tokens at or past valid_len get exactly zero gradient.
 */
int ssd_state_moments_bwd(const ssd_dims* dims, const float* d_m2, const float* d_m1,
                          const void* x, const float* dt, const float* A, const void* B,
                          const float* init, const int64_t* valid_len, void* d_x,
                          float* d_dt, float* d_A, void* d_B, float* d_init, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Participation ratio of the pooled moments (state_moments.rs page,
 * StateMoments::pr and StateMoments::trace), per (b, h) slice with
 * n = count[b], mu = m1 / n:
 *   Sigma = m2 / n  (center != 0: Sigma = m2 / n - mu mu^T)
 *   s     = max(tr Sigma, 2^-126)          (fp32's smallest normal)
 *   pr    = tr(Sigma/s)^2 / max(||Sigma/s||_F^2, 1e-12)
 *   trace = tr(m2) / n                     (raw, never centred)
 * The floors only act on a vanishing state: s on Sigma == 0, the 1e-12
 * denominator clamp once the state has collapsed (it then drags pr below 1).
 *   batch >= 0, nheads > 0, dstate in {16, 32, 64, 128} (as for the moments)
 *   m2     [b,h,r,r] in, fp32, 16-byte aligned
 *   m1     [b,h,r]   in, fp32; required when center != 0, else ignored (may be NULL)
 *   count  [b]       in, HOST int64, each > 0 (ssd_state_moments' count; the page
 *                    has one count for all rows, here each row has its own)
 *   pr     [b,h]     out, fp32
 *   trace  [b,h]     out, fp32, nullable (not written when NULL)
 * Sums and Sigma are formed in fp64; results are rounded to fp32 once.
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE (a dimension out of range, count <= 0),
 * SSD_ERR_UNSUPPORTED (dstate, alignment, size limit), SSD_ERR_HIP.  No workspace.
 */
int ssd_moments_pr(int64_t batch, int64_t nheads, int64_t dstate, const float* m2,
                   const float* m1, const int64_t* count, int center, float* pr, float* trace,
                   void* stream);

/*
 * Gradient of sum_{b,h} d_pr[b,h] * pr[b,h] with respect to m2 and m1, with the
 * normaliser s held fixed as on the page (it is detached there; the ratio does
 * not change with the scale of Sigma, so this is also the exact gradient of
 * (tr Sigma)^2 / ||Sigma||_F^2 wherever the 1e-12 clamp is inactive):
 *   G     = d_pr (2 tr1/tr2 I - 2 tr1^2/tr2^2 Sigma/s) / s,  tr1 = tr(Sigma)/s,
 *           tr2 = max(||Sigma/s||_F^2, 1e-12); the Sigma term is dropped while
 *           the clamp is active
 *   d_m2  = G / n                                   [b,h,r,r] out, fp32, 16-byte aligned
 *   d_m1  = -(G + G^T) mu / n when center, else 0   [b,h,r] out, fp32, nullable
 * d_pr [b,h] in, fp32; m2, m1, count, center as for ssd_moments_pr.  The result
 * stays finite for every state magnitude down to the floors.
 */
int ssd_moments_pr_bwd(int64_t batch, int64_t nheads, int64_t dstate, const float* d_pr,
                       const float* m2, const float* m1, const int64_t* count, int center,
                       float* d_m2, float* d_m1, void* stream);

/*
 * Gamma-weighted same-step correction of the Mamba-3 SSD (burn-mamba page
 * "mamba3/single_ssd/ssd/serial_recalculated/diag.rs": module doc and the
 * general MIMO path; at mimo_rank 1 its SISO path).  The term has no recurrence:
 * per token t of the flattened [b, n, l] axes and head h,
 *   qk[mo][mi]    = sum_r C[t,mo,h,r] B[t,mi,h,r]          (m x m, m = mimo_rank)
 *   y_diag[t,mo,h,p] = gamma[t,h] sum_mi qk[mo][mi] v[t,mi,h,p]
 * The Mamba-3 chunk scan adds it to its output; it is exposed here as its own
 * term (overwritten, not added).
 *   ntokens >= 0 (= b * n * l), mimo_rank in {1, 2, 4}, nheads > 0,
 *   headdim and dstate in {16, 32, 64, 128}
 *   v, y_diag   [T, m, h, p]  io dtype (the page's [b, n, l, m, h, p])
 *   B, C        [T, m, h, r]  io dtype
 *   gamma       [T, h]        fp32
 * io tensors 16-byte aligned (8-byte for bf16).  fp32 accumulation; bf16
 * outputs rounded to nearest even.  No workspace.  Errors: SSD_ERR_NULL,
 * SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED, SSD_ERR_DTYPE, SSD_ERR_HIP.
 */
int ssd_y_diag(int64_t ntokens, int64_t mimo_rank, int64_t nheads, int64_t headdim,
               int64_t dstate, int io_dtype, const void* v, const void* B, const void* C,
               const float* gamma, void* y_diag, void* stream);

/*
 * Gradients of <dy, y_diag> (the page's analytic backward of the correction):
 *   DV[mo][mi] = sum_p dy[mo,p] v[mi,p]
 *   d_gamma    = sum_{mo,mi} qk[mo][mi] DV[mo][mi]                [T, h] fp32
 *   d_v[mi,p]  = gamma sum_mo qk[mo][mi] dy[mo,p]                like v
 *   d_C[mo,r]  = gamma sum_mi DV[mo][mi] B[mi,r]                 like C
 *   d_B[mi,r]  = gamma sum_mo DV[mo][mi] C[mo,r]                 like B
 * dy like y_diag; all outputs required and overwritten.
 */
int ssd_y_diag_bwd(int64_t ntokens, int64_t mimo_rank, int64_t nheads, int64_t headdim,
                   int64_t dstate, int io_dtype, const void* dy, const void* v, const void* B,
                   const void* C, const float* gamma, void* d_v, void* d_B, void* d_C,
                   float* d_gamma, void* stream);

/*
 * Quaternion cumulative-product scan of the Mamba-3 rotation (burn-mamba page
 * "mamba3/quat_scan/backward.rs", module doc and "Gradient math").  For every
 * lane (b, h, j), with the Hamilton product (x) on components (w, x, y, z):
 *   cum[b,t,h,j] = q[b,t,h,j] (x) cum[b,t-1,h,j],   cum[b,-1,h,j] = init[b,h,j]
 *   q, cum   [b, s, h, j, 4]  fp32 (nquat = j quaternion blocks per head)
 *   init     [b, h, j, 4]     fp32, nullable (NULL = the identity quaternion)
 * batch >= 0, seq >= 0 (an empty sequence writes nothing), nheads, nquat > 0.
 * Quaternions need not be unit.  Tensors 16-byte aligned; the workspace
 * (ssd_quat_workspace_size, 256-byte aligned) is caller-owned and used by one
 * call at a time.  Products and carries are fp64; cum is rounded to fp32 once.
 * Results are bitwise reproducible: every segment's carry combines the same
 * records in the same order whatever the timing.
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED (size, alignment),
 * SSD_ERR_WORKSPACE, SSD_ERR_HIP.
 */
int ssd_quat_scan(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, const float* q,
                  const float* init, float* cum, void* ws, size_t ws_bytes, void* stream);

/*
 * Gradient of <d_cum, cum> (the page's recompute backward: only the leaves q and
 * init are taken; the scan is recomputed).  Exact for every quaternion: with
 * G_t = d_cum[t] + conj(q_{t+1}) (x) G_{t+1} (G past the end = 0),
 *   d_q[t] = G_t (x) conj(cum[t-1])     [b, s, h, j, 4] out, fp32
 *   d_init = conj(q_0) (x) G_0          [b, h, j, 4]    out, fp32, nullable
 * (for unit quaternions this equals the page's closed form S[0]).  d_cum like q.
 * An empty sequence sets d_init to 0.
 */
int ssd_quat_scan_bwd(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, const float* q,
                      const float* init, const float* d_cum, float* d_q, float* d_init, void* ws,
                      size_t ws_bytes, void* stream);

/* Workspace bytes of ssd_quat_scan (bwd == 0) or ssd_quat_scan_bwd (bwd != 0). */
int ssd_quat_workspace_size(int64_t batch, int64_t seq, int64_t nheads, int64_t nquat, int bwd,
                            size_t* bytes);

/*
 * Decode step: one token of the recurrence from a cached state (the
 * token-by-token `step` loop the burn-mamba "modules/state_moments.rs" page
 * refers to; the recurrence is the one the combined_backward.rs page chunks).
 * Per (b, h):
 *   new_state = exp(dt A) state + dt x (outer) B       [p, r]
 *   y         = new_state C + D x                       [p]
 * which is ssd_fwd over a single token with init = state (final = new_state).
 *   x, y      [b, h, p]     io dtype (the [b, n, l, h, p] layout at n = l = 1)
 *   dt        [b, h]        fp32
 *   A, D      [h]           fp32
 *   B, C      [b, h, r]     io dtype
 *   state, new_state [b, h, p, r]  fp32; new_state may equal state (updated in
 *             place), otherwise the two must not overlap (SSD_ERR_UNSUPPORTED)
 * batch >= 0; headdim and dstate in {16, 32, 64, 128}.  B, C, state, new_state
 * 16-byte aligned (B, C 8-byte for bf16).  No workspace.  Bitwise reproducible.
 * Errors: SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_UNSUPPORTED, SSD_ERR_DTYPE, SSD_ERR_HIP.
 */
int ssd_step(int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate, int io_dtype,
             const void* x, const float* dt, const float* A, const void* B, const void* C,
             const float* D, const float* state, float* new_state, void* y, void* stream);

/* Message for the last nonzero status returned on this thread ("" if none). */
const char* ssd_last_error(void);

/*
 * Debug mode (off by default; a process-wide switch).  While it is on, ssd_fwd,
 * ssd_bwd, ssd_state_moments and ssd_state_moments_bwd end by scanning every output
 * they wrote for a NaN or an infinity, which synchronises `stream`, and return
 * SSD_ERR_NONFINITE (ssd_last_error() names the first such output) instead of 0.
 * The outputs are written as usual.  Not for code under HIP graph capture (the
 * check synchronises).  The scan keeps one flag word per output in a small static
 * device array; a host lock held from clearing those words until their values are
 * back on the host makes checks of overlapping calls (other threads or streams)
 * run one after another, so each call reports only its own outputs.  Returns 0.
 */
int ssd_debug_enable(int on);

/*
 * Benchmark instrumentation (not part of the computation).  While enabled, every
 * kernel an entry point enqueues is bracketed by two HIP events recorded on the
 * caller's stream.  ssd_timing_collect() waits for the recorded events (a host
 * synchronisation), then writes per kernel name (NUL-terminated, at most
 * name_stride bytes each, into names[k * name_stride]) the summed elapsed
 * milliseconds and the number of launches, for up to max_kernels names, sets
 * *n_kernels to the number of distinct names and clears the records.  Returns 0
 * or SSD_ERR_NULL / SSD_ERR_HIP.
 */
int ssd_timing_enable(int on);
int ssd_timing_collect(int max_kernels, char* names, size_t name_stride, double* total_ms,
                       int64_t* launches, int* n_kernels);

/*
 * Benchmark instrumentation (not part of the computation): the HBM rate a plain
 * streaming kernel reaches for a mix of reads and writes, the ceiling that the
 * chunk kernels' byte rates are compared with (the nominal 8 TB/s is not reached
 * by mixes with writes).  Enqueues on `stream` one launch that reads `reads`
 * arrays of n16 16-byte elements from the device buffer src (array a at byte
 * offset 16 * n16 * a) and writes their elementwise float sum to `writes` arrays
 * in the device buffer dst (same layout); with writes = 0 nothing is written.
 * nontemporal != 0 makes every load and store non-temporal.  (reads, writes) is
 * one of (1,0), (6,1), (4,1), (3,1), (2,1), (1,1), (0,1); src must hold at least
 * reads * n16 and dst writes * n16 elements (dst at least n16 with writes = 0),
 * both 16-byte aligned; the caller owns them.  Returns 0, SSD_ERR_UNSUPPORTED for
 * another mix, SSD_ERR_NULL for a missing buffer, SSD_ERR_SHAPE for n16 < 0,
 * SSD_ERR_HIP if the launch fails.  (A grid-stride loop over at most 4096
 * workgroups covers any n16.)
 */
int ssd_stream_probe(int reads, int writes, int nontemporal, const void* src, void* dst,
                     int64_t n16, void* stream);

/*
 * Debug aid (not part of the computation): where ssd_bwd leaves its per-token
 * partials of the gradient w.r.t. the within-chunk cumsum of dt*A in the
 * workspace, so that a test can read them after the call.  They are the
 * pieces the combined_backward.rs page's CombinedGrads exposes for its test
 * of the local d_da: the BLUE + ORANGE gradient w.r.t. the cumsum through the
 * chunk's own terms (entry-state read-out and causal kernel, the entry states
 * held fixed), at the kernel chunk length, equals g1[t] + g2[t] with
 *   "g1"       fp32 [b, h, n*l]: the target-row side, C_t . d_C[t] (BLUE plus
 *              the ORANGE pairs (t, s < t));
 *   "g2"       fp32 [b, h, n*l]: the source-row side, minus the ORANGE pairs
 *              (t > s, s); the diagonal pair, which cancels, is in neither;
 *   "d_delta"  fp32 [b, h, n*l]: the chunk-end state term of the same
 *              gradient (not part of the local d_da).
 * Writes the region's byte offset into a workspace of ssd_workspace_size(dims,
 * SSD_OP_BWD) bytes and its size.  *bytes is 0 where ssd_bwd does not write the
 * region for these dims: g1 when the whole-chunk kernels run (kernel chunk
 * length 128 with headdim * dstate <= 8192), whose target-row kernel suffix-sums
 * g1 in registers, and every region of an empty problem.  Returns
 * SSD_ERR_SHAPE for an unknown name, SSD_ERR_NULL for a NULL argument.
 */
int ssd_bwd_partial_region(const ssd_dims* dims, const char* name, size_t* offset, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_CHUNKED_AMD_SSD_H */
