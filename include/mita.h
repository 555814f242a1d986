/*
 * mita.h - C ABI of the MI355X (gfx950) MiTA library (libmita.so): the forward
 * pass (mita_forward and its variants), its backward pass for training
 * (mita_forward_train, mita_backward), the dense-attention baseline the pages
 * compare against (mita_dense_attention) and peak probes for the roofline.
 *
 * MiTA (Mixture-of-Top-k Attention; Wen et al., arXiv 2602.01219 v6) replaces
 * each query's scan over N keys by m + s*k entries.  Per (b, h) head the
 * forward pass computes, as the MiTA tutorial (iwxt.cn/tutorials/mita-attention)
 * restates paper section 3.2, eqs. 5-12, in its chapter 4:
 *
 *   1. Q~ [m, d]: average pooling of Q over m windows of the token grid;
 *   2. landmark scores s~_ij = q~_i . k_j / sqrt(d) over all N keys;
 *   3. routed expert i = the top-k keys of row i (indices I [m, k]);
 *   4. shared values v~_i = sum_j softmax_j(s~_ij) v_j over all N keys;
 *   5. route every query to the s landmarks with the largest q . q~_i;
 *   6. one softmax over [q~_1..q~_m, the s*k routed keys] with values
 *      [v~_1..v~_m, the routed values]; o = V* softmax(K* q / sqrt(d)).
 *
 * Conventions fixed where the pages leave them open:
 *   - Q~ is the exact window mean rounded once (nearest, ties to even) to the
 *     input dtype; windows are adaptive, half-open
 *     [floor(i*G/P), ceil((i+1)*G/P)) per grid axis.
 *   - tokens n = row*grid_w + col and landmarks i = row*land_w + col
 *     (row-major, as the tutorial's 2x4 grid example in chapter 5);
 *   - top-k and top-s ties go to the lowest index; I rows are returned in
 *     ascending key index, routes by score descending then landmark index;
 *   - every logit is scaled by 1/sqrt(d) (mita_forward_variant can instead
 *     scale the shared logits by 1/d, as the authors' code does); the routing
 *     score is the unscaled q . q~ (same order);
 *   - non-causal: every query sees all m shared entries.
 *
 * Threading and ownership: the caller owns every buffer (inputs, outputs,
 * debug outputs and the workspace).  The library allocates no device memory
 * and keeps no state between calls; mita_forward only validates arguments and
 * enqueues kernels on the caller's HIP stream, then returns without
 * synchronising.  Buffers must stay valid until the stream reaches that point.
 * Calls on different streams must use different workspaces.
 *
 * Errors: every argument is validated before anything is enqueued; on an
 * error nothing is launched and no output is written.  Nothing is thrown
 * across the ABI.
 */
#ifndef MITA_H
#define MITA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MITA_OK = 0,
  MITA_ERR_NULL = 1,        /* a required pointer is NULL */
  MITA_ERR_SHAPE = 2,       /* B,H,N,d <= 0; N != grid_h*grid_w; m != land_h*land_w;
                               landmark grid larger than the token grid */
  MITA_ERR_PARAM = 3,       /* k not in [1, N]; s not in [1, m]; pointer not 16-byte aligned */
  MITA_ERR_UNSUPPORTED = 4, /* d not in {32, 64}; unknown dtype; s > 8; m > 4096;
                               N > 2^26; k > 2048 when N > 8192; B*H > 65535;
                               B*H*N > 2^31 - 1; (backward only) B*H*m*k > 2^31 - 1 */
  MITA_ERR_WORKSPACE = 5,   /* workspace smaller than mita_workspace_bytes() */
  MITA_ERR_HIP = 6          /* the HIP runtime reported an error while enqueueing */
} mita_status;

typedef enum { MITA_F32 = 0, MITA_BF16 = 1 } mita_dtype;

/* Pooling grid: N = grid_h * grid_w tokens, m = land_h * land_w landmarks.
 * A 1-D sequence uses grid_h = land_h = 1. */
typedef struct {
  int grid_h, grid_w, land_h, land_w;
} mita_pool;

/* Optional debug outputs (each may be NULL; the struct pointer may be NULL).
 *   topk   int32 [B, H, m, k]  routed-expert key indices, ascending per row
 *   route  int32 [B, H, N, s]  chosen landmarks, score descending then index
 *   vtilde float [B, H, m, d]  shared values v~ in float32
 *   qtilde dtype [B, H, m, d]  landmark queries q~ in the input dtype
 * They are filled by device-to-device copies enqueued on the same stream. */
typedef struct {
  int32_t* topk;
  int32_t* route;
  float* vtilde;
  void* qtilde;
} mita_debug;

/* Bytes of device workspace mita_forward needs for these arguments (0 if the
 * arguments are invalid).  Host-only; no HIP call. */
size_t mita_workspace_bytes(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool,
                            int m, int k, int s);

/* The MiTA forward pass (steps 1-6 above) for B*H independent heads.
 *   Q, K, V   device, dtype, contiguous [B, H, N, d] (d innermost), read only
 *   O         device, dtype, contiguous [B, H, N, d], written
 *   dbg       optional debug outputs (see mita_debug), or NULL
 *   workspace device buffer of at least mita_workspace_bytes(...) bytes,
 *             16-byte aligned, owned by the caller; contents need not be
 *             initialised and are overwritten
 *   stream    a hipStream_t (NULL = the default stream)
 * Inputs must be finite (non-finite values give unspecified, memory-safe
 * results) and every logit of the three softmaxes -- q~_i . k_j, q_n . q~_i
 * and q_n . k_j, times log2(e) / sqrt(d) -- must stay within 2^30 in
 * magnitude: each exponent is formed by one fused multiply-add of the fp32
 * score, whose rounding residual is half a unit in the last place of the
 * logit (above 2^30 that is more than 2^5, and exp2 can overflow).  Up to
 * 2^15 the residual is below the bf16 rounding of each probability; between
 * 2^15 and 2^30 the softmaxes are one-hot to within that residual.  V may use
 * the whole range of the input dtype.
 * Returns MITA_OK once all work is enqueued. */
mita_status mita_forward(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype,
                         int B, int H, int N, int d, mita_pool pool, int m, int k, int s,
                         const mita_debug* dbg, void* workspace, size_t workspace_bytes,
                         void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mita_forward
 * with no workspace argument.  Its scratch is a device array inside the
 * library, MITA_NOALLOC_SCRATCH_BYTES on every GPU it runs on, kept until the
 * process ends; a call whose mita_workspace_bytes(...) exceeds that returns
 * MITA_ERR_WORKSPACE before any launch (the vision-shaped workloads need
 * 15-22 MiB; long sequences need the caller's workspace and mita_forward).
 * The first call on a device looks the array's address up once (the device
 * that owns Q, K, V, O and the stream must be current, as for every launch).
 * Allocates nothing, synchronises nothing.  All calls on one GPU share its
 * array and each clears what it needs at its start: calls that overlap on one
 * GPU (other streams, other threads) race and give unspecified results --
 * serialise them.  Same arguments, validation and results as mita_forward
 * with dbg = NULL. */
#define MITA_NOALLOC_SCRATCH_BYTES (64u << 20)
mita_status mita_forward_noalloc(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype,
                                 int B, int H, int N, int d, mita_pool pool, int m, int k, int s,
                                 void* stream);

/* Profiling variant: identical work, and additionally records a pair of HIP
 * events around each stage on `stream`.  `events` holds 2 * mita_num_stages()
 * hipEvent_t handles made by mita_events_create (start, stop per stage); a
 * stage whose two handles are NULL is not timed (no record is enqueued).
 * Read the stage times with mita_events_elapsed after the stream finished. */
mita_status mita_forward_timed(const void* Q, const void* K, const void* V, void* O,
                               mita_dtype dtype, int B, int H, int N, int d, mita_pool pool,
                               int m, int k, int s, const mita_debug* dbg, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events);

/* Which entries and logit scales the step-6 softmax uses. */
typedef enum {
  /* 1/sqrt(d), like every other logit: the paper's eqs. 5-12 as the MiTA
   * tutorial's chapter 4 states them. */
  MITA_VARIANT_PAPER = 0,
  /* 1/d: the authors' released code pre-scales the shared key by d^-1/2 and
   * then applies the d^-1/2 logit scale (MiTA tutorial, chapter 8, third
   * check).  Routed logits stay q . k / sqrt(d); pooling, landmark scores,
   * top-k, shared values and routing are those of MITA_VARIANT_PAPER. */
  MITA_VARIANT_OFFICIAL = 1,
  /* Routing-only ablation (no shared branch): each query's softmax runs over
   * the s*k keys of its routed experts alone, with 1/sqrt(d).  Pooling,
   * landmark top-k and routing are unchanged; shared values are not computed
   * and dbg->vtilde is not written.  The pages' ablation matches the entries
   * per query (MiTA republication, "LRA" section): pass k + m/s as k. */
  MITA_VARIANT_ROUTED = 2
} mita_variant;

/* mita_forward / mita_forward_timed with the shared-logit scale chosen by
 * `variant` (any other value returns MITA_ERR_PARAM before any launch).
 * `events` is NULL, or 2 * mita_num_stages() handles as for
 * mita_forward_timed. */
mita_status mita_forward_variant(const void* Q, const void* K, const void* V, void* O,
                                 mita_dtype dtype, int B, int H, int N, int d, mita_pool pool,
                                 int m, int k, int s, mita_variant variant, const mita_debug* dbg,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events);

/* Dense (full) softmax attention O = softmax(Q K^T / sqrt(d)) V for B*H
 * independent heads, non-causal: the baseline of the pages' long-sequence
 * throughput test (MiTA tutorial, chapter 7, "LRA and synthetic long
 * sequences"; paper section 4.3, Fig. 5).  Q, K, V, O as for mita_forward
 * (device, dtype, contiguous [B, H, N, d], 16-byte aligned); no workspace, no
 * allocation, no synchronisation.  Errors: MITA_ERR_NULL (a NULL pointer),
 * MITA_ERR_SHAPE (B, H, N or d <= 0), MITA_ERR_PARAM (misaligned pointer),
 * MITA_ERR_UNSUPPORTED (d not in {32, 64}, unknown dtype, N > 2^26,
 * B*H > 65535), MITA_ERR_HIP (launch failure); nothing is launched on a
 * validation error. */
mita_status mita_dense_attention(const void* Q, const void* K, const void* V, void* O,
                                 mita_dtype dtype, int B, int H, int N, int d, void* stream);

/* ------------------------------------------------------------------------
 * Training: the forward pass that keeps what the backward pass needs, and the
 * backward pass.  The pages train MiTA models end to end (MiTA tutorial,
 * chapter 7: LRA training time) without writing a backward pass; the one here
 * differentiates steps 1-6 with the top-k experts (step 3) and the top-s
 * routes (step 5) held fixed -- choices are constant wherever they are
 * unique, so they pass no gradient -- and takes q~'s rounding to the input
 * dtype as the identity (pooling's adjoint spreads d q~_i / |W_i| over window
 * W_i).  Every other step is differentiated exactly, a key chosen by two of a
 * query's experts counting twice as in the forward.
 * ------------------------------------------------------------------------ */

/* Tensors kept by mita_forward_train for mita_backward: device buffers owned
 * by the caller, written by mita_forward_train, read by mita_backward.
 *   qtilde       dtype [B, H, m, d]  landmark queries q~ (step 1)
 *   vtilde       float [B, H, m, d]  shared values v~ (step 4) before the
 *                step-6 softmax rounded them to the input dtype
 *   topk         int32 [B, H, m, k]  experts (step 3)
 *   route        int32 [B, H, N, s]  routes (step 5)
 *   lse          float [B, H, N]     log2 of each query's step-6 normaliser,
 *                log2(sum_t exp(z_t)) over its logits z_t
 *   lse_landmark float [B, H, m]     log2(sum_j exp(q~_i . k_j / sqrt(d))),
 *                the normaliser of step 4
 *   out_f32      float [B, H, N, d]  the output before rounding to the input
 *                dtype (the backward's dO . o is taken from it: where one
 *                entry dominates a softmax, dP_t - dO . o cancels and the
 *                rounded output would leave a 2^-8 relative error in it)
 * qtilde, vtilde and out_f32 must be 16-byte aligned.  In MITA_VARIANT_ROUTED there is
 * no step 4: vtilde and lse_landmark are not written or read and may be
 * NULL.  mita_backward needs the contents written by mita_forward_train for
 * the same inputs and arguments; other contents give unspecified results (all
 * indices are clamped, so memory accesses stay in bounds). */
typedef struct {
  void* qtilde;
  float* vtilde;
  int32_t* topk;
  int32_t* route;
  float* lse;
  float* lse_landmark;
  float* out_f32;
} mita_saved;

/* mita_forward_variant (same arguments, same workspace size, same errors)
 * that also fills `saved` (MITA_ERR_NULL if saved or a required member is
 * NULL; MITA_ERR_PARAM if qtilde, vtilde or out_f32 is misaligned). */
mita_status mita_forward_train(const void* Q, const void* K, const void* V, void* O,
                               mita_dtype dtype, int B, int H, int N, int d, mita_pool pool,
                               int m, int k, int s, mita_variant variant, const mita_saved* saved,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace mita_backward needs (0 if the arguments are
 * invalid).  Host-only; no HIP call.  It holds, besides O(B*H*N) index and
 * scalar arrays, the routed key parts (s*B*H*m*k*2d fp32) and the
 * landmark-row partials of the two chunked passes. */
size_t mita_backward_workspace_bytes(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool,
                                     int m, int k, int s);

/* Gradients of sum(O * dO) with respect to Q, K and V.
 *   Q, K, V, O  the forward's inputs and output (device, dtype, [B, H, N, d];
 *               O is validated like the others but not read: saved->out_f32
 *               stands in for it)
 *   dO          device, dtype, [B, H, N, d]: the upstream gradient
 *   dQ, dK, dV  device, dtype, [B, H, N, d], written (accumulated in fp32,
 *               rounded once)
 *   variant     the variant the forward ran with
 *   saved       the tensors mita_forward_train kept
 *   workspace   device, >= mita_backward_workspace_bytes(...), 16-byte
 *               aligned, caller-owned, need not be initialised
 * All pointers 16-byte aligned.  Same shape limits and errors as
 * mita_forward (MITA_ERR_NULL also for a NULL dO, dQ, dK, dV or saved
 * member), and MITA_ERR_UNSUPPORTED when B*H*m*k > 2^31 - 1; nothing is
 * launched on a validation error.  A key held by several experts receives
 * their parts in an order that may change from call to call, so dK and dV
 * may differ in the last bits between calls; dQ is deterministic. */
mita_status mita_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                          void* dQ, void* dK, void* dV, mita_dtype dtype, int B, int H, int N, int d,
                          mita_pool pool, int m, int k, int s, mita_variant variant,
                          const mita_saved* saved, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Peak probes for the roofline (measurement only; no part of the forward or
 * backward pass uses them).  Each enqueues one kernel on `stream`.
 *   mita_probe_mfma  `blocks` workgroups of 256 threads; every wave runs
 *                    `iters` rounds of eight independent 16x16x32 bf16
 *                    matrix operations, blocks * 4 * iters * 8 * 16384 flops
 *                    in all; writes blocks * 256 floats to `out` (device).
 *   mita_probe_copy  copies `bytes` (a multiple of 16) from src to dst
 *                    (device, 16-byte aligned, not overlapping).
 *   mita_probe_step  the online-softmax step the attention kernels are built
 *                    on (MiTA tutorial (iwxt.cn) ch.4: softmax over
 *                    q~ . k / sqrt(d) weighting V; here d = 64, bf16), run
 *                    `iters` times per 16-row block with every operand in
 *                    registers: the ceiling of a kernel made of that step at
 *                    one launch shape.  `shape` 0: workgroups of 8 waves x 4
 *                    blocks (two waves per SIMD); 1: 16 waves x 1 block (four
 *                    per SIMD); 2: 8 waves x 2 blocks (two workgroups per
 *                    compute unit); 3: 16 waves x 2 blocks.  One step of one
 *                    block is 8 useful 16x16x32 products (scores and P.V,
 *                    131072 flops) plus one for the normaliser.  Writes
 *                    blocks * (512, or 1024 for shapes 1 and 3) floats to
 *                    `out` (device).
 * Errors: MITA_ERR_NULL (NULL pointer), MITA_ERR_PARAM (blocks or iters
 * <= 0, shape outside 0..3, bytes not a multiple of 16, misaligned pointer),
 * MITA_ERR_HIP. */
mita_status mita_probe_mfma(float* out, int blocks, int iters, void* stream);
mita_status mita_probe_copy(const void* src, void* dst, size_t bytes, void* stream);
mita_status mita_probe_step(float* out, int shape, int blocks, int iters, void* stream);

/* Number of timed stages and their names ("pool", "estimate", "score", ...). */
int mita_num_stages(void);
const char* mita_stage_name(int stage);

/* Create / destroy `count` HIP events with timing enabled and without the
 * system-scope memory fence (they time the stream; they do not make device
 * memory visible to the host), written to events[0..count).  Destroy skips
 * NULL handles.  mita_events_elapsed fills ms[i] with the time between
 * events[2i] and events[2i+1] for i < n_pairs, blocking until they complete;
 * a stage that launched nothing reports 0, a pair of NULL handles NaN. */
mita_status mita_events_create(void** events, int count);
mita_status mita_events_destroy(void** events, int count);
mita_status mita_events_elapsed(void* const* events, int n_pairs, float* ms);

/* Human-readable text for a status code (static storage). */
const char* mita_status_str(mita_status status);

/* Library version string. */
const char* mita_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MITA_H */
