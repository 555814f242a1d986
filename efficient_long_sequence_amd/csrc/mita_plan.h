// Host-side launch plan: every size, launch shape and workspace region of one
// mita_forward call, derived from the arguments alone (so sizing and running
// agree by construction).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mita {

// Rows of N up to this size keep every landmark score as a candidate ("dense"
// selection); above it a sampled threshold filters candidates first.
constexpr int NSMALL = 8192;
// Rows of N up to SMALL_N keys with k <= SMALL_K select their top-k on chip
// (k_topk_small) and write no candidates at all.
constexpr int SMALL_N = 2048;
constexpr int SMALL_K = 64;
// Candidate capacity per landmark row in sparse mode: the selection kernel
// gathers a row's candidates into LDS (up to 8192 x 8 bytes).  The threshold
// admits about 2.3 k keys per row, so the capacity follows k (8 k rounded up
// to a power of two, at least 2048), and a row past it falls back to the
// exact kernel; smaller buffers let more selection workgroups share a
// compute unit.
constexpr int CAPG = 8192;
constexpr int CAPG_MIN = 2048;
// Sparse mode: the least room for score records a lane keeps per (landmark
// row, key chunk, lane group) (more when the expected count is larger); a lane
// that needs more marks its row for the exact fallback.
constexpr int REC_MIN = 32;
constexpr int MAX_S = 8;
constexpr int MAX_M = 4096;
constexpr int MAX_K_SPARSE = 2048;
constexpr long long MAX_N = 1LL << 26;
// Stages reported by the profiling entry point.
enum Stage { ST_POOL = 0, ST_EST, ST_SCORE, ST_FINAL, ST_ROUTE, ST_BUCKET, ST_ATTEND, ST_COUNT };

struct WorkItem {
  int start;  // first position in the slot's permutation array
  int count;  // queries in this tile
  int be;     // bh * m + expert
  int pad;
};

// Outputs the forward keeps for the backward pass (each nullptr: not written).
struct TrainOut {
  float* lse;  // [BH, N] log2-sum-exp of each query's joint softmax
  float* o32;  // [BH, N, d] output before rounding to the input dtype
};

struct Plan {
  // arguments
  int dtype;  // 0 f32, 1 bf16
  int esize;  // bytes per element
  int B, H, BH, N, d, gh, gw, lh, lw, m, k, s;
  // landmark scoring
  int dense;      // 1: every score is a candidate
  int small;      // 1 (dense rows only): top-k selected on chip by k_topk_small
  int capg;       // candidate slots per landmark row
  int sc_nw, sc_ib, sc_R, sc_rt;  // waves, 16-row blocks per wave, rows per tile, row tiles
  int L, C;       // keys per chunk, chunks per head
  int s4;         // sparse mode: records per (row, chunk, lane group)
  // threshold estimate (sparse mode)
  int sigma;      // sample stride
  int NS;         // samples per head
  int G;          // sample groups per landmark row
  int J;          // rank of the threshold among the group maxima
  int est_gpb;    // groups per estimator workgroup
  int force_fallback;  // test hook: every row takes the exact fallback path
  // routing / attention
  int smax;       // compiled top-s list length (>= s)
  int at_nw, at_ib, T;  // attention waves, 16-query blocks per wave, queries per tile
  int UB;         // upper bound on work items per slot
  int fast;       // LDS-resident routing + shared part and per-expert attention
  int rs_qpw;     // queries per routing workgroup (resident path)
  int rs_nw;      // its waves: 8 (four 16-query blocks each), 12 (two) or 16 (one)
  int ex_nw, ex_ib;  // expert kernel waves and 16-query blocks per query group
  float cscale;   // log2(e) / sqrt(d)
  float cscale_sh;  // log2(e) times the scale of the shared logits (1/sqrt(d) or 1/d)
  int shared;       // 1: shared entries in the joint softmax; 0: routing-only variant

  // workspace regions
  void* qt;         // [BH, m, d] dtype
  float* gmax;      // [BH, m, G]
  float* tau;       // [BH, m] raw-score threshold
  float* mhat;      // [BH, m] sample maximum (raw)
  float* vpart;     // [BH, m, C, d + 4]: max, normaliser, 2 pad, d sums
  uint64_t* cand;   // [BH, m, capg]     (dense mode: every score as a candidate key)
  float* rec_sc;    // [BH, m, C, 4, s4, 8] sparse mode: the 8 raw scores of a lane step holding a candidate
  int32_t* rec_st;  // [BH, m, C, 4, s4]    its step inside the chunk
  int* rec_cnt;     // [BH, m, C, 4]        records the lane found (may exceed s4: the row falls back)
  int* counts;      // [s, BH, m]        (zeroed each call)
  int* cursor;      // [s, BH, m]        (zeroed each call)
  int* fail;        // [BH, m]
  int32_t* topk;    // [BH, m, k]
  float* vt32;      // [BH, m, d]
  void* vtT;        // [BH, m, d] dtype
  int32_t* route;   // [BH, N, s]
  int* gpre;        // [s, BH, m] exclusive prefix of counts
  int32_t* perm;    // [s, BH * N]
  WorkItem* wl;     // [s, UB]
  int* wl_count;    // [s]
  float* part;      // [s - 1, BH, N, d + 4]  (streaming path)
  float2* plse;     // [BH, N] (log2-sum-exp, row scale) of the finished part (resident path)
  void* po;         // [BH, N, d] output of the finished part divided by its row scale (fp16, |x| <= 1;
                    // fp32 with scale 1 for fp32 inputs)
  void* zero_begin;
  size_t zero_bytes;
  size_t total_bytes;

  // optional outputs kept for the backward pass (nullptr: not written)
  float* lse_out;   // [BH, N] log2-sum-exp of each query's joint softmax
  float* lse_lm;    // [BH, m] log2-sum-exp of each landmark row over all N keys
  float* o32;       // [BH, N, d] the output before rounding to the input dtype

  // call
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  hipStream_t stream;
};

// Launchers (one per translation unit); each enqueues on plan.stream.
void launch_pool(const Plan& p);  // also clears zero_bytes at zero_begin
void launch_estimate(const Plan& p);
void launch_score(const Plan& p);
void launch_final(const Plan& p);
void launch_route(const Plan& p);
void launch_bucket(const Plan& p);
// another work list over the same counts with items of at most T queries,
// recording each expert's full items (efirst) and partial item (epart)
void launch_items(const Plan& p, int T, int UB, WorkItem* wl, int* wl_count, int* efirst, int* epart);
void launch_attend(const Plan& p);
void launch_route_shared(const Plan& p);
void launch_expert(const Plan& p);
// dense softmax attention over B*H heads (the full-attention baseline)
void launch_dense(const void* Q, const void* K, const void* V, void* O, int dtype, int BH, int N, int d,
                  hipStream_t stream);
size_t resident_bytes(int dtype, int d, int E);

// Host-side plan of one backward call (mita_backward): sizes, launch shapes
// and workspace regions, derived from the arguments alone.
struct BPlan {
  int dtype, esize, BH, N, d, gh, gw, lh, lw, m, k, s;
  int shared;            // 1: shared entries in the joint softmax (not the routing-only variant)
  float cscale, cscale_sh;  // log2(e) x logit scale (routed / shared logits)
  float cnat, cnat_sh;      // the logit scales themselves
  int R;                 // stationary rows per workgroup
  int L1, C1;            // joint pass over queries: entries per chunk, chunks
  int L4, C4;            // shared-value pass over keys: entries per chunk, chunks
  Plan bk;               // query grouping by expert (counts, prefix, permutation, work list)

  // workspace
  float* Dn;      // [BH, N] dO . O per query
  int CH;         // queries per item of the routed-key pass
  int UB2;        // upper bound on its items per slot
  WorkItem* wl2;  // [s, UB2] its items
  int* wl2_count; // [s]
  int* efirst;    // [s, BH, m] first full item of each expert
  int* epart;     // [s, BH, m] partial item of each expert (-1: none)
  float* G;       // [s, UB2, k, 2d] routed dk, dv per (slot, item, expert row)
  float* Gs;      // [BH * m * k, 2d] each key's summed routed parts, at its first list position
  void* Qg;       // [s, BH * N, d] q in each slot's expert order
  void* dOg;      // [s, BH * N, d] dO likewise
  float* Lg;      // [s, BH * N] lse likewise
  float* Dg;      // [s, BH * N] dO . o likewise
  int* icnt;      // [BH * N] expert rows holding each key (zeroed each call)
  int* icur;      // [BH * N] fill cursors (zeroed each call)
  int* ipos;      // [BH * N] exclusive prefix of icnt
  int* bsum;      // per-block totals of the prefix
  int32_t* ilist; // [BH * m * k] (expert * k + row) of each key, grouped by key
  int32_t* ikey;  // [BH * m * k] the key (bh * N + j) of each list position
  float* part1;   // [BH, C1, m, 2d] per-chunk dq~ and dv~ of the joint softmax
  float* part4;   // [BH, C4, m, d] per-chunk dq~ of the shared-value softmax
  float* dqt;     // [BH, m, d] dq~
  float* dvt;     // [BH, m, d] dv~
  void* dvtT;     // [BH, m, d] dv~ in the input dtype (matrix-core operand)
  float* delta;   // [BH, m] dv~ . v~
  float* qpart;   // [s - 1, BH, N, d] dQ of slots 1 .. s-1
  // (vt, the input-dtype copy of the saved v~, is also a workspace region)
  void* zero_begin;
  size_t zero_bytes;
  size_t total_bytes;

  // call
  const void *Q, *K, *V, *O, *dO;
  void *dQ, *dK, *dV;
  const void* qt;         // saved q~ [BH, m, d]
  const float* vt32;      // saved v~ [BH, m, d] (fp32)
  void* vt;               // v~ rounded to the input dtype as the forward used it (workspace)
  const float* o32;       // saved output before rounding [BH, N, d]
  const int32_t* topk;    // saved experts [BH, m, k]
  const int32_t* route;   // saved routes [BH, N, s]
  const float* lse;       // saved [BH, N]
  const float* lse_lm;    // saved [BH, m]
  hipStream_t stream;
};
void launch_backward(const BPlan& p);
// peak probes (measurement only)
void launch_probe_mfma(float* out, int blocks, int iters, hipStream_t stream);
void launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
// the online-softmax step alone (shape 0: 8 waves x 4 blocks, 1: 16 x 1,
// 2: 8 x 2, 3: 16 x 2); probe_step_threads: its workgroup size
void launch_probe_step(float* out, int shape, int blocks, int iters, hipStream_t stream);
int probe_step_threads(int shape);
// stationary rows per workgroup of the backward's joint landmark pass for m
// landmarks (dtype 0 f32, 1 bf16)
int backward_rows(int dtype, int m);
// queries per workgroup of the backward's query pass (its work-item size)
int backward_query_rows(int dtype);
// landmark rows per workgroup of the shared-value landmark pass
int backward_lm4_rows(int dtype, int m);
// LDS a resident entry set may take (of 160 KB per compute unit).
constexpr size_t RES_MAX = 150 * 1024;

}  // namespace mita
