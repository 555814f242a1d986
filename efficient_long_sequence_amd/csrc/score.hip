// Steps 2-4 of MiTA: landmark scores, per-landmark top-k and shared values.
// (MiTA tutorial (iwxt.cn), ch.4 steps 2-3, paper section 3.2: every
// landmark q~_i scores all N keys with q~_i . k_j / sqrt(d); its top-k keys
// form routed expert i; the softmax of the same scores over all N keys
// weights V into the shared value v~_i.)
//
// Kernels, in launch order:
//   k_est     (large N only) scores every landmark against a strided sample of
//             the keys on the matrix cores and keeps the maximum of each of G
//             sample groups;
//   k_tau     per landmark row: the J-th largest group maximum becomes the
//             candidate threshold tau, the largest one the first softmax
//             offset;
//   k_score   one workgroup per (head, landmark-row tile, key chunk): the
//             score tile Q~ K^T on the matrix cores, an online softmax with
//             P.V on the matrix cores (partial v~ per chunk), and a record of
//             the 8 scores of every lane step holding a score >= tau (for
//             N <= 8192 rows with k > 64 or N > 2048: every score as a
//             candidate key).  Apart from that last case the m x N score
//             matrix never reaches HBM;
//   k_final   per landmark row: merges the v~ partials (the rescaled-sum
//             identity (Z1 o1 + Z2 o2)/(Z1 + Z2) of tutorial ch.4) and selects
//             the exact top-k from the candidates with a block radix select;
//   k_topk_small  (rows of at most 2048 keys, k <= 64, instead of the
//             candidate path) rescores 16 rows into LDS and selects each
//             row's top-k there with a wave-level bitwise search;
//   k_fallback exact streaming top-k for any row whose candidate count was
//             below k or above capacity (a threshold estimate that missed).
//
// Exactness of the selection: the candidates of a row are exactly the keys
// whose fp32 score is >= tau, an upper set of the score order.  If there are
// at least k of them, the k largest candidates (ties to the lower index) are
// the k largest keys of the whole row; otherwise the row is redone by
// k_fallback.  tau only decides how much work this takes, never the result.
#include <algorithm>

#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

__device__ __forceinline__ int sample_pos(int t, int sigma) {
  uint32_t h = (uint32_t)t * 2654435761u;
  h ^= h >> 15;
  return t * sigma + (int)(h % (uint32_t)sigma);
}

// ---------------------------------------------------------------------------
// sampled group maxima
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int IB>
__global__ __launch_bounds__(NW * 64) void k_est(const T* __restrict__ K, const T* __restrict__ Qt,
                                                 float* __restrict__ gmax, int N, int m, int sigma,
                                                 int NS, int G, int gpb) {
  constexpr int NT = NW * 64;
  using TL = TileLayout<T, D>;
  __shared__ __align__(16) T ks[TL::K_ELEMS];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int bh = blockIdx.z, rt = blockIdx.y;
  const int rbase = rt * (NW * 16 * IB) + wave * 16 * IB;
  const T* Kh = K + (size_t)bh * N * D;

  Frag<T> qf[IB][D / 32];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int row = rbase + b * 16 + li;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (row < m) load8(qf[b][dc], Qt + ((size_t)bh * m + row) * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
  }
  TileLoader<T, D, NT, false> ld;
  // Group g holds the samples t = u * G + g, u < Sg: its keys are spread over
  // the whole sequence, so runs of similar keys do not pile into one group.
  const int Sg = NS / G;
  for (int gl = 0; gl < gpb; ++gl) {
    const int grp = blockIdx.x * gpb + gl;
    if (grp >= G) break;
    float run[IB];
#pragma unroll
    for (int b = 0; b < IB; ++b) run[b] = -INFINITY;
    for (int u0 = 0; u0 < Sg; u0 += 32) {
      ld.load([&](int r) -> const T* {
                const int u = u0 + r;
                return u < Sg ? Kh + (size_t)sample_pos(u * G + grp, sigma) * D : nullptr;
              },
              [](int) -> const T* { return nullptr; });
      __syncthreads();
      ld.store(ks, nullptr);
      __syncthreads();
      StepFrags<T, D> f;
      f.load_keys(ks, li, lg);
      const int nv = min(32, Sg - u0);
#pragma unroll
      for (int b = 0; b < IB; ++b) {
        float sc[8];
        step_scores(f, qf[b], sc);
        if (nv < 32) {
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (slot_key(t, lg) >= nv) sc[t] = -INFINITY;
        }
        run[b] = fmaxf(run[b], max8(sc));
      }
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const float gm = wave_max_groups(run[b]);
      const int row = rbase + b * 16 + li;
      if (row < m && lg == 0) gmax[((size_t)bh * m + row) * G + grp] = gm;
    }
  }
}

__global__ void k_fill(float* __restrict__ p, int n, float v) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}


// ---------------------------------------------------------------------------
// fused scores, partial shared values and candidates
// ---------------------------------------------------------------------------
// Waves per SIMD the register budget must allow: the 16-row bf16 tiling keeps
// two 8-wave workgroups per CU.
template <typename T, int NW, int IB>
constexpr int score_waves_per_eu() { return (sizeof(T) == 2 && NW == 8 && IB == 1) ? 4 : 2; }

// Candidate output of the scoring kernel: SEL_SPARSE, score records of the
// lanes holding a score >= tau; SEL_DENSE, every score as a candidate key;
// SEL_NONE, nothing (small rows select on chip in k_topk_small).
enum { SEL_SPARSE = 0, SEL_DENSE = 1, SEL_NONE = 2 };

// SHARED = false (routing-only variant): keys only, no softmax, no P.V and no
// shared-value partials; the scores feed the candidates alone.
template <typename T, int D, int NW, int IB, int SEL, bool SHARED>
__global__ __launch_bounds__(NW * 64, (score_waves_per_eu<T, NW, IB>())) void k_score(
    const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Qt,
    const float* __restrict__ tau_in, const float* __restrict__ mhat_in, float* __restrict__ vpart,
    uint64_t* __restrict__ cand, float* __restrict__ rec_sc, int32_t* __restrict__ rec_st,
    int* __restrict__ rec_cnt, int N, int m, int L, int C, int capg, int s4, float cscale) {
  constexpr int NT = NW * 64;
  constexpr int R = NW * 16 * IB;
  using TL = TileLayout<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* buf0 = (T*)smem;
  T* buf1 = buf0 + TL::ELEMS;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const Frag<T> one = ones_frag<T>(li);
  const int ch = blockIdx.x, rt = blockIdx.y, bh = blockIdx.z;
  const int rbase = rt * R + wave * 16 * IB;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;
  const int j_begin = ch * L, j_end = min(N, j_begin + L);
  // sparse mode: every lane appends its own records (no cross-lane work on
  // the inner loop); rcnt[b] counts those of block b
  int rcnt[IB];
  uint32_t rbase32[IB];  // each block's first record of this lane (the plan keeps record indices in 32 bits)
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    rcnt[b] = 0;
    rbase32[b] = (uint32_t)(((((size_t)bh * m + rbase + b * 16 + li) * C + ch) * 4 + lg) * s4);
  }

  Frag<T> qf[IB][D / 32];
  float tau[IB];
  RunMax M[IB];
  f32x4 Z[IB];
  f32x4 acc[IB][D / 16];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int row = rbase + b * 16 + li;
    const bool valid = row < m;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (valid) load8(qf[b][dc], Qt + ((size_t)bh * m + row) * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
    M[b].set((mhat_in != nullptr && valid) ? mhat_in[(size_t)bh * m + row] * cscale : M0, cscale);
    tau[b] = SEL != SEL_SPARSE ? -INFINITY : (valid ? tau_in[(size_t)bh * m + row] : INFINITY);
    Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto rowK = [&](int j0) {
    return [=](int r) -> const T* { const int j = j0 + r; return j < j_end ? Kh + (size_t)j * D : nullptr; };
  };
  auto rowV = [&](int j0) {
    return [=](int r) -> const T* { const int j = j0 + r; return j < j_end ? Vh + (size_t)j * D : nullptr; };
  };

  // two register stages: the loads of step st + 2 are issued at the start of
  // step st, the tile of step st + 1 (loaded a step earlier) is stored at its
  // end; the two loaders swap roles every step (the loop is unrolled by two)
  TileLoader<T, D, NT, SHARED> la, lb;
  const int nsteps = (j_end - j_begin + 31) / 32;
  la.load(rowK(j_begin), rowV(j_begin));
  la.store(buf0, buf0 + TL::K_ELEMS);
  if (nsteps > 1) la.load(rowK(j_begin + 32), rowV(j_begin + 32));
  __syncthreads();
  // one 32-key step; MASKED: the chunk's last, partial step (its absent keys
  // get score -inf).  The partial step is peeled off the loop: with both
  // forms of the step in the loop body the kernel runs out of registers.
  auto body = [&](int st, auto masked, auto& lnext, auto& lfar) {
    constexpr bool MASKED = decltype(masked)::value;
    const int j0 = j_begin + st * 32;
    T* cur = (st & 1) ? buf1 : buf0;
    T* nxt = (st & 1) ? buf0 : buf1;
    const bool more = st + 1 < nsteps;
    if (st + 2 < nsteps) lfar.load(rowK(j0 + 64), rowV(j0 + 64));
    StepFrags<T, D> f;
    f.load_keys(cur, li, lg);
    if constexpr (SHARED) f.load_vals(cur + TL::K_ELEMS, li, lg);
    const int nv = min(32, j_end - j0);
    // per row block: every score of a small head is a candidate (DENSE);
    // otherwise a lane holding a score >= tau keeps a record: its 8 raw
    // scores and the step (the selection filters them against tau)
    auto cands = [&](int b, const float* sc, float mx) {
      const int row = rbase + b * 16 + li;
      if constexpr (SEL == SEL_DENSE) {
        if (row < m) {
          uint64_t* dst = cand + ((size_t)bh * m + row) * capg + j0;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int kl = slot_key(t, lg);
            if (kl < nv) dst[kl] = ckey(sc[t], (uint32_t)(j0 + kl));
          }
        }
      } else if (SEL == SEL_SPARSE) {
        // (rows past m have tau = +inf and never get here)
        if (mx >= tau[b]) {
          // past the lane's s4 records the last one is overwritten: the
          // count then exceeds s4 and the row takes the exact fallback
          const int c = rcnt[b];
          const uint32_t e = rbase32[b] + (uint32_t)min(c, s4 - 1);
          float4* dst = (float4*)(rec_sc + (size_t)e * 8);
          dst[0] = make_float4(sc[0], sc[1], sc[2], sc[3]);
          dst[1] = make_float4(sc[4], sc[5], sc[6], sc[7]);
          rec_st[e] = st;
          rcnt[b] = c + 1;
        }
      }
    };
    if constexpr (SHARED) attn_step<IB, MASKED>(f, one, qf, nv, lg, cscale, M, Z, acc, cands);
    else score_step<IB, MASKED>(f, qf, nv, lg, cands);
    if (more) lnext.store(nxt, nxt + TL::K_ELEMS);
    __syncthreads();
  };
  const int nfull = (j_end - j_begin) / 32;
  int st = 0;
  for (; st + 1 < nfull; st += 2) {
    body(st, BoolTag<false>{}, la, lb);
    body(st + 1, BoolTag<false>{}, lb, la);
  }
  if (st < nfull) {
    body(st, BoolTag<false>{}, la, lb);
    ++st;
    if (st < nsteps) body(st, BoolTag<true>{}, lb, la);
  } else if (st < nsteps) {
    body(st, BoolTag<true>{}, la, lb);
  }

  // partial shared values of this chunk: (max, normaliser, 2 pad, unnormalised sums)
  if constexpr (SHARED) {
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const float Zt = finish_z(Z[b], li);
      const int row = rbase + b * 16 + li;
      if (row < m) {
        float* dst = vpart + (((size_t)bh * m + row) * C + ch) * (D + 4);
        if (lg == 0) { dst[0] = M[b].M; dst[1] = Zt; }
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
          *(float4*)(dst + 4 + cb * 16 + 4 * lg) =
              make_float4(acc[b][cb][0], acc[b][cb][1], acc[b][cb][2], acc[b][cb][3]);
      }
    }
  }

  if constexpr (SEL == SEL_SPARSE) {
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const int row = rbase + b * 16 + li;
      if (row < m) rec_cnt[(((size_t)bh * m + row) * C + ch) * 4 + lg] = rcnt[b];
    }
  }
}

// ---------------------------------------------------------------------------
// selection and shared-value merge, one workgroup per landmark row
// ---------------------------------------------------------------------------
// Writes the k indices of the block-sorted keys a[0..k) (descending order)
// in ascending index order to out[0..k).  Reuses a[] as scratch.
__device__ void emit_topk(uint64_t* a, int k, int32_t* out) {
  const int Pk = next_pow2(k < 2 ? 2 : k);
  for (int j = threadIdx.x; j < Pk; j += blockDim.x)
    a[j] = j < k ? (uint64_t)ckey_idx(a[j]) : ~0ull;
  __syncthreads();
  block_bitonic_sort(a, Pk, false);
  for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = (int32_t)a[j];
}

// Ascending sort of 64 E values held E per lane (position lane * E + i) by
// one wave: a bitonic network whose strides below E swap registers and the
// others exchange with lane ^ (stride / E) by shuffles; no barrier.
template <int E>
__device__ __forceinline__ void wave_sort_asc(uint32_t (&v)[E], int lane) {
  constexpr int P = 64 * E;
#pragma unroll
  for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      if (stride >= E) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int p = lane * E + i;
          const uint32_t o = (uint32_t)__shfl_xor((int)v[i], stride / E);
          const bool asc = (p & size) == 0, lower = (p & stride) == 0;
          v[i] = asc == lower ? min(v[i], o) : max(v[i], o);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const int j = i ^ stride;
          if (j > i) {
            const bool asc = ((lane * E + i) & size) == 0;
            const uint32_t x = v[i], y = v[j];
            v[i] = asc ? min(x, y) : max(x, y);
            v[j] = asc ? max(x, y) : min(x, y);
          }
        }
      }
    }
  }
}

// emit_topk for k <= 64 E by wave 0 alone (the others return): the keys'
// indices sorted in registers, then written in order.
template <int E>
__device__ __forceinline__ void wave_emit_sorted(const uint64_t* a, int k, int32_t* out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  uint32_t v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = lane * E + i;
    v[i] = p < k ? ckey_idx(a[p]) : 0xFFFFFFFFu;
  }
  wave_sort_asc<E>(v, lane);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int p = lane * E + i;
    if (p < k) out[p] = (int32_t)v[i];
  }
}

// Per landmark row: the J-th largest of its G <= 512 sample-group maxima is
// the candidate threshold tau, the largest one the first softmax offset.
// One wave per row (four rows per workgroup): the maxima, as order-preserving
// keys, sorted in registers.
__global__ __launch_bounds__(256) void k_tau(const float* __restrict__ gmax, float* __restrict__ tau,
                                             float* __restrict__ mhat, int rows, int G, int J) {
  const int lane = threadIdx.x % 64;
  const size_t r = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
  if (r >= (size_t)rows) return;  // wave-uniform; no barrier follows
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = lane * 8 + i;
    v[i] = p < G ? fkey(gmax[r * G + p]) : 0u;  // 0: below every key of a score
  }
  wave_sort_asc<8>(v, lane);
  // position 511 holds the largest, 512 - J the J-th largest
  const int pj = 512 - J;
  uint32_t kj = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i == pj % 8) kj = v[i];
  kj = (uint32_t)__shfl((int)kj, pj / 8);
  const uint32_t kmax = (uint32_t)__shfl((int)v[7], 63);
  if (lane == 0) {
    tau[r] = fkey_inv(kj);
    mhat[r] = fkey_inv(kmax);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_final(const float* __restrict__ vpart, const uint64_t* __restrict__ cand,
                                               const float* __restrict__ rec_sc, const int32_t* __restrict__ rec_st,
                                               const int* __restrict__ rec_cnt, const float* __restrict__ tau,
                                               int32_t* __restrict__ topk, float* __restrict__ vt32,
                                               T* __restrict__ vtT, int* __restrict__ fail, float* __restrict__ lse_lm,
                                               int N, int k, int C, int L, int capg, int s4, int dense, int shared) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* a = (uint64_t*)smem;
  __shared__ float red[256];
  __shared__ float zred[256 / D];
  const size_t r = blockIdx.x;
  const int tid = threadIdx.x;
  constexpr int NG = 256 / D;  // chunk groups
  const float* pr = vpart + r * C * (D + 4);
  if (shared) {
    // shared values (not used by the routing-only variant): largest chunk maximum
    float mx = M0;
    for (int c = tid; c < C; c += 256) mx = fmaxf(mx, pr[(size_t)c * (D + 4)]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    const float Mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    // rescaled sums, chunk groups in parallel (rescaled-sum identity)
    {
      const int e = tid % D, cg = tid / D;
      float zs = 0.f, sv = 0.f;
#pragma unroll 4
      for (int c = cg; c < C; c += NG) {
        const float* q = pr + (size_t)c * (D + 4);
        const float w = __builtin_amdgcn_exp2f(q[0] - Mx);
        zs += q[1] * w;
        sv += q[4 + e] * w;
      }
      red[tid] = sv;
      if (e == 0) zred[cg] = zs;
    }
    __syncthreads();
    if (tid < D) {
      float sv = 0.f, zs = 0.f;
      for (int g = 0; g < NG; ++g) { sv += red[g * D + tid]; zs += zred[g]; }
      const float v = sv / zs;
      // the row's log2-sum-exp, kept for the backward pass when requested
      if (lse_lm && tid == 0) lse_lm[r] = Mx + __builtin_amdgcn_logf(zs);
      vt32[r * D + tid] = v;
      vtT[r * D + tid] = from_f32<T>(v);
    }
  }
  if (dense == 2) return;  // small rows: selected by k_topk_small
  __shared__ int s_over;
  int cnt;
  if (dense) {
    cnt = N;
    const uint64_t* src = cand + r * capg;
    for (int j = tid; j < cnt; j += 256) a[j] = src[j];
  } else {
    // gather the row's candidates from its records: every recorded score
    // >= tau.  The record counts of its (chunk, lane group) segments are
    // staged and prefix-summed in LDS; then each thread takes records
    // tid, tid + 256, ... of the row (its segment found by binary search),
    // and each wave reserves its hits' slots with one LDS atomic.
    int* s_pre = (int*)(a + capg);  // nseg + 1 prefix entries (reused by the selection later)
    __shared__ int s_wt[4], s_fill;
    if (tid == 0) { s_over = 0; s_fill = 0; }
    __syncthreads();
    const int nseg = 4 * C;
    const size_t seg0 = r * (size_t)nseg;
    // per-thread runs of consecutive segments, then a block scan of the run sums
    const int per = (nseg + 255) / 256;
    const int x0 = min(nseg, tid * per), x1 = min(nseg, x0 + per);
    int run = 0, over = 0;
    for (int x = x0; x < x1; ++x) {
      const int n = rec_cnt[seg0 + x];
      over |= n > s4;
      const int c = min(n, s4);
      s_pre[x] = c;
      run += c;
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if ((tid & 63) >= off) incl += y;
    }
    if ((tid & 63) == 63) s_wt[tid >> 6] = incl;
    if (wave_any(over != 0) && (tid & 63) == 0) s_over = 1;
    __syncthreads();
    int acc_ = incl - run;
    for (int w = 0; w < (tid >> 6); ++w) acc_ += s_wt[w];
    for (int x = x0; x < x1; ++x) {
      const int c = s_pre[x];
      s_pre[x] = acc_;
      acc_ += c;
    }
    const int total_rec = s_wt[0] + s_wt[1] + s_wt[2] + s_wt[3];
    if (tid == 0) s_pre[nseg] = total_rec;
    __syncthreads();
    const float tr = tau[r];
    for (int q0 = 0; q0 < total_rec; q0 += 256) {
      const int q = q0 + tid;
      int h = 0;
      float v[8];
      int j0 = 0, lgq = 0;
      if (q < total_rec) {
        // last segment whose start is <= q
        int lo = 0, hi = nseg;  // s_pre[lo] <= q < s_pre[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_pre[mid] <= q) lo = mid; else hi = mid;
        }
        const size_t e = (seg0 + lo) * s4 + (q - s_pre[lo]);
        const float4 a0 = ((const float4*)(rec_sc + e * 8))[0];
        const float4 a1 = ((const float4*)(rec_sc + e * 8))[1];
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
        j0 = (lo >> 2) * L + rec_st[e] * 32;
        lgq = lo & 3;
#pragma unroll
        for (int t = 0; t < 8; ++t) h += v[t] >= tr;
      }
      // wave prefix of the hit counts, one LDS reservation per wave
      int hi_ = h;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(hi_, off);
        if ((tid & 63) >= off) hi_ += y;
      }
      int wbase = 0;
      if ((tid & 63) == 63) wbase = atomicAdd(&s_fill, hi_);
      wbase = __shfl(wbase, 63);
      int pos = wbase + hi_ - h;
      if (h) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (v[t] >= tr) {
            if (pos < capg) a[pos] = ckey(v[t], (uint32_t)(j0 + slot_key(t, lgq)));
            ++pos;
          }
        }
      }
    }
    __syncthreads();
    const int total = s_fill;
    cnt = s_over ? -1 : total;
  }
  if (cnt < k || cnt > capg) {
    if (tid == 0) fail[r] = 1;
    return;
  }
  if (tid == 0) fail[r] = 0;
  __syncthreads();
  // radix select of the k-th largest key, 8 bits a pass; the keys are
  // distinct, so exactly k of them reach the final prefix.  The candidates
  // all lie near the top of the row, so their leading bits (sign, most of
  // the exponent) agree: the passes start at the highest bit where the
  // smallest and the largest key differ (a histogram of identical leading
  // digits would put every count on one LDS address).
  __shared__ int hist[256];
  __shared__ int s_b, s_above, s_in, s_nsel;
  __shared__ uint64_t s_lo[4], s_hi[4];
  {
    uint64_t lo = ~0ull, hi = 0;
    for (int j = tid; j < cnt; j += 256) {
      const uint64_t key = a[j];
      lo = key < lo ? key : lo;
      hi = key > hi ? key : hi;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t ol = __shfl_xor(lo, off), oh = __shfl_xor(hi, off);
      lo = ol < lo ? ol : lo;
      hi = oh > hi ? oh : hi;
    }
    if ((tid & 63) == 0) { s_lo[tid >> 6] = lo; s_hi[tid >> 6] = hi; }
  }
  __syncthreads();
  uint64_t klo = s_lo[0], khi = s_hi[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    klo = s_lo[w] < klo ? s_lo[w] : klo;
    khi = s_hi[w] > khi ? s_hi[w] : khi;
  }
  // bits above hb are the same in every key (cnt >= k >= 1 distinct keys)
  const int hb = klo == khi ? 0 : 63 - __builtin_clzll(klo ^ khi);
  uint64_t mask = hb >= 63 ? 0ull : ~((2ull << hb) - 1ull);
  uint64_t prefix = khi & mask;
  int krem = k;
  // (a digit may also cover known bits above the unknown ones: those are the
  // same in every key still matching the prefix, so the histogram is unchanged)
  for (int shift = hb >= 7 ? hb - 7 : 0;;) {
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < cnt; j += 256) {
      const uint64_t key = a[j];
      if ((key & mask) == prefix) atomicAdd(hist + ((int)(key >> shift) & 255), 1);
    }
    __syncthreads();
    if (tid < 64) {
      // one wave finds the bucket b with S(b) >= krem > S(b + 1), S(b) =
      // keys in buckets >= b: lane l holds buckets 4l..4l+3, suffix sums
      // across lanes by shuffles
      const int h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2], h3 = hist[4 * tid + 3];
      const int own = h0 + h1 + h2 + h3;
      int incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_down(incl, off);
        if (tid + off < 64) incl += v;
      }
      const int s4 = incl - own, s3 = s4 + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
      if (s3 >= krem && s4 < krem) { s_b = 4 * tid + 3; s_above = s4; s_in = h3; }
      if (s2 >= krem && s3 < krem) { s_b = 4 * tid + 2; s_above = s3; s_in = h2; }
      if (s1 >= krem && s2 < krem) { s_b = 4 * tid + 1; s_above = s2; s_in = h1; }
      if (s0 >= krem && s1 < krem) { s_b = 4 * tid; s_above = s1; s_in = h0; }
    }
    __syncthreads();
    prefix |= (uint64_t)s_b << shift;
    mask |= (uint64_t)0xFF << shift;
    krem -= s_above;
    const bool whole = s_in == krem;  // the bucket's keys are all taken
    __syncthreads();
    if (whole || shift == 0) break;  // (after the pass at bit 0 every bit is known)
    shift = shift >= 8 ? shift - 8 : 0;
  }
  uint64_t* sel = a + capg;
  if (tid == 0) s_nsel = 0;
  __syncthreads();
  for (int j = tid; j < cnt; j += 256) {
    const uint64_t key = a[j];
    if ((key & mask) >= prefix) sel[atomicAdd(&s_nsel, 1)] = key;
  }
  __syncthreads();
  // the selected indices in ascending order: one wave sorts up to 512 of
  // them in registers (a block-wide sort pays a barrier per network stage)
  int32_t* out = topk + r * k;
  if (k <= 64) wave_emit_sorted<1>(sel, k, out);
  else if (k <= 128) wave_emit_sorted<2>(sel, k, out);
  else if (k <= 256) wave_emit_sorted<4>(sel, k, out);
  else if (k <= 512) wave_emit_sorted<8>(sel, k, out);
  else emit_topk(sel, k, out);
}

// Exact streaming top-k of one landmark row over all N keys (fp32 dot
// products on the vector units), for rows k_final flagged.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_fallback(const T* __restrict__ K, const T* __restrict__ Qt,
                                                  const int* __restrict__ fail, int32_t* __restrict__ topk,
                                                  int N, int m, int k) {
  const size_t r = blockIdx.x;
  if (fail[r] == 0) return;
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* a = (uint64_t*)smem;
  __shared__ float q[D];
  __shared__ int nb;
  __shared__ uint64_t theta;
  const int tid = threadIdx.x;
  const size_t bh = r / m;
  const T* Kh = K + bh * (size_t)N * D;
  if (tid < D) q[tid] = to_f32<T>(Qt[r * D + tid]);
  if (tid == 0) { nb = 0; theta = 0ull; }
  __syncthreads();
  const int keep = 2 * k;
  for (int j0 = 0; j0 < N; j0 += 256) {
    const int j = j0 + tid;
    if (j < N) {
      const T* kr = Kh + (size_t)j * D;
      float s = 0.f;
      for (int c = 0; c < D; ++c) s = __builtin_fmaf(q[c], to_f32<T>(kr[c]), s);
      const uint64_t key = ckey(s, (uint32_t)j);
      if (key > theta) a[atomicAdd(&nb, 1)] = key;
    }
    __syncthreads();
    const int n = nb;
    if (n > keep) {
      const int P = next_pow2(n);
      for (int i = n + tid; i < P; i += blockDim.x) a[i] = 0ull;
      __syncthreads();
      block_bitonic_sort(a, P, true);
      if (tid == 0) { nb = k; theta = a[k - 1]; }
    }
    __syncthreads();
  }
  const int n = nb;
  const int P = next_pow2(n < 2 ? 2 : n);
  for (int i = n + tid; i < P; i += blockDim.x) a[i] = 0ull;
  __syncthreads();
  block_bitonic_sort(a, P, true);
  emit_topk(a, k, topk + r * k);
}


// ---------------------------------------------------------------------------
// small rows (N <= SMALL_N, k <= SMALL_K): top-k selected on chip
// ---------------------------------------------------------------------------
// One workgroup of sixteen waves per (head, 16 landmark rows).  The waves
// score the 16 rows against all N keys on the matrix cores (wave w takes the
// 32-key steps w, w + 16, ...; each key row is used by one wave only, so its
// operand fragments are read straight from global memory, one step ahead)
// into an LDS tile of raw fp32 scores; then each wave finishes one row with
// no barrier: a search for the k-th largest order-preserving score key (one
// bit a pass from the top, each pass counting the keys at or above a
// candidate value with one ballot per register of the row's keys; it stops
// as soon as exactly k keys lie at or above the known leading bits), one
// pass over the keys in index order that emits every key
// above that value and, among the keys equal to it, the lowest indices, in
// ascending order; and the merge of the row's shared-value partials (the
// rescaled-sum identity of tutorial ch.4, one output dimension per lane).
// Neither the scores nor candidate keys reach HBM.
// Wave-level selection helpers of k_topk_small.  A lane holds NU keys
// (register u: key index lane + 64 u of the set); nu of them are in use.
// Number of keys of the wave that are >= t (t >= 1: unused slots hold 0).
template <int NU>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&kk)[NU], int nu, uint32_t t) {
  int c = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (u < nu) c += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(kk[u] >= t));
  return c;
}
// Bitwise search for the k-th largest key T from bit `bit` down: on entry
// and exit, cge keys are >= prefix and every key that can reach the top k is
// >= prefix.  Stops when exactly k keys are >= prefix (they are the top k),
// when the bits run out (prefix = T), or once at most `stop` keys remain.
template <int NU>
__device__ __forceinline__ void wave_bit_search(const uint32_t (&kk)[NU], int nu, int k, int stop, int& bit,
                                                uint32_t& prefix, int& cge) {
  for (; bit >= 0 && cge != k && cge > stop; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int c = wave_count_ge(kk, nu, cand);
    if (c >= k) { prefix = cand; cge = c; }
  }
}
// Writes the top k in ascending index order: every key above T, then the
// first keys equal to T (by index) until k are taken; with exact (exactly k
// keys >= prefix) the keys >= prefix.  idx(u): this lane's key index in
// register u, or -1 for an unused slot; the set is in ascending index order
// (register-major, then lane).
template <int NU, class Idx>
__device__ __forceinline__ void wave_emit_topk(const uint32_t (&kk)[NU], int nu, int k, bool exact, uint32_t prefix,
                                               int cge, Idx idx, int32_t* out) {
  const int ngt = exact ? k : wave_count_ge(kk, nu, prefix + 1u);
  const int krem = k - ngt;
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u < nu) {
      const int j = idx(u);
      const bool valid = j >= 0;
      const bool gt = valid && (exact ? kk[u] >= prefix : kk[u] > prefix);
      const bool eq = valid && !exact && kk[u] == prefix;
      const uint64_t be = __builtin_amdgcn_ballot_w64(eq);
      const int er = eq_seen + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
      const bool take = gt || (eq && er < krem);
      const uint64_t bt = __builtin_amdgcn_ballot_w64(take);
      const int o = pos + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      if (take && o < k) out[o] = j;  // (exactly k are taken; the bound only guards memory)
      pos += (int)__builtin_popcountll(bt);
      eq_seen += (int)__builtin_popcountll(be);
    }
  }
}

// UMAX: keys per lane (N <= 64 UMAX); the kernel is compiled for 4, 8, 16
// and 32 so the per-key loops are unrolled to the row's length.
template <typename T, int D, int UMAX>
__global__ __launch_bounds__(1024, UMAX <= 8 ? 2 : 1) void k_topk_small(const T* __restrict__ K, const T* __restrict__ Qt,
                                                    const float* __restrict__ vpart, int32_t* __restrict__ topk,
                                                    float* __restrict__ vt32, T* __restrict__ vtT,
                                                    float* __restrict__ lse_lm, int N, int m, int k, int C,
                                                    int stride, int shared) {
  constexpr bool COMPACT = UMAX > 4;  // (the compaction area needs a row stride >= 256)
  extern __shared__ __align__(16) unsigned char smem[];
  float* S = (float*)smem;  // [16][stride] raw scores
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int bh = blockIdx.y, r0 = blockIdx.x * 16;
  const T* Kh = K + (size_t)bh * N * D;
  Frag<T> qf[D / 32];
  {
    const int row = r0 + li;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (row < m) load8(qf[dc], Qt + ((size_t)bh * m + row) * D + dc * 32 + 8 * lg);
      else zero(qf[dc]);
    }
  }
  // this wave's row: its first shared-value chunk partials are fetched now,
  // so their latency hides under the scoring and the selection (fewer for
  // short rows, whose workgroups run two to a compute unit on half the
  // registers)
  constexpr int CPRE = UMAX <= 8 ? 2 : 8;
  const size_t rw = (size_t)bh * m + min(r0 + wave, m - 1);
  const float* prw = vpart + rw * C * (D + 4);
  const int ew = lane < D ? lane : 0;
  float pq0[CPRE], pq1[CPRE], pqv[CPRE];
  if (shared) {
#pragma unroll
    for (int u = 0; u < CPRE; ++u) {
      const float* q = prw + (size_t)min(u, C - 1) * (D + 4);
      pq0[u] = q[0];
      pq1[u] = q[1];
      pqv[u] = q[4 + ew];
    }
  }
  const int nsteps = (N + 31) / 32;
  auto load_step = [&](StepFrags<T, D>& f, int st) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int j = st * 32 + jt * 16 + li;
#pragma unroll
      for (int dc = 0; dc < D / 32; ++dc) {
        if (j < N) load8(f.ka[jt][dc], Kh + (size_t)j * D + dc * 32 + 8 * lg);
        else zero(f.ka[jt][dc]);
      }
    }
  };
  // (rows of up to 512 keys: at most one step per wave, nothing to prefetch)
  constexpr bool PF = UMAX > 8;
  StepFrags<T, D> fn;
  if (PF && wave < nsteps) load_step(fn, wave);
  for (int st = wave; st < nsteps; st += 16) {
    StepFrags<T, D> f;
    if constexpr (PF) {
      f = fn;
      if (st + 16 < nsteps) load_step(fn, st + 16);
    } else {
      load_step(f, st);
    }
    float sc[8];
    step_scores(f, qf, sc);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int j = st * 32 + slot_key(t, lg);
      if (j < N) S[li * stride + j] = sc[t];
    }
  }
  __syncthreads();
  const int U = (N + 63) / 64;
  {
    const int rl = wave, row = r0 + rl;
    if (row >= m) return;  // wave-uniform; no barrier follows
    const float* Sr = S + rl * stride;
    const size_t r = (size_t)bh * m + row;
    uint32_t kf[UMAX];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const int j = lane + 64 * u;
      kf[u] = (u < U && j < N) ? fkey(Sr[j]) : 0u;  // 0: below every key of a score (the smallest is -inf's)
    }
    // the k-th largest key value T, one bit a pass from the top (counts are
    // ballots over the lane registers).  With more than four keys per lane,
    // once at most 128 keys can still reach the top k (those >= the bits
    // found so far) they are moved, in index order, to two registers per
    // lane through this row's LDS scores (no longer needed), and the search
    // and the emission continue on those.
    int32_t* out = topk + r * k;
    uint32_t prefix = 0;
    int cge = N;  // keys >= 0: every key of the row (unused slots hold 0)
    int bit = 31;
    wave_bit_search(kf, U, k, COMPACT ? 128 : -1, bit, prefix, cge);
    if (COMPACT && cge != k && bit >= 0) {
      uint32_t* kb = (uint32_t*)(S + rl * stride);  // cge <= 128 keys, then their indices
      int* ib = (int*)(kb + 128);
      int base = 0;
#pragma unroll
      for (int u = 0; u < UMAX; ++u) {
        if (u < U) {
          const int j = lane + 64 * u;
          const bool sel = j < N && kf[u] >= prefix;
          const uint64_t bs = __builtin_amdgcn_ballot_w64(sel);
          const int o = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0u));
          if (sel) { kb[o] = kf[u]; ib[o] = j; }
          base += (int)__builtin_popcountll(bs);
        }
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t kc[2];
      int ic[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int x = lane + 64 * v;
        kc[v] = x < base ? kb[x] : 0u;
        ic[v] = x < base ? ib[x] : -1;
      }
      wave_bit_search(kc, 2, k, -1, bit, prefix, cge);
      wave_emit_topk(kc, 2, k, cge == k, prefix, cge, [&](int v) { return ic[v]; }, out);
    } else {
      wave_emit_topk(kf, U, k, cge == k, prefix, cge,
                     [&](int u) { const int j = lane + 64 * u; return j < N ? j : -1; }, out);
    }
    // shared value of the row: merge its C chunk partials (lane e owns
    // output dim e); every load of a batch is in flight at once
    if (shared) {
      const float* pr = vpart + r * C * (D + 4);
      float mx = M0;
#pragma unroll
      for (int u = 0; u < CPRE; ++u)
        if (u < C) mx = fmaxf(mx, pq0[u]);
      if (C > CPRE) {
        for (int c = CPRE + lane; c < C; c += 64) mx = fmaxf(mx, pr[(size_t)c * (D + 4)]);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      }
      float zs = 0.f, sv = 0.f;
#pragma unroll
      for (int u = 0; u < CPRE; ++u) {
        if (u < C) {
          const float w = __builtin_amdgcn_exp2f(pq0[u] - mx);
          zs += pq1[u] * w;
          sv += pqv[u] * w;
        }
      }
      for (int c0 = CPRE; c0 < C; c0 += 8) {
        float q0[8], q1[8], qv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = min(c0 + u, C - 1);
          const float* q = pr + (size_t)c * (D + 4);
          q0[u] = q[0];
          q1[u] = q[1];
          qv[u] = q[4 + ew];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (c0 + u < C) {
            const float w = __builtin_amdgcn_exp2f(q0[u] - mx);
            zs += q1[u] * w;
            sv += qv[u] * w;
          }
        }
      }
      if (lane < D) {
        const float v = sv / zs;
        vt32[r * D + lane] = v;
        vtT[r * D + lane] = from_f32<T>(v);
      }
      if (lse_lm && lane == 0) lse_lm[r] = mx + __builtin_amdgcn_logf(zs);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int IB>
static void launch_score_t(const Plan& p) {
  using TL = TileLayout<T, D>;
  constexpr int R = NW * 16 * IB;
  const bool dense = p.dense != 0;
  if (!dense && p.force_fallback) {
    const int n = p.BH * p.m;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, p.stream, p.tau, n, INFINITY);
  } else if (!dense) {
    dim3 grid((unsigned)((p.G + p.est_gpb - 1) / p.est_gpb), (unsigned)p.sc_rt, (unsigned)p.BH);
    hipLaunchKernelGGL((k_est<T, D, NW, IB>), grid, dim3(NW * 64), 0, p.stream, (const T*)p.K, (const T*)p.qt,
                       p.gmax, p.N, p.m, p.sigma, p.NS, p.G, p.est_gpb);
    const int rows = p.BH * p.m;
    hipLaunchKernelGGL(k_tau, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, p.stream, p.gmax, p.tau, p.mhat, rows, p.G,
                       p.J);
  }
}

template <typename T, int D, int NW, int IB, bool SHARED>
static void launch_score_s(const Plan& p) {
  using TL = TileLayout<T, D>;
  constexpr int R = NW * 16 * IB;
  const bool dense = p.dense != 0;
  const size_t lds = 2 * TL::ELEMS * sizeof(T);
  dim3 grid((unsigned)p.C, (unsigned)p.sc_rt, (unsigned)p.BH);
  if (dense && p.small) {
    hipLaunchKernelGGL((k_score<T, D, NW, IB, SEL_NONE, SHARED>), grid, dim3(NW * 64), lds, p.stream, (const T*)p.K,
                       (const T*)p.V, (const T*)p.qt, nullptr, nullptr, p.vpart, nullptr, nullptr, nullptr, nullptr,
                       p.N, p.m, p.L, p.C, 0, 0, p.cscale);
    return;
  }
  if (dense) {
    hipLaunchKernelGGL((k_score<T, D, NW, IB, SEL_DENSE, SHARED>), grid, dim3(NW * 64), lds, p.stream, (const T*)p.K,
                       (const T*)p.V, (const T*)p.qt, nullptr, nullptr, p.vpart, p.cand, nullptr, nullptr, nullptr,
                       p.N, p.m, p.L, p.C, p.capg, 0, p.cscale);
    return;
  }
  hipLaunchKernelGGL((k_score<T, D, NW, IB, SEL_SPARSE, SHARED>), grid, dim3(NW * 64), lds, p.stream, (const T*)p.K,
                     (const T*)p.V, (const T*)p.qt, p.tau, p.force_fallback ? nullptr : p.mhat, p.vpart, nullptr,
                     p.rec_sc, p.rec_st, p.rec_cnt, p.N, p.m, p.L, p.C, p.capg, p.s4, p.cscale);
}

template <typename T, int D, int NW, int IB>
static void launch_score_main(const Plan& p) {
  if (p.shared) launch_score_s<T, D, NW, IB, true>(p);
  else launch_score_s<T, D, NW, IB, false>(p);
}

template <typename T, int D>
static void launch_final_t(const Plan& p) {
  if (p.small) {
    // top-k and the shared-value merge on chip; k_final is not needed
    const int stride = (p.N + 63) / 64 * 64 + 1;
    const size_t lds2 = (size_t)16 * stride * 4;
    auto go = [&](auto fn) {
      if (lds2 > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds2);
      hipLaunchKernelGGL(fn, dim3((unsigned)((p.m + 15) / 16), (unsigned)p.BH), dim3(1024), lds2, p.stream,
                         (const T*)p.K, (const T*)p.qt, p.vpart, p.topk, p.vt32, (T*)p.vtT, p.lse_lm, p.N, p.m, p.k,
                         p.C, stride, p.shared);
    };
    if (p.N <= 256) go(&k_topk_small<T, D, 4>);
    else if (p.N <= 512) go(&k_topk_small<T, D, 8>);
    else if (p.N <= 1024) go(&k_topk_small<T, D, 16>);
    else go(&k_topk_small<T, D, SMALL_N / 64>);
    return;
  }
  // candidates, then the selected keys (or, before the selection, the
  // per-segment record counts of a sparse row)
  const size_t sel = (size_t)next_pow2(p.k < 2 ? 2 : p.k) * 8;
  const size_t lds = p.small ? 0 : (size_t)p.capg * 8 + (p.dense ? sel : std::max(sel, ((size_t)4 * p.C + 1) * 4));
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_final<T, D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  hipLaunchKernelGGL((k_final<T, D>), dim3((unsigned)(p.BH * p.m)), dim3(256), lds, p.stream, p.vpart, p.cand,
                     p.rec_sc, p.rec_st, p.rec_cnt, p.tau, p.topk, p.vt32, (T*)p.vtT, p.fail, p.lse_lm, p.N, p.k,
                     p.C, p.L, p.capg, p.s4, p.small ? 2 : p.dense, p.shared);
  if (!p.dense) {
    const size_t lds2 = (size_t)next_pow2(2 * p.k + 256) * 8;
    hipLaunchKernelGGL((k_fallback<T, D>), dim3((unsigned)(p.BH * p.m)), dim3(256), lds2, p.stream,
                       (const T*)p.K, (const T*)p.qt, p.fail, p.topk, p.N, p.m, p.k);
  }
}

#define MITA_SCORE_DISPATCH(FN)                                                     \
  do {                                                                              \
    if (p.dtype == 0) {                                                             \
      if (p.d == 32) FN<float, 32, 4, 1>(p); else FN<float, 64, 4, 1>(p);           \
    } else if (p.d == 32) {                                                         \
      if (p.sc_nw == 4) FN<__bf16, 32, 4, 1>(p);                                    \
      else if (p.sc_ib == 1) FN<__bf16, 32, 8, 1>(p);                               \
      else if (p.sc_ib == 2) FN<__bf16, 32, 8, 2>(p);                               \
      else FN<__bf16, 32, 8, 4>(p);                                                 \
    } else {                                                                        \
      if (p.sc_nw == 4) FN<__bf16, 64, 4, 1>(p);                                    \
      else if (p.sc_ib == 1) FN<__bf16, 64, 8, 1>(p);                               \
      else if (p.sc_ib == 2) FN<__bf16, 64, 8, 2>(p);                               \
      else FN<__bf16, 64, 8, 4>(p);                                                 \
    }                                                                               \
  } while (0)

void launch_estimate(const Plan& p) { MITA_SCORE_DISPATCH(launch_score_t); }
void launch_score(const Plan& p) { MITA_SCORE_DISPATCH(launch_score_main); }
void launch_final(const Plan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_final_t<float, 32>(p); else launch_final_t<float, 64>(p);
  } else {
    if (p.d == 32) launch_final_t<__bf16, 32>(p); else launch_final_t<__bf16, 64>(p);
  }
}

}  // namespace mita
