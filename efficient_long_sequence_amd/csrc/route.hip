// Step 5 of MiTA: route every query to its top-s landmarks by q . q~_i
// (MiTA tutorial (iwxt.cn), ch.4 step 4, paper section 3.2: the score only
// selects experts, no gate mixes them), then group the queries by chosen
// expert so the attention kernel can stage each expert's keys once for all of
// its queries (the grouping the bit.fan article describes for the authors'
// Algorithm 1; here a counting sort on the device with no host round trip).
//
//   k_route   one workgroup per (head, 64*NW queries): Q Q~^T on the matrix
//             cores, landmarks streamed through LDS 32 at a time; each lane
//             keeps a sorted top-s list for its query (ties to the lower
//             landmark, which arrives first), the four lane groups of a query
//             are merged at the end; a per-workgroup histogram of the chosen
//             experts is added to the global per-(slot, head, expert) counts.
//   k_scan    one workgroup: exclusive prefix of the counts (the start of each
//             expert's bucket) and the work list of (expert, query tile)
//             items, per slot.
//   k_scatter writes each query into its expert's bucket (order inside a
//             bucket is immaterial: every query's output depends only on its
//             own row); per-workgroup LDS counts, one global reservation per
//             expert present in the workgroup.
#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

struct Cand {
  float v;
  int i;
};
__device__ __forceinline__ bool better(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Insert (v, i) into a list sorted by `better`, keeping its first S entries.
template <int S>
__device__ __forceinline__ void insert_full(float* lv, int* li, float v, int i) {
#pragma unroll
  for (int t = S - 1; t >= 0; --t) {
    const bool above = (t > 0) && better(v, i, lv[t - 1], li[t - 1]);
    const bool here = better(v, i, lv[t], li[t]);
    if (above) { lv[t] = lv[t - 1]; li[t] = li[t - 1]; }
    else if (here) { lv[t] = v; li[t] = i; }
  }
}

template <typename T, int D, int NW, int SMAX>
__global__ __launch_bounds__(NW * 64) void k_route(const T* __restrict__ Q, const T* __restrict__ Qt,
                                                   int32_t* __restrict__ route, int* __restrict__ counts,
                                                   int N, int m, int s, int BH, int hist_lds) {
  constexpr int NT = NW * 64;
  using TL = TileLayout<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  T* buf0 = (T*)smem;
  T* buf1 = buf0 + TL::K_ELEMS;
  int* hist = (int*)(buf1 + TL::K_ELEMS);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int bh = blockIdx.y;
  const int qbase = blockIdx.x * (NW * 64) + wave * 64;
  const T* Qh = Q + (size_t)bh * N * D;
  const T* Qth = Qt + (size_t)bh * m * D;

  if (hist_lds)
    for (int x = tid; x < s * m; x += NT) hist[x] = 0;

  Frag<T> qf[4][D / 32];
  float lv[4][SMAX];
  int lx[4][SMAX];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = qbase + b * 16 + li;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (n < N) load8(qf[b][dc], Qh + (size_t)n * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
#pragma unroll
    for (int t = 0; t < SMAX; ++t) { lv[b][t] = -INFINITY; lx[b][t] = 0x7FFFFFFF; }
  }

  TileLoader<T, D, NT, false> ld;
  auto rowL = [&](int i0) {
    return [=](int r) -> const T* { const int i = i0 + r; return i < m ? Qth + (size_t)i * D : nullptr; };
  };
  auto none = [](int) -> const T* { return nullptr; };
  const int nsteps = (m + 31) / 32;
  ld.load(rowL(0), none);
  ld.store(buf0, nullptr);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int i0 = st * 32;
    T* cur = (st & 1) ? buf1 : buf0;
    T* nxt = (st & 1) ? buf0 : buf1;
    const bool more = st + 1 < nsteps;
    if (more) ld.load(rowL(i0 + 32), none);
    StepFrags<T, D> f;
    f.load_keys(cur, li, lg);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float sc[8];
      step_scores(f, qf[b], sc);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = i0 + slot_key(t, lg);
        // within a lane landmarks arrive in increasing order: strict '>'
        // keeps the lower index on ties
        if (i < m && sc[t] > lv[b][SMAX - 1]) insert_full<SMAX>(lv[b], lx[b], sc[t], i);
      }
    }
    if (more) ld.store(nxt, nullptr);
    __syncthreads();
  }

  // merge the four lane groups of each query
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int sh = 16; sh <= 32; sh <<= 1) {
      float ov[SMAX];
      int ox[SMAX];
#pragma unroll
      for (int t = 0; t < SMAX; ++t) { ov[t] = __shfl_xor(lv[b][t], sh); ox[t] = __shfl_xor(lx[b][t], sh); }
#pragma unroll
      for (int t = 0; t < SMAX; ++t) insert_full<SMAX>(lv[b], lx[b], ov[t], ox[t]);
    }
    const int n = qbase + b * 16 + li;
    if (lg == 0 && n < N) {
      int32_t* dst = route + ((size_t)bh * N + n) * s;
#pragma unroll
      for (int t = 0; t < SMAX; ++t) {
        if (t < s) {
          // a valid list always holds s landmarks; the clamp only keeps
          // non-finite inputs (unspecified results) inside the buffers
          const int e = min(max(lx[b][t], 0), m - 1);
          dst[t] = e;
          if (hist_lds) atomicAdd(hist + t * m + e, 1);
          else atomicAdd(counts + ((size_t)t * BH + bh) * m + e, 1);
        }
      }
    }
  }
  if (hist_lds) {
    __syncthreads();
    for (int x = tid; x < s * m; x += NT) {
      const int c = hist[x];
      if (c) atomicAdd(counts + ((size_t)(x / m) * BH + bh) * m + (x % m), c);
    }
  }
}

// Exclusive prefix of the expert counts and the work list, for every slot.
// One workgroup of 1024 threads; each thread owns a contiguous segment.
// Optionally (efirst, epart not null) records where each expert's items
// went: its full items at efirst .. efirst + count / T - 1 and its partial
// item at epart (-1 if none).
// Work list order: first every item of a full T queries (experts in index
// order, so an expert's items stay adjacent), then each expert's partial
// item, larger ones first (a counting sort on the number of 16-query
// blocks), so the longest items start first and the short ones fill the tail.
constexpr int SCAN_BUCKETS = 128;  // T <= 2048 queries per item

// atomicAdd(&base[b], 1) for every lane with b >= 0.  When all of a
// wave's lanes that add use one b (small experts all fall in the first size
// bucket), the wave makes a single LDS atomic and hands out the slots by
// rank; otherwise each lane adds on its own.  Returns the lane's slot, or -1
// for b < 0.
__device__ __forceinline__ int wave_bucket_add(int* base, int b) {
  const uint64_t act = __builtin_amdgcn_ballot_w64(b >= 0);
  if (!act) return -1;
  const int lane = threadIdx.x % 64;
  const int first = (int)__builtin_ctzll(act);
  const int b0 = __shfl(b, first);
  const uint64_t same = __builtin_amdgcn_ballot_w64(b == b0) & act;
  if (same == act) {
    int old = 0;
    if (lane == first) old = atomicAdd(base + b0, (int)__builtin_popcountll(act));
    old = __shfl(old, first);
    return b >= 0 ? old + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0u))
                  : -1;
  }
  return b >= 0 ? atomicAdd(base + b, 1) : -1;
}

// Counts staged in LDS per slot (read coalesced, then each thread walks its
// contiguous segment there); above this many experts they are read from
// global memory directly.
constexpr int SCAN_STAGE = 8192;

__global__ __launch_bounds__(1024) void k_scan(const int* __restrict__ counts, int* __restrict__ gpre,
                                               WorkItem* __restrict__ wl, int* __restrict__ wl_count,
                                               int E, int m, int s, int T, int UB, int* __restrict__ efirst,
                                               int* __restrict__ epart) {
  __shared__ int sn[32], stl[32];  // wave totals, then exclusive wave offsets
  __shared__ int bcnt[SCAN_BUCKETS];
  __shared__ int cst[SCAN_STAGE];
  const int tid = threadIdx.x;
  const int seg = (E + 1023) / 1024;
  const int lo = min(E, tid * seg), hi = min(E, lo + seg);
  auto bucket = [&](int rem) { return min(SCAN_BUCKETS - 1, (rem + 15) / 16 - 1); };
  const bool staged = E <= SCAN_STAGE;
  for (int t = 0; t < s; ++t) {
    const int* cg = counts + (size_t)t * E;
    if (staged) {
      for (int x0 = tid; x0 < E; x0 += 8 * 1024) {  // eight loads in flight per thread
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = x0 + u * 1024 < E ? cg[x0 + u * 1024] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (x0 + u * 1024 < E) cst[x0 + u * 1024] = v[u];
      }
    }
    const int* c = staged ? cst : cg;
    if (tid < SCAN_BUCKETS) bcnt[tid] = 0;
    __syncthreads();
    int n_sum = 0, t_sum = 0;
    // (every thread runs the same trip count, so the wave-wide counting
    // below sees all its lanes)
    for (int i = 0; i < seg; ++i) {
      const int x = lo + i;
      const int n = x < hi ? c[x] : 0;
      n_sum += n;
      t_sum += n / T;
      wave_bucket_add(bcnt, n % T ? bucket(n % T) : -1);
    }
    // inclusive scan of the segment totals: within each wave by shuffles,
    // then over the 16 wave totals
    const int lane = tid % 64, wv = tid / 64;
    int in_n = n_sum, in_t = t_sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int yn = __shfl_up(in_n, off), yt = __shfl_up(in_t, off);
      if (lane >= off) { in_n += yn; in_t += yt; }
    }
    if (lane == 63) { sn[wv] = in_n; stl[wv] = in_t; }
    __syncthreads();
    if (wv == 0) {
      // wave totals -> exclusive wave offsets (lanes 0..15)
      int wn = lane < 16 ? sn[lane] : 0, wt = lane < 16 ? stl[lane] : 0;
      const int own_n = wn, own_t = wt;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int yn = __shfl_up(wn, off), yt = __shfl_up(wt, off);
        if (lane >= off) { wn += yn; wt += yt; }
      }
      const int nfull = __shfl(wt, 15);
      // partial items: bucket starts, largest bucket first; lane l holds
      // buckets 127 - 2l and 126 - 2l
      const int bh_ = SCAN_BUCKETS - 1 - 2 * lane, bl_ = bh_ - 1;
      const int ch = bcnt[bh_], cl = bcnt[bl_];
      int inc = ch + cl;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      const int start = nfull + inc - (ch + cl);
      bcnt[bh_] = start;
      bcnt[bl_] = start + ch;
      if (lane == 63) wl_count[t] = nfull + inc;
      if (lane < 16) { sn[lane + 16] = wn - own_n; stl[lane + 16] = wt - own_t; }
    }
    __syncthreads();
    int nb = in_n - n_sum + sn[16 + wv], tb = in_t - t_sum + stl[16 + wv];
    WorkItem* w = wl + (size_t)t * UB;
    for (int i = 0; i < seg; ++i) {
      const int x = lo + i;
      const bool in = x < hi;
      const int n = in ? c[x] : 0;
      const int nf = n / T;
      if (in) {
        gpre[(size_t)t * E + x] = nb;
        if (efirst) efirst[(size_t)t * E + x] = tb;
        for (int q = 0; q < nf; ++q) w[tb++] = WorkItem{nb + q * T, T, x, 0};
      }
      const int pi = wave_bucket_add(bcnt, in && n % T ? bucket(n % T) : -1);
      if (pi >= 0) w[pi] = WorkItem{nb + nf * T, n % T, x, 0};
      if (in && epart) epart[(size_t)t * E + x] = pi;
      nb += n;
    }
    __syncthreads();
  }
}

// Each workgroup counts its SC_QPW queries per expert in LDS, reserves one
// contiguous range per expert with a single global atomic, and writes the
// queries there (queries that share an expert in a block cost one atomic).
constexpr int SC_QPT = 8;              // queries per thread
constexpr int SC_QPW = 256 * SC_QPT;   // queries per workgroup

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ route, const int* __restrict__ gpre,
                                                 int* __restrict__ cursor, int32_t* __restrict__ perm, int N,
                                                 int m, int s, int BH) {
  extern __shared__ int s_cnt[];  // [m] counts, then [m] bases
  int* s_base = s_cnt + m;
  const int bh = blockIdx.y;
  const int n0 = blockIdx.x * SC_QPW + threadIdx.x;
  for (int t = 0; t < s; ++t) {
    for (int x = threadIdx.x; x < m; x += 256) s_cnt[x] = 0;
    __syncthreads();
    int e[SC_QPT], r[SC_QPT];
#pragma unroll
    for (int u = 0; u < SC_QPT; ++u) {
      const int n = n0 + u * 256;
      e[u] = n < N ? route[((size_t)bh * N + n) * s + t] : -1;
      r[u] = e[u] >= 0 ? atomicAdd(s_cnt + e[u], 1) : 0;
    }
    __syncthreads();
    const size_t xb = ((size_t)t * BH + bh) * m;
    for (int x = threadIdx.x; x < m; x += 256) {
      const int c = s_cnt[x];
      if (c) s_base[x] = gpre[xb + x] + atomicAdd(cursor + xb + x, c);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < SC_QPT; ++u)
      if (e[u] >= 0) perm[(size_t)t * BH * N + s_base[e[u]] + r[u]] = n0 + u * 256;
    __syncthreads();
  }
}

template <typename T, int D, int SMAX>
static void launch_route_t(const Plan& p) {
  using TL = TileLayout<T, D>;
  constexpr int NW = 4;
  const int hist_lds = (p.s * p.m <= 16384) ? 1 : 0;
  const size_t lds = 2 * TL::K_ELEMS * sizeof(T) + (hist_lds ? (size_t)p.s * p.m * 4 : 0);
  dim3 grid((unsigned)((p.N + NW * 64 - 1) / (NW * 64)), (unsigned)p.BH);
  hipLaunchKernelGGL((k_route<T, D, NW, SMAX>), grid, dim3(NW * 64), lds, p.stream, (const T*)p.Q,
                     (const T*)p.qt, p.route, p.counts, p.N, p.m, p.s, p.BH, hist_lds);
}

template <typename T, int D>
static void launch_route_s(const Plan& p) {
  switch (p.smax) {
    case 1: launch_route_t<T, D, 1>(p); break;
    case 2: launch_route_t<T, D, 2>(p); break;
    case 4: launch_route_t<T, D, 4>(p); break;
    default: launch_route_t<T, D, 8>(p); break;
  }
}

void launch_route(const Plan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_route_s<float, 32>(p); else launch_route_s<float, 64>(p);
  } else {
    if (p.d == 32) launch_route_s<__bf16, 32>(p); else launch_route_s<__bf16, 64>(p);
  }
}

void launch_bucket(const Plan& p) {
  const int E = p.BH * p.m;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, p.stream, p.counts, p.gpre, p.wl, p.wl_count, E, p.m, p.s,
                     p.T, p.UB, (int*)nullptr, (int*)nullptr);
  dim3 grid((unsigned)((p.N + SC_QPW - 1) / SC_QPW), (unsigned)p.BH);
  hipLaunchKernelGGL(k_scatter, grid, dim3(256), (size_t)2 * p.m * sizeof(int), p.stream, p.route, p.gpre, p.cursor,
                     p.perm, p.N, p.m, p.s, p.BH);
}

}  // namespace mita

namespace mita {
void launch_items(const Plan& p, int T, int UB, WorkItem* wl, int* wl_count, int* efirst, int* epart) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, p.stream, p.counts, p.gpre, wl, wl_count, p.BH * p.m, p.m,
                     p.s, T, UB, efirst, epart);
}
}  // namespace mita
