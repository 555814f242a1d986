// Backward pass of MiTA: dQ, dK and dV of sum(O * dO).
//
// What is differentiated is the forward of MiTA tutorial (iwxt.cn) ch.4
// (steps 1-6) as trained end to end (ch.7, LRA training).  The top-k keys of
// each landmark and the top-s landmarks of each query are choices, constant
// wherever they are unique, so they pass no gradient and are taken from the
// forward (its saved experts and routes); q~'s rounding to the input dtype is
// taken as the identity, so pooling's adjoint spreads d q~_i / |W_i| over the
// tokens of window W_i.
//
// Every softmax here is already finished: the forward kept each one's
// log2-sum-exp L, so a probability is exp2(score * cscale - L) with no
// running maximum.  The gradient of a softmax entry t is
// dS_t = P_t (dP_t - delta), with dP_t = g . w_t (g the upstream gradient of
// the softmax's output, w_t the entry's value) and delta = g . output; the
// matrix-core product that forms dP_t starts from -delta instead of zero, so
// it yields dP_t - delta directly.
//
// One step shape serves every pass: a workgroup keeps 16*IB*NW "stationary"
// rows in registers (matrix-core columns) and streams 32 "entries" at a time
// through double-buffered LDS.  Per step it forms S = X.Y and dP = W.Z (X, W
// the rows' two vectors; Y, Z the entries'), then P and dS, and accumulates
// dX += c dS Y and, when asked, dW += P Z, with c the logit scale.  The entry
// vectors are needed in two orders, row-major (operands of S and dP) and
// transposed (operands of the accumulations): bf16 tiles are staged once,
// row-major, and read transposed through the LDS transpose read; fp32 tiles
// are staged twice.  The slot permutation of the forward's layout cancels in
// every contraction.  The passes:
//
//   joint softmax, landmark rows over all queries    X q~, W v~,  Y q,  Z dO   -> dq~, dv~  (chunk partials)
//   joint softmax, expert key rows over its queries  X k,  W v,   Y q,  Z dO   -> dk, dv    (per expert row)
//   shared values, key rows over all landmarks       X k,  W v,   Y q~, Z dv~  -> dk, dv    (+ the above, final)
//
// A key can sit in several experts; its routed parts are gathered by the
// key's owner through the inverse of the expert lists (a counting sort), so
// every output row has exactly one writer and no atomics touch HBM.
//   shared values, landmark rows over all keys       X q~, W dv~, Y k,  Z v    -> dq~       (chunk partials)
//   joint softmax, query rows over [q~; expert keys] X q,  W dO,  Y,    Z      -> dq        (+ pooling's adjoint)
//
// In the shared-value softmax the stationary-landmark pass takes L and delta
// per row; every other pass takes them per entry (each entry is a query or a
// landmark row whose softmax it belongs to).
#include <cmath>

#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

// LDS of one step: Y (row-major + transposed), Z (likewise), then L and
// -delta of the 32 entries.
template <typename T, int D>
struct GradLds {
  using TL = TileLayout<T, D>;
  // bf16: one row-major tile per vector (both operand orders are read from
  // it, the transposed one with tr_frag); fp32: rows and a transposed copy
  static constexpr bool ROWS = sizeof(T) == 2;
  static constexpr size_t TILE_BYTES = (size_t)(ROWS ? TL::K_ELEMS : TL::ELEMS) * sizeof(T);
  static constexpr size_t STEP_BYTES = 2 * TILE_BYTES + 64 * sizeof(float);
  static_assert(TILE_BYTES % 16 == 0, "tiles must stay 16-byte aligned");
  __device__ static T* y(unsigned char* b) { return (T*)b; }
  __device__ static T* z(unsigned char* b) { return (T*)(b + TILE_BYTES); }
  __device__ static float* ent(unsigned char* b) { return (float*)(b + 2 * TILE_BYTES); }
};

template <typename T, int D, int NT, bool WANT_W, bool ENT>
struct GradLoader {
  using GL = GradLds<T, D>;
  using TL = TileLayout<T, D>;
  static constexpr bool TWO = !GL::ROWS;  // stage a transposed copy too (fp32)
  TileLoader<T, D, NT, TWO> ly;
  TileLoader<T, D, NT, TWO && WANT_W> lz;
  float2 e;
  template <class RY, class RZ, class RE>
  __device__ __forceinline__ void load(RY ry, RZ rz, RE re) {
    ly.load(ry, ry);
    lz.load(rz, rz);
    if constexpr (ENT) {
      if (threadIdx.x < 32) e = re((int)threadIdx.x);
    }
  }
  __device__ __forceinline__ void store(unsigned char* b) const {
    T* y = GL::y(b);
    T* z = GL::z(b);
    ly.store(y, y + TL::K_ELEMS);
    lz.store(z, z + TL::K_ELEMS);
    if constexpr (ENT) {
      if (threadIdx.x < 32) {
        float* f = GL::ent(b);
        f[threadIdx.x] = e.x;
        f[32 + threadIdx.x] = -e.y;
      }
    }
  }
};

// Scores of one 16-row block against the 32 entries of the step, added to
// c0 (entries 0-15) and c1 (entries 16-31) instead of to zero.
template <typename T, int D>
__device__ __forceinline__ void step_scores_from(const StepFrags<T, D>& f, const Frag<T>* qf, float* sc, f32x4 s0,
                                                 f32x4 s1) {
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc) {
    mma16(s0, f.ka[0][dc], qf[dc]);
    mma16(s1, f.ka[1][dc], qf[dc]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) { sc[r] = s0[r]; sc[4 + r] = s1[r]; }
}

// One 32-entry step for IB blocks of 16 stationary rows.  ROWL: L and delta
// per stationary row (Lr, Dr: this lane's row) instead of per entry (Le, and
// -delta in NDe, in LDS).  MASK: entries at offsets >= nv are absent.
//
// With per-row L (a pass with no P output), the softmax-gradient scale is
// folded into the exponent: exp2(s cscale - (L - log2 cnat)) = P cnat (exact
// for d = 64, where log2 cnat = -3), and dS comes out scaled.  With per-entry
// L and delta the step accumulates the unscaled dS: the caller multiplies
// the ax accumulators by cnat once at the end (scale_acc).
template <int IB, bool MASK, bool ROWL, bool WANT_W, typename T, int D>
__device__ __forceinline__ void grad_step(const StepFrags<T, D>& fy, const StepFrags<T, D>& fz,
                                          const Frag<T> (&xf)[IB][D / 32], const Frag<T> (&wf)[IB][D / 32],
                                          int nv, int lg, float cscale, float cnat, const float (&Lr)[IB],
                                          const float (&Dr)[IB], const float* Le, const float* NDe,
                                          f32x4 (&ax)[IB][D / 16], f32x4 (&aw)[IB][D / 16]) {
  static_assert(ROWL != WANT_W, "per-row statistics go with the no-P passes, per-entry ones with the others");
  constexpr bool FOLD = ROWL;
  const float lcn = FOLD ? __builtin_amdgcn_logf(cnat) : 0.f;
  // per entry: L of this lane's 8 entry slots, and -delta of its slots as
  // the starting values of the dP product (slots 0-3 are entries 4 lg ..,
  // slots 4-7 entries 16 + 4 lg .., the product's output rows)
  float le[8];
  f32x4 nd0 = {0.f, 0.f, 0.f, 0.f}, nd1 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (!ROWL) {
#pragma unroll
    for (int t = 0; t < 8; ++t) le[t] = Le[slot_key(t, lg)];
    nd0 = *(const f32x4*)(NDe + 4 * lg);
    nd1 = *(const f32x4*)(NDe + 16 + 4 * lg);
  }
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    float sc[8], dp[8];
    step_scores(fy, xf[b], sc);
    if constexpr (ROWL) {
      const f32x4 nd = {-Dr[b], -Dr[b], -Dr[b], -Dr[b]};
      step_scores_from(fz, wf[b], dp, nd, nd);
    } else {
      step_scores_from(fz, wf[b], dp, nd0, nd1);
    }
    float p[8], ds[8];
    const float Lb = FOLD ? Lr[b] - lcn : 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float L = FOLD ? Lb : le[t];
      float pt = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t], cscale, -L));
      if (MASK && slot_key(t, lg) >= nv) pt = 0.f;
      p[t] = pt;
      ds[t] = pt * dp[t];
    }
    Frag<T> df;
    set8(df, ds);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) mma16(ax[b][cb], fy.va[cb], df);
    if constexpr (WANT_W) {
      Frag<T> pf;
      set8(pf, p);
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) mma16(aw[b][cb], fz.va[cb], pf);
    }
  }
}

// Streams nsteps steps of entries from `src` through LDS and applies
// grad_step to the wave's blocks.  src.ry(st) / src.rz(st): row pointer
// functions of step st (nullptr past the end); src.re(st): (L, delta) of an
// entry; src.nv(st), src.cscale(st), src.cnat(st); src.prefetch(st), called
// a step before ry(st) (a source read through an index fetches it there).
// A wave with `active`
// false (none of its rows exists) only helps stage.  Ends with a barrier.
template <int IB, bool ROWL, bool WANT_W, bool ENT, int NT, typename T, int D, class Src>
__device__ __forceinline__ void grad_stream(unsigned char* smem, int nsteps, const Src& src,
                                            const Frag<T> (&xf)[IB][D / 32], const Frag<T> (&wf)[IB][D / 32],
                                            const float (&Lr)[IB], const float (&Dr)[IB],
                                            f32x4 (&ax)[IB][D / 16], f32x4 (&aw)[IB][D / 16], int li, int lg,
                                            bool active = true) {
  using GL = GradLds<T, D>;
  using TL = TileLayout<T, D>;
  GradLoader<T, D, NT, WANT_W, ENT> ld;
  unsigned char* b0 = smem;
  unsigned char* b1 = smem + GL::STEP_BYTES;
  if (nsteps > 0) {
    src.prefetch(0);
    ld.load(src.ry(0), src.rz(0), src.re(0));
    src.prefetch(1);
    ld.store(b0);
  }
  // Every load issued so far has landed on every path into the loop (the
  // stationary rows included): otherwise the compiler's wait bookkeeping
  // merges a path where one may still be pending and waits for the step's
  // own staging loads before the step's first product.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    unsigned char* cur = (st & 1) ? b1 : b0;
    unsigned char* nxt = (st & 1) ? b0 : b1;
    const bool more = st + 1 < nsteps;
    if (more) {
      ld.load(src.ry(st + 1), src.rz(st + 1), src.re(st + 1));
      src.prefetch(st + 2);
    }
    if (active) {
      StepFrags<T, D> fy, fz;
      const T* y = GL::y(cur);
      const T* z = GL::z(cur);
      fy.load_keys(y, li, lg);
      fz.load_keys(z, li, lg);
      if constexpr (GL::ROWS) {
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) tr_frag(fy.va[cb], y, TL::KS, 0, cb, li, lg);
        if constexpr (WANT_W) {
#pragma unroll
          for (int cb = 0; cb < D / 16; ++cb) tr_frag(fz.va[cb], z, TL::KS, 0, cb, li, lg);
        }
      } else {
        fy.load_vals(y + TL::K_ELEMS, li, lg);
        if constexpr (WANT_W) fz.load_vals(z + TL::K_ELEMS, li, lg);
      }
      const float* Le = GL::ent(cur);
      const int nv = src.nv(st);
      const float cs = src.cscale(st), cn = src.cnat(st);
      if (nv >= 32) grad_step<IB, false, ROWL, WANT_W>(fy, fz, xf, wf, nv, lg, cs, cn, Lr, Dr, Le, Le + 32, ax, aw);
      else grad_step<IB, true, ROWL, WANT_W>(fy, fz, xf, wf, nv, lg, cs, cn, Lr, Dr, Le, Le + 32, ax, aw);
    }
    if (more) ld.store(nxt);
    __syncthreads();
  }
}

// Entries = rows [j0, j1) of Y and Z (one head's base pointers); per-entry L
// and delta from Lv, Dv when given.
template <typename T, int D>
struct SrcRows {
  const T* Y;
  const T* Z;
  const float* Lv;
  const float* Dv;
  int j0, j1;
  float cs, cn;
  __device__ auto ry(int st) const {
    const T* b = Y;
    const int a = j0 + st * 32, e = j1;
    return [=](int r) -> const T* { const int j = a + r; return j < e ? b + (size_t)j * D : nullptr; };
  }
  __device__ auto rz(int st) const {
    const T* b = Z;
    const int a = j0 + st * 32, e = j1;
    return [=](int r) -> const T* { const int j = a + r; return j < e ? b + (size_t)j * D : nullptr; };
  }
  __device__ auto re(int st) const {
    const float* l = Lv;
    const float* d = Dv;
    const int a = j0 + st * 32, e = j1;
    return [=](int r) -> float2 { const int j = a + r; return j < e ? make_float2(l[j], d[j]) : make_float2(0.f, 0.f); };
  }
  __device__ int nv(int st) const { return min(32, j1 - j0 - st * 32); }
  __device__ void prefetch(int) const {}
  __device__ float cscale(int) const { return cs; }
  __device__ float cnat(int) const { return cn; }
};

// Entries = the queries perm[a .. e) of one head (rows of Y and Z; L and
// delta per entry from Lv, Dv), read through the permutation instead of from
// copies in that order.  Each thread's index for the step it stages next is
// fetched one step earlier (prefetch), so a row's address never waits on a
// global load: the fetched value is kept raw and only checked and clamped
// when it is used (a clamp at fetch time would make the wave wait for that
// load, and with it for the row loads issued just before).  bf16 staging
// map: thread t < 32 * CPR stages row t / CPR of a step (one 16-byte chunk),
// thread t < 32 the entry t.
template <typename T, int D>
struct SrcPerm {
  static_assert(sizeof(T) == 2, "the staging map above is the bf16 one");
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  const T* Y;
  const T* Z;
  const float* Lv;
  const float* Dv;
  const int32_t* perm;
  int a, e, N;
  float cs, cn;
  mutable int ridx = -1, eidx = -1;  // raw permutation entries (-1: none)
  __device__ void prefetch(int st) const {
    const int tid = threadIdx.x;
    const int j = a + st * 32 + tid / CPR, je = a + st * 32 + tid;
    ridx = -1;
    eidx = -1;
    if (tid < 32 * CPR && j < e) ridx = perm[j];
    if (tid < 32 && je < e) eidx = perm[je];
  }
  __device__ auto ry(int) const {
    const T* b = Y;
    const int x = ridx, n = N;
    return [=](int) -> const T* { return x >= 0 ? b + (size_t)min(x, n - 1) * D : nullptr; };
  }
  __device__ auto rz(int) const {
    const T* b = Z;
    const int x = ridx, n = N;
    return [=](int) -> const T* { return x >= 0 ? b + (size_t)min(x, n - 1) * D : nullptr; };
  }
  __device__ auto re(int) const {
    const float* l = Lv;
    const float* d = Dv;
    const int x = eidx, n = N;
    return [=](int) -> float2 {
      const int y = min(x, n - 1);
      return x >= 0 ? make_float2(l[y], d[y]) : make_float2(0.f, 0.f);
    };
  }
  __device__ int nv(int st) const { return min(32, e - a - st * 32); }
  __device__ float cscale(int) const { return cs; }
  __device__ float cnat(int) const { return cn; }
};

// Entries of one query tile: the m0 shared entries (q~, v~; padded to whole
// steps, so each step has one logit scale), then the expert's k keys (Ie:
// their indices, staged in LDS and already clamped into [0, N)).
template <typename T, int D>
struct SrcJoint {
  const T* qt;
  const T* vt;
  const T* K;
  const T* V;
  const int32_t* Ie;
  int m0, ns, k, N;
  float cs, cn, cs_sh, cn_sh;
  __device__ auto ry(int st) const { return rows(st, qt, K); }
  __device__ auto rz(int st) const { return rows(st, vt, V); }
  __device__ auto rows(int st, const T* shared, const T* raw) const {
    const int32_t* I = Ie;
    const int ns_ = ns, m0_ = m0, k_ = k;
    return [=](int r) -> const T* {
      if (st < ns_) {
        const int x = st * 32 + r;
        return x < m0_ ? shared + (size_t)x * D : nullptr;
      }
      const int x = (st - ns_) * 32 + r;
      return x < k_ ? raw + (size_t)I[x] * D : nullptr;
    };
  }
  __device__ auto re(int) const { return [](int) -> float2 { return make_float2(0.f, 0.f); }; }
  __device__ int nv(int st) const { return st < ns ? min(32, m0 - st * 32) : min(32, k - (st - ns) * 32); }
  __device__ void prefetch(int) const {}
  __device__ float cscale(int st) const { return st < ns ? cs_sh : cs; }
  __device__ float cnat(int st) const { return st < ns ? cn_sh : cn; }
};

template <typename T, int D, int IB, class RowPtr>
__device__ __forceinline__ void load_rows(Frag<T> (&f)[IB][D / 32], int lg, RowPtr row) {
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const T* p = row(b);
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (p) load8(f[b][dc], p + dc * 32 + 8 * lg);
      else zero(f[b][dc]);
    }
  }
}

template <int IB, int D>
__device__ __forceinline__ void zero_acc(f32x4 (&a)[IB][D / 16]) {
#pragma unroll
  for (int b = 0; b < IB; ++b)
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) a[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// The logit scale of a per-entry pass's dS, applied once to its sums.
template <int IB, int D>
__device__ __forceinline__ void scale_acc(f32x4 (&a)[IB][D / 16], float c) {
#pragma unroll
  for (int b = 0; b < IB; ++b)
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) a[b][cb][r] *= c;
}

// ---------------------------------------------------------------------------
// Landmark rows over one chunk of entries (all heads' chunks in the grid).
// JOINT: entries are queries (Y q, Z dO, per-entry lse and dO . o); outputs
// the chunk's dq~ (scaled by the shared-logit scale) and dv~.  Otherwise
// entries are keys (Y k, Z v) and L, delta are the landmark rows'; output
// the chunk's dq~ of the shared-value softmax.
template <typename T, int D, int NW, int IB, bool JOINT>
__global__ __launch_bounds__(NW * 64, 2) void k_bwd_lm(const T* __restrict__ Y, const T* __restrict__ Z,
                                                       const T* __restrict__ X, const T* __restrict__ W,
                                                       const float* __restrict__ Lv, const float* __restrict__ Dv,
                                                       float* __restrict__ part, int N, int m, int L, int C,
                                                       float cscale, float cnat) {
  constexpr int NT = NW * 64, PW = JOINT ? 2 * D : D;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int chunk = blockIdx.y, bh = blockIdx.z;
  const int i0 = blockIdx.x * (NW * 16 * IB) + wave * 16 * IB;
  Frag<T> xf[IB][D / 32], wf[IB][D / 32];
  float Lr[IB], Dr[IB];
  f32x4 ax[IB][D / 16], aw[IB][D / 16];
  auto rowp = [&](const T* base) {
    return [=](int b) -> const T* { const int i = i0 + b * 16 + li; return i < m ? base + ((size_t)bh * m + i) * D : nullptr; };
  };
  load_rows<T, D, IB>(xf, lg, rowp(X));
  load_rows<T, D, IB>(wf, lg, rowp(W));
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int i = i0 + b * 16 + li;
    Lr[b] = (!JOINT && i < m) ? Lv[(size_t)bh * m + i] : 0.f;
    Dr[b] = (!JOINT && i < m) ? Dv[(size_t)bh * m + i] : 0.f;
  }
  zero_acc<IB, D>(ax);
  zero_acc<IB, D>(aw);
  const int j0 = chunk * L, j1 = min(N, j0 + L);
  const SrcRows<T, D> src{Y + (size_t)bh * N * D, Z + (size_t)bh * N * D, JOINT ? Lv + (size_t)bh * N : nullptr,
                          JOINT ? Dv + (size_t)bh * N : nullptr, j0, j1, cscale, cnat};
  grad_stream<IB, !JOINT, JOINT, JOINT, NT, T, D>(smem, (j1 - j0 + 31) / 32, src, xf, wf, Lr, Dr, ax, aw, li, lg);
  if constexpr (JOINT) scale_acc<IB, D>(ax, cnat);
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int i = i0 + b * 16 + li;
    if (i >= m) continue;
    float* dst = part + (((size_t)bh * C + chunk) * m + i) * PW;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      *(float4*)(dst + cb * 16 + 4 * lg) = make_float4(ax[b][cb][0], ax[b][cb][1], ax[b][cb][2], ax[b][cb][3]);
      if constexpr (JOINT)
        *(float4*)(dst + D + cb * 16 + 4 * lg) = make_float4(aw[b][cb][0], aw[b][cb][1], aw[b][cb][2], aw[b][cb][3]);
    }
  }
}

// Key rows.  ROUTED: the k keys of expert e over one item (up to CH of the
// queries routed to e in a slot; a large expert is split into several items
// so no workgroup carries its whole list), read from the copies gathered in
// expert order so every step streams contiguous rows; writes the item's
// dk, dv parts of the expert rows to G [s, UB2, k, 2d].  Otherwise:
// every key over the nent landmark rows of the shared-value softmax (nent = 0
// in the routing-only variant), plus the sum of its routed parts (G here is
// the compact per-key sum k_bwd_route_sum wrote at ipos[key], present when
// icnt[key] > 0); writes dK, dV in the input dtype.  No atomics: every output
// row has one writer.
template <typename T, int D, int NW, int IB, bool ROUTED>
__global__ __launch_bounds__(NW * 64, 2) void k_bwd_keys(
    const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Ysrc, const T* __restrict__ Zsrc,
    const float* __restrict__ Lv, const float* __restrict__ Dv, const int32_t* __restrict__ qperm,
    const int32_t* __restrict__ topk, const WorkItem* __restrict__ wl2, const int* __restrict__ wl2_count,
    float* __restrict__ G, const int* __restrict__ icnt, const int* __restrict__ ipos, T* __restrict__ dK,
    T* __restrict__ dV, int N, int m, int k, int nent, int BH, int UB2, float cscale, float cnat) {
  constexpr int NT = NW * 64;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  int bh, cnt = 0, start = 0, slot = 0, e = 0, rt;
  if constexpr (ROUTED) {
    // grid x: (slot, item) of the slot's list, y: 16*IB*NW-row tiles of the expert
    slot = blockIdx.x / UB2;
    if ((int)(blockIdx.x % UB2) >= wl2_count[slot]) return;  // uniform over the block
    const WorkItem it = wl2[blockIdx.x];
    bh = it.be / m;
    e = it.be % m;
    start = it.start;
    cnt = it.count;
    rt = blockIdx.y;
  } else {
    bh = blockIdx.y;
    rt = blockIdx.x;
  }
  const int r0 = rt * (NW * 16 * IB) + wave * 16 * IB;
  int jr[IB];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int r = r0 + b * 16 + li;
    if constexpr (ROUTED) jr[b] = r < k ? min(max(topk[((size_t)bh * m + e) * k + r], 0), N - 1) : -1;
    else jr[b] = r < N ? r : -1;
  }
  Frag<T> xf[IB][D / 32], wf[IB][D / 32];
  load_rows<T, D, IB>(xf, lg, [&](int b) -> const T* { return jr[b] >= 0 ? K + ((size_t)bh * N + jr[b]) * D : nullptr; });
  load_rows<T, D, IB>(wf, lg, [&](int b) -> const T* { return jr[b] >= 0 ? V + ((size_t)bh * N + jr[b]) * D : nullptr; });
  float Lr[IB] = {}, Dr[IB] = {};
  f32x4 ax[IB][D / 16], aw[IB][D / 16];
  zero_acc<IB, D>(ax);
  zero_acc<IB, D>(aw);
  if constexpr (ROUTED) {
    const size_t so = (size_t)slot * BH * N;
    if constexpr (sizeof(T) == 2) {
      // the item's queries read through the slot's expert-order permutation
      // (q, dO, lse and dO . o in query order)
      const size_t hb = (size_t)bh * N;
      const SrcPerm<T, D> src{Ysrc + hb * D, Zsrc + hb * D, Lv + hb, Dv + hb, qperm + so, start, start + cnt, N,
                              cscale, cnat};
      grad_stream<IB, false, true, true, NT, T, D>(smem, (cnt + 31) / 32, src, xf, wf, Lr, Dr, ax, aw, li, lg);
      scale_acc<IB, D>(ax, cnat);
    } else {
      // the slot's queries gathered in expert order (q, dO, lse, dO . o)
      const SrcRows<T, D> src{Ysrc + so * D, Zsrc + so * D, Lv + so, Dv + so, start, start + cnt, cscale, cnat};
      grad_stream<IB, false, true, true, NT, T, D>(smem, (cnt + 31) / 32, src, xf, wf, Lr, Dr, ax, aw, li, lg);
      scale_acc<IB, D>(ax, cnat);
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const int r = r0 + b * 16 + li;
      if (r >= k) continue;
      float* dst = G + ((size_t)blockIdx.x * k + r) * (2 * D);
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        *(float4*)(dst + cb * 16 + 4 * lg) = make_float4(ax[b][cb][0], ax[b][cb][1], ax[b][cb][2], ax[b][cb][3]);
        *(float4*)(dst + D + cb * 16 + 4 * lg) = make_float4(aw[b][cb][0], aw[b][cb][1], aw[b][cb][2], aw[b][cb][3]);
      }
    }
  } else {
    const SrcRows<T, D> src{Ysrc + (size_t)bh * m * D, Zsrc + (size_t)bh * m * D, Lv + (size_t)bh * m,
                            Dv + (size_t)bh * m, 0, nent, cscale, cnat};
    grad_stream<IB, false, true, true, NT, T, D>(smem, (nent + 31) / 32, src, xf, wf, Lr, Dr, ax, aw, li, lg);
    scale_acc<IB, D>(ax, cnat);
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      if (jr[b] < 0) continue;
      const size_t key = (size_t)bh * N + jr[b];
      if (icnt[key] > 0) {  // the key's routed parts, summed by k_bwd_route_sum
        const float* g = G + (size_t)ipos[key] * (2 * D);
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const float4 a = *(const float4*)(g + cb * 16 + 4 * lg);
          const float4 c = *(const float4*)(g + D + cb * 16 + 4 * lg);
          ax[b][cb][0] += a.x; ax[b][cb][1] += a.y; ax[b][cb][2] += a.z; ax[b][cb][3] += a.w;
          aw[b][cb][0] += c.x; aw[b][cb][1] += c.y; aw[b][cb][2] += c.z; aw[b][cb][3] += c.w;
        }
      }
      const size_t o = key * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dK[o + cb * 16 + 4 * lg + r] = from_f32<T>(ax[b][cb][r]);
          dV[o + cb * 16 + 4 * lg + r] = from_f32<T>(aw[b][cb][r]);
        }
    }
  }
}

// The shared-value key pass with the landmarks resident in LDS (bf16): q~
// and dv~ are staged once per workgroup, row-major, and the workgroup loops
// over key tiles with no staging and no barrier in its inner loop.  The
// transposed operands (q~^T, dv~^T for dk += dS q~, dv += P dv~) come from
// the same row-major rows through the LDS transpose read (tr_frag).
template <int D, int NW, int IB>
__global__ __launch_bounds__(NW * 64, 2) void k_bwd_keys_res(
    const __bf16* __restrict__ K, const __bf16* __restrict__ V, const __bf16* __restrict__ Qt,
    const __bf16* __restrict__ dVt, const float* __restrict__ Lm, const float* __restrict__ Dm,
    const float* __restrict__ Gs, const int* __restrict__ icnt, const int* __restrict__ ipos,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int m, float cscale, float cnat) {
  using T = __bf16;
  constexpr int KS = TileLayout<T, D>::KS;
  constexpr int R = NW * 16 * IB;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = (m + 31) / 32 * 32;
  T* Yr = (T*)smem;
  T* Zr = Yr + (size_t)Mp * KS;
  float* Le = (float*)(Zr + (size_t)Mp * KS);
  float* De = Le + Mp;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int bh = blockIdx.y;
  // stage the head's landmarks once: rows past m are zero and their L, delta
  // zero (they are masked in the last step)
  constexpr int CPR = D / 8;
  for (int i = tid; i < Mp * CPR; i += NW * 64) {
    const int r = i / CPR, c = (i % CPR) * 8;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    if (r < m) {
      a = *(const uint4*)(Qt + ((size_t)bh * m + r) * D + c);
      b = *(const uint4*)(dVt + ((size_t)bh * m + r) * D + c);
    }
    *(uint4*)(Yr + (size_t)r * KS + c) = a;
    *(uint4*)(Zr + (size_t)r * KS + c) = b;
  }
  for (int r = tid; r < Mp; r += NW * 64) {
    Le[r] = r < m ? Lm[(size_t)bh * m + r] : 0.f;
    De[r] = r < m ? -Dm[(size_t)bh * m + r] : 0.f;  // -delta (see grad_step)
  }
  __syncthreads();
  const float Lr[IB] = {}, Dr[IB] = {};
  const int ntiles = (N + R - 1) / R;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int r0 = tile * R + wave * 16 * IB;
    int jr[IB];
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const int r = r0 + b * 16 + li;
      jr[b] = r < N ? r : -1;
    }
    Frag<T> xf[IB][D / 32], wf[IB][D / 32];
    load_rows<T, D, IB>(xf, lg, [&](int b) -> const T* { return jr[b] >= 0 ? K + ((size_t)bh * N + jr[b]) * D : nullptr; });
    load_rows<T, D, IB>(wf, lg, [&](int b) -> const T* { return jr[b] >= 0 ? V + ((size_t)bh * N + jr[b]) * D : nullptr; });
    f32x4 ax[IB][D / 16], aw[IB][D / 16];
    zero_acc<IB, D>(ax);
    zero_acc<IB, D>(aw);
    // full steps in the loop, the partial last one (m not a multiple of 32)
    // after it: one form of the step per loop body keeps the registers
    auto step = [&](int x0, auto masked) {
      StepFrags<T, D> fy, fz;
      fy.load_keys(Yr + (size_t)x0 * KS, li, lg);
      fz.load_keys(Zr + (size_t)x0 * KS, li, lg);
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        tr_frag(fy.va[cb], Yr, KS, x0, cb, li, lg);
        tr_frag(fz.va[cb], Zr, KS, x0, cb, li, lg);
      }
      grad_step<IB, decltype(masked)::value, false, true, T, D>(fy, fz, xf, wf, m - x0, lg, cscale, cnat, Lr, Dr,
                                                               Le + x0, De + x0, ax, aw);
    };
    int x0 = 0;
    for (; x0 + 32 <= m; x0 += 32) step(x0, BoolTag<false>{});
    if (x0 < m) step(x0, BoolTag<true>{});
    scale_acc<IB, D>(ax, cnat);
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      if (jr[b] < 0) continue;
      const size_t key = (size_t)bh * N + jr[b];
      if (icnt[key] > 0) {  // the key's routed parts, summed by k_bwd_route_sum
        const float* gp = Gs + (size_t)ipos[key] * (2 * D);
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const float4 a = *(const float4*)(gp + cb * 16 + 4 * lg);
          const float4 c = *(const float4*)(gp + D + cb * 16 + 4 * lg);
          ax[b][cb][0] += a.x; ax[b][cb][1] += a.y; ax[b][cb][2] += a.z; ax[b][cb][3] += a.w;
          aw[b][cb][0] += c.x; aw[b][cb][1] += c.y; aw[b][cb][2] += c.z; aw[b][cb][3] += c.w;
        }
      }
      const size_t o = key * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dK[o + cb * 16 + 4 * lg + r] = from_f32<T>(ax[b][cb][r]);
          dV[o + cb * 16 + 4 * lg + r] = from_f32<T>(aw[b][cb][r]);
        }
    }
  }
}

// delta = dO . o per query, in query order, from the forward's fp32 output
// (so that it equals sum_t P_t dP_t up to fp32 rounding even where one entry
// dominates and dP_t - delta cancels).  CPR lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_delta(const T* __restrict__ dO, const float* __restrict__ O32,
                                                   float* __restrict__ Dn, long long rows) {
  constexpr int EPC = 16 / (int)sizeof(T), CPR = D / EPC;
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long pos = g / CPR;
  const int c = (int)(g % CPR);
  float acc = 0.f;
  if (pos < rows) {
    const uint4 gv = *(const uint4*)(dO + pos * D + c * EPC);
    const T* pg = (const T*)&gv;
    const float4* po = (const float4*)(O32 + pos * D + c * EPC);
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      const float4 o = po[q];
      acc = __builtin_fmaf(o.x, to_f32(pg[4 * q]), acc);
      acc = __builtin_fmaf(o.y, to_f32(pg[4 * q + 1]), acc);
      acc = __builtin_fmaf(o.z, to_f32(pg[4 * q + 2]), acc);
      acc = __builtin_fmaf(o.w, to_f32(pg[4 * q + 3]), acc);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (pos < rows && c == 0) Dn[pos] = acc;
}

// Copies of q, dO, lse and delta = dO . o in each slot's expert order:
// position t * BH * N + x holds query perm_t[x] of head x / N (each head
// fills N consecutive positions of a slot).  delta is formed here from the
// forward's fp32 output (so that it equals sum_t P_t dP_t up to fp32 rounding
// even where one entry dominates and dP_t - delta cancels) and also written
// in query order (slot 0).  CPR lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_gather(const T* __restrict__ Q, const T* __restrict__ dO,
                                                    const float* __restrict__ O32, const float* __restrict__ lse,
                                                    const int32_t* __restrict__ perm, T* __restrict__ Qg,
                                                    T* __restrict__ dOg, float* __restrict__ Lg,
                                                    float* __restrict__ Dg, float* __restrict__ Dn, int N,
                                                    long long BHN, long long rows) {
  constexpr int EPC = 16 / (int)sizeof(T), CPR = D / EPC;
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long pos = g / CPR;  // over s * BH * N
  const int c = (int)(g % CPR);
  float acc = 0.f;
  long long src = 0;
  if (pos < rows) {
    const long long x = pos % BHN;
    src = (x / N) * N + min(max(perm[pos], 0), N - 1);
    const uint4 qv = *(const uint4*)(Q + src * D + c * EPC);
    const uint4 gv = *(const uint4*)(dO + src * D + c * EPC);
    *(uint4*)(Qg + pos * D + c * EPC) = qv;
    *(uint4*)(dOg + pos * D + c * EPC) = gv;
    const T* pg = (const T*)&gv;
    const float4* po = (const float4*)(O32 + src * D + c * EPC);
#pragma unroll
    for (int q = 0; q < EPC / 4; ++q) {
      const float4 o = po[q];
      acc = __builtin_fmaf(o.x, to_f32(pg[4 * q]), acc);
      acc = __builtin_fmaf(o.y, to_f32(pg[4 * q + 1]), acc);
      acc = __builtin_fmaf(o.z, to_f32(pg[4 * q + 2]), acc);
      acc = __builtin_fmaf(o.w, to_f32(pg[4 * q + 3]), acc);
    }
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (pos < rows && c == 0) {
    Lg[pos] = lse[src];
    Dg[pos] = acc;
    if (pos < BHN) Dn[src] = acc;
  }
}

// Sum of every routed part of a key (over its expert rows, slots and items)
// into Gs[ipos[key]] (a compact row per key that some expert holds).  The
// grid runs over positions of the inverse lists, which are grouped by key;
// the first position of each key sums its parts.  Each key's 2d values are
// spread over 2d/4 lanes with float4 loads.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_route_sum(const float* __restrict__ G, const int* __restrict__ counts,
                                                       const int* __restrict__ efirst, const int* __restrict__ epart,
                                                       const int* __restrict__ icnt, const int32_t* __restrict__ ikey,
                                                       const int32_t* __restrict__ ilist, float* __restrict__ Gs,
                                                       long long total, int N, int m, int k, int s, int BH, int CH,
                                                       int UB2) {
  constexpr int LPK = 2 * D / 4;  // lanes per key
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long p0 = g / LPK;
  const int c = (int)(g % LPK) * 4;
  if (p0 >= total) return;
  // the key's first (expert, row) slot is read beside the key itself and
  // that slot's item bounds in slot 0 beside the key's count, and its parts
  // are added before the loop over the rest (every key listed here has at
  // least one slot), so a key held by one expert row (most of them) waits
  // for three dependent loads (key and slot, item bounds, parts) instead of
  // five; the parts are added in the same order as before
  const int key = ikey[p0];
  const int er0 = ilist[p0];
  if (p0 > 0 && ikey[p0 - 1] == key) return;  // not the key's first position
  const int bh = key / N;
  const size_t E = (size_t)BH * m;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add_items = [&](int t, int r, int f0, int nf, int pi) {
    for (int q = f0; q < f0 + nf + (pi >= 0 ? 1 : 0); ++q) {
      const int item = q < f0 + nf ? q : pi;
      const float4 v = *(const float4*)(G + (((size_t)t * UB2 + item) * k + r) * (2 * D) + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  };
  const int n = icnt[key];
  {
    const size_t xe = (size_t)bh * m + er0 / k;
    add_items(0, er0 % k, efirst[xe], counts[xe] / CH, epart[xe]);
  }
  for (int x = 0; x < n; ++x) {
    const int er = x == 0 ? er0 : ilist[p0 + x];
    const int ee = er / k, r = er % k;
    for (int t = x == 0 ? 1 : 0; t < s; ++t) {
      const size_t xe = (size_t)t * E + (size_t)bh * m + ee;
      add_items(t, r, efirst[xe], counts[xe] / CH, epart[xe]);
    }
  }
  *(float4*)(Gs + (size_t)p0 * (2 * D) + c) = acc;
}

// Inverse of the experts: for every key, the (expert, row) slots holding it,
// by a counting sort (count, exclusive prefix over all keys, fill).
__global__ __launch_bounds__(256) void k_bwd_inv_count(const int32_t* __restrict__ topk, int* __restrict__ icnt,
                                                       int N, long long mk, long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long bh = i / mk;
  const int j = min(max(topk[i], 0), N - 1);
  atomicAdd(icnt + bh * N + j, 1);
}

__global__ __launch_bounds__(256) void k_bwd_inv_fill(const int32_t* __restrict__ topk, const int* __restrict__ ipos,
                                                      int* __restrict__ icur, int32_t* __restrict__ ilist,
                                                      int32_t* __restrict__ ikey, int N, long long mk,
                                                      long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const long long bh = i / mk;
  const int j = min(max(topk[i], 0), N - 1);
  const long long key = bh * N + j;
  const long long at = ipos[key] + atomicAdd(icur + key, 1);
  ilist[at] = (int32_t)(i - bh * mk);
  ikey[at] = (int32_t)key;
}

// Exclusive prefix sum of n ints in three passes: per-block scans of
// SCAN_PER_BLOCK elements with block totals, a one-workgroup scan of the
// totals, and the block offsets added.
constexpr int SCAN_EPT = 16;
constexpr int SCAN_PER_BLOCK = 256 * SCAN_EPT;

__device__ __forceinline__ int block_exclusive_scan256(int v, int* sh, int& total) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += sh[w];
  total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return wbase + x - v;
}

__global__ __launch_bounds__(256) void k_scan_local(const int* __restrict__ in, int* __restrict__ out,
                                                    int* __restrict__ bsum, long long n) {
  __shared__ int sh[4];
  const long long base = (long long)blockIdx.x * SCAN_PER_BLOCK + (long long)threadIdx.x * SCAN_EPT;
  int v[SCAN_EPT], sum = 0;
#pragma unroll
  for (int u = 0; u < SCAN_EPT; ++u) {
    v[u] = base + u < n ? in[base + u] : 0;
    sum += v[u];
  }
  int total;
  int run = block_exclusive_scan256(sum, sh, total);
#pragma unroll
  for (int u = 0; u < SCAN_EPT; ++u) {
    if (base + u < n) out[base + u] = run;
    run += v[u];
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(256) void k_scan_top(int* __restrict__ bsum, int nb) {
  __shared__ int sh[4];
  int carry = 0;
  for (int c0 = 0; c0 < nb; c0 += 256) {
    const int i = c0 + threadIdx.x;
    const int v = i < nb ? bsum[i] : 0;
    int total;
    const int ex = block_exclusive_scan256(v, sh, total);
    if (i < nb) bsum[i] = carry + ex;
    carry += total;
  }
}

__global__ __launch_bounds__(256) void k_scan_add(int* __restrict__ out, const int* __restrict__ bsum, long long n) {
  const long long base = (long long)blockIdx.x * SCAN_PER_BLOCK;
  const int add = bsum[blockIdx.x];
  for (int u = threadIdx.x; u < SCAN_PER_BLOCK; u += 256)
    if (base + u < n) out[base + u] += add;
}

// Query rows of one work item (expert e, a tile of the queries routed to it
// in `slot`) over the tile's joint-softmax entries.  Slots >= 1 store their
// dq part; the slot-0 pass (launched last) adds the m_shared shared entries,
// the stored parts and pooling's adjoint, and writes dQ.
template <typename T, int D, int NW, int IB, bool SLOT0>
__global__ __launch_bounds__(NW * 64, 2) void k_bwd_q(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ qt, const T* __restrict__ vt, const float* __restrict__ lse, const float* __restrict__ Dn,
    const int32_t* __restrict__ topk, const int32_t* __restrict__ perm, const WorkItem* __restrict__ wl,
    const int* __restrict__ wl_count, const float* __restrict__ dqt, float* __restrict__ qpart, T* __restrict__ dQ,
    int N, int m, int k, int s, int slot, int BH, int m_shared, int gh, int gw, int lh, int lw, float cscale,
    float cscale_sh, float cnat, float cnat_sh) {
  constexpr int NT = NW * 64;
  extern __shared__ __align__(16) unsigned char smem[];
  if ((int)blockIdx.x >= *wl_count) return;
  const WorkItem it = wl[blockIdx.x];
  const int bh = it.be / m;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  int qn[IB];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int local = wave * 16 * IB + b * 16 + li;
    qn[b] = local < it.count ? perm[it.start + local] : -1;
  }
  const size_t row0 = (size_t)bh * N;
  Frag<T> xf[IB][D / 32], wf[IB][D / 32];
  load_rows<T, D, IB>(xf, lg, [&](int b) -> const T* { return qn[b] >= 0 ? Q + (row0 + qn[b]) * D : nullptr; });
  load_rows<T, D, IB>(wf, lg, [&](int b) -> const T* { return qn[b] >= 0 ? dO + (row0 + qn[b]) * D : nullptr; });
  float Lr[IB], Dr[IB];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    Lr[b] = qn[b] >= 0 ? lse[row0 + qn[b]] : 0.f;
    Dr[b] = qn[b] >= 0 ? Dn[row0 + qn[b]] : 0.f;
  }
  f32x4 ax[IB][D / 16], aw[IB][D / 16];
  zero_acc<IB, D>(ax);
  const int m0 = SLOT0 ? m_shared : 0;
  const int ns = (m0 + 31) / 32;
  // the expert's key indices (from the forward; the clamp only keeps other
  // contents in bounds), staged after the two step buffers
  int32_t* s_idx = (int32_t*)(smem + 2 * GradLds<T, D>::STEP_BYTES);
  const int32_t* Ie = topk + (size_t)it.be * k;
  for (int x = tid; x < k; x += NT) s_idx[x] = min(max(Ie[x], 0), N - 1);
  __syncthreads();
  const SrcJoint<T, D> src{qt + (size_t)bh * m * D, vt + (size_t)bh * m * D, K + row0 * D, V + row0 * D,
                           s_idx, m0, ns, k, N, cscale, cnat, cscale_sh, cnat_sh};
  // the last tile of an expert is partly empty: waves with no query skip
  // the arithmetic
  const bool active = __builtin_amdgcn_readfirstlane(wave * 16 * IB) < it.count;
  grad_stream<IB, true, false, false, NT, T, D>(smem, ns + (k + 31) / 32, src, xf, wf, Lr, Dr, ax, aw, li, lg,
                                                active);

#pragma unroll
  for (int b = 0; b < IB; ++b) {
    if (qn[b] < 0) continue;
    const size_t qrow = row0 + qn[b];
    if constexpr (!SLOT0) {
      float* dst = qpart + ((size_t)(slot - 1) * BH * N + qrow) * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        *(float4*)(dst + cb * 16 + 4 * lg) = make_float4(ax[b][cb][0], ax[b][cb][1], ax[b][cb][2], ax[b][cb][3]);
    } else {
      float v[D / 16][4];
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[cb][r] = ax[b][cb][r];
      for (int t = 1; t < s; ++t) {
        const float* src_ = qpart + ((size_t)(t - 1) * BH * N + qrow) * D;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const float4 a = *(const float4*)(src_ + cb * 16 + 4 * lg);
          v[cb][0] += a.x; v[cb][1] += a.y; v[cb][2] += a.z; v[cb][3] += a.w;
        }
      }
      if (m_shared > 0) {
        // pooling's adjoint: token (y, x) lies in landmark windows
        // iy in [floor(y lh / gh), ceil((y + 1) lh / gh) - 1] (likewise x),
        // window iy spanning [floor(iy gh / lh), ceil((iy + 1) gh / lh))
        const long long y = qn[b] / gw, x = qn[b] % gw;
        const int ylo = (int)(y * lh / gh), yhi = min(lh - 1, (int)(((y + 1) * lh + gh - 1) / gh) - 1);
        const int xlo = (int)(x * lw / gw), xhi = min(lw - 1, (int)(((x + 1) * lw + gw - 1) / gw) - 1);
        for (int iy = ylo; iy <= yhi; ++iy) {
          const long long hy = ((long long)(iy + 1) * gh + lh - 1) / lh - (long long)iy * gh / lh;
          for (int ix = xlo; ix <= xhi; ++ix) {
            const long long hx = ((long long)(ix + 1) * gw + lw - 1) / lw - (long long)ix * gw / lw;
            const float w = 1.0f / (float)(hy * hx);
            const float* g = dqt + ((size_t)bh * m + (size_t)iy * lw + ix) * D;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) {
              const float4 a = *(const float4*)(g + cb * 16 + 4 * lg);
              v[cb][0] += w * a.x; v[cb][1] += w * a.y; v[cb][2] += w * a.z; v[cb][3] += w * a.w;
            }
          }
        }
      }
      T* dst = dQ + qrow * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[cb * 16 + 4 * lg + r] = from_f32<T>(v[cb][r]);
    }
  }
  (void)aw;
}

// ---------------------------------------------------------------------------
// small passes

// v~ in the input dtype, rounded as the forward rounded it for step 6.
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_cvt(const float* __restrict__ x, T* __restrict__ y, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = from_f32<T>(x[i]);
}

// Per-(slot, head, expert) query counts from the saved routes, which are
// copied (clamped into [0, m)) for the grouping kernels.
constexpr int CNT_PER_WG = 4096;
__global__ __launch_bounds__(256) void k_bwd_count(const int32_t* __restrict__ route_in, int32_t* __restrict__ route,
                                                   int* __restrict__ counts, int N, int m, int s, int BH, int hist_lds) {
  extern __shared__ int hist[];
  const int bh = blockIdx.y;
  if (hist_lds) {
    for (int x = threadIdx.x; x < s * m; x += 256) hist[x] = 0;
    __syncthreads();
  }
  const long long tot = (long long)N * s;
  const long long base = (long long)bh * tot;
  const long long e0 = (long long)blockIdx.x * CNT_PER_WG;
  for (int u = threadIdx.x; u < CNT_PER_WG; u += 256) {
    const long long x = e0 + u;
    if (x < tot) {
      const int e = min(max(route_in[base + x], 0), m - 1);
      route[base + x] = e;
      const int t = (int)(x % s);
      if (hist_lds) atomicAdd(hist + t * m + e, 1);
      else atomicAdd(counts + ((size_t)t * BH + bh) * m + e, 1);
    }
  }
  if (hist_lds) {
    __syncthreads();
    for (int x = threadIdx.x; x < s * m; x += 256) {
      const int c = hist[x];
      if (c) atomicAdd(counts + ((size_t)(x / m) * BH + bh) * m + (x % m), c);
    }
  }
}

// Sum of the joint pass's chunk partials per landmark row: dq~ (joint part),
// dv~ (fp32 and input dtype) and delta = dv~ . v~, taken with the rounded
// dv~ the matrix cores use for dA = dv~ . v_j and the fp32 v~, so that
// dA_j - delta = dv~ . (v_j - v~) holds without bf16 cancellation error.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_bwd_red1(const float* __restrict__ part, const float* __restrict__ vt32,
                                                 float* __restrict__ dqt, float* __restrict__ dvt,
                                                 T* __restrict__ dvtT, float* __restrict__ delta, int m, int C) {
  const size_t row = blockIdx.x;
  const size_t bh = row / m, i = row % m;
  const int c = threadIdx.x;
  float q = 0.f, v = 0.f;
  if (c < D) {
    const float* p = part + ((bh * C) * m + i) * 2 * D;
    for (int ch = 0; ch < C; ++ch, p += (size_t)m * 2 * D) {
      q += p[c];
      v += p[D + c];
    }
  }
  const T vr = from_f32<T>(v);
  float dd = c < D ? to_f32(vr) * vt32[row * D + c] : 0.f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dd += __shfl_xor(dd, off);
  if (c < D) {
    dqt[row * D + c] = q;
    dvt[row * D + c] = v;
    dvtT[row * D + c] = vr;
  }
  if (c == 0) delta[row] = dd;
}

// dq~ += the shared-value pass's chunk partials.
template <int D>
__global__ __launch_bounds__(64) void k_bwd_red4(const float* __restrict__ part, float* __restrict__ dqt, int m,
                                                 int C) {
  const size_t row = blockIdx.x;
  const size_t bh = row / m, i = row % m;
  const int c = threadIdx.x;
  if (c >= D) return;
  float q = 0.f;
  const float* p = part + ((bh * C) * m + i) * D;
  for (int ch = 0; ch < C; ++ch, p += (size_t)m * D) q += p[c];
  dqt[row * D + c] += q;
}

__global__ __launch_bounds__(256) void k_bwd_zero(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------------------
template <class F>
static void allow_lds(F fn, size_t lds) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// 16-row blocks per wave of a pass over `rows` stationary rows (bf16): a
// workgroup's tile should not be mostly empty rows (m or k of 128 or 256)
static int stat_blocks(int rows, int most) { return rows <= 128 ? 1 : (rows <= 256 || most == 2) ? 2 : 4; }

template <typename T, int D, int NW, int IBK>
static void launch_routed_keys(const BPlan& p, size_t lds) {
  constexpr int R = NW * 16 * IBK;
  auto fn = &k_bwd_keys<T, D, NW, IBK, true>;
  allow_lds(fn, lds);
  dim3 grid((unsigned)(p.s * p.UB2), (unsigned)((p.k + R - 1) / R));
  // bf16 reads the queries through the expert-order permutation; fp32 from
  // copies gathered in that order
  constexpr bool PERM = sizeof(T) == 2;
  hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, p.stream, (const T*)p.K, (const T*)p.V,
                     (const T*)(PERM ? p.Q : p.Qg), (const T*)(PERM ? p.dO : p.dOg), PERM ? p.lse : p.Lg,
                     PERM ? p.Dn : p.Dg, (const int32_t*)p.bk.perm, p.topk, p.wl2, p.wl2_count, p.G,
                     (const int*)nullptr, (const int*)nullptr, (T*)nullptr, (T*)nullptr, p.N, p.m, p.k, 0, p.BH,
                     p.UB2, p.cscale, p.cnat);
}

template <typename T, int D, int NW, int IBL>
static void launch_lm_joint(const BPlan& p, size_t lds) {
  constexpr int R = NW * 16 * IBL;
  auto fn = &k_bwd_lm<T, D, NW, IBL, true>;
  allow_lds(fn, lds);
  dim3 grid((unsigned)((p.m + R - 1) / R), (unsigned)p.C1, (unsigned)p.BH);
  hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, p.stream, (const T*)p.Q, (const T*)p.dO, (const T*)p.qt,
                     (const T*)p.vt, p.lse, p.Dn, p.part1, p.N, p.m, p.L1, p.C1, p.cscale_sh, p.cnat_sh);
}

template <typename T, int D, int NW, int IB4>
static void launch_lm_shared(const BPlan& p, size_t lds) {
  constexpr int R4 = NW * 16 * IB4;
  auto fn = &k_bwd_lm<T, D, NW, IB4, false>;
  allow_lds(fn, lds);
  dim3 grid((unsigned)((p.m + R4 - 1) / R4), (unsigned)p.C4, (unsigned)p.BH);
  hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, p.stream, (const T*)p.K, (const T*)p.V, (const T*)p.qt,
                     (const T*)p.dvtT, p.lse_lm, p.delta, p.part4, p.N, p.m, p.L4, p.C4, p.cscale, p.cnat);
}

template <typename T, int D, int NW, int IB>
static void launch_backward_t(const BPlan& p) {
  const size_t lds = 2 * GradLds<T, D>::STEP_BYTES;
  const hipStream_t st = p.stream;
  const int BH = p.BH, N = p.N, m = p.m, k = p.k, s = p.s;

  const size_t n16 = p.zero_bytes / 16;
  if (n16) {
    const int blocks = (int)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_bwd_zero, dim3(blocks), dim3(256), 0, st, (uint4*)p.zero_begin, n16);
  }
  if (p.shared) {
    const long long n = (long long)BH * m * D;
    hipLaunchKernelGGL((k_bwd_cvt<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p.vt32, (T*)p.vt, n);
  }
  {
    const int hist_lds = s * m <= 8192 ? 1 : 0;
    dim3 grid((unsigned)(((long long)N * s + CNT_PER_WG - 1) / CNT_PER_WG), (unsigned)BH);
    hipLaunchKernelGGL(k_bwd_count, grid, dim3(256), hist_lds ? (size_t)s * m * 4 : 0, st, p.route, p.bk.route,
                       p.bk.counts, N, m, s, BH, hist_lds);
  }
  launch_bucket(p.bk);

  // routed keys: per-(slot, expert, row) parts, and the inverse of the experts
  {
    constexpr int CPR = D * (int)sizeof(T) / 16;
    const long long BHN = (long long)BH * N, rows = (long long)s * BHN;
    if constexpr (sizeof(T) == 2) {
      // the routed pass reads the queries through the permutation: only delta
      hipLaunchKernelGGL((k_bwd_delta<T, D>), dim3((unsigned)((BHN * CPR + 255) / 256)), dim3(256), 0, st,
                         (const T*)p.dO, p.o32, p.Dn, BHN);
    } else {
      hipLaunchKernelGGL((k_bwd_gather<T, D>), dim3((unsigned)((rows * CPR + 255) / 256)), dim3(256), 0, st,
                         (const T*)p.Q, (const T*)p.dO, p.o32, p.lse, (const int32_t*)p.bk.perm, (T*)p.Qg,
                         (T*)p.dOg, p.Lg, p.Dg, p.Dn, N, BHN, rows);
    }
    launch_items(p.bk, p.CH, p.UB2, p.wl2, p.wl2_count, p.efirst, p.epart);
    if (sizeof(T) == 2 && stat_blocks(k, IB) == 1) launch_routed_keys<T, D, NW, 1>(p, lds);
    else launch_routed_keys<T, D, NW, IB>(p, lds);
    const long long mk = (long long)m * k, total = (long long)BH * mk, keys = (long long)BH * N;
    const unsigned gb = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(k_bwd_inv_count, dim3(gb), dim3(256), 0, st, p.topk, p.icnt, N, mk, total);
    const int nb = (int)((keys + SCAN_PER_BLOCK - 1) / SCAN_PER_BLOCK);
    hipLaunchKernelGGL(k_scan_local, dim3((unsigned)nb), dim3(256), 0, st, (const int*)p.icnt, p.ipos, p.bsum, keys);
    hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(256), 0, st, p.bsum, nb);
    hipLaunchKernelGGL(k_scan_add, dim3((unsigned)nb), dim3(256), 0, st, p.ipos, (const int*)p.bsum, keys);
    hipLaunchKernelGGL(k_bwd_inv_fill, dim3(gb), dim3(256), 0, st, p.topk, (const int*)p.ipos, p.icur, p.ilist,
                       p.ikey, N, mk, total);
  }
  if (p.shared) {
    if (sizeof(T) == 2 && stat_blocks(m, IB) == 1) launch_lm_joint<T, D, NW, 1>(p, lds);
    else launch_lm_joint<T, D, NW, IB>(p, lds);
    hipLaunchKernelGGL((k_bwd_red1<T, D>), dim3((unsigned)(BH * m)), dim3(64), 0, st, p.part1, p.vt32,
                       p.dqt, p.dvt, (T*)p.dvtT, p.delta, m, p.C1);
  }
  {
    const long long total = (long long)BH * m * k, thr = total * (2 * D / 4);
    hipLaunchKernelGGL((k_bwd_route_sum<D>), dim3((unsigned)((thr + 255) / 256)), dim3(256), 0, st, (const float*)p.G,
                       (const int*)p.bk.counts, (const int*)p.efirst, (const int*)p.epart, (const int*)p.icnt,
                       (const int32_t*)p.ikey, (const int32_t*)p.ilist, p.Gs, total, N, m, k, s, BH, p.CH, p.UB2);
  }
  // shared-value softmax for the keys plus their routed parts: final dK, dV;
  // bf16 with the landmarks resident in LDS when they fit
  const size_t res_lds = 2 * (size_t)((m + 31) / 32 * 32) * (TileLayout<T, D>::KS * sizeof(T) + 4);
  bool resident = false;
  if constexpr (sizeof(T) == 2) {
    if (p.shared && res_lds <= RES_MAX) {
      resident = true;
      constexpr int IBR = 2;
      auto fn = &k_bwd_keys_res<D, NW, IBR>;
      allow_lds(fn, res_lds);
      const int tiles = (N + NW * 16 * IBR - 1) / (NW * 16 * IBR);
      const int per_head = (256 + BH - 1) / BH;  // about one workgroup per compute unit in all
      dim3 grid((unsigned)(tiles < per_head ? tiles : per_head), (unsigned)BH);
      hipLaunchKernelGGL(fn, grid, dim3(NW * 64), res_lds, st, (const T*)p.K, (const T*)p.V, (const T*)p.qt,
                         (const T*)p.dvtT, p.lse_lm, p.delta, (const float*)p.Gs, (const int*)p.icnt,
                         (const int*)p.ipos, (T*)p.dK, (T*)p.dV, N, m, p.cscale, p.cnat);
    }
  }
  // (otherwise staged per step, one 16-row block per wave: with two this pass spills registers)
  if (!resident) {
    constexpr int IB3 = 1, R3 = NW * 16 * IB3;
    auto fn = &k_bwd_keys<T, D, NW, IB3, false>;
    allow_lds(fn, lds);
    dim3 grid((unsigned)((N + R3 - 1) / R3), (unsigned)BH);
    hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, st, (const T*)p.K, (const T*)p.V, (const T*)p.qt,
                       (const T*)p.dvtT, p.lse_lm, p.delta, (const int32_t*)nullptr, p.topk,
                       (const WorkItem*)nullptr, (const int*)nullptr,
                       p.Gs, (const int*)p.icnt, (const int*)p.ipos, (T*)p.dK, (T*)p.dV, N, m, k,
                       p.shared ? m : 0, BH, p.UB2, p.cscale, p.cnat);
  }
  if (p.shared) {
    // four 16-row blocks per wave for bf16 (one accumulator only in this pass)
    if constexpr (sizeof(T) == 2) {
      const int b4 = stat_blocks(m, 4);
      if (b4 == 1) launch_lm_shared<T, D, NW, 1>(p, lds);
      else if (b4 == 2) launch_lm_shared<T, D, NW, 2>(p, lds);
      else launch_lm_shared<T, D, NW, 4>(p, lds);
    } else {
      launch_lm_shared<T, D, NW, IB>(p, lds);
    }
    hipLaunchKernelGGL((k_bwd_red4<D>), dim3((unsigned)(BH * m)), dim3(64), 0, st, p.part4, p.dqt, m, p.C4);
  }
  // queries: slots s-1 .. 1 store parts, slot 0 finishes dQ
  {
    // three 16-query blocks per wave for bf16 (no transposed values or
    // second accumulator in this pass leaves the registers for it), in
    // four-wave workgroups: two per compute unit, so one's per-step barrier
    // and staging overlap the other's arithmetic
    constexpr int IBQ = sizeof(T) == 2 ? 3 : IB;
    constexpr int NWQ = sizeof(T) == 2 ? 4 : NW;
    auto f1 = &k_bwd_q<T, D, NWQ, IBQ, false>;
    auto f0 = &k_bwd_q<T, D, NWQ, IBQ, true>;
    const size_t lq = lds + (size_t)k * 4;
    allow_lds(f1, lq);
    allow_lds(f0, lq);
    for (int t = s - 1; t >= 0; --t) {
      const int32_t* perm = p.bk.perm + (size_t)t * BH * N;
      const WorkItem* wl = p.bk.wl + (size_t)t * p.bk.UB;
      const int* wlc = p.bk.wl_count + t;
      hipLaunchKernelGGL(t > 0 ? f1 : f0, dim3((unsigned)p.bk.UB), dim3(NWQ * 64), lq, st, (const T*)p.Q,
                         (const T*)p.K, (const T*)p.V, (const T*)p.dO, (const T*)p.qt, (const T*)p.vt, p.lse, p.Dn,
                         p.topk, perm, wl, wlc, p.dqt, p.qpart, (T*)p.dQ, N, m, k, s, t, BH, p.shared ? m : 0,
                         p.gh, p.gw, p.lh, p.lw, p.cscale, p.cscale_sh, p.cnat, p.cnat_sh);
    }
  }
}

// Rows per workgroup of every backward kernel for a dtype (the plan's R).
int backward_rows(int dtype, int m) { return dtype == 1 ? 8 * 16 * stat_blocks(m, 2) : 4 * 16 * 1; }
int backward_query_rows(int dtype) { return dtype == 1 ? 4 * 16 * 3 : 4 * 16 * 1; }
int backward_lm4_rows(int dtype, int m) { return dtype == 1 ? 8 * 16 * stat_blocks(m, 4) : 4 * 16 * 1; }

void launch_backward(const BPlan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_backward_t<float, 32, 4, 1>(p); else launch_backward_t<float, 64, 4, 1>(p);
  } else {
    if (p.d == 32) launch_backward_t<__bf16, 32, 8, 2>(p); else launch_backward_t<__bf16, 64, 8, 2>(p);
  }
}

}  // namespace mita
