// LDS-resident routing and attention (used when the m landmark entries and
// the k entries of one expert each fit in LDS).
//
// MiTA's joint softmax (MiTA tutorial (iwxt.cn), ch.4 steps 5-6) runs over
// the m shared entries (q~_i, v~_i), the same for every query of a head, and
// the k entries of the query's expert.  Both kernels below keep their entry
// set in LDS for the lifetime of the workgroup (keys row-major, values
// transposed for the P.V matrix product) and let every wave stream its own
// queries through it with no barrier in the inner loop:
//
//   k_route_shared  per (head, range of queries): q . q~_i for all m
//                   landmarks on the matrix cores.  The raw scores pick the
//                   top-s experts (routing, tutorial ch.4 step 4) and, scaled
//                   by 1/sqrt(d), are the shared logits of the joint softmax
//                   (the reuse the tutorial's cost count of ch.6 assumes), so
//                   the shared part of the output is finished here and stored
//                   as a partial: log2-sum-exp, and the output row divided by
//                   its largest magnitude (fp16, so every stored element lies
//                   in [-1, 1] whatever the scale of V) with that magnitude
//                   kept in fp32.
//   k_expert        per (expert, range of its queries): the expert's k
//                   gathered key/value rows staged once, the routed logits
//                   and values on the matrix cores, then the merge with the
//                   stored partial by the rescaled-sum identity
//                   (Z1 o1 + Z2 o2) / (Z1 + Z2) of tutorial ch.4.  One launch
//                   per routing slot; the last one writes O.
#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

typedef _Float16 f16;

// Storage type of the finished-part output between kernels: fp16 for bf16
// inputs, fp32 for fp32.  An fp16 row is stored divided by its largest
// magnitude (a per-query fp32 scale kept beside it), so it never overflows
// and its rounding is at most 2^-11 of the row's largest element, below the
// bf16 rounding of the output itself; fp32 rows are stored as they are
// (scale 1).
template <typename T> struct PartT { typedef f16 type; };
template <> struct PartT<float> { typedef float type; };

// The per-query scale of a row of 16 values per lane (the four lane groups of
// a query hold its d = 64 outputs): 1 / max|x| for the stored values and
// max|x| * mul for the fp32 scale.  A row of zeros (or one below 1e-30 in
// magnitude, whose rounding to zero is far inside any tolerance) gets 0 and 0.
template <typename P, int NCB>
__device__ __forceinline__ void row_scale(const f32x4 (&x)[NCB], float mul, float& inv_store, float& scale) {
  if constexpr (sizeof(P) == 4) {
    inv_store = 1.0f;
    scale = mul;
  } else {
    float a = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) a = fmaxf(a, fabsf(x[cb][r]));
    a = wave_max_groups(a);
    const bool nz = a > 1e-30f;
    inv_store = nz ? 1.0f / a : 0.f;
    scale = nz ? a * mul : 0.f;
  }
}

// Row layout of the finished-part output: lane group g of a query holds
// output dims cb*16 + 4g + r (cb < D/16, r < 4) in its accumulator tiles, and
// stores them as one contiguous run at positions g*D/4 + cb*4 + r, so the
// four lane groups of a query write (and later read) the whole row.
template <int D>
__device__ __forceinline__ int part_pos(int g, int cb) { return g * (D / 4) + cb * 4; }

template <typename P> struct Vec4;
template <> struct Vec4<f16> { typedef __attribute__((__vector_size__(4 * sizeof(f16)))) f16 type; };
template <> struct Vec4<float> { typedef __attribute__((__vector_size__(4 * sizeof(float)))) float type; };

template <typename T, int D>
struct Resident {
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int KS = D + EPC;  // key row stride (as TileLayout)
  static constexpr int CPR = D / EPC;
  __host__ __device__ static int pad(int E) { return (E + 31) / 32 * 32; }
  __host__ __device__ static size_t bytes(int Ep) { return ((size_t)Ep * KS + (size_t)D * (Ep + 4)) * sizeof(T); }

  // Stage E entries: key row x from rk(x), value row from rv(x); rows E..Ep-1
  // are zero.  Keys row-major [Ep][KS]; values transposed [D][Ep + 4].  Each
  // thread issues its global loads in batches of 8 before the LDS stores, so
  // a batch costs one memory latency instead of eight.
  template <class RK, class RV>
  __device__ static void load(T* Ks, T* Vs, int E, int Ep, RK rk, RV rv) {
    constexpr int U = 8;
    const int vs = Ep + 4, nt = blockDim.x, tid = threadIdx.x;
    const int nk = Ep * CPR;
    for (int base = 0; base < nk; base += U * nt) {
      uint4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * nt + tid, x = i / CPR;
        r[u] = make_uint4(0, 0, 0, 0);
        if (i < nk && x < E) r[u] = *(const uint4*)(rk(x) + (i % CPR) * EPC);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * nt + tid;
        if (i < nk) *(uint4*)(Ks + (i / CPR) * KS + (i % CPR) * EPC) = r[u];
      }
    }
    if constexpr (sizeof(T) == 2) {
      // two value rows per task, packed into 32-bit transposed writes
      const int ntask = (Ep / 2) * CPR;
      for (int base = 0; base < ntask; base += (U / 2) * nt) {
        uint4 ra[U / 2], rb[U / 2];
#pragma unroll
        for (int u = 0; u < U / 2; ++u) {
          const int i = base + u * nt + tid, xp = i / CPR, c0 = (i % CPR) * EPC;
          ra[u] = make_uint4(0, 0, 0, 0);
          rb[u] = make_uint4(0, 0, 0, 0);
          if (i < ntask && 2 * xp < E) ra[u] = *(const uint4*)(rv(2 * xp) + c0);
          if (i < ntask && 2 * xp + 1 < E) rb[u] = *(const uint4*)(rv(2 * xp + 1) + c0);
        }
#pragma unroll
        for (int u = 0; u < U / 2; ++u) {
          const int i = base + u * nt + tid, xp = i / CPR, c0 = (i % CPR) * EPC;
          if (i >= ntask) continue;
          const uint32_t* a = (const uint32_t*)&ra[u];
          const uint32_t* b = (const uint32_t*)&rb[u];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            *(uint32_t*)(Vs + (c0 + 2 * w) * vs + 2 * xp) = (a[w] & 0xFFFFu) | (b[w] << 16);
            *(uint32_t*)(Vs + (c0 + 2 * w + 1) * vs + 2 * xp) = (a[w] >> 16) | (b[w] & 0xFFFF0000u);
          }
        }
      }
    } else {
      for (int base = 0; base < nk; base += U * nt) {
        float4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = base + u * nt + tid, x = i / CPR;
          r[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (i < nk && x < E) r[u] = *(const float4*)(rv(x) + (i % CPR) * EPC);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = base + u * nt + tid, x = i / CPR, c0 = (i % CPR) * EPC;
          if (i >= nk) continue;
          Vs[(c0 + 0) * vs + x] = r[u].x;
          Vs[(c0 + 1) * vs + x] = r[u].y;
          Vs[(c0 + 2) * vs + x] = r[u].z;
          Vs[(c0 + 3) * vs + x] = r[u].w;
        }
      }
    }
  }

  // Matrix-core operands of the 32 entries starting at x0.
  __device__ static void frags(StepFrags<T, D>& f, const T* Ks, const T* Vs, int Ep, int x0, int li, int g) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int dc = 0; dc < D / 32; ++dc) load8(f.ka[jt][dc], Ks + (x0 + jt * 16 + li) * KS + dc * 32 + 8 * g);
    const int vs = Ep + 4;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const T* row = Vs + (cb * 16 + li) * vs + x0;
      load4x2(f.va[cb], row + 4 * g, row + 16 + 4 * g);
    }
  }
};

// Query fragments of one group of 16*IB queries (rows given by qrow(b), or
// -1 for an empty slot).
template <typename T, int D, int IB, class QR>
__device__ __forceinline__ void load_queries(Frag<T> (&qf)[IB][D / 32], const T* Q, int lg, QR qrow) {
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const long long r = qrow(b);
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (r >= 0) load8(qf[b][dc], Q + (size_t)r * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
  }
}

template <int S>
__device__ __forceinline__ void list_insert(float* lv, int* lx, float v, int i) {
#pragma unroll
  for (int t = S - 1; t >= 0; --t) {
    const bool above = (t > 0) && (v > lv[t - 1] || (v == lv[t - 1] && i < lx[t - 1]));
    const bool here = v > lv[t] || (v == lv[t] && i < lx[t]);
    if (above) { lv[t] = lv[t - 1]; lx[t] = lx[t - 1]; }
    else if (here) { lv[t] = v; lx[t] = i; }
  }
}

// ---------------------------------------------------------------------------
// IB: 16-query blocks per wave group (four with eight waves; one with sixteen
// waves, four per SIMD, for mid-size heads)
template <typename T, int D, int NW, int SMAX, int IB>
__global__ __launch_bounds__(NW * 64, NW >= 16 ? 4 : NW >= 12 ? 3 : 1) void k_route_shared(
    const T* __restrict__ Q, const T* __restrict__ Qt, const T* __restrict__ VtT, int32_t* __restrict__ route,
    int* __restrict__ counts, float2* __restrict__ plse, typename PartT<T>::type* __restrict__ po, int N, int m, int s,
    int BH, int qpw, int hist_lds, float cscale) {  // cscale: log2(e) x the shared-logit scale
  using RL = Resident<T, D>;
  using P = typename PartT<T>::type;
  using PV = typename Vec4<P>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Mp = RL::pad(m);
  T* Ks = (T*)smem;
  T* Vs = Ks + (size_t)Mp * RL::KS;
  int* hist = (int*)(smem + RL::bytes(Mp));
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const Frag<T> one = ones_frag<T>(li);
  const int bh = blockIdx.y;
  const int q0 = blockIdx.x * qpw, q1 = min(N, q0 + qpw);
  const T* Qh = Q + (size_t)bh * N * D;
  if (hist_lds)
    for (int x = tid; x < s * m; x += NW * 64) hist[x] = 0;
  RL::load(Ks, Vs, m, Mp, [&](int x) { return Qt + ((size_t)bh * m + x) * D; },
           [&](int x) { return VtT + ((size_t)bh * m + x) * D; });
  __syncthreads();

  constexpr int GQ = 16 * IB;
  const int ngroups = (q1 - q0 + GQ - 1) / GQ;
  auto group_rows = [&](int gi) {
    return [=](int b) -> long long { const int n = q0 + gi * GQ + b * 16 + li; return n < q1 ? n : -1; };
  };
  // the next group's query rows are fetched while the current one computes
  Frag<T> qn[IB][D / 32];
  if (wave < ngroups) load_queries<T, D, IB>(qn, Qh, lg, group_rows(wave));
  for (int gi = wave; gi < ngroups; gi += NW) {
    const int qb = q0 + gi * GQ;
    Frag<T> qf[IB][D / 32];
#pragma unroll
    for (int b = 0; b < IB; ++b)
#pragma unroll
      for (int dc = 0; dc < D / 32; ++dc) qf[b][dc] = qn[b][dc];
    if (gi + NW < ngroups) load_queries<T, D, IB>(qn, Qh, lg, group_rows(gi + NW));
    float lv[IB][SMAX];
    RunMax M[IB];
    f32x4 Z[IB];
    int lx[IB][SMAX];
    f32x4 acc[IB][D / 16];
#pragma unroll
    for (int b = 0; b < IB; ++b) {
#pragma unroll
      for (int t = 0; t < SMAX; ++t) { lv[b][t] = -INFINITY; lx[b][t] = 0x7FFFFFFF; }
      M[b].set(M0, cscale);
      Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int x0 = 0;
    // landmarks reach a lane in increasing order: strict '>' keeps the lower
    // index on ties
    auto topsel = [&](int b, const float* sc, float mx) {
      if constexpr (SMAX == 1) {
        // top-1: the first of this lane's slots holding its maximum (slots
        // ascend with the landmark index), taken when it beats the best so far
        int tf = 7;
#pragma unroll
        for (int t = 6; t >= 0; --t) tf = sc[t] == mx ? t : tf;
        if (mx > lv[b][0]) {
          lv[b][0] = mx;
          lx[b][0] = x0 + 4 * lg + tf + (tf >= 4 ? 12 : 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (sc[t] > lv[b][SMAX - 1]) list_insert<SMAX>(lv[b], lx[b], sc[t], x0 + slot_key(t, lg));
      }
    };
    for (; x0 + 32 <= m; x0 += 32) {
      StepFrags<T, D> f;
      RL::frags(f, Ks, Vs, Mp, x0, li, lg);
      attn_step<IB, false>(f, one, qf, 32, lg, cscale, M, Z, acc, topsel);
    }
    if (x0 < m) {
      StepFrags<T, D> f;
      RL::frags(f, Ks, Vs, Mp, x0, li, lg);
      attn_step<IB, true>(f, one, qf, m - x0, lg, cscale, M, Z, acc, topsel);
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) {
#pragma unroll
      for (int sh = 16; sh <= 32; sh <<= 1) {
        float ov[SMAX];
        int ox[SMAX];
#pragma unroll
        for (int t = 0; t < SMAX; ++t) { ov[t] = __shfl_xor(lv[b][t], sh); ox[t] = __shfl_xor(lx[b][t], sh); }
#pragma unroll
        for (int t = 0; t < SMAX; ++t) list_insert<SMAX>(lv[b], lx[b], ov[t], ox[t]);
      }
      const float Zt = finish_z(Z[b], li);
      const int n = qb + b * 16 + li;
      if (n >= q1) continue;
      const size_t qrow = (size_t)bh * N + n;
      // the stored row: acc / max|acc|; its scale: max|acc| / Z
      float sn, scl;
      row_scale<P, D / 16>(acc[b], 1.0f / Zt, sn, scl);
      if (lg == 0) {
        int32_t* dst = route + qrow * s;
#pragma unroll
        for (int t = 0; t < SMAX; ++t) {
          if (t < s) {
            // a valid list holds s landmarks; the clamp only keeps non-finite
            // inputs (unspecified results) inside the buffers
            const int e = min(max(lx[b][t], 0), m - 1);
            dst[t] = e;
            if (hist_lds) atomicAdd(hist + t * m + e, 1);
            else atomicAdd(counts + ((size_t)t * BH + bh) * m + e, 1);
          }
        }
        plse[qrow] = make_float2(M[b].M + __builtin_amdgcn_logf(Zt), scl);
      }
      P* o = po + qrow * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        PV h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (P)(acc[b][cb][r] * sn);
        *(PV*)(o + part_pos<D>(lg, cb)) = h;
      }
    }
  }
  if (hist_lds) {
    __syncthreads();
    for (int x = tid; x < s * m; x += NW * 64) {
      const int c = hist[x];
      if (c) atomicAdd(counts + ((size_t)(x / m) * BH + bh) * m + (x % m), c);
    }
  }
}

// ---------------------------------------------------------------------------
// One group of IB blocks of 16 queries (query rows qn[b], -1 for an empty
// slot) against the expert's k resident entries, merged with the stored
// finished part.  EARLY: the stored part is fetched before the key loop (it
// arrives while the loop computes; for the launch shapes with registers to
// hold it), else after it.  issue() starts the caller's own loads for later
// (the next group's query rows) once the group's own are in.
template <int IB, typename T, int D, bool EARLY, class IS>
__device__ __forceinline__ void expert_group(const Frag<T> (&qf)[IB][D / 32], const int (&qn)[IB], const T* Ks,
                                             const T* Vs, int Kp, int k, const Frag<T>& one, size_t row0,
                                             float2* __restrict__ plse, typename PartT<T>::type* __restrict__ po,
                                             T* __restrict__ O, TrainOut tr, int merge_in, int last, float cscale, int li,
                                             int lg, IS issue) {
  using RL = Resident<T, D>;
  using P = typename PartT<T>::type;
  using PV = typename Vec4<P>::type;
  RunMax M[IB];
  f32x4 Z[IB];
  f32x4 acc[IB][D / 16];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    M[b].set(M0, cscale);
    Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the stored part (none before the first routed slot of the routing-only
  // variant): (log2-sum-exp, scale) and the scaled row
  float2 plv[IB];
  PV hv[IB][D / 16];
  auto fetch = [&](int b) {
    plv[b] = make_float2(M0, 0.f);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) hv[b][cb] = PV{};
    if (merge_in && qn[b] >= 0) {
      const size_t qrow = row0 + qn[b];
      plv[b] = plse[qrow];
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) hv[b][cb] = *(const PV*)(po + qrow * D + part_pos<D>(lg, cb));
    }
  };
  if constexpr (EARLY) {
    // the query rows first: the loop needs them at once, and with their loads
    // still counted the compiler would wait for these ones inside the loop too
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int b = 0; b < IB; ++b) fetch(b);
  }
  issue();
  int x0 = 0;
  for (; x0 + 32 <= k; x0 += 32) {
    StepFrags<T, D> f;
    RL::frags(f, Ks, Vs, Kp, x0, li, lg);
    attn_step<IB, false>(f, one, qf, 32, lg, cscale, M, Z, acc, NoHook{});
  }
  if (x0 < k) {
    StepFrags<T, D> f;
    RL::frags(f, Ks, Vs, Kp, x0, li, lg);
    attn_step<IB, true>(f, one, qf, k - x0, lg, cscale, M, Z, acc, NoHook{});
  }
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const float Zt = finish_z(Z[b], li);
    if (qn[b] < 0) continue;
    const size_t qrow = row0 + qn[b];
    // merge with the stored part: weights 2^lse of the two parts; the stored
    // row comes back multiplied by its scale
    float2 pl;
    if constexpr (EARLY) pl = plv[b];
    else pl = merge_in ? plse[qrow] : make_float2(M0, 0.f);
    const float la = pl.x;
    const float lb = M[b].M + __builtin_amdgcn_logf(Zt);
    const float mx = fmaxf(la, lb);
    const float wa = __builtin_amdgcn_exp2f(la - mx), wb = __builtin_amdgcn_exp2f(lb - mx);
    const float den = wa + wb;
    const float ca = wa / den * pl.y, cb_ = wb / (den * Zt);
    P* o = po + qrow * D;
    f32x4 v[D / 16];
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      PV h = PV{};
      if constexpr (EARLY) h = hv[b][cb];
      else if (merge_in) h = *(const PV*)(o + part_pos<D>(lg, cb));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float hf = (float)h[r];
        // (converted on its own: folded into a mixed-precision multiply-add
        // the merge was not reproducible from run to run)
        if constexpr (EARLY) asm volatile("" : "+v"(hf));
        v[cb][r] = ca * hf + cb_ * acc[b][cb][r];
      }
    }
    // the log2-sum-exp of everything merged so far: the next slot's input,
    // or after the last slot the query's whole normaliser (kept for the
    // backward pass when requested)
    const float lse = mx + __builtin_amdgcn_logf(den);
    if (last) {
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        T* dst = O + qrow * D + cb * 16 + 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(v[cb][r]);
        if (tr.o32) *(float4*)(tr.o32 + qrow * D + cb * 16 + 4 * lg) = make_float4(v[cb][0], v[cb][1], v[cb][2], v[cb][3]);
      }
      if (lg == 0 && tr.lse) tr.lse[qrow] = lse;
    } else {
      float sn, scl;
      row_scale<P, D / 16>(v, 1.0f, sn, scl);
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        PV w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (P)(v[cb][r] * sn);
        *(PV*)(o + part_pos<D>(lg, cb)) = w;
      }
      if (lg == 0) plse[qrow] = make_float2(lse, scl);
    }
  }
}

template <int IBX, typename T, int D, bool EARLY, class QR>
__device__ __forceinline__ void expert_blocks(const T* Qh, QR qrow, const T* Ks, const T* Vs, int Kp, int k,
                                              const Frag<T>& one, size_t row0, float2* plse,
                                              typename PartT<T>::type* po, T* O, TrainOut tr, int merge_in, int last,
                                              float cscale, int li, int lg) {
  Frag<T> qf[IBX][D / 32];
  int qn[IBX];
  load_queries<T, D, IBX>(qf, Qh, lg, qrow);
#pragma unroll
  for (int b = 0; b < IBX; ++b) qn[b] = (int)qrow(b);
  expert_group<IBX, T, D, EARLY>(qf, qn, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg,
                                 [] {});
}

template <typename T, int D, int NW, int IB>
// (for bf16 sixteen waves of one 16-query block, four per SIMD, or twelve of
// two, three per SIMD with the registers to fetch the stored part early: one
// wave's dependency stalls are covered by the others)
__global__ __launch_bounds__(NW * 64, NW >= 16 ? 4 : NW >= 12 ? 3 : 2) void k_expert(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const int32_t* __restrict__ topk,
    const int32_t* __restrict__ perm, const WorkItem* __restrict__ wl, const int* __restrict__ wl_count,
    float2* __restrict__ plse, typename PartT<T>::type* __restrict__ po, T* __restrict__ O, TrainOut tr, int N, int m, int k,
    int merge_in, int last, float cscale) {
  using RL = Resident<T, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  // The list holds the largest items first; the hardware deals workgroups
  // to the XCDs in turn, which spreads them evenly.
  if ((int)blockIdx.x >= *wl_count) return;
  const WorkItem it = wl[blockIdx.x];
  const int Kp = RL::pad(k);
  T* Ks = (T*)smem;
  T* Vs = Ks + (size_t)Kp * RL::KS;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const Frag<T> one = ones_frag<T>(li);
  const int bh = it.be / m;
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;
  // the expert's key indices and the item's query indices, staged in LDS
  int* s_idx = (int*)(smem + RL::bytes(Kp));
  int* s_q = s_idx + Kp;
  const int32_t* Ie = topk + (size_t)it.be * k;
  for (int x = tid; x < k; x += NW * 64) s_idx[x] = Ie[x];
  for (int x = tid; x < it.count; x += NW * 64) s_q[x] = perm[it.start + x];
  __syncthreads();
  RL::load(Ks, Vs, k, Kp, [&](int x) { return Kh + (size_t)s_idx[x] * D; },
           [&](int x) { return Vh + (size_t)s_idx[x] * D; });
  __syncthreads();

  constexpr int GQ = 16 * IB;
  const T* Qh = Q + (size_t)bh * N * D;
  const size_t row0 = (size_t)bh * N;
  // whole rounds of full groups (one per wave) ...
  const int nfull = it.count / (NW * GQ) * NW;
  auto group_rows = [&](int gi) {
    return [=](int b) -> long long { return s_q[gi * GQ + b * 16 + li]; };
  };
  // the stored part is fetched before each group's key loop where the
  // registers allow (sixteen waves of one block, twelve of two: 0.44 -> 0.415
  // ms at N = 1M, 62 -> 60 us at 64K); the next group's query rows while the
  // current one computes (not with twelve waves of two blocks: no registers
  // for both, and the other waves of the SIMD cover the load)
  constexpr bool EARLY = NW >= 12;
  constexpr bool PREFETCH = !(NW == 12 && IB == 2);
  Frag<T> qnx[PREFETCH ? IB : 1][D / 32];
  if constexpr (PREFETCH)
    if (wave < nfull) load_queries<T, D, IB>(qnx, Qh, lg, group_rows(wave));
  for (int gi = wave; gi < nfull; gi += NW) {
    Frag<T> qf[IB][D / 32];
    int qn[IB];
    if constexpr (PREFETCH) {
#pragma unroll
      for (int b = 0; b < IB; ++b)
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) qf[b][dc] = qnx[b][dc];
    } else {
      load_queries<T, D, IB>(qf, Qh, lg, group_rows(gi));
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) qn[b] = s_q[gi * GQ + b * 16 + li];
    expert_group<IB, T, D, EARLY>(qf, qn, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg,
                                  [&] {
                                    if constexpr (PREFETCH)
                                      if (gi + NW < nfull) load_queries<T, D, IB>(qnx, Qh, lg, group_rows(gi + NW));
                                  });
  }
  // ... then the rest in blocks of 16 queries dealt to the waves in turn, so
  // a short remainder keeps every wave busy on narrower groups
  const int r0 = nfull * GQ;
  const int nblk = (it.count - r0 + 15) / 16;
  const int mine = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;  // at most IB
  auto rem_rows = [&](int b) -> long long {
    const int l = r0 + (wave + b * NW) * 16 + li;
    return l < it.count ? s_q[l] : -1;
  };
  if constexpr (IB >= 4) {
    if (mine == 4) expert_blocks<4, T, D, EARLY>(Qh, rem_rows, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg);
    if (mine == 3) expert_blocks<3, T, D, EARLY>(Qh, rem_rows, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg);
  }
  if constexpr (IB >= 2) {
    if (mine == 2) expert_blocks<2, T, D, EARLY>(Qh, rem_rows, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg);
  }
  if (mine == 1) expert_blocks<1, T, D, EARLY>(Qh, rem_rows, Ks, Vs, Kp, k, one, row0, plse, po, O, tr, merge_in, last, cscale, li, lg);
}

// ---------------------------------------------------------------------------
size_t resident_bytes(int dtype, int d, int E) {
  const int Ep = (E + 31) / 32 * 32;
  if (dtype == 1) return d == 64 ? Resident<__bf16, 64>::bytes(Ep) : Resident<__bf16, 32>::bytes(Ep);
  return d == 64 ? Resident<float, 64>::bytes(Ep) : Resident<float, 32>::bytes(Ep);
}

template <typename T, int D, int SMAX, int NW, int IB>
static void launch_route_shared_t(const Plan& p) {
  const int hist_lds = (p.s * p.m <= 4096) ? 1 : 0;
  const size_t lds = resident_bytes(p.dtype, D, p.m) + (hist_lds ? (size_t)p.s * p.m * 4 : 0);
  auto fn = &k_route_shared<T, D, NW, SMAX, IB>;
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  dim3 grid((unsigned)((p.N + p.rs_qpw - 1) / p.rs_qpw), (unsigned)p.BH);
  hipLaunchKernelGGL(fn, grid, dim3(NW * 64), lds, p.stream, (const T*)p.Q, (const T*)p.qt, (const T*)p.vtT, p.route,
                     p.counts, p.plse, (typename PartT<T>::type*)p.po, p.N, p.m, p.s, p.BH, p.rs_qpw, hist_lds, p.cscale_sh);
}

template <typename T, int D>
static void launch_route_shared_d(const Plan& p) {
  if (p.rs_nw == 12) {  // (top-1 routing only)
    launch_route_shared_t<T, D, 1, 12, 2>(p);
    return;
  }
  if (p.rs_nw == 16) {
    switch (p.smax) {
      case 1: launch_route_shared_t<T, D, 1, 16, 1>(p); break;
      case 2: launch_route_shared_t<T, D, 2, 16, 1>(p); break;
      case 4: launch_route_shared_t<T, D, 4, 16, 1>(p); break;
      default: launch_route_shared_t<T, D, 8, 16, 1>(p); break;
    }
    return;
  }
  switch (p.smax) {
    case 1: launch_route_shared_t<T, D, 1, 8, 4>(p); break;
    case 2: launch_route_shared_t<T, D, 2, 8, 4>(p); break;
    case 4: launch_route_shared_t<T, D, 4, 8, 4>(p); break;
    default: launch_route_shared_t<T, D, 8, 8, 4>(p); break;
  }
}

void launch_route_shared(const Plan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_route_shared_d<float, 32>(p); else launch_route_shared_d<float, 64>(p);
  } else {
    if (p.d == 32) launch_route_shared_d<__bf16, 32>(p); else launch_route_shared_d<__bf16, 64>(p);
  }
}

template <typename T, int D, int NW, int IB>
static void launch_expert_t(const Plan& p) {
  const int Kp = (p.k + 31) / 32 * 32;
  const size_t lds = resident_bytes(p.dtype, D, p.k) + (size_t)(Kp + p.T) * 4;
  auto fn = &k_expert<T, D, NW, IB>;
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  for (int t = 0; t < p.s; ++t) {
    const int32_t* perm = p.perm + (size_t)t * p.BH * p.N;
    const WorkItem* wl = p.wl + (size_t)t * p.UB;
    hipLaunchKernelGGL(fn, dim3((unsigned)(p.UB + 8)), dim3(NW * 64), lds, p.stream, (const T*)p.Q, (const T*)p.K,
                       (const T*)p.V, p.topk, perm, wl, p.wl_count + t, p.plse, (typename PartT<T>::type*)p.po, (T*)p.O, TrainOut{p.lse_out, p.o32}, p.N, p.m, p.k,
                       (t > 0 || p.shared) ? 1 : 0, t == p.s - 1 ? 1 : 0, p.cscale);
  }
}

template <typename T, int D>
static void launch_expert_d(const Plan& p) {
  if (p.ex_nw == 1 && p.ex_ib == 1) launch_expert_t<T, D, 1, 1>(p);
  else if (p.ex_nw == 1) launch_expert_t<T, D, 1, 2>(p);
  else if (p.ex_nw == 4) launch_expert_t<T, D, 4, 4>(p);
  else if (p.ex_ib == 1) launch_expert_t<T, D, 16, 1>(p);
  else launch_expert_t<T, D, 12, 2>(p);
}

void launch_expert(const Plan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_expert_t<float, 32, 1, 1>(p); else launch_expert_t<float, 64, 1, 1>(p);
  } else {
    if (p.d == 32) launch_expert_d<__bf16, 32>(p); else launch_expert_d<__bf16, 64>(p);
  }
}

}  // namespace mita
