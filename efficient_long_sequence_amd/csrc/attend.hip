// Step 6 of MiTA: one joint softmax per query over the m shared entries
// (q~_i, v~_i) and the s*k raw entries of its chosen experts (MiTA tutorial
// (iwxt.cn), ch.4 steps 5-6 and V* = [V~, V^(e1), ..., V^(es)]; shared and
// routed entries compete for one total weight).
//
// One workgroup per work item (expert e of head bh, a tile of up to T of the
// queries routed to e).  The workgroup streams the entry list
// [q~_1..q~_m, k_j for j in I_e] (values [v~_1..v~_m, v_j]) through LDS 32
// entries at a time; keys and values of the expert are gathered rows of K and
// V.  Every wave owns 16*IB queries as matrix-core columns, so each staged
// entry is reused by all queries of the tile.  The softmax is online in fp32:
// running maximum, normaliser and unnormalised output per query.
//
// With s >= 2 a query is visited once per slot.  Slots 1..s-1 cover only
// their expert's k entries and store (max, normaliser, unnormalised output);
// the slot-0 pass, launched last, adds the m shared entries and its own
// expert, merges the stored parts with the rescaled-sum identity
// (Z1 o1 + Z2 o2) / (Z1 + Z2) (tutorial ch.4) and writes O.  Keys shared by
// two chosen experts are therefore counted twice, as the entry count m + s k
// requires.
#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

template <typename T, int D, int NW, int IB, bool SLOT0>
__global__ __launch_bounds__(NW * 64) void k_attend(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ Qt,
    const T* __restrict__ VtT, const int32_t* __restrict__ topk, const int32_t* __restrict__ perm,
    const WorkItem* __restrict__ wl, const int* __restrict__ wl_count, float* __restrict__ part,
    T* __restrict__ O, float* __restrict__ lse_out, float* __restrict__ o32, int N, int m, int k, int s, int slot, int BH, int m_shared,
    float cscale, float cscale_sh) {
  constexpr int NT = NW * 64;
  using TL = TileLayout<T, D>;
  __shared__ __align__(16) T smem[2 * TL::ELEMS];
  extern __shared__ __align__(16) int32_t s_idx[];  // the expert's k key indices (dynamic LDS)
  if ((int)blockIdx.x >= *wl_count) return;
  const WorkItem it = wl[blockIdx.x];
  const int bh = it.be / m;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const Frag<T> one = ones_frag<T>(li);
  const T* Kh = K + (size_t)bh * N * D;
  const T* Vh = V + (size_t)bh * N * D;
  const T* Qth = Qt + (size_t)bh * m * D;
  const T* Vth = VtT + (size_t)bh * m * D;
  const int32_t* Ie = topk + (size_t)it.be * k;

  Frag<T> qf[IB][D / 32];
  int qn[IB];
  RunMax M[IB];
  f32x4 Z[IB];
  f32x4 acc[IB][D / 16];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int local = wave * 16 * IB + b * 16 + li;
    qn[b] = local < it.count ? perm[it.start + local] : -1;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (qn[b] >= 0) load8(qf[b][dc], Q + ((size_t)bh * N + qn[b]) * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
    M[b].set(M0, cscale_sh);
    Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // shared entries first (slot 0 only; none in the routing-only variant),
  // then the expert's entries from a
  // fresh step, so every step has one logit scale (the shared logits may be
  // scaled differently, see mita_forward_variant)
  const int m0 = SLOT0 ? m_shared : 0;
  const int ns = (m0 + 31) / 32, nsteps = ns + (k + 31) / 32;
  auto rowK = [&](int st) {
    return [=](int r) -> const T* {
      if (st < ns) { const int x = st * 32 + r; return x < m0 ? Qth + (size_t)x * D : nullptr; }
      const int x = (st - ns) * 32 + r;
      return x < k ? Kh + (size_t)s_idx[x] * D : nullptr;
    };
  };
  auto rowV = [&](int st) {
    return [=](int r) -> const T* {
      if (st < ns) { const int x = st * 32 + r; return x < m0 ? Vth + (size_t)x * D : nullptr; }
      const int x = (st - ns) * 32 + r;
      return x < k ? Vh + (size_t)s_idx[x] * D : nullptr;
    };
  };

  // the expert's indices go to LDS first, so a staged row's address does not
  // wait on a global load of its index (the clamp only keeps other contents
  // in bounds)
  for (int x = tid; x < k; x += NT) s_idx[x] = min(max(Ie[x], 0), N - 1);
  __syncthreads();

  TileLoader<T, D, NT, true> ld;
  T* buf0 = smem;
  T* buf1 = smem + TL::ELEMS;
  ld.load(rowK(0), rowV(0));
  ld.store(buf0, buf0 + TL::K_ELEMS);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    T* cur = (st & 1) ? buf1 : buf0;
    T* nxt = (st & 1) ? buf0 : buf1;
    const bool more = st + 1 < nsteps;
    if (more) ld.load(rowK(st + 1), rowV(st + 1));
    StepFrags<T, D> f;
    f.load_keys(cur, li, lg);
    f.load_vals(cur + TL::K_ELEMS, li, lg);
    const int nv = st < ns ? min(32, m0 - st * 32) : min(32, k - (st - ns) * 32);
    const float sc = st < ns ? cscale_sh : cscale;
    if (st == ns && ns > 0) {  // the logit scale may change with the routed entries
#pragma unroll
      for (int b = 0; b < IB; ++b) M[b].set(M[b].M, cscale);
    }
    if (nv == 32) attn_step<IB, false>(f, one, qf, nv, lg, sc, M, Z, acc, NoHook{});
    else attn_step<IB, true>(f, one, qf, nv, lg, sc, M, Z, acc, NoHook{});
    if (more) ld.store(nxt, nxt + TL::K_ELEMS);
    __syncthreads();
  }

#pragma unroll
  for (int b = 0; b < IB; ++b) {
    float Zt = finish_z(Z[b], li);
    if (qn[b] < 0) continue;
    const size_t qrow = (size_t)bh * N + qn[b];
    if constexpr (!SLOT0) {
      float* dst = part + ((size_t)(slot - 1) * BH * N + qrow) * (D + 4);
      if (lg == 0) { dst[0] = M[b].M; dst[1] = Zt; }
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
        *(float4*)(dst + 4 + cb * 16 + 4 * lg) = make_float4(acc[b][cb][0], acc[b][cb][1], acc[b][cb][2], acc[b][cb][3]);
    } else {
      float Mx = M[b].M;
      for (int t = 1; t < s; ++t) {
        const float* src = part + ((size_t)(t - 1) * BH * N + qrow) * (D + 4);
        const float Mt = src[0], Zp = src[1];
        const float nM = fmaxf(Mx, Mt);
        const float w0 = __builtin_amdgcn_exp2f(Mx - nM), w1 = __builtin_amdgcn_exp2f(Mt - nM);
        Zt = Zt * w0 + Zp * w1;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
          const float4 o = *(const float4*)(src + 4 + cb * 16 + 4 * lg);
          acc[b][cb][0] = acc[b][cb][0] * w0 + o.x * w1;
          acc[b][cb][1] = acc[b][cb][1] * w0 + o.y * w1;
          acc[b][cb][2] = acc[b][cb][2] * w0 + o.z * w1;
          acc[b][cb][3] = acc[b][cb][3] * w0 + o.w * w1;
        }
        Mx = nM;
      }
      if (lse_out && lg == 0) lse_out[qrow] = Mx + __builtin_amdgcn_logf(Zt);  // kept for the backward pass
      const float inv = 1.0f / Zt;
      T* dst = O + qrow * D;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[cb * 16 + 4 * lg + r] = from_f32<T>(acc[b][cb][r] * inv);
      if (o32)
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
          *(float4*)(o32 + qrow * D + cb * 16 + 4 * lg) =
              make_float4(acc[b][cb][0] * inv, acc[b][cb][1] * inv, acc[b][cb][2] * inv, acc[b][cb][3] * inv);
    }
  }
}

template <typename T, int D, int NW, int IB>
static void launch_attend_t(const Plan& p) {
  const size_t dyn = (size_t)p.k * 4, stat = 2 * TileLayout<T, D>::ELEMS * sizeof(T);
  if (stat + dyn > 65536) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attend<T, D, NW, IB, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attend<T, D, NW, IB, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
  }
  for (int t = p.s - 1; t >= 0; --t) {
    const int32_t* perm = p.perm + (size_t)t * p.BH * p.N;
    const WorkItem* wl = p.wl + (size_t)t * p.UB;
    const int* wlc = p.wl_count + t;
    if (t > 0)
      hipLaunchKernelGGL((k_attend<T, D, NW, IB, false>), dim3((unsigned)p.UB), dim3(NW * 64), dyn, p.stream,
                         (const T*)p.Q, (const T*)p.K, (const T*)p.V, (const T*)p.qt, (const T*)p.vtT, p.topk, perm,
                         wl, wlc, p.part, (T*)p.O, p.lse_out, p.o32, p.N, p.m, p.k, p.s, t, p.BH, p.shared ? p.m : 0, p.cscale, p.cscale_sh);
    else
      hipLaunchKernelGGL((k_attend<T, D, NW, IB, true>), dim3((unsigned)p.UB), dim3(NW * 64), dyn, p.stream,
                         (const T*)p.Q, (const T*)p.K, (const T*)p.V, (const T*)p.qt, (const T*)p.vtT, p.topk, perm,
                         wl, wlc, p.part, (T*)p.O, p.lse_out, p.o32, p.N, p.m, p.k, p.s, t, p.BH, p.shared ? p.m : 0, p.cscale, p.cscale_sh);
  }
}

template <typename T, int D>
static void launch_attend_d(const Plan& p) {
  if (p.at_nw == 1) launch_attend_t<T, D, 1, 1>(p);
  else if (p.at_ib == 1) launch_attend_t<T, D, 4, 1>(p);
  else if (p.at_nw == 4) launch_attend_t<T, D, 4, 4>(p);
  else launch_attend_t<T, D, 8, 4>(p);
}

void launch_attend(const Plan& p) {
  if (p.dtype == 0) {
    if (p.d == 32) launch_attend_t<float, 32, 1, 1>(p); else launch_attend_t<float, 64, 1, 1>(p);
  } else {
    if (p.d == 32) launch_attend_d<__bf16, 32>(p); else launch_attend_d<__bf16, 64>(p);
  }
}

}  // namespace mita
