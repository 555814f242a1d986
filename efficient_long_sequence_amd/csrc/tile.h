// A 32-row step of keys (and values) staged in LDS for the matrix cores.
//
// Keys are stored row-major, Ks[j][c] with a padded row stride KS, which is
// the A-operand order of the score product (key rows, d along K).  Values are
// stored transposed, Vs[c][j] with row stride VS, which is the A-operand
// order of O^T = V^T P^T (d rows, keys along K).  Each thread first pulls its
// 16-byte chunks of the step into registers (so the global loads of step
// i+1 overlap the matrix work of step i) and then writes them to LDS; the
// transposing write packs two key rows per 32-bit word for bf16.
#pragma once
#include "mita_dev.h"

namespace mita {

template <typename T, int D>
struct TileLayout {
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16 bytes
  static constexpr int KS = D + EPC;   // padded key row (elements); 16-byte aligned rows
  static constexpr int VS = 36;        // padded V^T row (elements); 8-byte (bf16) / 16-byte (f32) aligned
  static constexpr int K_ELEMS = 32 * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int ELEMS = K_ELEMS + V_ELEMS;
};

template <typename T, int D, int NT, bool WITH_V>
struct TileLoader {
  using L = TileLayout<T, D>;
  static constexpr int EPC = L::EPC;
  static constexpr int CPR = D / EPC;                  // 16-byte chunks per row
  static constexpr int KCH = 32 * CPR;
  static constexpr int KPT = (KCH + NT - 1) / NT;
  static constexpr int VROWS = sizeof(T) == 2 ? 2 : 1;  // rows per transposing task
  static constexpr int VCH = WITH_V ? (32 / VROWS) * CPR : 0;
  static constexpr int VPT = WITH_V ? (VCH + NT - 1) / NT : 0;
  static constexpr int VS = L::VS;
  // Split placement (bf16, when the block has room): key chunks go to the
  // first threads and the value transpose, in tasks of two rows by four
  // elements, to the last ones.  A SIMD runs waves w and w + NT/256 of the
  // block, so each SIMD then carries one key-loading and one value-loading
  // wave and the per-step barrier waits less for the slowest.
  static constexpr int VFINE = WITH_V ? 16 * (D / 4) : 0;
  static constexpr bool SPLIT = WITH_V && sizeof(T) == 2 && KCH + VFINE <= NT;

  uint4 kreg[KPT];
  uint4 vreg[SPLIT ? 1 : (VPT > 0 ? VPT : 1)][SPLIT ? 1 : VROWS];
  uint2 vfine[SPLIT ? 2 : 1];

  // rk(j) / rv(j): pointer to key / value row j of the step, or nullptr for a
  // row past the end (it is staged as zeros).
  template <class RK, class RV>
  __device__ __forceinline__ void load(RK rk, RV rv) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int i = tid + c * NT;
      kreg[c] = make_uint4(0, 0, 0, 0);
      if (i < KCH) {
        const T* p = rk(i / CPR);
        if (p) kreg[c] = *(const uint4*)(p + (i % CPR) * EPC);
      }
    }
    if constexpr (SPLIT) {
      const int i = tid - (NT - VFINE);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        vfine[r] = make_uint2(0, 0);
        if (i >= 0) {
          const T* p = rv(2 * (i / (D / 4)) + r);
          if (p) vfine[r] = *(const uint2*)(p + (i % (D / 4)) * 4);
        }
      }
    } else if constexpr (WITH_V) {
#pragma unroll
      for (int c = 0; c < VPT; ++c) {
        const int i = tid + c * NT;
#pragma unroll
        for (int r = 0; r < VROWS; ++r) {
          vreg[c][r] = make_uint4(0, 0, 0, 0);
          if (i < VCH) {
            const T* p = rv((i / CPR) * VROWS + r);
            if (p) vreg[c][r] = *(const uint4*)(p + (i % CPR) * EPC);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* Ks, T* Vs) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int i = tid + c * NT;
      if (i < KCH) *(uint4*)(Ks + (i / CPR) * L::KS + (i % CPR) * EPC) = kreg[c];
    }
    if constexpr (SPLIT) {
      const int i = tid - (NT - VFINE);
      if (i >= 0) {
        const int jp = i / (D / 4), c0 = (i % (D / 4)) * 4;
        const uint32_t* a = (const uint32_t*)&vfine[0];
        const uint32_t* b = (const uint32_t*)&vfine[1];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          // elements 2u, 2u+1 of rows 2jp (a) and 2jp+1 (b)
          *(uint32_t*)(Vs + (c0 + 2 * u) * VS + 2 * jp) = (a[u] & 0xFFFFu) | (b[u] << 16);
          *(uint32_t*)(Vs + (c0 + 2 * u + 1) * VS + 2 * jp) = (a[u] >> 16) | (b[u] & 0xFFFF0000u);
        }
      }
    } else if constexpr (WITH_V) {
#pragma unroll
      for (int c = 0; c < VPT; ++c) {
        const int i = tid + c * NT;
        if (i < VCH) {
          const int jp = i / CPR, c0 = (i % CPR) * EPC;
          if constexpr (sizeof(T) == 2) {
            const uint32_t* a = (const uint32_t*)&vreg[c][0];
            const uint32_t* b = (const uint32_t*)&vreg[c][1];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              // elements 2u, 2u+1 of rows 2jp (a) and 2jp+1 (b)
              const uint32_t lo = (a[u] & 0xFFFFu) | (b[u] << 16);
              const uint32_t hi = (a[u] >> 16) | (b[u] & 0xFFFF0000u);
              *(uint32_t*)(Vs + (c0 + 2 * u) * VS + 2 * jp) = lo;
              *(uint32_t*)(Vs + (c0 + 2 * u + 1) * VS + 2 * jp) = hi;
            }
          } else {
            const float* a = (const float*)&vreg[c][0];
#pragma unroll
            for (int u = 0; u < 4; ++u) Vs[(c0 + u) * VS + jp] = a[u];
          }
        }
      }
    }
  }
};

// Per-lane key slot -> key offset inside a 32-key step.
__device__ __forceinline__ int slot_key(int t, int g) { return t < 4 ? 4 * g + t : 16 + 4 * g + (t - 4); }

// A operands of one step for a wave: keys (2 tiles of 16 x D) and V^T.
template <typename T, int D>
struct StepFrags {
  Frag<T> ka[2][D / 32];
  Frag<T> va[D / 16];
  __device__ __forceinline__ void load_keys(const T* Ks, int li, int g) {
    using L = TileLayout<T, D>;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int dc = 0; dc < D / 32; ++dc) load8(ka[jt][dc], Ks + (jt * 16 + li) * L::KS + dc * 32 + 8 * g);
  }
  __device__ __forceinline__ void load_vals(const T* Vs, int li, int g) {
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const T* row = Vs + (cb * 16 + li) * TileLayout<T, D>::VS;
      load4x2(va[cb], row + 4 * g, row + 16 + 4 * g);
    }
  }
};

// Scores of one 16-query block against the 32 keys of the step: 8 per lane.
template <typename T, int D>
__device__ __forceinline__ void step_scores(const StepFrags<T, D>& f, const Frag<T>* qf, float* sc) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc) {
    mma16(s0, f.ka[0][dc], qf[dc]);
    mma16(s1, f.ka[1][dc], qf[dc]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) { sc[r] = s0[r]; sc[4 + r] = s1[r]; }
}

// A-operand block whose first row is all ones: multiplied with the
// probability fragment it yields the softmax normaliser on the matrix cores
// (row 0 of the output tile, i.e. element 0 in lane group 0), summing the
// same rounded probabilities the P.V product uses.
template <typename T>
__device__ __forceinline__ Frag<T> ones_frag(int li) {
  Frag<T> f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = (T)(li == 0 ? 1.0f : 0.0f);
  return f;
}
// The normaliser of query li (held by lane li of group 0), in every lane.
__device__ __forceinline__ float finish_z(const f32x4& Z, int li) { return __shfl(Z[0], li); }

// Running maximum of one 16-query block: M in the scaled log2 domain
// (identical in the four lane groups of a query) and Mt = (M + THRESH) /
// cscale, the raw score above which the maximum is raised, so the common
// step compares raw lane maxima with no scaling.
struct RunMax {
  float M, Mt;
  __device__ __forceinline__ void set(float m, float cscale) {
    M = m;
    Mt = (m + THRESH) / cscale;
  }
};

// Online-softmax update of one 16-query block with the 8 raw scores of this
// lane (already -inf where masked) and their maximum mx_raw.  Z is the
// normaliser tile (see ones_frag), acc the O^T accumulator.
template <typename T, int D>
__device__ __forceinline__ void softmax_step(const StepFrags<T, D>& f, const Frag<T>& one, const float* sc,
                                             float mx_raw, float cscale, RunMax& R, f32x4& Z, f32x4* acc) {
  if (wave_any(mx_raw > R.Mt)) {
    // The decision uses the query's own maximum over its four lane groups
    // with the same comparison, so each query's running maximum (and every
    // rounding that follows from it) is independent of which other queries
    // share the wave.
    const float gm = wave_max_groups(mx_raw);
    if (gm > R.Mt) {
      const float nm = gm * cscale;
      const float alpha = __builtin_amdgcn_exp2f(R.M - nm);
      Z[0] *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[cb][r] *= alpha;
      R.set(nm, cscale);
    }
  }
  const float nm = -R.M;
  float p[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t], cscale, nm));
  Frag<T> pf;
  set8(pf, p);
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) mma16(acc[cb], f.va[cb], pf);
  mma16(Z, one, pf);
}

// chained so the compiler forms three-input maxima (v_max3_f32)
__device__ __forceinline__ float max8(const float* s) {
  float m = fmaxf(fmaxf(s[0], s[1]), s[2]);
  m = fmaxf(fmaxf(m, s[3]), s[4]);
  m = fmaxf(fmaxf(m, s[5]), s[6]);
  return fmaxf(m, s[7]);
}

// The two halves of one 32-entry step for IB blocks of 16 queries.
// attn_scores: the score tiles of all blocks on the matrix cores.
template <int IB, typename T, int D>
__device__ __forceinline__ void attn_scores(const StepFrags<T, D>& f, const Frag<T> (&qf)[IB][D / 32],
                                            float (&sc)[IB][8]) {
#pragma unroll
  for (int b = 0; b < IB; ++b) step_scores(f, qf[b], sc[b]);
}

// attn_finish: the hook `on(b, scores, lane_max)` of each block
// (candidates, routing), then one check of every block's running maximum (a
// single, rarely taken branch), and last the exponentials and P.V of all
// blocks as one branch-free stretch.  MASK marks the last, partial step:
// entries at offsets >= nv get score -inf.
template <int IB, bool MASK, typename T, int D, class On>
__device__ __forceinline__ void attn_finish(const StepFrags<T, D>& f, const Frag<T>& one, float (&sc)[IB][8], int nv,
                                            int lg, float cscale, RunMax (&M)[IB], f32x4 (&Z)[IB],
                                            f32x4 (&acc)[IB][D / 16], On on) {
  if constexpr (MASK) {
#pragma unroll
    for (int b = 0; b < IB; ++b)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (slot_key(t, lg) >= nv) sc[b][t] = -INFINITY;
  }
  float mx[IB];
  bool up = false;
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    mx[b] = max8(sc[b]);
    on(b, sc[b], mx[b]);
    up |= mx[b] > M[b].Mt;
  }
  if (wave_any(up)) {
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      // the query's own maximum over its four lane groups decides, so each
      // query's running maximum is independent of the others in the wave
      const float gm = wave_max_groups(mx[b]);
      if (gm > M[b].Mt) {
        const float nm = gm * cscale;
        const float alpha = __builtin_amdgcn_exp2f(M[b].M - nm);
        Z[b][0] *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[b][cb][r] *= alpha;
        M[b].set(nm, cscale);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const float nm = -M[b].M;
    float p[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][t], cscale, nm));
    Frag<T> pf;
    set8(pf, p);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) mma16(acc[b][cb], f.va[cb], pf);
    mma16(Z[b], one, pf);
  }
}

// One whole 32-entry step: the score tiles of all blocks first, then
// attn_finish, so the scheduler can overlap one block's vector work with
// another's matrix work.
template <int IB, bool MASK, typename T, int D, class On>
__device__ __forceinline__ void attn_step(const StepFrags<T, D>& f, const Frag<T>& one,
                                          const Frag<T> (&qf)[IB][D / 32], int nv, int lg, float cscale,
                                          RunMax (&M)[IB], f32x4 (&Z)[IB], f32x4 (&acc)[IB][D / 16], On on) {
  float sc[IB][8];
  attn_scores<IB>(f, qf, sc);
  attn_finish<IB, MASK>(f, one, sc, nv, lg, cscale, M, Z, acc, on);
}

struct NoHook {
  __device__ __forceinline__ void operator()(int, const float*, float) const {}
};

// Scores of one 32-entry step for IB blocks and the hook on(b, scores,
// lane_max), with no softmax (keys only; the step's value operands are not
// needed).  MASK as for attn_step.
template <int IB, bool MASK, typename T, int D, class On>
__device__ __forceinline__ void score_step(const StepFrags<T, D>& f, const Frag<T> (&qf)[IB][D / 32], int nv,
                                           int lg, On on) {
  float sc[IB][8];
#pragma unroll
  for (int b = 0; b < IB; ++b) step_scores(f, qf[b], sc[b]);
  if constexpr (MASK) {
#pragma unroll
    for (int b = 0; b < IB; ++b)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (slot_key(t, lg) >= nv) sc[b][t] = -INFINITY;
  }
#pragma unroll
  for (int b = 0; b < IB; ++b) on(b, sc[b], max8(sc[b]));
}

}  // namespace mita
