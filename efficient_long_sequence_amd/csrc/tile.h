// A 32-row step of keys (and values) staged in LDS for the matrix cores.
//
// Keys are stored row-major, Ks[j][c] with a padded row stride KS, which is
// the A-operand order of the score product (key rows, d along K).  The
// product O^T = V^T P^T needs the values transposed (d rows, keys along K):
// bf16 values are stored row-major too, with row stride VSR, and read
// transposed by the LDS transpose read (tr_frag), so key and value rows are
// staged alike, one 16-byte chunk per thread and step; fp32 values are
// stored transposed, Vs[c][j] with row stride VS.  Each thread first pulls
// its chunks of the step into registers (so the global loads of step i+1
// overlap the matrix work of step i) and then writes them to LDS.  (A key
// row stride of 72 elements keeps the row-wise key reads free of LDS bank
// conflicts and a value row stride of 80 the transposed value reads, with
// 32 or 64 banks of 4 bytes alike.)
#pragma once
#include "mita_dev.h"

namespace mita {

template <typename T, int D>
struct TileLayout {
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16 bytes
  static constexpr int KS = D + EPC;   // padded key row (elements); 16-byte aligned rows
  static constexpr int VS = 36;        // padded V^T row (elements); 8-byte (bf16) / 16-byte (f32) aligned
  // bf16: value rows are staged as they come, padded to VSR elements, and
  // read transposed (ds_read_b64_tr_b16)
  static constexpr bool ROWV = sizeof(T) == 2;
  static constexpr int VSR = D + 16;
  static constexpr int K_ELEMS = 32 * KS;
  static constexpr int V_ELEMS = ROWV ? 32 * VSR : D * VS;
  static constexpr int ELEMS = K_ELEMS + V_ELEMS;
};

template <typename T, int D, int NT, bool WITH_V>
struct TileLoader {
  using L = TileLayout<T, D>;
  static constexpr int EPC = L::EPC;
  static constexpr int CPR = D / EPC;  // 16-byte chunks per row
  static constexpr int KCH = 32 * CPR;
  // bf16 with values: key and value rows alike, 2 KCH chunks over the block
  // (with 512 threads, one each: the first half keys, the second values)
  static constexpr bool ROWV = WITH_V && sizeof(T) == 2;
  static constexpr int TCH = ROWV ? 2 * KCH : KCH;
  static constexpr int RPT = (TCH + NT - 1) / NT;
  // fp32 with values: the value transpose, one row chunk per task
  static constexpr bool TRV = WITH_V && !ROWV;
  static constexpr int VPT = TRV ? (KCH + NT - 1) / NT : 0;

  uint4 rreg[RPT];
  uint4 vreg[VPT > 0 ? VPT : 1];

  // rk(j) / rv(j): pointer to key / value row j of the step, or nullptr for a
  // row past the end (it is staged as zeros).
  template <class RK, class RV>
  __device__ __forceinline__ void load(RK rk, RV rv) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < RPT; ++c) {
      const int i = tid + c * NT;
      rreg[c] = make_uint4(0, 0, 0, 0);
      if (i < TCH) {
        const int ii = i < KCH ? i : i - KCH;
        const T* p = i < KCH ? rk(ii / CPR) : rv(ii / CPR);
        if (p) rreg[c] = *(const uint4*)(p + (ii % CPR) * EPC);
      }
    }
    if constexpr (TRV) {
#pragma unroll
      for (int c = 0; c < VPT; ++c) {
        const int i = tid + c * NT;
        vreg[c] = make_uint4(0, 0, 0, 0);
        if (i < KCH) {
          const T* p = rv(i / CPR);
          if (p) vreg[c] = *(const uint4*)(p + (i % CPR) * EPC);
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* Ks, T* Vs) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < RPT; ++c) {
      const int i = tid + c * NT;
      if (i < TCH) {
        const int ii = i < KCH ? i : i - KCH;
        T* dst = i < KCH ? Ks + (ii / CPR) * L::KS : Vs + (ii / CPR) * L::VSR;
        *(uint4*)(dst + (ii % CPR) * EPC) = rreg[c];
      }
    }
    if constexpr (TRV) {
#pragma unroll
      for (int c = 0; c < VPT; ++c) {
        const int i = tid + c * NT;
        if (i < KCH) {
          const int j = i / CPR, c0 = (i % CPR) * EPC;
          const float* a = (const float*)&vreg[c];
#pragma unroll
          for (int u = 0; u < 4; ++u) Vs[(c0 + u) * L::VS + j] = a[u];
        }
      }
    }
  }
};

// The V^T-order operand of one 16-column block `cb` for the 32 rows x0 ..
// x0+31 of a row-major bf16 tile (row stride KS), in the slot permutation of
// the score layout (slot t < 4: row x0 + 4g + t; t >= 4: row x0 + 16 + 4g +
// t - 4), read with the LDS transpose read ds_read_b64_tr_b16: in each
// 16-lane group, lane i receives element i mod 4 of the 8-byte words supplied
// by lanes i/4 + 4t (t = 0..3); lane j supplies row x0 + 4g + j/4, columns
// 16 cb + 4 (j mod 4) .. + 3, so lane (li, g) receives column 16 cb + li of
// the four rows of its slots.  The two results are joined as whole vectors.
typedef short tr_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void tr_frag(Frag<__bf16>& f, const __bf16* rows, int KS, int x0, int cb, int lane16,
                                        int g) {
  const int r = lane16 / 4, c = cb * 16 + 4 * (lane16 % 4);
  const tr_v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr_v4s*)(rows + (size_t)(x0 + 4 * g + r) * KS + c));
  const tr_v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr_v4s*)(rows + (size_t)(x0 + 16 + 4 * g + r) * KS + c));
  const bf16x4 a4 = __builtin_bit_cast(bf16x4, a), b4 = __builtin_bit_cast(bf16x4, b);
  f.v = __builtin_shufflevector(a4, b4, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void tr_frag(Frag<float>&, const float*, int, int, int, int, int) {}

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
    if constexpr (TileLayout<T, D>::ROWV) {
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) tr_frag(va[cb], Vs, TileLayout<T, D>::VSR, 0, cb, li, g);
    } else {
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        const T* row = Vs + (cb * 16 + li) * TileLayout<T, D>::VS;
        load4x2(va[cb], row + 4 * g, row + 16 + 4 * g);
      }
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
