// Device-side building blocks shared by the MiTA kernels (gfx950 only).
//
// Matrix-core conventions.  All contractions use the 16x16 output tile of
// v_mfma_f32_16x16x32_bf16 (bf16 inputs) or eight v_mfma_f32_16x16x4_f32
// (fp32 inputs) over a 32-wide K chunk.  In a wave of 64 lanes, lane l has
// column c = l % 16 and group g = l / 16:
//   A operand  row  l%16, K elements 8g .. 8g+7   (one Frag per lane)
//   B operand  col  l%16, K elements 8g .. 8g+7
//   D (4 fp32) col  l%16, rows 4g .. 4g+3
// Scores are produced transposed (keys as rows, queries as columns), so a
// lane owns one query and eight keys of a 32-key step; the probability
// fragment then feeds the P.V product directly as the B operand of
// O^T = V^T P^T, and the O^T accumulator keeps each query in one lane column.
// The permutation of the 32 keys inside a step (slot t < 4 -> key 4g+t,
// t >= 4 -> key 16+4g+t-4) is applied identically to P and to V^T, so it
// cancels in the sum.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Large negative start value for running maxima: exp2(x - M0) underflows to
// 0 for every finite x we meet, and M0 - M stays finite (unlike -inf - -inf).
constexpr float M0 = -1.0e30f;
// A running maximum is only raised when a score exceeds it by more than this
// many binades; until then probabilities may reach 2^THRESH, which fp32 and
// bf16 hold without overflow.
constexpr float THRESH = 8.0f;

// A compile-time flag passed as a value (selects a template form in a generic lambda).
template <bool B> struct BoolTag { static constexpr bool value = B; };

template <typename T> struct Frag;
template <> struct Frag<__bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma16(f32x4& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], acc, 0, 0, 0);
}

// 8 consecutive elements.
__device__ __forceinline__ void load8(Frag<__bf16>& f, const __bf16* p) { f.v = *(const bf16x8*)p; }
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
  float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// Two runs of 4 consecutive elements (slots 0-3 and 4-7).
__device__ __forceinline__ void load4x2(Frag<__bf16>& f, const __bf16* p0, const __bf16* p1) {
  bf16x4 a = *(const bf16x4*)p0, b = *(const bf16x4*)p1;
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void load4x2(Frag<float>& f, const float* p0, const float* p1) {
  float4 a = *(const float4*)p0, b = *(const float4*)p1;
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
template <typename T> __device__ __forceinline__ void zero(Frag<T>& f) {
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = (T)0.0f;
}
// Probability fragment from 8 fp32 values (round to nearest even for bf16).
__device__ __forceinline__ void set8(Frag<__bf16>& f, const float* x) {
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = (__bf16)x[t];
}
__device__ __forceinline__ void set8(Frag<float>& f, const float* x) {
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = x[t];
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// Order-preserving map of a float to uint32 (-0 is folded onto +0 first).
__device__ __forceinline__ uint32_t fkey(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Composite candidate key: larger key = higher score, then lower index.
__device__ __forceinline__ uint64_t ckey(float s, uint32_t idx) {
  return ((uint64_t)fkey(s) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t ckey_idx(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

__device__ __forceinline__ float wave_max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum_groups(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// In-place bitonic sort of a[0..P) in LDS (P a power of two) by the whole
// block; `descending` selects the final order.  Ends with a barrier.
template <typename K>
__device__ void block_bitonic_sort(K* a, int P, bool descending) {
  const int nt = blockDim.x, tid = threadIdx.x;
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P >> 1); i += nt) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = ((lo & size) == 0) != descending;  // this pair's order
        K x = a[lo], y = a[hi];
        if ((x > y) == up) { a[lo] = y; a[hi] = x; }
      }
      __syncthreads();
    }
  }
}

__host__ __device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace mita
