// Step 1: landmark queries by average pooling of Q (MiTA tutorial (iwxt.cn),
// ch.4 step 1, paper section 3.2; gist.science summary, section 2.2).
//
// One workgroup per (head, landmark).  Its window is a rectangle of the token
// grid (adaptive bounds [floor(iG/P), ceil((i+1)G/P)) per axis, tokens
// row-major); every window row is a contiguous run of tokens, and every
// thread loads whole 16-byte chunks of token rows, so the reads coalesce.
// Sums are kept in fp64 (exact for the value ranges met in practice: every
// input value is a bf16 or fp32 number and a window holds at most a few
// thousand of them), divided once by the window size, and rounded once to the
// input dtype, nearest with ties to even.
#include "mita_dev.h"
#include "mita_plan.h"

namespace mita {

// float64 -> bf16, round to nearest even, from the 64-bit pattern (a detour
// through float32 would round twice).  Values below the bf16 normal range
// (|x| < 2^-126, never a mean of realistic data) go through float32.
__device__ __forceinline__ __bf16 f64_to_bf16(double x) {
  if (fabs(x) < 1.1754943508222875e-38) return (__bf16)(float)x;
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);  // half ulp - 1, plus lsb
  u &= ~0x00001FFFFFFFFFFFull;                      // keep 1 + 7 significand bits
  return (__bf16)(float)__longlong_as_double((long long)u);  // both casts exact
}
__device__ __forceinline__ void store_rounded(__bf16* p, double x) { *p = f64_to_bf16(x); }
__device__ __forceinline__ void store_rounded(float* p, double x) { *p = (float)x; }

// The pooling launch also clears the workspace's zero-initialised counters
// (z16 16-byte words at zp), a grid-strided slice per workgroup, so the
// forward needs no launch of its own for it (and no memset node when a
// caller captures it in a graph).
__device__ __forceinline__ void clear_slice(uint4* __restrict__ zp, size_t z16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < z16; i += (size_t)gridDim.x * blockDim.x)
    zp[i] = make_uint4(0, 0, 0, 0);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ Q, T* __restrict__ Qt, int N,
                                              int gh, int gw, int lh, int lw, uint4* __restrict__ zp, size_t z16) {
  clear_slice(zp, z16);
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPT = D / EPC;              // chunks per token row
  constexpr int TPP = 256 / CPT;            // tokens per pass of the block
  const int m = lh * lw;
  const int bh = blockIdx.x / m, i = blockIdx.x % m;
  const long long lr = i / lw, lc = i % lw;
  const int r0 = (int)((lr * gh) / lh), r1 = (int)(((lr + 1) * gh + lh - 1) / lh);
  const int c0 = (int)((lc * gw) / lw), c1 = (int)(((lc + 1) * gw + lw - 1) / lw);
  const int wc = c1 - c0, W = (r1 - r0) * wc;
  const int chunk = threadIdx.x % CPT, tslot = threadIdx.x / CPT;

  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  const T* base = Q + (size_t)bh * N * D + chunk * EPC;
  // two independent loads in flight per thread before they are accumulated
  // (fewer loads per pass made the pass faster: four 62.5 -> two 57.7 us at
  // N = 1M, 16.6 -> 14.8 us at 256K; eight 87 us)
  constexpr int U = 2;
  for (int w0 = tslot; w0 < W; w0 += U * TPP) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + u * TPP;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (w < W) {
        const long long n = (long long)(r0 + w / wc) * gw + c0 + w % wc;
        raw[u] = *(const uint4*)(base + (size_t)n * D);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const T* v = (const T*)&raw[u];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += (double)(float)v[e];
    }
  }
  __shared__ double red[256][EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[threadIdx.x][e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x, ch = c / EPC, e = c % EPC;
    double s = 0.0;
    for (int ts = 0; ts < TPP; ++ts) s += red[ts * CPT + ch][e];
    store_rounded(Qt + ((size_t)bh * m + i) * D + c, s / (double)W);
  }
}

// Short windows (at most 64 tokens, the vision shapes): one wave per
// landmark, four landmarks per workgroup.  A token row is read by CPT lanes
// (16 bytes each), 64 / CPT rows a pass; the per-lane fp64 sums are then
// added across the rows of a pass with lane shuffles (no LDS, no barrier).
// The fp64 sums are the same as k_pool's (exact for the value ranges met in
// practice, see above), so the results agree bit for bit.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool_short(const T* __restrict__ Q, T* __restrict__ Qt, int N, int BHm,
                                                    int gh, int gw, int lh, int lw, uint4* __restrict__ zp,
                                                    size_t z16) {
  clear_slice(zp, z16);
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CPT = D / EPC;   // lanes per token row
  constexpr int TPW = 64 / CPT;  // token rows per pass of the wave
  const int m = lh * lw;
  const int lane = threadIdx.x % 64;
  const int g = blockIdx.x * 4 + threadIdx.x / 64;
  if (g >= BHm) return;  // wave-uniform; no barrier follows
  const int bh = g / m, i = g % m;
  const long long lr = i / lw, lc = i % lw;
  const int r0 = (int)((lr * gh) / lh), r1 = (int)(((lr + 1) * gh + lh - 1) / lh);
  const int c0 = (int)((lc * gw) / lw), c1 = (int)(((lc + 1) * gw + lw - 1) / lw);
  const int wc = c1 - c0, W = (r1 - r0) * wc;
  const int chunk = lane % CPT, tslot = lane / CPT;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  const T* base = Q + (size_t)bh * N * D + chunk * EPC;
  for (int w = tslot; w < W; w += TPW) {
    const long long n = (long long)(r0 + w / wc) * gw + c0 + w % wc;
    const uint4 raw = *(const uint4*)(base + (size_t)n * D);
    const T* v = (const T*)&raw;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += (double)(float)v[e];
  }
#pragma unroll
  for (int off = CPT; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (tslot == 0) {
    T* dst = Qt + (size_t)g * D + chunk * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) store_rounded(dst + e, acc[e] / (double)W);
  }
}

template <typename T, int D>
static bool launch_pool_short(const Plan& p) {
  // the largest window: ceil(G/P) + 1 rows and columns at most
  const long long wr = (p.gh + p.lh - 1) / p.lh + 1, wcl = (p.gw + p.lw - 1) / p.lw + 1;
  if (wr * wcl > 64) return false;
  const int BHm = p.BH * p.m;
  hipLaunchKernelGGL((k_pool_short<T, D>), dim3((unsigned)((BHm + 3) / 4)), dim3(256), 0, p.stream, (const T*)p.Q,
                     (T*)p.qt, p.N, BHm, p.gh, p.gw, p.lh, p.lw, (uint4*)p.zero_begin, p.zero_bytes / 16);
  return true;
}

void launch_pool(const Plan& p) {
  if (p.dtype == 1 && p.d == 64 && launch_pool_short<__bf16, 64>(p)) return;
  if (p.dtype == 1 && p.d == 32 && launch_pool_short<__bf16, 32>(p)) return;
  if (p.dtype == 0 && p.d == 64 && launch_pool_short<float, 64>(p)) return;
  if (p.dtype == 0 && p.d == 32 && launch_pool_short<float, 32>(p)) return;
  dim3 grid((unsigned)(p.BH * p.m));
  if (p.dtype == 1 && p.d == 64)
    hipLaunchKernelGGL((k_pool<__bf16, 64>), grid, dim3(256), 0, p.stream, (const __bf16*)p.Q, (__bf16*)p.qt, p.N, p.gh, p.gw, p.lh, p.lw,
                       (uint4*)p.zero_begin, p.zero_bytes / 16);
  else if (p.dtype == 1 && p.d == 32)
    hipLaunchKernelGGL((k_pool<__bf16, 32>), grid, dim3(256), 0, p.stream, (const __bf16*)p.Q, (__bf16*)p.qt, p.N, p.gh, p.gw, p.lh, p.lw,
                       (uint4*)p.zero_begin, p.zero_bytes / 16);
  else if (p.dtype == 0 && p.d == 64)
    hipLaunchKernelGGL((k_pool<float, 64>), grid, dim3(256), 0, p.stream, (const float*)p.Q, (float*)p.qt, p.N, p.gh, p.gw, p.lh, p.lw,
                       (uint4*)p.zero_begin, p.zero_bytes / 16);
  else
    hipLaunchKernelGGL((k_pool<float, 32>), grid, dim3(256), 0, p.stream, (const float*)p.Q, (float*)p.qt, p.N, p.gh, p.gw, p.lh, p.lw,
                       (uint4*)p.zero_begin, p.zero_bytes / 16);
}

}  // namespace mita
