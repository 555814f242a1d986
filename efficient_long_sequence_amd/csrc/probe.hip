// Peak probes for the roofline: what this GPU sustains on its own, measured
// beside the spec-sheet peaks.
//
//   k_probe_mfma  every wave issues `iters` rounds of eight independent
//                 16x16x32 bf16 matrix operations on varied operands (no
//                 loads, no vector work), so the matrix cores, at the clock
//                 they hold under that load, are the only limit; the
//                 accumulators are written once so nothing is dropped.
//   k_probe_copy  a 16-byte-per-thread device copy with four loads in
//                 flight per thread (reads + writes bytes through HBM once
//                 each), grid-strided.
#include "mita_dev.h"
#include "mita_plan.h"

namespace mita {

__global__ __launch_bounds__(256, 2) void k_probe_mfma(float* __restrict__ out, int iters) {
  // eight chains, each with its own operands of varied bits (an integer hash
  // of lane, chain and element), so the multipliers toggle as they do on
  // real data and the clock settles where it does under a real load
  const uint32_t lane = threadIdx.x % 64 + 64u * blockIdx.x;
  Frag<__bf16> a[8], b[8];
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t h = (lane * 8u + (uint32_t)t) * 2654435761u ^ (uint32_t)(u + 1) * 40503u;
      h ^= h >> 13;
      h *= 0x5bd1e995u;
      h ^= h >> 15;
      a[u].v[t] = (__bf16)((float)(h & 0xFFFF) * (1.0f / 32768.0f) - 1.0f);
      b[u].v[t] = (__bf16)((float)(h >> 16) * (1.0f / 32768.0f) - 1.0f);
    }
    acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u) mma16(acc[u], a[u], b[u]);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// four 16-byte loads in flight per thread, then their stores
typedef __attribute__((__vector_size__(16))) unsigned int v4u;
__global__ __launch_bounds__(256) void k_probe_copy(const v4u* __restrict__ src, v4u* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(x0, dst + i);
    __builtin_nontemporal_store(x1, dst + i + stride);
    __builtin_nontemporal_store(x2, dst + i + 2 * stride);
    __builtin_nontemporal_store(x3, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

void launch_probe_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
}

void launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_probe_copy, dim3(8192), dim3(256), 0, stream, (const v4u*)src, (v4u*)dst, n16);
}

}  // namespace mita
