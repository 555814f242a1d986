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
//   k_probe_step  the attention kernels' own online-softmax step (attn_step:
//                 scores on the matrix cores, running-maximum check,
//                 exponentials, bf16 packing, P.V and the normaliser product)
//                 with every operand already in registers: no loads, no
//                 barriers, no hooks.  Its rate is the ceiling of a kernel
//                 built on that step at the same waves per workgroup and
//                 16-row blocks per wave.
#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

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

template <int NW, int IB, int WPE>
__global__ __launch_bounds__(NW * 64, WPE) void k_probe_step(float* __restrict__ out, int iters) {
  typedef __bf16 T;
  constexpr int D = 64;
  const int lane = threadIdx.x % 64, li = lane % 16, lg = lane / 16;
  StepFrags<T, D> f;
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
      for (int t = 0; t < 8; ++t) f.ka[jt][dc].v[t] = (T)(0.01f * ((lane + t + jt + dc) % 7) - 0.03f);
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
    for (int t = 0; t < 8; ++t) f.va[cb].v[t] = (T)(0.02f * ((lane * 3 + t + cb) % 5));
  Frag<T> qf[IB][D / 32];
#pragma unroll
  for (int b = 0; b < IB; ++b)
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
      for (int t = 0; t < 8; ++t) qf[b][dc].v[t] = (T)(0.01f * ((lane + 2 * t + b + dc) % 9) - 0.04f);
  const Frag<T> one = ones_frag<T>(li);
  const float cscale = 0.18033688f;  // log2(e) / sqrt(64)
  RunMax M[IB];
  f32x4 Z[IB];
  f32x4 acc[IB][D / 16];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    M[b].set(1.0f, cscale);
    Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = 0; i < iters; ++i) {
    attn_step<IB, false>(f, one, qf, 32, lg, cscale, M, Z, acc, NoHook{});
    // a loop-carried key operand keeps the score products inside the loop
    f.ka[0][0].v[0] = (T)((float)f.ka[0][0].v[0] + 1e-30f * Z[0][0]);
  }
  float s = 0.f;
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    s += Z[b][0];
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) s += acc[b][cb][0] + acc[b][cb][1] + acc[b][cb][2] + acc[b][cb][3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

int probe_step_threads(int shape) { return (shape == 1 || shape == 3) ? 1024 : 512; }

void launch_probe_step(float* out, int shape, int blocks, int iters, hipStream_t stream) {
  // shape 0: 8 waves x 4 blocks (two waves per SIMD); 1: 16 waves x 1 block
  // (four per SIMD); 2: 8 waves x 2 blocks (two workgroups per compute
  // unit); 3: 16 waves x 2 blocks (four per SIMD)
  if (shape == 0)
    hipLaunchKernelGGL((k_probe_step<8, 4, 2>), dim3((unsigned)blocks), dim3(512), 0, stream, out, iters);
  else if (shape == 1)
    hipLaunchKernelGGL((k_probe_step<16, 1, 4>), dim3((unsigned)blocks), dim3(1024), 0, stream, out, iters);
  else if (shape == 2)
    hipLaunchKernelGGL((k_probe_step<8, 2, 2>), dim3((unsigned)blocks), dim3(512), 0, stream, out, iters);
  else
    hipLaunchKernelGGL((k_probe_step<16, 2, 4>), dim3((unsigned)blocks), dim3(1024), 0, stream, out, iters);
}

void launch_probe_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_mfma, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
}

void launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_probe_copy, dim3(8192), dim3(256), 0, stream, (const v4u*)src, (v4u*)dst, n16);
}

}  // namespace mita
