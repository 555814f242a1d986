// Dense (full) softmax attention, O = softmax(Q K^T / sqrt(d)) V per head,
// non-causal: the baseline MiTA is compared against in the pages' long-sequence
// throughput test (MiTA tutorial (iwxt.cn), ch.7, "LRA and synthetic long
// sequences", paper section 4.3 / Fig. 5: a three-layer model of width 128,
// full attention against MiTA with m*k ~ N/4).
//
// One workgroup per (head, 16*IB*NW queries): every wave keeps 16*IB queries
// as matrix-core columns in registers and the block streams all N keys and
// values through double-buffered LDS tiles of 32, with the same online
// softmax (fp32, lazy running maximum) and matrix-core layout as the MiTA
// kernels.  Workgroups of one head are dealt to the XCDs in turn and stream
// the keys in the same order, so a tile fetched from HBM serves the other
// workgroups through the caches.
#include <cmath>

#include "mita_dev.h"
#include "mita_plan.h"
#include "tile.h"

namespace mita {

template <typename T, int D, int NW, int IB>
__global__ __launch_bounds__(NW * 64, 2) void k_dense(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, T* __restrict__ O, int N,
                                                   float cscale) {
  constexpr int NT = NW * 64;
  using TL = TileLayout<T, D>;
  __shared__ __align__(16) T smem[2 * TL::ELEMS];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, li = lane % 16, lg = lane / 16;
  const int bh = blockIdx.y;
  const size_t hb = (size_t)bh * N * D;
  const int qbase = blockIdx.x * (NW * 16 * IB) + wave * 16 * IB;
  const Frag<T> one = ones_frag<T>(li);

  Frag<T> qf[IB][D / 32];
  RunMax M[IB];
  f32x4 Z[IB];
  f32x4 acc[IB][D / 16];
#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const int n = qbase + b * 16 + li;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      if (n < N) load8(qf[b][dc], Q + hb + (size_t)n * D + dc * 32 + 8 * lg);
      else zero(qf[b][dc]);
    }
    M[b].set(M0, cscale);
    Z[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) acc[b][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto rowK = [&](int j0) {
    return [=](int r) -> const T* { const int j = j0 + r; return j < N ? K + hb + (size_t)j * D : nullptr; };
  };
  auto rowV = [&](int j0) {
    return [=](int r) -> const T* { const int j = j0 + r; return j < N ? V + hb + (size_t)j * D : nullptr; };
  };
  // two register stages: the loads of step st + 2 are issued at the start of
  // step st, the tile of step st + 1 (loaded a step earlier) is stored at its
  // end; the two loaders swap roles every step (the loop is unrolled by two).
  // The partial last step is peeled off the loop: with both forms of the step
  // in the loop body the kernel runs out of registers.
  TileLoader<T, D, NT, true> la, lb;
  T* buf0 = smem;
  T* buf1 = smem + TL::ELEMS;
  const int nsteps = (N + 31) / 32;
  la.load(rowK(0), rowV(0));
  la.store(buf0, buf0 + TL::K_ELEMS);
  if (nsteps > 1) la.load(rowK(32), rowV(32));
  __syncthreads();
  auto body = [&](int st, auto masked, auto& lnext, auto& lfar) {
    constexpr bool MASKED = decltype(masked)::value;
    const int j0 = st * 32;
    T* cur = (st & 1) ? buf1 : buf0;
    T* nxt = (st & 1) ? buf0 : buf1;
    if (st + 2 < nsteps) lfar.load(rowK(j0 + 64), rowV(j0 + 64));
    StepFrags<T, D> f;
    f.load_keys(cur, li, lg);
    f.load_vals(cur + TL::K_ELEMS, li, lg);
    attn_step<IB, MASKED>(f, one, qf, min(32, N - j0), lg, cscale, M, Z, acc, NoHook{});
    if (st + 1 < nsteps) lnext.store(nxt, nxt + TL::K_ELEMS);
    __syncthreads();
  };
  const int nfull = N / 32;
  int st = 0;
  for (; st + 1 < nfull; st += 2) {
    body(st, BoolTag<false>{}, la, lb);
    body(st + 1, BoolTag<false>{}, lb, la);
  }
  if (st < nfull) {
    body(st, BoolTag<false>{}, la, lb);
    ++st;
    if (st < nsteps) body(st, BoolTag<true>{}, lb, la);
  } else if (st < nsteps) {
    body(st, BoolTag<true>{}, la, lb);
  }

#pragma unroll
  for (int b = 0; b < IB; ++b) {
    const float inv = 1.0f / finish_z(Z[b], li);
    const int n = qbase + b * 16 + li;
    if (n >= N) continue;
    T* o = O + hb + (size_t)n * D;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[cb * 16 + 4 * lg + r] = from_f32<T>(acc[b][cb][r] * inv);
  }
}

template <typename T, int D, int NW, int IB>
static void launch_dense_t(const void* Q, const void* K, const void* V, void* O, int BH, int N, float cscale,
                           hipStream_t stream) {
  constexpr int QPB = NW * 16 * IB;
  dim3 grid((unsigned)((N + QPB - 1) / QPB), (unsigned)BH);
  hipLaunchKernelGGL((k_dense<T, D, NW, IB>), grid, dim3(NW * 64), 0, stream, (const T*)Q, (const T*)K,
                     (const T*)V, (T*)O, N, cscale);
}

void launch_dense(const void* Q, const void* K, const void* V, void* O, int dtype, int BH, int N, int d,
                  hipStream_t stream) {
  const float cscale = (float)(1.4426950408889634 / std::sqrt((double)d));
  if (dtype == 0) {
    if (d == 32) launch_dense_t<float, 32, 4, 1>(Q, K, V, O, BH, N, cscale, stream);
    else launch_dense_t<float, 64, 4, 1>(Q, K, V, O, BH, N, cscale, stream);
  } else {
    if (d == 32) launch_dense_t<__bf16, 32, 8, 4>(Q, K, V, O, BH, N, cscale, stream);
    else launch_dense_t<__bf16, 64, 8, 4>(Q, K, V, O, BH, N, cscale, stream);
  }
}

}  // namespace mita
