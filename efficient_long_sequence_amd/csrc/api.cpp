// C ABI of libmita: argument validation, the launch plan and workspace
// carve-up, and the enqueue order of the forward pass.  No device memory is
// allocated and no state is kept between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mita.h"
#include "mita_plan.h"

using namespace mita;

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

mita_status validate(const void* Q, const void* K, const void* V, const void* O, mita_dtype dtype, int B, int H,
                     int N, int d, mita_pool pool, int m, int k, int s, bool check_ptrs) {
  if (check_ptrs && (!Q || !K || !V || !O)) return MITA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return MITA_ERR_SHAPE;
  if (pool.grid_h <= 0 || pool.grid_w <= 0 || pool.land_h <= 0 || pool.land_w <= 0) return MITA_ERR_SHAPE;
  if ((long long)pool.grid_h * pool.grid_w != N) return MITA_ERR_SHAPE;
  if ((long long)pool.land_h * pool.land_w != m) return MITA_ERR_SHAPE;
  if (pool.land_h > pool.grid_h || pool.land_w > pool.grid_w) return MITA_ERR_SHAPE;
  if (k < 1 || k > N) return MITA_ERR_PARAM;
  if (s < 1 || s > m) return MITA_ERR_PARAM;
  if (check_ptrs) {
    const uintptr_t mis = ((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u;
    if (mis) return MITA_ERR_PARAM;
  }
  if (dtype != MITA_F32 && dtype != MITA_BF16) return MITA_ERR_UNSUPPORTED;
  if (d != 32 && d != 64) return MITA_ERR_UNSUPPORTED;
  if (s > MAX_S || m > MAX_M || (long long)N > MAX_N) return MITA_ERR_UNSUPPORTED;
  if (N > NSMALL && k > MAX_K_SPARSE) return MITA_ERR_UNSUPPORTED;
  if ((long long)B * H > 65535) return MITA_ERR_UNSUPPORTED;
  // query positions of a slot (bucket offsets, work items) are 32-bit
  if ((long long)B * H * N > 0x7FFFFFFFLL) return MITA_ERR_UNSUPPORTED;
  return MITA_OK;
}

// Sizes, launch shapes and workspace regions.  With base == nullptr only the
// sizes are meaningful (used by mita_workspace_bytes).
Plan make_plan(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool, int m, int k, int s, char* base) {
  Plan p;
  std::memset(&p, 0, sizeof(p));
  p.dtype = dtype == MITA_BF16 ? 1 : 0;
  p.esize = p.dtype ? 2 : 4;
  p.B = B; p.H = H; p.BH = B * H; p.N = N; p.d = d;
  p.gh = pool.grid_h; p.gw = pool.grid_w; p.lh = pool.land_h; p.lw = pool.land_w;
  p.m = m; p.k = k; p.s = s;
  p.cscale = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.cscale_sh = p.cscale;
  p.shared = 1;

  // landmark scoring: rows per workgroup tile
  if (p.dtype == 0 || m <= 64) { p.sc_nw = 4; p.sc_ib = 1; }
  else if (m <= 128) { p.sc_nw = 8; p.sc_ib = 1; }
  else if (m <= 256) { p.sc_nw = 8; p.sc_ib = 2; }
  else { p.sc_nw = 8; p.sc_ib = 4; }
  p.sc_R = p.sc_nw * 16 * p.sc_ib;
  p.sc_rt = ceil_div(m, p.sc_R);
  // key chunks: about as many workgroups as fit on the chip at once (8-wave
  // tiles of two or four 16-row blocks per wave run one workgroup per compute
  // unit, the others two)
  const long long target = (p.sc_nw == 8 && p.sc_ib >= 2) ? 256 : 512;
  int C = ceil_div(target, (long long)p.BH * p.sc_rt);
  C = C < 1 ? 1 : C;
  const int max_c = ceil_div(N, 32);
  C = C > max_c ? max_c : C;
  int L = ceil_div(N, C);
  L = (L + 31) / 32 * 32;
  if (L > (1 << 23)) L = 1 << 23;
  p.L = L;
  p.C = ceil_div(N, L);

  p.dense = N <= NSMALL ? 1 : 0;
  p.small = (N <= SMALL_N && k <= SMALL_K) ? 1 : 0;
  {
    int cap = CAPG_MIN;
    while (cap < 8 * k && cap < CAPG) cap *= 2;
    p.capg = p.dense ? N : cap;
  }
  if (!p.dense) {
    p.sigma = k / 32 > 1 ? k / 32 : 1;
    p.NS = N / p.sigma;
    p.G = p.NS < 512 ? p.NS : 512;
    const double lam = (double)k / p.sigma;
    int J = (int)std::ceil(lam + 6.0 * std::sqrt(lam) + 3.0);
    p.J = J > p.G ? p.G : J;
    const long long est_target = 2048;  // (few sample groups per workgroup: each costs a load round trip)
    int gpb = ceil_div((long long)p.G * p.BH * p.sc_rt, est_target);
    p.est_gpb = gpb < 1 ? 1 : gpb;
    // records per (row, chunk, lane group): the threshold admits about 2.3 k
    // keys per row and a record holds one or more of them, so a lane group
    // holds at most e = 0.35 k L / N records per chunk on average (the
    // seeded 1M-key inputs give 0.5 to 0.6 e); clustered keys come in bursts
    // of up to about 10 times the mean, so room is left for 20 e and at least
    // REC_MIN; a lane keeps at most one record per 32-key step
    const int steps = ceil_div(p.L, 32);
    const double e = 0.35 * (double)k * p.L / N;
    int s4 = (int)std::ceil(20.0 * e);
    s4 = s4 < REC_MIN ? REC_MIN : s4;
    s4 = steps < s4 ? steps : s4;
    // the scoring kernel indexes records with 32 bits (segs < 2^32 under the
    // argument limits above, B*H <= 65535 and m <= 4096, so s4 stays >= 1)
    const long long segs = (long long)p.BH * m * p.C * 4;
    const long long most = (long long)UINT32_MAX / segs;
    p.s4 = s4 < most ? s4 : (int)most;
    // Test hook (host-forced): MITA_TEST_FORCE_FALLBACK=1 sets every candidate
    // threshold to +inf, so no row collects candidates and every row is
    // selected by the exact fallback kernel instead.
    const char* ff = std::getenv("MITA_TEST_FORCE_FALLBACK");
    p.force_fallback = (ff != nullptr && ff[0] == '1') ? 1 : 0;
  }

  // routing and attention tiles
  p.smax = s <= 1 ? 1 : s <= 2 ? 2 : s <= 4 ? 4 : 8;
  const double avg = (double)N / m;  // queries per expert and slot, on average
  const size_t hist_bytes = (size_t)s * m <= 4096 ? (size_t)s * m * 4 : 0;
  // (the expert kernel also stages its k key indices and up to 2048 query
  // indices in LDS)
  p.fast = (resident_bytes(p.dtype, d, m) + hist_bytes <= RES_MAX &&
            resident_bytes(p.dtype, d, k) + (size_t)(k + 32 + 2048) * 4 <= RES_MAX) ? 1 : 0;
  if (p.fast) {
    // routing workgroups: about 256 in all (one per compute unit at a
    // time, so each stages its landmarks once for many queries), 512
    // queries at least
    long long qpw = ((long long)p.BH * N + 255) / 256;
    qpw = (qpw + 511) / 512 * 512;
    p.rs_qpw = (int)(qpw < 512 ? 512 : qpw);
    // bf16: sixteen waves of one 16-query block each (four per SIMD, which
    // cover each other's dependency stalls; N = 1M: 0.373 -> 0.357 ms,
    // DeiT-S: 18 -> 13.5 us), or for top-1 routing over 512 or more
    // landmarks twelve waves of two blocks (three per SIMD, the two blocks'
    // chains interleaved: N = 1M 0.413-0.416 -> 0.398-0.399 ms; level at
    // m = 256, 128; 1 us slower at DeiT-S); fp32: eight waves of four blocks
    p.rs_nw = p.dtype == 1 ? (m >= 512 && s == 1 ? 12 : 16) : 8;
    if (p.dtype == 0 || avg <= 16) { p.ex_nw = 1; p.ex_ib = 1; }
    else if (avg <= 64) { p.ex_nw = 1; p.ex_ib = 2; }
    else if (avg <= 256) { p.ex_nw = 4; p.ex_ib = 4; }
    // experts of up to ~1K queries: sixteen waves of one 16-query block
    // (four waves per SIMD; 64K: 0.079 -> 0.067 ms, 256K: 0.082 -> 0.075 ms);
    // larger ones two blocks (N = 1M: 0.424 -> 0.404 ms with sixteen waves
    // against eight waves of four), in twelve waves, which leaves the
    // registers to fetch the stored shared part before the key loop
    // (0.44 -> 0.415 ms)
    else if (avg <= 1024) { p.ex_nw = 16; p.ex_ib = 1; }
    else { p.ex_nw = 12; p.ex_ib = 2; }
    // queries per work item: about twice the average expert (at least 64),
    // in whole groups of the launch shape, at most 2048 queries (the
    // work-list scan's size classes): an expert that fits one item stages
    // its keys once, while smaller items spread a large expert over more
    // workgroups (measured: DeiT-S 19.5 -> 17.6 us, ADE 32x32 18 -> 15,
    // 40x40 21 -> 17, N = 64K 69 -> 60 us, against items of about the
    // average; N = 256K 68-72 -> 64-66 us with items of 2048 queries
    // instead of 1024)
    const int per = p.ex_nw * 16 * p.ex_ib;
    const double want = 2.0 * avg > 64.0 ? 2.0 * avg : 64.0;
    const int gmax = 2048 / per;
    int gpw = (int)(want / per + 0.5);
    gpw = gpw < 1 ? 1 : gpw > gmax ? gmax : gpw;
    p.T = per * gpw;
  } else {
    if (p.dtype == 0 || avg <= 16) { p.at_nw = 1; p.at_ib = 1; }
    else if (avg <= 64) { p.at_nw = 4; p.at_ib = 1; }
    // (four waves of four 16-query blocks also for large experts: that form
    // keeps all its registers at one wave per SIMD, the 8-wave one spills)
    else { p.at_nw = 4; p.at_ib = 4; }
    p.T = p.at_nw * 16 * p.at_ib;
  }
  p.UB = (int)((long long)p.BH * (ceil_div(N, p.T) + m));  // <= B*H*N/16 + B*H*m: fits (see validate)

  // workspace
  const size_t BH = p.BH, Mr = (size_t)p.BH * m;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* ptr = base ? base + off : nullptr;
    off = align_up(off + bytes, 256);
    return ptr;
  };
  p.qt = take(Mr * d * p.esize);
  p.gmax = (float*)take(p.dense ? 0 : Mr * p.G * 4);
  p.tau = (float*)take(Mr * 4);
  p.mhat = (float*)take(Mr * 4);
  p.vpart = (float*)take(Mr * p.C * (d + 4) * 4);
  p.cand = (uint64_t*)take(p.dense && !p.small ? Mr * p.capg * 8 : 0);
  const size_t nseg = p.dense ? 0 : Mr * p.C * 4;
  p.rec_sc = (float*)take(nseg * p.s4 * 8 * 4);
  p.rec_st = (int32_t*)take(nseg * p.s4 * 4);
  p.rec_cnt = (int*)take(nseg * 4);
  const size_t zoff = off;
  p.counts = (int*)take((size_t)s * Mr * 4);
  p.cursor = (int*)take((size_t)s * Mr * 4);
  p.zero_begin = base ? base + zoff : nullptr;
  p.zero_bytes = off - zoff;
  p.fail = (int*)take(Mr * 4);
  p.topk = (int32_t*)take(Mr * k * 4);
  p.vt32 = (float*)take(Mr * d * 4);
  p.vtT = take(Mr * d * p.esize);
  p.route = (int32_t*)take(BH * N * s * 4);
  p.gpre = (int*)take((size_t)s * Mr * 4);
  p.perm = (int32_t*)take((size_t)s * BH * N * 4);
  p.wl = (WorkItem*)take((size_t)s * p.UB * sizeof(WorkItem));
  p.wl_count = (int*)take(MAX_S * 4);
  p.part = (float*)take(!p.fast && s > 1 ? (size_t)(s - 1) * BH * N * (d + 4) * 4 : 0);
  p.plse = (float2*)take(p.fast ? BH * N * 8 : 0);
  p.po = take(p.fast ? BH * N * d * (p.dtype ? 2 : 4) : 0);  // fp16 / fp32
  p.total_bytes = off;
  return p;
}

bool valid_variant(int v) {
  return v == MITA_VARIANT_PAPER || v == MITA_VARIANT_OFFICIAL || v == MITA_VARIANT_ROUTED;
}

mita_status check_saved(const mita_saved* sv, int variant) {
  if (!sv || !sv->qtilde || !sv->topk || !sv->route || !sv->lse || !sv->out_f32) return MITA_ERR_NULL;
  const bool shared = variant != MITA_VARIANT_ROUTED;
  if (shared && (!sv->vtilde || !sv->lse_landmark)) return MITA_ERR_NULL;
  if (((uintptr_t)sv->qtilde | (uintptr_t)sv->out_f32 | (shared ? (uintptr_t)sv->vtilde : 0)) & 15u)
    return MITA_ERR_PARAM;
  return MITA_OK;
}

struct Timer {
  void* const* ev;
  hipStream_t st;
  // a stage whose handles are NULL is not timed
  void begin(int stage) const {
    if (ev && ev[2 * stage]) (void)hipEventRecord((hipEvent_t)ev[2 * stage], st);
  }
  void end(int stage) const {
    if (ev && ev[2 * stage + 1]) (void)hipEventRecord((hipEvent_t)ev[2 * stage + 1], st);
    // Diagnostics (host-set MITA_DEBUG_SYNC): name each stage whose launches
    // reported an error; with 1 also wait for the stage to finish.
    if (debug_sync) {
      const hipError_t e1 = hipGetLastError();
      const hipError_t e2 = debug_sync == 1 ? hipStreamSynchronize(st) : hipSuccess;
      if (e1 != hipSuccess || e2 != hipSuccess)
        std::fprintf(stderr, "mita: stage %d: %s\n", stage, hipGetErrorString(e1 != hipSuccess ? e1 : e2));
    }
  }
  int debug_sync = 0;
};

mita_status run(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B, int H, int N,
                int d, mita_pool pool, int m, int k, int s, int variant, const mita_debug* dbg, void* workspace,
                size_t workspace_bytes, void* stream, void* const* events, const mita_saved* sv = nullptr,
                bool want_saved = false) {
  mita_status st = validate(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, true);
  if (st != MITA_OK) return st;
  if (!valid_variant(variant)) return MITA_ERR_PARAM;
  if (want_saved && (st = check_saved(sv, variant)) != MITA_OK) return st;
  if (!workspace) return MITA_ERR_NULL;
  if ((uintptr_t)workspace & 15u) return MITA_ERR_PARAM;
  Plan p = make_plan(dtype, B, H, N, d, pool, m, k, s, (char*)workspace);
  if (workspace_bytes < p.total_bytes) return MITA_ERR_WORKSPACE;
  p.Q = Q; p.K = K; p.V = V; p.O = O;
  p.stream = (hipStream_t)stream;
  if (variant == MITA_VARIANT_OFFICIAL) p.cscale_sh = (float)(1.4426950408889634 / (double)d);
  p.shared = variant == MITA_VARIANT_ROUTED ? 0 : 1;
  if (sv) {
    p.lse_out = sv->lse;
    p.lse_lm = p.shared ? sv->lse_landmark : nullptr;
    p.o32 = sv->out_f32;
  }
  Timer tm{events, p.stream};
  {
    const char* ds = std::getenv("MITA_DEBUG_SYNC");
    tm.debug_sync = ds == nullptr ? 0 : ds[0] == '1' ? 1 : ds[0] == '2' ? 2 : 0;
  }

  (void)hipGetLastError();  // clear any earlier sticky launch error
  tm.begin(ST_POOL);
  launch_pool(p);  // (also clears the zero-initialised counters)
  tm.end(ST_POOL);
  tm.begin(ST_EST);
  if (!p.dense) launch_estimate(p);
  tm.end(ST_EST);
  tm.begin(ST_SCORE);
  launch_score(p);
  tm.end(ST_SCORE);
  tm.begin(ST_FINAL);
  launch_final(p);
  tm.end(ST_FINAL);
  tm.begin(ST_ROUTE);
  if (p.fast && p.shared) launch_route_shared(p);
  else launch_route(p);  // routing only (the shared part, if any, is done by the streaming attention)
  tm.end(ST_ROUTE);
  tm.begin(ST_BUCKET);
  launch_bucket(p);
  tm.end(ST_BUCKET);
  tm.begin(ST_ATTEND);
  if (p.fast) launch_expert(p);
  else launch_attend(p);
  tm.end(ST_ATTEND);

  if (dbg) {
    const size_t Mr = (size_t)p.BH * m;
    if (dbg->topk) (void)hipMemcpyAsync(dbg->topk, p.topk, Mr * k * 4, hipMemcpyDeviceToDevice, p.stream);
    if (dbg->route)
      (void)hipMemcpyAsync(dbg->route, p.route, (size_t)p.BH * N * s * 4, hipMemcpyDeviceToDevice, p.stream);
    if (dbg->vtilde && p.shared)
      (void)hipMemcpyAsync(dbg->vtilde, p.vt32, Mr * d * 4, hipMemcpyDeviceToDevice, p.stream);
    if (dbg->qtilde)
      (void)hipMemcpyAsync(dbg->qtilde, p.qt, Mr * d * p.esize, hipMemcpyDeviceToDevice, p.stream);
  }
  if (sv) {
    const size_t Mr = (size_t)p.BH * m;
    (void)hipMemcpyAsync(sv->qtilde, p.qt, Mr * d * p.esize, hipMemcpyDeviceToDevice, p.stream);
    if (p.shared) (void)hipMemcpyAsync(sv->vtilde, p.vt32, Mr * d * 4, hipMemcpyDeviceToDevice, p.stream);
    (void)hipMemcpyAsync(sv->topk, p.topk, Mr * k * 4, hipMemcpyDeviceToDevice, p.stream);
    (void)hipMemcpyAsync(sv->route, p.route, (size_t)p.BH * N * s * 4, hipMemcpyDeviceToDevice, p.stream);
  }
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

// Sizes, launch shapes and workspace regions of one backward call.
BPlan make_bplan(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool, int m, int k, int s, char* base) {
  BPlan p;
  std::memset(&p, 0, sizeof(p));
  p.dtype = dtype == MITA_BF16 ? 1 : 0;
  p.esize = p.dtype ? 2 : 4;
  p.BH = B * H; p.N = N; p.d = d;
  p.gh = pool.grid_h; p.gw = pool.grid_w; p.lh = pool.land_h; p.lw = pool.land_w;
  p.m = m; p.k = k; p.s = s;
  p.shared = 1;
  p.cnat = (float)(1.0 / std::sqrt((double)d));
  p.cnat_sh = p.cnat;
  p.cscale = (float)(1.4426950408889634 / std::sqrt((double)d));
  p.cscale_sh = p.cscale;
  p.R = backward_rows(p.dtype, m);
  // landmark-row passes: about 256 workgroups in all (one per compute unit: fewer chunks mean fewer partials to sum), whole 32-entry steps
  auto chunks = [&](int& L, int& C, int rows) {
    const long long rt = ceil_div(m, rows);
    long long c = ceil_div(256, rt * p.BH);
    c = c < 1 ? 1 : c;
    const long long cmax = ceil_div(N, 32);
    c = c > cmax ? cmax : c;
    L = ceil_div(N, c);
    L = (L + 31) / 32 * 32;
    C = ceil_div(N, L);
  };
  chunks(p.L1, p.C1, p.R);
  chunks(p.L4, p.C4, backward_lm4_rows(p.dtype, m));
  // query grouping: tiles of R queries
  Plan& b = p.bk;
  b.dtype = p.dtype; b.esize = p.esize; b.B = B; b.H = H; b.BH = p.BH; b.N = N; b.d = d;
  b.m = m; b.k = k; b.s = s;
  b.T = backward_query_rows(p.dtype);
  b.UB = (int)((long long)p.BH * (ceil_div(N, b.T) + m));

  const size_t BH = p.BH, Mr = (size_t)p.BH * m, Nr = (size_t)p.BH * N;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* ptr = base ? base + off : nullptr;
    off = align_up(off + bytes, 256);
    return ptr;
  };
  const size_t zoff = off;
  b.counts = (int*)take((size_t)s * Mr * 4);
  b.cursor = (int*)take((size_t)s * Mr * 4);
  p.icnt = (int*)take(Nr * 4);
  p.icur = (int*)take(Nr * 4);
  p.zero_begin = base ? base + zoff : nullptr;
  p.zero_bytes = off - zoff;
  p.Dn = (float*)take(Nr * 4);
  p.ipos = (int*)take(Nr * 4);
  p.bsum = (int*)take(((Nr + 4095) / 4096 + 1) * 4);
  p.ilist = (int32_t*)take(Mr * k * 4);
  p.ikey = (int32_t*)take(Mr * k * 4);
  // routed-key pass: items of at most CH queries (large experts split)
  p.CH = 2048;
  p.UB2 = (int)((long long)p.BH * (ceil_div(N, p.CH) + m));
  p.wl2 = (WorkItem*)take((size_t)s * p.UB2 * sizeof(WorkItem));
  p.wl2_count = (int*)take(MAX_S * 4);
  p.efirst = (int*)take((size_t)s * Mr * 4);
  p.epart = (int*)take((size_t)s * Mr * 4);
  p.G = (float*)take((size_t)s * p.UB2 * k * 2 * d * 4);
  p.Gs = (float*)take(Mr * k * 2 * d * 4);
  // expert-order copies of the queries (fp32 only: bf16 reads them through
  // the permutation)
  const size_t gath = p.dtype == 0 ? (size_t)s * Nr : 0;
  p.Qg = take(gath * d * p.esize);
  p.dOg = take(gath * d * p.esize);
  p.Lg = (float*)take(gath * 4);
  p.Dg = (float*)take(gath * 4);
  b.route = (int32_t*)take(Nr * s * 4);
  b.gpre = (int*)take((size_t)s * Mr * 4);
  b.perm = (int32_t*)take((size_t)s * Nr * 4);
  b.wl = (WorkItem*)take((size_t)s * b.UB * sizeof(WorkItem));
  b.wl_count = (int*)take(MAX_S * 4);
  p.part1 = (float*)take(BH * p.C1 * m * 2 * d * 4);
  p.part4 = (float*)take(BH * p.C4 * m * d * 4);
  p.dqt = (float*)take(Mr * d * 4);
  p.dvt = (float*)take(Mr * d * 4);
  p.dvtT = take(Mr * d * p.esize);
  p.vt = take(Mr * d * p.esize);
  p.delta = (float*)take(Mr * 4);
  p.qpart = (float*)take(s > 1 ? (size_t)(s - 1) * Nr * d * 4 : 0);
  p.total_bytes = off;
  return p;
}

const char* const kStageNames[ST_COUNT] = {"pool", "estimate", "score", "select", "route", "bucket", "attend"};

}  // namespace

// Scratch of mita_forward_noalloc: a file-scope device array, one copy on
// every GPU the library runs on, held until the process ends.  Host code uses
// the device address hipGetSymbolAddress returns for the current device
// (kept per device below), never the array's name, which on the host is only
// a stand-in for the symbol.
static __device__ __align__(256) unsigned char scratch[MITA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (nullptr: not looked up yet)

// The scratch array's address on the current device, looked up once per
// device (with that device current).
mita_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MITA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MITA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MITA_OK;
}

}  // namespace

extern "C" {

size_t mita_workspace_bytes(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool, int m, int k, int s) {
  if (validate(nullptr, nullptr, nullptr, nullptr, dtype, B, H, N, d, pool, m, k, s, false) != MITA_OK) return 0;
  return make_plan(dtype, B, H, N, d, pool, m, k, s, nullptr).total_bytes;
}

mita_status mita_forward(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B, int H,
                         int N, int d, mita_pool pool, int m, int k, int s, const mita_debug* dbg, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return run(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, MITA_VARIANT_PAPER, dbg, workspace, workspace_bytes,
             stream, nullptr);
}

mita_status mita_forward_noalloc(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B,
                                 int H, int N, int d, mita_pool pool, int m, int k, int s, void* stream) {
  mita_status st = validate(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, true);
  if (st != MITA_OK) return st;
  if (make_plan(dtype, B, H, N, d, pool, m, k, s, nullptr).total_bytes > MITA_NOALLOC_SCRATCH_BYTES)
    return MITA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MITA_OK) return st;
  return run(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, MITA_VARIANT_PAPER, nullptr, ws,
             MITA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

mita_status mita_forward_timed(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B,
                               int H, int N, int d, mita_pool pool, int m, int k, int s, const mita_debug* dbg,
                               void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return MITA_ERR_NULL;
  return run(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, MITA_VARIANT_PAPER, dbg, workspace, workspace_bytes,
             stream, events);
}

mita_status mita_forward_variant(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B,
                                 int H, int N, int d, mita_pool pool, int m, int k, int s, mita_variant variant,
                                 const mita_debug* dbg, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events) {
  return run(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, (int)variant, dbg, workspace, workspace_bytes, stream,
             events);
}

mita_status mita_dense_attention(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B,
                                 int H, int N, int d, void* stream) {
  if (!Q || !K || !V || !O) return MITA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return MITA_ERR_SHAPE;
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u) return MITA_ERR_PARAM;
  if (dtype != MITA_F32 && dtype != MITA_BF16) return MITA_ERR_UNSUPPORTED;
  if (d != 32 && d != 64) return MITA_ERR_UNSUPPORTED;
  if ((long long)N > MAX_N || (long long)B * H > 65535) return MITA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  launch_dense(Q, K, V, O, dtype == MITA_BF16 ? 1 : 0, B * H, N, d, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

mita_status mita_forward_train(const void* Q, const void* K, const void* V, void* O, mita_dtype dtype, int B,
                               int H, int N, int d, mita_pool pool, int m, int k, int s, mita_variant variant,
                               const mita_saved* saved, void* workspace, size_t workspace_bytes, void* stream) {
  return run(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, (int)variant, nullptr, workspace, workspace_bytes, stream,
             nullptr, saved, true);
}

size_t mita_backward_workspace_bytes(mita_dtype dtype, int B, int H, int N, int d, mita_pool pool, int m, int k,
                                     int s) {
  if (validate(nullptr, nullptr, nullptr, nullptr, dtype, B, H, N, d, pool, m, k, s, false) != MITA_OK) return 0;
  if ((long long)B * H * m * k > 0x7FFFFFFFLL) return 0;
  return make_bplan(dtype, B, H, N, d, pool, m, k, s, nullptr).total_bytes;
}

mita_status mita_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO, void* dQ,
                          void* dK, void* dV, mita_dtype dtype, int B, int H, int N, int d, mita_pool pool, int m,
                          int k, int s, mita_variant variant, const mita_saved* saved, void* workspace,
                          size_t workspace_bytes, void* stream) {
  mita_status st = validate(Q, K, V, O, dtype, B, H, N, d, pool, m, k, s, true);
  if (st != MITA_OK) return st;
  if (!dO || !dQ || !dK || !dV) return MITA_ERR_NULL;
  if (((uintptr_t)dO | (uintptr_t)dQ | (uintptr_t)dK | (uintptr_t)dV) & 15u) return MITA_ERR_PARAM;
  if (!valid_variant((int)variant)) return MITA_ERR_PARAM;
  if ((st = check_saved(saved, (int)variant)) != MITA_OK) return st;
  // positions in the keys' inverse lists are 32-bit
  if ((long long)B * H * m * k > 0x7FFFFFFFLL) return MITA_ERR_UNSUPPORTED;
  if (!workspace) return MITA_ERR_NULL;
  if ((uintptr_t)workspace & 15u) return MITA_ERR_PARAM;
  BPlan p = make_bplan(dtype, B, H, N, d, pool, m, k, s, (char*)workspace);
  if (workspace_bytes < p.total_bytes) return MITA_ERR_WORKSPACE;
  p.shared = variant == MITA_VARIANT_ROUTED ? 0 : 1;
  if (variant == MITA_VARIANT_OFFICIAL) {
    p.cnat_sh = (float)(1.0 / (double)d);
    p.cscale_sh = (float)(1.4426950408889634 / (double)d);
  }
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.dO = dO;
  p.dQ = dQ; p.dK = dK; p.dV = dV;
  p.qt = saved->qtilde;
  p.vt32 = p.shared ? saved->vtilde : nullptr;
  p.o32 = saved->out_f32;
  p.topk = saved->topk;
  p.route = saved->route;
  p.lse = saved->lse;
  p.lse_lm = p.shared ? saved->lse_landmark : nullptr;
  p.stream = (hipStream_t)stream;
  p.bk.stream = p.stream;
  (void)hipGetLastError();
  launch_backward(p);
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

mita_status mita_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out) return MITA_ERR_NULL;
  if (blocks <= 0 || iters <= 0 || ((uintptr_t)out & 15u)) return MITA_ERR_PARAM;
  (void)hipGetLastError();
  launch_probe_mfma(out, blocks, iters, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

mita_status mita_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return MITA_ERR_NULL;
  if (bytes % 16 || (((uintptr_t)src | (uintptr_t)dst) & 15u)) return MITA_ERR_PARAM;
  (void)hipGetLastError();
  launch_probe_copy(src, dst, bytes, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

mita_status mita_probe_step(float* out, int shape, int blocks, int iters, void* stream) {
  if (!out) return MITA_ERR_NULL;
  if (shape < 0 || shape > 3 || blocks <= 0 || iters <= 0 || ((uintptr_t)out & 15u)) return MITA_ERR_PARAM;
  (void)hipGetLastError();
  launch_probe_step(out, shape, blocks, iters, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MITA_OK : MITA_ERR_HIP;
}

int mita_num_stages(void) { return ST_COUNT; }

const char* mita_stage_name(int stage) { return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "?"; }

mita_status mita_events_create(void** events, int count) {
  if (!events || count <= 0) return MITA_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    // timing only: no system-scope fence at each record, so a record between
    // two kernels adds no cache write-back
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return MITA_ERR_HIP;
    events[i] = (void*)e;
  }
  return MITA_OK;
}

mita_status mita_events_destroy(void** events, int count) {
  if (!events || count <= 0) return MITA_ERR_NULL;
  for (int i = 0; i < count; ++i)
    if (events[i]) (void)hipEventDestroy((hipEvent_t)events[i]);
  return MITA_OK;
}

mita_status mita_events_elapsed(void* const* events, int n_pairs, float* ms) {
  if (!events || !ms || n_pairs <= 0) return MITA_ERR_NULL;
  for (int i = 0; i < n_pairs; ++i) {
    if (!events[2 * i] || !events[2 * i + 1]) {
      ms[i] = std::nanf("");
      continue;
    }
    if (hipEventSynchronize((hipEvent_t)events[2 * i + 1]) != hipSuccess) return MITA_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, (hipEvent_t)events[2 * i], (hipEvent_t)events[2 * i + 1]) != hipSuccess)
      return MITA_ERR_HIP;
    ms[i] = t;
  }
  return MITA_OK;
}

const char* mita_status_str(mita_status status) {
  switch (status) {
    case MITA_OK: return "ok";
    case MITA_ERR_NULL: return "a required pointer is NULL";
    case MITA_ERR_SHAPE: return "inconsistent shape (B, H, N, d, pooling grid or m)";
    case MITA_ERR_PARAM: return "k or s out of range, or a pointer is not 16-byte aligned";
    case MITA_ERR_UNSUPPORTED: return "unsupported configuration (d, dtype, s, m, N or k limit)";
    case MITA_ERR_WORKSPACE: return "workspace smaller than mita_workspace_bytes()";
    case MITA_ERR_HIP: return "HIP runtime error while enqueueing";
  }
  return "unknown status";
}

const char* mita_version(void) { return "mita-gfx950 0.1"; }

}  // extern "C"
