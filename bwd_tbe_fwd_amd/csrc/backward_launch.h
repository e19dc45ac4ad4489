// Host launcher of the short-run and long-apply kernels for one weight format.
#pragma once

#include "backward_kernels.h"

namespace tbe {

namespace detail {

constexpr int kShortUnroll = 4;
// gradient rows in flight per run for the short-run grids on a shared counter (held to part of
// every CU beside the dense rows): fewer waves, so more rows each (skewed batch 9.40 -> 9.25 ms;
// at full occupancy 8 rows cost the uniform batch's tiny runs 7 %)
constexpr int kShortUnrollShared = 8;
constexpr int kTinyUnroll = 2;

// float4 column chunks per lane: one (BD / 4 lanes per run) up to 256 columns, then all 64
// lanes with BD / 256 chunks.  Steps of tiny runs of rows 64 .. 256 wide take two chunks
// (half the lanes per run); narrower rows already put 8 or more runs in a wave step, wider
// rows hold 8 or 16 floats a lane, and more would cost waves
constexpr int short_chunks(int BD, bool tiny) {
  const int np = BD >= 256 ? BD / 256 : 1;
  return (tiny && BD >= 64 && BD <= 256) ? 2 : np;
}

// reserve > 0: the grid leaves that share (in 1/512) of every SIMD free for a kernel on another
// stream: of the workgroups a CU holds (a workgroup is one wave on each of its four SIMDs), the
// grid takes the share 1 - reserve / 512, at least one
template <int DT, int BD, int OPT, bool WEIGHTED>
tbe_status short_go(void* W, float* momentum, const float* psw, const float* grad_out,
                    const uint32_t* pay, const uint32_t* bag_of, const uint4* list,
                    const int32_t* count, int tiny, int64_t cap, const tbe_tables* tb,
                    float lr, float eps, int reserve, int32_t* work, hipStream_t s) {
  using S = typename Fmt<DT>::S;
  constexpr int NPS = short_chunks(BD, false), NPT = short_chunks(BD, true);
  constexpr int RPW = 2 * kWave / (BD / (4 * NPS));  // runs per wave step
  const int64_t waves = (cap + RPW - 1) / RPW;
  // the shared-counter grids (unweighted only: they serve batches with dense rows) take more
  // rows in flight; the first (beside other kernels, reserve > 0) and the second grid are
  // separate instantiations of the same code
  auto kernel = short_run_kernel<DT, BD, NPS, NPT, OPT, WEIGHTED, kShortUnroll, kTinyUnroll, 0>;
  if constexpr (WEIGHTED) {
    // the shared counter comes with the dense rows, which per-sample weights rule out; a grid
    // that ignored it would serve every run a second time
    if (work) {
      set_error("shared short-run grids serve batches without per-sample weights only");
      return TBE_ERR_ARG;
    }
  } else {
    if (work)
      kernel = reserve > 0 ? short_run_kernel<DT, BD, NPS, NPT, OPT, WEIGHTED, kShortUnrollShared, kTinyUnroll, 1>
                           : short_run_kernel<DT, BD, NPS, NPT, OPT, WEIGHTED, kShortUnrollShared, kTinyUnroll, 2>;
  }
  const int64_t want = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  int grid = resident_grid(kernel, want);
  // when the whole upstream gradient fits the 256 MB Infinity Cache, a grid of four times what
  // the CUs hold balances the waves (a slot that frees up takes the next workgroup) at no cost in
  // locality (mixed-width batch, 252 MB: 1.07 -> 0.93 ms); a larger gradient needs the resident
  // grid's window of runs in key order, whose tables' gradient slices stay in that cache (skewed
  // 3.48 -> 4.23 ms and uniform 4.16 -> 4.34 ms at four times)
  if (!work && static_cast<int64_t>(tb->B) * tb->out_width * 4 <= kInfinityCacheBytes)
    grid = static_cast<int>(hmin(want, 4 * static_cast<int64_t>(grid)));
  // the second grid on a shared counter is timed under its own name, so that the first one's
  // time is the short runs' span
  if (reserve > 0) {
    const int fit = hmax(1, blocks_per_cu(reinterpret_cast<const void*>(kernel)) * (512 - reserve) / 512);
    grid = static_cast<int>(hmin(grid, static_cast<int64_t>(device_cu_count()) * fit));
  }
  ProfScope ps(work && reserve == 0 ? "short_run_more" : "short_run", s);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s,
                     static_cast<S*>(W), momentum, grad_out, pay, bag_of, psw, list, count, cap, tiny,
                     tb->meta, tb->B, tb->out_width, lr, eps, work);
  return check_launch("short_run");
}

template <int DT, int OPT, bool WEIGHTED>
tbe_status short_bucket(int b, void* W, float* momentum, const float* psw, const float* grad_out,
                        const uint32_t* pay, const uint32_t* bag_of, const uint4* list,
                        const int32_t* count, int tiny, int64_t cap,
                        const tbe_tables* tb, float lr, float eps, int reserve, int32_t* work,
                        hipStream_t s) {
#define TBE_SB(BD) short_go<DT, BD, OPT, WEIGHTED>(W, momentum, psw, grad_out, pay, bag_of, list, count, tiny, cap, tb, lr, eps, reserve, work, s)
  switch (b) {
    case 0: return TBE_SB(4);
    case 1: return TBE_SB(8);
    case 2: return TBE_SB(16);
    case 3: return TBE_SB(32);
    case 4: return TBE_SB(64);
    case 5: return TBE_SB(128);
    case 6: return TBE_SB(256);
    case 7: return TBE_SB(512);
    default: return TBE_SB(1024);
  }
#undef TBE_SB
}

template <int DT, int OPT>
tbe_status apply_go(void* W, float* momentum, const uint4* long_list, const uint32_t* long_table,
                    const int32_t* counters, int64_t cap, const tbe_tables* tb, int chunk,
                    const float* partial, const uint32_t* long_flag, float lr, float eps, hipStream_t s) {
  using S = typename Fmt<DT>::S;
  const auto kernel = long_apply_kernel<DT, OPT>;
  const int grid = resident_grid(kernel, cap);
  ProfScope ps("long_apply", s);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<S*>(W),
                     momentum, long_list, long_table, counters, tb->meta, chunk, tb->max_D, partial, long_flag,
                     lr, eps);
  return check_launch("long_apply");
}

template <int DT, int OPT, bool WEIGHTED>
tbe_status fused_go(void* W, float* momentum, const float* psw, const float* grad_out, char* ws,
                    const BwdLayout& L, int final_buf, const Config& cfg, const uint32_t* order,
                    const tbe_tables* tb, float lr, float eps, hipStream_t s) {
  using S = typename Fmt<DT>::S;
  const int64_t batches = (L.cap_chunk + kFusedBatch - 1) / kFusedBatch;
  const auto kernel = long_fused_kernel<DT, OPT, WEIGHTED>;
  const int grid = resident_grid(kernel, (batches + kWavesPerBlock - 1) / kWavesPerBlock);
  ProfScope ps("long_fused", s);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s,
                     static_cast<S*>(W), momentum, grad_out,
                     reinterpret_cast<const uint32_t*>(ws + L.pay[final_buf]),
                     WEIGHTED ? reinterpret_cast<const uint32_t*>(ws + L.bag_of) : nullptr, psw,
                     reinterpret_cast<const uint4*>(ws + L.long_list),
                     reinterpret_cast<const uint32_t*>(ws + L.long_table),
                     reinterpret_cast<uint32_t*>(ws + L.long_count),
                     reinterpret_cast<const uint2*>(ws + L.chunk_list), order,
                     reinterpret_cast<const int32_t*>(ws + L.counters), tb->meta, tb->B, tb->out_width,
                     cfg.chunk, tb->max_D, reinterpret_cast<float*>(ws + L.partial), lr, eps);
  return check_launch("long_fused");
}

}  // namespace detail

tbe_status launch_grad_accum(const tbe_tables* tb, const float* psw, const float* grad_out,
                             char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                             hipStream_t s);

// the long runs' chunks and their apply on s
template <int DT>
tbe_status long_runs_and_apply(const tbe_tables* tb, void* W, float* momentum, int opt,
                               const float* psw, const float* grad_out, float lr, float eps,
                               char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                               hipStream_t s);

template <int DT>
tbe_status launch_short_and_apply(const tbe_tables* tb, void* W, float* momentum, int opt,
                                  const float* psw, const float* grad_out, float lr, float eps,
                                  char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                                  hipStream_t s, hipStream_t s_long) {
  const int32_t* counters = reinterpret_cast<const int32_t*>(ws + L.counters);
  const uint32_t* pay = reinterpret_cast<const uint32_t*>(ws + L.pay[final_buf]);
  const uint32_t* bag_of = psw ? reinterpret_cast<const uint32_t*>(ws + L.bag_of) : nullptr;
  // the short runs of every bucket on stream ss, the grid leaving `reserve` free
  auto short_runs = [&](hipStream_t ss, int reserve) -> tbe_status {
    for (int b = 0; b < TBE_NUM_BUCKETS; ++b) {
      if (!L.cap_short[b]) continue;
      const uint4* list = reinterpret_cast<const uint4*>(ws + L.short_list[b]);
      const int64_t cap = L.cap_short[b];
      const int32_t* cnt = counters + kShort0 + b;
#define TBE_SHORT(OPT, WTD) \
  detail::short_bucket<DT, OPT, WTD>(b, W, momentum, psw, grad_out, pay, bag_of, list, cnt, cfg.tiny, cap, tb, lr, eps, \
                                     reserve, cfg.short_work, ss)
      const tbe_status st = opt == kOptSGD ? (psw ? TBE_SHORT(kOptSGD, true) : TBE_SHORT(kOptSGD, false))
                                           : (psw ? TBE_SHORT(kOptAdagrad, true) : TBE_SHORT(kOptAdagrad, false));
#undef TBE_SHORT
      if (st) return st;
    }
    return TBE_OK;
  };
  if (tbe_status st = short_runs(s, cfg.short_reserve)) return st;
  // long runs touch other rows than short runs: s_long may be a second stream
  if (tbe_status st = long_runs_and_apply<DT>(tb, W, momentum, opt, psw, grad_out, lr, eps, ws, L, final_buf,
                                          cfg, s_long))
    return st;
  // with a shared work counter, a second short-run grid on the long runs' stream, after them,
  // takes the short runs the first grid has not reached (one wave step at a time)
  if (cfg.short_work && s_long != s) return short_runs(s_long, 0);
  return TBE_OK;
}

template <int DT>
tbe_status long_runs_and_apply(const tbe_tables* tb, void* W, float* momentum, int opt,
                               const float* psw, const float* grad_out, float lr, float eps,
                               char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                               hipStream_t s) {
  const int32_t* counters = reinterpret_cast<const int32_t*>(ws + L.counters);
  if (L.cap_long == 0) return TBE_OK;
  if (cfg.fused_long) {
    const uint32_t* order = nullptr;
    if (tbe_status st = launch_chunk_order(tb, psw, ws, L, final_buf, cfg, &order, s)) return st;
    if (opt == kOptSGD)
      return psw ? detail::fused_go<DT, kOptSGD, true>(W, momentum, psw, grad_out, ws, L, final_buf, cfg, order, tb, lr, eps, s)
                 : detail::fused_go<DT, kOptSGD, false>(W, momentum, psw, grad_out, ws, L, final_buf, cfg, order, tb, lr, eps, s);
    return psw ? detail::fused_go<DT, kOptAdagrad, true>(W, momentum, psw, grad_out, ws, L, final_buf, cfg, order, tb, lr, eps, s)
               : detail::fused_go<DT, kOptAdagrad, false>(W, momentum, psw, grad_out, ws, L, final_buf, cfg, order, tb, lr, eps, s);
  }
  if (tbe_status st = launch_grad_accum(tb, psw, grad_out, ws, L, final_buf, cfg, s)) return st;
  const uint4* long_list = reinterpret_cast<const uint4*>(ws + L.long_list);
  const uint32_t* long_table = reinterpret_cast<const uint32_t*>(ws + L.long_table);
  const float* partial = reinterpret_cast<const float*>(ws + L.partial);
  // dense rows picked from the long runs: their slots are skipped
  const uint32_t* long_flag =
      L.dense_on && !L.dense_presort ? reinterpret_cast<const uint32_t*>(ws + L.long_flag) : nullptr;
  if (opt == kOptSGD)
    return detail::apply_go<DT, kOptSGD>(W, momentum, long_list, long_table, counters, L.cap_long, tb, cfg.chunk, partial, long_flag, lr, eps, s);
  return detail::apply_go<DT, kOptAdagrad>(W, momentum, long_list, long_table, counters, L.cap_long, tb, cfg.chunk, partial, long_flag, lr, eps, s);
}

}  // namespace tbe
