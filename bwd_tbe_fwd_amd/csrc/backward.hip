// Long-run gradient accumulation (split into fixed-size chunks) and the
// backward's update orchestration.
//
// After PyTorch blog "Modernizing Table Batched Embeddings with FBTriton",
// section 4 (problem 1) and section 3 (grad_accum, then an apply kernel): a
// run at or above the threshold is cut into 256-lookup chunks, so that one hot
// row's lookups are summed by many waves at once, like a split reduction.
// Here every chunk writes its own fp32 partial row into the workspace (no
// atomics), and the apply kernel adds a run's partials in a fixed order and
// steps the optimizer, so the result does not depend on scheduling.
#include "backward_kernels.h"

namespace tbe {
namespace {

// One wave per chunk (accumulate_chunk in backward_kernels.h).
template <bool WEIGHTED, int UNROLL>
__global__ __launch_bounds__(kBlock) void grad_accum_kernel(
    const float* __restrict__ grad_out, const uint32_t* __restrict__ pay,
    const uint32_t* __restrict__ bag_of, const float* __restrict__ psw,
    const uint4* __restrict__ long_list, const uint32_t* __restrict__ long_table,
    const uint2* __restrict__ chunk_list, const int32_t* __restrict__ counters,
    const int64_t* __restrict__ meta, int32_t B, int32_t out_width, int chunk, int max_D,
    const uint32_t* __restrict__ order, const uint32_t* __restrict__ long_flag,
    float* __restrict__ partial) {
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
  const int64_t n = counters[kChunks];
  for (int64_t i = wave; i < n; i += nwaves) {
    const int64_t cix = order ? order[i] : i;
    const uint2 ch = chunk_list[cix];
    if (long_flag && long_flag[ch.x]) continue;  // a dense row: updated by the dense path
    const uint4 L = long_list[ch.x];
    const int t = static_cast<int>(long_table[ch.x]);
    const TableMeta m = load_meta(meta, t);
    const uint32_t lo = L.y + ch.y * static_cast<uint32_t>(chunk);
    const uint32_t hi = min(lo + static_cast<uint32_t>(chunk), L.y + L.z);
    accumulate_chunk<WEIGHTED, UNROLL>(grad_out, pay, bag_of, psw, m, t, B, out_width, lo, hi,
                                       partial + cix * max_D);
  }
}

// Long-run chunk ordering: the chunks are regrouped by (table, window of bags of
// their first lookup), so that chunks processed at the same time read gradient
// rows of the same few thousand bags - rows that many long runs share - and find
// them in L2.  A counting sort: units counted, scanned, then chunks scattered.
__global__ __launch_bounds__(kBlock) void chunk_units_kernel(
    const uint2* __restrict__ chunk_list, const uint4* __restrict__ long_list,
    const uint32_t* __restrict__ long_table, const uint32_t* __restrict__ pay,
    const uint32_t* __restrict__ bag_of, const int32_t* __restrict__ counters, int chunk, int B,
    int nwin, int win_size, uint32_t* __restrict__ chunk_unit, uint32_t* __restrict__ unit_cnt) {
  const int64_t n = counters[kChunks];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; c < n; c += stride) {
    const uint2 ch = chunk_list[c];
    const uint4 L = long_list[ch.x];
    const uint32_t t = long_table[ch.x];
    const uint32_t p = pay[L.y + ch.y * static_cast<uint32_t>(chunk)];
    const int64_t bag = bag_of ? static_cast<int64_t>(bag_of[p]) : static_cast<int64_t>(p);
    int64_t b = bag - static_cast<int64_t>(t) * B;
    b = min(max(b, static_cast<int64_t>(0)), static_cast<int64_t>(B - 1));
    const uint32_t u = t * static_cast<uint32_t>(nwin) + static_cast<uint32_t>(b / win_size);
    chunk_unit[c] = u;
    atomicAdd(&unit_cnt[u], 1u);
  }
}

// exclusive scan of the unit counts in place (one workgroup, units <= 4096)
__global__ __launch_bounds__(kBlock) void unit_scan_kernel(uint32_t* __restrict__ cnt, int units) {
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int ipt = (units + kBlock - 1) / kBlock;
  const int i0 = threadIdx.x * ipt;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    v[q] = (q < ipt && i0 + q < units) ? cnt[i0 + q] : 0u;
    sum += v[q];
  }
  uint32_t inc = sum;
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  if (lane == kWave - 1) s_tmp[w] = inc;
  __syncthreads();
  uint32_t run = inc - sum;
  for (int k = 0; k < w; ++k) run += s_tmp[k];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < ipt && i0 + q < units) cnt[i0 + q] = run;
    run += v[q];
  }
}

__global__ __launch_bounds__(kBlock) void chunk_scatter_kernel(const uint32_t* __restrict__ chunk_unit,
                                                               uint32_t* __restrict__ unit_pos,
                                                               const int32_t* __restrict__ counters,
                                                               uint32_t* __restrict__ order) {
  const int64_t n = counters[kChunks];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; c < n; c += stride)
    order[atomicAdd(&unit_pos[chunk_unit[c]], 1u)] = static_cast<uint32_t>(c);
}

template <bool WEIGHTED>
tbe_status accum_go(const tbe_tables* tb, const float* psw, const float* grad_out, char* ws,
                    const BwdLayout& L, int final_buf, const Config& cfg, hipStream_t s) {
  const int64_t work = (L.cap_chunk + kWavesPerBlock - 1) / kWavesPerBlock;
  const uint32_t* pay = reinterpret_cast<const uint32_t*>(ws + L.pay[final_buf]);
  const uint32_t* bag_of = WEIGHTED ? reinterpret_cast<const uint32_t*>(ws + L.bag_of) : nullptr;
  const uint32_t* order = nullptr;
  if (tbe_status st = launch_chunk_order(tb, psw, ws, L, final_buf, cfg, &order, s)) return st;
  // dense rows picked from the long runs: their chunks are skipped
  const uint32_t* long_flag =
      L.dense_on && !L.dense_presort ? reinterpret_cast<const uint32_t*>(ws + L.long_flag) : nullptr;
  ProfScope ps("grad_accum", s);
  // eight times the workgroups the CUs hold (at most one wave per chunk): each wave takes
  // about one chunk, and a slot that frees up takes the next workgroup, so the CUs that drew
  // slow chunks do not set the end (skewed batch 1.02 -> 0.96 ms alone, mixed 0.67 -> 0.65 ms)
#define TBE_ACC(U)                                                                                 \
  hipLaunchKernelGGL((grad_accum_kernel<WEIGHTED, U>),                                             \
                     dim3(hmin(work, 8 * static_cast<int64_t>(resident_grid(grad_accum_kernel<WEIGHTED, U>, work)))), \
                     dim3(kBlock), 0, s, grad_out, pay,                                             \
                     bag_of, psw, reinterpret_cast<const uint4*>(ws + L.long_list),               \
                     reinterpret_cast<const uint32_t*>(ws + L.long_table),                        \
                     reinterpret_cast<const uint2*>(ws + L.chunk_list),                           \
                     reinterpret_cast<const int32_t*>(ws + L.counters), tb->meta, tb->B,           \
                     tb->out_width, cfg.chunk, tb->max_D, order, long_flag,                       \
                     reinterpret_cast<float*>(ws + L.partial))
  if (cfg.bwd_unroll <= 2) TBE_ACC(2);
  else if (cfg.bwd_unroll <= 4) TBE_ACC(4);
  else TBE_ACC(8);
#undef TBE_ACC
  return check_launch("grad_accum");
}

}  // namespace

tbe_status launch_chunk_order(const tbe_tables* tb, const float* psw, char* ws, const BwdLayout& L,
                              int final_buf, const Config& cfg, const uint32_t** order, hipStream_t s) {
  *order = nullptr;
  if (L.nwin <= 1) return TBE_OK;
  const int64_t maxb = static_cast<int64_t>(device_cu_count()) * 8;
  const uint32_t* pay = reinterpret_cast<const uint32_t*>(ws + L.pay[final_buf]);
  const uint32_t* bag_of = psw ? reinterpret_cast<const uint32_t*>(ws + L.bag_of) : nullptr;
  uint32_t* unit_cnt = reinterpret_cast<uint32_t*>(ws + L.unit_cnt);
  uint32_t* chunk_unit = reinterpret_cast<uint32_t*>(ws + L.chunk_unit);
  uint32_t* chunk_order = reinterpret_cast<uint32_t*>(ws + L.chunk_order);
  if (tbe_status st = launch_fill_i32(reinterpret_cast<int32_t*>(unit_cnt), 0, L.units, s)) return st;
  const int g2 = static_cast<int>(hmax(1, hmin((L.cap_chunk + kBlock - 1) / kBlock, maxb)));
  ProfScope ps("chunk_order", s);
  hipLaunchKernelGGL(chunk_units_kernel, dim3(g2), dim3(kBlock), 0, s,
                     reinterpret_cast<const uint2*>(ws + L.chunk_list),
                     reinterpret_cast<const uint4*>(ws + L.long_list),
                     reinterpret_cast<const uint32_t*>(ws + L.long_table), pay, bag_of,
                     reinterpret_cast<const int32_t*>(ws + L.counters), cfg.chunk, tb->B, L.nwin,
                     L.win_size, chunk_unit, unit_cnt);
  hipLaunchKernelGGL(unit_scan_kernel, dim3(1), dim3(kBlock), 0, s, unit_cnt, L.units);
  hipLaunchKernelGGL(chunk_scatter_kernel, dim3(g2), dim3(kBlock), 0, s, chunk_unit, unit_cnt,
                     reinterpret_cast<const int32_t*>(ws + L.counters), chunk_order);
  if (tbe_status st = check_launch("chunk_order")) return st;
  *order = chunk_order;
  return TBE_OK;
}

tbe_status launch_grad_accum(const tbe_tables* tb, const float* psw, const float* grad_out,
                             char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                             hipStream_t s) {
  if (psw) return accum_go<true>(tb, psw, grad_out, ws, L, final_buf, cfg, s);
  return accum_go<false>(tb, psw, grad_out, ws, L, final_buf, cfg, s);
}

tbe_status launch_backward_update(const tbe_tables* tb, void* W, float* momentum, int opt,
                                  const float* psw, const float* grad_out, float lr, float eps,
                                  char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                                  hipStream_t s, hipStream_t s_long) {
  if (L.N == 0) return TBE_OK;
  switch (tb->w_dtype) {
    case TBE_F32:
      return launch_short_and_apply<0>(tb, W, momentum, opt, psw, grad_out, lr, eps, ws, L, final_buf, cfg, s, s_long);
    case TBE_F16:
      return launch_short_and_apply<1>(tb, W, momentum, opt, psw, grad_out, lr, eps, ws, L, final_buf, cfg, s, s_long);
    default:
      return launch_short_and_apply<2>(tb, W, momentum, opt, psw, grad_out, lr, eps, ws, L, final_buf, cfg, s, s_long);
  }
}

}  // namespace tbe
