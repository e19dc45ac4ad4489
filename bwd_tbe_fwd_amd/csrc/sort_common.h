// Device helpers of the sorting and routing kernels (transpose.hip).
#pragma once

#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {

// ---------------------------------------------------------------------------
// block-wide scans (256 threads)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* s_tmp,
                                                        uint32_t* total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  uint32_t inc = v;
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  if (lane == kWave - 1) s_tmp[w] = inc;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k) {
    const uint32_t x = s_tmp[k];
    if (k < w) pre += x;
    tot += x;
  }
  __syncthreads();
  if (total) *total = tot;
  return pre + inc - v;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* s_tmp) {
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) s_tmp[w] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k) t += s_tmp[k];
  __syncthreads();
  return t;
}

// lanes whose digit equals this lane's digit, among the lanes in `valid`
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int bits, uint64_t valid) {
  uint64_t peers = valid;
  for (int b = 0; b < bits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// Short-run descriptor lists, one per width bucket next_pow2(D) (capacity 0: not written).
struct ShortLists {
  uint4* p[TBE_NUM_BUCKETS];
  int64_t cap[TBE_NUM_BUCKETS];
};

constexpr int kCats = 1 + TBE_NUM_BUCKETS;  // run categories: 0 long, 1 + b short in bucket b
constexpr int kClsRows = kCats + 1;         // + the chunks of the long runs

}  // namespace tbe
