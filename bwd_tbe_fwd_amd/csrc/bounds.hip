// Bounds check and repair of offsets and indices.
//
// PyTorch blog "Modernizing Table Batched Embeddings with FBTriton", section 2,
// "Bounds checking": invalid inputs are validated and repaired before the
// forward, and offsets get their own small repair step; "Table-Batched
// Embeddings in Triton", Pitfalls: an id outside its table silently reads
// another table's row.  The pages give no repair rule.  The rule here:
//   offsets: o'[0] = 0, o'[T*B] = N, o'[i] = max(o'[i-1], clamp(o[i], 0, N))
//            (a running maximum, so bags stay disjoint and ordered);
//   indices: an id outside [0, E_t) of the table owning its position
//            (positions [o'[t*B], o'[(t+1)*B])) becomes 0.
// Every changed entry is counted; counts = {indices repaired, offsets changed}.
//
// The running maximum is a device-wide scan done reduce-then-scan: per-block
// maxima, one small scan of them, then each block rescans its segment seeded
// with its prefix.  Counts use one atomic per block.
#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {
namespace {

constexpr int kBoundsBlocks = 1024;

__global__ void bounds_init_kernel(int64_t* counts) {
  if (threadIdx.x < 2) counts[threadIdx.x] = 0;
}

template <typename OT>
__device__ __forceinline__ int64_t clamped_offset(const OT* o, int64_t i, int64_t nb, int64_t N) {
  if (i == 0) return 0;
  if (i == nb) return N;
  int64_t v = static_cast<int64_t>(o[i]);
  return min(max(v, static_cast<int64_t>(0)), N);
}

__device__ __forceinline__ int64_t block_max(int64_t v, int64_t* s_tmp) {
  for (int m = 1; m < kWave; m <<= 1) v = max(v, static_cast<int64_t>(__shfl_xor(v, m)));
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) s_tmp[w] = v;
  __syncthreads();
  int64_t r = s_tmp[0];
  for (int i = 1; i < kWavesPerBlock; ++i) r = max(r, s_tmp[i]);
  __syncthreads();
  return r;
}

template <typename OT>
__global__ __launch_bounds__(kBlock) void bounds_offsets_reduce(const OT* __restrict__ off,
                                                                 int64_t nb, int64_t N, int64_t seg,
                                                                 int64_t* __restrict__ bmax) {
  __shared__ int64_t s_tmp[kWavesPerBlock];
  const int64_t lo = blockIdx.x * seg, hi = min(lo + seg, nb + 1);
  int64_t v = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) v = max(v, clamped_offset(off, i, nb, N));
  v = block_max(v, s_tmp);
  if (threadIdx.x == 0) bmax[blockIdx.x] = v;
}

// exclusive running maximum of the block maxima (one workgroup, <= 4 per thread)
__global__ __launch_bounds__(kBlock) void bounds_offsets_scan(const int64_t* __restrict__ bmax,
                                                               int64_t* __restrict__ prefix, int nblk) {
  __shared__ int64_t s_wave[kWavesPerBlock];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int64_t v[4];
  int64_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * threadIdx.x + k;
    v[k] = i < nblk ? bmax[i] : 0;
    m = max(m, v[k]);
  }
  int64_t inc = m;  // inclusive wave scan of the per-thread maxima
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t u = __shfl_up(inc, d);
    if (lane >= d) inc = max(inc, u);
  }
  if (lane == kWave - 1) s_wave[w] = inc;
  __syncthreads();
  int64_t pre = 0;
  for (int k = 0; k < w; ++k) pre = max(pre, s_wave[k]);
  int64_t ex = __shfl_up(inc, 1);
  if (lane == 0) ex = 0;
  int64_t run = max(pre, ex);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * threadIdx.x + k;
    if (i < nblk) prefix[i] = run;
    run = max(run, v[k]);
  }
}

template <typename OT>
__global__ __launch_bounds__(kBlock) void bounds_offsets_apply(OT* __restrict__ off, int64_t nb,
                                                                int64_t N, int64_t seg,
                                                                const int64_t* __restrict__ prefix,
                                                                int64_t* __restrict__ counts) {
  __shared__ int64_t s_wave[kWavesPerBlock];
  __shared__ int64_t s_carry;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int64_t lo = blockIdx.x * seg, hi = min(lo + seg, nb + 1);
  if (threadIdx.x == 0) s_carry = prefix[blockIdx.x];
  __syncthreads();
  int64_t changed = 0;
  for (int64_t base = lo; base < hi; base += kBlock) {
    const int64_t i = base + threadIdx.x;
    const bool valid = i < hi;
    int64_t v = valid ? clamped_offset(off, i, nb, N) : 0;
    // inclusive running max within the wave, then across waves, then the carry
    for (int d = 1; d < kWave; d <<= 1) {
      const int64_t u = __shfl_up(v, d);
      if (lane >= d) v = max(v, u);
    }
    if (lane == kWave - 1) s_wave[w] = v;
    __syncthreads();
    int64_t pre = s_carry;
    for (int k = 0; k < w; ++k) pre = max(pre, s_wave[k]);
    v = max(v, pre);
    if (valid) {
      const int64_t old = static_cast<int64_t>(off[i]);
      if (old != v) {
        off[i] = static_cast<OT>(v);
        ++changed;
      }
    }
    __syncthreads();
    if (threadIdx.x == kBlock - 1) s_carry = v;  // invalid lanes held 0, so this is the tile max
    __syncthreads();
  }
  // one atomic per block
  for (int m = 1; m < kWave; m <<= 1) changed += __shfl_xor(changed, m);
  if (lane == 0) s_wave[w] = changed;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t c = 0;
    for (int k = 0; k < kWavesPerBlock; ++k) c += s_wave[k];
    if (c) atomicAdd(reinterpret_cast<unsigned long long*>(&counts[1]), static_cast<unsigned long long>(c));
  }
}

// the table owning position p: largest t with start[t] <= p, start[t] = o'[t*B]
template <typename OT>
__device__ __forceinline__ int owner_table(const OT* off, const int64_t* s_start, int T, int64_t B,
                                           int64_t p) {
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t v = s_start ? s_start[mid] : static_cast<int64_t>(off[mid * B]);
    if (v <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kLdsTables = 2048;

// Each thread checks 4 positions per step, a grid stride apart, so four
// independent loads are in flight; the owning table is found by binary search
// over the repaired table starts held in LDS.
template <typename IT, typename OT>
__global__ __launch_bounds__(kBlock) void bounds_indices(IT* __restrict__ idx, int64_t N,
                                                          const OT* __restrict__ off,
                                                          const int64_t* __restrict__ meta, int T,
                                                          int64_t B, int64_t* __restrict__ counts) {
  __shared__ int64_t s_start[kLdsTables + 1];
  __shared__ int64_t s_E[kLdsTables];
  __shared__ int64_t s_cnt[kWavesPerBlock];
  const bool lds = T <= kLdsTables;
  if (lds)
    for (int t = threadIdx.x; t <= T; t += kBlock) {
      s_start[t] = static_cast<int64_t>(off[t * B]);
      if (t < T) s_E[t] = meta[4 * (t + 1)] - meta[4 * t];
    }
  __syncthreads();
  const int64_t lo_t = lds ? s_start[0] : static_cast<int64_t>(off[0]);
  const int64_t hi_t = lds ? s_start[T] : static_cast<int64_t>(off[T * B]);
  int64_t fixed = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t p0 = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; p0 < N; p0 += 4 * stride) {
    int64_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t p = p0 + k * stride;
      v[k] = p < N ? static_cast<int64_t>(idx[p]) : 0;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t p = p0 + k * stride;
      if (p >= N || p < lo_t || p >= hi_t) continue;  // outside every bag: cannot happen after repair
      const int t = owner_table(off, lds ? s_start : nullptr, T, B, p);
      const int64_t E = lds ? s_E[t] : meta[4 * (t + 1)] - meta[4 * t];
      if (static_cast<uint64_t>(v[k]) >= static_cast<uint64_t>(E)) {
        idx[p] = 0;
        ++fixed;
      }
    }
  }
  for (int m = 1; m < kWave; m <<= 1) fixed += __shfl_xor(fixed, m);
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) s_cnt[w] = fixed;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t c = 0;
    for (int k = 0; k < kWavesPerBlock; ++k) c += s_cnt[k];
    if (c) atomicAdd(reinterpret_cast<unsigned long long*>(&counts[0]), static_cast<unsigned long long>(c));
  }
}

template <typename OT>
tbe_status offsets_go(const tbe_tables* tb, void* offsets, int64_t N, int64_t* counts, void* ws,
                      hipStream_t s) {
  const int64_t nb = static_cast<int64_t>(tb->T) * tb->B;
  int64_t* bmax = static_cast<int64_t*>(ws);
  int64_t* prefix = bmax + kBoundsBlocks;
  const int64_t seg0 = (nb + 1 + kBoundsBlocks - 1) / kBoundsBlocks;
  const int64_t seg = ((seg0 + kBlock - 1) / kBlock) * kBlock;
  const int nblk = static_cast<int>((nb + 1 + seg - 1) / seg);
  {
    ProfScope ps("bounds_init", s);
    hipLaunchKernelGGL(bounds_init_kernel, dim3(1), dim3(64), 0, s, counts);
  }
  if (tbe_status st = check_launch("bounds_init")) return st;
  ProfScope ps("bounds_offsets", s);
  hipLaunchKernelGGL((bounds_offsets_reduce<OT>), dim3(nblk), dim3(kBlock), 0, s,
                     static_cast<const OT*>(offsets), nb, N, seg, bmax);
  hipLaunchKernelGGL(bounds_offsets_scan, dim3(1), dim3(kBlock), 0, s, bmax, prefix, nblk);
  hipLaunchKernelGGL((bounds_offsets_apply<OT>), dim3(nblk), dim3(kBlock), 0, s,
                     static_cast<OT*>(offsets), nb, N, seg, prefix, counts);
  return check_launch("bounds_offsets");
}

template <typename IT, typename OT>
tbe_status indices_go(const tbe_tables* tb, void* indices, const void* offsets, int64_t N,
                      int64_t* counts, hipStream_t s) {
  if (N <= 0) return TBE_OK;
  const int64_t want = (N + kBlock * 16 - 1) / (kBlock * 16);
  const int grid = static_cast<int>(hmax(1, hmin(want, static_cast<int64_t>(device_cu_count()) * 8)));
  ProfScope ps("bounds_indices", s);
  hipLaunchKernelGGL((bounds_indices<IT, OT>), dim3(grid), dim3(kBlock), 0, s,
                     static_cast<IT*>(indices), N, static_cast<const OT*>(offsets), tb->meta,
                     tb->T, static_cast<int64_t>(tb->B), counts);
  return check_launch("bounds_indices");
}

}  // namespace

size_t bounds_workspace(const tbe_tables*) { return 2 * kBoundsBlocks * sizeof(int64_t); }

tbe_status launch_bounds_offsets(const tbe_tables* tb, void* offsets, int otype, int64_t N,
                                 int64_t* counts, void* ws, hipStream_t s) {
  if (otype == TBE_I32) return offsets_go<int32_t>(tb, offsets, N, counts, ws, s);
  return offsets_go<int64_t>(tb, offsets, N, counts, ws, s);
}

tbe_status launch_bounds_indices(const tbe_tables* tb, void* indices, int itype, const void* offsets,
                                 int otype, int64_t N, int64_t* counts, hipStream_t s) {
  if (itype == TBE_I32) {
    if (otype == TBE_I32) return indices_go<int32_t, int32_t>(tb, indices, offsets, N, counts, s);
    return indices_go<int32_t, int64_t>(tb, indices, offsets, N, counts, s);
  }
  if (otype == TBE_I32) return indices_go<int64_t, int32_t>(tb, indices, offsets, N, counts, s);
  return indices_go<int64_t, int64_t>(tb, indices, offsets, N, counts, s);
}

tbe_status launch_bounds(const tbe_tables* tb, void* indices, int itype, void* offsets, int otype,
                         int64_t N, int64_t* counts, void* ws, hipStream_t s) {
  if (tbe_status st = launch_bounds_offsets(tb, offsets, otype, N, counts, ws, s)) return st;
  return launch_bounds_indices(tb, indices, itype, offsets, otype, N, counts, s);
}

}  // namespace tbe
