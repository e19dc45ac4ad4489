// Backward of the small histogram table: per-bag lookup counts times the
// output gradient on MFMA, then one optimizer step per touched row.
//
// PyTorch blog "Modernizing Table Batched Embeddings with FBTriton", section 2,
// "forward-state reuse and preprocessing": for the table the histogram forward
// serves, exact row-wise Adagrad takes its gradient from the bags' row counts
// (a dense counts-transposed times grad_out product accumulated in fp32) instead
// of a per-lookup scatter, and then applies the optimizer.  For row r of a table
// with at most 64 rows,
//     g[r, :] = sum_b count_b[r] * grad_out[b, col_t : col_t + D],
// which equals the sum over every lookup of r of its bag's gradient row: the
// same gradient the sorted-run path produces, read from the B x D gradient slice
// once instead of once per lookup.
//
// gfx950 mapping.  A workgroup takes 64 consecutive bags per step.  Each of its
// four waves counts ALL lookups of 16 of those bags (not only a bag's first
// 256: the counts are never rounded to fp16 here) into the shared LDS array
// count[64 bags][64 rows], reading the bags' ids as one contiguous coalesced
// range and finding each id's bag by a 4-step search of the 17 offsets.  After
// a barrier, wave w multiplies the counts by gradient columns 32 w .. 32 w + 31
// of the 64 bags on v_mfma_f32_16x16x4_f32 in fp32: the counts (integers, exact
// in fp32) are the A operand (rows x bags), the gradient the B operand (bags x
// columns), so no high/low fp16 split of the gradient is needed and every
// product is the fp32 product of an exact count and the fp32 gradient.  The
// 64 x 32 accumulator (4 x 2 MFMA tiles) stays in registers across the steps and
// is written once per workgroup as a partial.  The apply kernel sums a row's
// partials in a fixed order and applies SGD or row-wise Adagrad to rows whose
// count is nonzero, so results are bitwise repeatable.
//
// After the hoisted forward, the counts of each bag's first 256 lookups are the
// ones the histogram forward already made (kept as u16 in the workspace): a wave
// loads them into LDS and reads only the ids past a bag's first 256, so the
// id stream of this table is read once per training step instead of twice.
// The counts are the same integers either way, so the results are bitwise equal.
#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kHbRows = 64;     // table rows: MFMA M, 4 tiles of 16
constexpr int kHbCols = 128;    // max D; each wave owns 32 columns (2 MFMA N tiles)
constexpr int kHbWaveBags = 16; // bags one wave counts per step
constexpr int kHbBags = kHbWaveBags * kWavesPerBlock;  // bags per workgroup step: MFMA K, 16 steps of 4
constexpr int kHbLoads = 8;     // id loads in flight per lane while counting
constexpr int kHbHead = 256;    // ids per bag the histogram forward counts (its saved counts)

__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_wave_barrier(); }

// Workgroup step over 64 consecutive bags: wave w counts bags 16 w .. 16 w + 15
// into the shared count[64 bags][64 rows]; after a barrier every wave multiplies
// the counts by its 32 gradient columns (K = 64 bags).
template <typename IT, typename OT>
__global__ __launch_bounds__(kBlock) void hist_bwd_partial_kernel(
    const IT* __restrict__ indices, const OT* __restrict__ offsets,
    const float* __restrict__ grad_out, int64_t bag0, int32_t B, int32_t E, int32_t D,
    int64_t col_base, int32_t out_width, int64_t N, const uint16_t* __restrict__ saved,
    float* __restrict__ partial, int32_t* __restrict__ pcount) {
  __shared__ __align__(16) uint32_t s_cnt[kHbBags * kHbRows];
  __shared__ int32_t s_off[kWavesPerBlock][kHbWaveBags + 1];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = 32 * w;                 // this wave's first column
  const int c2 = cw + 2 * (lane & 15);   // B operand / result columns c2 (tile 0), c2 + 1 (tile 1)
  float4_t acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt][0] = acc[mt][1] = float4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t rowcnt[4] = {0u, 0u, 0u, 0u};
  uint32_t* mycnt = s_cnt + kHbWaveBags * kHbRows * w;
  int32_t* off = s_off[w];

  const int64_t steps = (static_cast<int64_t>(B) + kHbBags - 1) / kHbBags;
  for (int64_t st = blockIdx.x; st < steps; st += gridDim.x) {
    const int64_t b0 = st * kHbBags;                    // first bag of the workgroup step
    const int nb = static_cast<int>(min<int64_t>(kHbBags, static_cast<int64_t>(B) - b0));
    const int64_t bw = b0 + kHbWaveBags * w;            // first bag this wave counts
    const int nbw = max(0, min(kHbWaveBags, nb - kHbWaveBags * w));
    // gradient rows: lane l holds bags 4 ks + l / 16, columns c2, c2 + 1
    f32x2 gv[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const int i = 4 * ks + (lane >> 4);
      gv[ks] = f32x2{0.f, 0.f};
      if (i < nb && c2 < D)
        gv[ks] = *reinterpret_cast<const f32x2*>(grad_out + (b0 + i) * out_width + col_base + c2);
    }
    // the 17 offsets of this wave's bags, clamped to [0, N] and made monotone (running max)
    int32_t o = 0;
    if (lane <= kHbWaveBags) {
      // waves past the last bag (nbw = 0) read the table's end offset, not beyond it
      const int64_t v = static_cast<int64_t>(offsets[bag0 + min(bw + min(lane, nbw), static_cast<int64_t>(B))]);
      o = static_cast<int32_t>(min(max(v, static_cast<int64_t>(0)), N));
    }
    for (int d = 1; d < 32; d <<= 1) {
      const int32_t u = __shfl_up(o, d);
      if (lane >= d) o = max(o, u);
    }
    const int32_t o0 = read_lane(o, 0);
    const int32_t n = read_lane(o, kHbWaveBags) - o0;
    __syncthreads();  // every wave is done reading the previous step's counts
    if (lane <= kHbWaveBags) off[lane] = o - o0;
    if (saved) {
      // the forward's counts of the 16 bags (the forward pads the last tile with zero counts;
      // a wave past the last bag has none)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = 8 * (k * kWave + lane);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (nbw > 0) v = *reinterpret_cast<const u32x4*>(saved + bw * kHbRows + e);
        reinterpret_cast<u32x4*>(mycnt + e)[0] = u32x4{v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16};
        reinterpret_cast<u32x4*>(mycnt + e)[1] = u32x4{v.z & 0xffffu, v.z >> 16, v.w & 0xffffu, v.w >> 16};
      }
      wave_sync();
      // ids past each bag's first 256
      for (int i = 0; i < nbw; ++i) {
        const int32_t e = off[i + 1];
        for (int32_t j = off[i] + kHbHead + lane; j < e; j += kWave) {
          const int64_t r = static_cast<int64_t>(indices[o0 + j]);
          if (static_cast<uint64_t>(r) < static_cast<uint64_t>(E))
            atomicAdd(&mycnt[i * kHbRows + static_cast<int>(r)], 1u);
        }
      }
    } else {
#pragma unroll
      for (int x = lane; x < kHbWaveBags * kHbRows / 4; x += kWave)
        reinterpret_cast<u32x4*>(mycnt)[x] = u32x4{0u, 0u, 0u, 0u};
      wave_sync();
      // count every lookup of the wave's 16 bags; ids outside [0, E) are dropped
      for (int32_t j0 = 0; j0 < n; j0 += kHbLoads * kWave) {
        int64_t r[kHbLoads];
#pragma unroll
        for (int u = 0; u < kHbLoads; ++u) {
          const int32_t j = j0 + u * kWave + lane;
          r[u] = j < n ? static_cast<int64_t>(indices[o0 + j]) : -1;
        }
#pragma unroll
        for (int u = 0; u < kHbLoads; ++u) {
          const int32_t j = j0 + u * kWave + lane;
          if (static_cast<uint64_t>(r[u]) < static_cast<uint64_t>(E)) {
            int b = 0;  // largest b in [0, 16) with off[b] <= j: the bag of lookup j
#pragma unroll
            for (int step = 8; step > 0; step >>= 1)
              if (off[b + step] <= j) b += step;
            atomicAdd(&mycnt[b * kHbRows + static_cast<int>(r[u])], 1u);
          }
        }
      }
    }
    __syncthreads();  // all 64 bags counted
    // acc[mt][q] += counts^T (rows 16 mt + m, bags 4 ks + k) x grad (bags 4 ks + k, columns cw + 2 n + q)
    // (all four row tiles: rows >= E have zero counts; columns >= D have zero gradient)
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint32_t c = s_cnt[(4 * ks + (lane >> 4)) * kHbRows + 16 * mt + (lane & 15)];
        rowcnt[mt] += c;
        const float a = static_cast<float>(c);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, gv[ks].x, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, gv[ks].y, acc[mt][1], 0, 0, 0);
      }
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bounds the count reads in flight
    }
  }
  // MFMA result layout: lane l holds rows 16 mt + 4 (l / 16) + i, columns c2 + q in acc[mt][q][i]
  float* dst = partial + static_cast<int64_t>(blockIdx.x) * kHbRows * kHbCols;
  if (c2 < D) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * (lane >> 4) + i;
        if (row < E)
          *reinterpret_cast<f32x2*>(dst + row * kHbCols + c2) = f32x2{acc[mt][0][i], acc[mt][1][i]};
      }
    }
  }
  // per-row lookup totals: lanes l, l ^ 16, l ^ 32, l ^ 48 share row 16 mt + l % 16
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    rowcnt[mt] += __shfl_xor(rowcnt[mt], 16);
    rowcnt[mt] += __shfl_xor(rowcnt[mt], 32);
    const int row = 16 * mt + lane;
    if (w == 0 && lane < 16 && row < E)
      pcount[static_cast<int64_t>(blockIdx.x) * kHbRows + row] = static_cast<int32_t>(rowcnt[mt]);
  }
}

// One workgroup per table row.  Thread (k, q) sums partials k, k + 8, ... of
// column quad q in increasing order; the eight sums are added in k order; then
// the row's optimizer step (skipped when no lookup hit the row).
template <int OPT>
__global__ __launch_bounds__(kBlock) void hist_bwd_apply_kernel(
    uint16_t* __restrict__ Wt, float* __restrict__ momentum, const int64_t* __restrict__ meta,
    int t, int32_t D, int P, const float* __restrict__ partial, const int32_t* __restrict__ pcount,
    float lr, float eps) {
  constexpr int kGroups = kBlock / (kHbCols / 4);  // 8
  __shared__ __align__(16) float s_part[kGroups][kHbCols];
  const int r = blockIdx.x;
  int hit = 0;
  for (int p = threadIdx.x; p < P; p += kBlock) hit |= pcount[static_cast<int64_t>(p) * kHbRows + r];
  if (!__syncthreads_or(hit)) return;  // untouched row: no update, weights and state unchanged
  const int q = threadIdx.x & (kHbCols / 4 - 1), k = threadIdx.x / (kHbCols / 4);
  const int col = 4 * q;
  if (col < D) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    const float* src = partial + static_cast<int64_t>(r) * kHbCols + col;
    int p = k;
    for (; p + 3 * kGroups < P; p += 4 * kGroups) {
      const f32x4 x0 = load_f4(src + static_cast<int64_t>(p) * kHbRows * kHbCols);
      const f32x4 x1 = load_f4(src + static_cast<int64_t>(p + kGroups) * kHbRows * kHbCols);
      const f32x4 x2 = load_f4(src + static_cast<int64_t>(p + 2 * kGroups) * kHbRows * kHbCols);
      const f32x4 x3 = load_f4(src + static_cast<int64_t>(p + 3 * kGroups) * kHbRows * kHbCols);
      a += x0; a += x1; a += x2; a += x3;
    }
    for (; p < P; p += kGroups) a += load_f4(src + static_cast<int64_t>(p) * kHbRows * kHbCols);
    *reinterpret_cast<f32x4*>(&s_part[k][col]) = a;
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  // wave 0 finishes: lane l owns columns 4 l .. 4 l + 3 (lanes >= D / 4 idle)
  const int lane = threadIdx.x;
  const int c = 4 * lane;
  const bool act = lane < (kHbCols / 4) && c < D;
  float gv[4] = {0.f, 0.f, 0.f, 0.f};
  float wv[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t row_base = meta[4 * t];
  uint16_t* wrow = Wt + static_cast<int64_t>(r) * D;
  if (act) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = s_part[0][c + e];
#pragma unroll
      for (int kk = 1; kk < kGroups; ++kk) s += s_part[kk][c + e];
      gv[e] = s;
    }
    load_vec<1, 4>(wrow + c, wv);
  }
  if constexpr (OPT == kOptSGD) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] -= lr * gv[e];
  } else {
    float ss = gv[0] * gv[0] + gv[1] * gv[1] + gv[2] * gv[2] + gv[3] * gv[3];
    for (int msk = 1; msk < kWave; msk <<= 1) ss += __shfl_xor(ss, msk);
    const float mnew = momentum[row_base + r] + ss / static_cast<float>(D);
    const float denom = sqrtf(mnew) + eps;
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] -= lr * gv[e] / denom;
    if (lane == 0) momentum[row_base + r] = mnew;
  }
  if (act) store_vec4<1>(wrow + c, wv);
}

template <typename IT, typename OT>
tbe_status hist_partial_go(const tbe_tables* tb, const IndexArgs& ia, const float* grad_out,
                           const uint16_t* saved, int P, float* partial, int32_t* pcount, hipStream_t s) {
  ProfScope ps("hist_bwd_partial", s);
  hipLaunchKernelGGL((hist_bwd_partial_kernel<IT, OT>), dim3(P), dim3(kBlock), 0, s,
                     static_cast<const IT*>(ia.indices), static_cast<const OT*>(ia.offsets), grad_out,
                     static_cast<int64_t>(tb->hist_table) * tb->B, tb->B, tb->hist_E, tb->hist_D,
                     static_cast<int64_t>(tb->hist_col), tb->out_width, ia.N, saved, partial, pcount);
  return check_launch("hist_bwd_partial");
}

}  // namespace

int hist_partial_blocks_per_cu() {
  return blocks_per_cu(reinterpret_cast<const void*>(hist_bwd_partial_kernel<int64_t, int64_t>));
}

tbe_status launch_hist_backward(const tbe_tables* tb, void* W, float* momentum, int opt,
                                const IndexArgs& ia, const float* grad_out, float lr, float eps,
                                char* ws, const BwdLayout& L, const uint16_t* saved, hipStream_t s,
                                int wgs_per_cu) {
  if (tb->B == 0 || tb->hist_table < 0) return TBE_OK;
  if (tb->hist_table >= tb->T || tb->hist_E < 1 || tb->hist_E > kHbRows || tb->hist_D > kHbCols || tb->hist_D % 16 || tb->w_dtype != TBE_F16) {
    set_error("histogram table outside E <= 64, D <= 128, D %% 16 == 0, fp16");
    return TBE_ERR_UNSUPPORTED;
  }
  // one partial per workgroup; each workgroup step covers 64 bags
  const int64_t steps = (static_cast<int64_t>(tb->B) + kHbBags - 1) / kHbBags;
  int64_t P64 = hmin(kHistBwdBlocks, steps);
  if (wgs_per_cu > 0) P64 = hmin(P64, static_cast<int64_t>(device_cu_count()) * wgs_per_cu);
  const int P = static_cast<int>(hmax(1, P64));
  float* partial = reinterpret_cast<float*>(ws + L.hist_partial);
  int32_t* pcount = reinterpret_cast<int32_t*>(ws + L.hist_count);
  tbe_status st;
  if (ia.itype == TBE_I32)
    st = ia.otype == TBE_I32 ? hist_partial_go<int32_t, int32_t>(tb, ia, grad_out, saved, P, partial, pcount, s)
                             : hist_partial_go<int32_t, int64_t>(tb, ia, grad_out, saved, P, partial, pcount, s);
  else
    st = ia.otype == TBE_I32 ? hist_partial_go<int64_t, int32_t>(tb, ia, grad_out, saved, P, partial, pcount, s)
                             : hist_partial_go<int64_t, int64_t>(tb, ia, grad_out, saved, P, partial, pcount, s);
  if (st) return st;
  uint16_t* Wt = static_cast<uint16_t*>(W) + tb->hist_w_base;
  ProfScope ps("hist_bwd_apply", s);
  if (opt == kOptSGD)
    hipLaunchKernelGGL((hist_bwd_apply_kernel<kOptSGD>), dim3(tb->hist_E), dim3(kBlock), 0, s, Wt,
                       momentum, tb->meta, tb->hist_table, tb->hist_D, P, partial, pcount, lr, eps);
  else
    hipLaunchKernelGGL((hist_bwd_apply_kernel<kOptAdagrad>), dim3(tb->hist_E), dim3(kBlock), 0, s, Wt,
                       momentum, tb->meta, tb->hist_table, tb->hist_D, P, partial, pcount, lr, eps);
  return check_launch("hist_bwd_apply");
}

}  // namespace tbe
