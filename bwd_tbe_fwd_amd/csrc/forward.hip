// TBE forward: pooled gather-sum over T tables in one launch, plus the
// small-table histogram path on MFMA.
//
// PyTorch blog "Modernizing Table Batched Embeddings with FBTriton", section 2:
// every bag of every table gathers its rows, scales each by its per-sample
// weight when there is one, and sums them into one D-wide output row; fp16 /
// bf16 tables accumulate in fp32 and fp32 tables in fp64.  "The general gather
// path" there keeps several independent row loads in flight per program and
// lets each program walk the tables for its bags; "The small-table histogram
// and tensor-core path" counts the first 256 ids of each bag of a table with at
// most 64 rows and multiplies the counts by the table on tensor cores.
//
// gfx950 mapping (generic path): one wave pools one bag at a time.  A row of D
// elements is read by a group of D/VEC lanes with 16-byte (fp16/bf16: 8
// elements, fp32: 4) or 8-byte vector loads, so one wave instruction fetches
// 64/(D/VEC) rows; UNROLL such instructions are issued before any is summed.
// The bag's ids are loaded coalesced, one per lane, and handed to the row
// groups with lane shuffles; the consecutive bags a wave takes per grid step
// (up to 64, the bags-per-wave knob) have their offsets fetched in one
// coalesced load.  Per-group partial sums are combined with xor shuffles and
// one group writes the output row.  With the fused bounds check (REPAIR), an
// id outside its table is read as row 0, rewritten to 0 in place and counted.
#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {
namespace {

// Pools the lookups [s, e) of one bag into acc (this lane's VEC columns, row group
// lane >> lg).  The bag's first 64 ids (and weights) arrive already loaded in
// first_id / first_w: they were fetched while the previous bag's rows were in
// flight.  REPAIR (fused bounds check): an id outside [0, E) is read as row 0,
// rewritten to 0 in place (once, on the first column block) and counted.
template <int DT, typename IT, bool PSW, int VEC, typename ACC, int UNROLL, bool REPAIR>
__device__ __forceinline__ void pool_bag(const typename Fmt<DT>::S* __restrict__ Wt, int64_t E,
                                         int D, IT* __restrict__ indices,
                                         const float* __restrict__ psw, int64_t s, int64_t e,
                                         int lg, int col, bool act, int64_t first_id, float first_w,
                                         bool first_block, int64_t& fixed, ACC (&acc)[VEC]) {
  const int lane = lane_id();
  const int G = kWave >> lg;  // rows per wave instruction
  const int g = lane >> lg;   // this lane's row group
  for (int64_t j0 = s; j0 < e; j0 += kWave) {
    const int n = static_cast<int>(min<int64_t>(kWave, e - j0));
    int64_t r = first_id;
    float myw = first_w;
    if (j0 != s) {
      r = lane < n ? static_cast<int64_t>(indices[j0 + lane]) : -1;
      if constexpr (PSW) myw = lane < n ? psw[j0 + lane] : 0.f;
    }
    const bool bad = lane < n && static_cast<uint64_t>(r) >= static_cast<uint64_t>(E);
    int32_t myrow = (lane < n && !bad) ? static_cast<int32_t>(r) : -1;
    if constexpr (REPAIR) {
      if (bad) {
        myrow = 0;
        if (first_block) {
          indices[j0 + lane] = 0;
          ++fixed;
        }
      }
    }
    for (int q0 = 0; q0 < n; q0 += G * UNROLL) {
      RawVec<DT, VEC> raw[UNROLL];
      float wq[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int q = q0 + u * G + g;
        const int row = __shfl(myrow, q & (kWave - 1));
        if constexpr (PSW) wq[u] = __shfl(myw, q & (kWave - 1));
        if (q < n && row >= 0 && act) load_raw<DT, VEC>(Wt + static_cast<int64_t>(row) * D + col, raw[u]);
        else zero_raw(raw[u]);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        float v[VEC];
        unpack_raw(raw[u], v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          if constexpr (PSW) acc[i] += static_cast<ACC>(wq[u]) * static_cast<ACC>(v[i]);
          else acc[i] += static_cast<ACC>(v[i]);
        }
      }
    }
  }
}

// fp16 / bf16 tables without per-sample weights, up to 4 rows in flight, are held to at
// least 6 waves per SIMD (80 registers): the kernel is bound by its row-load latency, and the
// fused id check's instantiation otherwise takes 82 registers and 5 waves (skewed batch:
// 2.66 -> 2.49 ms).  With per-sample weights, fp32 tables (fp64 sums) or 8 rows in flight
// the bound would spill.
template <int DT, typename IT, typename OT, bool PSW, int VEC, typename ACC, int UNROLL, bool REPAIR>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu((PSW || DT == 0 || UNROLL > 4) ? 1 : 6)))
void fwd_gather_kernel(
    const typename Fmt<DT>::S* __restrict__ W, IT* __restrict__ indices,
    const OT* __restrict__ offsets, const float* __restrict__ psw, float* __restrict__ out,
    const int64_t* __restrict__ meta, int32_t skip_t, int32_t n_tables, int32_t B,
    int32_t out_width, int64_t N, int32_t group, int64_t* __restrict__ counts) {
  const int lane = lane_id();
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
  const int64_t slots = static_cast<int64_t>(n_tables) * B;
  int cur_t = -1;
  TableMeta m{};
  int64_t fixed = 0;
  for (int64_t base = wave * group; base < slots; base += nwaves * group) {
    // one bag per lane (group <= 64 of them): its table, batch row and clamped [start, end)
    const int64_t slot = lane < group ? base + lane : slots;
    int64_t s = 0, e = 0;
    int32_t bt = 0, bb = 0;
    if (slot < slots) {
      const int32_t ti = static_cast<int32_t>(slot / B);
      bb = static_cast<int32_t>(slot - static_cast<int64_t>(ti) * B);
      bt = (skip_t >= 0 && ti >= skip_t) ? ti + 1 : ti;  // every table but skip_t
      const int64_t bag = static_cast<int64_t>(bt) * B + bb;
      s = static_cast<int64_t>(offsets[bag]);
      e = static_cast<int64_t>(offsets[bag + 1]);
      s = min(max(s, static_cast<int64_t>(0)), N);
      e = min(max(e, s), N);
    }
    const int nb = static_cast<int>(min<int64_t>(group, slots - base));
    // ids of the first bag; each later bag's first ids are fetched one bag ahead
    int64_t nxt_id = -1;
    float nxt_w = 0.f;
    {
      const int64_t s0 = read_lane64(s, 0), e0 = read_lane64(e, 0);
      if (lane < e0 - s0) {
        nxt_id = static_cast<int64_t>(indices[s0 + lane]);
        if constexpr (PSW) nxt_w = psw[s0 + lane];
      }
    }
    for (int k = 0; k < nb; ++k) {
      const int64_t sk = read_lane64(s, k), ek = read_lane64(e, k);
      const int t = read_lane(bt, k), b = read_lane(bb, k);
      const int64_t cur_id = nxt_id;
      const float cur_w = nxt_w;
      if (k + 1 < nb) {
        const int64_t s1 = read_lane64(s, k + 1), e1 = read_lane64(e, k + 1);
        nxt_id = -1;
        if (lane < e1 - s1) {
          nxt_id = static_cast<int64_t>(indices[s1 + lane]);
          if constexpr (PSW) nxt_w = psw[s1 + lane];
        }
      }
      if (t != cur_t) {
        m = load_meta(meta, t);
        cur_t = t;
      }
      const int D = static_cast<int>(m.D);
      float* orow = out + static_cast<int64_t>(b) * out_width + m.col_base;
      for (int cb = 0; cb < D; cb += kWave * VEC) {
        const int w = min(D - cb, kWave * VEC);
        const int lpr = pow2_ceil((w + VEC - 1) / VEC);
        const int lg = __builtin_ctz(lpr);
        const int c = lane & (lpr - 1);
        const int col = cb + c * VEC;
        const bool act = c * VEC < w;
        ACC acc[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] = 0;
        pool_bag<DT, IT, PSW, VEC, ACC, UNROLL, REPAIR>(W + m.w_base, m.E, D, indices, psw, sk, ek,
                                                        lg, col, act, cur_id, cur_w, cb == 0, fixed,
                                                        acc);
        for (int msk = lpr; msk < kWave; msk <<= 1) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], msk);
        }
        if ((lane >> lg) == 0 && act) {
#pragma unroll
          for (int i = 0; i < VEC; i += 4) {
            f32x4 o = {static_cast<float>(acc[i]), static_cast<float>(acc[i + 1]),
                       static_cast<float>(acc[i + 2]), static_cast<float>(acc[i + 3])};
            store_f4_stream(orow + col + i, o);  // the pooled rows are not read back here
          }
        }
      }
    }
  }
  if constexpr (REPAIR) {  // one atomic per wave
    for (int msk = 1; msk < kWave; msk <<= 1) fixed += __shfl_xor(fixed, msk);
    if (lane == 0 && fixed)
      atomicAdd(reinterpret_cast<unsigned long long*>(counts), static_cast<unsigned long long>(fixed));
  }
}

// ---------------------------------------------------------------------------
// histogram + MFMA path for one small table (E <= 64, 64 <= D <= 128, fp16)
// ---------------------------------------------------------------------------
// One wave owns 16 consecutive bags (one 16-row MFMA tile).  Their ids are one
// contiguous range, read coalesced with several loads in flight; the wave
// counts each bag's first 256 ids into an LDS histogram (16 x 64), turns it
// into the fp16 A operand (counts <= 256 are exact in fp16), and multiplies it
// by the table held transposed in LDS as the B operand with
// v_mfma_f32_16x16x16_f16 (fp32 accumulation).  The products count * w are
// exact in fp32; only the accumulation rounds.  Ids beyond the first 256 of a
// bag are gathered and added to the tile; the finished tile leaves through LDS,
// 64 columns at a time, as 16-byte row-contiguous stores.  The count area and
// the output stage share one 16 x 68-word LDS area per wave (the counts are in
// registers by the time the products are staged), and eight waves share the
// table, so a CU holds 24 waves.  With REPAIR, ids outside the table are
// repaired to 0 in place and counted, as in the gather.  With save_counts, the
// tile's counts also go to HBM as u16 (bag-major, 64 rows a bag), the forward
// state the histogram backward reuses.
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kHistRows = 64;   // K of the contraction (table rows, zero padded)
constexpr int kHistCols = 128;  // max D
constexpr int kHistBags = 16;   // M of one MFMA tile
constexpr int kHistHead = 256;  // ids per bag counted into the histogram
constexpr int kHistLoads = 8;   // id loads in flight per lane while counting
constexpr int kHistWaves = 8;   // waves per workgroup, sharing one copy of the table
constexpr int kHistThreads = kHistWaves * kWave;
constexpr int kHistHalf = 64;   // output columns staged at a time
// LDS strides padded against bank conflicts (32 banks of 4 bytes): a table column holds its
// 64 rows in 68 halves, so the 16 columns of an MFMA B operand start in 16 different bank
// pairs; a bag's counts (and a staged output row of 64 columns) take 68 words, so the 16 bags
// of the A operand spread over the banks and the four row groups of an MFMA result land in
// two bank halves
constexpr int kHistWStride = kHistRows + 4;
constexpr int kHistStride = kHistRows + 4;

template <typename IT, typename OT, bool REPAIR>
__global__ __launch_bounds__(kHistThreads) __attribute__((amdgpu_waves_per_eu(6))) void fwd_hist_kernel(
    const uint16_t* __restrict__ Wt, IT* __restrict__ indices, const OT* __restrict__ offsets,
    float* __restrict__ out, int64_t bag0, int32_t B, int32_t E, int32_t D, int64_t col_base,
    int32_t out_width, int64_t N, int64_t* __restrict__ counts, uint16_t* __restrict__ save_counts) {
  __shared__ __align__(16) uint16_t s_wT[kHistCols * kHistWStride];           // [col][row]
  __shared__ __align__(16) uint32_t s_tile[kHistWaves][kHistBags * kHistStride];
  __shared__ int32_t s_off[kHistWaves][kHistBags + 1];
  const int lane = lane_id();
  const int w = threadIdx.x >> 6;
  // the table (16 KB, once per workgroup), stored transposed: lane l of a wave takes row l,
  // so neighbouring lanes write neighbouring halves of a column
  for (int i = threadIdx.x; i < kHistRows * (kHistCols / 4); i += kHistThreads) {
    const int row = i % kHistRows, col = 4 * (i / kHistRows);
    u32x2 v = {0u, 0u};
    if (row < E && col < D) v = *reinterpret_cast<const u32x2*>(Wt + static_cast<int64_t>(row) * D + col);
    s_wT[(col + 0) * kHistWStride + row] = static_cast<uint16_t>(v.x);
    s_wT[(col + 1) * kHistWStride + row] = static_cast<uint16_t>(v.x >> 16);
    s_wT[(col + 2) * kHistWStride + row] = static_cast<uint16_t>(v.y);
    s_wT[(col + 3) * kHistWStride + row] = static_cast<uint16_t>(v.y >> 16);
  }
  __syncthreads();
  uint32_t* cnt = s_tile[w];                          // counts [bag][row], then ...
  float* otile = reinterpret_cast<float*>(s_tile[w]);  // ... the staged output [bag][column - c0]
  int32_t* off = s_off[w];
  int64_t fixed = 0;
  const int64_t tiles = (static_cast<int64_t>(B) + kHistBags - 1) / kHistBags;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kHistWaves + w; tile < tiles;
       tile += static_cast<int64_t>(gridDim.x) * kHistWaves) {
    const int64_t b0 = tile * kHistBags;
    const int nbag = static_cast<int>(min<int64_t>(kHistBags, B - b0));
    // the 17 offsets of the tile, clamped to [0, N] and made monotone, so that the
    // tile's ids are one contiguous range [o0, o0 + n)
    int32_t o = 0;
    if (lane <= kHistBags) {
      const int64_t v = static_cast<int64_t>(offsets[bag0 + b0 + min(lane, nbag)]);
      o = static_cast<int32_t>(min(max(v, static_cast<int64_t>(0)), N));
    }
    for (int d = 1; d < 32; d <<= 1) {
      const int32_t u = __shfl_up(o, d);
      if (lane >= d) o = max(o, u);
    }
    const int32_t o0 = read_lane(o, 0);
    const int32_t n = read_lane(o, kHistBags) - o0;
    if (lane <= kHistBags) off[lane] = o - o0;
    for (int i = lane; i < kHistBags * kHistStride; i += kWave) cnt[i] = 0u;
    __builtin_amdgcn_wave_barrier();
    // each bag's first 256 ids, read as one coalesced range with kHistLoads loads in
    // flight per lane; positions only grow, so a lane's bag search continues from its last
    // bag (off[16] = n ends it).  The next round's ids are requested before this round is
    // counted, so a tile waits on one load latency instead of one a round.
    int bcur = 0;
    int64_t rn[kHistLoads];  // the round in flight
    int32_t r[kHistLoads];   // the round being counted: its rows, -1 for an id outside the table
    auto fetch = [&](int32_t j0) {
#pragma unroll
      for (int u = 0; u < kHistLoads; ++u) {
        const int32_t j = j0 + u * kWave + lane;
        rn[u] = j < n ? static_cast<int64_t>(indices[o0 + j]) : 0;
      }
    };
    auto take = [&]() {
#pragma unroll
      for (int u = 0; u < kHistLoads; ++u)
        r[u] = static_cast<uint64_t>(rn[u]) < static_cast<uint64_t>(E) ? static_cast<int32_t>(rn[u]) : -1;
    };
    fetch(0);
    take();
    for (int32_t j0 = 0; j0 < n; j0 += kHistLoads * kWave) {
      if (j0 + kHistLoads * kWave < n) fetch(j0 + kHistLoads * kWave);
#pragma unroll
      for (int u = 0; u < kHistLoads; ++u) {
        const int32_t j = j0 + u * kWave + lane;
        if (j < n) {
          while (off[bcur + 1] <= j) ++bcur;
          const int b = bcur;
          if (j - off[b] < kHistHead) {
            int32_t row = r[u];
            if (row < 0) {
              if constexpr (REPAIR) {  // repaired to row 0, in place, and counted
                indices[o0 + j] = 0;
                ++fixed;
                row = 0;
              }
            }
            if (row >= 0) atomicAdd(&cnt[b * kHistStride + row], 1u);
          }
        }
      }
      take();
    }
    __builtin_amdgcn_wave_barrier();
    if (save_counts) {  // 16 bags x 64 rows as u16 (the padding bags of the last tile hold zeros)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = 8 * (k * kWave + lane);  // bag e / 64, rows e % 64 + [0, 8)
        const int c = (e / kHistRows) * kHistStride + e % kHistRows;
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(&cnt[c]);
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(&cnt[c + 4]);
        const u32x4 v = {c0.x | (c0.y << 16), c0.z | (c0.w << 16), c1.x | (c1.y << 16), c1.z | (c1.w << 16)};
        *reinterpret_cast<u32x4*>(save_counts + b0 * kHistRows + e) = v;
      }
    }
    // A operand: lane l holds bag l%16, rows 16s + 4(l/16) + [0, 4), read 16 bytes at a time
    half4_t a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(&cnt[(lane & 15) * kHistStride + 16 * s + 4 * (lane >> 4)]);
      a[s][0] = static_cast<_Float16>(static_cast<float>(c.x));
      a[s][1] = static_cast<_Float16>(static_cast<float>(c.y));
      a[s][2] = static_cast<_Float16>(static_cast<float>(c.z));
      a[s][3] = static_cast<_Float16>(static_cast<float>(c.w));
    }
    __builtin_amdgcn_wave_barrier();  // the counts are in registers: the area takes the output
    for (int c0 = 0; c0 < D; c0 += kHistHalf) {
      const int nc = min(kHistHalf, D - c0);
      for (int nt = 0; nt < nc / 16; ++nt) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // B operand: lane l holds column c0 + 16n + l%16, rows 16s + 4(l/16) + [0, 4)
          const half4_t bf = *reinterpret_cast<const half4_t*>(
              &s_wT[(c0 + 16 * nt + (lane & 15)) * kHistWStride + 16 * s + 4 * (lane >> 4)]);
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a[s], bf, acc, 0, 0, 0);
        }
        // result: lane l holds column c0 + 16n + l%16 of bags 4(l/16) + [0, 4)
#pragma unroll
        for (int q = 0; q < 4; ++q) otile[(4 * (lane >> 4) + q) * kHistStride + 16 * nt + (lane & 15)] = acc[q];
      }
      __builtin_amdgcn_wave_barrier();
      // ids past the first 256 of a bag: gathered from the LDS copy of the table (the
      // repair, and its count, happen on the first column block)
      for (int i = 0; i < nbag; ++i) {
        const int32_t s = o0 + off[i], e = o0 + off[i + 1];
        for (int32_t j = s + kHistHead; j < e; ++j) {
          int64_t r = static_cast<int64_t>(indices[j]);
          if (static_cast<uint64_t>(r) >= static_cast<uint64_t>(E)) {
            if constexpr (REPAIR) {
              __builtin_amdgcn_wave_barrier();
              if (lane == 0 && c0 == 0) {
                indices[j] = 0;
                ++fixed;
              }
              r = 0;
            } else {
              continue;
            }
          }
          for (int col = lane; col < nc; col += kWave)
            otile[i * kHistStride + col] += static_cast<float>(
                __builtin_bit_cast(_Float16, s_wT[(c0 + col) * kHistWStride + r]));
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int c4n = nc / 4;
      for (int x = lane; x < nbag * c4n; x += kWave) {
        const int i = x / c4n, c4 = x - i * c4n;
        const f32x4 v = *reinterpret_cast<const f32x4*>(&otile[i * kHistStride + 4 * c4]);
        store_f4_stream(out + (b0 + i) * out_width + col_base + c0 + 4 * c4, v);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  if constexpr (REPAIR) {  // one atomic per wave
    for (int msk = 1; msk < kWave; msk <<= 1) fixed += __shfl_xor(fixed, msk);
    if (lane == 0 && fixed)
      atomicAdd(reinterpret_cast<unsigned long long*>(counts), static_cast<unsigned long long>(fixed));
  }
}


// One workgroup per kWavesPerBlock groups of bags, not a grid sized to what the CUs hold: the
// dispatcher gives each slot that frees up the next workgroup, so CUs and waves that drew heavy
// bags or slow rows do not set the kernel's end, while the workgroups still start in bag order
// (skewed batch 2.50 -> 2.41 ms, uniform 1.56 -> 1.40 ms with the bag groups below).
template <int DT, typename IT, typename OT, bool PSW, int VEC, typename ACC>
tbe_status gather_go(const tbe_tables* tb, const void* W, const IndexArgs& ia, const float* psw,
                     float* out, int skip, int nt, int unroll, int group, int64_t* repair_counts, hipStream_t s) {
  const int64_t slots = static_cast<int64_t>(nt) * tb->B;
  const int64_t work = ((slots + group - 1) / group + kWavesPerBlock - 1) / kWavesPerBlock;
  using S = typename Fmt<DT>::S;
  ProfScope ps("fwd_gather", s);
#define TBE_FWD_LAUNCH(U, R)                                                                     \
  hipLaunchKernelGGL((fwd_gather_kernel<DT, IT, OT, PSW, VEC, ACC, U, R>),                       \
                     dim3(static_cast<int>(hmax(1, hmin(work, int64_t{1} << 30)))),                \
                     dim3(kBlock), 0, s, static_cast<const S*>(W),                                  \
                     const_cast<IT*>(static_cast<const IT*>(ia.indices)),                           \
                     static_cast<const OT*>(ia.offsets), psw, out, tb->meta, skip, nt, tb->B,         \
                     tb->out_width, ia.N, group, repair_counts)
  if (repair_counts) {
    if (unroll <= 4) TBE_FWD_LAUNCH(4, true);
    else TBE_FWD_LAUNCH(8, true);
  } else if (unroll <= 2) {
    TBE_FWD_LAUNCH(2, false);
  } else if (unroll <= 4) {
    TBE_FWD_LAUNCH(4, false);
  } else {
    TBE_FWD_LAUNCH(8, false);
  }
#undef TBE_FWD_LAUNCH
  return check_launch("fwd_gather");
}

template <int DT, typename IT, typename OT>
tbe_status gather_dispatch_psw(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                               const float* psw, float* out, int skip, int nt, int unroll, int group,
                               int64_t* rc, hipStream_t s) {
  if constexpr (DT == 0) {
    if (psw) return gather_go<DT, IT, OT, true, 4, double>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
    return gather_go<DT, IT, OT, false, 4, double>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
  } else {
    if (tb->all_D_mult8) {
      if (psw) return gather_go<DT, IT, OT, true, 8, float>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
      return gather_go<DT, IT, OT, false, 8, float>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
    }
    if (psw) return gather_go<DT, IT, OT, true, 4, float>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
    return gather_go<DT, IT, OT, false, 4, float>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
  }
}

template <int DT>
tbe_status gather_dispatch_idx(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                               const float* psw, float* out, int skip, int nt, int unroll, int group,
                               int64_t* rc, hipStream_t s) {
  if (ia.itype == TBE_I32) {
    if (ia.otype == TBE_I32)
      return gather_dispatch_psw<DT, int32_t, int32_t>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
    return gather_dispatch_psw<DT, int32_t, int64_t>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
  }
  if (ia.otype == TBE_I32)
    return gather_dispatch_psw<DT, int64_t, int32_t>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
  return gather_dispatch_psw<DT, int64_t, int64_t>(tb, W, ia, psw, out, skip, nt, unroll, group, rc, s);
}

template <typename IT, typename OT>
tbe_status hist_go(const tbe_tables* tb, const void* W, const IndexArgs& ia, float* out,
                   int64_t* repair_counts, uint16_t* save_counts, hipStream_t s) {
  const int64_t tiles = (static_cast<int64_t>(tb->B) + kHistBags - 1) / kHistBags;
  const int64_t work = (tiles + kHistWaves - 1) / kHistWaves;
  ProfScope ps("fwd_hist", s);
#define TBE_HIST_LAUNCH(R)                                                                         \
  hipLaunchKernelGGL((fwd_hist_kernel<IT, OT, R>),                                               \
                     dim3(resident_grid(fwd_hist_kernel<IT, OT, R>, work, 0, kHistThreads)),      \
                     dim3(kHistThreads), 0, s,                                                    \
                     static_cast<const uint16_t*>(W) + tb->hist_w_base,                           \
                     const_cast<IT*>(static_cast<const IT*>(ia.indices)),                         \
                     static_cast<const OT*>(ia.offsets), out,                                     \
                     static_cast<int64_t>(tb->hist_table) * tb->B, tb->B, tb->hist_E, tb->hist_D,   \
                     static_cast<int64_t>(tb->hist_col), tb->out_width, ia.N, repair_counts,     \
                     save_counts)
  if (repair_counts) TBE_HIST_LAUNCH(true);
  else TBE_HIST_LAUNCH(false);
#undef TBE_HIST_LAUNCH
  return check_launch("fwd_hist");
}

}  // namespace

tbe_status launch_forward_gather(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                                 const float* psw, float* out, int skip_table,
                                 int unroll, int group, int64_t* rc, hipStream_t s) {
  const int n_tables = skip_table >= 0 ? tb->T - 1 : tb->T;
  if (n_tables <= 0 || tb->B == 0) return TBE_OK;
  if (group < 1 || group > kWave) {
    // automatic: the smallest power of two from 8 that keeps the launch within 65536
    // workgroups (one group of bags a wave)
    const int64_t slots = static_cast<int64_t>(n_tables) * tb->B;
    group = 8;
    while (group < kWave && slots > static_cast<int64_t>(group) * kWavesPerBlock * 65536) group *= 2;
  }
  switch (tb->w_dtype) {
    case TBE_F32: return gather_dispatch_idx<0>(tb, W, ia, psw, out, skip_table, n_tables, unroll, group, rc, s);
    case TBE_F16: return gather_dispatch_idx<1>(tb, W, ia, psw, out, skip_table, n_tables, unroll, group, rc, s);
    default: return gather_dispatch_idx<2>(tb, W, ia, psw, out, skip_table, n_tables, unroll, group, rc, s);
  }
}

tbe_status launch_forward_hist(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                               float* out, int64_t* rc, uint16_t* sc, hipStream_t s) {
  if (tb->B == 0 || tb->hist_table < 0) return TBE_OK;
  if (ia.itype == TBE_I32) {
    if (ia.otype == TBE_I32) return hist_go<int32_t, int32_t>(tb, W, ia, out, rc, sc, s);
    return hist_go<int32_t, int64_t>(tb, W, ia, out, rc, sc, s);
  }
  if (ia.otype == TBE_I32) return hist_go<int64_t, int32_t>(tb, W, ia, out, rc, sc, s);
  return hist_go<int64_t, int64_t>(tb, W, ia, out, rc, sc, s);
}

}  // namespace tbe
