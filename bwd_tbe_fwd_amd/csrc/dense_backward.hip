// Backward of the hottest rows of large tables as a dense product.
//
// PyTorch blog "Modernizing Table Batched Embeddings with FBTriton", section 2
// ("forward-state reuse and preprocessing") computes the gradient of the small
// histogram table as per-bag row counts times grad_out on tensor cores instead
// of a per-lookup gather.  The same identity holds for any set of rows R of any
// table t: for r in R,
//     g[r, :] = sum_b count_b[r] * grad_out[b, col_t : col_t + D],
// which is the sum over every lookup of r of its bag's gradient row.  On the
// sorted-run path a row with n lookups reads n gradient rows (n * 4D bytes);
// here the table's B x D gradient slice is read once for all rows of R
// together, plus the table's ids (or one two-byte slot per lookup).  For rows
// looked up thousands of times (the head of a skewed id distribution) that
// replaces most of the long-run gradient traffic.
//
// gfx950 mapping.  dense_select (one wave per table) takes a table's long runs
// of at least dense_min lookups (the kDenseRows longest when more qualify) and
// records their row ids (ascending).  In large batches the rows are picked
// before the sort, from a sample of the lookups: dense_sample writes the keys
// of 64 positions out of every hot_stride, which are sorted and run-length
// encoded on their own, the runs that reach dense_min scaled to the sample are
// taken, and their keys go into a hashed key set that linearize consults:
// their lookups get the sentinel key, so the sort, the run-length encoding and
// the run kernels never see them, and every position gets a dense slot (its
// row's rank among the table's dense rows, and its bag modulo 16).  Otherwise
// (the sample's twenty-odd launches would cost more than they save) the rows
// come from the batch's own long runs after the sort, and their long-list
// slots are flagged so that the chunk and apply kernels skip them.
// dense_partial: workgroup (t, p) takes the table's 64-bag steps p, p + P, ...;
// each of its four waves counts the lookups of 16 of the step's bags that hit
// a selected row (from the dense slots, or else through a bit filter in LDS, a
// 7-step search of the sorted row ids and a 4-step search of the bag offsets)
// into the shared count[128 rows][64 bags] (fp32, so that a count below 256 is
// its own bf16 value; uint32 for a wave whose bags hold 2^24 lookups or more);
// then wave w multiplies the counts by gradient columns 32 w .. 32 w + 31 of
// the 64 bags on v_mfma_f32_16x16x32_bf16.  The blog's
// compensated high/low product, made exact: the fp32 gradient is split into
// three bf16 parts whose sum is exactly its value, counts are exact in bf16
// (byte by byte above 255), so every product is exact and only the fp32
// accumulation rounds.  (fp32 MFMA would be 16x slower per flop: 128 rows x 64
// bags x D per step is 137 GFLOP over the large skewed batch.)  The 128 x 32
// accumulator (8 x 2 tiles) stays in registers across the steps and is
// written once as the workgroup's partial.  dense_apply sums a row's P
// partials in a fixed order and applies SGD or row-wise Adagrad: results are
// bitwise repeatable.  With per-sample weights the counts become per-bag sums
// of the weights (see dense_partial_kernel), the same identity with each
// lookup's gradient row scaled by its weight.
#include "backward_launch.h"

namespace tbe {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kDnCols = 128;     // max D; each wave owns 32 columns (2 MFMA N tiles)
constexpr int kDnWaveBags = 16;  // bags one wave counts per step
constexpr int kDnBags = kDnWaveBags * kWavesPerBlock;  // bags per step: the MFMA K, two blocks of 32
constexpr int kDnLoads = 8;      // id loads in flight per lane while counting

__device__ __forceinline__ bool dense_table_ok(int D, int t, int hist_t) {
  return t != hist_t && D >= 16 && D <= kDnCols && D % 16 == 0;
}

// The sample: wave j takes positions stride * j + [0, 64).  A position's table is the last
// table whose first offset is at or below it; lookups of tables the dense path does not take,
// positions no table covers and ids outside their table (unless invalid_as_row0, when they
// count as row 0) get the sentinel key, which the sort leaves out.
template <typename IT, typename OT>
__global__ __launch_bounds__(kBlock) void dense_sample_kernel(
    const IT* __restrict__ indices, const OT* __restrict__ offsets, const int64_t* __restrict__ meta, int T,
    int32_t B, int64_t N, int64_t stride, int64_t nsamp, int hist_t, int invalid_as_row0, uint32_t sentinel,
    uint32_t* __restrict__ keys, uint32_t* __restrict__ pay) {
  const int lane = lane_id();
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
  auto first = [&](int t) {  // table t's first lookup, clamped to [0, N]
    const int64_t v = static_cast<int64_t>(offsets[static_cast<int64_t>(t) * B]);
    return min(max(v, static_cast<int64_t>(0)), N);
  };
  const int64_t lo0 = first(0), hiT = first(T);
  for (int64_t j = wave; j < nsamp; j += nwaves) {
    const int64_t p = j * stride + lane;
    uint32_t key = sentinel;
    if (p >= lo0 && p < hiT) {
      int lo = 0, hi = T - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first(mid) <= p) lo = mid; else hi = mid - 1;
      }
      const TableMeta m = load_meta(meta, lo);
      if (dense_table_ok(static_cast<int>(m.D), lo, hist_t)) {
        const int64_t r = static_cast<int64_t>(indices[p]);
        if (static_cast<uint64_t>(r) < static_cast<uint64_t>(m.E)) key = static_cast<uint32_t>(m.row_base + r);
        else if (invalid_as_row0) key = static_cast<uint32_t>(m.row_base);
      }
    }
    keys[j * kWave + lane] = key;
    pay[j * kWave + lane] = 0u;
  }
}

// One wave per table: the table's long runs (long-list slots [lo, hi), in key order) of at
// least min_len lookups become its dense rows, in ascending order; when more than kDenseRows
// qualify, the kDenseRows longest (among equal lengths, the smaller keys).
// Picked from the sorted sample (hot_set != NULL): their keys and ranks go into the key set
// (linear probing over records; the most records a lookup reads into *probe_max) and its filter.  Picked from
// the batch's own runs (long_flag != NULL): each slot's flag says whether the chunk and apply
// kernels leave it to the dense path.
__global__ __launch_bounds__(kBlock) void dense_select_kernel(
    const uint4* __restrict__ long_list, const uint32_t* __restrict__ long_table,
    const int32_t* __restrict__ counters, int64_t cap_long, const int64_t* __restrict__ meta, int T,
    int hist_t, uint32_t min_len, int32_t* __restrict__ dense_rows, int32_t* __restrict__ dense_cnt,
    uint32_t* __restrict__ long_flag, uint32_t* __restrict__ hot_set,
    uint32_t hot_mask, uint32_t* __restrict__ hot_filter, int32_t* __restrict__ probe_max) {
  const int lane = lane_id();
  const int t = static_cast<int>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t n = min(static_cast<int64_t>(counters[kLong]), cap_long);
  // first slot of table t and of table t + 1
  auto lower = [&](uint32_t v) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
      const int64_t mid = (lo + hi) >> 1;
      if (long_table[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  const int64_t s0 = lower(static_cast<uint32_t>(t)), s1 = lower(static_cast<uint32_t>(t) + 1);
  const TableMeta m = load_meta(meta, t);
  const bool ok = dense_table_ok(static_cast<int>(m.D), t, hist_t);
  const uint32_t* len_of = reinterpret_cast<const uint32_t*>(long_list) + 2;  // len_of[4 s]
  // runs of at least v lookups (and the longest run)
  auto count_ge = [&](uint32_t v, uint32_t* longest) {
    int64_t c = 0;
    uint32_t mx = 0;
    for (int64_t s = s0 + lane; s - lane < s1; s += kWave) {
      const uint32_t len = s < s1 ? len_of[4 * s] : 0u;
      c += __popcll(__ballot(len >= v && len > 0));
      mx = max(mx, len);
    }
    if (longest) {
      for (int d = 1; d < kWave; d <<= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), d)));
      *longest = mx;
    }
    return c;
  };
  // kept: every run longer than tau, and the first `quota` runs of exactly tau lookups
  uint32_t tau = max(min_len, 1u);
  int64_t quota = int64_t{1} << 40;
  if (ok) {
    uint32_t hi;
    if (count_ge(tau, &hi) > kDenseRows) {
      uint32_t lo = tau;  // the largest v with at least kDenseRows runs of >= v lookups
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo + 1) / 2;
        if (count_ge(mid, nullptr) >= kDenseRows) lo = mid; else hi = mid - 1;
      }
      tau = lo;
      quota = kDenseRows - count_ge(tau + 1, nullptr);
    }
  }
  int taken = 0;
  int64_t eq_seen = 0;  // runs of exactly tau lookups before this step
  for (int64_t s = s0 + lane; s - lane < s1; s += kWave) {
    const bool in = s < s1;
    uint4 L = make_uint4(0u, 0u, 0u, 0u);
    if (in) L = long_list[s];
    const bool eq = in && L.z == tau;
    const uint64_t em = __ballot(eq);
    const bool want = in && ok && (L.z > tau || (eq && eq_seen + __popcll(em & lanemask_lt()) < quota));
    eq_seen += __popcll(em);
    const uint64_t wm = __ballot(want);
    const int rank = taken + __popcll(wm & lanemask_lt());
    const bool take = want && rank < kDenseRows;
    if (take) dense_rows[static_cast<int64_t>(t) * kDenseRows + rank] = static_cast<int32_t>(L.x - m.row_base);
    if (long_flag && in) long_flag[s] = take ? 1u : 0u;
    if (hot_set && take) {
      const uint32_t key = L.x;
      const uint32_t h = hot_slot(key, hot_mask);
      // the set holds at least 6 slots per possible key: a free slot is always found
      int g = 0;
      for (bool placed = false; !placed; ++g) {
        const uint32_t rec = (h + 4 * g) & hot_mask;
        for (int j = 0; j < kHotSlotsPerRecord && !placed; ++j) {
          const uint32_t prev = atomicCAS(&hot_set[rec + j], kHotEmpty, key);
          if (prev == kHotEmpty)  // its rank into byte j of the record's rank word
            reinterpret_cast<uint8_t*>(hot_set + rec + kHotSlotsPerRecord)[j] = static_cast<uint8_t>(rank);
          placed = prev == kHotEmpty || prev == key;
        }
      }
      atomicMax(probe_max, g);  // records a lookup reads at most
      const uint32_t f = hot_filter_bit(key);
      atomicOr(&hot_filter[f >> 5], 1u << (f & 31));
    }
    taken = min(kDenseRows, taken + __popcll(wm));
  }
  if (lane == 0) dense_cnt[t] = taken;
}

// bf16 bits of a float whose low 16 bits are zero (exact)
__device__ __forceinline__ short bf16_bits(float x) {
  return static_cast<short>(__builtin_bit_cast(uint32_t, x) >> 16);
}
// x = hi + mid + lo exactly: each part keeps the top 8 significand bits of what is left
// (truncation, so every subtraction is exact in fp32)
__device__ __forceinline__ void split3(float x, short& hi, short& mid, short& lo) {
  const float h = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & 0xffff0000u);
  const float r = x - h;
  const float m = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, r) & 0xffff0000u);
  const float l = r - m;  // at most 8 significant bits left
  hi = bf16_bits(h);
  mid = bf16_bits(m);
  lo = static_cast<short>(__builtin_bit_cast(uint32_t, l) >> 16);
}

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// acc[q] += A (16 rows x 32 bags, bf16) x the gradient's three bf16 parts (32 bags x 16 columns,
// column tile q)
__device__ __forceinline__ void dense_mfma(float4_t (&acc)[2], bf16x8 a, const s16x8 (&bh)[2],
                                           const s16x8 (&bm)[2], const s16x8 (&bl)[2]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bh[q]), acc[q], 0, 0, 0);
    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bm[q]), acc[q], 0, 0, 0);
    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bl[q]), acc[q], 0, 0, 0);
  }
}

// The 17 offsets of a wave's 16 bags (lanes 0..16; waves past the last bag read the
// table's end offset), clamped to [0, N].
template <typename OT>
__device__ __forceinline__ int32_t wave_offsets(const OT* __restrict__ offsets, int64_t bag0, int64_t bw,
                                                int nbw, int32_t B, int64_t N) {
  const int lane = lane_id();
  int32_t o = 0;
  if (lane <= kDnWaveBags) {
    const int64_t v = static_cast<int64_t>(offsets[bag0 + min(bw + min(lane, nbw), static_cast<int64_t>(B))]);
    o = static_cast<int32_t>(min(max(v, static_cast<int64_t>(0)), N));
  }
  return o;
}

// Workgroup (t, p) = blockIdx.x: table t's 64-bag steps p, p + P, ...
// The product runs on v_mfma_f32_16x16x32_bf16 with every operand exact in bf16: the gradient
// as three bf16 parts (hi + mid + lo = its fp32 value), a count below 256 as itself, larger
// counts byte by byte (each byte times its power of 256).  Every product is therefore exact,
// and only the fp32 accumulation rounds, as in the fp32 sums of the chunk path.  A step's
// gradient rows and ids are requested together, and the next step's offsets before this
// step's counting, so a step waits on memory about once.
// SLOTS: each lookup's row rank and bag come from dense_slot (two bytes a position, written
// by linearize with the pre-sort pick) instead of its id, the filter, the search of the row
// list and the search of the bag offsets.
// WEIGHTED: a (row, bag) entry is the sum of the per-sample weights of the bag's lookups of the
// row instead of their count, so that entry x gradient row is the sum of the weighted gradient
// rows.  The lanes resolve their lookups' rows in parallel and stage (rank, weight) in LDS by
// position; then one lane per bag adds its bag's staged weights in position order (no atomics:
// every sum is formed in one fixed order).  The sums, fp32 values, are split into three bf16
// parts as the gradient is: each of the nine part products is exact, and only the fp32 sums
// round.
template <typename IT, typename OT, bool SLOTS, bool WEIGHTED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(WEIGHTED ? 2 : 3))) void dense_partial_kernel(
    const IT* __restrict__ indices, const OT* __restrict__ offsets, const float* __restrict__ grad_out,
    const int64_t* __restrict__ meta, int32_t B, int32_t out_width, int64_t N, int P,
    const int32_t* __restrict__ dense_rows, const int32_t* __restrict__ dense_cnt,
    const uint16_t* __restrict__ dense_slot, const float* __restrict__ psw, float* __restrict__ partial) {
  constexpr int kStride = kDnBags + 4;   // counts [row][bag]; rows padded against bank conflicts
  constexpr int kBloomWords = 1024;      // 32768-bit filter of the selected rows (id mod 32768)
  // counts as fp32 (exact integers below 2^24): a count below 256 is then its own bf16 value
  // in the high half of its bits; a wave whose 16 bags hold 2^24 lookups or more counts in
  // uint32 instead (s_intc)
  __shared__ __align__(16) float s_cnt[kDenseRows * kStride];
  __shared__ uint32_t s_bloom[kBloomWords];
  __shared__ int32_t s_rows[kDenseRows];
  __shared__ int32_t s_off[kWavesPerBlock][kDnWaveBags + 1];
  __shared__ int32_t s_intc[kWavesPerBlock];  // 1: the wave's counts of this step are uint32
  const int t = static_cast<int>(blockIdx.x) / P, p = static_cast<int>(blockIdx.x) % P;
  const int nd = dense_cnt[t];
  if (nd == 0) return;  // uniform over the workgroup
  const int ntiles = (nd + 15) / 16;
  const TableMeta m = load_meta(meta, t);
  const int D = static_cast<int>(m.D);
  const int64_t E = m.E;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cw = 32 * w;                // this wave's first column
  const int c2 = cw + 2 * (lane & 15);  // result columns c2 (tile 0) and c2 + 1 (tile 1)
  // the selected rows, ascending (the unused tail padded with a value no id matches), and
  // the filter that lets most ids skip the search
  for (int i = threadIdx.x; i < kBloomWords; i += kBlock) s_bloom[i] = 0u;
  for (int i = threadIdx.x; i < kDenseRows; i += kBlock)
    s_rows[i] = i < nd ? dense_rows[static_cast<int64_t>(t) * kDenseRows + i] : 0x7fffffff;
  __syncthreads();
  for (int i = threadIdx.x; i < nd; i += kBlock) {
    const uint32_t h = static_cast<uint32_t>(s_rows[i]) & (32 * kBloomWords - 1);
    atomicOr(&s_bloom[h >> 5], 1u << (h & 31));
  }
  float4_t acc[kDenseRows / 16][2];
#pragma unroll
  for (int mt = 0; mt < kDenseRows / 16; ++mt) acc[mt][0] = acc[mt][1] = float4_t{0.f, 0.f, 0.f, 0.f};
  int32_t* off = s_off[w];
  const int64_t bag0 = static_cast<int64_t>(t) * B;
  const int64_t steps = (static_cast<int64_t>(B) + kDnBags - 1) / kDnBags;
  auto wave_bags = [&](int64_t st, int64_t& bw, int& nbw) {
    const int nb = static_cast<int>(min<int64_t>(kDnBags, static_cast<int64_t>(B) - st * kDnBags));
    bw = st * kDnBags + kDnWaveBags * w;
    nbw = max(0, min(kDnWaveBags, nb - kDnWaveBags * w));
  };
  int32_t o_next = 0;
  if (p < steps) {
    int64_t bw;
    int nbw;
    wave_bags(p, bw, nbw);
    o_next = wave_offsets(offsets, bag0, bw, nbw, B, N);
  }
  for (int64_t st = p; st < steps; st += P) {
    const int64_t b0 = st * kDnBags;
    const int nb = static_cast<int>(min<int64_t>(kDnBags, static_cast<int64_t>(B) - b0));
    // this wave's bag range from the offsets fetched one step ahead (monotone running max)
    int32_t o = o_next;
    for (int d = 1; d < 32; d <<= 1) {
      const int32_t u = __shfl_up(o, d);
      if (lane >= d) o = max(o, u);
    }
    const int32_t o0 = read_lane(o, 0);
    const int32_t n = read_lane(o, kDnWaveBags) - o0;
    // an fp32 count stops growing at 2^24, which only a wave whose bags hold 2^24 lookups or
    // more can reach: such a wave counts with integer adds on the same slots (its columns are
    // then read as uint32 below; its step always takes the byte-by-byte path, since one of its
    // 16 bags has at least 2^20 lookups)
    const bool intc = n >= (1 << 24);
    // SLOTS: the first slot bytes are requested before the gradient, so that counting (which
    // waits only for them) overlaps the gradient's arrival
    uint32_t sl0[kDnLoads];
    if constexpr (SLOTS && !WEIGHTED) {
#pragma unroll
      for (int u = 0; u < kDnLoads; ++u) {
        const int32_t j = u * kWave + lane;
        sl0[u] = j < n ? dense_slot[o0 + j] : kNoDenseSlot;
      }
    }
    // gradient values: gv[8 kk + j] = bag 32 kk + 8 (l / 16) + j, columns c2, c2 + 1
    f32x2 gv[16];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * kk + 8 * (lane >> 4) + j;
        gv[8 * kk + j] = f32x2{0.f, 0.f};
        if (i < nb && c2 < D)
          gv[8 * kk + j] = *reinterpret_cast<const f32x2*>(grad_out + (b0 + i) * out_width + m.col_base + c2);
      }
    }
    if (st + P < steps) {
      int64_t bw;
      int nbw;
      wave_bags(st + P, bw, nbw);
      o_next = wave_offsets(offsets, bag0, bw, nbw, B, N);
    }
    __syncthreads();  // every wave is done with the previous step's counts (and the filter is set)
    if (lane <= kDnWaveBags) off[lane] = o - o0;
    if (lane == 0) s_intc[w] = intc ? 1 : 0;
    // this wave's 16 bag columns of every row
#pragma unroll
    for (int x = lane; x < kDenseRows * (kDnWaveBags / 4); x += kWave)
      *reinterpret_cast<f32x4*>(&s_cnt[(x >> 2) * kStride + kDnWaveBags * w + 4 * (x & 3)]) = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_wave_barrier();
    // every lookup of the wave's 16 bags that hits a selected row
    if constexpr (WEIGHTED) {
      // rounds of kDnLoads x 64 lookups: every lane resolves its lookups' rows and stages
      // (row, weight) in LDS by position; then lane l < 16 adds bag l's staged weights in
      // position order, from LDS
      __shared__ uint2 s_stage[kWavesPerBlock][kDnLoads * kWave];
      uint2* stage = s_stage[w];
      for (int32_t j0 = 0; j0 < n; j0 += kDnLoads * kWave) {
        int64_t r[kDnLoads];
        float pw[kDnLoads];
#pragma unroll
        for (int u = 0; u < kDnLoads; ++u) {
          const int32_t j = j0 + u * kWave + lane;
          if constexpr (SLOTS) r[u] = j < n ? static_cast<int64_t>(dense_slot[o0 + j]) : kNoDenseSlot;
          else r[u] = j < n ? static_cast<int64_t>(indices[o0 + j]) : -1;
          pw[u] = j < n ? psw[o0 + j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kDnLoads; ++u) {
          uint32_t k = 0xffffffffu;  // the row's rank, or none
          if constexpr (SLOTS) {
            const uint32_t rank = static_cast<uint32_t>(r[u]) & 0xffu;
            if (rank < static_cast<uint32_t>(nd)) k = rank;
          } else if (static_cast<uint64_t>(r[u]) < static_cast<uint64_t>(E)) {
            const int32_t id = static_cast<int32_t>(r[u]);
            const uint32_t h = static_cast<uint32_t>(id) & (32 * kBloomWords - 1);
            if ((s_bloom[h >> 5] >> (h & 31)) & 1u) {
              int kk = 0;  // largest kk with s_rows[kk] <= id (or 0)
#pragma unroll
              for (int step = kDenseRows / 2; step > 0; step >>= 1)
                if (s_rows[kk + step] <= id) kk += step;
              if (s_rows[kk] == id) k = static_cast<uint32_t>(kk);
            }
          }
          stage[u * kWave + lane] = make_uint2(k, __builtin_bit_cast(uint32_t, pw[u]));
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < kDnWaveBags) {
          float* col = &s_cnt[kDnWaveBags * w + lane];  // row k of this bag's column at k * kStride
          const int32_t hi = min(off[lane + 1], j0 + kDnLoads * kWave);
          for (int32_t j = max(off[lane], j0); j < hi; ++j) {
            const uint2 e = stage[j - j0];
            if (e.x < static_cast<uint32_t>(nd)) col[e.x * kStride] += __builtin_bit_cast(float, e.y);
          }
        }
        __builtin_amdgcn_wave_barrier();  // the stage is read before the next round overwrites it
      }
    }
    if constexpr (SLOTS && !WEIGHTED) {
      for (int32_t j0 = 0; j0 < n; j0 += kDnLoads * kWave) {
        uint32_t sl[kDnLoads];
#pragma unroll
        for (int u = 0; u < kDnLoads; ++u) {
          const int32_t j = j0 + u * kWave + lane;
          sl[u] = j0 == 0 ? sl0[u] : (j < n ? dense_slot[o0 + j] : kNoDenseSlot);
        }
#pragma unroll
        for (int u = 0; u < kDnLoads; ++u) {
          if (j0 + u * kWave >= n) break;  // uniform: no lane has a lookup left
          const uint32_t rank = sl[u] & 0xffu;
          if (rank < static_cast<uint32_t>(nd)) {  // the wave's bags start at a multiple of 16
            float* c = &s_cnt[rank * kStride + kDnWaveBags * w + ((sl[u] >> 8) & 15u)];
            if (intc) atomicAdd(reinterpret_cast<uint32_t*>(c), 1u);
            else atomicAdd(c, 1.f);
          }
        }
      }
    }
    for (int32_t j0 = 0; !SLOTS && !WEIGHTED && j0 < n; j0 += kDnLoads * kWave) {
      int64_t r[kDnLoads];
#pragma unroll
      for (int u = 0; u < kDnLoads; ++u) {
        const int32_t j = j0 + u * kWave + lane;
        r[u] = j < n ? static_cast<int64_t>(indices[o0 + j]) : -1;
      }
#pragma unroll
      for (int u = 0; u < kDnLoads; ++u) {
        if (j0 + u * kWave >= n) break;  // uniform: no lane has an id left
        const int32_t j = j0 + u * kWave + lane;
        if (static_cast<uint64_t>(r[u]) < static_cast<uint64_t>(E)) {
          const int32_t id = static_cast<int32_t>(r[u]);
          const uint32_t h = static_cast<uint32_t>(id) & (32 * kBloomWords - 1);
          if ((s_bloom[h >> 5] >> (h & 31)) & 1u) {
            int k = 0;  // largest k with s_rows[k] <= id (or 0)
#pragma unroll
            for (int step = kDenseRows / 2; step > 0; step >>= 1)
              if (s_rows[k + step] <= id) k += step;
            if (s_rows[k] == id) {
              int b = 0;  // the bag of lookup j
#pragma unroll
              for (int step = 8; step > 0; step >>= 1)
                if (off[b + step] <= j) b += step;
              float* c = &s_cnt[k * kStride + kDnWaveBags * w + b];
              if (intc) atomicAdd(reinterpret_cast<uint32_t*>(c), 1u);
              else atomicAdd(c, 1.f);
            }
          }
        }
      }
    }
    __syncthreads();  // all 64 bags counted
    // a count can reach 256 only in a bag of at least 256 lookups: lane l checks bag l % 16
    // of wave l / 16 (bags past the last have no lookups)
    const bool any_big =
        __ballot(s_off[lane >> 4][(lane & 15) + 1] - s_off[lane >> 4][lane & 15] >= 256) != 0;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s16x8 bh[2], bm[2], bl[2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          short h, mi, lo;
          split3(q ? gv[8 * kk + j].y : gv[8 * kk + j].x, h, mi, lo);
          bh[q][j] = h;
          bm[q][j] = mi;
          bl[q][j] = lo;
        }
      }
#pragma unroll
      for (int mt = 0; mt < kDenseRows / 16; ++mt) {
        if (mt < ntiles) {
          const float* src = &s_cnt[(16 * mt + (lane & 15)) * kStride + 32 * kk + 8 * (lane >> 4)];
          const u32x4 c0 = *reinterpret_cast<const u32x4*>(src);
          const u32x4 c1 = *reinterpret_cast<const u32x4*>(src + 4);
          if constexpr (WEIGHTED) {
            // the weight sums as three bf16 parts each, against the gradient's three parts
            const uint32_t cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            s16x8 ah, am, al;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              short h, mi, lo;
              split3(__builtin_bit_cast(float, cv[j]), h, mi, lo);
              ah[j] = h;
              am[j] = mi;
              al[j] = lo;
            }
            dense_mfma(acc[mt], __builtin_bit_cast(bf16x8, ah), bh, bm, bl);
            dense_mfma(acc[mt], __builtin_bit_cast(bf16x8, am), bh, bm, bl);
            dense_mfma(acc[mt], __builtin_bit_cast(bf16x8, al), bh, bm, bl);
          } else if (!any_big) {
            // every count is below 256: the high halves of the fp32 counts are their bf16 values
            const u32x4 pk = {__builtin_amdgcn_perm(c0.y, c0.x, 0x07060302u),
                              __builtin_amdgcn_perm(c0.w, c0.z, 0x07060302u),
                              __builtin_amdgcn_perm(c1.y, c1.x, 0x07060302u),
                              __builtin_amdgcn_perm(c1.w, c1.z, 0x07060302u)};
            dense_mfma(acc[mt], __builtin_bit_cast(bf16x8, pk), bh, bm, bl);
          } else {
            // byte by byte: byte lv of a count times 256^lv has at most 8 significant bits.
            // The lane's 8 bag columns belong to wave 2 kk + lane / 32, whose counts are fp32
            // or (intc) uint32
            const uint32_t cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const bool ic = s_intc[2 * kk + (lane >> 5)] != 0;
#pragma unroll 1
            for (int lv = 0; lv < 4; ++lv) {
              u32x4 pk;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t a = ic ? cv[2 * j] : static_cast<uint32_t>(__builtin_bit_cast(float, cv[2 * j]));
                const uint32_t b = ic ? cv[2 * j + 1] : static_cast<uint32_t>(__builtin_bit_cast(float, cv[2 * j + 1]));
                const float lo = static_cast<float>(((a >> (8 * lv)) & 255u) << (8 * lv));
                const float hi = static_cast<float>(((b >> (8 * lv)) & 255u) << (8 * lv));
                pk[j] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                                              0x07060302u);
              }
              dense_mfma(acc[mt], __builtin_bit_cast(bf16x8, pk), bh, bm, bl);
            }
          }
        }
      }
    }
  }
  // every workgroup of the table writes its partial (zeros when it had no step)
  float* dst = partial + static_cast<int64_t>(blockIdx.x) * kDenseRows * kDnCols;
  if (c2 < D) {
#pragma unroll
    for (int mt = 0; mt < kDenseRows / 16; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * mt + 4 * (lane >> 4) + i;
        if (row < nd) *reinterpret_cast<f32x2*>(dst + row * kDnCols + c2) = f32x2{acc[mt][0][i], acc[mt][1][i]};
      }
    }
  }
}

// Workgroup (t, k) = blockIdx.x: selected row k of table t.  Thread (g, q) sums partials
// g, g + 8, ... of column quad q in increasing order, the eight sums are added in g order,
// then the row's optimizer step.
template <int DT, int OPT>
__global__ __launch_bounds__(kBlock) void dense_apply_kernel(
    typename Fmt<DT>::S* __restrict__ W, float* __restrict__ momentum, const int64_t* __restrict__ meta,
    int P, const int32_t* __restrict__ dense_rows, const int32_t* __restrict__ dense_cnt,
    const float* __restrict__ partial, float lr, float eps) {
  using S = typename Fmt<DT>::S;
  constexpr int kGroups = kBlock / (kDnCols / 4);  // 8
  __shared__ __align__(16) float s_part[kGroups][kDnCols];
  const int t = static_cast<int>(blockIdx.x) / kDenseRows, k = static_cast<int>(blockIdx.x) % kDenseRows;
  if (k >= dense_cnt[t]) return;
  const TableMeta m = load_meta(meta, t);
  const int D = static_cast<int>(m.D);
  const int q = threadIdx.x & (kDnCols / 4 - 1), g = threadIdx.x / (kDnCols / 4);
  const int col = 4 * q;
  if (col < D) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    const float* src = partial + (static_cast<int64_t>(t) * P * kDenseRows + k) * kDnCols + col;
    const int64_t pstride = static_cast<int64_t>(kDenseRows) * kDnCols;
    int pp = g;
    for (; pp + 3 * kGroups < P; pp += 4 * kGroups) {
      const f32x4 x0 = load_f4(src + pp * pstride);
      const f32x4 x1 = load_f4(src + (pp + kGroups) * pstride);
      const f32x4 x2 = load_f4(src + (pp + 2 * kGroups) * pstride);
      const f32x4 x3 = load_f4(src + (pp + 3 * kGroups) * pstride);
      a += x0; a += x1; a += x2; a += x3;
    }
    for (; pp < P; pp += kGroups) a += load_f4(src + pp * pstride);
    *reinterpret_cast<f32x4*>(&s_part[g][col]) = a;
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  // wave 0 finishes: lane l owns columns 4 l .. 4 l + 3
  const int lane = threadIdx.x;
  const int c = 4 * lane;
  const bool act = lane < kDnCols / 4 && c < D;
  const int64_t row = dense_rows[static_cast<int64_t>(t) * kDenseRows + k];
  S* wrow = W + m.w_base + row * D;
  float gv[4] = {0.f, 0.f, 0.f, 0.f};
  float wv[4] = {0.f, 0.f, 0.f, 0.f};
  if (act) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s = s_part[0][c + e];
#pragma unroll
      for (int gg = 1; gg < kGroups; ++gg) s += s_part[gg][c + e];
      gv[e] = s;
    }
    load_vec<DT, 4>(wrow + c, wv);
  }
  if constexpr (OPT == kOptSGD) {
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] -= lr * gv[e];
  } else {
    float ss = gv[0] * gv[0] + gv[1] * gv[1] + gv[2] * gv[2] + gv[3] * gv[3];
    for (int msk = 1; msk < kWave; msk <<= 1) ss += __shfl_xor(ss, msk);
    const int64_t key = m.row_base + row;
    const float mnew = momentum[key] + ss / static_cast<float>(D);
    const float denom = sqrtf(mnew) + eps;
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[e] -= lr * gv[e] / denom;
    if (lane == 0) momentum[key] = mnew;
  }
  if (act) store_vec4<DT>(wrow + c, wv);
}

template <typename IT, typename OT, bool SLOTS, bool WEIGHTED>
void partial_launch(const tbe_tables* tb, const IndexArgs& ia, const float* grad_out, const float* psw,
                    char* ws, const BwdLayout& L, int P, const uint16_t* slot, hipStream_t s) {
  hipLaunchKernelGGL((dense_partial_kernel<IT, OT, SLOTS, WEIGHTED>), dim3(tb->T * P), dim3(kBlock), 0, s,
                     static_cast<const IT*>(ia.indices), static_cast<const OT*>(ia.offsets), grad_out,
                     tb->meta, tb->B, tb->out_width, ia.N, P,
                     reinterpret_cast<const int32_t*>(ws + L.dense_rows),
                     reinterpret_cast<const int32_t*>(ws + L.dense_cnt), slot, psw,
                     reinterpret_cast<float*>(ws + L.dense_partial));
}

template <typename IT, typename OT>
tbe_status partial_go(const tbe_tables* tb, const IndexArgs& ia, const float* grad_out, const float* psw,
                      char* ws, const BwdLayout& L, int P, hipStream_t s) {
  ProfScope ps("dense_partial", s);
  const uint16_t* slot = L.dense_presort ? reinterpret_cast<const uint16_t*>(ws + L.dense_slot) : nullptr;
  if (slot) {
    if (psw) partial_launch<IT, OT, true, true>(tb, ia, grad_out, psw, ws, L, P, slot, s);
    else partial_launch<IT, OT, true, false>(tb, ia, grad_out, psw, ws, L, P, slot, s);
  } else {
    if (psw) partial_launch<IT, OT, false, true>(tb, ia, grad_out, psw, ws, L, P, slot, s);
    else partial_launch<IT, OT, false, false>(tb, ia, grad_out, psw, ws, L, P, slot, s);
  }
  return check_launch("dense_partial");
}

template <int DT, int OPT>
tbe_status apply_dense_go(const tbe_tables* tb, void* W, float* momentum, char* ws, const BwdLayout& L,
                          int P, float lr, float eps, hipStream_t s) {
  using S = typename Fmt<DT>::S;
  ProfScope ps("dense_apply", s);
  hipLaunchKernelGGL((dense_apply_kernel<DT, OPT>), dim3(tb->T * kDenseRows), dim3(kBlock), 0, s,
                     static_cast<S*>(W), momentum, tb->meta, P,
                     reinterpret_cast<const int32_t*>(ws + L.dense_rows),
                     reinterpret_cast<const int32_t*>(ws + L.dense_cnt),
                     reinterpret_cast<const float*>(ws + L.dense_partial), lr, eps);
  return check_launch("dense_apply");
}

template <typename IT, typename OT>
tbe_status sample_go(const tbe_tables* tb, const IndexArgs& ia, int hist_t, int invalid_as_row0, char* ws,
                     const BwdLayout& L, hipStream_t s) {
  const SortPlan& P = L.sample;
  const int64_t nsamp = P.N / kWave;
  const auto kernel = dense_sample_kernel<IT, OT>;
  const int grid = resident_grid(kernel, (nsamp + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<const IT*>(ia.indices),
                     static_cast<const OT*>(ia.offsets), tb->meta, tb->T, tb->B, ia.N,
                     static_cast<int64_t>(L.hot_stride), nsamp, hist_t, invalid_as_row0,
                     static_cast<uint32_t>(tb->total_rows), reinterpret_cast<uint32_t*>(ws + P.keys[0]),
                     reinterpret_cast<uint32_t*>(ws + P.pay[0]));
  return check_launch("dense_sample");
}

}  // namespace

tbe_status launch_dense_sample(const tbe_tables* tb, const IndexArgs& ia, int hist_t, int invalid_as_row0,
                               char* ws, const BwdLayout& L, hipStream_t s) {
  if (ia.itype == TBE_I32)
    return ia.otype == TBE_I32 ? sample_go<int32_t, int32_t>(tb, ia, hist_t, invalid_as_row0, ws, L, s)
                               : sample_go<int32_t, int64_t>(tb, ia, hist_t, invalid_as_row0, ws, L, s);
  return ia.otype == TBE_I32 ? sample_go<int64_t, int32_t>(tb, ia, hist_t, invalid_as_row0, ws, L, s)
                             : sample_go<int64_t, int64_t>(tb, ia, hist_t, invalid_as_row0, ws, L, s);
}

tbe_status launch_dense_select(const tbe_tables* tb, char* ws, const BwdLayout& L, int hist_t,
                               hipStream_t s) {
  const SortPlan& P = L.sample;
  hipLaunchKernelGGL(dense_select_kernel, dim3((tb->T + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, s,
                     reinterpret_cast<const uint4*>(ws + P.long_list),
                     reinterpret_cast<const uint32_t*>(ws + P.long_table),
                     reinterpret_cast<const int32_t*>(ws + P.counters), P.cap_long, tb->meta, tb->T, hist_t, 0u,
                     reinterpret_cast<int32_t*>(ws + L.dense_rows), reinterpret_cast<int32_t*>(ws + L.dense_cnt),
                     nullptr, reinterpret_cast<uint32_t*>(ws + L.hot_set),
                     static_cast<uint32_t>(L.hot_set_size - 1),
                     reinterpret_cast<uint32_t*>(ws + L.hot_bloom),
                     reinterpret_cast<int32_t*>(ws + L.counters) + kHotProbe);
  return check_launch("dense_select");
}

tbe_status launch_dense_select_runs(const tbe_tables* tb, char* ws, const BwdLayout& L, int hist_t,
                                    const Config& cfg, hipStream_t s) {
  ProfScope ps("dense_select", s);
  hipLaunchKernelGGL(dense_select_kernel, dim3((tb->T + kWavesPerBlock - 1) / kWavesPerBlock), dim3(kBlock), 0, s,
                     reinterpret_cast<const uint4*>(ws + L.long_list),
                     reinterpret_cast<const uint32_t*>(ws + L.long_table),
                     reinterpret_cast<const int32_t*>(ws + L.counters), L.cap_long, tb->meta, tb->T, hist_t,
                     static_cast<uint32_t>(cfg.dense_min), reinterpret_cast<int32_t*>(ws + L.dense_rows),
                     reinterpret_cast<int32_t*>(ws + L.dense_cnt), reinterpret_cast<uint32_t*>(ws + L.long_flag),
                     nullptr, 0u, nullptr, nullptr);
  return check_launch("dense_select");
}

int dense_partial_blocks_per_cu() {
  return blocks_per_cu(reinterpret_cast<const void*>(dense_partial_kernel<int64_t, int64_t, true, false>));
}

tbe_status launch_dense_backward(const tbe_tables* tb, void* W, float* momentum, int opt,
                                 const IndexArgs& ia, const float* psw, const float* grad_out, float lr,
                                 float eps, char* ws, const BwdLayout& L, hipStream_t s, int wgs_per_cu) {
  // partials per table: as many workgroups as the GPU holds at once over all tables (one
  // round, no tail), or wgs_per_cu a CU, at most the workspace's dense_P
  // (the weighted instance holds fewer workgroups a CU: registers and its LDS stage)
  const void* k = psw ? reinterpret_cast<const void*>(dense_partial_kernel<int64_t, int64_t, false, true>)
                      : reinterpret_cast<const void*>(dense_partial_kernel<int64_t, int64_t, false, false>);
  const int64_t resident = static_cast<int64_t>(device_cu_count()) * (wgs_per_cu > 0 ? wgs_per_cu : blocks_per_cu(k));
  const int P = static_cast<int>(hmax(1, hmin(L.dense_P, resident / tb->T)));
  tbe_status st;
  if (ia.itype == TBE_I32)
    st = ia.otype == TBE_I32 ? partial_go<int32_t, int32_t>(tb, ia, grad_out, psw, ws, L, P, s)
                             : partial_go<int32_t, int64_t>(tb, ia, grad_out, psw, ws, L, P, s);
  else
    st = ia.otype == TBE_I32 ? partial_go<int64_t, int32_t>(tb, ia, grad_out, psw, ws, L, P, s)
                             : partial_go<int64_t, int64_t>(tb, ia, grad_out, psw, ws, L, P, s);
  if (st) return st;
#define TBE_DA(DT) \
  (opt == kOptSGD ? apply_dense_go<DT, kOptSGD>(tb, W, momentum, ws, L, P, lr, eps, s) \
                  : apply_dense_go<DT, kOptAdagrad>(tb, W, momentum, ws, L, P, lr, eps, s))
  switch (tb->w_dtype) {
    case TBE_F32: return TBE_DA(0);
    case TBE_F16: return TBE_DA(1);
    default: return TBE_DA(2);
  }
#undef TBE_DA
}

}  // namespace tbe
