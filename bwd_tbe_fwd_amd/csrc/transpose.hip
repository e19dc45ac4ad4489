// Backward transpose and routing: linearize, stable LSD radix sort, run-length
// encoding, and classification of runs by segment length with D buckets.
//
// PyTorch blog "Modernizing Table Batched Embeddings with FBTriton", section 3:
// transpose_embedding_input inverts the batch into runs, each one unique
// (table, row) with the lookups that touched it, so that no two runs write the
// same row; runs are routed by segment length (SL, the lookups of a run):
// SL < 256 to short_run, longer runs to 256-lookup chunks.  Section 4, problem 3:
// short runs are bucketed by next_pow2(D) during classification, and run counts
// stay on the device (stream compaction with one atomic per block and a
// prefix sum inside the block), so nothing is read back.
// "Table-Batched Embeddings in Triton", section 2: the linearized id is the
// table's first row plus the local id, sorted stably.
//
// gfx950 design:
//  - linearize: a wave takes 64 consecutive bags (their offsets in one load),
//    and its lanes walk the contiguous lookups of those bags, 8 positions a
//    lane per step, each lane finding its bag by a 6-step binary search over
//    the 64 end offsets (lane shuffles).  With the dense rows picked before the
//    sort, their lookups get the sentinel key (a filter in LDS, then a probe of
//    the hashed key set) and every position gets its dense slot.
//  - sort: reduce-then-scan LSD radix, up to 9 bits a pass (26-bit keys take 3
//    passes); the first pass leaves the sentinel keys out, and the later
//    kernels read the kept count from the device.  When the largest table needs
//    fewer bits than the linearized ids, each table's keys are sorted on their
//    own on local row bits (same order, smaller digits; see the radix section).
//    The dense-row pick sorts its sample with the same kernels (sort_route).  A
//    fixed number of blocks each own a contiguous segment; per pass:
//    upsweep (digit counts per block), a per-digit scan across blocks, and a
//    downsweep that ranks each 4096-key tile stably in LDS (wave ballots find
//    the lanes holding the same digit; the lowest lane adds the count), sorts
//    the tile by digit in LDS and writes each digit's keys contiguously.  No
//    inter-block waiting, so every wave always finishes.
//  - RLE: head flags counted per block, scanned, then written in order.
//  - classify: per-block category counts, a scan across blocks, an ordered
//    write: lists in key order, no global atomics.
#include "sort_common.h"
#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {
namespace {

// ---------------------------------------------------------------------------
// linearize
// ---------------------------------------------------------------------------
// One wave takes 64 consecutive bags; lane l finds, for each lookup position p
// of the group, the bag that owns it by a 6-step search of the lanes' end
// offsets.  Lookups of table skip_t (>= 0: its rows are updated elsewhere) are
// left out and the positions after them close up, so the sort sees
// N - (lookups of skip_t) keys; that count goes to *n_eff.  Positions that no
// bag covers (possible only with offsets that break the documented contract)
// get the sentinel key, so every key and payload the sort reads is defined.
// hot_set != NULL: keys in the dense-row key set (hot_mask + 1 words of records; the most
// records a lookup reads in *hot_probes) get the sentinel key too, and every position of a bag (and
// every position no bag covers) gets its dense slot: the rank of its row among its table's
// dense rows and its bag modulo 16, or kNoDenseSlot (positions of the table left out,
// skip_t, are not written): those lookups are the
// dense path's.  The set's filter goes into LDS; keys that pass it probe the set (a
// whole copy in LDS measured slower: it cost occupancy, and most probes are hits anyway).
constexpr int kLinU = 8;  // positions per lane per step
template <typename IT, typename OT, bool WEIGHTED>
__global__ __launch_bounds__(kBlock) void linearize_kernel(
    const IT* __restrict__ indices, const OT* __restrict__ offsets, const int64_t* __restrict__ meta,
    int32_t B, int64_t nbags, int32_t N, uint32_t sentinel, int skip_t, int invalid_as_row0,
    const uint32_t* __restrict__ hot_filter, const uint32_t* __restrict__ hot_set,
    uint32_t hot_mask, const int32_t* __restrict__ hot_probes,
    uint16_t* __restrict__ dense_slot, uint32_t* __restrict__ keys,
    uint32_t* __restrict__ pay, uint32_t* __restrict__ bag_of, int32_t* __restrict__ n_eff) {
  __shared__ __align__(16) uint32_t s_filter[kHotBloomWords];
  int hot_max = 0;
  if (hot_set) {
    for (int i = 4 * threadIdx.x; i < kHotBloomWords; i += 4 * kBlock)
      *reinterpret_cast<u32x4*>(s_filter + i) = *reinterpret_cast<const u32x4*>(hot_filter + i);
    hot_max = *hot_probes;
    __syncthreads();
  }
  const int lane = lane_id();
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
  auto clampN = [N](int64_t v, int64_t lo) {
    return static_cast<int32_t>(min(max(v, lo), static_cast<int64_t>(N)));
  };
  // the skipped table's lookups [skip_lo, skip_lo + skip_len)
  int32_t skip_lo = 0, skip_len = 0;
  if (skip_t >= 0) {
    skip_lo = clampN(static_cast<int64_t>(offsets[static_cast<int64_t>(skip_t) * B]), 0);
    skip_len = clampN(static_cast<int64_t>(offsets[static_cast<int64_t>(skip_t + 1) * B]), skip_lo) - skip_lo;
    if (wave == 0 && lane == 0) *n_eff = N - skip_len;
  }
  auto compact = [skip_lo, skip_len](int32_t p) { return p - min(max(p - skip_lo, 0), skip_len); };
  auto fill = [&](int32_t lo, int32_t hi) {
    for (int32_t p = lo + lane; p < hi; p += kWave) {
      const int32_t q = compact(p);
      keys[q] = sentinel;
      if (hot_set) dense_slot[p] = kNoDenseSlot;
      if constexpr (WEIGHTED) {
        pay[q] = static_cast<uint32_t>(p);
        bag_of[p] = 0u;
      } else {
        pay[q] = 0u;
      }
    }
  };
  if (nbags == 0 && wave == 0) fill(0, N);
  for (int64_t g0 = wave * kWave; g0 < nbags; g0 += nwaves * kWave) {
    const int64_t glast = min(g0 + kWave, nbags) - 1;
    if (skip_t >= 0 && g0 / B == skip_t && glast / B == skip_t) continue;  // all 64 bags skipped
    const int64_t bag = g0 + lane;
    const int32_t S = clampN(static_cast<int64_t>(offsets[g0]), 0);
    int32_t e = S;
    int64_t rb = 0, E = 0;
    bool skip = false;
    if (bag < nbags) {
      e = clampN(static_cast<int64_t>(offsets[bag + 1]), S);
      const int t = static_cast<int>(bag / B);
      rb = meta[4 * t];
      E = meta[4 * (t + 1)] - rb;
      skip = t == skip_t;
    }
    const int64_t tb0 = (g0 / B) * B;  // first bag of the group's first table
    // monotone end offsets across the 64 lanes (inclusive running max)
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t u = __shfl_up(e, d);
      if (lane >= d) e = max(e, u);
    }
    const int32_t Eend = __shfl(e, kWave - 1);
    const uint64_t skip_mask = __ballot(skip);
    // kLinU positions a lane per step: their ids (and then their key-set probes) are
    // requested together
    for (int32_t base = S; base < Eend; base += kLinU * kWave) {
      int32_t p[kLinU];
      int k[kLinU];
      bool act[kLinU];
      uint32_t key[kLinU];
#pragma unroll
      for (int u = 0; u < kLinU; ++u) {
        p[u] = base + u * kWave + lane;
        // first lane l with e_l > p
        int lo = 0, hi = kWave - 1;
#pragma unroll
        for (int step = 0; step < 6; ++step) {
          const int mid = (lo + hi) >> 1;
          const int32_t em = __shfl(e, mid);
          if (em > p[u]) hi = mid; else lo = mid + 1;
        }
        k[u] = lo;
        act[u] = p[u] < Eend && !((skip_mask >> lo) & 1ull);
      }
      int64_t r[kLinU];
#pragma unroll
      for (int u = 0; u < kLinU; ++u) r[u] = act[u] ? static_cast<int64_t>(indices[p[u]]) : 0;
#pragma unroll
      for (int u = 0; u < kLinU; ++u) {
        const int64_t rbk = __shfl(rb, k[u]);
        const int64_t Ek = __shfl(E, k[u]);
        key[u] = (static_cast<uint64_t>(r[u]) < static_cast<uint64_t>(Ek))
                     ? static_cast<uint32_t>(rbk + r[u])
                     : (invalid_as_row0 ? static_cast<uint32_t>(rbk) : sentinel);
      }
      uint32_t slot[kLinU];  // rank among the table's dense rows, or kNoDenseSlot
#pragma unroll
      for (int u = 0; u < kLinU; ++u) slot[u] = kNoDenseSlot;
      if (hot_set) {
        // the filter, then every candidate's first record (three keys and their ranks, one
        // 16-byte load) at once; the rare full record without the key sends its lanes to the
        // next records, all together
        bool pend[kLinU];
        uint32_t h[kLinU];
        u32x4 v[kLinU];
#pragma unroll
        for (int u = 0; u < kLinU; ++u) {
          const uint32_t f = hot_filter_bit(key[u]);
          pend[u] = act[u] && key[u] != sentinel && ((s_filter[f >> 5] >> (f & 31)) & 1u);
          h[u] = hot_slot(key[u], hot_mask);
        }
        for (int g = 0; g < hot_max; ++g) {
#pragma unroll
          for (int u = 0; u < kLinU; ++u) {
            if (!pend[u]) continue;
            const uint32_t e = (h[u] + 4 * g) & hot_mask;
            v[u] = *reinterpret_cast<const u32x4*>(hot_set + e);
          }
          bool more = false;
#pragma unroll
          for (int u = 0; u < kLinU; ++u) {
            if (!pend[u]) continue;
            const uint32_t kk = key[u];
            const bool hit = v[u].x == kk || v[u].y == kk || v[u].z == kk;
            const bool gap = v[u].x == kHotEmpty || v[u].y == kHotEmpty || v[u].z == kHotEmpty;
            if (hit) {
              const int j = v[u].x == kk ? 0 : (v[u].y == kk ? 1 : 2);
              slot[u] = (v[u].w >> (8 * j)) & 0xffu;  // the bag's part is added below
              key[u] = sentinel;
            }
            pend[u] = !hit && !gap;
            more |= pend[u];
          }
          if (!__ballot(more)) break;
        }
      }
#pragma unroll
      for (int u = 0; u < kLinU; ++u) {
        if (hot_set && p[u] < Eend) {
          // the bag's index within its table, modulo 16 (the group's 64 bags start in table
          // g0 / B: one step past a table's end per table crossed)
          int32_t local = static_cast<int32_t>(g0 + k[u] - tb0);
          while (local >= B) local -= B;
          const uint32_t bb = static_cast<uint32_t>(local & 15);
          dense_slot[p[u]] = static_cast<uint16_t>(slot[u] == kNoDenseSlot ? slot[u] : (slot[u] | (bb << 8)));
        }
        if (!act[u]) continue;
        const int32_t q = compact(p[u]);
        keys[q] = key[u];
        const uint32_t b = static_cast<uint32_t>(g0 + k[u]);
        if constexpr (WEIGHTED) {
          pay[q] = static_cast<uint32_t>(p[u]);
          bag_of[p[u]] = b;
        } else {
          pay[q] = b;
        }
      }
    }
    // positions no bag covers: before the first bag, and between this group's end
    // and the next group's start
    if (g0 == 0) fill(0, S);
    const int32_t Snext = g0 + kWave < nbags ? clampN(static_cast<int64_t>(offsets[g0 + kWave]), 0) : N;
    fill(Eend, Snext);
  }
}

// ---------------------------------------------------------------------------
// radix sort
// ---------------------------------------------------------------------------
// Two plans share the kernels below.  Global: the keys are sorted on their whole value, and
// block b owns [b seg, (b + 1) seg) of a pass's input.  BY_TABLE: linearize leaves each table's
// lookups together, in the batch's table order, and a key of table t is its row base plus the
// local row, so sorting each table's range on its own, on the bits of the local row, gives the
// order of the global sort — with fewer bits a pass when the largest table is much smaller
// than all tables together (2M-row tables of a 64M-row batch: three 7-bit passes instead of
// three 9-bit ones, so a 4096-key tile holds about 32 keys of a digit instead of 8, written out
// as longer contiguous pieces).  A pass's blocks are dealt to the tables: table t takes blocks
// [f(t), f(t + 1)) with f(t) = t + (nblk - T) start_t / n (at least one each, the rest in
// proportion to the keys), which split the table's range evenly.  The per-digit scan over
// blocks is the global one; a block of table t derives its digit bases from it, and each
// table's first block records where the table starts in the pass's output (the next pass's
// start_t).  start_t must be non-decreasing, start_0 = 0 and start_T = n, the pass's keys.

// f(t): the first block of table t (f(T) = nblk)
__device__ __forceinline__ int table_first_block(const int32_t* __restrict__ start, int T, int nblk, int t) {
  if (t >= T) return nblk;
  const int64_t n = start[T];
  return t + static_cast<int>(n > 0 ? static_cast<int64_t>(nblk - T) * start[t] / n : 0);
}

struct TableRange {
  int t, first, last;  // the block's table and that table's blocks [first, last)
  int32_t lo, hi;      // the block's keys
};

__device__ TableRange table_range(const int32_t* __restrict__ start, int T, int nblk, int b) {
  int lo = 0, hi = T;  // f(lo) <= b < f(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (table_first_block(start, T, nblk, mid) <= b) lo = mid;
    else hi = mid;
  }
  TableRange r;
  r.t = lo;
  r.first = table_first_block(start, T, nblk, lo);
  r.last = table_first_block(start, T, nblk, lo + 1);
  const int64_t s0 = start[lo], s1 = max(start[lo + 1], start[lo]);
  const int64_t per = (s1 - s0 + (r.last - r.first) - 1) / (r.last - r.first);
  const int64_t a = min(s0 + static_cast<int64_t>(b - r.first) * per, s1);
  r.lo = static_cast<int32_t>(a);
  r.hi = static_cast<int32_t>(min(a + per, s1));
  return r;
}

// BY_TABLE plan, before the first pass: where each table's keys start in linearize's output (the
// batch's table order, the left-out table's lookups closed up), clamped into [0, n] and made
// non-decreasing; start[T] = n = N - (the left-out table's lookups), the keys linearize wrote.
// One workgroup.
template <typename OT>
__global__ __launch_bounds__(kBlock) void table_starts_kernel(const OT* __restrict__ offsets, int T, int32_t B,
                                                             int32_t N, int skip_t, int32_t* __restrict__ start) {
  __shared__ int32_t s_tmp[kWavesPerBlock];
  auto at = [&](int64_t i) {
    return static_cast<int32_t>(min(max(static_cast<int64_t>(offsets[i]), int64_t{0}), static_cast<int64_t>(N)));
  };
  int32_t skip_lo = 0, skip_len = 0;
  if (skip_t >= 0) {
    skip_lo = at(static_cast<int64_t>(skip_t) * B);
    skip_len = max(at(static_cast<int64_t>(skip_t + 1) * B), skip_lo) - skip_lo;
  }
  const int32_t n = N - skip_len;
  const int ipt = (T + 1 + kBlock - 1) / kBlock;
  const int i0 = threadIdx.x * ipt;
  int32_t run = 0;  // running maximum over this thread's entries
  for (int q = 0; q < ipt; ++q) {
    const int t = i0 + q;
    if (t > T) break;
    int32_t v = n;
    if (t == 0) {
      v = 0;
    } else if (t < T) {
      const int32_t p = at(static_cast<int64_t>(t) * B);
      v = p - min(max(p - skip_lo, 0), skip_len);
    }
    run = max(run, v);
  }
  // exclusive maximum over the threads before this one (all values are >= 0)
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int32_t inc = run;
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t u = __shfl_up(inc, d);
    if (lane >= d) inc = max(inc, u);
  }
  if (lane == kWave - 1) s_tmp[w] = inc;
  __syncthreads();
  int32_t pre = __shfl_up(inc, 1);
  if (lane == 0) pre = 0;
  for (int k = 0; k < w; ++k) pre = max(pre, s_tmp[k]);
  run = pre;
  for (int q = 0; q < ipt; ++q) {
    const int t = i0 + q;
    if (t > T) break;
    int32_t v = n;
    if (t == 0) {
      v = 0;
    } else if (t < T) {
      const int32_t p = at(static_cast<int64_t>(t) * B);
      v = p - min(max(p - skip_lo, 0), skip_len);
    }
    run = max(run, v);
    start[t] = t == T ? n : run;
  }
}

// drop: a key equal to it is not counted (the first pass leaves out the sentinel keys;
// later passes pass a value no key has)
template <bool BY_TABLE>
__global__ __launch_bounds__(kBlock) void radix_upsweep(const uint32_t* __restrict__ keys, int64_t N,
                                                        const int32_t* __restrict__ n_eff,
                                                        int64_t seg, int shift, int bits, uint32_t drop,
                                                        uint32_t* __restrict__ hist, int nblk,
                                                        const int32_t* __restrict__ tstart,
                                                        const int64_t* __restrict__ meta, int T) {
  __shared__ uint32_t s_cnt[kWavesPerBlock][kRadixDigits];
  __shared__ int32_t s_rng[3];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int ndig = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(ndig - 1);
  for (int i = lane; i < ndig; i += kWave) s_cnt[w][i] = 0;
  int64_t lo, hi;
  uint32_t rb = 0;  // the row base subtracted before the digit is taken
  if constexpr (BY_TABLE) {
    if (threadIdx.x == 0) {
      const TableRange r = table_range(tstart, T, nblk, blockIdx.x);
      s_rng[0] = r.t;
      s_rng[1] = r.lo;
      s_rng[2] = r.hi;
    }
    __syncthreads();
    rb = static_cast<uint32_t>(meta[4 * s_rng[0]]);
    lo = s_rng[1];
    hi = s_rng[2];
  } else {
    if (n_eff) N = min(N, static_cast<int64_t>(*n_eff));
    lo = blockIdx.x * seg;
    hi = min(lo + seg, N);
    __builtin_amdgcn_wave_barrier();
  }
  // each wave reads 4 x 256 consecutive keys per step, 16 bytes per lane per load, from the
  // 16-byte boundary at or below lo
  for (int64_t base = (lo & ~int64_t{3}) + w * 16 * kWave; base < hi; base += 16 * kBlock) {
    uint32_t k[16];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t i = base + s * 4 * kWave + 4 * lane;
      if (i >= lo && i + 3 < hi) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(keys + i);
        k[4 * s] = v.x; k[4 * s + 1] = v.y; k[4 * s + 2] = v.z; k[4 * s + 3] = v.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) k[4 * s + q] = (i + q >= lo && i + q < hi) ? keys[i + q] : 0u;
      }
    }
    // counts are order-free: one LDS atomic add per key, except where keys repeat.  After the
    // first pass a hot row's lookups lie side by side, so whole groups of four (and whole
    // waves of groups) carry one digit, and adding them one by one would serialize on one
    // LDS address: such a group adds 4 at once, such a wave 256 from one lane.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t i0 = base + s * 4 * kWave + 4 * lane;
      uint32_t d[4];
      bool ok[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        d[q] = ((k[4 * s + q] - rb) >> shift) & mask;
        ok[q] = i0 + q >= lo && i0 + q < hi && k[4 * s + q] != drop;
      }
      const bool same4 = ok[0] && ok[1] && ok[2] && ok[3] && d[1] == d[0] && d[2] == d[0] && d[3] == d[0];
      const uint32_t dw = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(d[0])));
      if (__ballot(!(same4 && d[0] == dw)) == 0) {
        if (lane == 0) atomicAdd(&s_cnt[w][dw], 4u * kWave);
      } else if (same4) {
        atomicAdd(&s_cnt[w][d[0]], 4u);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (ok[q]) atomicAdd(&s_cnt[w][d[q]], 1u);
      }
    }
  }
  __syncthreads();
  for (int d = threadIdx.x; d < ndig; d += kBlock) {
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) c += s_cnt[q][d];
    hist[static_cast<int64_t>(d) * nblk + blockIdx.x] = c;
  }
}

// per digit (one workgroup each): exclusive scan of its per-block counts, total to tot[d]
__global__ __launch_bounds__(kBlock) void radix_scan(uint32_t* __restrict__ hist, int nblk,
                                                     uint32_t* __restrict__ tot) {
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  uint32_t* row = hist + static_cast<int64_t>(blockIdx.x) * nblk;
  const int ipt = (nblk + kBlock - 1) / kBlock;
  const int i0 = threadIdx.x * ipt;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    v[q] = (q < ipt && i0 + q < nblk) ? row[i0 + q] : 0u;
    sum += v[q];
  }
  uint32_t total;
  uint32_t run = block_exclusive_sum(sum, s_tmp, &total);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < ipt && i0 + q < nblk) row[i0 + q] = run;
    run += v[q];
  }
  if (threadIdx.x == 0) tot[blockIdx.x] = total;
}

// DIG: digits the LDS counters hold (>= 1 << bits).  With at most 128 the kernel takes 36 KB of
// LDS and is held to 128 registers, so a CU holds 4 workgroups instead of 3 (skewed batch, three
// 7-bit passes: 1.10 -> 1.05 ms).
template <bool BY_TABLE, int DIG>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(DIG <= 128 ? 4 : 1))) void radix_downsweep(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ pin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ pout, int64_t N, const int32_t* __restrict__ n_eff, int64_t seg,
    int shift, int bits, uint32_t drop, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ tot,
    int nblk, int32_t* __restrict__ n_kept, const int32_t* __restrict__ tstart,
    int32_t* __restrict__ tstart_next, const int64_t* __restrict__ meta, int T) {
  // drop: keys equal to it are left out (not ranked, not written); the keys kept, over all
  // blocks, go to *n_kept (block 0), the count every later kernel reads
  __shared__ uint32_t s_base[DIG];
  __shared__ uint32_t s_wcnt[kWavesPerBlock][DIG];
  __shared__ uint32_t s_toff[DIG];
  __shared__ uint32_t s_tcnt[DIG];
  __shared__ uint32_t s_key[kRadixTile];
  __shared__ uint32_t s_pay[kRadixTile];
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  __shared__ uint32_t s_kept;  // keys of the current tile that are kept
  __shared__ int32_t s_rng[5];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int ndig = 1 << bits;
  const uint32_t mask = static_cast<uint32_t>(ndig - 1);
  int64_t lo, hi;
  uint32_t rb = 0;  // the row base subtracted before the digit is taken
  const int d0 = 2 * threadIdx.x, d1 = d0 + 1;
  if constexpr (BY_TABLE) {
    if (threadIdx.x == 0) {
      const TableRange r = table_range(tstart, T, nblk, blockIdx.x);
      s_rng[0] = r.t;
      s_rng[1] = r.first;
      s_rng[2] = r.last;
      s_rng[3] = r.lo;
      s_rng[4] = r.hi;
    }
    __syncthreads();
    const int t = s_rng[0], first = s_rng[1], last = s_rng[2];
    rb = static_cast<uint32_t>(meta[4 * t]);
    lo = s_rng[3];
    hi = s_rng[4];
    // hist[d][b] holds the keys of digit d in the blocks before b (all tables), tot[d] all of
    // them.  The table's keys start after the earlier tables' keys, the sum over digits of the
    // prefix at its first block; its digit d after its keys of smaller digits; this block's
    // after the table's earlier blocks' keys of digit d.
    auto col = [&](int d, int b) -> uint32_t {
      return d < ndig ? (b < nblk ? hist[static_cast<int64_t>(d) * nblk + b] : tot[d]) : 0u;
    };
    const uint32_t a0 = col(d0, first), a1 = col(d1, first);
    const uint32_t c0 = col(d0, last) - a0, c1 = col(d1, last) - a1;  // the table's keys per digit
    const uint32_t o0 = col(d0, blockIdx.x) - a0, o1 = col(d1, blockIdx.x) - a1;
    const uint32_t t0 = d0 < ndig ? tot[d0] : 0u, t1 = d1 < ndig ? tot[d1] : 0u;
    const uint32_t start_out = block_sum(a0 + a1, s_tmp);
    const uint32_t all = block_sum(t0 + t1, s_tmp);
    const uint32_t ex = block_exclusive_sum(c0 + c1, s_tmp, nullptr);
    if (d0 < ndig) s_base[d0] = start_out + ex + o0;
    if (d1 < ndig) s_base[d1] = start_out + ex + c0 + o1;
    if (threadIdx.x == 0) {
      if (static_cast<int>(blockIdx.x) == first) tstart_next[t] = static_cast<int32_t>(start_out);
      if (blockIdx.x == 0) {
        tstart_next[T] = static_cast<int32_t>(all);
        if (n_kept) *n_kept = static_cast<int32_t>(all);
      }
    }
  } else {
    if (n_eff) N = min(N, static_cast<int64_t>(*n_eff));
    // global base of each digit for this block: digits below + earlier blocks
    const uint32_t a = d0 < ndig ? tot[d0] : 0u, b = d1 < ndig ? tot[d1] : 0u;
    uint32_t all;
    const uint32_t ex = block_exclusive_sum(a + b, s_tmp, &all);
    if (d0 < ndig) s_base[d0] = ex + hist[static_cast<int64_t>(d0) * nblk + blockIdx.x];
    if (d1 < ndig) s_base[d1] = ex + a + hist[static_cast<int64_t>(d1) * nblk + blockIdx.x];
    if (n_kept && blockIdx.x == 0 && threadIdx.x == 0) *n_kept = static_cast<int32_t>(all);
    lo = blockIdx.x * seg;
    hi = min(lo + seg, N);
  }
  __syncthreads();
  for (int64_t tile = lo; tile < hi; tile += kRadixTile) {
    for (int i = lane; i < ndig; i += kWave) s_wcnt[w][i] = 0;
    uint32_t k[kRadixItems], p[kRadixItems], r[kRadixItems];
    const int64_t wbase = tile + w * (kRadixItems * kWave);
#pragma unroll
    for (int s = 0; s < kRadixItems; ++s) {
      const int64_t i = wbase + s * kWave + lane;
      const bool valid = i < hi;
      k[s] = valid ? kin[i] : 0u;
      p[s] = valid ? pin[i] : 0u;
    }
    __builtin_amdgcn_wave_barrier();
    // Stable rank of each key among the wave's keys of its digit: the lowest lane of
    // each group of equal digits adds the group size to the wave's digit counter
    // with one LDS atomic that returns the count before it (a wave's LDS operations
    // execute in order, so the 8 atomics of a half need no wait in between), then
    // every lane adds the returned base, read from its group's lowest lane, to its
    // place in the group.  r packs the place (bits 0-7) and the lowest lane (bits
    // 8-15).  Two halves of 8 items keep 8 returned bases live instead of 16.
#pragma unroll
    for (int h = 0; h < kRadixItems; h += kRadixItems / 2) {
      uint32_t base[kRadixItems / 2];
#pragma unroll
      for (int q = 0; q < kRadixItems / 2; ++q) {
        const int s = h + q;
        const bool valid = wbase + s * kWave + lane < hi && k[s] != drop;
        const uint32_t d = ((k[s] - rb) >> shift) & mask;
        const uint64_t peers = match_digit(d, bits, __ballot(valid));
        const int lead = __ffsll(static_cast<long long>(peers)) - 1;
        base[q] = 0u;
        if (valid && lane == lead) base[q] = atomicAdd(&s_wcnt[w][d], static_cast<uint32_t>(__popcll(peers)));
        r[s] = static_cast<uint32_t>(__popcll(peers & lanemask_lt())) | (static_cast<uint32_t>(lead & 63) << 8);
      }
#pragma unroll
      for (int q = 0; q < kRadixItems / 2; ++q) {
        const int s = h + q;
        r[s] = (r[s] & 0xffu) + static_cast<uint32_t>(__shfl(static_cast<int>(base[q]), static_cast<int>(r[s] >> 8)));
      }
    }
    __builtin_amdgcn_wave_barrier();
    __syncthreads();
    for (int d = threadIdx.x; d < ndig; d += kBlock) {
      const uint32_t c0 = s_wcnt[0][d], c1 = s_wcnt[1][d], c2 = s_wcnt[2][d], c3 = s_wcnt[3][d];
      s_wcnt[0][d] = 0;
      s_wcnt[1][d] = c0;
      s_wcnt[2][d] = c0 + c1;
      s_wcnt[3][d] = c0 + c1 + c2;
      s_tcnt[d] = c0 + c1 + c2 + c3;
    }
    __syncthreads();
    {
      const int d0 = 2 * threadIdx.x, d1 = d0 + 1;
      const uint32_t a = d0 < ndig ? s_tcnt[d0] : 0u, b = d1 < ndig ? s_tcnt[d1] : 0u;
      uint32_t kept;
      const uint32_t ex = block_exclusive_sum(a + b, s_tmp, &kept);
      if (d0 < ndig) s_toff[d0] = ex;
      if (d1 < ndig) s_toff[d1] = ex + a;
      if (threadIdx.x == 0) s_kept = kept;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kRadixItems; ++s) {
      if (wbase + s * kWave + lane < hi && k[s] != drop) {
        const uint32_t d = ((k[s] - rb) >> shift) & mask;
        const uint32_t pos = s_toff[d] + s_wcnt[w][d] + r[s];
        s_key[pos] = k[s];
        s_pay[pos] = p[s];
      }
    }
    __syncthreads();
    const int kn = static_cast<int>(s_kept);  // the tile's keys, less those dropped
    for (int j = threadIdx.x; j < kn; j += kBlock) {
      const uint32_t key = s_key[j];
      const uint32_t d = ((key - rb) >> shift) & mask;
      const uint32_t g = s_base[d] + (static_cast<uint32_t>(j) - s_toff[d]);
      kout[g] = key;
      pout[g] = s_pay[j];
    }
    __syncthreads();
    for (int d = threadIdx.x; d < ndig; d += kBlock) s_base[d] += s_tcnt[d];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// run-length encoding
// ---------------------------------------------------------------------------
constexpr int kRleItems = 4;

__global__ __launch_bounds__(kBlock) void rle_count(const uint32_t* __restrict__ keys, int64_t N,
                                                    const int32_t* __restrict__ n_eff,
                                                    int64_t seg, uint32_t* __restrict__ cnt) {
  if (n_eff) N = min(N, static_cast<int64_t>(*n_eff));
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  const int64_t lo = blockIdx.x * seg, hi = min(lo + seg, N);
  uint32_t c = 0;
  // four keys (and their predecessors) in flight per thread
  for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += 4 * kBlock) {
    uint32_t k[4], pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q * kBlock;
      k[q] = i < hi ? keys[i] : 0u;
      pk[q] = (i < hi && i > 0) ? keys[i - 1] : ~0u;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q * kBlock;
      c += (i < hi && (i == 0 || k[q] != pk[q])) ? 1u : 0u;
    }
  }
  c = block_sum(c, s_tmp);
  if (threadIdx.x == 0) cnt[blockIdx.x] = c;
}

// exclusive scan of the per-block head counts (one workgroup); run count to counters
__global__ __launch_bounds__(kBlock) void rle_scan(uint32_t* __restrict__ cnt, int nblk,
                                                   int32_t* __restrict__ counters,
                                                   uint32_t* __restrict__ run_start, int64_t N,
                                                   const int32_t* __restrict__ n_eff) {
  if (n_eff) N = min(N, static_cast<int64_t>(*n_eff));
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  const int ipt = (nblk + kBlock - 1) / kBlock;
  const int i0 = threadIdx.x * ipt;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    v[q] = (q < ipt && i0 + q < nblk) ? cnt[i0 + q] : 0u;
    sum += v[q];
  }
  uint32_t total;
  uint32_t run = block_exclusive_sum(sum, s_tmp, &total);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < ipt && i0 + q < nblk) cnt[i0 + q] = run;
    run += v[q];
  }
  if (threadIdx.x == 0) {
    counters[kRuns] = static_cast<int32_t>(total);
    run_start[total] = static_cast<uint32_t>(N);
  }
}

__global__ __launch_bounds__(kBlock) void rle_write(const uint32_t* __restrict__ keys, int64_t N,
                                                    const int32_t* __restrict__ n_eff,
                                                    int64_t seg, const uint32_t* __restrict__ cnt,
                                                    uint32_t* __restrict__ run_key,
                                                    uint32_t* __restrict__ run_start) {
  if (n_eff) N = min(N, static_cast<int64_t>(*n_eff));
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  __shared__ uint32_t s_base;
  const int64_t lo = blockIdx.x * seg, hi = min(lo + seg, N);
  if (threadIdx.x == 0) s_base = cnt[blockIdx.x];
  __syncthreads();
  for (int64_t tile = lo; tile < hi; tile += kBlock * kRleItems) {
    const int64_t i0 = tile + threadIdx.x * kRleItems;
    uint32_t k[kRleItems];
    bool head[kRleItems];
    uint32_t c = 0;
    uint32_t prev = (i0 > 0 && i0 < hi) ? keys[i0 - 1] : 0u;
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
      const int64_t i = i0 + q;
      k[q] = i < hi ? keys[i] : 0u;
      head[q] = i < hi && (i == 0 || k[q] != prev);
      prev = k[q];
      c += head[q] ? 1u : 0u;
    }
    uint32_t total;
    uint32_t r = s_base + block_exclusive_sum(c, s_tmp, &total);
#pragma unroll
    for (int q = 0; q < kRleItems; ++q) {
      if (head[q]) {
        run_key[r] = k[q];
        run_start[r] = static_cast<uint32_t>(i0 + q);
        ++r;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) s_base += total;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// classification: long runs (with chunk plan) and short runs per D bucket
// ---------------------------------------------------------------------------
// Three passes over the runs, with no atomics on global memory: per-block counts
// of every category, an exclusive scan of those counts across blocks, then an
// ordered write.  The lists come out in run (= key) order, so runs of one table
// stay together, and the result is the same on every run.  The block segments
// are derived on the device from the run count.
constexpr int kLdsTables = 2048;

// row bases and widths of the tables in dynamic LDS (sized for T at launch: a few hundred
// bytes for tens of tables, so LDS does not limit the workgroups a CU holds)
struct TableLds {
  int64_t* rb;  // [T + 1]
  int32_t* D;   // [T]
};
inline size_t table_lds_bytes(int T) {
  return T <= kLdsTables ? static_cast<size_t>(T + 1) * 8 + static_cast<size_t>(T) * 4 : 0;
}

__device__ __forceinline__ TableLds load_tables(const int64_t* __restrict__ meta, int T) {
  extern __shared__ __align__(8) char s_dyn[];
  TableLds s{reinterpret_cast<int64_t*>(s_dyn), reinterpret_cast<int32_t*>(s_dyn + static_cast<size_t>(T + 1) * 8)};
  if (T <= kLdsTables)
    for (int t = threadIdx.x; t <= T; t += kBlock) {
      s.rb[t] = meta[4 * t];
      if (t < T) s.D[t] = static_cast<int32_t>(meta[4 * t + 3]);
    }
  __syncthreads();
  return s;
}

__device__ __forceinline__ int lds_table_of_key(const TableLds& s, const int64_t* __restrict__ meta, int T,
                                                uint32_t key, int& D) {
  if (T > kLdsTables) {
    const int t = table_of_key(meta, T, key);
    D = static_cast<int>(meta[4 * t + 3]);
    return t;
  }
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.rb[mid] <= static_cast<int64_t>(key)) lo = mid; else hi = mid - 1;
  }
  D = s.D[lo];
  return lo;
}

__device__ __forceinline__ void block_segment(int64_t n, int64_t& lo, int64_t& hi) {
  int64_t seg = (n + gridDim.x - 1) / gridDim.x;
  seg = (seg + kBlock - 1) / kBlock * kBlock;
  lo = min(n, static_cast<int64_t>(blockIdx.x) * seg);
  hi = min(n, lo + seg);
}

// category of a run (-1: ids outside their table, dropped) and its chunk count
__device__ __forceinline__ int run_category(const TableLds& s, const int64_t* __restrict__ meta, int T,
                                            uint32_t total_rows, int threshold, int chunk, uint32_t key,
                                            uint32_t len, int& t, uint32_t& nch) {
  nch = 0;
  t = 0;
  if (key >= total_rows) return -1;
  int D;
  t = lds_table_of_key(s, meta, T, key, D);
  if (len >= static_cast<uint32_t>(threshold)) {
    nch = (len + chunk - 1) / chunk;
    return 0;
  }
  return 1 + bucket_of_D(D);
}

// one_bucket >= 0: every table's short runs fall in that bucket, so a run's category follows
// from its key's validity and its length alone (no table search).  Each wave adds its
// counts with one LDS atomic per category (a lane per run would serialize on one address).
__global__ __launch_bounds__(kBlock) void classify_count(
    const uint32_t* __restrict__ run_key, const uint32_t* __restrict__ run_start,
    const int32_t* __restrict__ counters, const int64_t* __restrict__ meta, int T,
    uint32_t total_rows, int threshold, int chunk, int one_bucket, uint32_t* __restrict__ cls_cnt) {
  __shared__ uint32_t s_cnt[kClsRows];
  if (threadIdx.x < kClsRows) s_cnt[threadIdx.x] = 0;
  const TableLds s_tab = load_tables(meta, T);
  const int lane = lane_id();
  int64_t lo, hi;
  block_segment(counters[kRuns], lo, hi);
  for (int64_t tile = lo; tile < hi; tile += kBlock) {  // uniform trip count (ballots below)
    const int64_t r = tile + threadIdx.x;
    int cat = -1;
    uint32_t nch = 0;
    if (r < hi) {
      const uint32_t key = run_key[r];
      const uint32_t len = run_start[r + 1] - run_start[r];
      if (one_bucket >= 0) {
        if (key < total_rows) {
          const bool lng = len >= static_cast<uint32_t>(threshold);
          cat = lng ? 0 : 1 + one_bucket;
          nch = lng ? (len + chunk - 1) / chunk : 0u;
        }
      } else {
        int t;
        cat = run_category(s_tab, meta, T, total_rows, threshold, chunk, key, len, t, nch);
      }
    }
#pragma unroll
    for (int c = 0; c < kCats; ++c) {
      const uint64_t m = __ballot(cat == c);
      if (lane == 0 && m) atomicAdd(&s_cnt[c], static_cast<uint32_t>(__popcll(m)));
    }
    for (int d = 1; d < kWave; d <<= 1) nch += __shfl_xor(nch, d);
    if (lane == 0 && nch) atomicAdd(&s_cnt[kCats], nch);
  }
  __syncthreads();
  if (threadIdx.x < kClsRows) cls_cnt[threadIdx.x * gridDim.x + blockIdx.x] = s_cnt[threadIdx.x];
}

// one workgroup per category row: exclusive scan over blocks, total into counters
__global__ __launch_bounds__(kBlock) void classify_scan(uint32_t* __restrict__ cls_cnt, int nblk,
                                                        int32_t* __restrict__ counters) {
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  uint32_t* row = cls_cnt + static_cast<int64_t>(blockIdx.x) * nblk;
  const int ipt = (nblk + kBlock - 1) / kBlock;
  const int i0 = threadIdx.x * ipt;
  uint32_t v[16];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    v[q] = (q < ipt && i0 + q < nblk) ? row[i0 + q] : 0u;
    sum += v[q];
  }
  uint32_t total;
  uint32_t run = block_exclusive_sum(sum, s_tmp, &total);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < ipt && i0 + q < nblk) row[i0 + q] = run;
    run += v[q];
  }
  if (threadIdx.x == 0) {
    const int c = blockIdx.x;
    const int dst = c == 0 ? kLong : (c == kCats ? kChunks : kShort0 + c - 1);
    counters[dst] = static_cast<int32_t>(total);
  }
}

__global__ __launch_bounds__(kBlock) void classify_write(
    const uint32_t* __restrict__ run_key, const uint32_t* __restrict__ run_start,
    const int32_t* __restrict__ counters, const int64_t* __restrict__ meta, int T,
    uint32_t total_rows, int threshold, int chunk, const uint32_t* __restrict__ cls_cnt,
    uint4* __restrict__ long_list, uint32_t* __restrict__ long_table, uint32_t* __restrict__ long_count,
    uint2* __restrict__ chunk_list, int64_t cap_long, int64_t cap_chunk, ShortLists lists) {
  __shared__ uint32_t s_base[kClsRows];
  __shared__ uint32_t s_wcnt[kWavesPerBlock][kCats];
  __shared__ uint32_t s_tmp[kWavesPerBlock];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  if (threadIdx.x < kClsRows) s_base[threadIdx.x] = cls_cnt[threadIdx.x * gridDim.x + blockIdx.x];
  const TableLds s_tab = load_tables(meta, T);
  int64_t lo, hi;
  block_segment(counters[kRuns], lo, hi);
  for (int64_t tile = lo; tile < hi; tile += kBlock) {
    const int64_t r = tile + threadIdx.x;
    int cat = -1, t = 0;
    uint32_t key = 0, start = 0, len = 0, nch = 0;
    if (r < hi) {
      key = run_key[r];
      start = run_start[r];
      len = run_start[r + 1] - start;
      cat = run_category(s_tab, meta, T, total_rows, threshold, chunk, key, len, t, nch);
    }
    uint32_t wrank = 0;
#pragma unroll
    for (int c = 0; c < kCats; ++c) {
      const uint64_t m = __ballot(cat == c);
      if (cat == c) wrank = __popcll(m & lanemask_lt());
      if (lane == 0) s_wcnt[w][c] = __popcll(m);
    }
    uint32_t ch_total;
    const uint32_t ch_off = block_exclusive_sum(nch, s_tmp, &ch_total);  // synchronizes
    if (cat >= 0) {
      uint32_t pre = s_base[cat];
      for (int k = 0; k < w; ++k) pre += s_wcnt[k][cat];
      const int64_t slot = static_cast<int64_t>(pre) + wrank;
      if (cat == 0) {
        const int64_t cb = static_cast<int64_t>(s_base[kCats]) + ch_off;
        if (slot < cap_long) {
          long_list[slot] = make_uint4(key, start, len, static_cast<uint32_t>(cb));
          long_table[slot] = static_cast<uint32_t>(t);
          long_count[slot] = nch;  // countdown of the fused long-run kernel
          for (uint32_t c = 0; c < nch; ++c)
            if (cb + c < cap_chunk) chunk_list[cb + c] = make_uint2(static_cast<uint32_t>(slot), c);
        }
      } else if (slot < lists.cap[cat - 1]) {
        lists.p[cat - 1][slot] = make_uint4(key, start, len, static_cast<uint32_t>(t));
      }
    }
    __syncthreads();
    if (threadIdx.x < kCats) {
      uint32_t add = 0;
      for (int k = 0; k < kWavesPerBlock; ++k) add += s_wcnt[k][threadIdx.x];
      s_base[threadIdx.x] += add;
    }
    if (threadIdx.x == kCats) s_base[kCats] += ch_total;
    __syncthreads();
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// the dense-row key set linearize consults (NULL set: none)
struct HotSet {
  const uint32_t* filter;
  const uint32_t* set;
  uint32_t mask;
  const int32_t* probes;
  uint16_t* slot;  // per position: its dense slot (rank and bag modulo 16), or kNoDenseSlot
};

template <typename IT, typename OT>
tbe_status linearize_go(const tbe_tables* tb, const IndexArgs& ia, int weighted, uint32_t* keys,
                        uint32_t* pay, uint32_t* bag_of, int skip_t, int invalid_as_row0,
                        const HotSet& hot, int32_t* n_eff, hipStream_t s) {
  const int64_t nbags = static_cast<int64_t>(tb->T) * tb->B;
  const int64_t groups = (nbags + kWave - 1) / kWave;
  const int64_t work = (groups + kWavesPerBlock - 1) / kWavesPerBlock;
  const uint32_t sentinel = static_cast<uint32_t>(tb->total_rows);
  // one workgroup per four groups of 64 bags, not a grid sized to the CUs: a slot that frees up
  // takes the next workgroup, and in the hoisted forward the pooling's workgroups and these
  // share the CUs as they come (skewed 0.52 -> 0.50 ms; hoisted step 9.25 -> 9.22 ms)
  ProfScope ps("linearize", s);
  if (weighted)
    hipLaunchKernelGGL((linearize_kernel<IT, OT, true>), dim3(static_cast<int>(hmax(1, hmin(work, int64_t{1} << 30)))),
                       dim3(kBlock), 0, s,
                       static_cast<const IT*>(ia.indices), static_cast<const OT*>(ia.offsets), tb->meta,
                       tb->B, nbags, static_cast<int32_t>(ia.N), sentinel, skip_t, invalid_as_row0, hot.filter,
                       hot.set, hot.mask, hot.probes, hot.slot, keys, pay, bag_of, n_eff);
  else
    hipLaunchKernelGGL((linearize_kernel<IT, OT, false>), dim3(static_cast<int>(hmax(1, hmin(work, int64_t{1} << 30)))),
                       dim3(kBlock), 0, s,
                       static_cast<const IT*>(ia.indices), static_cast<const OT*>(ia.offsets), tb->meta,
                       tb->B, nbags, static_cast<int32_t>(ia.N), sentinel, skip_t, invalid_as_row0, hot.filter,
                       hot.set, hot.mask, hot.probes, hot.slot, keys, pay, bag_of, n_eff);
  return check_launch("linearize");
}

// Radix sort of the plan's keys[0] (with payloads) over `passes` passes, run-length encoding
// and classification.  Keys equal to `drop` (the sentinel) are left out by the first pass;
// n_in != NULL bounds the keys read (the count linearize leaves).  A run of at least
// `threshold` lookups is long; short runs go to `lists` (capacity 0: not written).
// names: the profiling names of the five phases.
struct RouteNames {
  const char *up, *scan, *down, *rle, *cls;
};
constexpr RouteNames kMainNames = {"radix_upsweep", "radix_scan", "radix_downsweep", "rle", "classify"};
constexpr RouteNames kQuietNames = {"-", "-", "-", "-", "-"};

// R.by_table: tstart holds the first pass's table starts (table_starts_kernel) and room for
// the next pass's
tbe_status sort_route(const tbe_tables* tb, char* ws, const SortPlan& P, const RadixPlan& R, int32_t* tstart,
                      const int32_t* n_in, uint32_t drop, int threshold, int chunk, const ShortLists& lists,
                      const RouteNames& nm, int* final_buf, hipStream_t s) {
  const int64_t N = P.N;
  int32_t* counters = reinterpret_cast<int32_t*>(ws + P.counters);
  uint32_t* keys[2] = {reinterpret_cast<uint32_t*>(ws + P.keys[0]), reinterpret_cast<uint32_t*>(ws + P.keys[1])};
  uint32_t* pay[2] = {reinterpret_cast<uint32_t*>(ws + P.pay[0]), reinterpret_cast<uint32_t*>(ws + P.pay[1])};
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + P.sort_hist);
  uint32_t* tot = hist + static_cast<int64_t>(kRadixDigits) * P.nblocks;
  int32_t* n_sorted = counters + kSorted;
  tbe_status st;
  int cur = 0;
  const int T = tb->T;
  for (int pass = 0; pass < R.passes; ++pass) {
    const int ndig = 1 << R.bits[pass];
    const int32_t* n_p = pass == 0 ? n_in : n_sorted;
    const uint32_t d = pass == 0 ? drop : ~0u;
    // by table: this pass's table starts, and where the next pass's go
    const int32_t* ts_in = R.by_table ? tstart + (pass & 1) * (T + 1) : nullptr;
    int32_t* ts_out = R.by_table ? tstart + ((pass + 1) & 1) * (T + 1) : nullptr;
    {
      ProfScope ps(nm.up, s);
      if (R.by_table)
        hipLaunchKernelGGL(radix_upsweep<true>, dim3(P.nblocks), dim3(kBlock), 0, s, keys[cur], N, n_p, P.seg,
                           R.shift[pass], R.bits[pass], d, hist, P.nblocks, ts_in, tb->meta, T);
      else
        hipLaunchKernelGGL(radix_upsweep<false>, dim3(P.nblocks), dim3(kBlock), 0, s, keys[cur], N, n_p, P.seg,
                           R.shift[pass], R.bits[pass], d, hist, P.nblocks, ts_in, tb->meta, T);
    }
    if ((st = check_launch("radix_upsweep"))) return st;
    {
      ProfScope ps(nm.scan, s);
      hipLaunchKernelGGL(radix_scan, dim3(ndig), dim3(kBlock), 0, s, hist, P.nblocks, tot);
    }
    if ((st = check_launch("radix_scan"))) return st;
    {
      ProfScope ps(nm.down, s);
#define TBE_DOWN(BT, DG)                                                                             \
  hipLaunchKernelGGL((radix_downsweep<BT, DG>), dim3(P.nblocks), dim3(kBlock), 0, s, keys[cur], pay[cur], \
                     keys[cur ^ 1], pay[cur ^ 1], N, n_p, P.seg, R.shift[pass], R.bits[pass], d, hist, tot, \
                     P.nblocks, pass == 0 ? n_sorted : nullptr, ts_in, ts_out, tb->meta, T)
      if (R.by_table) {
        if (ndig <= 128) TBE_DOWN(true, 128);
        else TBE_DOWN(true, kRadixDigits);
      } else {
        if (ndig <= 128) TBE_DOWN(false, 128);
        else TBE_DOWN(false, kRadixDigits);
      }
#undef TBE_DOWN
    }
    if ((st = check_launch("radix_downsweep"))) return st;
    cur ^= 1;
  }
  *final_buf = cur;
  uint32_t* run_key = reinterpret_cast<uint32_t*>(ws + P.run_key);
  uint32_t* run_start = reinterpret_cast<uint32_t*>(ws + P.run_start);
  uint32_t* seg_cnt = reinterpret_cast<uint32_t*>(ws + P.seg_cnt);
  {
    ProfScope ps(nm.rle, s);
    hipLaunchKernelGGL(rle_count, dim3(P.nblocks), dim3(kBlock), 0, s, keys[cur], N, n_sorted, P.seg, seg_cnt);
    hipLaunchKernelGGL(rle_scan, dim3(1), dim3(kBlock), 0, s, seg_cnt, P.nblocks, counters, run_start, N, n_sorted);
    hipLaunchKernelGGL(rle_write, dim3(P.nblocks), dim3(kBlock), 0, s, keys[cur], N, n_sorted, P.seg, seg_cnt,
                       run_key, run_start);
  }
  if ((st = check_launch("rle"))) return st;
  {
    uint32_t* cls_cnt = reinterpret_cast<uint32_t*>(ws + P.cls_cnt);
    const uint32_t total_rows = static_cast<uint32_t>(tb->total_rows);
    ProfScope ps(nm.cls, s);
    const size_t lds = table_lds_bytes(tb->T);
    int one_bucket = -1;  // the only short-run bucket any table falls in, if there is one
    for (int b = 0; b < TBE_NUM_BUCKETS; ++b)
      if (tb->bucket_rows[b] > 0) one_bucket = one_bucket == -1 ? b : -2;
    hipLaunchKernelGGL(classify_count, dim3(P.cls_blocks), dim3(kBlock), lds, s, run_key, run_start,
                       counters, tb->meta, tb->T, total_rows, threshold, chunk, one_bucket < 0 ? -1 : one_bucket,
                       cls_cnt);
    hipLaunchKernelGGL(classify_scan, dim3(kClsRows), dim3(kBlock), 0, s, cls_cnt, P.cls_blocks, counters);
    hipLaunchKernelGGL(classify_write, dim3(P.cls_blocks), dim3(kBlock), lds, s, run_key, run_start,
                       counters, tb->meta, tb->T, total_rows, threshold, chunk, cls_cnt,
                       reinterpret_cast<uint4*>(ws + P.long_list), reinterpret_cast<uint32_t*>(ws + P.long_table),
                       reinterpret_cast<uint32_t*>(ws + P.long_count),
                       P.cap_chunk ? reinterpret_cast<uint2*>(ws + P.chunk_list) : nullptr, P.cap_long,
                       P.cap_chunk, lists);
  }
  return check_launch("classify");
}

}  // namespace

tbe_status launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return TBE_OK;
  ProfScope ps("init", s);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return check_launch("init");
}

tbe_status launch_transpose(const tbe_tables* tb, const IndexArgs& ia, int weighted, char* ws,
                            const BwdLayout& L, const Config& cfg, int skip_table,
                            int invalid_as_row0, int dense, int* final_buf, hipStream_t s) {
  int32_t* counters = reinterpret_cast<int32_t*>(ws + L.counters);
  if (tbe_status st = launch_fill_i32(counters, 0, kNumCounters, s)) return st;
  const int64_t N = L.N;
  *final_buf = 0;
  // without the dense rows (or with no lookups) no table has any: a backward that takes these
  // runs as they are leaves every row to them
  if (L.dense_on && L.dense_presort && (!dense || N == 0))
    if (tbe_status st = launch_fill_i32(reinterpret_cast<int32_t*>(ws + L.dense_cnt), 0, tb->T, s)) return st;
  dense = dense && L.dense_on && L.dense_presort;
  if (N == 0) {
    uint32_t* rs = reinterpret_cast<uint32_t*>(ws + L.run_start);
    return launch_fill_i32(reinterpret_cast<int32_t*>(rs), 0, 1, s);
  }
  // with a skipped table the sort covers only the other tables' lookups, a count
  // known on the device once linearize has run
  if (skip_table >= 0 && weighted) {
    set_error("a table can be left out of the runs only without per-sample weights");
    return TBE_ERR_ARG;
  }
  const uint32_t sentinel = static_cast<uint32_t>(tb->total_rows);
  tbe_status st;
  // the dense rows, picked from a sample of the lookups before the sort
  HotSet hot{nullptr, nullptr, 0u, nullptr, nullptr};
  if (dense) {
    ProfScope ps("dense_sample", s);
    const SortPlan& P = L.sample;
    if ((st = launch_fill_i32(reinterpret_cast<int32_t*>(ws + P.counters), 0, kNumCounters, s))) return st;
    if ((st = launch_fill_i32(reinterpret_cast<int32_t*>(ws + L.hot_set), -1, L.hot_set_size, s))) return st;
    if ((st = launch_fill_i32(reinterpret_cast<int32_t*>(ws + L.hot_bloom), 0, kHotBloomWords, s))) return st;
    if ((st = launch_dense_sample(tb, ia, skip_table, invalid_as_row0, ws, L, s))) return st;
    ShortLists none;
    for (int b = 0; b < TBE_NUM_BUCKETS; ++b) {
      none.p[b] = nullptr;
      none.cap[b] = 0;
    }
    int fb;
    if ((st = sort_route(tb, ws, P, L.sample_radix, nullptr, nullptr, sentinel, L.hot_thr, 1 << 30, none,
                         kQuietNames, &fb, s)))
      return st;
    if ((st = launch_dense_select(tb, ws, L, skip_table, s))) return st;
    hot = HotSet{reinterpret_cast<const uint32_t*>(ws + L.hot_bloom),
                 reinterpret_cast<const uint32_t*>(ws + L.hot_set),
                 static_cast<uint32_t>(L.hot_set_size - 1), counters + kHotProbe,
                 reinterpret_cast<uint16_t*>(ws + L.dense_slot)};
  }
  uint32_t* keys0 = reinterpret_cast<uint32_t*>(ws + L.keys[0]);
  uint32_t* pay0 = reinterpret_cast<uint32_t*>(ws + L.pay[0]);
  uint32_t* bag_of = weighted ? reinterpret_cast<uint32_t*>(ws + L.bag_of) : nullptr;
  int32_t* n_eff = skip_table >= 0 ? counters + kNeff : nullptr;
  if (ia.itype == TBE_I32)
    st = ia.otype == TBE_I32 ? linearize_go<int32_t, int32_t>(tb, ia, weighted, keys0, pay0, bag_of, skip_table, invalid_as_row0, hot, n_eff, s)
                             : linearize_go<int32_t, int64_t>(tb, ia, weighted, keys0, pay0, bag_of, skip_table, invalid_as_row0, hot, n_eff, s);
  else
    st = ia.otype == TBE_I32 ? linearize_go<int64_t, int32_t>(tb, ia, weighted, keys0, pay0, bag_of, skip_table, invalid_as_row0, hot, n_eff, s)
                             : linearize_go<int64_t, int64_t>(tb, ia, weighted, keys0, pay0, bag_of, skip_table, invalid_as_row0, hot, n_eff, s);
  if (st) return st;
  // the first pass leaves out the sentinel keys (ids outside their table, lookups the dense
  // rows take, positions no bag covers): later kernels see only the kept keys
  SortPlan M;
  M.N = N;
  for (int i = 0; i < 2; ++i) {
    M.keys[i] = L.keys[i];
    M.pay[i] = L.pay[i];
  }
  M.run_key = L.run_key;
  M.run_start = L.run_start;
  M.sort_hist = L.sort_hist;
  M.seg_cnt = L.seg_cnt;
  M.cls_cnt = L.cls_cnt;
  M.counters = L.counters;
  M.long_list = L.long_list;
  M.long_table = L.long_table;
  M.long_count = L.long_count;
  M.chunk_list = L.chunk_list;
  M.cap_long = L.cap_long;
  M.cap_chunk = L.cap_chunk;
  M.seg = L.seg;
  M.nblocks = L.nblocks;
  M.cls_blocks = L.cls_blocks;
  ShortLists lists;
  for (int b = 0; b < TBE_NUM_BUCKETS; ++b) {
    lists.p[b] = L.cap_short[b] ? reinterpret_cast<uint4*>(ws + L.short_list[b]) : nullptr;
    lists.cap[b] = L.cap_short[b];
  }
  int32_t* tstart = nullptr;
  if (L.radix.by_table) {
    // each table's first key in linearize's output
    tstart = reinterpret_cast<int32_t*>(ws + L.tstart);
    ProfScope ps("table_starts", s);
    if (ia.otype == TBE_I32)
      hipLaunchKernelGGL(table_starts_kernel<int32_t>, dim3(1), dim3(kBlock), 0, s,
                         static_cast<const int32_t*>(ia.offsets), tb->T, tb->B, static_cast<int32_t>(N),
                         skip_table, tstart);
    else
      hipLaunchKernelGGL(table_starts_kernel<int64_t>, dim3(1), dim3(kBlock), 0, s,
                         static_cast<const int64_t*>(ia.offsets), tb->T, tb->B, static_cast<int32_t>(N),
                         skip_table, tstart);
    if ((st = check_launch("table_starts"))) return st;
  }
  return sort_route(tb, ws, M, L.radix, tstart, n_eff, sentinel, cfg.threshold, cfg.chunk, lists, kMainNames,
                    final_buf, s);
}

}  // namespace tbe
