// Host-side internals shared by the TBE translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tbe.h"
#include "../../include/tbe_measure.h"

namespace tbe {

// ---------------------------------------------------------------------------
// errors and kernel timing
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
tbe_status check_launch(const char* what);

// Records a pair of events around a launch when the kernel is the one
// selected with tbe_profile_select.
struct ProfScope {
  ProfScope(const char* kernel, hipStream_t s);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};

// ---------------------------------------------------------------------------
// launch geometry
// ---------------------------------------------------------------------------
constexpr int kBlock = 256;            // threads per workgroup in every kernel
constexpr int kWavesPerBlock = kBlock / 64;
int device_cu_count();                 // compute units of the current device (cached)
inline int64_t hmin(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t hmax(int64_t a, int64_t b) { return a > b ? a : b; }
// Workgroups of kBlock threads of `kernel` one CU holds at once (its registers and
// LDS, with dyn_lds bytes of dynamic LDS, decide), queried once per kernel and size.
int blocks_per_cu(const void* kernel, size_t dyn_lds = 0, int threads = kBlock);
// Grid of a grid-stride kernel: every workgroup resident at once (a workgroup that
// has to wait for a free slot would start its whole share late), at most work_blocks.
template <typename K>
int resident_grid(K* kernel, int64_t work_blocks, size_t dyn_lds = 0, int threads = kBlock) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) *
                      blocks_per_cu(reinterpret_cast<const void*>(kernel), dyn_lds, threads);
  return static_cast<int>(hmax(1, hmin(work_blocks, cap)));
}

// MI355X's Infinity Cache (the last level before HBM)
constexpr int64_t kInfinityCacheBytes = int64_t{256} << 20;

// Radix sort geometry (least-significant digit first, up to 9 bits a pass)
constexpr int kRadixMaxBits = 9;
constexpr int kRadixDigits = 1 << kRadixMaxBits;
constexpr int kRadixItems = 16;                       // keys per thread per tile
constexpr int kRadixTile = kBlock * kRadixItems;      // 4096 keys

struct Config {
  int threshold, chunk, hist_enable, fwd_unroll, bwd_unroll, sort_blocks, bag_windows, fused_long;
  int pretransposed, bags_per_wave, bwd_streams;
  int tiny;  // wave steps of short runs of at most this many lookups: half the lanes per run
  int dense_min;  // rows of at least this many lookups (the 128 longest a table) take the dense path (0: off)
  int dense_presort;  // dense rows picked before the sort: 1 always, -1 never, 0 large batches
  int sort_by_table;  // each table's lookups sorted on their own: 1 when possible, -1 never, 0 auto
  int short_reserve;  // set by the backward: the share (in 1/512) of every SIMD's registers the
                     // short-run grid leaves free for a kernel on another stream (0: none)
  int32_t* short_work;  // set by the backward: a zeroed device counter from which the short-run
                        // waves take their work (NULL: each wave takes fixed steps); with the
                        // long runs on a second stream a second short-run grid follows them there
};
Config resolve_config(const tbe_config* c);

// Buffers of one sort + run-length encoding + classification (byte offsets into the workspace)
struct SortPlan {
  int64_t N;                                   // keys at most
  size_t keys[2], pay[2], run_key, run_start, sort_hist, seg_cnt, cls_cnt, counters;
  size_t long_list, long_table, long_count, chunk_list;
  int64_t cap_long, cap_chunk;
  int64_t seg;        // keys per sort / RLE block (multiple of kRadixTile)
  int nblocks;        // sort / RLE blocks
  int cls_blocks;     // classification blocks
};

// Radix passes (least-significant digit first): each pass's digit position and width.
// by_table: each table's keys are sorted on their own, on the bits of the local row id (key -
// the table's row base); the batch keeps a table's lookups together, so the result is the
// order of the linearized ids.
struct RadixPlan {
  int passes;
  int shift[4], bits[4];
  int by_table;
};

// Workspace carve-up of the backward / transpose (byte offsets, 256-aligned)
struct BwdLayout {
  int64_t N;
  size_t keys[2], pay[2], bag_of, run_key, run_start;
  size_t long_list, long_table, long_count, chunk_list, partial, short_list[TBE_NUM_BUCKETS];
  size_t sort_hist, seg_cnt, cls_cnt, counters, total;
  size_t chunk_unit, chunk_order, unit_cnt;  // long-run chunk ordering by (table, bag window)
  size_t hist_partial, hist_count;             // histogram backward: per-block partial sums
  size_t hist_saved;                           // per-bag counts the histogram forward saves (u16)
  // dense hot rows: per table kDenseRows selected row ids and their count, dense_P partials of
  // kDenseRows x 128 floats per table.  With dense_presort the rows are chosen before the sort
  // from a sample of the lookups (64 positions every hot_stride, sorted and run-length encoded
  // on their own: runs of at least hot_thr sampled lookups), and their keys go into an
  // open-addressing set (hot_set: hot_set_size words, 16-byte records of three key slots and
  // their ranks, at most a sixth of the slots used) with a
  // 65536-bit filter, which linearize consults; otherwise they come from the batch's long runs
  // after the sort, with a flag per long-list slot (long_flag) that the chunk and apply
  // kernels read
  // (dense_slot: two bytes per lookup position, its row's rank or none and its bag modulo 16,
  // written by linearize and read by the dense partial kernel instead of the ids)
  size_t dense_rows, dense_cnt, dense_partial, hot_set, hot_bloom, long_flag, dense_slot;
  int dense_P, dense_on, dense_presort, hot_stride, hot_thr;
  int64_t hot_set_size;
  SortPlan sample;
  int nwin, win_size, units;
  int64_t cap_long, cap_chunk, cap_short[TBE_NUM_BUCKETS];
  int64_t seg;        // keys per sort / RLE block (multiple of kRadixTile)
  int nblocks;        // sort / RLE blocks
  int cls_blocks;     // classification blocks
  RadixPlan radix;    // the sort of the batch's keys
  RadixPlan sample_radix;  // the sort of the dense-row sample (always on the linearized ids)
  size_t tstart;      // by-table sort: 2 x (T + 1) int32, each table's start in a pass's input / output
  int key_bits;
  int final_buf;      // key / payload buffer holding the sorted result
};
BwdLayout bwd_layout(const tbe_tables* tb, int64_t N, int weighted, const Config& cfg);

constexpr int kOptSGD = 0;
constexpr int kOptAdagrad = 1;

// kNeff: keys the sort covers when a table is left out of the runs; kSorted: keys kept by the
// first radix pass (sentinel keys left out), the length of the sorted arrays; kHotProbe: the
// longest probe sequence of the dense-row key set
enum Counter { kRuns = 0, kLong = 1, kChunks = 2, kShort0 = 3, kNeff = 12, kSorted = 13, kHotProbe = 14,
               kShortWork = 15, kNumCounters = 16 };
static_assert(kShort0 + TBE_NUM_BUCKETS <= kNeff, "counter slots overlap");

// ---------------------------------------------------------------------------
// launchers (each returns TBE_OK or the launch error)
// ---------------------------------------------------------------------------
struct IndexArgs {
  const void* indices; int itype;
  const void* offsets; int otype;
  int64_t N;
};

tbe_status launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

tbe_status launch_forward_gather(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                                 const float* psw, float* out, int skip_table, int unroll,
                                 int bags_per_wave, int64_t* repair_counts, hipStream_t s);
// repair_counts != NULL: ids outside the table are repaired to 0 in place and counted there;
// save_counts != NULL: each bag's counts (its first 256 ids, 64 u16 a bag) are kept for the
// backward
tbe_status launch_forward_hist(const tbe_tables* tb, const void* W, const IndexArgs& ia,
                               float* out, int64_t* repair_counts, uint16_t* save_counts,
                               hipStream_t s);

tbe_status launch_bounds(const tbe_tables* tb, void* indices, int itype, void* offsets, int otype,
                         int64_t N, int64_t* counts, void* ws, hipStream_t s);
size_t bounds_workspace(const tbe_tables* tb);
tbe_status launch_bounds_offsets(const tbe_tables* tb, void* offsets, int otype, int64_t N,
                                 int64_t* counts, void* ws, hipStream_t s);
tbe_status launch_bounds_indices(const tbe_tables* tb, void* indices, int itype, const void* offsets,
                                 int otype, int64_t N, int64_t* counts, hipStream_t s);

// skip_table >= 0: that table's lookups are left out of the runs (its rows are
// updated by the histogram backward)
// invalid_as_row0: an id outside its table counts as row 0 (the value the bounds
// repair writes) instead of being dropped
// dense (with L.dense_on and L.dense_presort): the dense rows are picked first and their
// lookups are left out of the runs (the backward's transpose; tbe_transpose keeps every
// lookup)
tbe_status launch_transpose(const tbe_tables* tb, const IndexArgs& ia, int weighted,
                            char* ws, const BwdLayout& L, const Config& cfg, int skip_table,
                            int invalid_as_row0, int dense, int* final_buf, hipStream_t s);

// histogram backward of the small table (counts x gradient on MFMA, then the optimizer)
constexpr int kHistBwdBlocks = 512;  // max partials (workgroups) of the histogram backward
// dense hot rows of large tables (counts x gradient on MFMA).  With dense_presort, before the
// sort: the sampled keys (into L.sample's first key buffer), then, from the sample's sorted
// runs, the rows of each table and the key set linearize consults.  The backward updates
// those rows.
constexpr int kDenseRows = 128;  // rows per table at most
constexpr int kHotBloomWords = 2048;  // 65536-bit filter of the dense-row keys
tbe_status launch_dense_sample(const tbe_tables* tb, const IndexArgs& ia, int hist_t, int invalid_as_row0,
                               char* ws, const BwdLayout& L, hipStream_t s);
tbe_status launch_dense_select(const tbe_tables* tb, char* ws, const BwdLayout& L, int hist_t,
                               hipStream_t s);
// the rows from the batch's sorted long runs instead (without dense_presort), flagging their
// long-list slots
tbe_status launch_dense_select_runs(const tbe_tables* tb, char* ws, const BwdLayout& L, int hist_t,
                                    const Config& cfg, hipStream_t s);
// wgs_per_cu > 0: the partial kernel's grid is that many workgroups per CU (else as many as fit);
// psw != NULL: the per-sample weights of the lookups
tbe_status launch_dense_backward(const tbe_tables* tb, void* W, float* momentum, int opt,
                                 const IndexArgs& ia, const float* psw, const float* grad_out, float lr,
                                 float eps, char* ws, const BwdLayout& L, hipStream_t s, int wgs_per_cu = 0);
// workgroups per CU the dense partial kernel holds at once
int dense_partial_blocks_per_cu();

// saved_counts: the counts the histogram forward kept (then only ids past a bag's first 256
// are read), or NULL to count every id
// wgs_per_cu > 0: the partial kernel's grid is at most that many workgroups per CU
tbe_status launch_hist_backward(const tbe_tables* tb, void* W, float* momentum, int opt,
                                const IndexArgs& ia, const float* grad_out, float lr, float eps,
                                char* ws, const BwdLayout& L, const uint16_t* saved_counts,
                                hipStream_t s, int wgs_per_cu = 0);
// workgroups per CU the histogram partial kernel holds at once
int hist_partial_blocks_per_cu();

// groups long-run chunks by (table, bag window); *order = NULL when not grouped
tbe_status launch_chunk_order(const tbe_tables* tb, const float* psw, char* ws, const BwdLayout& L,
                              int final_buf, const Config& cfg, const uint32_t** order, hipStream_t s);

// short runs on s, long runs (chunks, apply) on s_long (s itself, or a fork of it)
tbe_status launch_backward_update(const tbe_tables* tb, void* W, float* momentum, int opt,
                                  const float* psw, const float* grad_out, float lr, float eps,
                                  char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                                  hipStream_t s, hipStream_t s_long);

// A second stream forked from s: work enqueued on side() starts after everything
// enqueued on s before the fork, and join() makes later work on s wait for it.
// One per device, made on first use, default priority; a Fork holds a lock until
// it is joined, so forks of concurrent calls on one device take turns.
class Fork {
 public:
  explicit Fork(hipStream_t s);
  ~Fork();
  tbe_status status() const { return st_; }
  hipStream_t side() const { return side_; }
  tbe_status join();

 private:
  hipStream_t main_, side_ = nullptr;
  void* done_ = nullptr;  // hipEvent_t
  tbe_status st_ = TBE_OK;
  bool joined_ = true;
};

}  // namespace tbe
