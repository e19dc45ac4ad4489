// C ABI of the TBE library: argument validation, workspace layout, dispatch.
// Declarations and the meaning of every argument are in include/tbe.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local char g_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

tbe_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return TBE_ERR_HIP;
  }
  return TBE_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
namespace {
struct ProfState {
  std::mutex mu;
  std::string selected;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t used = 0;
};
ProfState& prof() {
  static ProfState* p = new ProfState();  // never destroyed: events outlive static teardown
  return *p;
}
}  // namespace

ProfScope::ProfScope(const char* kernel, hipStream_t s) : slot(-1), stream(s) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  if (P.selected.empty() || P.selected != kernel) return;
  if (P.used == P.events.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    P.events.emplace_back(a, b);
  }
  slot = static_cast<int>(P.used++);
  (void)hipEventRecord(P.events[slot].first, s);
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  ProfState& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  (void)hipEventRecord(P.events[slot].second, stream);
}

// ---------------------------------------------------------------------------
// device properties
// ---------------------------------------------------------------------------
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int blocks_per_cu(const void* kernel, size_t dyn_lds, int threads) {
  struct Entry {
    const void* kernel;
    size_t lds;
    int threads, n;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.kernel == kernel && e.lds == dyn_lds && e.threads == threads) return e.n;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, dyn_lds) != hipSuccess || n < 1) {
    (void)hipGetLastError();  // not sticky; fall back to 32 waves
    n = 32 * kWave / threads;
  }
  cache.push_back(Entry{kernel, dyn_lds, threads, n});
  return n;
}

// ---------------------------------------------------------------------------
// config and workspace layout
// ---------------------------------------------------------------------------
Config resolve_config(const tbe_config* c) {
  tbe_config d;
  tbe_config_default(&d);
  if (!c) c = &d;
  Config r;
  r.threshold = c->long_threshold > 0 ? c->long_threshold : d.long_threshold;
  r.chunk = c->chunk > 0 ? c->chunk : d.chunk;
  r.hist_enable = c->hist_enable;
  r.fwd_unroll = c->fwd_unroll > 0 ? c->fwd_unroll : d.fwd_unroll;
  r.bwd_unroll = c->bwd_unroll > 0 ? c->bwd_unroll : d.bwd_unroll;
  r.sort_blocks = c->sort_blocks;
  r.bag_windows = c->bag_windows;
  r.fused_long = c->fused_long;
  r.pretransposed = c->pretransposed;
  r.bags_per_wave = (c->bags_per_wave >= 1 && c->bags_per_wave <= 64) ? c->bags_per_wave : 0;
  r.bwd_streams = (c->bwd_streams == 1 || c->bwd_streams == 2) ? c->bwd_streams : 0;
  r.tiny = c->tiny_runs > 0 ? static_cast<int>(hmin(c->tiny_runs, r.threshold - 1)) : 0;
  // a dense row is a long run
  r.dense_min = c->dense_min > 0 ? static_cast<int>(hmax(c->dense_min, r.threshold)) : 0;
  r.dense_presort = c->dense_presort > 0 ? 1 : (c->dense_presort < 0 ? -1 : 0);
  r.sort_by_table = c->sort_by_table > 0 ? 1 : (c->sort_by_table < 0 ? -1 : 0);
  r.short_reserve = 0;
  r.short_work = nullptr;
  return r;
}

// The table the histogram kernels take in this call, or -1: the eligible table, when
// the histogram paths are on and there are no per-sample weights.
int histogram_table(const tbe_tables* tb, const Config& cfg, const float* psw) {
  return (cfg.hist_enable && !psw && tb->hist_table >= 0) ? tb->hist_table : -1;
}

namespace {
constexpr size_t kAlign = 256;
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return at;
  }
};
constexpr int kDefaultSortBlocks = 4096;
constexpr int kClsBlocks = 4096;  // classification workgroups at most (the scan takes up to 4096)
constexpr int kMaxSortBlocks = 4096;
}  // namespace

// sort / RLE block segments and classification blocks for n keys
// Sort blocks: sort_blocks (4096 by default) segments of whole 4096-key tiles; by default, when
// the sort covers all n keys (no table left out), at least two tiles a block when that still
// leaves 1024 blocks and 2T (which the sort by table needs): a block's fixed work, and the scan
// over blocks, then pay off (mixed-width batch's 15.7M keys, downsweep 0.32 -> 0.29 ms), while
// smaller sorts, and sorts whose n is only a bound, keep a block per tile
static void sort_geometry(int64_t n, const Config& cfg, int T, bool all_keys, int64_t* seg, int* nblocks,
                          int* cls_blocks) {
  const int64_t n1 = n > 0 ? n : 1;
  const int64_t tiles = (n1 + kRadixTile - 1) / kRadixTile;
  int64_t want = cfg.sort_blocks > 0 ? cfg.sort_blocks : kDefaultSortBlocks;
  if (want > kMaxSortBlocks) want = kMaxSortBlocks;
  if (want > tiles) want = tiles;
  const int64_t two = (tiles + 1) / 2;  // blocks of two tiles
  if (all_keys && cfg.sort_blocks <= 0 && want > two && two >= hmax(1024, 2 * static_cast<int64_t>(T))) want = two;
  const int64_t per = (tiles + want - 1) / want;  // tiles per block
  *seg = per * kRadixTile;
  *nblocks = static_cast<int>((n1 + *seg - 1) / *seg);
  *cls_blocks = static_cast<int>(hmax(1, hmin(kClsBlocks, (n1 + kBlock - 1) / kBlock)));
}

BwdLayout bwd_layout(const tbe_tables* tb, int64_t N, int weighted, const Config& cfg) {
  BwdLayout L;
  std::memset(&L, 0, sizeof(L));
  L.N = N;
  const int64_t n1 = N > 0 ? N : 1;
  Carver c;
  for (int i = 0; i < 2; ++i) {
    L.keys[i] = c.take(n1 * 4);
    L.pay[i] = c.take(n1 * 4);
  }
  L.bag_of = weighted ? c.take(n1 * 4) : 0;
  L.run_key = c.take(n1 * 4);
  L.run_start = c.take((n1 + 1) * 4);
  L.cap_long = N / cfg.threshold + 1;
  L.cap_chunk = N / cfg.chunk + L.cap_long;
  L.long_list = c.take(L.cap_long * 16);
  L.long_table = c.take(L.cap_long * 4);
  L.long_count = c.take(L.cap_long * 4);
  L.chunk_list = c.take(L.cap_chunk * 8);
  L.partial = c.take(static_cast<size_t>(L.cap_chunk) * tb->max_D * 4);
  for (int b = 0; b < TBE_NUM_BUCKETS; ++b) {
    L.cap_short[b] = tb->bucket_rows[b] > 0 ? (tb->bucket_rows[b] < N ? tb->bucket_rows[b] : N) : 0;
    L.short_list[b] = L.cap_short[b] ? c.take(L.cap_short[b] * 16) : 0;
  }
  // the histogram table's lookups, when its kernels take them, leave the sort
  const bool hist_out = cfg.hist_enable && tb->hist_table >= 0 && !weighted;
  sort_geometry(N, cfg, tb->T, !hist_out, &L.seg, &L.nblocks, &L.cls_blocks);
  L.sort_hist = c.take((static_cast<size_t>(kRadixDigits) * L.nblocks + kRadixDigits) * 4);
  L.seg_cnt = c.take(static_cast<size_t>(L.nblocks) * 4);
  L.cls_cnt = c.take(static_cast<size_t>(TBE_NUM_BUCKETS + 2) * L.cls_blocks * 4);
  // long-run chunks grouped by (table, window of bags); at most 4096 groups
  L.nwin = 1;
  if (cfg.bag_windows > 1 && tb->B > 1) {
    int64_t nw = hmin(cfg.bag_windows, hmax(1, 4096 / tb->T));
    nw = hmin(nw, tb->B);
    L.nwin = static_cast<int>(nw);
  }
  if (L.nwin > 1) {
    L.win_size = static_cast<int>((tb->B + L.nwin - 1) / L.nwin);
    L.units = tb->T * L.nwin;
    L.chunk_unit = c.take(L.cap_chunk * 4);
    L.chunk_order = c.take(L.cap_chunk * 4);
    L.unit_cnt = c.take(static_cast<size_t>(L.units) * 4);
  }
  if (cfg.hist_enable && tb->hist_table >= 0 && !weighted) {
    L.hist_partial = c.take(static_cast<size_t>(kHistBwdBlocks) * 64 * 128 * 4);
    L.hist_count = c.take(static_cast<size_t>(kHistBwdBlocks) * 64 * 4);
    L.hist_saved = c.take(static_cast<size_t>((tb->B + 15) / 16 * 16) * 64 * 2);
  }
  if (cfg.dense_min > 0 && !cfg.fused_long && tb->B > 0) {
    // partials per table: about 2048 workgroups in all, at most 64 a table, at most one per
    // 64-bag step
    const int64_t steps = (static_cast<int64_t>(tb->B) + 63) / 64;
    L.dense_on = 1;
    L.dense_P = static_cast<int>(hmax(1, hmin(hmin(64, 2048 / tb->T), steps)));
    L.dense_rows = c.take(static_cast<size_t>(tb->T) * kDenseRows * 4);
    L.dense_cnt = c.take(static_cast<size_t>(tb->T) * 4);
    L.dense_partial = c.take(static_cast<size_t>(tb->T) * L.dense_P * kDenseRows * 128 * 4);
    // automatic: the rows are picked before the sort from 2^26 lookups on, where the sort
    // work they take away outweighs the sample's fixed cost (about twenty short launches)
    L.dense_presort = cfg.dense_presort > 0 || (cfg.dense_presort == 0 && N >= (int64_t{1} << 26));
  }
  if (L.dense_on && !L.dense_presort) L.long_flag = c.take(L.cap_long * 4);
  if (L.dense_on && L.dense_presort) {
    // the sample: 64 positions in every hot_stride, at most 2^20 keys (every lookup of
    // batches up to 2^20 lookups); a row is taken when its sampled lookups reach dense_min
    // scaled to the sample
    L.hot_stride = 64;
    while (64 * ((N + L.hot_stride - 1) / L.hot_stride) > (int64_t{1} << 20)) L.hot_stride *= 2;
    L.hot_thr = static_cast<int>(hmax(1, (static_cast<int64_t>(cfg.dense_min) * 64 + L.hot_stride - 1) / L.hot_stride));
    SortPlan& P = L.sample;
    P.N = 64 * ((N + L.hot_stride - 1) / L.hot_stride);
    const int64_t m1 = P.N > 0 ? P.N : 1;
    for (int i = 0; i < 2; ++i) {
      P.keys[i] = c.take(m1 * 4);
      P.pay[i] = c.take(m1 * 4);
    }
    P.run_key = c.take(m1 * 4);
    P.run_start = c.take((m1 + 1) * 4);
    P.cap_long = P.N / L.hot_thr + 1;
    P.cap_chunk = 0;
    P.long_list = c.take(P.cap_long * 16);
    P.long_table = c.take(P.cap_long * 4);
    P.long_count = c.take(P.cap_long * 4);
    P.chunk_list = 0;
    sort_geometry(P.N, cfg, tb->T, true, &P.seg, &P.nblocks, &P.cls_blocks);
    P.sort_hist = c.take((static_cast<size_t>(kRadixDigits) * P.nblocks + kRadixDigits) * 4);
    P.seg_cnt = c.take(static_cast<size_t>(P.nblocks) * 4);
    P.cls_cnt = c.take(static_cast<size_t>(TBE_NUM_BUCKETS + 2) * P.cls_blocks * 4);
    P.counters = c.take(kNumCounters * 4);
    // words of 16-byte records, three key slots each: at most a sixth of the slots used
    int64_t hs = 1024;
    while (hs < 8 * static_cast<int64_t>(kDenseRows) * tb->T) hs <<= 1;
    L.hot_set_size = hs;
    L.hot_set = c.take(static_cast<size_t>(hs) * 4);
    L.dense_slot = c.take(static_cast<size_t>(n1) * 2);
    L.hot_bloom = c.take(static_cast<size_t>(kHotBloomWords) * 4);
  }
  // keys are in [0, total_rows]; total_rows itself marks an id outside its table
  uint32_t maxkey = static_cast<uint32_t>(tb->total_rows);
  int kb = 1;
  while (kb < 32 && (maxkey >> kb) != 0) ++kb;
  L.key_bits = kb;
  auto plan = [](int bits_total, int by_table, RadixPlan& R) {
    R.passes = (bits_total + kRadixMaxBits - 1) / kRadixMaxBits;
    int shift = 0;
    for (int p = 0; p < R.passes; ++p) {
      const int bits = bits_total / R.passes + (p < bits_total % R.passes ? 1 : 0);
      R.shift[p] = shift;
      R.bits[p] = bits;
      shift += bits;
    }
    R.by_table = by_table;
  };
  plan(kb, 0, L.sample_radix);
  L.radix = L.sample_radix;
  // by table: the local row ids of the largest table in no more passes, at least one sort block
  // per table and most blocks dealt by keys (at most half as many tables as blocks)
  const int lb = tb->row_bits > 0 ? tb->row_bits : 1;
  const bool can_by_table = tb->T >= 2 && 2 * static_cast<int64_t>(tb->T) <= L.nblocks &&
                            (lb + kRadixMaxBits - 1) / kRadixMaxBits <= L.sample_radix.passes;
  if (cfg.sort_by_table > 0 ? can_by_table : (cfg.sort_by_table == 0 && can_by_table && lb < kb)) {
    plan(lb, 1, L.radix);
    L.tstart = c.take(static_cast<size_t>(2) * (tb->T + 1) * 4);
  }
  L.counters = c.take(kNumCounters * 4);
  L.total = c.off;
  // the radix passes alternate buffers from buffer 0
  L.final_buf = L.radix.passes & 1;
  return L;
}

}  // namespace tbe

using namespace tbe;

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
namespace {

tbe_status check_tables(const tbe_tables* tb) {
  if (!tb) { set_error("tables is NULL"); return TBE_ERR_ARG; }
  if (tb->T < 1 || tb->B < 0) { set_error("bad geometry T=%d B=%d", tb->T, tb->B); return TBE_ERR_ARG; }
  if (tb->w_dtype < TBE_F32 || tb->w_dtype > TBE_BF16) { set_error("bad w_dtype %d", tb->w_dtype); return TBE_ERR_UNSUPPORTED; }
  if (!tb->meta) { set_error("tables->meta (device copy of the table metadata) is NULL"); return TBE_ERR_ARG; }
  if (tb->max_D < 4 || tb->max_D > TBE_MAX_D) { set_error("max_D %d outside [4, %d]", tb->max_D, TBE_MAX_D); return TBE_ERR_UNSUPPORTED; }
  if (tb->total_rows < 1 || tb->total_rows >= (1ll << 31) - 1) { set_error("total rows %lld outside [1, 2^31-1)", (long long)tb->total_rows); return TBE_ERR_UNSUPPORTED; }
  if (static_cast<int64_t>(tb->T) * tb->B >= (1ll << 31)) { set_error("T*B must be < 2^31"); return TBE_ERR_UNSUPPORTED; }
  return TBE_OK;
}

tbe_status check_index_args(const tbe_tables* tb, const void* indices, int itype, const void* offsets,
                            int otype, int64_t N) {
  if (itype != TBE_I32 && itype != TBE_I64) { set_error("bad index type %d", itype); return TBE_ERR_ARG; }
  if (otype != TBE_I32 && otype != TBE_I64) { set_error("bad offset type %d", otype); return TBE_ERR_ARG; }
  // positions are 32-bit in the kernels, with room for a step of a few hundred past the end
  if (N < 0 || N > TBE_MAX_LOOKUPS) { set_error("num_indices %lld outside [0, 2^31 - 4096]", (long long)N); return TBE_ERR_UNSUPPORTED; }
  if (N > 0 && !indices) { set_error("indices is NULL"); return TBE_ERR_ARG; }
  if (!offsets) { set_error("offsets is NULL"); return TBE_ERR_ARG; }
  if (itype == TBE_I32 && N > 0 && (reinterpret_cast<uintptr_t>(indices) & 3)) { set_error("indices misaligned"); return TBE_ERR_ARG; }
  if (reinterpret_cast<uintptr_t>(offsets) & (otype == TBE_I32 ? 3 : 7)) { set_error("offsets misaligned"); return TBE_ERR_ARG; }
  (void)tb;
  return TBE_OK;
}

tbe_status check_rows(const void* p, const char* what, size_t align) {
  if (!p) { set_error("%s is NULL", what); return TBE_ERR_ARG; }
  if (reinterpret_cast<uintptr_t>(p) % align) { set_error("%s is not %zu-byte aligned", what, align); return TBE_ERR_ARG; }
  return TBE_OK;
}

size_t weight_align(const tbe_tables* tb) { return tb->w_dtype == TBE_F32 ? 16 : (tb->all_D_mult8 ? 16 : 8); }

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* tbe_status_string(tbe_status s) {
  switch (s) {
    case TBE_OK: return "ok";
    case TBE_ERR_ARG: return "invalid argument";
    case TBE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TBE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TBE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* tbe_last_error(void) { return g_error; }

void tbe_config_default(tbe_config* cfg) {
  if (!cfg) return;
  cfg->long_threshold = 256;
  cfg->chunk = 256;
  cfg->hist_enable = 1;
  cfg->fwd_unroll = 4;
  cfg->bwd_unroll = 8;
  cfg->sort_blocks = 0;
  cfg->bag_windows = 1;
  cfg->fused_long = 0;
  cfg->pretransposed = 0;
  cfg->bags_per_wave = 0;
  cfg->bwd_streams = 0;
  cfg->tiny_runs = 8;
  cfg->dense_min = 1024;
  cfg->dense_presort = 0;
  cfg->sort_by_table = 0;
}

int64_t tbe_meta_entries(int32_t T) { return T >= 0 ? static_cast<int64_t>(TBE_META_FIELDS) * (T + 1) : 0; }

tbe_status tbe_tables_derive(int32_t T, int32_t B, int32_t w_dtype, const int64_t* E_host,
                             const int32_t* D_host, const int32_t* pooling_hint_host,
                             int64_t* meta_host, tbe_tables* out) {
  g_error[0] = 0;
  if (!out || !E_host || !D_host || !meta_host) { set_error("NULL argument"); return TBE_ERR_ARG; }
  if (T < 1 || B < 0) { set_error("bad geometry T=%d B=%d", T, B); return TBE_ERR_ARG; }
  if (w_dtype < TBE_F32 || w_dtype > TBE_BF16) { set_error("bad w_dtype %d", w_dtype); return TBE_ERR_UNSUPPORTED; }
  std::memset(out, 0, sizeof(*out));
  out->T = T;
  out->B = B;
  out->w_dtype = w_dtype;
  out->hist_table = -1;
  out->all_D_mult8 = 1;
  int64_t rows = 0, elems = 0, cols = 0;
  int maxD = 0;
  out->row_bits = 1;
  for (int t = 0; t < T; ++t) {
    const int64_t E = E_host[t];
    const int32_t D = D_host[t];
    if (E < 1) { set_error("table %d has %lld rows", t, (long long)E); return TBE_ERR_ARG; }
    while (out->row_bits < 32 && ((E - 1) >> out->row_bits) != 0) ++out->row_bits;
    if (D < 4 || D > TBE_MAX_D || D % 4) { set_error("table %d: D=%d not in [4, %d] or not a multiple of 4", t, D, TBE_MAX_D); return TBE_ERR_UNSUPPORTED; }
    meta_host[4 * t + 0] = rows;
    meta_host[4 * t + 1] = elems;
    meta_host[4 * t + 2] = cols;
    meta_host[4 * t + 3] = D;
    if (D % 8) out->all_D_mult8 = 0;
    if (D > maxD) maxD = D;
    out->bucket_rows[bucket_of_D(D)] += E;
    if (out->hist_table < 0 && pooling_hint_host && E <= 64 && D >= 64 && D <= 128 && D % 16 == 0 &&
        w_dtype == TBE_F16 && pooling_hint_host[t] >= 64) {
      out->hist_table = t;
      out->hist_E = static_cast<int32_t>(E);
      out->hist_D = D;
      out->hist_col = static_cast<int32_t>(cols);
      out->hist_w_base = elems;
    }
    rows += E;
    elems += E * D;
    cols += D;
    if (rows >= (1ll << 31) - 1) { set_error("sum of rows must be < 2^31 - 1"); return TBE_ERR_UNSUPPORTED; }
    if (cols >= (1ll << 31)) { set_error("sum of D too large"); return TBE_ERR_UNSUPPORTED; }
  }
  meta_host[4 * T + 0] = rows;
  meta_host[4 * T + 1] = elems;
  meta_host[4 * T + 2] = cols;
  meta_host[4 * T + 3] = 0;
  out->max_D = maxD;
  out->out_width = static_cast<int32_t>(cols);
  out->total_rows = rows;
  out->total_elems = elems;
  out->meta = nullptr;
  return TBE_OK;
}

size_t tbe_bounds_check_workspace_bytes(const tbe_tables* tables) { return bounds_workspace(tables); }

tbe_status tbe_bounds_check(const tbe_tables* tables, void* indices, int32_t index_type, void* offsets,
                            int32_t offset_type, int64_t num_indices, int64_t* error_counts,
                            void* workspace, size_t workspace_bytes, tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (!error_counts) { set_error("error_counts is NULL"); return TBE_ERR_ARG; }
  if (!workspace || workspace_bytes < bounds_workspace(tables) || (reinterpret_cast<uintptr_t>(workspace) & 255)) {
    set_error("bounds workspace needs %zu bytes, 256-byte aligned", bounds_workspace(tables));
    return TBE_ERR_WORKSPACE;
  }
  return launch_bounds(tables, indices, index_type, offsets, offset_type, num_indices, error_counts,
                       workspace, static_cast<hipStream_t>(stream));
}

tbe_status tbe_forward(const tbe_tables* tables, const void* weights, const void* indices,
                       int32_t index_type, const void* offsets, int32_t offset_type, int64_t num_indices,
                       const float* per_sample_weights, float* out, const tbe_config* config,
                       tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (tables->B == 0) return TBE_OK;
  if (tbe_status st = check_rows(weights, "weights", weight_align(tables))) return st;
  if (tbe_status st = check_rows(out, "out", 16)) return st;
  const Config cfg = resolve_config(config);
  IndexArgs ia{indices, index_type, offsets, offset_type, num_indices};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int hist = histogram_table(tables, cfg, per_sample_weights);
  if (hist >= 0)
    if (tbe_status st = launch_forward_hist(tables, weights, ia, out, nullptr, nullptr, s)) return st;
  return launch_forward_gather(tables, weights, ia, per_sample_weights, out, hist, cfg.fwd_unroll,
                               cfg.bags_per_wave, nullptr, s);
}

// Forward after the offsets are final: the histogram table (if used) and the
// gather; with error_counts, out-of-range ids are repaired on the way.
static tbe_status forward_body(const tbe_tables* tables, const void* weights, const IndexArgs& ia,
                               const float* psw, float* out, int64_t* error_counts, const Config& cfg,
                               uint16_t* save_counts, hipStream_t s) {
  const int hist = histogram_table(tables, cfg, psw);
  // both kernels repair the ids they read (the histogram table's, everyone else's)
  if (hist >= 0)
    if (tbe_status st = launch_forward_hist(tables, weights, ia, out, error_counts, save_counts, s))
      return st;
  return launch_forward_gather(tables, weights, ia, psw, out, hist, cfg.fwd_unroll, cfg.bags_per_wave,
                               error_counts, s);
}

static tbe_status check_bounds_ws(const tbe_tables* tables, const void* workspace, size_t bytes) {
  if (!workspace || bytes < bounds_workspace(tables) || (reinterpret_cast<uintptr_t>(workspace) & 255)) {
    set_error("bounds workspace needs %zu bytes, 256-byte aligned", bounds_workspace(tables));
    return TBE_ERR_WORKSPACE;
  }
  return TBE_OK;
}

static tbe_status check_repair_args(const tbe_tables* tables, const void* weights, void* indices,
                                    int32_t index_type, void* offsets, int32_t offset_type,
                                    int64_t num_indices, const float* out, const int64_t* error_counts) {
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (!error_counts) { set_error("error_counts is NULL"); return TBE_ERR_ARG; }
  if (tables->B > 0) {
    if (tbe_status st = check_rows(weights, "weights", weight_align(tables))) return st;
    if (tbe_status st = check_rows(out, "out", 16)) return st;
  }
  return TBE_OK;
}

// tbe_forward_repair once its arguments are checked; workspace holds the offsets repair's
// block partials (bounds_workspace bytes)
static tbe_status forward_repair_body(const tbe_tables* tables, const void* weights, void* indices,
                                      int32_t index_type, void* offsets, int32_t offset_type,
                                      int64_t num_indices, const float* per_sample_weights, float* out,
                                      int64_t* error_counts, void* workspace, const tbe_config* config,
                                      tbe_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tbe_status st = launch_bounds_offsets(tables, offsets, offset_type, num_indices, error_counts,
                                            workspace, s))
    return st;
  if (tables->B == 0) return launch_bounds_indices(tables, indices, index_type, offsets, offset_type,
                                                   num_indices, error_counts, s);
  const Config cfg = resolve_config(config);
  IndexArgs ia{indices, index_type, offsets, offset_type, num_indices};
  return forward_body(tables, weights, ia, per_sample_weights, out, error_counts, cfg, nullptr, s);
}

tbe_status tbe_forward_repair(const tbe_tables* tables, const void* weights, void* indices,
                              int32_t index_type, void* offsets, int32_t offset_type, int64_t num_indices,
                              const float* per_sample_weights, float* out, int64_t* error_counts,
                              void* workspace, size_t workspace_bytes, const tbe_config* config,
                              tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_repair_args(tables, weights, indices, index_type, offsets, offset_type,
                                        num_indices, out, error_counts))
    return st;
  if (tbe_status st = check_bounds_ws(tables, workspace, workspace_bytes)) return st;
  return forward_repair_body(tables, weights, indices, index_type, offsets, offset_type, num_indices,
                             per_sample_weights, out, error_counts, workspace, config, stream);
}

// ---------------------------------------------------------------------------
// The entry point that allocates nothing.  The offsets repair's block partials live in a
// static device array, one copy per GPU, held until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per device (its first
// call there, with that device current) and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int64_t scratch[TBE_NOALLOC_SCRATCH_BYTES / sizeof(int64_t)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

static tbe_status scratch_of_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    set_error("hipGetDevice failed or device id out of range");
    return TBE_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return TBE_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TBE_OK;
}

tbe_status tbe_forward_repair_noalloc(const tbe_tables* tables, const void* weights, void* indices,
                                      int32_t index_type, void* offsets, int32_t offset_type,
                                      int64_t num_indices, const float* per_sample_weights, float* out,
                                      int64_t* error_counts, const tbe_config* config, tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_repair_args(tables, weights, indices, index_type, offsets, offset_type,
                                        num_indices, out, error_counts))
    return st;
  if (bounds_workspace(tables) > sizeof(scratch)) {
    set_error("the offsets repair needs %zu bytes of scratch, more than the %zu bytes the library holds",
              bounds_workspace(tables), sizeof(scratch));
    return TBE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (tbe_status st = scratch_of_current_device(&ws)) return st;
  return forward_repair_body(tables, weights, indices, index_type, offsets, offset_type, num_indices,
                             per_sample_weights, out, error_counts, ws, config, stream);
}

// ---------------------------------------------------------------------------
// second stream (hoisted transpose, concurrent long runs)
// ---------------------------------------------------------------------------
namespace {
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];
}  // namespace

Fork::Fork(hipStream_t s) : main_(s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("hipGetDevice failed or device id out of range");
    st_ = TBE_ERR_HIP;
    return;
  }
  g_side_mu.lock();
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    // default priority; does not synchronize with the null stream
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      set_error("could not create the side stream or its events");
      st_ = TBE_ERR_HIP;
      ss.stream = nullptr;
      g_side_mu.unlock();
      return;
    }
  }
  if (hipEventRecord(ss.fork, s) != hipSuccess || hipStreamWaitEvent(ss.stream, ss.fork, 0) != hipSuccess) {
    set_error("fork to the side stream failed");
    st_ = TBE_ERR_HIP;
    g_side_mu.unlock();
    return;
  }
  side_ = ss.stream;
  done_ = ss.join;
  joined_ = false;
}

tbe_status Fork::join() {
  if (joined_) return st_;
  joined_ = true;
  const bool ok = hipEventRecord(static_cast<hipEvent_t>(done_), side_) == hipSuccess &&
                  hipStreamWaitEvent(main_, static_cast<hipEvent_t>(done_), 0) == hipSuccess;
  g_side_mu.unlock();
  if (!ok) {
    set_error("join of the side stream failed");
    st_ = TBE_ERR_HIP;
  }
  return st_;
}

Fork::~Fork() { join(); }

tbe_status tbe_forward_hoisted(const tbe_tables* tables, const void* weights, void* indices,
                               int32_t index_type, void* offsets, int32_t offset_type,
                               int64_t num_indices, const float* per_sample_weights, float* out,
                               int64_t* error_counts, void* bounds_workspace,
                               size_t bounds_workspace_bytes, void* bwd_workspace,
                               size_t bwd_workspace_bytes, const tbe_config* config,
                               tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (error_counts)
    if (tbe_status st = check_bounds_ws(tables, bounds_workspace, bounds_workspace_bytes)) return st;
  if (tables->B > 0) {
    if (tbe_status st = check_rows(weights, "weights", weight_align(tables))) return st;
    if (tbe_status st = check_rows(out, "out", 16)) return st;
  }
  const Config cfg = resolve_config(config);
  const int weighted = per_sample_weights ? 1 : 0;
  const BwdLayout L = bwd_layout(tables, num_indices, weighted, cfg);
  if (!bwd_workspace || bwd_workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(bwd_workspace) & 255)) {
    set_error("backward workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total, bwd_workspace_bytes);
    return TBE_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (error_counts)
    if (tbe_status st = launch_bounds_offsets(tables, offsets, offset_type, num_indices, error_counts,
                                              bounds_workspace, s))
      return st;
  IndexArgs ia{indices, index_type, offsets, offset_type, num_indices};
  // the backward skips the transpose when there are no bags or no lookups
  if (tables->B == 0 || num_indices == 0) {
    if (tables->B == 0)
      return error_counts ? launch_bounds_indices(tables, indices, index_type, offsets, offset_type,
                                                  num_indices, error_counts, s)
                          : TBE_OK;
    return forward_body(tables, weights, ia, per_sample_weights, out, error_counts, cfg, nullptr, s);
  }
  const int hist = histogram_table(tables, cfg, per_sample_weights);
  // forward-state reuse: the histogram forward keeps its counts for the backward
  uint16_t* saved = hist >= 0 ? reinterpret_cast<uint16_t*>(static_cast<char*>(bwd_workspace) + L.hist_saved)
                              : nullptr;
  Fork fork(s);
  if (tbe_status st = fork.status()) return st;
  int final_buf = 0;
  const tbe_status st_t = launch_transpose(tables, ia, weighted, static_cast<char*>(bwd_workspace), L,
                                           cfg, hist, error_counts ? 1 : 0, 1, &final_buf, fork.side());
  const tbe_status st_f = st_t ? TBE_OK
                               : forward_body(tables, weights, ia, per_sample_weights, out, error_counts,
                                              cfg, saved, s);
  // joined even after a failed launch, so that the streams stay ordered
  const tbe_status st_j = fork.join();
  return st_t ? st_t : (st_f ? st_f : st_j);
}

size_t tbe_backward_workspace_bytes(const tbe_tables* tables, int64_t num_indices, int32_t weighted,
                                    const tbe_config* config) {
  if (!tables || num_indices < 0) return 0;
  return bwd_layout(tables, num_indices, weighted ? 1 : 0, resolve_config(config)).total;
}

static tbe_status backward_common(const tbe_tables* tables, void* weights, float* momentum, int opt,
                                  const void* indices, int32_t index_type, const void* offsets,
                                  int32_t offset_type, int64_t num_indices, const float* psw,
                                  const float* grad_out, float lr, float eps, void* workspace,
                                  size_t workspace_bytes, const tbe_config* config, tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (tables->B == 0 || num_indices == 0) return TBE_OK;
  if (tbe_status st = check_rows(weights, "weights", weight_align(tables))) return st;
  if (tbe_status st = check_rows(grad_out, "grad_out", 16)) return st;
  if (opt == kOptAdagrad && !momentum) { set_error("momentum is NULL"); return TBE_ERR_ARG; }
  const Config cfg = resolve_config(config);
  const BwdLayout L = bwd_layout(tables, num_indices, psw ? 1 : 0, cfg);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) {
    set_error("backward workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total, workspace_bytes);
    return TBE_ERR_WORKSPACE;
  }
  IndexArgs ia{indices, index_type, offsets, offset_type, num_indices};
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // the small table's rows are updated from per-bag counts x gradient (MFMA) instead of runs
  const int hist = histogram_table(tables, cfg, psw);
  // pretransposed: tbe_forward_hoisted left the sorted runs in the workspace, the sorted
  // payloads in buffer L.final_buf
  int final_buf = L.final_buf;
  if (!cfg.pretransposed)
    if (tbe_status st = launch_transpose(tables, ia, psw ? 1 : 0, ws, L, cfg, hist, 0, 1, &final_buf, s)) return st;
  // without dense_presort the dense rows come from the long runs (flags read by the chunk and
  // apply kernels)
  if (L.dense_on && !L.dense_presort)
    if (tbe_status st = launch_dense_select_runs(tables, ws, L, hist, cfg, s)) return st;
  // automatic: short runs of several widths are several short launches, whose tails leave
  // room for the long runs
  int buckets = 0;
  for (int b = 0; b < TBE_NUM_BUCKETS; ++b) buckets += L.cap_short[b] > 0;
  const int streams = cfg.bwd_streams ? cfg.bwd_streams : (buckets >= 2 ? 2 : 1);
  // (with per-sample weights the dense rows run on the short runs' stream or after the long runs:
  // the shared-counter short-run grids serve unweighted batches only)
  const bool beside =
      cfg.bwd_streams == 0 && streams < 2 && ((L.dense_on && L.dense_presort && !psw) || hist >= 0);
  if (hist >= 0 && !beside) {
    // with the hoisted forward's state, its saved counts replace counting the first 256 ids
    const uint16_t* saved = cfg.pretransposed ? reinterpret_cast<const uint16_t*>(ws + L.hist_saved) : nullptr;
    if (tbe_status st = launch_hist_backward(tables, weights, momentum, opt, ia, grad_out, lr, eps, ws, L,
                                             saved, s))
      return st;
  }
  const bool side_dense = L.dense_on && L.dense_presort && !psw;
  if (beside) {
    // the histogram table's backward and the dense rows' kernels (matrix cores and LDS
    // counting) on the second stream, launched first with one workgroup per CU, beside the
    // short runs (bound by gradient-row reads), whose grid leaves that workgroup's share of
    // every SIMD free (disjoint rows throughout)
    // with the long runs on the second stream, the short runs take their work from a counter
    // (cleared before the fork, so the second stream's work starts after it): a second
    // short-run grid follows the long runs there and takes what the first has not reached
    int32_t* work = side_dense ? reinterpret_cast<int32_t*>(ws + L.counters) + kShortWork : nullptr;
    if (work)
      if (tbe_status st = launch_fill_i32(work, 0, 1, s)) return st;
    Fork fork(s);
    if (tbe_status st = fork.status()) return st;
    tbe_status st = TBE_OK;
    int reserve = 0;  // the side kernels' share of a SIMD's registers, in 1/512
    if (hist >= 0) {
      const uint16_t* saved = cfg.pretransposed ? reinterpret_cast<const uint16_t*>(ws + L.hist_saved) : nullptr;
      st = launch_hist_backward(tables, weights, momentum, opt, ia, grad_out, lr, eps, ws, L, saved, fork.side(), 1);
      reserve = hmax(reserve, (512 + hist_partial_blocks_per_cu() - 1) / hist_partial_blocks_per_cu());
    }
    if (!st && side_dense) {
      st = launch_dense_backward(tables, weights, momentum, opt, ia, psw, grad_out, lr, eps, ws, L, fork.side(), 1);
      reserve = hmax(reserve, (512 + dense_partial_blocks_per_cu() - 1) / dense_partial_blocks_per_cu());
    }
    Config c2 = cfg;
    c2.short_reserve = reserve;
    c2.short_work = work;
    // with the dense rows picked before the sort, the long runs follow the dense kernels on the
    // second stream: their chunks start in the slots the dense kernel leaves while the short
    // runs go on (skewed batch 9.72 -> 9.64 ms)
    if (!st)
      st = launch_backward_update(tables, weights, momentum, opt, psw, grad_out, lr, eps, ws, L, final_buf, c2,
                                  s, side_dense ? fork.side() : s);
    // dense rows picked from the long runs after the sort: after the chunk kernels on s
    if (!st && L.dense_on && !L.dense_presort)
      st = launch_dense_backward(tables, weights, momentum, opt, ia, psw, grad_out, lr, eps, ws, L, s);
    const tbe_status st_j = fork.join();
    return st ? st : st_j;
  }
  if (streams < 2 || L.cap_long == 0) {
    if (tbe_status st = launch_backward_update(tables, weights, momentum, opt, psw, grad_out, lr, eps, ws,
                                               L, final_buf, cfg, s, s))
      return st;
    return L.dense_on ? launch_dense_backward(tables, weights, momentum, opt, ia, psw, grad_out, lr, eps, ws, L, s)
                      : TBE_OK;
  }
  // long runs (and the dense rows) on a second stream, concurrent with the short runs
  // (disjoint rows)
  Fork fork(s);
  if (tbe_status st = fork.status()) return st;
  tbe_status st = launch_backward_update(tables, weights, momentum, opt, psw, grad_out, lr, eps, ws, L,
                                         final_buf, cfg, s, fork.side());
  if (!st && L.dense_on)
    st = launch_dense_backward(tables, weights, momentum, opt, ia, psw, grad_out, lr, eps, ws, L, fork.side());
  const tbe_status st_j = fork.join();
  return st ? st : st_j;
}

tbe_status tbe_backward_sgd(const tbe_tables* tables, void* weights, const void* indices,
                            int32_t index_type, const void* offsets, int32_t offset_type,
                            int64_t num_indices, const float* per_sample_weights, const float* grad_out,
                            float lr, void* workspace, size_t workspace_bytes, const tbe_config* config,
                            tbe_stream_t stream) {
  return backward_common(tables, weights, nullptr, kOptSGD, indices, index_type, offsets, offset_type,
                         num_indices, per_sample_weights, grad_out, lr, 0.f, workspace, workspace_bytes,
                         config, stream);
}

tbe_status tbe_backward_rowwise_adagrad(const tbe_tables* tables, void* weights, float* momentum,
                                        const void* indices, int32_t index_type, const void* offsets,
                                        int32_t offset_type, int64_t num_indices,
                                        const float* per_sample_weights, const float* grad_out, float lr,
                                        float eps, void* workspace, size_t workspace_bytes,
                                        const tbe_config* config, tbe_stream_t stream) {
  return backward_common(tables, weights, momentum, kOptAdagrad, indices, index_type, offsets,
                         offset_type, num_indices, per_sample_weights, grad_out, lr, eps, workspace,
                         workspace_bytes, config, stream);
}

tbe_status tbe_transpose(const tbe_tables* tables, const void* indices, int32_t index_type,
                         const void* offsets, int32_t offset_type, int64_t num_indices, int32_t weighted,
                         void* workspace, size_t workspace_bytes, const tbe_config* config,
                         tbe_runs_view* view, tbe_stream_t stream) {
  g_error[0] = 0;
  if (tbe_status st = check_tables(tables)) return st;
  if (tbe_status st = check_index_args(tables, indices, index_type, offsets, offset_type, num_indices)) return st;
  if (!view) { set_error("view is NULL"); return TBE_ERR_ARG; }
  const Config cfg = resolve_config(config);
  const BwdLayout L = bwd_layout(tables, num_indices, weighted ? 1 : 0, cfg);
  if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255)) {
    set_error("transpose workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total, workspace_bytes);
    return TBE_ERR_WORKSPACE;
  }
  IndexArgs ia{indices, index_type, offsets, offset_type, num_indices};
  char* ws = static_cast<char*>(workspace);
  // pretransposed: describe what tbe_forward_hoisted left in the workspace (sorted keys and
  // payloads in buffer L.final_buf)
  int final_buf = L.final_buf;
  tbe_status st = TBE_OK;
  if (!cfg.pretransposed)
    st = launch_transpose(tables, ia, weighted ? 1 : 0, ws, L, cfg, -1, 0, 0, &final_buf,
                          static_cast<hipStream_t>(stream));
  std::memset(view, 0, sizeof(*view));
  view->sorted_keys = reinterpret_cast<const uint32_t*>(ws + L.keys[final_buf]);
  view->sorted_payload = reinterpret_cast<const uint32_t*>(ws + L.pay[final_buf]);
  view->run_key = reinterpret_cast<const uint32_t*>(ws + L.run_key);
  view->run_start = reinterpret_cast<const uint32_t*>(ws + L.run_start);
  view->counters = reinterpret_cast<const int32_t*>(ws + L.counters);
  view->long_list = reinterpret_cast<const uint32_t*>(ws + L.long_list);
  view->long_table = reinterpret_cast<const uint32_t*>(ws + L.long_table);
  view->chunk_list = reinterpret_cast<const uint32_t*>(ws + L.chunk_list);
  for (int b = 0; b < TBE_NUM_BUCKETS; ++b) {
    view->short_list[b] = L.cap_short[b] ? reinterpret_cast<const uint32_t*>(ws + L.short_list[b]) : nullptr;
    view->short_capacity[b] = L.cap_short[b];
  }
  view->long_capacity = L.cap_long;
  view->chunk_capacity = L.cap_chunk;
  view->payload_is_position = weighted ? 1 : 0;
  view->radix_passes = L.radix.passes;
  view->sorted_by_table = L.radix.by_table;
  if (L.dense_on && L.dense_presort) {
    view->dense_rows = reinterpret_cast<const int32_t*>(ws + L.dense_rows);
    view->dense_count = reinterpret_cast<const int32_t*>(ws + L.dense_cnt);
  }
  return st;
}

tbe_status tbe_profile_select(const char* kernel_name) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  P.selected = kernel_name ? kernel_name : "";
  P.used = 0;
  return TBE_OK;
}

tbe_status tbe_profile_read(int64_t* launches, double* total_ms) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  double ms = 0.0;
  for (size_t i = 0; i < P.used; ++i) {
    if (hipEventSynchronize(P.events[i].second) != hipSuccess) {
      set_error("hipEventSynchronize failed");
      return TBE_ERR_HIP;
    }
    float f = 0.f;
    if (hipEventElapsedTime(&f, P.events[i].first, P.events[i].second) != hipSuccess) {
      set_error("hipEventElapsedTime failed");
      return TBE_ERR_HIP;
    }
    ms += f;
  }
  if (launches) *launches = static_cast<int64_t>(P.used);
  if (total_ms) *total_ms = ms;
  P.used = 0;
  return TBE_OK;
}

}  // extern "C"
