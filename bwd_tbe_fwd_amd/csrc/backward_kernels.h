// Backward gradient reduction and optimizer kernels (templates; instantiated
// per weight format in backward_f32.hip / backward_f16.hip / backward_bf16.hip).
//
// Routing after PyTorch blog "Modernizing Table Batched Embeddings with
// FBTriton", sections 3 and 4 (problem 3).  Here, a run of fewer than 256
// lookups goes to short_run_kernel, where one lane group reads every gradient
// row of the run, sums them in registers, runs the optimizer and stores the
// row: nothing else writes that row, so no atomics are needed.  A run of 256
// or more is split into 256-lookup chunks: grad_accum_kernel writes one fp32
// partial row per chunk into the workspace and long_apply_kernel adds a run's
// partials and steps the optimizer.  With per-sample weights, the kernels
// multiply a lookup's gradient row by its weight as they add it.  Short runs
// are launched once per width bucket next_pow2(D), and the bucket fixes how
// many lanes serve one run.  The optimizer is the backward's epilogue: SGD (w - lr*g) or
// exact row-wise Adagrad ("Table-Batched Embeddings in Triton", section 5:
// m += mean_d g_d^2, w -= lr*g/(sqrt(m)+eps) with the new m).
//
// gfx950 mapping: gradients are fp32 rows of D floats, read as float4 per lane,
// so a run of bucket BD is served by BD/4 lanes (BD >= 256: all 64 lanes with
// BD/256 column passes) and a wave owns 64/(BD/4) short runs at once - no lane
// is masked off for D = BD, and the per-run metadata (one 16-byte descriptor)
// is amortized over the lanes of the run.  UNROLL gradient rows are in flight
// per lane before they are summed.  A wave step whose runs are all tiny (a few
// lookups each: their time goes to waiting on the descriptor, payload and row
// loads, not to bandwidth) serves twice as many runs with half the lanes each.  The weight row and the Adagrad state are
// loaded before the gradient loop so their latency overlaps it.  Accumulation
// is fp32 throughout; no float atomics anywhere, so results are deterministic.
#pragma once

#include "tbe_device.h"
#include "tbe_internal.h"

namespace tbe {

// One short run, owned by a group of LPR lanes (c: this lane's place in the group); each
// lane holds NP float4 column chunks of the row.
template <int DT, int NP, int LPR, int OPT, bool WEIGHTED, int UNROLL>
__device__ __forceinline__ void short_run_one(
    typename Fmt<DT>::S* __restrict__ W, float* __restrict__ momentum,
    const float* __restrict__ grad_out, const uint32_t* __restrict__ pay,
    const uint32_t* __restrict__ bag_of, const float* __restrict__ psw, const uint4 dsc, int c,
    const int64_t* __restrict__ meta, int32_t B, int32_t out_width, float lr, float eps) {
  using S = typename Fmt<DT>::S;
  const uint32_t key = dsc.x, start = dsc.y, len = dsc.z;
  const int t = static_cast<int>(dsc.w);
  const TableMeta m = load_meta(meta, t);
  const int D = static_cast<int>(m.D);
  S* wrow = W + m.w_base + (static_cast<int64_t>(key) - m.row_base) * D;
  const int64_t bag_lo = static_cast<int64_t>(t) * B;
  float w[NP][4];
  bool act[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int col = p * 4 * LPR + c * 4;
    act[p] = col < D;
    if (act[p]) {
      load_vec<DT, 4, true>(wrow + col, w[p]);  // read once, written back below
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) w[p][q] = 0.f;
    }
  }
  float mom = 0.f;
  if constexpr (OPT == kOptAdagrad) mom = __builtin_nontemporal_load(momentum + key);
  float acc[NP][4];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[p][q] = 0.f;
  for (uint32_t j0 = 0; j0 < len; j0 += LPR) {
    const int nb = static_cast<int>(min<uint32_t>(LPR, len - j0));
    int32_t myb = -1;
    float myw = 1.f;
    if (c < nb) {
      const uint32_t pv = pay[start + j0 + c];
      int64_t bag;
      if constexpr (WEIGHTED) {
        bag = bag_of[pv];
        myw = psw[pv];
      } else {
        bag = pv;
      }
      const int64_t br = bag - bag_lo;
      myb = (br >= 0 && br < B) ? static_cast<int32_t>(br) : -1;
    }
    for (int q0 = 0; q0 < nb; q0 += UNROLL) {
      float v[UNROLL][NP][4];
      float wq[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int q = q0 + u;
        const int b = __shfl(myb, q, LPR);
        wq[u] = WEIGHTED ? __shfl(myw, q, LPR) : 1.f;
        const bool ok = q < nb && b >= 0;
        const float* grow = grad_out + static_cast<int64_t>(b) * out_width + m.col_base;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (ok && act[p]) {
            const f32x4 x = load_f4(grow + p * 4 * LPR + c * 4);
            v[u][p][0] = x.x; v[u][p][1] = x.y; v[u][p][2] = x.z; v[u][p][3] = x.w;
          } else {
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) v[u][p][q2] = 0.f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            if constexpr (WEIGHTED) acc[p][q2] += wq[u] * v[u][p][q2];
            else acc[p][q2] += v[u][p][q2];
          }
    }
  }
  if constexpr (OPT == kOptSGD) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) w[p][q] -= lr * acc[p][q];
  } else {
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) ss += act[p] ? acc[p][q] * acc[p][q] : 0.f;
#pragma unroll
    for (int msk = 1; msk < LPR; msk <<= 1) ss += __shfl_xor(ss, msk);
    const float mnew = mom + ss / static_cast<float>(D);
    const float denom = sqrtf(mnew) + eps;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) w[p][q] -= lr * acc[p][q] / denom;
    if (c == 0) store_pol<true>(momentum + key, mnew);  // written once, not read back here
  }
#pragma unroll
  for (int p = 0; p < NP; ++p)
    if (act[p]) store_vec4<DT, true>(wrow + p * 4 * LPR + c * 4, w[p]);
}

constexpr int kShortGrab = 16;  // wave steps a short-run wave takes from the shared counter at once

// Short runs of one D bucket, list[0 .. n).  A wave step takes 2 x RPW_S consecutive runs.
// When every run of the step has at most `tiny` lookups, each is served by LPR_T = LPR_S / 2
// lanes holding NPT = 2 float4 chunks a lane, all of them at once (twice the runs in flight:
// such runs wait on memory, not on bandwidth); otherwise the step runs as two halves of
// RPW_S runs with LPR_S lanes each.  Rows wider than 256 columns or narrower than 64 have
// one mode only (NPT == NPS).
// SHARED > 0: the wave steps come from the counter `work` (kShortGrab at a time), which other
// launches share (1: the first grid, 2: a second one, the same code under its own name, so that
// profiles time the two apart); 0: wave w takes steps w, w + waves, ...
template <int DT, int BD, int NPS, int NPT, int OPT, bool WEIGHTED, int US, int UT, int SHARED>
__global__ __launch_bounds__(kBlock) void short_run_kernel(
    typename Fmt<DT>::S* __restrict__ W, float* __restrict__ momentum,
    const float* __restrict__ grad_out, const uint32_t* __restrict__ pay,
    const uint32_t* __restrict__ bag_of, const float* __restrict__ psw,
    const uint4* __restrict__ list, const int32_t* __restrict__ count_ptr, int64_t cap, int tiny,
    const int64_t* __restrict__ meta, int32_t B, int32_t out_width, float lr, float eps,
    int32_t* __restrict__ work) {
  constexpr int LPR_S = BD / (4 * NPS), LPR_T = BD / (4 * NPT);  // lanes per run
  constexpr int RPW_S = kWave / LPR_S;                            // runs per half step
  static_assert(LPR_S >= 1 && LPR_S <= kWave && (LPR_S & (LPR_S - 1)) == 0, "lanes per run");
  static_assert(NPT == NPS || LPR_T * 2 == LPR_S, "tiny steps halve the lanes per run");
  const int lane = lane_id();
  const int64_t n = min(static_cast<int64_t>(*count_ptr), cap);
  // one wave step: runs [i0, i0 + 2 RPW_S)
  auto step = [&](int64_t i0) {
    if constexpr (NPT != NPS) {
      const int64_t it = i0 + lane / LPR_T;
      const uint4 dsc = it < n ? list[it] : make_uint4(0u, 0u, 0u, 0u);
      if (__ballot(it < n && dsc.z > static_cast<uint32_t>(tiny)) == 0) {
        if (it < n)
          short_run_one<DT, NPT, LPR_T, OPT, WEIGHTED, UT>(W, momentum, grad_out, pay, bag_of, psw, dsc,
                                                           lane % LPR_T, meta, B, out_width, lr, eps);
        return;
      }
    }
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      const int64_t i = i0 + h * RPW_S + lane / LPR_S;
      if (i < n)
        short_run_one<DT, NPS, LPR_S, OPT, WEIGHTED, US>(W, momentum, grad_out, pay, bag_of, psw, list[i],
                                                         lane % LPR_S, meta, B, out_width, lr, eps);
    }
  };
  if constexpr (SHARED > 0) {
    // steps taken from the shared counter, kShortGrab at a time, until every step is taken (by
    // this grid or by another launch that shares the counter); each run is still served by
    // exactly one wave, in the same way, so the result does not depend on which
    const int64_t nsteps = (n + 2 * RPW_S - 1) / (2 * RPW_S);
    for (;;) {
      int32_t g0 = 0;
      if (lane == 0) g0 = atomicAdd(work, kShortGrab);
      g0 = __shfl(g0, 0);
      if (g0 >= nsteps) break;
      const int64_t g1 = min(static_cast<int64_t>(g0) + kShortGrab, nsteps);
      for (int64_t g = g0; g < g1; ++g) step(g * 2 * RPW_S);
    }
  } else {
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
    for (int64_t i0 = wave * 2 * RPW_S; i0 < n; i0 += nwaves * 2 * RPW_S) step(i0);
  }
}

// Sums the gradient rows of lookups [lo, hi) of one long run (table t) into
// dst[0 .. D).  One wave: lanes form groups of D/4 (at most 64) lanes; each group
// reads one gradient row per instruction as float4 per lane, UNROLL
// instructions in flight; the groups' sums are combined with xor shuffles.
template <bool WEIGHTED, int UNROLL>
__device__ __forceinline__ void accumulate_chunk(const float* __restrict__ grad_out,
                                                 const uint32_t* __restrict__ pay,
                                                 const uint32_t* __restrict__ bag_of,
                                                 const float* __restrict__ psw, const TableMeta& m,
                                                 int t, int32_t B, int32_t out_width, uint32_t lo,
                                                 uint32_t hi, float* __restrict__ dst) {
  const int lane = lane_id();
  const int D = static_cast<int>(m.D);
  const int64_t bag_lo = static_cast<int64_t>(t) * B;
  for (int cb = 0; cb < D; cb += 4 * kWave) {
    const int wcols = min(D - cb, 4 * kWave);
    const int lpr = pow2_ceil(wcols / 4);
    const int lg = __builtin_ctz(lpr);
    const int G = kWave >> lg;
    const int g = lane >> lg;
    const int cc = lane & (lpr - 1);
    const int col = cb + cc * 4;
    const bool act = cc * 4 < wcols;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t j0 = lo; j0 < hi; j0 += kWave) {
      const int nb = static_cast<int>(min<uint32_t>(kWave, hi - j0));
      int32_t myb = -1;
      float myw = 1.f;
      if (lane < nb) {
        const uint32_t pv = pay[j0 + lane];
        int64_t bag;
        if constexpr (WEIGHTED) {
          bag = bag_of[pv];
          myw = psw[pv];
        } else {
          bag = pv;
        }
        const int64_t br = bag - bag_lo;
        myb = (br >= 0 && br < B) ? static_cast<int32_t>(br) : -1;
      }
      for (int q0 = 0; q0 < nb; q0 += G * UNROLL) {
        f32x4 v[UNROLL];
        float wq[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int q = q0 + u * G + g;
          const int b = __shfl(myb, q & (kWave - 1));
          wq[u] = WEIGHTED ? __shfl(myw, q & (kWave - 1)) : 1.f;
          if (q < nb && b >= 0 && act)
            v[u] = load_f4(grad_out + static_cast<int64_t>(b) * out_width + m.col_base + col);
          else
            v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          if constexpr (WEIGHTED) acc += wq[u] * v[u];
          else acc += v[u];
        }
      }
    }
    for (int msk = lpr; msk < kWave; msk <<= 1) {
      acc.x += __shfl_xor(acc.x, msk);
      acc.y += __shfl_xor(acc.y, msk);
      acc.z += __shfl_xor(acc.z, msk);
      acc.w += __shfl_xor(acc.w, msk);
    }
    if (g == 0 && act) store_f4(dst + col, acc);
  }
}

// Fused long runs (blog section 4, problem 5: fence, then countdown): chunks write
// their partial rows, a device-scope fence makes them visible, then each run's
// countdown (initialised to its chunk count) is decremented; the wave that takes
// a run's count to zero sums all of its partials in chunk order and applies the
// optimizer in the same launch.  No wave ever waits for another.  On gfx950 a
// device-scope release writes back the XCD's L2, so a wave fences once per batch
// of kFusedBatch chunks rather than once per chunk.
constexpr int kFusedBatch = 16;

template <int DT, int OPT>
__device__ __forceinline__ void apply_long_run(typename Fmt<DT>::S* __restrict__ W,
                                               float* __restrict__ momentum, const uint4& L,
                                               const TableMeta& m, int chunk, int max_D,
                                               const float* __restrict__ partial, float lr,
                                               float eps) {
  using S = typename Fmt<DT>::S;
  constexpr int NP = TBE_MAX_D / (4 * kWave);  // column blocks of 256
  const int lane = lane_id();
  const int D = static_cast<int>(m.D);
  const uint32_t nch = (L.z + chunk - 1) / chunk;
  const int64_t cb = L.w;
  f32x4 g[NP];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    g[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int col = p * 4 * kWave + 4 * lane;
    if (col < D) {
      for (uint32_t k = 0; k < nch; ++k) g[p] += load_f4(partial + (cb + k) * max_D + col);
      ss += g[p].x * g[p].x + g[p].y * g[p].y + g[p].z * g[p].z + g[p].w * g[p].w;
    }
  }
  S* wrow = W + m.w_base + (static_cast<int64_t>(L.x) - m.row_base) * D;
  float denom = 1.f;  // SGD: w - lr * g; Adagrad: w - lr * g / (sqrt(m) + eps)
  if constexpr (OPT == kOptAdagrad) {
    for (int msk = 1; msk < kWave; msk <<= 1) ss += __shfl_xor(ss, msk);
    const float mnew = momentum[L.x] + ss / static_cast<float>(D);
    if (lane == 0) momentum[L.x] = mnew;
    denom = sqrtf(mnew) + eps;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int col = p * 4 * kWave + 4 * lane;
    if (col < D) {
      float wv[4];
      load_vec<DT, 4>(wrow + col, wv);
      if constexpr (OPT == kOptAdagrad) {
        wv[0] -= lr * g[p].x / denom; wv[1] -= lr * g[p].y / denom;
        wv[2] -= lr * g[p].z / denom; wv[3] -= lr * g[p].w / denom;
      } else {
        wv[0] -= lr * g[p].x; wv[1] -= lr * g[p].y; wv[2] -= lr * g[p].z; wv[3] -= lr * g[p].w;
      }
      store_vec4<DT>(wrow + col, wv);
    }
  }
}

template <int DT, int OPT, bool WEIGHTED>
__global__ __launch_bounds__(kBlock) void long_fused_kernel(
    typename Fmt<DT>::S* __restrict__ W, float* __restrict__ momentum,
    const float* __restrict__ grad_out, const uint32_t* __restrict__ pay,
    const uint32_t* __restrict__ bag_of, const float* __restrict__ psw,
    const uint4* __restrict__ long_list, const uint32_t* __restrict__ long_table,
    uint32_t* __restrict__ countdown, const uint2* __restrict__ chunk_list,
    const uint32_t* __restrict__ order, const int32_t* __restrict__ counters,
    const int64_t* __restrict__ meta, int32_t B, int32_t out_width, int chunk, int max_D,
    float* __restrict__ partial, float lr, float eps) {
  const int lane = lane_id();
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kBlock) >> 6;
  const int64_t n = counters[kChunks];
  for (int64_t i0 = wave * kFusedBatch; i0 < n; i0 += nwaves * kFusedBatch) {
    const int nb = static_cast<int>(min<int64_t>(kFusedBatch, n - i0));
    uint32_t my_run = 0;  // lane j < nb: long-run slot of the batch's j-th chunk
    for (int j = 0; j < nb; ++j) {
      const int64_t cix = order ? order[i0 + j] : i0 + j;
      const uint2 ch = chunk_list[cix];
      const uint4 L = long_list[ch.x];
      const int t = static_cast<int>(long_table[ch.x]);
      const TableMeta m = load_meta(meta, t);
      const uint32_t lo = L.y + ch.y * static_cast<uint32_t>(chunk);
      const uint32_t hi = min(lo + static_cast<uint32_t>(chunk), L.y + L.z);
      accumulate_chunk<WEIGHTED, 2>(grad_out, pay, bag_of, psw, m, t, B, out_width, lo, hi,
                                    partial + cix * max_D);
      if (lane == j) my_run = ch.x;
    }
    __threadfence();  // this batch's partials are visible device-wide before its countdowns
    uint32_t left = 0;
    if (lane < nb) left = atomicSub(&countdown[my_run], 1u);
    uint64_t last = __ballot(lane < nb && left == 1u);
    if (!last) continue;
    __threadfence();  // the other chunks' partials of those runs are visible to this wave
    while (last) {
      const int j = __ffsll(static_cast<long long>(last)) - 1;
      last &= last - 1;
      const uint32_t li = __shfl(my_run, j);
      const uint4 L = long_list[li];
      const TableMeta m = load_meta(meta, static_cast<int>(long_table[li]));
      apply_long_run<DT, OPT>(W, momentum, L, m, chunk, max_D, partial, lr, eps);
    }
  }
}

// One workgroup per long run: the four waves sum interleaved chunk partials
// (chunk k goes to wave k % 4, always in increasing k), the four sums are added
// in wave order, and the optimizer is applied by all 256 threads, 4 columns each.
template <int DT, int OPT>
__global__ __launch_bounds__(kBlock) void long_apply_kernel(
    typename Fmt<DT>::S* __restrict__ W, float* __restrict__ momentum,
    const uint4* __restrict__ long_list, const uint32_t* __restrict__ long_table,
    const int32_t* __restrict__ counters, const int64_t* __restrict__ meta, int chunk, int max_D,
    const float* __restrict__ partial, const uint32_t* __restrict__ long_flag, float lr, float eps) {
  using S = typename Fmt<DT>::S;
  __shared__ __align__(16) float s_red[kWavesPerBlock][TBE_MAX_D];
  __shared__ float s_tmp[kWavesPerBlock];
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int64_t n = counters[kLong];
  for (int64_t li = blockIdx.x; li < n; li += gridDim.x) {
    if (long_flag && long_flag[li]) continue;  // a dense row: updated by the dense path
    const uint4 L = long_list[li];
    const int t = static_cast<int>(long_table[li]);
    const TableMeta m = load_meta(meta, t);
    const int D = static_cast<int>(m.D);
    const uint32_t nch = (L.z + chunk - 1) / chunk;
    const int64_t cb = L.w;
    for (int col = 4 * lane; col < D; col += 4 * kWave) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      for (uint32_t k = w; k < nch; k += kWavesPerBlock) a += load_f4(partial + (cb + k) * max_D + col);
      *reinterpret_cast<f32x4*>(&s_red[w][col]) = a;
    }
    __syncthreads();
    const int col = 4 * threadIdx.x;
    const bool act = col < D;
    float gv[4] = {0.f, 0.f, 0.f, 0.f};
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
    S* wrow = W + m.w_base + (static_cast<int64_t>(L.x) - m.row_base) * D;
    if (act) {
      load_vec<DT, 4>(wrow + col, wv);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        gv[q] = ((s_red[0][col + q] + s_red[1][col + q]) + s_red[2][col + q]) + s_red[3][col + q];
    }
    if constexpr (OPT == kOptSGD) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[q] -= lr * gv[q];
    } else {
      float ss = gv[0] * gv[0] + gv[1] * gv[1] + gv[2] * gv[2] + gv[3] * gv[3];
      for (int msk = 1; msk < kWave; msk <<= 1) ss += __shfl_xor(ss, msk);
      if (lane == 0) s_tmp[w] = ss;
      __syncthreads();
      ss = ((s_tmp[0] + s_tmp[1]) + s_tmp[2]) + s_tmp[3];
      const float mnew = momentum[L.x] + ss / static_cast<float>(D);
      const float denom = sqrtf(mnew) + eps;
#pragma unroll
      for (int q = 0; q < 4; ++q) wv[q] -= lr * gv[q] / denom;
      __syncthreads();
      if (threadIdx.x == 0) momentum[L.x] = mnew;
    }
    if (act) store_vec4<DT>(wrow + col, wv);
    __syncthreads();
  }
}

// launchers per weight format (backward_f32/f16/bf16.hip)
template <int DT>
tbe_status launch_short_and_apply(const tbe_tables* tb, void* W, float* momentum, int opt,
                                  const float* psw, const float* grad_out, float lr, float eps,
                                  char* ws, const BwdLayout& L, int final_buf, const Config& cfg,
                                  hipStream_t s, hipStream_t s_long);

}  // namespace tbe
