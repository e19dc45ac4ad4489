// Device-side helpers shared by the TBE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage formats: 0 = fp32, 1 = fp16, 2 = bf16 (matches tbe_dtype)
// ---------------------------------------------------------------------------
template <int DT> struct Fmt;

template <> struct Fmt<0> {
  using S = float;
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};

template <> struct Fmt<1> {
  using S = uint16_t;
  static __device__ __forceinline__ float to_f(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
  }
  // fp32 -> fp16, round to nearest even (v_cvt_f16_f32 in the default mode)
  static __device__ __forceinline__ uint16_t from_f(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
};

template <> struct Fmt<2> {
  using S = uint16_t;
  static __device__ __forceinline__ float to_f(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  // fp32 -> bf16, round to nearest even on the bit pattern; NaN stays NaN
  static __device__ __forceinline__ uint16_t from_f(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Loads VEC consecutive elements of format DT at p (aligned to the vector size); NT: with the
// streaming cache policy, for data read once (the short runs' weight rows and state: uniform
// batch short_run 4.13 -> 4.08 ms).
template <int DT, int VEC, bool NT = false>
__device__ __forceinline__ void load_vec(const typename Fmt<DT>::S* p, float (&v)[VEC]) {
  if constexpr (DT == 0) {
    static_assert(VEC % 4 == 0, "fp32 vectors are float4 based");
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      f32x4 x;
      if constexpr (NT) x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
      else x = *reinterpret_cast<const f32x4*>(p + i);
      v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
    }
  } else if constexpr (VEC == 4) {
    u32x2 x;
    if constexpr (NT) x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    else x = *reinterpret_cast<const u32x2*>(p);
    v[0] = Fmt<DT>::to_f(static_cast<uint16_t>(x.x));
    v[1] = Fmt<DT>::to_f(static_cast<uint16_t>(x.x >> 16));
    v[2] = Fmt<DT>::to_f(static_cast<uint16_t>(x.y));
    v[3] = Fmt<DT>::to_f(static_cast<uint16_t>(x.y >> 16));
  } else {
    static_assert(VEC % 8 == 0, "16-bit vectors are 4 or 8k wide");
#pragma unroll
    for (int i = 0; i < VEC; i += 8) {
      u32x4 x = *reinterpret_cast<const u32x4*>(p + i);
      v[i + 0] = Fmt<DT>::to_f(static_cast<uint16_t>(x.x));
      v[i + 1] = Fmt<DT>::to_f(static_cast<uint16_t>(x.x >> 16));
      v[i + 2] = Fmt<DT>::to_f(static_cast<uint16_t>(x.y));
      v[i + 3] = Fmt<DT>::to_f(static_cast<uint16_t>(x.y >> 16));
      v[i + 4] = Fmt<DT>::to_f(static_cast<uint16_t>(x.z));
      v[i + 5] = Fmt<DT>::to_f(static_cast<uint16_t>(x.z >> 16));
      v[i + 6] = Fmt<DT>::to_f(static_cast<uint16_t>(x.w));
      v[i + 7] = Fmt<DT>::to_f(static_cast<uint16_t>(x.w >> 16));
    }
  }
}

// VEC elements of format DT kept as loaded (32-bit words), so that rows in
// flight cost VEC*sizeof(S)/4 registers rather than VEC.
template <int DT, int VEC>
struct RawVec {
  static constexpr int kWords = VEC * static_cast<int>(sizeof(typename Fmt<DT>::S)) / 4;
  uint32_t w[kWords];
};

template <int DT, int VEC>
__device__ __forceinline__ void load_raw(const typename Fmt<DT>::S* p, RawVec<DT, VEC>& r) {
  constexpr int W = RawVec<DT, VEC>::kWords;
  if constexpr (W == 2) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    r.w[0] = x.x; r.w[1] = x.y;
  } else {
    static_assert(W % 4 == 0, "vectors of 8 or 16k bytes");
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint32_t*>(p) + i);
      r.w[i] = x.x; r.w[i + 1] = x.y; r.w[i + 2] = x.z; r.w[i + 3] = x.w;
    }
  }
}

template <int DT, int VEC>
__device__ __forceinline__ void zero_raw(RawVec<DT, VEC>& r) {
#pragma unroll
  for (int i = 0; i < RawVec<DT, VEC>::kWords; ++i) r.w[i] = 0u;
}

template <int DT, int VEC>
__device__ __forceinline__ void unpack_raw(const RawVec<DT, VEC>& r, float (&v)[VEC]) {
  if constexpr (DT == 0) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __uint_as_float(r.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      v[2 * i] = Fmt<DT>::to_f(static_cast<uint16_t>(r.w[i]));
      v[2 * i + 1] = Fmt<DT>::to_f(static_cast<uint16_t>(r.w[i] >> 16));
    }
  }
}

// Stores 4 floats rounded to format DT at p (aligned to the vector size).
template <int DT, bool NT = false>
__device__ __forceinline__ void store_vec4(typename Fmt<DT>::S* p, const float (&v)[4]) {
  if constexpr (DT == 0) {
    f32x4 x = {v[0], v[1], v[2], v[3]};
    if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = x;
  } else {
    u32x2 x;
    x.x = static_cast<uint32_t>(Fmt<DT>::from_f(v[0])) |
          (static_cast<uint32_t>(Fmt<DT>::from_f(v[1])) << 16);
    x.y = static_cast<uint32_t>(Fmt<DT>::from_f(v[2])) |
          (static_cast<uint32_t>(Fmt<DT>::from_f(v[3])) << 16);
    if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(p));
    else *reinterpret_cast<u32x2*>(p) = x;
  }
}

__device__ __forceinline__ f32x4 load_f4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void store_f4(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
// A store with the streaming (non-temporal) cache policy, for data that nothing reads back
// soon: it does not displace lines the kernel re-reads (the pooling's weight rows: skewed
// batch fwd_gather 2.45 -> 2.39 ms; the short runs' gradient rows: short_run 3.50 ->
// 3.47 ms).  Not for scattered partial-line writes, which then reach memory unmerged (radix
// downsweep 1.04 -> 1.65 ms).
__device__ __forceinline__ void store_f4_stream(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
template <bool NT, typename T>
__device__ __forceinline__ void store_pol(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// value of a wave-uniform expression held in lane `src` (src uniform)
__device__ __forceinline__ int32_t read_lane(int32_t v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ int64_t read_lane64(int64_t v, int src) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32);
  lo = __builtin_amdgcn_readlane(lo, src);
  hi = __builtin_amdgcn_readlane(hi, src);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// smallest power of two >= x (x >= 1, x <= 2^30)
__host__ __device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Table metadata row t: {row base, weight base, column base, D}
struct TableMeta {
  int64_t row_base, w_base, col_base, D, E;
};
__device__ __forceinline__ TableMeta load_meta(const int64_t* __restrict__ meta, int t) {
  TableMeta m;
  m.row_base = meta[4 * t + 0];
  m.w_base = meta[4 * t + 1];
  m.col_base = meta[4 * t + 2];
  m.D = meta[4 * t + 3];
  m.E = meta[4 * (t + 1) + 0] - m.row_base;
  return m;
}

// table owning linearized row `key`: largest t with row_base[t] <= key (T >= 1)
__device__ __forceinline__ int table_of_key(const int64_t* __restrict__ meta, int T, uint32_t key) {
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (meta[4 * mid] <= static_cast<int64_t>(key)) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The key set of the dense rows: open addressing with linear probing over a power-of-two
// array of 16-byte records, each three key slots (kHotEmpty marks a free one) and a word
// holding their keys' ranks among their tables' dense rows (byte j for slot j), so that one
// load answers a probe: a lookup reads whole records (one, nearly always) and stops at the
// first record with a free slot; a 65536-bit filter turns most other keys away first.  Both
// hashes are multiplicative (Knuth's golden-ratio constant and a second odd multiplier).
constexpr uint32_t kHotEmpty = 0xffffffffu;
constexpr int kHotSlotsPerRecord = 3;
// A lookup's dense slot: bits 0-7 the rank of its row among its table's dense rows (0xff:
// none), bits 8-11 its bag's index within the table modulo 16
constexpr uint16_t kNoDenseSlot = 0x00ff;
__device__ __forceinline__ uint32_t hot_slot(uint32_t key, uint32_t mask) {
  const uint32_t h = key * 0x9e3779b1u;
  return ((h ^ (h >> 15)) << 2) & mask;  // first word of a record
}
__device__ __forceinline__ uint32_t hot_filter_bit(uint32_t key) { return (key * 0x85ebca6bu) >> 16; }

// short-run bucket of width D: log2(next_pow2(D)) - 2, for 4 <= D <= 1024
__host__ __device__ __forceinline__ int bucket_of_D(int D) {
  int b = 0, p = 4;
  while (p < D) { p <<= 1; ++b; }
  return b;
}

}  // namespace tbe
