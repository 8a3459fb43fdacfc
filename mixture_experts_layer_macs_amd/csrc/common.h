// Internal helpers shared by the HIP sources of the MoE-layer library.
// Written for gfx950 (CDNA4): 64-lane wavefronts, 64-bit ballots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_macs.h"

#define MOE_WAVE 64

namespace moe {

// Host side: translate the last launch error into the ABI status.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Index of the current device, or -1 if there is none below 64.
inline int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64 ? dev : -1;
}

// Compute units of the current device (cached per device; 256 if unknown).
inline int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// ----------------------------------------------------------------- device
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t lanemask_le() {
  const int l = lane_id();
  return l == 63 ? ~0ull : ((2ull << l) - 1ull);
}

// ------------------------------------------------ DPP wave primitives
// Cross-lane steps use DPP row operations (a VALU operand modifier, a few
// cycles each) instead of LDS-crossbar shuffles (ds_bpermute, about a
// hundred cycles each), so a full-wave reduction or scan costs six dependent
// VALU steps.  Every lane of the wave must be active.
enum : int {
  DPP_QUAD_1032 = 0xb1,  // lane ^ 1 inside each quad
  DPP_QUAD_2301 = 0x4e,  // lane ^ 2 inside each quad
  DPP_ROW_SHR1 = 0x111,  // lane - n inside each row of 16
  DPP_ROW_SHR2 = 0x112,
  DPP_ROW_SHR4 = 0x114,
  DPP_ROW_SHR8 = 0x118,
  DPP_ROW_HALF_MIRROR = 0x141,  // lane 7-i inside each half-row of 8
  DPP_ROW_BCAST15 = 0x142,  // lane 15 of each row into the next row
  DPP_ROW_BCAST31 = 0x143,  // lane 31 into rows 2 and 3
};

// Value of the DPP source lane; lanes without a source (or outside
// ROW_MASK) get `old`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      static_cast<int>(old), static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp64(uint64_t old, uint64_t v) {
  const uint32_t lo = dpp<CTRL, ROW_MASK>(static_cast<uint32_t>(old),
                                          static_cast<uint32_t>(v));
  const uint32_t hi = dpp<CTRL, ROW_MASK>(static_cast<uint32_t>(old >> 32),
                                          static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t bits_of(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t bits_of(int v) { return static_cast<uint32_t>(v); }
__device__ __forceinline__ uint32_t bits_of(uint32_t v) { return v; }
template <typename T> __device__ __forceinline__ T from_bits(uint32_t b);
template <> __device__ __forceinline__ float from_bits<float>(uint32_t b) { return __uint_as_float(b); }
template <> __device__ __forceinline__ int from_bits<int>(uint32_t b) { return static_cast<int>(b); }
template <> __device__ __forceinline__ uint32_t from_bits<uint32_t>(uint32_t b) { return b; }

template <typename T, int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ T dpp_t(T ident, T v) {
  return from_bits<T>(dpp<CTRL, ROW_MASK>(bits_of(ident), bits_of(v)));
}

// Full-wave reduction; the result (lane 63's total) is returned to every
// lane.  `ident` is the identity of `op`.
template <typename T, class Op>
__device__ __forceinline__ T wave_reduce(T v, T ident, Op op) {
  v = op(v, dpp_t<T, DPP_QUAD_1032>(ident, v));
  v = op(v, dpp_t<T, DPP_QUAD_2301>(ident, v));
  v = op(v, dpp_t<T, DPP_ROW_SHR4>(ident, v));
  v = op(v, dpp_t<T, DPP_ROW_SHR8>(ident, v));
  v = op(v, dpp_t<T, DPP_ROW_BCAST15, 0xa>(ident, v));
  v = op(v, dpp_t<T, DPP_ROW_BCAST31, 0xc>(ident, v));
  return from_bits<T>(static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(bits_of(v)), 63)));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce<T>(v, T(0), [](T a, T b) { return a + b; });
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce<float>(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ int wave_max(int v) {
  return wave_reduce<int>(v, INT32_MIN, [](int a, int b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp64<DPP_QUAD_1032>(0ull, v));
  v = mx(v, dpp64<DPP_QUAD_2301>(0ull, v));
  v = mx(v, dpp64<DPP_ROW_SHR4>(0ull, v));
  v = mx(v, dpp64<DPP_ROW_SHR8>(0ull, v));
  v = mx(v, dpp64<DPP_ROW_BCAST15, 0xa>(0ull, v));
  v = mx(v, dpp64<DPP_ROW_BCAST31, 0xc>(0ull, v));
  return readlane64(v, 63);
}

// Inclusive prefix sum across the wave (lane order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  v = v + dpp_t<T, DPP_ROW_SHR1>(T(0), v);
  v = v + dpp_t<T, DPP_ROW_SHR2>(T(0), v);
  v = v + dpp_t<T, DPP_ROW_SHR4>(T(0), v);
  v = v + dpp_t<T, DPP_ROW_SHR8>(T(0), v);
  v = v + dpp_t<T, DPP_ROW_BCAST15, 0xa>(T(0), v);
  v = v + dpp_t<T, DPP_ROW_BCAST31, 0xc>(T(0), v);
  return v;
}

// Value held by `lane` (wave-uniform lane index).
__device__ __forceinline__ int read_lane(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

// Wait until this wave's global stores have completed (vector memory
// counter at zero; LDS and export counters left alone).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Store visible at agent scope once it completes (written through the
// XCD's L2, which is not coherent with the other XCDs' L2s): a workgroup
// that hands results to a workgroup on another XCD stores them this way and
// waits for its stores, instead of writing back its whole L2.
__device__ __forceinline__ void store_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Monotone unsigned image of an fp32 value: a > b  <=>  key(a) > key(b);
// -0.0 is folded onto +0.0 first so the two compare equal.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key that ranks larger value first, then lower index first, under max().
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
  return (static_cast<uint64_t>(f32_order_key(v)) << 32) |
         static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int rank_key_index(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}

// Lanes of the wave whose `key` equals this lane's key (only lanes with
// valid != 0 take part; invalid lanes get 0).  nbits = bits needed for key.
__device__ __forceinline__ uint64_t match_any(int key, int valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t on = __ballot(valid && bit);
    peers &= bit ? on : ~on;
  }
  return valid ? peers : 0ull;
}

// Inverse of f32_order_key (-0.0 comes back as +0.0).
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float rank_key_value(uint64_t key) {
  return f32_from_order_key(static_cast<uint32_t>(key >> 32));
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
  uint64_t u = static_cast<uint64_t>(v);
  u += dpp64<DPP_QUAD_1032>(0ull, u);
  u += dpp64<DPP_QUAD_2301>(0ull, u);
  u += dpp64<DPP_ROW_SHR4>(0ull, u);
  u += dpp64<DPP_ROW_SHR8>(0ull, u);
  u += dpp64<DPP_ROW_BCAST15, 0xa>(0ull, u);
  u += dpp64<DPP_ROW_BCAST31, 0xc>(0ull, u);
  return static_cast<int64_t>(readlane64(u, 63));
}

// Full-wave sum of doubles in a fixed lane order (deterministic).
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto step = [](double x, uint64_t y) { return x + __longlong_as_double(static_cast<long long>(y)); };
  auto bits = [](double x) { return static_cast<uint64_t>(__double_as_longlong(x)); };
  v = step(v, dpp64<DPP_QUAD_1032>(0ull, bits(v)));
  v = step(v, dpp64<DPP_QUAD_2301>(0ull, bits(v)));
  v = step(v, dpp64<DPP_ROW_SHR4>(0ull, bits(v)));
  v = step(v, dpp64<DPP_ROW_SHR8>(0ull, bits(v)));
  v = step(v, dpp64<DPP_ROW_BCAST15, 0xa>(0ull, bits(v)));
  v = step(v, dpp64<DPP_ROW_BCAST31, 0xc>(0ull, bits(v)));
  return __longlong_as_double(static_cast<long long>(readlane64(bits(v), 63)));
}

// Block-wide sum of one int64 per thread; result valid in every thread.
__device__ inline int64_t block_sum_i64(int64_t v, int64_t* red) {
  const int wave = threadIdx.x / MOE_WAVE, W = blockDim.x / MOE_WAVE;
  v = wave_sum_i64(v);
  __syncthreads();
  if (lane_id() == 0) red[wave] = v;
  __syncthreads();
  int64_t s = 0;
  for (int i = 0; i < W; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Block-wide sums of two int64 values per thread (one set of barriers).
__device__ inline void block_sum2_i64(int64_t& a, int64_t& b, int64_t* red) {
  const int wave = threadIdx.x / MOE_WAVE, W = blockDim.x / MOE_WAVE;
  a = wave_sum_i64(a);
  b = wave_sum_i64(b);
  __syncthreads();
  if (lane_id() == 0) {
    red[wave] = a;
    red[16 + wave] = b;
  }
  __syncthreads();
  int64_t sa = 0, sb = 0;
  for (int i = 0; i < W; ++i) {
    sa += red[i];
    sb += red[16 + i];
  }
  __syncthreads();
  a = sa;
  b = sb;
}

// Exclusive prefix over groups of G consecutive lanes (G a power of two,
// G <= 16, groups aligned to G): returns the sum of v over the lanes of the
// group below this one's position; *total gets the group's sum.
template <int G>
__device__ __forceinline__ int32_t group_excl_scan(int32_t v, int32_t* total) {
  const int pos = lane_id() & (G - 1);
  int32_t x = v;
  if constexpr (G > 1) { const int32_t y = dpp_t<int, DPP_ROW_SHR1>(0, x); x += pos >= 1 ? y : 0; }
  if constexpr (G > 2) { const int32_t y = dpp_t<int, DPP_ROW_SHR2>(0, x); x += pos >= 2 ? y : 0; }
  if constexpr (G > 4) { const int32_t y = dpp_t<int, DPP_ROW_SHR4>(0, x); x += pos >= 4 ? y : 0; }
  if constexpr (G > 8) { const int32_t y = dpp_t<int, DPP_ROW_SHR8>(0, x); x += pos >= 8 ? y : 0; }
  // the group's last lane holds its total
  *total = __shfl(x, (lane_id() | (G - 1)), MOE_WAVE);
  return x - v;
}

// Ordered per-key inclusive prefix of item weights inside one workgroup.
// Items idx = 0..n-1 are in sequence order; key(idx) < 0 means "no item";
// weights lie in [0, 2^16] (token weights in units of 2^-16 token).
// On return incl[idx] = sum of w over items j <= idx with the same key, and
// part_row[key] = the block total of that key.  run: LDS [waves * N].
// UNIT: every item weighs 1, so a lane's in-wave prefix is a popcount.
template <bool UNIT = false, class Get>
__device__ inline void key_prefix(int n, int N, int nbits, int32_t* run, Get get,
                           int32_t* incl, int32_t* part_row,
                           uint32_t* act_bits) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int W = nthr / MOE_WAVE, wave = tid / MOE_WAVE, lane = lane_id();
  for (int i = tid; i < W * N; i += nthr) run[i] = 0;
  __syncthreads();
  const int per = (((n + W - 1) / W) + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
  const int beg = wave * per;
  const int end = min(n, beg + per);
  int32_t* myrun = run + wave * N;
  for (int b = beg; b < end; b += MOE_WAVE) {
    const int idx = b + lane;
    int key = -1;
    int32_t w = 0;
    if (idx < end) get(idx, key, w);
    const int valid = key >= 0;
    const uint64_t peers = match_any(key, valid, nbits);
    const uint64_t m = peers & lanemask_le();
    int32_t local = 0;
    if constexpr (UNIT) {
      local = __popcll(m);
    } else {
      // weighted prefix over the peers at or below this lane, bit plane by
      // bit plane: sum_b 2^b * |{peers j <= lane : bit b of w_j set}|
      // (weights are 0 .. 2^16, so 17 planes; no shuffles, no loops
      // whose length depends on the data)
#pragma unroll
      for (int b = 0; b < 17; ++b) {
        const uint64_t plane = __ballot(valid && ((w >> b) & 1));
        local += static_cast<int32_t>(__popcll(m & plane)) << b;
      }
    }
    if (valid) {
      const int32_t inc = myrun[key] + local;
      incl[idx] = inc;
      if (act_bits) atomicOr(&act_bits[key >> 5], 1u << (key & 31));
      if (lane == 63 - __clzll(static_cast<long long>(peers))) myrun[key] = inc;
    }
  }
  __syncthreads();
  // exclusive scan over the waves of every key: W consecutive lanes per key
  // (W = 4 or 16, a power of two), DPP row shifts inside the lane group
  for (int i = tid; i < W * N; i += nthr) {
    const int e = i / W, v = i % W;
    const int32_t x = run[v * N + e];
    int32_t tot;
    const int32_t ex = W == 16 ? group_excl_scan<16>(x, &tot)
                     : W == 8 ? group_excl_scan<8>(x, &tot)
                     : W == 4 ? group_excl_scan<4>(x, &tot)
                     : W == 2 ? group_excl_scan<2>(x, &tot)
                              : group_excl_scan<1>(x, &tot);
    run[v * N + e] = ex;
    if (v == 0) part_row[e] = tot;
  }
  __syncthreads();
  for (int idx = tid; idx < n; idx += nthr) {
    int key = -1;
    int32_t w = 0;
    get(idx, key, w);
    if (key >= 0) incl[idx] += run[(idx / per) * N + key];
  }
  __syncthreads();
}

// Column-wise exclusive prefix of a [G][N] int32 matrix held in global
// memory (one row per token block): excl[g][e] = sum_{g' < g} in[g'][e],
// column totals to tot[e] (either output may be null).  Columns are staged
// through LDS (lds: lds_elems int32) with batches of independent loads, so
// the cost is a few memory round trips rather than one per block.
template <class OutT>
__device__ void column_scan(const int32_t* in, OutT* excl, OutT* tot, int G,
                            int N, int32_t* lds, int lds_elems) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int EC = max(1, min(N, lds_elems / max(G, 1)));
  for (int e0 = 0; e0 < N; e0 += EC) {
    const int ec = min(EC, N - e0);
    const int n = G * ec;
    for (int i0 = tid; i0 < n; i0 += nthr * 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * nthr;
        v[u] = i < n ? in[static_cast<size_t>(i / ec) * N + e0 + i % ec] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * nthr;
        if (i < n) lds[i] = v[u];
      }
    }
    __syncthreads();
    for (int c = tid; c < ec; c += nthr) {
      OutT acc = 0;
      for (int g0 = 0; g0 < G; g0 += 8) {  // 8 reads in flight per step
        int32_t p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = g0 + u < G ? lds[(g0 + u) * ec + c] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (g0 + u < G) {
            if (excl) excl[static_cast<size_t>(g0 + u) * N + e0 + c] = acc;
            acc += p[u];
          }
        }
      }
      if (tot) tot[e0 + c] = acc;
    }
    __syncthreads();
  }
}

}  // namespace moe
