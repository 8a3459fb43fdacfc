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

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    T o = __shfl_xor(v, off, MOE_WAVE);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl(static_cast<uint32_t>(v), src, MOE_WAVE);
  uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src, MOE_WAVE);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, MOE_WAVE);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, MOE_WAVE);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Inclusive prefix sum across the wave (lane order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T o = __shfl_up(v, off, MOE_WAVE);
    if (l >= off) v += o;
  }
  return v;
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
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, MOE_WAVE);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32),
                             off, MOE_WAVE);
    v += static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  }
  return v;
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

// Ordered per-key inclusive prefix of item weights inside one workgroup.
// Items idx = 0..n-1 are in sequence order; key(idx) < 0 means "no item".
// On return incl[idx] = sum of w over items j <= idx with the same key, and
// part_row[key] = the block total of that key.  run: LDS [waves * N].
template <class Get>
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
    uint64_t m = peers & lanemask_le();
    const int maxcnt = wave_max(__popcll(m));
    int32_t local = 0;
    for (int c = 0; c < maxcnt; ++c) {  // uniform trip count: all lanes shuffle
      const int j = m ? (__ffsll(static_cast<long long>(m)) - 1) : lane;
      const int32_t v = __shfl(w, j, MOE_WAVE);
      if (m) {
        local += v;
        m &= m - 1;
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
  for (int e = tid; e < N; e += nthr) {
    int32_t acc = 0;
    for (int v = 0; v < W; ++v) {
      const int32_t t = run[v * N + e];
      run[v * N + e] = acc;
      acc += t;
    }
    part_row[e] = acc;
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
      for (int g = 0; g < G; ++g) {
        const int32_t p = lds[g * ec + c];
        if (excl) excl[static_cast<size_t>(g) * N + e0 + c] = acc;
        acc += p;
      }
      if (tot) tot[e0 + c] = acc;
    }
    __syncthreads();
  }
}

}  // namespace moe
