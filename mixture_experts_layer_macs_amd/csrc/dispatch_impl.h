// Stable counting sort of the kept slots into expert-major rows, (token,
// slot) ascending inside each expert: device phases and workspace layout,
// shared by the dispatch kernel and the fused routing kernel.
#pragma once

#include <algorithm>

#include "common.h"

namespace moe {
namespace disp {

struct Args {
  const int32_t* slot;
  int T, N, k, nbits;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* slot_row;
  int32_t* rank;   // [T*k]  1-based rank of the slot inside its block/expert
  int32_t* part;   // [G*N]  per-block per-expert counts
  int32_t* base;   // [G*N]  rows of each expert in earlier blocks
  unsigned* ticket;
  int TB, G, lds_scan;
};

__device__ void count_block(const Args& a, int g, int t0, int t1,
                            int32_t* run) {
  const int k = a.k;
  const int32_t* slot = a.slot + static_cast<size_t>(t0) * k;
  key_prefix<true>((t1 - t0) * k, a.N, a.nbits, run,
             [&](int idx, int& key, int32_t& w) {
               key = slot[idx];
               w = 1;
             },
             a.rank + static_cast<size_t>(t0) * k,
             a.part + static_cast<size_t>(g) * a.N, nullptr);
}

// Expert offsets = exclusive scan of the per-expert totals; per-block bases
// (exclusive prefix over the blocks, without the expert offset).
__device__ void scan_offsets(const Args& a, int32_t* tot, int32_t* stage) {
  const int tid = threadIdx.x, nthr = blockDim.x, N = a.N, G = a.G;
  if (G == 1) {
    for (int e = tid; e < N; e += nthr) {
      tot[e] = a.part[e];
      a.base[e] = 0;
    }
  } else {
    column_scan<int32_t>(a.part, a.base, tot, G, N, stage, a.lds_scan);
  }
  // block scan over the N totals in chunks of blockDim, carried between
  // chunks: DPP scan inside each wave, then wave 0 scans the wave totals
  __shared__ int32_t wsum[16];
  __shared__ int32_t wexcl[17];
  int32_t carry = 0;
  const int W = nthr / MOE_WAVE, wave = tid / MOE_WAVE, lane = lane_id();
  __syncthreads();  // tot complete
  for (int c0 = 0; c0 < N; c0 += nthr) {
    const int e = c0 + tid;
    const int32_t v = e < N ? tot[e] : 0;
    const int32_t inc = wave_incl_scan(v);
    if (lane == MOE_WAVE - 1) wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
      const int32_t x = lane < W ? wsum[lane] : 0;
      const int32_t xi = wave_incl_scan(x);
      if (lane < W) wexcl[lane] = xi - x;
      if (lane == MOE_WAVE - 1) wexcl[16] = xi;
    }
    __syncthreads();
    const int32_t pre = carry + wexcl[wave];
    if (e < N) a.offsets[e] = pre + inc - v;  // exclusive
    if (e == N - 1) a.offsets[N] = pre + inc;
    carry += wexcl[16];
    __syncthreads();
  }
}

__device__ void scatter_block(const Args& a, int g, int t0, int t1) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k, N = a.N;
  const int32_t* base = a.base + static_cast<size_t>(g) * N;
  for (int i = t0 * k + tid; i < t1 * k; i += nthr) {
    const int e = a.slot[i];
    if (e < 0) {
      a.slot_row[i] = -1;
      continue;
    }
    const int row = a.offsets[e] + base[e] + a.rank[i] - 1;
    a.slot_row[i] = row;
    a.row_token[row] = i / k;
    a.row_slot[row] = i % k;
  }
}

// Whole batch in one workgroup (G == 1): count, offsets and scatter.
__device__ void dispatch_single(const Args& a, unsigned char* smem) {
  int32_t* tot = reinterpret_cast<int32_t*>(smem);
  int32_t* run = tot + a.N;
  count_block(a, 0, 0, a.T, run);
  scan_offsets(a, tot, run);
  __syncthreads();
  scatter_block(a, 0, 0, a.T);
}

struct Layout {
  int G, TB, threads;
  size_t ticket, rank, part, base, bytes;
};

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout layout(int T, int N, int k) {
  Layout L{};
  const long items = static_cast<long>(T) * k;
  if (items <= 4096) {
    L.G = 1;
    L.TB = T > 0 ? T : 1;
    L.threads = 1024;
  } else {
    L.TB = k >= 1024 ? 1 : 1024 / k;
    L.G = (T + L.TB - 1) / L.TB;
    L.threads = 256;
  }
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o = align_up(o + n);
    return at;
  };
  const size_t GN = static_cast<size_t>(L.G) * N;
  L.ticket = take(sizeof(unsigned));
  L.rank = take(sizeof(int32_t) * static_cast<size_t>(T) * k);
  L.part = take(sizeof(int32_t) * GN);
  L.base = take(sizeof(int32_t) * GN);
  L.bytes = o;
  return L;
}


inline Args make_args(const int32_t* slot_expert, int T, int N, int k,
                      int32_t* expert_offsets, int32_t* row_token,
                      int32_t* row_slot, int32_t* slot_row, char* ws,
                      const Layout& L) {
  Args a{};
  a.slot = slot_expert;
  a.T = T;
  a.N = N;
  a.k = k;
  int nb = 1;
  while ((1 << nb) < N) ++nb;
  a.nbits = nb;
  a.offsets = expert_offsets;
  a.row_token = row_token;
  a.row_slot = row_slot;
  a.slot_row = slot_row;
  a.rank = reinterpret_cast<int32_t*>(ws + L.rank);
  a.part = reinterpret_cast<int32_t*>(ws + L.part);
  a.base = reinterpret_cast<int32_t*>(ws + L.base);
  a.ticket = reinterpret_cast<unsigned*>(ws + L.ticket);
  a.TB = L.TB;
  a.G = L.G;
  a.lds_scan = std::max((L.threads / MOE_WAVE) * N, 8192);
  return a;
}

// Dynamic LDS: [tot: N int32][run table / scan staging: lds_scan int32].
inline size_t lds_bytes(const Args& a) { return sizeof(int32_t) * (a.N + a.lds_scan); }
}  // namespace disp
}  // namespace moe
