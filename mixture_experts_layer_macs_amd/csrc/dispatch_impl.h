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

__device__ void exclusive_offsets(const int32_t* tot, int N, int32_t* dst);

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
  __syncthreads();  // tot complete
  exclusive_offsets(tot, N, a.offsets);
}

// dst[e] = sum of tot[0 .. e-1] for e <= N (dst may be global or LDS): a
// block scan over the N totals in chunks of blockDim, carried between
// chunks; DPP scan inside each wave, then wave 0 scans the wave totals.
// tot must be complete (a barrier) before the call.
__device__ void exclusive_offsets(const int32_t* tot, int N, int32_t* dst) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  __shared__ int32_t wsum[16];
  __shared__ int32_t wexcl[17];
  int32_t carry = 0;
  const int W = nthr / MOE_WAVE, wave = tid / MOE_WAVE, lane = lane_id();
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
    if (e < N) dst[e] = pre + inc - v;  // exclusive
    if (e == N - 1) dst[N] = pre + inc;
    carry += wexcl[16];
    __syncthreads();
  }
}

// offsets: the expert offsets; base: this block's rows of each expert in
// earlier blocks (both [N], global or LDS); the first skip slots of the
// block are left out.
__device__ void scatter_block(const Args& a, int t0, int t1, const int32_t* offsets,
                              const int32_t* base, int skip = 0) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k;
  for (int i = t0 * k + skip + tid; i < t1 * k; i += nthr) {
    const int e = a.slot[i];
    if (e < 0) {
      a.slot_row[i] = -1;
      continue;
    }
    const int row = offsets[e] + base[e] + a.rank[i] - 1;
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
  scatter_block(a, 0, a.T, a.offsets, a.base);
}

// Blocks of a batch of at most DEC_MAX_G blocks, in the launch after the
// count launch: with no serial step in between, every block sums the
// per-block counts itself, over all blocks (the expert totals, scanned into
// the offsets, which block 0 also writes out) and over the blocks before it
// (its base), then scatters its slots.  With N a multiple of 4, V = N / 4
// threads cover a block's row of counts with 16-byte loads and P groups of
// them split the blocks, so a thread issues up to 16 loads at once; the
// partial sums meet in LDS in a fixed order.
// smem: [tot N][base N][offsets N + 1][partials 2 * P * N] int32.
constexpr int DEC_MAX_G = 128;
__device__ void scatter_dec(const Args& a, int g, unsigned char* smem) {
  const int tid = threadIdx.x, nthr = blockDim.x, N = a.N, G = a.G, k = a.k;
  int32_t* tot = reinterpret_cast<int32_t*>(smem);
  int32_t* bse = tot + N;
  int32_t* off = bse + N;
  int32_t* red = off + N + 1;
  // the block's slots and ranks are read first, so their latency overlaps
  // the sums (a block has at most 1024 slots: PF per thread)
  constexpr int PF = 4;
  const int t0 = g * a.TB, t1 = min(a.T, t0 + a.TB);
  const int i0 = t0 * k + tid, i1 = t1 * k;
  int32_t pe[PF], pr[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int i = i0 + u * nthr;
    pe[u] = i < i1 ? a.slot[i] : -1;
    pr[u] = i < i1 ? a.rank[i] : 0;
  }
  if ((N & 3) == 0 && N / 4 <= nthr) {
    const int V = N / 4, P = max(1, min(nthr / V, G));
    const int v = tid % V, q = tid / V;
    if (q < P) {
      int32_t before[4] = {0, 0, 0, 0}, all[4] = {0, 0, 0, 0};
      for (int b0 = q; b0 < G; b0 += 16 * P) {
        int4 x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int b = b0 + u * P;
          x[u] = b < G ? *reinterpret_cast<const int4*>(a.part + static_cast<size_t>(b) * N + 4 * v)
                       : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          all[0] += x[u].x;
          all[1] += x[u].y;
          all[2] += x[u].z;
          all[3] += x[u].w;
          if (b0 + u * P < g) {
            before[0] += x[u].x;
            before[1] += x[u].y;
            before[2] += x[u].z;
            before[3] += x[u].w;
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        red[q * N + 4 * v + c] = before[c];
        red[(P + q) * N + 4 * v + c] = all[c];
      }
    }
    __syncthreads();
    for (int e = tid; e < N; e += nthr) {
      int32_t b = red[e], t = red[P * N + e];
      for (int p = 1; p < P; ++p) {
        b += red[p * N + e];
        t += red[(P + p) * N + e];
      }
      bse[e] = b;
      tot[e] = t;
    }
  } else {
    for (int e = tid; e < N; e += nthr) {
      int32_t b = 0, t = 0;
      for (int blk = 0; blk < G; ++blk) {
        const int32_t x = a.part[static_cast<size_t>(blk) * N + e];
        t += x;
        if (blk < g) b += x;
      }
      bse[e] = b;
      tot[e] = t;
    }
  }
  __syncthreads();
  exclusive_offsets(tot, N, off);
  __syncthreads();
  if (g == 0)
    for (int e = tid; e <= N; e += nthr) a.offsets[e] = off[e];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int i = i0 + u * nthr;
    if (i >= i1) break;
    const int e = pe[u];
    if (e < 0) {
      a.slot_row[i] = -1;
      continue;
    }
    const int row = off[e] + bse[e] + pr[u] - 1;
    a.slot_row[i] = row;
    a.row_token[row] = i / k;
    a.row_slot[row] = i % k;
  }
  // slots beyond PF per thread (more than PF * blockDim in the block)
  if (i1 - t0 * k > PF * nthr) scatter_block(a, t0, t1, off, bse, PF * nthr);
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
