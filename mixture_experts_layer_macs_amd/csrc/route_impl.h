// Router softmax and top-k for one token ("MACS", §3.1 Eq. 1), shared by the
// stand-alone route kernel and the fused routing kernel.
//
// A group of GT threads (a whole number of waves) owns one token.  Its N
// logits become 64-bit rank keys in LDS (order-preserving image of the fp32
// value, then the inverted expert index, so a larger key means a better rank
// and equal logits fall to the lower index).  The rank of expert e is the
// number of keys above its own, counted directly: every thread compares one
// expert's key against a span of the others (LDS broadcast reads, no
// cross-lane traffic), and the partial counts meet in an LDS atomic.  The
// k + R best ranks are then written straight to their output positions.  No
// step depends on the previous pick, so the latency is a few hundred cycles
// instead of k + R dependent wave-wide reductions.
#pragma once

#include "common.h"

namespace moe {
namespace rt {

// LDS per token group: keys u64[N], ranks i32[N], reduction slots f32[GT/64]
// (rounded up to 16 bytes so consecutive groups stay aligned).
__host__ __device__ constexpr size_t token_lds_bytes(int N, int GT) {
  return (static_cast<size_t>(N) * 12 + static_cast<size_t>(GT / MOE_WAVE) * 4 +
          15) & ~static_cast<size_t>(15);
}

// Reduction over the GT threads of one token group.  Every thread of the
// workgroup must call it (it synchronises the workgroup).
template <int GT, bool MAX>
__device__ __forceinline__ float group_reduce(float v, float* red) {
  v = MAX ? wave_max(v) : wave_sum(v);
  if constexpr (GT > MOE_WAVE) {
    const int wv = (threadIdx.x % GT) / MOE_WAVE;
    if (lane_id() == 0) red[wv] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < GT / MOE_WAVE; ++i) v = MAX ? fmaxf(v, red[i]) : v + red[i];
    __syncthreads();
  }
  return v;
}

// Route token t, whose N logits start at `row` (global memory or LDS;
// live == false: a padding group that only joins the workgroup barriers and
// reads nothing).  Writes topk_ids[t][0..k), topk_gates[t][0..k) and
// fallback_ids[t][0..R) in rank order; the ids with agent-scope stores, so
// that another workgroup of the same launch can read them after a
// hand-off without a write-back of this XCD's L2.
template <int GT>
__device__ void route_token(const float* __restrict__ row, int N, int k,
                            int R, int t, bool live, unsigned char* lds,
                            int32_t* __restrict__ topk_ids,
                            float* __restrict__ topk_gates,
                            int32_t* __restrict__ fallback_ids) {
  uint64_t* key = reinterpret_cast<uint64_t*>(lds);
  int* rank = reinterpret_cast<int*>(lds + static_cast<size_t>(N) * 8);
  float* red = reinterpret_cast<float*>(lds + static_cast<size_t>(N) * 12);
  const int g = threadIdx.x % GT;

  float mx = -INFINITY;
  if (live)
    for (int j = g; j < N; j += GT) {
      const float v = row[j];
      key[j] = rank_key(v, j);
      rank[j] = 0;
      mx = fmaxf(mx, v);
    }
  mx = group_reduce<GT, true>(mx, red);  // exact: the order does not matter
  // The softmax denominator is summed in one fixed order whatever GT is:
  // lane l of the group's first wave adds the experts j = l (mod 64) in
  // increasing j, then the wave tree combines the 64 partial sums.  The
  // gates are therefore the same bits for every group size.  (The keys are
  // visible to the whole group: the max reduction synchronised it.)
  float se = 0.f;
  if (g < MOE_WAVE) {
    if (live)
      for (int j = g; j < N; j += MOE_WAVE) se += expf(rank_key_value(key[j]) - mx);
    se = wave_sum(se);
  }
  if constexpr (GT > MOE_WAVE) {
    if (g == 0) red[0] = se;
    __syncthreads();
    se = red[0];
  } else {
    __syncthreads();  // every key and zeroed rank visible to the whole group
  }

  if (live) {
    if (N <= GT) {
      // S threads per expert, each counting over one span of the keys
      const int S = GT / N;
      const int e = g % N, s = g / N;
      if (s < S) {
        const int span = (N + S - 1) / S;
        const int j0 = s * span, j1 = min(N, j0 + span);
        const uint64_t ke = key[e];
        int c = 0;
#pragma unroll 8
        for (int j = j0; j < j1; ++j) c += key[j] > ke ? 1 : 0;
        if (c) atomicAdd(&rank[e], c);
      }
    } else {
      for (int e = g; e < N; e += GT) {
        const uint64_t ke = key[e];
        int c = 0;
#pragma unroll 8
        for (int j = 0; j < N; ++j) c += key[j] > ke ? 1 : 0;
        rank[e] = c;
      }
    }
  }
  __syncthreads();
  if (live)
    for (int e = g; e < N; e += GT) {
      const int r = rank[e];
      if (r < k) {
        store_agent(&topk_ids[static_cast<size_t>(t) * k + r], e);
        topk_gates[static_cast<size_t>(t) * k + r] =
            expf(rank_key_value(key[e]) - mx) / se;
      } else if (r < k + R) {
        store_agent(&fallback_ids[static_cast<size_t>(t) * R + (r - k)], e);
      }
    }
}

// One wave ranks one token whose N <= 64 * KPL logits start at `row`
// (global memory or LDS), with every key in registers: lane l holds experts
// l, l + 64, ...  The outputs are route_token's, bit for bit (the same max,
// the same softmax denominator order, the same gate expression).
//
//   1. the (k + R)-th largest order key theta is found by a most-significant-
//      bit-first search: bit b is kept iff at least k + R keys are >= the
//      candidate (one ballot per register); the search stops as soon as
//      exactly k + R keys qualify;
//   2. the selected set is every key above theta plus the lowest-index keys
//      equal to theta (ranks of equal logits go to the lower index);
//   3. the selected keys are compacted into `cand` (LDS, k + R entries of
//      this wave's own) and each one's rank is the number of selected keys
//      that beat it.
// A dead token (live == false) returns at once: the wave takes no part in
// any workgroup barrier.  ranked (optional, LDS or global): the k + R ids in
// rank order, for a consumer in the same workgroup.
template <int KPL>
__device__ void route_token_wave(const float* __restrict__ row, int N, int k,
                                 int R, int t, bool live, uint64_t* cand,
                                 int32_t* __restrict__ topk_ids,
                                 float* __restrict__ topk_gates,
                                 int32_t* __restrict__ fallback_ids,
                                 int32_t* ranked = nullptr) {
  if (!live) return;
  const int lane = lane_id();
  const int M = k + R;
  float v[KPL];
  uint32_t u[KPL];
  float mx = -INFINITY;
  // every load issued before the first use (clamped index: a lane past N
  // reads a valid logit and ignores it)
#pragma unroll
  for (int i = 0; i < KPL; ++i) v[i] = row[min(lane + MOE_WAVE * i, N - 1)];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int j = lane + MOE_WAVE * i;
    u[i] = j < N ? f32_order_key(v[i]) : 0u;  // 0: below every finite key
    if (j < N) mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  // softmax denominator: lane l adds its experts in increasing index, then
  // the wave tree -- route_token's order
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    if (lane + MOE_WAVE * i < N) se += expf(f32_from_order_key(u[i]) - mx);
  se = wave_sum(se);

  uint32_t theta = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand_t = theta | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < KPL; ++i) cnt += __popcll(__ballot(u[i] >= cand_t));
    if (cnt >= M) {
      theta = cand_t;
      if (cnt == M) break;
    }
  }
  int above = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) above += __popcll(__ballot(u[i] > theta));
  const int need = M - above;  // keys equal to theta to take, lowest index first
  const uint64_t lt = lanemask_lt();
  int ties = 0, base = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const uint64_t eq = __ballot(u[i] == theta);
    const bool sel = u[i] > theta || (u[i] == theta && ties + __popcll(eq & lt) < need);
    ties += __popcll(eq);
    const uint64_t sb = __ballot(sel);
    if (sel)
      cand[base + __popcll(sb & lt)] =
          (static_cast<uint64_t>(u[i]) << 32) |
          static_cast<uint32_t>(0xffffffffu - static_cast<uint32_t>(lane + MOE_WAVE * i));
    base += __popcll(sb);
  }
  // the wave's own LDS writes are visible to its later reads
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int c = lane; c < M; c += MOE_WAVE) {
    const uint64_t kc = cand[c];
    int r = 0;
    for (int c2 = 0; c2 < M; ++c2) r += cand[c2] > kc ? 1 : 0;
    const int e = rank_key_index(kc);
    if (ranked) ranked[r] = e;
    if (r < k) {
      store_agent(&topk_ids[static_cast<size_t>(t) * k + r], e);
      topk_gates[static_cast<size_t>(t) * k + r] = expf(rank_key_value(kc) - mx) / se;
    } else {
      store_agent(&fallback_ids[static_cast<size_t>(t) * R + (r - k)], e);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace rt
}  // namespace moe
