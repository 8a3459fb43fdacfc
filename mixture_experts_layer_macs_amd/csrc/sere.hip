// moe_sere_reroute: SERE similarity-guided expert re-routing (multi-image QA
// inference write-up, §4.1 algorithm, §4.2 protection matrix, §4.3 fused
// operator).
//
// One fused workgroup of 1024 threads, no host round trip, no sort:
//   1. the batch union P of every token's ranks 1..K' and the set of experts
//      that appear as secondaries are built as bitsets in LDS;
//   2. the re-route target depends only on the source expert, so it is
//      computed once per secondary expert e outside P: one wave scans the
//      similarity row of e (coalesced, read once) masked by P, takes the
//      argmax (ties to the lowest expert index), and checks the single
//      protection bit Prot[e][p*] -- a blocked p* keeps e;
//   3. every slot is rewritten through the per-expert target table in LDS.
// Similarity and protection share one [N][N] row-major layout, so the one
// protection byte read sits at the same offset as the winning similarity.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(1024) void sere_kernel(
    const int32_t* __restrict__ topk, int T, int N, int k, int kprime,
    float rho, const float* __restrict__ sim, const uint8_t* __restrict__ prot,
    int32_t* __restrict__ slot_expert, uint8_t* __restrict__ flags) {
  __shared__ uint32_t in_p[32];     // union of primaries (N <= 1024)
  __shared__ uint32_t is_sec[32];   // experts appearing as secondaries
  __shared__ int16_t target[1024];  // re-route target per source expert

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  if (tid < 32) {
    in_p[tid] = 0u;
    is_sec[tid] = 0u;
  }
  __syncthreads();

  const long total = static_cast<long>(T) * k;
  for (long i = tid; i < total; i += nthr) {
    const int s = static_cast<int>(i % k);
    const int e = topk[i];
    if (s < kprime)
      atomicOr(&in_p[e >> 5], 1u << (e & 31));
    else
      atomicOr(&is_sec[e >> 5], 1u << (e & 31));
  }
  __syncthreads();

  // 8 lanes per source expert, nthr/8 experts in flight per pass; each
  // lane scans every 8th candidate of the similarity row, then the 8 lanes
  // combine their best keys with three xor-shuffles.
  constexpr int LPE = 8;
  const int sub = tid % LPE;
  for (int e0 = 0; e0 < N; e0 += nthr / LPE) {
    const int e = e0 + tid / LPE;
    bool want = false;
    if (e < N) {
      const bool e_in_p = (in_p[e >> 5] >> (e & 31)) & 1u;
      const bool e_sec = (is_sec[e >> 5] >> (e & 31)) & 1u;
      want = e_sec && !e_in_p;
    }
    uint64_t best = 0ull;
    if (want) {
      const float* srow = sim + static_cast<size_t>(e) * N;
#pragma unroll 4
      for (int p = sub; p < N; p += LPE) {
        if ((in_p[p >> 5] >> (p & 31)) & 1u) {
          const uint64_t key = rank_key(srow[p], p);
          best = key > best ? key : best;
        }
      }
    }
#pragma unroll
    for (int off = LPE / 2; off > 0; off >>= 1) {
      const uint64_t o = shfl_u64(best, lane_id() ^ off);
      best = o > best ? o : best;
    }
    if (e < N && sub == 0) {
      int tgt = e;
      if (want && best != 0ull) {
        const int ps = rank_key_index(best);
        if (rank_key_value(best) > rho && prot[static_cast<size_t>(e) * N + ps] == 0)
          tgt = ps;
      }
      target[e] = static_cast<int16_t>(tgt);
    }
  }
  __syncthreads();

  for (long i = tid; i < total; i += nthr) {
    const int s = static_cast<int>(i % k);
    const int e = topk[i];
    int o = e;
    if (s >= kprime && !((in_p[e >> 5] >> (e & 31)) & 1u)) o = target[e];
    slot_expert[i] = o;
    flags[i] = o != e ? MOE_FLAG_SERE : 0;
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_sere_reroute(const int32_t* topk_ids, int T, int N, int k,
                                int kprime, float rho, const float* sim,
                                const uint8_t* prot, int32_t* slot_expert,
                                uint8_t* flags, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      kprime < 1 || kprime > k)
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !sim || !prot || !slot_expert || !flags) return MOE_EINVAL;
  hipLaunchKernelGGL(sere_kernel, dim3(1), dim3(1024), 0, as_stream(stream),
                     topk_ids, T, N, k, kprime, rho, sim, prot, slot_expert,
                     flags);
  return launch_status();
}
