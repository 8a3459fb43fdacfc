// SERE similarity-guided expert re-routing over one batch, run by a single
// workgroup (multi-image QA inference write-up, §4.1 algorithm, §4.2
// protection matrix, §4.3 fused operator).  Shared by the stand-alone SERE
// kernel and the fused routing kernel.
//
//   1. the batch union P of every token's ranks 1..K' and the set of experts
//      that appear as secondaries become LDS byte flags (plain stores of 1:
//      no atomics, so no serialisation on popular experts);
//   2. the re-route target depends only on the source expert, so it is
//      computed once per secondary expert e outside P: 8 lanes read the
//      similarity row of e and the protection row of e with 16-byte and
//      4-byte vector loads (all issued before any is used, so the row costs
//      one memory round trip), keep the best primary p by (S[e][p] desc,
//      p asc) together with its protection byte, and combine their
//      candidates with two DPP quad permutes and one half-row mirror; a
//      blocked p* keeps e;
//   3. every slot is rewritten through the per-expert target table in LDS.
// Similarity and protection share one [N][N] row-major layout, so the lane
// that holds S[e][p] also holds Prot[e][p]: the protection bit is checked
// once, for the winner only, with no second dependent load.
#pragma once

#include "common.h"

namespace moe {
namespace sr {

struct alignas(16) SereLds {
  uint8_t in_p[1024];    // 1 = in the union of primaries (N <= 1024)
  uint8_t is_sec[1024];  // 1 = appears as a secondary
  int16_t target[1024];  // re-route target per source expert
};

__device__ void sere_block(const int32_t* __restrict__ topk, int T, int N,
                           int k, int kprime, float rho,
                           const float* __restrict__ sim,
                           const uint8_t* __restrict__ prot,
                           int32_t* __restrict__ slot_expert,
                           uint8_t* __restrict__ flags, SereLds& L) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  for (int e = tid; e < N; e += nthr) {
    L.in_p[e] = 0;
    L.is_sec[e] = 0;
  }
  __syncthreads();

  const int total = T * k;
  for (int i = tid; i < total; i += nthr) {
    const int e = topk[i];
    if (i % k < kprime)
      L.in_p[e] = 1;
    else
      L.is_sec[e] = 1;
  }
  __syncthreads();

  constexpr int LPE = 8;  // lanes per source expert: half a DPP row
  const int sub = tid % LPE;
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(sim) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(prot) & 3) == 0;
  for (int e0 = 0; e0 < N; e0 += nthr / LPE) {  // uniform trip count
    const int e = e0 + tid / LPE;
    const bool want = e < N && L.is_sec[e] && !L.in_p[e];
    uint64_t best = 0ull;
    uint32_t bprot = 0u;
    if (want) {
      const float* srow = sim + static_cast<size_t>(e) * N;
      const uint8_t* prow = prot + static_cast<size_t>(e) * N;
      if (vec) {
        // batches of QB quads per lane: every load of a batch is issued
        // before the first is used (one memory round trip per batch)
        constexpr int QB = 8;
        const int nq = N / 4;
        const uint32_t* pflag4 = reinterpret_cast<const uint32_t*>(L.in_p);
        for (int q0 = sub; q0 < nq; q0 += LPE * QB) {
          float4 s4[QB];
          uint32_t p4[QB];
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            const int q = q0 + b * LPE;
            if (q < nq) {
              s4[b] = *reinterpret_cast<const float4*>(srow + 4 * q);
              p4[b] = *reinterpret_cast<const uint32_t*>(prow + 4 * q);
            }
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            const int q = q0 + b * LPE;
            if (q < nq) {
              const uint32_t f4 = pflag4[q];
              const float sv[4] = {s4[b].x, s4[b].y, s4[b].z, s4[b].w};
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint64_t key = rank_key(sv[i], 4 * q + i);
                if (((f4 >> (8 * i)) & 0xffu) && key > best) {
                  best = key;
                  bprot = (p4[b] >> (8 * i)) & 0xffu;
                }
              }
            }
          }
        }
      } else {
#pragma unroll 8
        for (int p = sub; p < N; p += LPE) {
          const float sv = srow[p];
          const uint32_t pv = prow[p];
          const uint64_t key = rank_key(sv, p);
          if (L.in_p[p] && key > best) {
            best = key;
            bprot = pv;
          }
        }
      }
    }
    // combine the 8 lanes: partner lane ^ 1, ^ 2, then the mirrored lane
    // of the other quad (all lanes take part)
    {
      const uint64_t o = dpp64<DPP_QUAD_1032>(0ull, best);
      const uint32_t op = dpp<DPP_QUAD_1032>(0u, bprot);
      if (o > best) {
        best = o;
        bprot = op;
      }
    }
    {
      const uint64_t o = dpp64<DPP_QUAD_2301>(0ull, best);
      const uint32_t op = dpp<DPP_QUAD_2301>(0u, bprot);
      if (o > best) {
        best = o;
        bprot = op;
      }
    }
    {
      const uint64_t o = dpp64<DPP_ROW_HALF_MIRROR>(0ull, best);
      const uint32_t op = dpp<DPP_ROW_HALF_MIRROR>(0u, bprot);
      if (o > best) {
        best = o;
        bprot = op;
      }
    }
    if (e < N && sub == 0) {
      int tgt = e;
      if (want && best != 0ull && rank_key_value(best) > rho && bprot == 0u)
        tgt = rank_key_index(best);
      L.target[e] = static_cast<int16_t>(tgt);
    }
  }
  __syncthreads();

  for (int i = tid; i < total; i += nthr) {
    const int e = topk[i];
    int o = e;
    if (i % k >= kprime && !L.in_p[e]) o = L.target[e];
    slot_expert[i] = o;
    flags[i] = o != e ? MOE_FLAG_SERE : 0;
  }
}

}  // namespace sr
}  // namespace moe
