// SERE similarity-guided expert re-routing over one batch, run by a single
// workgroup (multi-image QA inference write-up, §4.1 algorithm, §4.2
// protection matrix, §4.3 fused operator).  Shared by the stand-alone SERE
// kernel and the fused routing kernel.
//
//   1. the batch union P of every token's ranks 1..K' and the set of experts
//      that appear as secondaries become LDS byte flags (plain stores of 1:
//      no atomics, so no serialisation on popular experts);
//   2. the re-route target depends only on the source expert, so it is
//      computed once per movable expert e (a secondary outside P): wave 0
//      compacts the movable experts into a list with ballots, then 8 lanes
//      per listed expert read the similarity row of e and the protection
//      row of e with 16-byte and 4-byte vector loads (all issued before any
//      is used, so the row costs one memory round trip), keep the best
//      primary p by (S[e][p] desc, p asc) with plain fp32 compares (a lane
//      visits its p in ascending order and only a strictly larger value
//      replaces its candidate), and combine the 8 candidates with two DPP
//      quad permutes and one half-row mirror; a blocked p* keeps e;
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
  int16_t list[1024];    // movable experts (secondaries outside P)
  int count;             // entries of list
};

// A lane's candidate is its best similarity so far, that primary (INT32_MAX:
// none yet) and the primary's protection byte.  The other lane's candidate
// (ov, op) beats this one (v, p) if its S is larger, or equal with a lower
// index.
__device__ __forceinline__ bool beats(float ov, int op, float v, int p) {
  return ov > v || (ov == v && op < p);
}

__device__ __forceinline__ void sere_block(const int32_t* __restrict__ topk, int T, int N,
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

  // targets default to the expert itself; wave 0 lists the movable ones
  for (int e = tid; e < N; e += nthr) L.target[e] = static_cast<int16_t>(e);
  if (tid < MOE_WAVE) {
    int base = 0;
    for (int e0 = 0; e0 < N; e0 += MOE_WAVE) {
      const int e = e0 + tid;
      const bool mv = e < N && L.is_sec[e] && !L.in_p[e];
      const uint64_t bal = __ballot(mv);
      if (mv) L.list[base + __popcll(bal & lanemask_lt())] = static_cast<int16_t>(e);
      base += __popcll(bal);
    }
    if (tid == 0) L.count = base;
  }
  __syncthreads();

  constexpr int LPE = 8;  // lanes per listed expert: half a DPP row
  const int sub = tid % LPE;
  const int count = L.count;
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(sim) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(prot) & 3) == 0;
  // uniform trip count: every lane takes part in the DPP steps
  for (int m0 = 0; m0 < count; m0 += nthr / LPE) {
    const int m = m0 + tid / LPE;
    const bool want = m < count;
    const int e = want ? L.list[m] : 0;
    float bv = -INFINITY;
    int bp = INT32_MAX;
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
            const int q = min(q0 + b * LPE, nq - 1);
            s4[b] = *reinterpret_cast<const float4*>(srow + 4 * q);
            p4[b] = *reinterpret_cast<const uint32_t*>(prow + 4 * q);
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            const int q = q0 + b * LPE;
            const uint32_t f4 = q < nq ? pflag4[q] : 0u;
            const float sv[4] = {s4[b].x, s4[b].y, s4[b].z, s4[b].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (((f4 >> (8 * i)) & 0xffu) && (sv[i] > bv || bp == INT32_MAX)) {
                bv = sv[i];
                bp = 4 * q + i;
                bprot = (p4[b] >> (8 * i)) & 0xffu;
              }
            }
          }
        }
      } else {
#pragma unroll 8
        for (int p = sub; p < N; p += LPE) {
          const float sv = srow[p];
          const uint32_t pv = prow[p];
          if (L.in_p[p] && (sv > bv || bp == INT32_MAX)) {
            bv = sv;
            bp = p;
            bprot = pv;
          }
        }
      }
    }
    // combine the 8 lanes: partner lane ^ 1, ^ 2, then the mirrored lane
    // of the other quad (all lanes take part)
    {
      const float ov = dpp_t<float, DPP_QUAD_1032>(-INFINITY, bv);
      const int op = dpp_t<int, DPP_QUAD_1032>(INT32_MAX, bp);
      const uint32_t opr = dpp<DPP_QUAD_1032>(0u, bprot);
      if (beats(ov, op, bv, bp)) {
        bv = ov;
        bp = op;
        bprot = opr;
      }
    }
    {
      const float ov = dpp_t<float, DPP_QUAD_2301>(-INFINITY, bv);
      const int op = dpp_t<int, DPP_QUAD_2301>(INT32_MAX, bp);
      const uint32_t opr = dpp<DPP_QUAD_2301>(0u, bprot);
      if (beats(ov, op, bv, bp)) {
        bv = ov;
        bp = op;
        bprot = opr;
      }
    }
    {
      const float ov = dpp_t<float, DPP_ROW_HALF_MIRROR>(-INFINITY, bv);
      const int op = dpp_t<int, DPP_ROW_HALF_MIRROR>(INT32_MAX, bp);
      const uint32_t opr = dpp<DPP_ROW_HALF_MIRROR>(0u, bprot);
      if (beats(ov, op, bv, bp)) {
        bv = ov;
        bp = op;
        bprot = opr;
      }
    }
    if (want && sub == 0 && bp != INT32_MAX && bv > rho && bprot == 0u)
      L.target[e] = static_cast<int16_t>(bp);
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
