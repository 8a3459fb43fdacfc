// Routing of a very small decode batch (at most 8 tokens and 64 slots) in
// one workgroup: router top-k ("MACS", §3.1 Eq. 1), SERE re-routing
// (multi-image QA inference write-up, §4.1-§4.3), MACS weights, capacities
// and re-route-else-drop ("MACS", §3.2 Eq. 5-6, §3.3 Eq. 7, §3.1 Eq. 3, §1
// and Fig. 1) and the expert-major dispatch.
//
// At this size every batch-wide step is a handful of instructions, and the
// cost of the general tail is its chain of workgroup barriers and memory
// round trips.  Here the workgroup splits the work by what it depends on:
//   - wave t < T ranks token t with its logits in registers and leaves the
//     k + R ranked ids in LDS as well as in the outputs;
//   - at the same time wave T, which needs no ranking, forms the token
//     weights, W, W_vis, R_v and every capacity, and clears the tables;
//   - after one workgroup barrier, wave 0 alone runs the rest with one lane
//     per slot (slot i = t k + s in lane i): SERE, round-0 admission, the
//     fallback rounds (on one lane per token) and the dispatch maps.  Lanes
//     meet through ballots, DPP row shifts and LDS behind wave-local
//     ordering only.
// In a single wave the cost is the length of its dependent instruction
// chain and of its memory round trips, so each step is arranged to keep
// both short: every LDS or memory read is issued unconditionally (clamped
// index) and before its first use, so a batch of reads costs one round
// trip; the SERE step reads only the similarity and protection entries it
// compares (from a decode step's cold caches, copying the matrices to LDS
// costs more than it saves); the fallback rounds are unrolled with their
// candidate, group and capacity terms fetched up front; the dispatch row
// comes from ballot bit planes, without a scan.  The results equal the
// general tail's bit for bit.
#pragma once

#include <cmath>
#include <type_traits>

#include "common.h"
#include "dtail_impl.h"
#include "route_impl.h"

namespace moe {
namespace tiny {

constexpr int MAX_T = 8, MAX_K = 8, MAX_R = 8, MAX_N = 256, MAX_SLOTS = 64;
constexpr int MAX_THREADS = (MAX_T + 1) * MOE_WAVE;
constexpr int MAX_IDS = MAX_T * (MAX_K + MAX_R);

inline bool supported(int T, int N, int k, int R) {
  return T >= 1 && T <= MAX_T && T * k <= MAX_SLOTS && k <= MAX_K && R <= MAX_R &&
         N <= MAX_N;
}

// Threads of the workgroup: the routing waves and the helper wave.
inline int threads(int T) { return MOE_WAVE * (T + 1); }

struct Args {
  dtail::Args d;  // the batch-wide steps' inputs (d.topk, d.fb, d.sim_lds unused) and outputs
  const float* logits;
  int32_t* topk_ids;
  float* topk_gates;
  int32_t* fallback_ids;
};

// Orders this wave's LDS accesses: the writes before it are seen by every
// lane's reads after it (a wave's LDS operations complete in order).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bit e of a 256-bit set held as four wave-uniform words.
__device__ __forceinline__ bool in_set(const uint64_t (&m)[4], int e) {
  const uint64_t w = e < 64 ? m[0] : e < 128 ? m[1] : e < 192 ? m[2] : m[3];
  return (w >> (e & 63)) & 1u;
}

// Offers of the token lanes (lanes 0..7, one row of 16 lanes) in packed
// form ((expert + 1) << 17 | weight, 0 for no offer): adds the weight of the
// offer of lane l - D when it goes to the same expert.
template <int D>
__device__ __forceinline__ uint32_t same_offer(uint32_t pk, uint32_t acc) {
  const uint32_t o = dpp<0x110 + D>(0u, pk);  // row_shr:D
  return acc + ((o >> 17) == (pk >> 17) ? (o & 0x1ffffu) : 0u);
}

struct Lds {
  uint64_t cand[MAX_IDS];                  // the routing waves' selections
  int32_t ids[MAX_IDS];                    // ranked ids, token-major
  int32_t wq[MAX_T];                       // token weights
  int32_t cap[MAX_N];                      // capacity, clamped to 2^30
  uint32_t load0[MAX_N];                   // round-0 load (capacity off: the load)
  uint32_t got[MAX_N];                     // weight placed by the fallback rounds
  uint32_t cnt[MAX_N];                     // kept slots per expert
  int32_t cur[MAX_SLOTS];                  // slot experts after round 0
  int32_t plist[MAX_SLOTS];                // the primaries, ascending
  uint8_t active[MAX_N];                   // experts with a round-0 slot
  uint8_t inp[MAX_N];                      // experts in the primary union
};

template <int KPL>
__global__ __launch_bounds__(MAX_THREADS) void routing_kernel(Args A) {
  __shared__ Lds L;
  const dtail::Args& a = A.d;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int T = a.T, N = a.N, k = a.k, R = a.R, M = k + R, Tk = T * k;

  if (wave < T) {
    rt::route_token_wave<KPL>(A.logits + static_cast<size_t>(wave) * N, N, k, R, wave,
                              true, L.cand + wave * M, A.topk_ids, A.topk_gates,
                              A.fallback_ids, L.ids + wave * M);
  } else if (wave == T) {
    // ---- helper wave: token weights, W and W_vis, R_v, capacities
    uint8_t vis = 0;
    float ew = 0.f;
    int8_t modv[4] = {0, 0, 0, 0};
    {  // (clamped indices: every load issued at once, the extra ones unused)
      const uint8_t v0 = a.vis[min(lane, T - 1)];
      const float w0 = a.ew[min(lane, T - 1)];
#pragma unroll
      for (int j = 0; j < 4; ++j) modv[j] = a.mod[min(lane + 64 * j, N - 1)];
      if (lane < T) {
        vis = v0;
        ew = w0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // every entry, so that reads need no bound
      const int e = lane + 64 * j;
      L.active[e] = 0;
      L.inp[e] = 0;
      L.load0[e] = 0u;
      L.got[e] = 0u;
      L.cnt[e] = 0u;
    }
    const int32_t wq = lane < T ? dtail::quant_weight(vis, ew) : 0;
    if (lane < T) L.wq[lane] = wq;
    const int64_t W = wave_sum_i64(wq), Wv = wave_sum_i64(vis ? wq : 0);
    const double rv = W > 0 ? static_cast<double>(Wv) / static_cast<double>(W) : 0.5;
    if (lane == 0) {
      a.r_v[0] = rv;
      a.stats[0] = W;
      a.stats[1] = Wv;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e >= N) continue;
      if (a.cap_on) {
        const int64_t c = dtail::capacity(a, rv, modv[j]);
        a.cap_q[e] = c;
        L.cap[e] = static_cast<int32_t>(c < (int64_t(1) << 30) ? c : (int64_t(1) << 30));
      } else {
        a.cap_q[e] = INT64_MAX;
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // ---- wave 0: lane i holds slot i = t k + s
  const bool valid = lane < Tk;
  int t = 0;  // lane / k, by compares (k <= 8, lane < 64)
#pragma unroll
  for (int u = 1; u < MAX_T; ++u) t += valid && lane >= u * k ? 1 : 0;
  const int s = valid ? lane - t * k : 0;
  const int id0 = L.ids[t * M + s];
  const int e0 = valid ? min(max(id0, 0), N - 1) : 0;
  int cur = e0;
  bool moved = false;

  // ---- SERE: secondaries outside the primary union P move to their most
  // similar primary (ascending scan, strictly greater wins: ties keep the
  // lower id) if that similarity exceeds rho and the pair is not protected
  if (a.kprime > 0) {
    if (valid && s < a.kprime) L.inp[e0] = 1;
    wave_sync();
    uint64_t pm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool f = L.inp[lane + 64 * j] != 0;  // entries >= N are zero
      pm[j] = __ballot(f);
    }
    int np = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((pm[j] >> lane) & 1u) L.plist[np + __popcll(pm[j] & lanemask_lt())] = lane + 64 * j;
      np += __popcll(pm[j]);
    }
    wave_sync();
    const bool movable = valid && s >= a.kprime && !in_set(pm, e0);
    if (movable) {
      float bv = 0.f;
      int bp = -1;
      uint32_t bpr = 0u;
      const size_t row = static_cast<size_t>(e0) * N;
      for (int c0 = 0; c0 < np; c0 += 16) {
        int ps[16];
        float v[16];
        uint8_t pr[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) ps[q] = L.plist[min(c0 + q, np - 1)];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          v[q] = a.sim[row + ps[q]];
          pr[q] = a.prot[row + ps[q]];
        }
        // branch-free (short-circuit forms compile to a branch per entry)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const bool take = (c0 + q < np) & ((bp < 0) | (v[q] > bv));
          bv = take ? v[q] : bv;
          bp = take ? ps[q] : bp;
          bpr = take ? pr[q] : bpr;
        }
      }
      moved = bv > a.rho && bpr == 0u;  // np >= 1 whenever a slot is movable
      if (moved) cur = bp;
    }
    if (valid) a.slot_sere[lane] = cur;
  }

  // the token weights (lane u < T holds token u's)
  const int32_t wq_l = L.wq[min(lane, MAX_T - 1)];
  const int32_t wtok = lane < T ? wq_l : 0;

  bool over = false, placed = false;
  if (!a.cap_on) {
    // everything kept; the load is the plain weight total
    if (valid) atomicAdd(&L.load0[cur], static_cast<uint32_t>(L.wq[t]));
  } else {
    // ---- round 0: each expert admits its slots in (token, slot) order while
    // the running weight stays within its capacity.  A slot's running weight
    // sums its peers (same expert) at or before it, token by token.
    const uint64_t peers = match_any(cur, valid, a.nbits);
    const uint64_t ple = peers & lanemask_le();
    const uint64_t tmask = (1ull << k) - 1ull;  // k <= 8
    uint32_t incl = 0u;
#pragma unroll
    for (int u = 0; u < MAX_T; ++u) {
      if (u >= T) break;
      const uint32_t wu = static_cast<uint32_t>(__builtin_amdgcn_readlane(wtok, u));
      incl += static_cast<uint32_t>(__popcll(ple & (tmask << (u * k)))) * wu;
    }
    const int32_t capc = L.cap[cur];
    const bool adm = valid && static_cast<int32_t>(incl) <= capc;
    over = valid && !adm;
    const uint64_t admb = __ballot(adm);
    if (valid) {
      L.active[cur] = 1;
      L.cur[lane] = cur;
      if (adm && lane == 63 - __clzll(static_cast<long long>(peers & admb)))
        L.load0[cur] = incl;  // the admitted slots of an expert form a prefix
    }
    wave_sync();

    // ---- fallback rounds: lane u < T owns token u
    const uint64_t overb = __ballot(over);
    if (R > 0 && overb) {
      // fallback ranks that could be offered, tested in lane j = 8 t + q for
      // token t's rank q: the expert has a round-0 slot and no kept slot of
      // the token holds it (kept slots never move; the full test is made at
      // the offer).  A token's fallback ids are distinct, so placing a slot
      // on rank q's expert rules out no other rank.
      uint32_t cand;
      {
        const int ct = lane >> 3, cq = lane & 7;
        const bool live = ct < T && cq < R;
        const int c = min(max(L.ids[min(ct * M + k + cq, MAX_IDS - 1)], 0), N - 1);
        int cv[MAX_K];
#pragma unroll
        for (int x = 0; x < MAX_K; ++x) cv[x] = L.cur[min(ct * k + x, MAX_SLOTS - 1)];
        const bool act = L.active[c] != 0;
        bool held = false;
#pragma unroll
        for (int x = 0; x < MAX_K; ++x)
          held |= (x < k) & !((overb >> ((ct * k + x) & 63)) & 1u) & (cv[x] == c);
        const bool cnd = live & act & !held;
        const uint64_t cb = __ballot(cnd);
        cand = lane < T ? static_cast<uint32_t>(cb >> (lane * 8)) & 0xffu : 0u;
      }
      const bool tok = lane < T;
      uint32_t ov = tok ? static_cast<uint32_t>(overb >> (lane * k)) & static_cast<uint32_t>(tmask)
                        : 0u;
      uint32_t pl = 0u;
      int tc[MAX_K], fbr[MAX_R];
      int32_t room[MAX_R];  // capacity left after round 0 for each fallback rank
#pragma unroll
      for (int x = 0; x < MAX_K; ++x) {
        const int v = L.cur[min(lane * k + x, MAX_SLOTS - 1)];
        tc[x] = tok && x < k ? v : -1;
      }
#pragma unroll
      for (int q = 0; q < MAX_R; ++q) {
        const int v = L.ids[min(lane * M + k + q, MAX_IDS - 1)];
        fbr[q] = tok && q < R ? min(max(v, 0), N - 1) : 0;
      }
#pragma unroll
      for (int q = 0; q < MAX_R; ++q)
        room[q] = L.cap[fbr[q]] - static_cast<int32_t>(L.load0[fbr[q]]);
      // ONE: every expert in one group (no group test, no division)
      auto rounds = [&](auto one_tag) {
        constexpr bool ONE = decltype(one_tag)::value;
        int fbg[MAX_R], tcg[MAX_K];  // expert groups, up front
        if constexpr (!ONE) {
#pragma unroll
          for (int q = 0; q < MAX_R; ++q) fbg[q] = fbr[q] / a.group;
#pragma unroll
          for (int x = 0; x < MAX_K; ++x) tcg[x] = tc[x] < 0 ? 0 : tc[x] / a.group;
        }
#pragma unroll
        for (int r = 1; r <= MAX_R; ++r) {
          if (r > R) break;
          // stop once no token has an overflowed slot with a candidate left
          if (!__ballot(ov != 0u && (cand >> (r - 1)) != 0u)) break;
          const int c = fbr[r - 1];
          const uint32_t got = L.got[c];
          bool offer = false;
          int s0 = 0;
          if (ov != 0u && ((cand >> (r - 1)) & 1u)) {
            s0 = __builtin_ctz(ov);
            bool held = false;
#pragma unroll
            for (int x = 0; x < MAX_K; ++x) held |= tc[x] == c;
            bool same_group = true;
            if constexpr (!ONE) {
              int g0 = 0;
#pragma unroll
              for (int x = 0; x < MAX_K; ++x)
                if (x == s0) g0 = tcg[x];
              same_group = g0 == fbg[r - 1];
            }
            offer = !held && same_group;
          }
          // the offers to one expert are admitted in token order while their
          // running weight stays within what the expert has left
          const uint32_t pk = offer ? (static_cast<uint32_t>(c + 1) << 17) |
                                          static_cast<uint32_t>(wtok)
                                    : 0u;
          uint32_t pre = static_cast<uint32_t>(wtok);
          pre = same_offer<1>(pk, pre);
          pre = same_offer<2>(pk, pre);
          pre = same_offer<3>(pk, pre);
          pre = same_offer<4>(pk, pre);
          pre = same_offer<5>(pk, pre);
          pre = same_offer<6>(pk, pre);
          pre = same_offer<7>(pk, pre);
          if (offer && static_cast<int32_t>(pre) <= room[r - 1] - static_cast<int32_t>(got)) {
#pragma unroll
            for (int x = 0; x < MAX_K; ++x)
              if (x == s0) {
                tc[x] = c;
                if constexpr (!ONE) tcg[x] = fbg[r - 1];
              }
            ov &= ~(1u << s0);
            pl |= 1u << s0;
            atomicAdd(&L.got[c], static_cast<uint32_t>(wtok));
          }
          wave_sync();
        }
      };
      if (a.group >= N)
        rounds(std::true_type{});
      else
        rounds(std::false_type{});
      if (tok) {
#pragma unroll
        for (int x = 0; x < MAX_K; ++x)
          if (x < k) L.cur[lane * k + x] = tc[x];
      }
      wave_sync();
      const uint32_t ovt = __shfl(ov, t), plt = __shfl(pl, t);
      over = valid && ((ovt >> s) & 1u);
      placed = valid && ((plt >> s) & 1u);
      const int cfin = L.cur[lane];
      if (placed) cur = cfin;
    }
  }

  // ---- final slots, flags, loads and counts
  const bool kept = valid && !over;
  const int fe = kept ? cur : -1;
  if (valid) {
    a.slot_expert[lane] = fe;
    a.flags[lane] = static_cast<uint8_t>((moved ? MOE_FLAG_SERE : 0) |
                                         (over ? MOE_FLAG_DROP : 0) |
                                         (placed ? MOE_FLAG_MACS : 0));
  }
  const int n_drop = __popcll(__ballot(over)), n_macs = __popcll(__ballot(placed));
  if (lane == 0) {
    a.stats[2] = n_drop;
    a.stats[3] = n_macs;
  }

  // ---- dispatch: kept slots in (expert, token, slot) order.  From the
  // top bit of the expert id down, `eq` keeps the kept lanes that agree with
  // this one so far and `less` counts those that fell below it; at the end
  // eq holds the peers, and the row is less + the peers before this lane.
  uint64_t eq = __ballot(kept);
  uint32_t less = 0u;
  for (int b = a.nbits - 1; b >= 0; --b) {
    const bool bit = kept && ((fe >> b) & 1);
    const uint64_t on = __ballot(bit);
    if (bit) less += static_cast<uint32_t>(__popcll(eq & ~on));
    eq &= bit ? on : ~on;
  }
  if (valid) {
    if (kept) {
      const int row = static_cast<int>(less) + __popcll(eq & lanemask_lt());
      a.slot_row[lane] = row;
      a.row_token[row] = t;
      a.row_slot[row] = s;
      if (lane == 63 - __clzll(static_cast<long long>(eq)))
        L.cnt[fe] = static_cast<uint32_t>(__popcll(eq));
    } else {
      a.slot_row[lane] = -1;
    }
  }
  wave_sync();  // the expert counts and the capacity-off loads
  {
    int32_t v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      v[q] = e < N ? static_cast<int32_t>(L.cnt[e]) : 0;
      sum += v[q];
    }
    const int32_t incl_sum = wave_incl_scan(sum);
    int32_t run = incl_sum - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < N) a.offsets[e] = run;
      run += v[q];
    }
    if (lane == 63) a.offsets[N] = incl_sum;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < N) a.load_q[e] = static_cast<int64_t>(L.load0[e]) + L.got[e];
  }
}

}  // namespace tiny
}  // namespace moe
