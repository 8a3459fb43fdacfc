// MACS entropy-weighted load, modality-adaptive capacity and
// re-route-else-drop ("MACS", §3.1 Eq. 3, §3.2 Eq. 5-6, §3.3 Eq. 7 with the
// expert modality indicator m_j, §1 and Fig. 1 for the two-stage overflow
// handling): device phases and workspace layout, shared by the capacity
// kernels and the fused routing kernel.
//
// The capacity is computed in IEEE double, one rounded operation per step,
// in a fixed order (floating-point contraction is off inside capacity_of).
//
// Work decomposition.  Tokens are split into G contiguous blocks of TB
// tokens, one workgroup each.  Every round has the same shape:
//   propose  each workgroup lists its proposals in (token, slot) order and
//            computes, per expert, the inclusive running weight of its own
//            proposals (an ordered per-key prefix: 64-lane chunks, peers
//            found by ballots over the key bits, a per-wave running total in
//            LDS, then a per-expert scan over the waves);
//   global   the last workgroup to finish (an atomic ticket that wraps back
//            to zero) scans the per-workgroup totals over the blocks, so
//            every proposal's global running weight is block base + local;
//   apply    at the start of the next launch each proposal is admitted iff
//            its global running weight is within the expert's remaining
//            capacity -- exactly the sequential prefix rule, because block
//            order is token order.
// Loads, sums and capacities are integers in units of 2^-16 token, so the
// parallel sums equal the sequential ones bit for bit.  When the whole batch
// fits one workgroup (decode), all rounds run in one launch.
#pragma once

#include <math.h>

#include <algorithm>
#include <cmath>

#include "common.h"

namespace moe {
namespace cap {

enum : uint8_t { ST_KEPT = 0, ST_OVER = 1, ST_PLACED = 2, ST_MASK = 3,
                 ST_SERE = 4 };

enum : unsigned { PH_RUN = 0, PH_FINISH = 1, PH_DONE = 2 };

constexpr int64_t CAP_CLAMP = int64_t(1) << 62;

struct Args {
  const int32_t* topk;
  const int32_t* slot_in;
  const int32_t* fallback;
  const uint8_t* is_visual;
  const float* entropy_w;
  const int8_t* modality;
  int T, N, k, R, group, nbits;
  double gamma, lam;
  int32_t* slot_out;
  uint8_t* flags;
  int64_t* load_q;
  int64_t* cap_q;
  int64_t* stats;
  double* r_v;
  // workspace
  int32_t* wq;         // [T]      token weight (fixed point)
  int32_t* cur;        // [T*k]    current expert of each slot
  uint8_t* st;         // [T*k]    slot state | ST_SERE
  int32_t* incl_slot;  // [T*k]    in-block running weight, round 0
  int32_t* incl_tok;   // [T]      in-block running weight, rounds >= 1
  int32_t* offer_s;    // [T]      offered slot this round (-1 = none)
  int32_t* offer_c;    // [T]      offered expert this round
  int32_t* part;       // [G*N]    per-block per-expert proposal weight
  int64_t* base;       // [G*N]    exclusive block prefix of part
  int64_t* wsum;       // [G*4]    per-block {W, W_vis, dropped, rerouted}
  int64_t* capv;       // [N]
  int64_t* drem;       // [N]      capacity left for the pending round
  uint8_t* active;     // [N]
  // control words: zero between calls (each is cleared after its last use)
  unsigned* ticket;                 // [1]
  // progress of a multi-launch call, set by the first launch: PH_RUN, then
  // PH_FINISH once no overflowed slot is left unplaced, PH_DONE once the
  // slots are final; pending counts the unplaced overflowed slots
  unsigned* phase;                  // [1]
  unsigned long long* pending;      // [1] (two's complement sum)
  uint32_t* act_bits;               // [32]  experts with a round-0 proposer
  unsigned long long* adm;          // [3][N] max admitted running weight
  unsigned long long* total;        // [N]   proposal weight (capacity off)
  // decentralised multi-launch call (dec != 0): the launch that finalised
  // the slots early (0 = none yet)
  unsigned* fin;                    // [1]
  int TB, G, lds_scan, dec;
};

__device__ __forceinline__ int32_t quant_weight(uint8_t vis, float w) {
  if (!vis) return MOE_WEIGHT_ONE;
  if (isnan(w)) w = 1.f;
  w = fminf(fmaxf(w, 0.f), 1.f);
  return static_cast<int32_t>(rintf(w * 65536.f));  // exact scale, half-even
}

__device__ int64_t capacity_of(const Args& a, double rv, int e) {
#pragma clang fp contract(off)
  const double base = ((a.gamma * static_cast<double>(a.T)) *
                       static_cast<double>(a.k)) / static_cast<double>(a.N);
  const double scale = a.lam * static_cast<double>(a.modality[e]);
  double c = base * (1.0 + scale * (rv - 0.5));
  c = (1.0 > c) ? 1.0 : c;
  const double cq = c * 65536.0;
  return cq >= 4611686018427387904.0 ? CAP_CLAMP
                                     : static_cast<int64_t>(floor(cq));
}

// ---------------------------------------------------------------- phases
// Round-0 proposals: every slot, in (token, slot) order.
__device__ void propose0(const Args& a, int g, int t0, int t1, int32_t* run,
                         uint32_t* act_bits, int64_t* red, int32_t* part_row) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k;
  int64_t w_all = 0, w_vis = 0;
  for (int t = t0 + tid; t < t1; t += nthr) {
    const int32_t q = quant_weight(a.is_visual[t], a.entropy_w[t]);
    a.wq[t] = q;
    w_all += q;
    if (a.is_visual[t]) w_vis += q;
  }
  for (int i = t0 * k + tid; i < t1 * k; i += nthr) {
    const int32_t e = a.slot_in[i];
    a.cur[i] = e;
    a.st[i] = (e != a.topk[i]) ? ST_SERE : ST_KEPT;
  }
  if (tid < 32) act_bits[tid] = 0u;
  block_sum2_i64(w_all, w_vis, red);
  if (tid == 0) {
    a.wsum[g * 4 + 0] = w_all;
    a.wsum[g * 4 + 1] = w_vis;
  }
  const int32_t* cur = a.cur + static_cast<size_t>(t0) * k;
  const int32_t* wq = a.wq;
  key_prefix((t1 - t0) * k, a.N, a.nbits, run,
             [&](int idx, int& key, int32_t& w) {
               key = cur[idx];
               w = wq[t0 + idx / k];
             },
             a.incl_slot + static_cast<size_t>(t0) * k, part_row, act_bits);
  if (tid < 32 && act_bits[tid]) atomicOr(&a.act_bits[tid], act_bits[tid]);
}

// Offers of fallback round r >= 1: one per token with an unplaced overflow.
// An expert is a candidate iff it had a round-0 proposer: active[c], or,
// when active is null, bit c of the global act_bits.
__device__ void propose_round(const Args& a, int r, int g, int t0, int t1,
                              int32_t* run, const uint8_t* active,
                              int32_t* part_row) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k;
  for (int t = t0 + tid; t < t1; t += nthr) {
    const int32_t* cs = a.cur + static_cast<size_t>(t) * k;
    const uint8_t* ss = a.st + static_cast<size_t>(t) * k;
    // no early exits: the k loads of each scan are independent and can all
    // be in flight together
    int s_off = -1;
    for (int s = k - 1; s >= 0; --s)
      if ((ss[s] & ST_MASK) == ST_OVER) s_off = s;
    int c = -1;
    if (s_off >= 0) {
      c = a.fallback[static_cast<size_t>(t) * a.R + (r - 1)];
      const int e = cs[s_off];
      const bool act = active ? active[c] != 0 : ((a.act_bits[c >> 5] >> (c & 31)) & 1u) != 0;
      bool ok = act && (c / a.group) == (e / a.group);
      bool held = false;
      for (int s = 0; s < k; ++s) held |= cs[s] == c;
      if (!ok || held) s_off = -1;
    }
    a.offer_s[t] = s_off;
    a.offer_c[t] = s_off >= 0 ? c : -1;
  }
  __syncthreads();
  const int32_t* oc = a.offer_c + t0;
  const int32_t* wq = a.wq + t0;
  key_prefix(t1 - t0, a.N, a.nbits, run,
             [&](int idx, int& key, int32_t& w) {
               key = oc[idx];
               w = wq[idx];
             },
             a.incl_tok + t0, part_row, nullptr);
}

// Admit or refuse the proposals of round r against base (this block's
// exclusive prefix of round r's proposal weight over the earlier blocks;
// null for a single workgroup, where it is zero) and
// drem (capacity left before round r).  amax (LDS) ends with this block's
// largest admitted running weight per expert, also folded into adm[] with
// atomicMax unless adm is null.
// pending (may be null): LDS count of overflowed slots not yet placed;
// round 0 adds its overflows, later rounds subtract their admissions.
__device__ void apply(const Args& a, int r, int t0, int t1,
                      unsigned long long* amax, int* pending,
                      const int64_t* base, const int64_t* drem,
                      unsigned long long* adm) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k, N = a.N;
  for (int e = tid; e < N; e += nthr) amax[e] = 0ull;
  __syncthreads();
  int moved = 0;
  if (r == 0) {
    for (int i = t0 * k + tid; i < t1 * k; i += nthr) {
      const int e = a.cur[i];
      const int64_t v = (base ? base[e] : 0) + a.incl_slot[i];
      if (v <= drem[e]) {
        atomicMax(&amax[e], static_cast<unsigned long long>(v));
      } else {
        a.st[i] = (a.st[i] & ST_SERE) | ST_OVER;
        ++moved;
      }
    }
  } else {
    for (int t = t0 + tid; t < t1; t += nthr) {
      const int s = a.offer_s[t];
      if (s < 0) continue;
      const int c = a.offer_c[t];
      const int64_t v = (base ? base[c] : 0) + a.incl_tok[t];
      if (v <= drem[c]) {
        const size_t i = static_cast<size_t>(t) * k + s;
        a.st[i] = (a.st[i] & ST_SERE) | ST_PLACED;
        a.cur[i] = c;
        atomicMax(&amax[c], static_cast<unsigned long long>(v));
        --moved;
      }
    }
  }
  if (pending) {  // one LDS atomic per wave
    const int w = wave_sum(moved);
    if (lane_id() == 0 && w != 0) atomicAdd(pending, w);
  }
  __syncthreads();
  if (adm)
    for (int e = tid; e < N; e += nthr)
      if (amax[e]) atomicMax(&adm[e], amax[e]);
}

// Final slot values and flags of the block; the drop / re-route counts go to
// wsum (or, with add_stats, straight into stats[2..3] by integer atomics).
__device__ void finalize_slots(const Args& a, int g, int t0, int t1,
                               int64_t* red, bool add_stats = false) {
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k;
  int64_t n_drop = 0, n_macs = 0;
  for (int i = t0 * k + tid; i < t1 * k; i += nthr) {
    const uint8_t s = a.st[i];
    uint8_t f = (s & ST_SERE) ? MOE_FLAG_SERE : 0;
    int32_t o = a.cur[i];
    if ((s & ST_MASK) == ST_OVER) {
      o = -1;
      f |= MOE_FLAG_DROP;
      ++n_drop;
    } else if ((s & ST_MASK) == ST_PLACED) {
      f |= MOE_FLAG_MACS;
      ++n_macs;
    }
    a.slot_out[i] = o;
    a.flags[i] = f;
  }
  block_sum2_i64(n_drop, n_macs, red);
  if (tid == 0) {
    if (add_stats) {
      if (n_drop) atomicAdd(reinterpret_cast<unsigned long long*>(a.stats + 2),
                            static_cast<unsigned long long>(n_drop));
      if (n_macs) atomicAdd(reinterpret_cast<unsigned long long*>(a.stats + 3),
                            static_cast<unsigned long long>(n_macs));
    } else {
      a.wsum[g * 4 + 2] = n_drop;
      a.wsum[g * 4 + 3] = n_macs;
    }
  }
}

// Global step after round r's proposals (r <= R) or after the last apply
// (r == R + 1).  Run by exactly one workgroup.
// adm: the largest admitted running weight of round r-1 per expert -- the
// global atomicMax target a.adm with several workgroups (cleared here after
// use), or the single workgroup's own LDS maxima (cleared by its next apply).
__device__ void global_step(const Args& a, int r, int64_t* red, int32_t* lds,
                            unsigned long long* adm) {
  const int tid = threadIdx.x, nthr = blockDim.x, N = a.N, G = a.G;
  __shared__ double s_rv;
  if (r == 0) {
    int64_t w_all = 0, w_vis = 0;
    for (int g = tid; g < G; g += nthr) {
      w_all += a.wsum[g * 4 + 0];
      w_vis += a.wsum[g * 4 + 1];
    }
    block_sum2_i64(w_all, w_vis, red);
    if (tid == 0) {
      const double rv = w_all > 0 ? static_cast<double>(w_vis) /
                                        static_cast<double>(w_all)
                                  : 0.5;
      s_rv = rv;
      a.r_v[0] = rv;
      a.stats[0] = w_all;
      a.stats[1] = w_vis;
    }
    __syncthreads();
    const double rv = s_rv;
    for (int e = tid; e < N; e += nthr) {
      const int64_t c = capacity_of(a, rv, e);
      a.capv[e] = c;
      a.cap_q[e] = c;
      a.drem[e] = c;
      a.active[e] = (a.act_bits[e >> 5] >> (e & 31)) & 1u;
      if (G > 1) a.adm[e] = 0ull;  // a decentralised call may leave one round's maxima
    }
    __syncthreads();
    if (tid < 32) a.act_bits[tid] = 0u;
    if (G > 1 && tid == 0) {
      *a.phase = PH_RUN;
      *a.pending = 0ull;
    }
  } else {
    for (int e = tid; e < N; e += nthr) {
      const int64_t m = static_cast<int64_t>(adm[e]);
      if (G > 1) adm[e] = 0ull;
      const int64_t d = a.drem[e] - m;
      a.drem[e] = d;
      if (r > a.R) a.load_q[e] = a.capv[e] - d;
    }
  }
  // every workgroup added its change of the pending count before the
  // ticket: none left after round r - 1 means rounds r .. R offer nothing
  if (G > 1 && r >= 1 && r <= a.R && tid == 0 && atomicAdd(a.pending, 0ull) == 0ull)
    *a.phase = PH_FINISH;
  if (r <= a.R) {
    // one workgroup: no earlier block, every prefix base is zero (apply is
    // passed no base array)
    if (G > 1) column_scan<int64_t>(a.part, a.base, nullptr, G, N, lds, a.lds_scan);
  } else {
    int64_t nd = 0, nm = 0;
    for (int g = tid; g < G; g += nthr) {
      nd += a.wsum[g * 4 + 2];
      nm += a.wsum[g * 4 + 3];
    }
    block_sum2_i64(nd, nm, red);
    if (tid == 0) {
      a.stats[2] = nd;
      a.stats[3] = nm;
    }
  }
}

// Whether an unplaced overflowed slot of the block could still be placed in
// rounds r..R (call after round r-1's admissions, before round r's offers).
// Every condition of an offer only tightens from round to round: A and the
// groups are fixed, a token's held experts only grow, the capacity left
// only shrinks.  So if no token has a candidate c that passes them all now
// -- c in A, in the group of one of its overflowed slots, not held, and at
// least the token's weight of capacity left -- no later round admits
// anything, and the slots can be finalised at once.
__device__ bool any_placeable(const Args& a, int r, int t0, int t1,
                              const unsigned long long* adm) {
  __shared__ int s_any;
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k;
  if (tid == 0) s_any = 0;
  __syncthreads();
  // one (token, round) pair per step: the pairs are independent, so their
  // loads overlap; with one group of all N experts (the one-GPU case) the
  // group test, an integer division per slot otherwise, drops out
  const bool one_group = a.group >= a.N;
  const int nr = a.R - r + 1;
  const int npairs = (t1 - t0) * nr;
  for (int p = tid; p < npairs; p += nthr) {
    const int t = t0 + p / nr, rr = r + p % nr;
    const int32_t* cs = a.cur + static_cast<size_t>(t) * k;
    const uint8_t* ss = a.st + static_cast<size_t>(t) * k;
    const int c = a.fallback[static_cast<size_t>(t) * a.R + (rr - 1)];
    const int gc = one_group ? 0 : c / a.group;
    bool held = false, grp = false;
    for (int s = 0; s < k; ++s) {
      const int e = cs[s];
      held |= e == c;
      grp |= (ss[s] & ST_MASK) == ST_OVER && (one_group || e / a.group == gc);
    }
    if (grp && !held && a.active[c] &&
        a.drem[c] - static_cast<int64_t>(adm[c]) >= a.wq[t])
      s_any = 1;
  }
  __syncthreads();
  return s_any != 0;
}

// True in every thread of the workgroup that finished last (G > 1).  An
// agent-scope fence writes back or invalidates the XCD's L2 on gfx950, so
// one thread fences for the whole workgroup after every wave has waited for
// its own stores.
__device__ bool last_block(const Args& a) {
  __shared__ int s_last;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned prev = atomicInc(a.ticket, static_cast<unsigned>(a.G - 1));
    s_last = prev == static_cast<unsigned>(a.G - 1);
    if (s_last) __threadfence();
  }
  __syncthreads();
  return s_last != 0;
}

// Workgroup g of the token-block decomposition (g = 0 when one workgroup
// covers the batch).  smem: dynamic LDS [N u64][lds_scan int32].
__device__ void cap_rounds(const Args& a, int g, int r_first, int r_last,
                           unsigned char* smem) {
  // [amax: N u64][run table / column-scan staging: lds_scan int32]
  unsigned long long* amax = reinterpret_cast<unsigned long long*>(smem);
  int32_t* run = reinterpret_cast<int32_t*>(smem + sizeof(unsigned long long) * a.N);
  __shared__ uint32_t act_bits[32];
  __shared__ int64_t red[32];
  __shared__ int s_pending;
  const int t0 = g * a.TB, t1 = min(a.T, t0 + a.TB);
  // One workgroup running every round can stop re-routing as soon as no
  // overflowed slot is left unplaced (the overflow set only shrinks), or as
  // soon as none of them has a candidate left that could be admitted: the
  // remaining rounds could admit nothing.
  const bool track = a.G == 1 && r_first == 0 && r_last == a.R + 1;
  const bool multi = a.G > 1;
  if (threadIdx.x == 0) s_pending = 0;
  if (multi && r_first >= 1) {
    // a launch after the first: skip the rounds that can place nothing
    __shared__ unsigned s_phase;
    if (threadIdx.x == 0) s_phase = *a.phase;  // set by an earlier launch
    __syncthreads();
    const unsigned ph = s_phase;
    if (ph == PH_DONE) return;
    if (ph == PH_FINISH) {
      finalize_slots(a, g, t0, t1, red);
      if (!last_block(a)) return;
      global_step(a, a.R + 1, red, run, a.adm);
      if (threadIdx.x == 0) *a.phase = PH_DONE;
      return;
    }
  }
  for (int r = r_first; r <= r_last; ++r) {
    if (r >= 1) {
      const int before = s_pending;
      apply(a, r - 1, t0, t1, amax, (track || multi) ? &s_pending : nullptr,
            multi ? a.base + static_cast<size_t>(g) * a.N : nullptr, a.drem,
            multi ? a.adm : nullptr);
      __syncthreads();
      if (multi && threadIdx.x == 0 && s_pending != 0)
        atomicAdd(a.pending, static_cast<unsigned long long>(static_cast<long long>(s_pending)));
      // the placeability check runs after round 0's admission and after
      // any round that placed nothing
      if (track && r <= a.R &&
          (s_pending == 0 ||
           ((r == 1 || s_pending == before) && !any_placeable(a, r, t0, t1, amax)))) {
        finalize_slots(a, g, t0, t1, red);
        __syncthreads();
        global_step(a, a.R + 1, red, run, amax);
        __syncthreads();
        return;
      }
    }
    if (r == 0)
      propose0(a, g, t0, t1, run, act_bits, red, a.part + static_cast<size_t>(g) * a.N);
    else if (r <= a.R)
      propose_round(a, r, g, t0, t1, run, a.active, a.part + static_cast<size_t>(g) * a.N);
    else
      finalize_slots(a, g, t0, t1, red);
    if (a.G > 1) {
      if (!last_block(a)) return;
    } else {
      __syncthreads();
    }
    global_step(a, r, red, run, multi ? a.adm : amax);
    __syncthreads();
  }
}

// Multi-launch call with no serial global step (dec: 2 <= G <= DEC_MAX_G).
// Launch r runs round r in every block; what the last block's global step
// publishes in the other form, each block derives itself from the earlier
// launches' results:
//   - D, the capacity left before round r-1's admissions (LDS): D = C (from
//     R_v, each block summing the block weight totals) for r = 1, else the
//     previous launch's D (stored by block 0) minus round r-2's admitted
//     weight (the atomicMax of every block's largest admitted running
//     weight);
//   - its exclusive prefix over the earlier blocks of round r-1's proposal
//     weight, summed from their per-block totals.
// Buffers rotate by round so that no block overwrites what another block of
// the same launch may still read: part by 2, D by 2, adm by 3.  Block 0 of
// launch 0 clears adm, load_q, the drop and re-route counts and the early
// finish marker; the launch that finalises clears act_bits.  Once no
// overflowed slot is left unplaced (pending == 0 at a launch's start, r >= 2)
// that launch finalises and records itself in fin; later launches return.
constexpr int DEC_MAX_G = 128;

__device__ void cap_rounds_dec(const Args& a, int g, int r, unsigned char* smem) {
  const int tid = threadIdx.x, nthr = blockDim.x, N = a.N, G = a.G;
  // [amax: N u64][D: N i64][prefix: N i64][run / key-prefix staging]
  unsigned long long* amax = reinterpret_cast<unsigned long long*>(smem);
  int64_t* dv = reinterpret_cast<int64_t*>(smem + 8 * static_cast<size_t>(N));
  int64_t* bv = reinterpret_cast<int64_t*>(smem + 16 * static_cast<size_t>(N));
  int32_t* run = reinterpret_cast<int32_t*>(smem + 24 * static_cast<size_t>(N));
  __shared__ uint32_t act_bits[32];
  __shared__ int64_t red[32];
  __shared__ int s_pending;
  __shared__ unsigned s_fin;
  __shared__ unsigned long long s_pend;
  __shared__ double s_rv;
  const int t0 = g * a.TB, t1 = min(a.T, t0 + a.TB);
  const size_t GN = static_cast<size_t>(G) * N;
  if (r == 0) {
    if (g == 0) {
      for (int i = tid; i < 3 * N; i += nthr) a.adm[i] = 0ull;
      for (int e = tid; e < N; e += nthr) a.load_q[e] = 0;
      if (tid == 0) {
        a.stats[2] = 0;
        a.stats[3] = 0;
        *a.fin = 0u;
        *a.pending = 0ull;
      }
    }
    propose0(a, g, t0, t1, run, act_bits, red, a.part + static_cast<size_t>(g) * N);
    return;
  }
  if (tid == 0) {
    s_fin = *a.fin;
    s_pend = *a.pending;
    s_pending = 0;
  }
  __syncthreads();
  if (s_fin != 0u && s_fin < static_cast<unsigned>(r)) return;
  const bool last = r == a.R + 1;
  const bool finish = !last && r >= 2 && s_pend == 0ull;

  if (r == 1) {
    int64_t w_all = 0, w_vis = 0;
    for (int b = tid; b < G; b += nthr) {
      w_all += a.wsum[b * 4 + 0];
      w_vis += a.wsum[b * 4 + 1];
    }
    block_sum2_i64(w_all, w_vis, red);
    if (tid == 0) {
      const double rv = w_all > 0 ? static_cast<double>(w_vis) /
                                        static_cast<double>(w_all)
                                  : 0.5;
      s_rv = rv;
      if (g == 0) {
        a.r_v[0] = rv;
        a.stats[0] = w_all;
        a.stats[1] = w_vis;
      }
    }
    __syncthreads();
    const double rv = s_rv;
    for (int e = tid; e < N; e += nthr) {
      const int64_t c = capacity_of(a, rv, e);
      dv[e] = c;
      if (g == 0) {
        a.capv[e] = c;
        a.cap_q[e] = c;
        a.drem[e] = c;
      }
    }
  } else {
    const int64_t* dprev = a.drem + static_cast<size_t>((r - 2) & 1) * N;
    const unsigned long long* aprev = a.adm + static_cast<size_t>((r - 2) % 3) * N;
    for (int e = tid; e < N; e += nthr) {
      const int64_t d = dprev[e] - static_cast<int64_t>(aprev[e]);
      dv[e] = d;
      if (g == 0) {
        a.drem[static_cast<size_t>((r - 1) & 1) * N + e] = d;
        a.adm[static_cast<size_t>(r % 3) * N + e] = 0ull;
      }
    }
  }
  if (finish) {
    __syncthreads();
    finalize_slots(a, g, t0, t1, red, true);
    if (g == 0) {
      for (int e = tid; e < N; e += nthr) a.load_q[e] = a.capv[e] - dv[e];
      if (tid < 32) a.act_bits[tid] = 0u;
      if (tid == 0) *a.fin = static_cast<unsigned>(r);
    }
    return;
  }
  // this block's prefix over the earlier blocks of round r-1's proposals.
  // With N a multiple of 4, V = N / 4 threads cover a block's row with
  // 16-byte loads and P = nthr / V such groups split the earlier blocks, so
  // a thread issues all of its (at most 16) loads at once; otherwise one
  // thread per expert.  The partial sums meet in LDS in a fixed order.
  {
    const int32_t* pp = a.part + static_cast<size_t>((r - 1) & 1) * GN;
    int64_t* red64 = reinterpret_cast<int64_t*>(run);  // free until the offers
    if ((N & 3) == 0 && N / 4 <= nthr) {
      const int V = N / 4, P = max(1, min(nthr / V, g));  // no more groups than blocks
      const int v = tid % V, part = tid / V;
      int64_t acc[4] = {0, 0, 0, 0};
      if (part < P) {
        for (int b0 = part; b0 < g; b0 += 16 * P) {
          int4 x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int b = b0 + u * P;
            x[u] = b < g ? *reinterpret_cast<const int4*>(pp + static_cast<size_t>(b) * N + 4 * v)
                         : make_int4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            acc[0] += x[u].x;
            acc[1] += x[u].y;
            acc[2] += x[u].z;
            acc[3] += x[u].w;
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) red64[part * N + 4 * v + c] = acc[c];
      }
      __syncthreads();
      for (int e = tid; e < N; e += nthr) {
        int64_t t = red64[e];
        for (int q = 1; q < P; ++q) t += red64[q * N + e];
        bv[e] = t;
      }
      __syncthreads();
    } else {
      for (int e = tid; e < N; e += nthr) {
        int64_t t = 0;
        for (int b = 0; b < g; ++b) t += pp[static_cast<size_t>(b) * N + e];
        bv[e] = t;
      }
      __syncthreads();
    }
  }
  apply(a, r - 1, t0, t1, amax, &s_pending, bv, dv,
        last ? nullptr : a.adm + static_cast<size_t>((r - 1) % 3) * N);
  __syncthreads();
  if (!last) {
    if (tid == 0 && s_pending != 0)
      atomicAdd(a.pending, static_cast<unsigned long long>(static_cast<long long>(s_pending)));
    propose_round(a, r, g, t0, t1, run, nullptr,
                  a.part + static_cast<size_t>(r & 1) * GN + static_cast<size_t>(g) * N);
    return;
  }
  finalize_slots(a, g, t0, t1, red, true);
  // load = C - D + the round's admitted weight: the max over the blocks
  for (int e = tid; e < N; e += nthr) {
    const int64_t c = r == 1 ? dv[e] : a.capv[e];
    const int64_t v = c - dv[e] + static_cast<int64_t>(amax[e]);
    atomicMax(reinterpret_cast<unsigned long long*>(a.load_q + e),
              static_cast<unsigned long long>(v));
  }
  if (g == 0 && tid < 32) a.act_bits[tid] = 0u;
}

// Capacity off: everything kept; loads are the plain weight totals.
// smem: dynamic LDS [N u64].
__device__ void cap_off(const Args& a, int g, unsigned char* smem) {
  unsigned long long* tot = reinterpret_cast<unsigned long long*>(smem);
  __shared__ int64_t red[32];
  const int tid = threadIdx.x, nthr = blockDim.x, k = a.k, N = a.N;
  const int t0 = g * a.TB, t1 = min(a.T, t0 + a.TB);
  for (int e = tid; e < N; e += nthr) tot[e] = 0ull;
  __syncthreads();
  int64_t w_all = 0, w_vis = 0;
  for (int t = t0 + tid; t < t1; t += nthr) {
    const int32_t q = quant_weight(a.is_visual[t], a.entropy_w[t]);
    w_all += q;
    if (a.is_visual[t]) w_vis += q;
  }
  // one thread per slot (the token weight is recomputed, not passed along)
  for (int i = t0 * k + tid; i < t1 * k; i += nthr) {
    const int t = i / k;
    const int32_t q = quant_weight(a.is_visual[t], a.entropy_w[t]);
    const int32_t e = a.slot_in[i];
    atomicAdd(&tot[e], static_cast<unsigned long long>(q));
    a.slot_out[i] = e;
    a.flags[i] = (e != a.topk[i]) ? MOE_FLAG_SERE : 0;
  }
  block_sum2_i64(w_all, w_vis, red);
  if (tid == 0) {
    a.wsum[g * 4 + 0] = w_all;
    a.wsum[g * 4 + 1] = w_vis;
  }
  if (a.G > 1) {
    for (int e = tid; e < N; e += nthr)
      if (tot[e]) atomicAdd(&a.total[e], tot[e]);
    if (!last_block(a)) return;
  } else {
    __syncthreads();
  }
  int64_t W = w_all, Wv = w_vis;
  if (a.G > 1) {
    W = Wv = 0;
    for (int b = tid; b < a.G; b += nthr) {
      W += a.wsum[b * 4 + 0];
      Wv += a.wsum[b * 4 + 1];
    }
    block_sum2_i64(W, Wv, red);
  }
  if (tid == 0) {
    a.r_v[0] = W > 0 ? static_cast<double>(Wv) / static_cast<double>(W) : 0.5;
    a.stats[0] = W;
    a.stats[1] = Wv;
    a.stats[2] = 0;
    a.stats[3] = 0;
  }
  for (int e = tid; e < N; e += nthr) {
    if (a.G > 1) {
      a.load_q[e] = static_cast<int64_t>(a.total[e]);
      a.total[e] = 0ull;
    } else {
      a.load_q[e] = static_cast<int64_t>(tot[e]);
    }
    a.cap_q[e] = INT64_MAX;
  }
}

// ------------------------------------------------------------------ host
// Workspace: a fixed control block (zero between calls, independent of T so
// one workspace serves any batch size), then the per-call arrays.  The
// ticket's 256-byte block also holds the phase (byte 64), pending count
// (byte 128) and early-finish launch (byte 192) of a multi-launch call; the
// first launch sets them, so they need not be zero between calls.
constexpr size_t CTRL_TICKET = 0;
constexpr size_t CTRL_ACT = 256;
constexpr size_t CTRL_ADM = 512;
constexpr size_t CTRL_TOTAL = CTRL_ADM + 3 * 8 * 1024;
constexpr size_t CTRL_BYTES = CTRL_TOTAL + 8 * 1024;
constexpr int SCAN_LDS = 8192;  // int32 staging for the block-prefix scan

struct Layout {
  int G, TB, threads, dec;
  size_t wq, cur, st, incl_slot, incl_tok, offer_s, offer_c, part, base, wsum,
      capv, drem, active, bytes;
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
  L.dec = L.G > 1 && L.G <= DEC_MAX_G;
  size_t o = CTRL_BYTES;
  auto take = [&](size_t n) {
    const size_t at = o;
    o = align_up(o + n);
    return at;
  };
  const size_t Tk = static_cast<size_t>(T) * k, GN = static_cast<size_t>(L.G) * N;
  L.wq = take(sizeof(int32_t) * T);
  L.cur = take(sizeof(int32_t) * Tk);
  L.st = take(Tk);
  L.incl_slot = take(sizeof(int32_t) * Tk);
  L.incl_tok = take(sizeof(int32_t) * T);
  L.offer_s = take(sizeof(int32_t) * T);
  L.offer_c = take(sizeof(int32_t) * T);
  L.part = take(sizeof(int32_t) * GN * (L.G > 1 ? 2 : 1));
  L.base = take(sizeof(int64_t) * GN);
  L.wsum = take(sizeof(int64_t) * 4 * L.G);
  L.capv = take(sizeof(int64_t) * N);
  L.drem = take(sizeof(int64_t) * N * 2);
  L.active = take(N);
  L.bytes = o;
  return L;
}

// Argument block of one call: caller arrays plus the workspace carve-up.
inline Args make_args(const int32_t* topk_ids, const int32_t* slot_in,
                      const int32_t* fallback_ids, const uint8_t* is_visual,
                      const float* entropy_w, const int8_t* modality, int T,
                      int N, int k, int R, int group, double gamma, double lam,
                      int32_t* slot_out, uint8_t* flags, int64_t* load_q,
                      int64_t* cap_q, int64_t* stats, double* r_v, char* ws,
                      const Layout& L) {
  Args a{};
  a.topk = topk_ids;
  a.slot_in = slot_in;
  a.fallback = fallback_ids;
  a.is_visual = is_visual;
  a.entropy_w = entropy_w;
  a.modality = modality;
  a.T = T;
  a.N = N;
  a.k = k;
  a.R = R;
  a.group = group;
  int nb = 1;
  while ((1 << nb) < N) ++nb;
  a.nbits = nb;
  a.gamma = gamma;
  a.lam = lam;
  a.slot_out = slot_out;
  a.flags = flags;
  a.load_q = load_q;
  a.cap_q = cap_q;
  a.stats = stats;
  a.r_v = r_v;
  a.wq = reinterpret_cast<int32_t*>(ws + L.wq);
  a.cur = reinterpret_cast<int32_t*>(ws + L.cur);
  a.st = reinterpret_cast<uint8_t*>(ws + L.st);
  a.incl_slot = reinterpret_cast<int32_t*>(ws + L.incl_slot);
  a.incl_tok = reinterpret_cast<int32_t*>(ws + L.incl_tok);
  a.offer_s = reinterpret_cast<int32_t*>(ws + L.offer_s);
  a.offer_c = reinterpret_cast<int32_t*>(ws + L.offer_c);
  a.part = reinterpret_cast<int32_t*>(ws + L.part);
  a.base = reinterpret_cast<int64_t*>(ws + L.base);
  a.wsum = reinterpret_cast<int64_t*>(ws + L.wsum);
  a.capv = reinterpret_cast<int64_t*>(ws + L.capv);
  a.drem = reinterpret_cast<int64_t*>(ws + L.drem);
  a.active = reinterpret_cast<uint8_t*>(ws + L.active);
  a.ticket = reinterpret_cast<unsigned*>(ws + CTRL_TICKET);
  a.phase = reinterpret_cast<unsigned*>(ws + CTRL_TICKET + 64);
  a.pending = reinterpret_cast<unsigned long long*>(ws + CTRL_TICKET + 128);
  a.fin = reinterpret_cast<unsigned*>(ws + CTRL_TICKET + 192);
  a.act_bits = reinterpret_cast<uint32_t*>(ws + CTRL_ACT);
  a.adm = reinterpret_cast<unsigned long long*>(ws + CTRL_ADM);
  a.total = reinterpret_cast<unsigned long long*>(ws + CTRL_TOTAL);
  a.TB = L.TB;
  a.G = L.G;
  a.dec = L.dec;
  a.lds_scan = std::max((L.threads / MOE_WAVE) * N, SCAN_LDS);
  return a;
}

// Dynamic LDS of the capacity rounds (capacity on) and of the capacity-off
// pass.
inline size_t rounds_lds_bytes(const Args& a) {
  return sizeof(unsigned long long) * a.N + sizeof(int32_t) * a.lds_scan;
}
inline size_t off_lds_bytes(const Args& a) { return sizeof(unsigned long long) * a.N; }
inline size_t dec_lds_bytes(const Args& a) {
  return 24 * static_cast<size_t>(a.N) + sizeof(int32_t) * a.lds_scan;
}

}  // namespace cap
}  // namespace moe
