// Batch-wide routing steps of a decode batch in one workgroup: SERE
// re-routing (multi-image QA inference write-up, §4.1-§4.3), MACS weights,
// capacity and re-route-else-drop ("MACS", §3.2 Eq. 5-6, §3.3 Eq. 7, §3.1
// Eq. 3, §1 and Fig. 1) and the expert-major dispatch, run after the route
// kernel has ranked every token.
//
// The steps are a chain of short dependent phases over a few thousand
// slots, so their cost is the number of workgroup barriers and dependent
// LDS round trips, not arithmetic.  The design keeps both small:
//   - every input is read from global memory once, with all loads of a
//     thread issued before any is used; the similarity and protection rows
//     (N <= 128) are copied into LDS in the same batch;
//   - the per-expert ordered prefixes (round-0 admission, dispatch ranks)
//     give each wave a contiguous range of slots: ballots over the expert
//     id find a lane's peers, 17 ballot bit planes give its weighted prefix
//     among them, a per-wave running table carries the prefix across the
//     wave's chunks, and one scan over the waves joins them;
//   - a fallback round costs two barriers: a token's state (its slots'
//     experts, which are still overflowed, its fallback ranks) stays in the
//     registers of one thread, which sets the token's bit in the offer mask
//     of the expert it offers to; one lane per expert then takes that
//     expert's offers in token order and admits them while the running
//     weight fits the capacity left (kept in the lane's registers across
//     rounds), and each offering token reads its bit back.
// Integer sums in units of 2^-16 token make every order of summation give
// the same result as the sequential rule.
#pragma once

#include <cmath>
#include <type_traits>

#include "common.h"

namespace moe {
namespace dtail {

constexpr int NT = 512;                 // threads of the workgroup
constexpr int NW = NT / MOE_WAVE;       // 8 waves
constexpr int MAX_N = 256, MAX_T = 256, MAX_K = 16, MAX_R = 16;
constexpr int MAX_SLOTS = 2048, MAX_FB = 4096;
constexpr int SPT = MAX_SLOTS / NT;     // slots per thread
constexpr int FPT = MAX_FB / NT;        // fallback entries per thread
constexpr int SIM_LDS_N = 128;          // similarity rows kept in LDS up to this N
constexpr int OM_W = MAX_T / 64;        // 64-bit words of a token mask

enum : uint8_t { ST_OVER = 1, ST_PLACED = 2, ST_SERE = 4 };

struct Args {
  const int32_t* topk;
  const int32_t* fb;
  const uint8_t* vis;
  const float* ew;
  const int8_t* mod;
  const float* sim;
  const uint8_t* prot;
  int T, N, k, R, kprime, group, nbits;
  float rho;
  double gamma, lam;
  int cap_on, sim_lds;
  int32_t* slot_sere;
  int32_t* slot_expert;
  uint8_t* flags;
  int64_t* load_q;
  int64_t* cap_q;
  int64_t* stats;
  double* r_v;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* slot_row;
};

inline bool supported(int T, int N, int k, int R) {
  return T >= 1 && T <= MAX_T && N <= MAX_N && k <= MAX_K && R <= MAX_R &&
         T * k <= MAX_SLOTS && T * R <= MAX_FB;
}

// Dynamic LDS: the similarity and protection rows when they are kept there.
inline size_t dyn_lds(int N, bool sim_lds) {
  return sim_lds ? static_cast<size_t>(N) * N * 5 : 0;
}

__device__ __forceinline__ int32_t quant_weight(uint8_t vis, float w) {
  if (!vis) return MOE_WEIGHT_ONE;
  if (isnan(w)) w = 1.f;
  w = fminf(fmaxf(w, 0.f), 1.f);
  return static_cast<int32_t>(rintf(w * 65536.f));  // exact scale, half-even
}

// Capacity of expert e in units of 2^-16 token: one rounded double operation
// per step, left to right, no contraction.
__device__ int64_t capacity(const Args& a, double rv, int m) {
#pragma clang fp contract(off)
  const double base = ((a.gamma * static_cast<double>(a.T)) *
                       static_cast<double>(a.k)) / static_cast<double>(a.N);
  const double scale = a.lam * static_cast<double>(m);
  double c = base * (1.0 + scale * (rv - 0.5));
  c = (1.0 > c) ? 1.0 : c;
  const double cq = c * 65536.0;
  return cq >= 4611686018427387904.0 ? (int64_t(1) << 62)
                                     : static_cast<int64_t>(floor(cq));
}

// Weighted inclusive prefix of w over the lanes at or below this one whose
// key equals this lane's (peers: those lanes, from match_any).
__device__ __forceinline__ uint32_t peer_prefix(uint64_t peers, bool valid, uint32_t w) {
  const uint64_t m = peers & lanemask_le();
  uint32_t local = 0;
#pragma unroll
  for (int b = 0; b < 17; ++b) {
    const uint64_t plane = __ballot(valid && ((w >> b) & 1u));
    local += static_cast<uint32_t>(__popcll(m & plane)) << b;
  }
  return local;
}

// Makes a loaded value live in a register at this point: a batch of
// independent LDS reads followed by pin() of each value costs one wait,
// where the compiler would otherwise sink each read into the branch that
// uses it and wait for each in turn.
template <class T>
__device__ __forceinline__ void pin(T& v) {
  int x = static_cast<int>(v);
  asm volatile("" : "+v"(x));
  v = static_cast<T>(x);
}

__device__ __forceinline__ bool beats(float ov, int op, float v, int p) {
  return ov > v || (ov == v && op < p);
}

template <int CTRL>
__device__ __forceinline__ void sere_combine(float& bv, int& bp, uint32_t& bprot) {
  const float ov = dpp_t<float, CTRL>(-INFINITY, bv);
  const int op = dpp_t<int, CTRL>(INT32_MAX, bp);
  const uint32_t opr = dpp<CTRL>(0u, bprot);
  if (beats(ov, op, bv, bp)) {
    bv = ov;
    bp = op;
    bprot = opr;
  }
}

// Ordered per-expert inclusive prefix over items idx = 0..n-1 (slot order):
// wave w owns items [w*per, (w+1)*per) in chunks of 64; key(idx) < 0 means
// no item.  Returns, per chunk c of this lane (idx = w*per + 64c + lane),
// the prefix in incl[c]; afterwards run[w][e] holds the exclusive prefix of
// expert e over the earlier waves and tot[e] its total.  run must be zero on
// entry and is left holding the wave bases.  Two barriers.
template <bool UNIT, class Get>
__device__ __forceinline__ void ordered_prefix(int n, int N, int nbits, uint32_t* run,
                                               uint32_t* tot, Get get,
                                               uint32_t (&incl)[SPT], int (&key)[SPT]) {
  const int tid = threadIdx.x, wave = tid / MOE_WAVE, lane = lane_id();
  const int per = (((n + NW - 1) / NW) + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
  uint32_t* myrun = run + wave * MAX_N;
#pragma unroll
  for (int c = 0; c < SPT; ++c) {
    const int idx = wave * per + c * MOE_WAVE + lane;
    int e = -1;
    uint32_t w = 0;
    if (c * MOE_WAVE < per && idx < n) get(idx, e, w);
    key[c] = e;
    incl[c] = 0;
    if (c * MOE_WAVE >= per) continue;  // uniform: per is the same in every lane
    const bool valid = e >= 0;
    const uint64_t peers = match_any(e, valid, nbits);
    const uint32_t local = UNIT ? static_cast<uint32_t>(__popcll(peers & lanemask_le()))
                                : peer_prefix(peers, valid, w);
    if (valid) {
      const uint32_t inc = myrun[e] + local;
      incl[c] = inc;
      if (lane == 63 - __clzll(static_cast<long long>(peers))) myrun[e] = inc;
    }
  }
  __syncthreads();
  // exclusive scan over the waves of every expert (8 consecutive lanes)
  for (int i = tid; i < NW * N; i += NT) {
    const int e = i / NW, v = i % NW;
    const int32_t x = static_cast<int32_t>(run[v * MAX_N + e]);
    int32_t t;
    const int32_t ex = group_excl_scan<NW>(x, &t);
    run[v * MAX_N + e] = static_cast<uint32_t>(ex);
    if (v == 0) tot[e] = static_cast<uint32_t>(t);
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < SPT; ++c)
    if (key[c] >= 0) incl[c] += myrun[key[c]];
}

// LDS of the compact tail (every instantiation of run() shares one block).
struct Lds {
  int16_t s_e[MAX_SLOTS];      // router experts, then final experts
  int16_t s_cur[MAX_SLOTS];    // post-SERE experts, then placed ones
  uint8_t s_st[MAX_SLOTS];
  int16_t s_fb[MAX_FB];
  int32_t s_wq[MAX_T];
  uint8_t s_inp[MAX_N], s_sec[MAX_N], s_active[MAX_N];
  int16_t s_target[MAX_N];
  uint32_t s_run[NW * MAX_N];   // round 0
  uint32_t s_drun[NW * MAX_N];  // dispatch
  uint32_t s_tot[MAX_N];
  int32_t s_cap[MAX_N];        // capacity, clamped to 2^30
  uint32_t s_load0[MAX_N];
  uint32_t s_U[MAX_N];          // weight placed by the fallback rounds
  unsigned long long s_om[2 * MAX_N * OM_W];  // offer masks, by round parity
  unsigned long long s_load_off[MAX_N];
  int32_t s_off[MAX_N + 1];
  unsigned long long s_sum[4];  // W, W_vis, dropped, re-routed
  uint8_t s_pend[8];            // token waves with a pending overflow, by round parity
};

// The batch-wide steps, run by one workgroup of NT threads once every
// token's ranks are visible in a.topk and a.fb; k <= MK and R <= MR (the
// per-token loops of the fallback rounds are unrolled to these bounds).
// dyn: dynamic LDS of at least dyn_lds(N, a.sim_lds) bytes
// ([N*N f32 sim][N*N u8 prot]).
template <int MK, int MR>
__device__ __forceinline__ void run(const Args& a, unsigned char* dyn, Lds& L) {
  auto& s_e = L.s_e;
  auto& s_cur = L.s_cur;
  auto& s_st = L.s_st;
  auto& s_fb = L.s_fb;
  auto& s_wq = L.s_wq;
  auto& s_inp = L.s_inp;
  auto& s_sec = L.s_sec;
  auto& s_active = L.s_active;
  auto& s_target = L.s_target;
  auto& s_run = L.s_run;
  auto& s_drun = L.s_drun;
  auto& s_tot = L.s_tot;
  auto& s_cap = L.s_cap;
  auto& s_load0 = L.s_load0;
  auto& s_U = L.s_U;
  auto& s_om = L.s_om;
  auto& s_load_off = L.s_load_off;
  auto& s_off = L.s_off;
  auto& s_sum = L.s_sum;
  auto& s_pend = L.s_pend;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int T = a.T, N = a.N, k = a.k, R = a.R, Tk = T * k, TR = T * R;
  const bool sere = a.kprime > 0;
  float* s_sim = reinterpret_cast<float*>(dyn);
  uint8_t* s_prot = dyn + static_cast<size_t>(N) * N * 4;

  // ---- every input, one batch of loads: each issued unconditionally at a
  // clamped index and held (pin) until all are issued, so the batch costs
  // one round trip (a load behind a per-lane condition is waited for on its
  // own); the lane conditions apply afterwards.  (Ids are clamped to
  // [0, N): an id out of range could never index past an array.)
  int e_in[SPT], fbv[FPT];
  uint8_t vis;
  float ew;
  int mod;
  {
    int re[SPT], rf[FPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) re[j] = a.topk[min(tid + j * NT, Tk - 1)];
    const int32_t* fbp = TR > 0 ? a.fb : a.topk;  // (R = 0: no fallback array)
    const int fbn = TR > 0 ? TR : Tk;
#pragma unroll
    for (int j = 0; j < FPT; ++j) rf[j] = fbp[min(tid + j * NT, fbn - 1)];
    int rv = a.vis[min(tid, T - 1)];
    float rw = a.ew[min(tid, T - 1)];
    int rm = a.mod[min(tid, N - 1)];
#pragma unroll
    for (int j = 0; j < SPT; ++j) pin(re[j]);
#pragma unroll
    for (int j = 0; j < FPT; ++j) pin(rf[j]);
    pin(rv);
    pin(rm);
    int rwi = __float_as_int(rw);
    pin(rwi);
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      e_in[j] = tid + j * NT < Tk ? min(max(re[j], 0), N - 1) : -1;
#pragma unroll
    for (int j = 0; j < FPT; ++j)
      fbv[j] = tid + j * NT < TR ? min(max(rf[j], 0), N - 1) : 0;
    vis = tid < T ? static_cast<uint8_t>(rv) : 0;
    ew = tid < T ? __int_as_float(rwi) : 0.f;
    mod = tid < N ? rm : 0;
  }
  if (sere && a.sim_lds) {
    // N <= 128: every thread issues all its 16-byte loads (8 of the rows,
    // 2 of the protection bytes) before the first store, so the copy costs
    // one memory round trip (issued after the batch above, not with it:
    // one batch of both measured slower)
    const int nn = N * N;
    if ((nn & 15) == 0 && ((reinterpret_cast<uintptr_t>(a.sim) |
                           reinterpret_cast<uintptr_t>(a.prot)) & 15) == 0) {
      constexpr int QS = SIM_LDS_N * SIM_LDS_N / 4 / NT, QP = SIM_LDS_N * SIM_LDS_N / 16 / NT;
      const int n4 = nn / 4, n16 = nn / 16;
      float4 sv[QS];
      uint4 pv[QP];
      // (clamped indices: every load in bounds, the extra ones unused)
#pragma unroll
      for (int j = 0; j < QS; ++j)
        sv[j] = reinterpret_cast<const float4*>(a.sim)[min(tid + j * NT, n4 - 1)];
#pragma unroll
      for (int j = 0; j < QP; ++j)
        pv[j] = reinterpret_cast<const uint4*>(a.prot)[min(tid + j * NT, n16 - 1)];
      // held until all are issued (each value's only use is a guarded store,
      // into which the compiler would otherwise sink its load and wait)
#pragma unroll
      for (int j = 0; j < QS; ++j)
        asm volatile("" : "+v"(sv[j].x), "+v"(sv[j].y), "+v"(sv[j].z), "+v"(sv[j].w));
#pragma unroll
      for (int j = 0; j < QP; ++j)
        asm volatile("" : "+v"(pv[j].x), "+v"(pv[j].y), "+v"(pv[j].z), "+v"(pv[j].w));
#pragma unroll
      for (int j = 0; j < QS; ++j) {
        const int q = tid + j * NT;
        if (q < n4) reinterpret_cast<float4*>(s_sim)[q] = sv[j];
      }
#pragma unroll
      for (int j = 0; j < QP; ++j) {
        const int q = tid + j * NT;
        if (q < n16) reinterpret_cast<uint4*>(s_prot)[q] = pv[j];
      }
    } else {
      for (int q = tid; q < nn; q += NT) {
        s_sim[q] = a.sim[q];
        s_prot[q] = a.prot[q];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = tid + j * NT;
    if (i < Tk) s_e[i] = static_cast<int16_t>(e_in[j]);
  }
#pragma unroll
  for (int j = 0; j < FPT; ++j) {
    const int i = tid + j * NT;
    if (i < TR) s_fb[i] = static_cast<int16_t>(fbv[j]);
  }
  const int32_t wq = tid < T ? quant_weight(vis, ew) : 0;
  if (tid < T) s_wq[tid] = wq;
  for (int i = tid; i < NW * MAX_N; i += NT) {
    s_run[i] = 0u;
    s_drun[i] = 0u;
  }
  for (int i = tid; i < 2 * MAX_N * OM_W; i += NT) s_om[i] = 0ull;
  if (tid < MAX_N) {
    s_inp[tid] = 0;
    s_sec[tid] = 0;
    s_active[tid] = 0;
    s_load0[tid] = 0u;
    s_U[tid] = 0u;
    s_load_off[tid] = 0ull;
  }
  if (tid < 4) s_sum[tid] = 0ull;
  __syncthreads();

  // ---- token weights: W and W_vis (integer sums, any order)
  {
    const int64_t wa = wave_sum_i64(wq), wv = wave_sum_i64(vis ? wq : 0);
    if (lane == 0 && (wa | wv)) {
      atomicAdd(&s_sum[0], static_cast<unsigned long long>(wa));
      atomicAdd(&s_sum[1], static_cast<unsigned long long>(wv));
    }
  }

  // ---- SERE: primary union P, one target per movable expert, slots moved
  int slot_pos[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = tid + j * NT;
    slot_pos[j] = i < Tk ? i % k : 0;
  }
  int cur_in[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) cur_in[j] = e_in[j];
  if (sere) {
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (e_in[j] >= 0) {
        if (slot_pos[j] < a.kprime) s_inp[e_in[j]] = 1;
        else s_sec[e_in[j]] = 1;
      }
    __syncthreads();
    // LPE lanes per expert, each over every LPE-th primary in ascending
    // order; candidates combined with quad DPP steps (all lanes take part)
    const int LPE = N <= 128 ? 4 : 2;
    const int e = tid / LPE, sub = tid % LPE;
    const bool mv = e < N && s_sec[e] && !s_inp[e];
    float bv = -INFINITY;
    int bp = INT32_MAX;
    uint32_t bprot = 0u;
    if (a.sim_lds) {
      // P as a bit mask (N <= 128: two words, the same in every lane); lane
      // sub scans the 32 columns [32 sub, 32 sub + 32) of row e: all 32
      // reads issued at once, then the compares in registers.  The 16
      // experts of a wave start at different columns (rotation by e), so
      // their rows, 128 words apart, do not hit one LDS bank together; the
      // compare (value, then the lower column) does not depend on the order
      // the columns are visited in.
      const uint64_t pm0 = __ballot(lane < N && s_inp[lane]);
      const uint64_t pm1 = __ballot(lane + 64 < N && s_inp[lane + 64]);
      if (mv) {
        const float* srow = s_sim + static_cast<size_t>(e) * N;
        const int p0 = sub * 32, rot = e & 31;
        float v[32];
#pragma unroll
        for (int q = 0; q < 32; ++q)  // (clamped: columns past N have no primary bit)
          v[q] = srow[min(p0 + ((q + rot) & 31), N - 1)];
        const uint64_t pw = sub < 2 ? pm0 : pm1;
        const uint32_t bits = static_cast<uint32_t>(pw >> ((sub & 1) * 32));
        // branch-free: the test of beats() with bitwise operators and two
        // selects per column (short-circuit forms compile to a divergent
        // branch per column)
#pragma unroll
        for (int q = 0; q < 32; ++q) {
          const int c = (q + rot) & 31, pc = p0 + c;
          const bool take = ((bits >> c) & 1u) != 0u &
                            ((v[q] > bv) | ((v[q] == bv) & (pc < bp)));
          bv = take ? v[q] : bv;
          bp = take ? pc : bp;
        }
      }
    } else if (mv) {
      const float* srow = a.sim + static_cast<size_t>(e) * N;
      const uint8_t* prow = a.prot + static_cast<size_t>(e) * N;
      for (int p = sub; p < N; p += LPE) {
        if (!s_inp[p]) continue;
        const float sv = srow[p];
        if (bp == INT32_MAX || sv > bv) {
          bv = sv;
          bp = p;
          bprot = prow[p];
        }
      }
    }
    sere_combine<DPP_QUAD_1032>(bv, bp, bprot);
    if (LPE == 4) sere_combine<DPP_QUAD_2301>(bv, bp, bprot);
    // the protection byte of the winner only (the LDS copy; the global
    // path carried it along)
    if (a.sim_lds && mv && sub == 0 && bp != INT32_MAX) bprot = s_prot[e * N + bp];
    if (e < N && sub == 0)
      s_target[e] = static_cast<int16_t>(
          mv && bp != INT32_MAX && bv > a.rho && bprot == 0u ? bp : e);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = tid + j * NT;
      if (e_in[j] < 0) continue;
      const int ee = e_in[j];
      const int o = (slot_pos[j] >= a.kprime && !s_inp[ee]) ? s_target[ee] : ee;
      cur_in[j] = o;
      a.slot_sere[i] = o;
    }
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = tid + j * NT;
    if (e_in[j] < 0) continue;
    s_cur[i] = static_cast<int16_t>(cur_in[j]);
    s_st[i] = cur_in[j] != e_in[j] ? ST_SERE : 0;
  }
  __syncthreads();  // s_cur / s_st / W sums complete

  // ---- R_v and the capacities
  const int64_t W = static_cast<int64_t>(s_sum[0]), Wv = static_cast<int64_t>(s_sum[1]);
  const double rv = W > 0 ? static_cast<double>(Wv) / static_cast<double>(W) : 0.5;
  if (tid == 0) {
    a.r_v[0] = rv;
    a.stats[0] = W;
    a.stats[1] = Wv;
  }
  if (tid < N) {
    if (a.cap_on) {
      const int64_t c = capacity(a, rv, mod);
      a.cap_q[tid] = c;
      s_cap[tid] = static_cast<int32_t>(c < (int64_t(1) << 30) ? c : (int64_t(1) << 30));
    } else {
      a.cap_q[tid] = INT64_MAX;
    }
  }

  uint32_t incl[SPT];
  int key[SPT];
  if (!a.cap_on) {
    // capacity off: everything kept, the load is the plain weight total
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = tid + j * NT;
      if (e_in[j] < 0) continue;
      atomicAdd(&s_load_off[cur_in[j]], static_cast<unsigned long long>(s_wq[i / k]));
    }
  } else {
    __syncthreads();  // s_cap
    // ---- round 0: per-expert running weight in (token, slot) order
    ordered_prefix<false>(Tk, N, a.nbits, s_run, s_tot,
                          [&](int idx, int& e, uint32_t& w) {
                            e = s_cur[idx];
                            w = static_cast<uint32_t>(s_wq[idx / k]);
                          },
                          incl, key);
    const int per = (((Tk + NW - 1) / NW) + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
#pragma unroll
    for (int c = 0; c < SPT; ++c) {
      const int e = key[c];
      if (e < 0) continue;
      const int idx = wave * per + c * MOE_WAVE + lane;
      s_active[e] = 1;
      if (static_cast<int32_t>(incl[c]) <= s_cap[e])
        atomicMax(&s_load0[e], incl[c]);  // kept slots of e form a prefix
      else
        s_st[idx] |= ST_OVER;
    }
    __syncthreads();

    // ---- fallback rounds: thread t owns token t.  Every LDS read below is
    // issued unconditionally (clamped index) and its value pinned right after
    // the batch (pin), so that the compiler cannot sink each read into the
    // branch that uses it and wait for it there: a batch costs one round trip.
    const bool tok = tid < T;
    int cur[MK];
    uint32_t over = 0u, placed = 0u;
    {
      int cv[MK];
      uint8_t sv[MK];
#pragma unroll
      for (int s = 0; s < MK; ++s) {
        const int i = min(tid * k + s, MAX_SLOTS - 1);
        cv[s] = s_cur[i];
        sv[s] = s_st[i];
      }
#pragma unroll
      for (int s = 0; s < MK; ++s) {
        pin(cv[s]);
        pin(sv[s]);
      }
#pragma unroll
      for (int s = 0; s < MK; ++s) {
        const bool own = tok && s < k;
        cur[s] = own ? cv[s] : -1;
        if (own && (sv[s] & ST_OVER)) over |= 1u << s;
      }
    }
    const int tw = (T + MOE_WAVE - 1) / MOE_WAVE;  // waves holding tokens
    int fbr[MR];
#pragma unroll
    for (int q = 0; q < MR; ++q) {
      fbr[q] = s_fb[min(tid * R + q, MAX_FB - 1)];
    }
#pragma unroll
    for (int q = 0; q < MR; ++q) pin(fbr[q]);
#pragma unroll
    for (int q = 0; q < MR; ++q) fbr[q] = tok && q < R ? fbr[q] : 0;
    // A (experts with a round-0 proposer) as four 64-bit words, the same in
    // every lane (entries past N are zero)
    uint64_t am[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool f = s_active[q * 64 + lane] != 0;
      am[q] = __ballot(f);
    }
    // the token's fallback ranks that could still be offered: in A and not
    // held for good by a kept slot (A is fixed; a kept or placed slot never
    // moves, so its expert stays held; an overflowed slot's expert is held
    // only until that slot is placed elsewhere, so it does not rule a rank
    // out here); the full held test and the group test stay at the offer.
    // Rounds stop once no token with an unplaced overflowed slot has a
    // candidate left: no later round could offer anything.  A token's
    // fallback ids are distinct, so placing a slot rules out no other rank.
    uint32_t cand = 0u;
    if (tok && over) {
#pragma unroll
      for (int q = 0; q < MR; ++q) {
        const int c = fbr[q];
        bool held = false;
#pragma unroll
        for (int s = 0; s < MK; ++s) held |= !((over >> s) & 1u) && cur[s] == c;
        const uint64_t aw = c < 64 ? am[0] : c < 128 ? am[1] : c < 192 ? am[2] : am[3];
        if (q < R && ((aw >> (c & 63)) & 1u) && !held) cand |= 1u << q;
      }
    }
    // Admission of a round's offers to expert c: in token order, while the
    // running weight stays within the capacity left.  Weights are
    // non-negative, so the running weight never falls: the admitted offers
    // are the ones before the first refusal, and lane c of the walker waves
    // (threads below N) takes the set bits of c's offer mask lowest first
    // and stops there.  It keeps c's capacity left in a register across
    // rounds, writes the admitted bits back over the mask and clears the
    // other parity's mask for the next round.
    int32_t rem = 0;
    uint32_t placed_w = 0;
    if (tid < N) rem = s_cap[tid] - static_cast<int32_t>(s_load0[tid]);
    // ONE: every expert in one group (no group test, no division).  The
    // rounds are unrolled, so the candidate of round r and the earlier
    // rounds' admissions are static register indices.
    auto rounds = [&](auto one_tag) {
      constexpr bool ONE = decltype(one_tag)::value;
      int fbg[MR], cg[MK];  // expert groups, up front
      if constexpr (!ONE) {
#pragma unroll
        for (int q = 0; q < MR; ++q) fbg[q] = fbr[q] / a.group;
#pragma unroll
        for (int s = 0; s < MK; ++s) cg[s] = cur[s] < 0 ? 0 : cur[s] / a.group;
      }
#pragma unroll
      for (int r = 1; r <= MR; ++r) {
        if (r > R) break;
        bool offer = false;
        const int c = fbr[r - 1];
        int s0 = 0;
        unsigned long long* om = s_om + (r & 1) * MAX_N * OM_W;
        if (wave < tw) {  // uniform: waves without tokens only meet the barriers
          if (tok && over && ((cand >> (r - 1)) & 1u)) {
            s0 = __builtin_ctz(over);
            bool held = false;
#pragma unroll
            for (int s = 0; s < MK; ++s) held |= cur[s] == c;
            bool same_group = true;
            if constexpr (!ONE) {
              int g0 = 0;  // the offered slot's group (static indices)
#pragma unroll
              for (int s = 0; s < MK; ++s)
                if (s == s0) g0 = cg[s];
              same_group = g0 == fbg[r - 1];
            }
            offer = !held && same_group;
          }
          if (offer) atomicOr(&om[c * OM_W + (tid >> 6)], 1ull << (tid & 63));
          // this wave's pending flag for round r (parity slot)
          const bool pend = __ballot(over != 0u && (cand >> (r - 1)) != 0u) != 0ull;
          if (lane == 0) s_pend[(r & 1) * 4 + wave] = pend;
        }
        // publishes the masks and the flags: stop once no token has an
        // unplaced overflowed slot (no later round could offer anything)
        __syncthreads();
        bool any = false;
        {
          uint8_t pv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) pv[v] = s_pend[(r & 1) * 4 + v];
#pragma unroll
          for (int v = 0; v < 4; ++v) any |= v < tw && pv[v] != 0;
        }
        if (!any) break;
        if (tid < N) {
          unsigned long long m[OM_W];
#pragma unroll
          for (int w = 0; w < OM_W; ++w) m[w] = om[tid * OM_W + w];
#pragma unroll
          for (int w = 0; w < OM_W; ++w) {  // both halves held, as pin() does
            uint32_t lo = static_cast<uint32_t>(m[w]), hi = static_cast<uint32_t>(m[w] >> 32);
            asm volatile("" : "+v"(lo), "+v"(hi));
            m[w] = (static_cast<unsigned long long>(hi) << 32) | lo;
          }
          uint32_t run = 0;
          bool stop = false;
#pragma unroll
          for (int w = 0; w < OM_W; ++w) {
            unsigned long long left = m[w], adm = 0ull;
            while (left != 0ull && !stop) {
              const int b = __builtin_ctzll(left);
              const uint32_t x = static_cast<uint32_t>(s_wq[w * 64 + b]);
              if (static_cast<int32_t>(run + x) <= rem) {
                run += x;
                adm |= 1ull << b;
              } else {
                stop = true;
              }
              left &= left - 1;
            }
            om[tid * OM_W + w] = adm;
            s_om[((r + 1) & 1) * MAX_N * OM_W + tid * OM_W + w] = 0ull;
          }
          rem -= static_cast<int32_t>(run);
          placed_w += run;
        }
        __syncthreads();  // the admitted bits
        if (offer && ((om[c * OM_W + (tid >> 6)] >> (tid & 63)) & 1ull)) {
#pragma unroll
          for (int s = 0; s < MK; ++s)
            if (s == s0) {
              cur[s] = c;
              if constexpr (!ONE) cg[s] = fbg[r - 1];
            }
          over &= ~(1u << s0);
          placed |= 1u << s0;
        }
      }
    };
    if (a.group >= N)
      rounds(std::true_type{});
    else
      rounds(std::false_type{});
    if (tid < N) s_U[tid] = placed_w;
    if (tok) {
#pragma unroll
      for (int s = 0; s < MK; ++s)
        if (s < k) {
          const int i = tid * k + s;
          s_cur[i] = static_cast<int16_t>(cur[s]);
          s_st[i] = (s_st[i] & ST_SERE) | ((over >> s) & 1u ? ST_OVER : 0) |
                    ((placed >> s) & 1u ? ST_PLACED : 0);
        }
    }
  }
  __syncthreads();  // final slots; for capacity off, the loads

  // ---- final slots, flags, loads and counts
  {
    uint32_t n_drop = 0, n_macs = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = tid + j * NT;
      if (i >= Tk) continue;
      const uint8_t st = s_st[i];
      uint8_t f = (st & ST_SERE) ? MOE_FLAG_SERE : 0;
      int o = s_cur[i];
      if (st & ST_OVER) {
        o = -1;
        f |= MOE_FLAG_DROP;
        ++n_drop;
      } else if (st & ST_PLACED) {
        f |= MOE_FLAG_MACS;
        ++n_macs;
      }
      a.slot_expert[i] = o;
      a.flags[i] = f;
      s_e[i] = static_cast<int16_t>(o);
    }
    n_drop = wave_sum(n_drop);
    n_macs = wave_sum(n_macs);
    if (lane == 0 && (n_drop | n_macs)) {
      atomicAdd(&s_sum[2], static_cast<unsigned long long>(n_drop));
      atomicAdd(&s_sum[3], static_cast<unsigned long long>(n_macs));
    }
    if (tid < N) {
      int64_t l;
      if (a.cap_on) {
        l = static_cast<int64_t>(s_load0[tid]) + s_U[tid];
      } else {
        l = static_cast<int64_t>(s_load_off[tid]);
      }
      a.load_q[tid] = l;
    }
  }
  __syncthreads();
  if (tid == 0) {
    a.stats[2] = static_cast<int64_t>(s_sum[2]);
    a.stats[3] = static_cast<int64_t>(s_sum[3]);
  }

  // ---- dispatch: rank of every kept slot inside its expert, (t,s) order
  ordered_prefix<true>(Tk, N, a.nbits, s_drun, s_tot,
                       [&](int idx, int& e, uint32_t& w) {
                         e = s_e[idx];
                         w = 1u;
                       },
                       incl, key);
  // expert offsets: exclusive scan of the totals (wave 0, 4 experts a lane)
  if (wave == 0) {
    int32_t v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      v[q] = e < N ? static_cast<int32_t>(s_tot[e]) : 0;
      sum += v[q];
    }
    const int32_t incl_sum = wave_incl_scan(sum);
    int32_t run = incl_sum - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      if (e < N) s_off[e] = run;
      run += v[q];
    }
    if (lane == 63) s_off[N] = incl_sum;
  }
  __syncthreads();
  if (tid <= N) a.offsets[tid] = s_off[tid];
  const int per = (((Tk + NW - 1) / NW) + MOE_WAVE - 1) / MOE_WAVE * MOE_WAVE;
#pragma unroll
  for (int c = 0; c < SPT; ++c) {
    const int idx = wave * per + c * MOE_WAVE + lane;
    if (c * MOE_WAVE >= per || idx >= Tk) continue;
    const int e = key[c];
    if (e < 0) {
      a.slot_row[idx] = -1;
      continue;
    }
    const int row = s_off[e] + static_cast<int>(incl[c]) - 1;
    a.slot_row[idx] = row;
    a.row_token[row] = idx / k;
    a.row_slot[row] = idx % k;
  }
}

}  // namespace dtail
}  // namespace moe
