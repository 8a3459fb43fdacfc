// moe_routing_fused: router top-k, SERE re-routing, MACS capacity with
// re-route-else-drop, and dispatch in ONE launch, for decode-sized batches
// ("MACS", §3.1 Eq. 1 and Eq. 3, §3.2 Eq. 5-6, §3.3 Eq. 7, §1 and Fig. 1;
// multi-image QA inference write-up, §4.1-§4.3: the re-route operator is a
// single fused kernel with no host round trip and feeds the fused MoE
// directly).
//
// The grid routes the tokens (one group of GT threads per token, rank
// counting in LDS).  The workgroup that finishes last (atomic ticket that
// wraps back to zero) sees every token's ranks and runs the batch-wide
// steps on its own: the SERE union and re-route, the capacity rounds (all of
// them, or the capacity-off pass), and the counting sort into expert-major
// rows.  Each step is the same device code as the stand-alone entry points,
// so the results are identical to calling them in order.
//
// The batch-wide steps are a chain of short dependent phases, so each
// global-memory round trip would cost about a microsecond.  The last
// workgroup therefore loads every per-slot and per-token input into LDS
// with one batch of independent loads, runs every phase on LDS copies (the
// workspace arrays and control words of the capacity and dispatch steps
// live in LDS too), and writes the results out once, coalesced.  Shapes
// whose tail does not fit in LDS are not supported here (the separate entry
// points cover them).
#include <atomic>
#include <cmath>

#include "capacity_impl.h"
#include "dispatch_impl.h"
#include "dtail_impl.h"
#include "route_impl.h"
#include "sere_impl.h"
#include "tiny_impl.h"

namespace moe {
namespace fused {

// Byte offsets of the tail's arrays in dynamic LDS (16-byte aligned).
struct TailLayout {
  unsigned topk, fb, sere, slot, flags, vis, ew, mod;  // inputs and outputs
  unsigned wq, cur, st, incl_slot, incl_tok, offer_s, offer_c;  // capacity
  unsigned part, base, wsum, capv, drem, active, act_bits, adm, total;
  unsigned drank, dpart, dbase, doff;  // dispatch
  unsigned scratch;                    // phase scratch: [N u64][W*N int32]
  unsigned bytes;
  int lds_scan;
};

// Dynamic LDS the tail may use (the static LDS of the kernel comes on top).
constexpr size_t TAIL_LDS_MAX = 150 * 1024;

// Threads per workgroup.  The tail runs a long chain of short phases, and
// every wave executes each phase's whole instruction stream, so more waves
// cost more instruction issue, fewer waves longer loops and less latency
// hiding.  Measured on the qwen3 decode batch (tail and route phase
// together): 16 waves 20.1 us, 8 waves 19.1 us, 4 waves 24.8 us; on a
// 256-token batch with capacity rounds: 91.7, 85.9, 99.7 us.
#ifndef MOE_FUSED_THREADS
#define MOE_FUSED_THREADS 512
#endif
constexpr int FT = MOE_FUSED_THREADS;
static_assert(FT == 256 || FT == 512 || FT == 1024, "fused workgroup size");

__host__ __device__ inline TailLayout tail_layout(int T, int N, int k, int R,
                                                  int waves) {
  TailLayout L{};
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o = (o + n + 15) & ~size_t(15);
    return static_cast<unsigned>(at);
  };
  const size_t Tk = static_cast<size_t>(T) * k;
  L.topk = take(4 * Tk);
  L.fb = take(4 * static_cast<size_t>(T) * R);
  L.sere = take(4 * Tk);
  L.slot = take(4 * Tk);
  L.flags = take(Tk);
  L.vis = take(T);
  L.ew = take(4 * static_cast<size_t>(T));
  L.mod = take(N);
  L.wq = take(4 * static_cast<size_t>(T));
  L.cur = take(4 * Tk);
  L.st = take(Tk);
  L.incl_slot = take(4 * Tk);
  L.incl_tok = take(4 * static_cast<size_t>(T));
  L.offer_s = take(4 * static_cast<size_t>(T));
  L.offer_c = take(4 * static_cast<size_t>(T));
  L.part = take(4 * static_cast<size_t>(N));
  L.base = take(8 * static_cast<size_t>(N));
  L.wsum = take(8 * 4);
  L.capv = take(8 * static_cast<size_t>(N));
  L.drem = take(8 * static_cast<size_t>(N));
  L.active = take(N);
  L.act_bits = take(4 * 32);
  L.adm = take(8 * static_cast<size_t>(N));
  L.total = take(8 * static_cast<size_t>(N));
  L.drank = take(4 * Tk);
  L.dpart = take(4 * static_cast<size_t>(N));
  L.dbase = take(4 * static_cast<size_t>(N));
  L.doff = take(4 * (static_cast<size_t>(N) + 1));
  L.lds_scan = waves * N;
  L.scratch = take(8 * static_cast<size_t>(N) + 4 * static_cast<size_t>(L.lds_scan));
  L.bytes = static_cast<unsigned>(o);
  return L;
}

struct Args {
  const float* logits;
  const float* sim;
  const uint8_t* prot;
  int32_t* topk_ids;
  float* topk_gates;
  int32_t* fallback_ids;
  int32_t* slot_sere;
  int32_t* slot_expert;
  uint8_t* flags;
  int32_t* expert_offsets;
  int T, N, k, R, kprime;
  float rho;
  bool cap_on;
  unsigned* ticket;
  TailLayout tl;
};

// The batch-wide steps, run by the last workgroup on LDS copies.  cg and dg
// carry the caller's inputs and outputs; their workspace pointers are
// replaced by LDS arrays here.
__device__ void tail(const Args& f, const cap::Args& cg, const disp::Args& dg,
                     unsigned char* smem, sr::SereLds& sl) {
  const TailLayout& L = f.tl;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int T = f.T, N = f.N, k = f.k, R = f.R;
  const int Tk = T * k, TR = T * R;
  int32_t* topk = reinterpret_cast<int32_t*>(smem + L.topk);
  int32_t* fb = reinterpret_cast<int32_t*>(smem + L.fb);
  int32_t* sere = reinterpret_cast<int32_t*>(smem + L.sere);
  int32_t* slot = reinterpret_cast<int32_t*>(smem + L.slot);
  uint8_t* flags = smem + L.flags;
  uint8_t* vis = smem + L.vis;
  float* ew = reinterpret_cast<float*>(smem + L.ew);
  int8_t* mod = reinterpret_cast<int8_t*>(smem + L.mod);
  uint32_t* act_bits = reinterpret_cast<uint32_t*>(smem + L.act_bits);
  unsigned long long* adm = reinterpret_cast<unsigned long long*>(smem + L.adm);
  unsigned long long* total = reinterpret_cast<unsigned long long*>(smem + L.total);
  int32_t* doff = reinterpret_cast<int32_t*>(smem + L.doff);

  // one batch of independent loads brings every input in; the control
  // words start at zero
  const int n_in = max(max(Tk, TR), max(T, N));
  for (int i = tid; i < n_in; i += nthr) {
    if (i < Tk) topk[i] = f.topk_ids[i];
    if (i < TR) fb[i] = f.fallback_ids[i];
    if (i < T) {
      vis[i] = cg.is_visual[i];
      ew[i] = cg.entropy_w[i];
    }
    if (i < N) {
      mod[i] = cg.modality[i];
      adm[i] = 0ull;
      total[i] = 0ull;
    }
    if (i < 32) act_bits[i] = 0u;
  }
  __syncthreads();

  const int32_t* slot_in = topk;
  if (f.kprime > 0) {
    sr::sere_block(topk, T, N, k, f.kprime, f.rho, f.sim, f.prot, sere, flags, sl);
    __syncthreads();
    slot_in = sere;
  }

  cap::Args c = cg;
  c.topk = topk;
  c.slot_in = slot_in;
  c.fallback = fb;
  c.is_visual = vis;
  c.entropy_w = ew;
  c.modality = mod;
  c.slot_out = slot;
  c.flags = flags;
  c.wq = reinterpret_cast<int32_t*>(smem + L.wq);
  c.cur = reinterpret_cast<int32_t*>(smem + L.cur);
  c.st = smem + L.st;
  c.incl_slot = reinterpret_cast<int32_t*>(smem + L.incl_slot);
  c.incl_tok = reinterpret_cast<int32_t*>(smem + L.incl_tok);
  c.offer_s = reinterpret_cast<int32_t*>(smem + L.offer_s);
  c.offer_c = reinterpret_cast<int32_t*>(smem + L.offer_c);
  c.part = reinterpret_cast<int32_t*>(smem + L.part);
  c.base = reinterpret_cast<int64_t*>(smem + L.base);
  c.wsum = reinterpret_cast<int64_t*>(smem + L.wsum);
  c.capv = reinterpret_cast<int64_t*>(smem + L.capv);
  c.drem = reinterpret_cast<int64_t*>(smem + L.drem);
  c.active = smem + L.active;
  c.ticket = nullptr;
  c.act_bits = act_bits;
  c.adm = adm;
  c.total = total;
  c.lds_scan = L.lds_scan;
  if (f.cap_on)
    cap::cap_rounds(c, 0, 0, R + 1, smem + L.scratch);
  else
    cap::cap_off(c, 0, smem + L.scratch);
  __syncthreads();

  disp::Args d = dg;
  d.slot = slot;
  d.offsets = doff;
  d.rank = reinterpret_cast<int32_t*>(smem + L.drank);
  d.part = reinterpret_cast<int32_t*>(smem + L.dpart);
  d.base = reinterpret_cast<int32_t*>(smem + L.dbase);
  d.ticket = nullptr;
  d.lds_scan = L.lds_scan;
  disp::dispatch_single(d, smem + L.scratch);
  __syncthreads();

  const int n_out = max(Tk, N + 1);
  for (int i = tid; i < n_out; i += nthr) {
    if (i < Tk) {
      f.slot_expert[i] = slot[i];
      f.flags[i] = flags[i];
      if (f.kprime > 0) f.slot_sere[i] = sere[i];
    }
    if (i <= N) f.expert_offsets[i] = doff[i];
  }
}

// DT: the batch-wide steps run as dtail::run (decode batches within its
// limits), else as tail() above.
#ifndef MOE_SIM_LDS_MIN_SLOTS
#define MOE_SIM_LDS_MIN_SLOTS 64
#endif
// Counters of the hand-off, one per 128 bytes.
constexpr unsigned TICKET_STRIDE = 32;

template <int GT, bool DT>
__global__ __launch_bounds__(FT) void routing_kernel(Args f, cap::Args ca,
                                                       disp::Args da, dtail::Args dta) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_last;
  constexpr int TPB = FT / GT;
  const int grp = threadIdx.x / GT;
  const int t = blockIdx.x * TPB + grp;
  // The tail's SERE step scans similarity and protection rows that are cold
  // in HBM.  The first threads of the grid read them once now, 16 bytes
  // each, so that the memory-side cache holds them by the time the tail
  // asks; the loads complete under the route step (the hand-off waits for
  // every outstanding load anyway).
  int4 pf = make_int4(0, 0, 0, 0);
  bool pf_on = false;
  if (f.kprime > 0 && ((reinterpret_cast<uintptr_t>(f.sim) |
                         reinterpret_cast<uintptr_t>(f.prot)) & 15) == 0) {
    const size_t sc = static_cast<size_t>(f.N) * f.N / 4;   // 16-byte chunks of sim
    const size_t pc = static_cast<size_t>(f.N) * f.N / 16;  // and of prot
    const size_t i = static_cast<size_t>(blockIdx.x) * FT + threadIdx.x;
    if (i < sc) {
      pf = reinterpret_cast<const int4*>(f.sim)[i];
      pf_on = true;
    } else if (i < sc + pc) {
      pf = reinterpret_cast<const int4*>(f.prot)[i - sc];
      pf_on = true;
    }
  }
  // The tail's arguments are first read by the last workgroup, after the
  // hand-off; a cold read of the argument block there costs about 1 us.
  // Every workgroup reads one word of each 64-byte line of it now, so that
  // the line sits in the scalar cache of the CU that runs the tail.
  constexpr int ARG_WORDS =
      static_cast<int>((sizeof(Args) + sizeof(cap::Args) + sizeof(disp::Args) +
                        sizeof(dtail::Args)) / 4);
  typedef __attribute__((address_space(4))) const uint32_t karg_word;
  const karg_word* kargs = (const karg_word*)(__builtin_amdgcn_kernarg_segment_ptr());
  uint32_t kacc = 0;
#pragma unroll
  for (int i = 0; i < ARG_WORDS; i += 16) kacc ^= kargs[i];
  rt::route_token<GT>(f.logits + static_cast<size_t>(t) * f.N, f.N, f.k, f.R, t, t < f.T,
                      smem + grp * rt::token_lds_bytes(f.N, GT), f.topk_ids,
                      f.topk_gates, f.fallback_ids);

  // Hand-off to the last workgroup.  The tail reads only the ranked ids of
  // the route step, which route_token writes with agent-scope stores
  // (through the XCD's L2): once every wave has waited for its stores they
  // are visible on every XCD, so the workgroup counts itself without a
  // release fence (on gfx950 that writes back the whole XCD L2, about 2 us
  // at this point of a decode step).  More than 8 workgroups count in two
  // levels, so that no more than a few increments of one counter queue
  // behind each other: workgroup p counts on counter p % 8 (128 bytes
  // apart), and the last of each such group on the top counter.  Each count
  // wraps to zero (atomicInc's limit), leaving the workspace zero.  The last
  // workgroup invalidates its L2 (acquire) before reading the ids; a single
  // workgroup reads its own stores.
  wait_stores();
  // never true (T >= 0): only keeps the warming loads from being dropped
  if (pf_on && f.T < 0 && (pf.x | pf.y | pf.z | pf.w) == 0) s_last = 0;
  if (f.T < 0 && kacc == 0) s_last = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned G = gridDim.x, x = blockIdx.x % 8;
    bool last = true;  // a single workgroup hands off to itself
    if (G > 8) {
      const unsigned nx = G / 8 + (x < G % 8 ? 1u : 0u);  // members of group x
      last = atomicInc(f.ticket + TICKET_STRIDE * (1 + x), nx - 1) == nx - 1 &&
             atomicInc(f.ticket, 7u) == 7u;
    } else if (G > 1) {
      last = atomicInc(f.ticket, G - 1) == G - 1;
    }
    s_last = last;
    if (last && G > 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return;

  if constexpr (DT) {
    __shared__ dtail::Lds dl;
    if (dta.k <= 8 && dta.R <= 8)
      dtail::run<8, 8>(dta, smem, dl);
    else
      dtail::run<dtail::MAX_K, dtail::MAX_R>(dta, smem, dl);
  } else {
    __shared__ sr::SereLds sl;
    tail(f, ca, da, smem, sl);
  }
}

// Dynamic LDS of the kernel: the larger of the routing groups and the tail.
inline size_t kernel_lds(const TailLayout& L, int N, int GT) {
  const size_t route = static_cast<size_t>(FT / GT) * rt::token_lds_bytes(N, GT);
  return std::max(route, static_cast<size_t>(L.bytes));
}

inline bool supported(int T, int N, int k, int R) {
  return tail_layout(T, N, k, R, FT / MOE_WAVE).bytes <= TAIL_LDS_MAX;
}

constexpr size_t WS_BYTES = 9 * TICKET_STRIDE * 4;  // the two-level ticket

}  // namespace fused
}  // namespace moe

using namespace moe;

extern "C" size_t moe_routing_workspace_size(int T, int N, int k, int R) {
  if (T < 0 || N < 1 || N > 1024 || k < 1 || k > N || R < 0 || R > N - k ||
      !fused::supported(T, N, k, R))
    return 0;
  return fused::WS_BYTES;
}

extern "C" int moe_routing_fused(
    const float* logits, const uint8_t* is_visual, const float* entropy_w,
    const int8_t* modality, const float* sim, const uint8_t* prot, int T,
    int N, int k, int R, int kprime, float rho, int group, double gamma,
    double lam, int32_t* topk_ids, float* topk_gates, int32_t* fallback_ids,
    int32_t* slot_sere, int32_t* slot_expert, uint8_t* flags, int64_t* load_q,
    int64_t* cap_q, int64_t* stats, double* r_v, int32_t* expert_offsets,
    int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      R < 0 || R > N - k || group < 1 || group > N || kprime < 0 ||
      kprime > k)
    return MOE_EINVAL;
  if (std::isnan(gamma) || gamma <= 0.0 || (!std::isinf(gamma) && gamma > 1e30) ||
      !std::isfinite(lam))
    return MOE_EINVAL;
  if (!fused::supported(T, N, k, R)) return MOE_EUNSUP;
  if (!expert_offsets) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !is_visual || !entropy_w || !modality || !topk_ids ||
      !topk_gates || (R > 0 && !fallback_ids) || !slot_expert || !flags ||
      !load_q || !cap_q || !stats || !r_v || !row_token || !row_slot ||
      !slot_row || !workspace)
    return MOE_EINVAL;
  if (kprime > 0 && (!sim || !prot || !slot_sere)) return MOE_EINVAL;
  if (workspace_bytes < fused::WS_BYTES) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);

  char* ws = static_cast<char*>(workspace);

  fused::Args f{};
  f.logits = logits;
  f.sim = sim;
  f.prot = prot;
  f.topk_ids = topk_ids;
  f.topk_gates = topk_gates;
  f.fallback_ids = fallback_ids;
  f.slot_sere = slot_sere;
  f.slot_expert = slot_expert;
  f.flags = flags;
  f.expert_offsets = expert_offsets;
  f.T = T;
  f.N = N;
  f.k = k;
  f.R = R;
  f.kprime = kprime;
  f.rho = rho;
  f.cap_on = !std::isinf(gamma);
  f.ticket = reinterpret_cast<unsigned*>(ws);
  f.tl = fused::tail_layout(T, N, k, R, fused::FT / MOE_WAVE);
  // Caller-side arrays only: the tail points every workspace array of these
  // argument blocks at LDS.
  cap::Args ca{};
  ca.is_visual = is_visual;
  ca.entropy_w = entropy_w;
  ca.modality = modality;
  ca.T = T;
  ca.N = N;
  ca.k = k;
  ca.R = R;
  ca.group = group;
  int nb = 1;
  while ((1 << nb) < N) ++nb;
  ca.nbits = nb;
  ca.gamma = gamma;
  ca.lam = lam;
  ca.load_q = load_q;
  ca.cap_q = cap_q;
  ca.stats = stats;
  ca.r_v = r_v;
  ca.TB = T;
  ca.G = 1;
  disp::Args da{};
  da.T = T;
  da.N = N;
  da.k = k;
  da.nbits = nb;
  da.row_token = row_token;
  da.row_slot = row_slot;
  da.slot_row = slot_row;
  da.TB = T;
  da.G = 1;

  // Threads per token: a whole workgroup per token while that still leaves
  // at most one token per CU (the route phase then spreads over T CUs),
  // else one wave (N <= 128) or four per token.
#ifndef MOE_FUSED_GT
#define MOE_FUSED_GT 0
#endif
  const int GT = MOE_FUSED_GT ? MOE_FUSED_GT
                              : (T <= cu_count() ? fused::FT : (N <= 128 ? 64 : 256));
  const int TPB = fused::FT / GT;
  const dim3 grid((T + TPB - 1) / TPB), block(fused::FT);

  // Decode batches within the compact tail's limits run it as the last
  // workgroup's steps.
  static_assert(fused::FT == dtail::NT, "the compact tail runs in one routing workgroup");
  const bool dt = dtail::supported(T, N, k, R);
  dtail::Args d{};
  if (dt) {
    d.topk = topk_ids;
    d.fb = fallback_ids;
    d.vis = is_visual;
    d.ew = entropy_w;
    d.mod = modality;
    d.sim = sim;
    d.prot = prot;
    d.T = T;
    d.N = N;
    d.k = k;
    d.R = R;
    d.kprime = kprime;
    d.group = group;
    d.nbits = nb;
    d.rho = rho;
    d.gamma = gamma;
    d.lam = lam;
    d.cap_on = !std::isinf(gamma);
    // S and Prot go to LDS for the SERE step unless the batch is so small
    // that the few rows it reads cost less from memory than the copy
    d.sim_lds = kprime > 0 && N <= dtail::SIM_LDS_N && T * k > MOE_SIM_LDS_MIN_SLOTS;
    d.slot_sere = slot_sere;
    d.slot_expert = slot_expert;
    d.flags = flags;
    d.load_q = load_q;
    d.cap_q = cap_q;
    d.stats = stats;
    d.r_v = r_v;
    d.offsets = expert_offsets;
    d.row_token = row_token;
    d.row_slot = row_slot;
    d.slot_row = slot_row;
  }
  // Batches of at most 8 tokens and 64 slots: one workgroup, every
  // batch-wide step in one wave.
#ifndef MOE_TINY_ROUTING
#define MOE_TINY_ROUTING 1
#endif
  if (MOE_TINY_ROUTING && tiny::supported(T, N, k, R)) {
    tiny::Args ta{};
    ta.d = d;
    ta.logits = logits;
    ta.topk_ids = topk_ids;
    ta.topk_gates = topk_gates;
    ta.fallback_ids = fallback_ids;
    auto launch_tiny = [&](auto kern) -> int {
      hipLaunchKernelGGL(kern, dim3(1), dim3(tiny::threads(T)), 0, s, ta);
      return launch_status();
    };
    if (N <= 64) return launch_tiny(tiny::routing_kernel<1>);
    if (N <= 128) return launch_tiny(tiny::routing_kernel<2>);
    return launch_tiny(tiny::routing_kernel<4>);
  }
  const size_t route_lds = static_cast<size_t>(TPB) * rt::token_lds_bytes(N, GT);
  const size_t lds = dt ? std::max(route_lds, dtail::dyn_lds(N, d.sim_lds))
                        : fused::kernel_lds(f.tl, N, GT);
  auto launch = [&](auto kern) -> int {
    const void* fn = reinterpret_cast<const void*>(kern);
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return static_cast<int>(MOE_EHIP);
    hipLaunchKernelGGL(kern, grid, block, lds, s, f, ca, da, d);
    return launch_status();
  };
  if (dt) {
    if (GT == 64) return launch(fused::routing_kernel<64, true>);
    if (GT == 256) return launch(fused::routing_kernel<256, true>);
    return launch(fused::routing_kernel<fused::FT, true>);
  }
  if (GT == 64) return launch(fused::routing_kernel<64, false>);
  if (GT == 256) return launch(fused::routing_kernel<256, false>);
  return launch(fused::routing_kernel<fused::FT, false>);
}
