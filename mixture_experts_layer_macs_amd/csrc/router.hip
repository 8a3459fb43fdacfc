// moe_router_topk: the router network's scores z_t = W_g x_t for every token
// and expert ("MACS", §3.1: the router G scores the N experts; Eq. 1 then
// takes the top k by score and weighs them by the softmax), fused with the
// route step: the scores of a token tile never leave the workgroup before
// they are ranked.
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation).  A
// workgroup of 16 waves owns a tile of 32 tokens and every expert (N rounded
// up to NP = 32, 64, 128 or 256 columns), over one range of the H axis:
//   - the token rows (x, streamed once from HBM) and the weight rows (W_g,
//     N*H*2 bytes, re-read by every tile from L2) travel global -> LDS by
//     direct-to-LDS loads into two rings.  One wave issues every x load and
//     two waves share the W_g loads: a wave's load counter then covers only
//     its own stream, so the x ring can keep SA - 2 slices in flight (the
//     HBM latency) while the W_g ring, served from L2, stays shallow;
//   - wave w < NP / 32 multiplies the tile's rows by column block w; the
//     other waves only join the ring's barriers.  They exist for the route
//     step, which ranks one token per wave: with 16 waves each ranks two of
//     the tile's tokens, and their instruction streams hide each other's
//     latencies.
// Short batches split the H axis over up to 8 workgroups per tile so that
// the chip is filled; the partial scores go to the workspace, and the last
// workgroup of a tile (an atomic ticket that wraps back to zero) adds them in
// split order.  The scores of a tile are then staged in LDS, written out
// when the caller asks for them, and ranked one token per wave with every
// key in registers (route_impl.h, route_token_wave), which gives exactly
// what moe_route gives for the same scores.
//
// fp32 path: one workgroup per 32-token tile, one thread per (token, expert)
// score with a sequential fused multiply-add over H in increasing order; the
// same epilogue.
#include <algorithm>

#include "dma.h"
#include "route_impl.h"

namespace moe {
namespace rtr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 32;          // tokens per tile
constexpr int BK = 64;          // H slice: 128 bytes of every row
constexpr int NTHR = 1024;      // 16 waves: the MFMA work needs at most 8, the
                                // route step ranks one token per wave
constexpr int SA = 8;           // x ring stages
constexpr int MAX_SPLIT = 8;    // H-axis splits per tile
constexpr int FILL = 256;       // workgroups that fill the chip (256 CUs)

__host__ __device__ constexpr int stages_b(int np) { return np >= 256 ? 3 : 6; }
__host__ __device__ constexpr int pitch(int np) { return np + 4; }  // floats per LDS row
__host__ __device__ constexpr int cand_slots(int np) { return np; }  // >= k + R per wave
__host__ __device__ constexpr int keys_per_lane(int np) { return np <= 64 ? 1 : np / 64; }

struct Args {
  const void* x;          // [T,H]
  const void* w;          // [N,H]
  int T, N, H, k, R;
  float* logits;          // [T,N] or null
  int32_t* topk_ids;
  float* topk_gates;
  int32_t* fallback_ids;
  float* part;            // [tiles][KS][BM][NP] partial scores (KS > 1)
  unsigned* ticket;       // [tiles] arrivals (zero between calls)
  int KS, kc;             // splits per tile, H slices per split
  int NP;
};

// Scores of the tile (LDS [BM][pitch]) -> optional logits rows, then the
// route step for each live token: one wave per token, wave w taking tokens
// w and w + 16 of the tile (route_token_wave, keys in registers).
template <int KPL>
__device__ void finish_tile(const Args& a, const float* tile, int t0,
                            unsigned char* route_lds) {
  const int tid = threadIdx.x;
  const int P = pitch(a.NP);
  const int rows = min(BM, a.T - t0);
  if (a.logits) {
    for (int i = tid; i < rows * a.N; i += NTHR) {
      const int r = i / a.N, c = i - r * a.N;
      a.logits[static_cast<size_t>(t0 + r) * a.N + c] = tile[r * P + c];
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  uint64_t* cand = reinterpret_cast<uint64_t*>(route_lds) + wave * cand_slots(a.NP);
  for (int lt = wave; lt < rows; lt += NTHR / MOE_WAVE)
    rt::route_token_wave<KPL>(tile + lt * P, a.N, a.k, a.R, t0 + lt, true, cand,
                              a.topk_ids, a.topk_gates, a.fallback_ids);
}

template <int NP>
__global__ __launch_bounds__(NTHR) void router_bf16_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int SB = stages_b(NP);
  constexpr int A_BYTES = BM * BK * 2;       // 4 KB
  constexpr int B_BYTES = NP * BK * 2;       // NP * 128 bytes
  constexpr int QA = BM / 8;                 // x loads per slice (wave 0)
  constexpr int QB = NP / 16;                // W_g loads per slice per wave (waves 1, 2)
  constexpr int NCB = NP / 32;               // 32-column blocks, one per wave
  constexpr int P = pitch(NP);
  static_assert(SA * A_BYTES + SB * B_BYTES <= 160 * 1024, "LDS");

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  // workgroup b is split b % KS of tile b / KS: with 8 splits, every XCD
  // (they receive workgroups round-robin) reads one H range of W_g
  const int tile = blockIdx.x / a.KS, ks = blockIdx.x % a.KS;
  const int t0 = tile * BM;
  const int nk = a.H / BK;
  const int s0 = ks * a.kc;
  const int ns = min(nk, s0 + a.kc) - s0;    // >= 1 (host)
  const uint32_t row_bytes = static_cast<uint32_t>(a.H) * 2;

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));
  const uint32_t lds_b = lds_base + SA * A_BYTES;

  // This wave's loads: 16 bytes per lane, lane -> (row, 16-byte slot) of an
  // 8-row group; the lane filling LDS slot s of row r fetches chunk
  // s ^ ((r >> 1) & 7) of that row, so fragment reads are conflict free.
  // Rows past the batch or past N get an offset outside their resource.
  const int lrow = lane / 8, lslot = lane % 8;
  i32x4 rsrc = {0, 0, 0, 0};
  uint32_t voff[QB > QA ? QB : QA];
  if (wave == 0) {
    rsrc = buffer_rsrc(a.x, static_cast<uint32_t>(a.T) * row_bytes);
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int r = q * 8 + lrow;
      const int ch = lslot ^ ((r >> 1) & 7);
      voff[q] = t0 + r < a.T ? static_cast<uint32_t>(t0 + r) * row_bytes + ch * 16 : OOB_OFF;
    }
  } else if (wave <= 2) {
    rsrc = buffer_rsrc(a.w, static_cast<uint32_t>(a.N) * row_bytes);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int r = ((wave - 1) * QB + q) * 8 + lrow;
      const int ch = lslot ^ ((r >> 1) & 7);
      voff[q] = r < a.N ? static_cast<uint32_t>(r) * row_bytes + ch * 16 : OOB_OFF;
    }
  }
  // Slice s of the split goes to stage s % SA (x) or s % SB (W_g); requests
  // past the last slice re-fetch it into a stage that is never read again,
  // so every iteration issues the same number of loads.
  auto issue = [&](int s) {
    const uint32_t koff = static_cast<uint32_t>((s0 + min(s, ns - 1)) * BK * 2);
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < QA; ++q)
        lds_dma16(rsrc, voff[q], koff, lds_base + (s % SA) * A_BYTES + q * 1024);
    } else if (wave <= 2) {
#pragma unroll
      for (int q = 0; q < QB; ++q)
        lds_dma16(rsrc, voff[q], koff,
                  lds_b + (s % SB) * B_BYTES + ((wave - 1) * QB + q) * 1024);
    }
  };

  const bool mma_wave = wave < NCB;          // wave w owns column block w
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) const unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  const int frow = lane & 31, fhalf = lane >> 5;

  // Ring protocol: x slices SA - 1 ahead (wave 0), W_g slices SB - 1 ahead
  // (waves 1 and 2).  At the top of iteration s a loading wave waits until
  // its own loads of slice s have landed, the barrier publishes everyone's,
  // and slice s + S - 1 of each ring is requested into the stage of slice
  // s - 1, which every wave finished reading before the barrier.
  for (int s = 0; s + 1 < SA; ++s) {
    if (wave == 0 || s + 1 < SB) issue(s);
  }
  for (int s = 0; s < ns; ++s) {
    if (wave == 0)
      wait_vmcnt<(SA - 2) * QA>();
    else
      wait_vmcnt<(SB - 2) * QB>();
    wg_barrier();
    issue(s + (wave == 0 ? SA : SB) - 1);
    if (mma_wave) {
      lds_byte* A_ = lds0 + (s % SA) * A_BYTES;
      lds_byte* B_ = lds0 + SA * A_BYTES + (s % SB) * B_BYTES;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int sw = ((kk * 2 + fhalf) ^ ((frow >> 1) & 7)) << 4;
        const bf16x8 fa = *(lds_frag*)(A_ + frow * (BK * 2) + sw);
        const bf16x8 fb = *(lds_frag*)(B_ + (wave * 32 + frow) * (BK * 2) + sw);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc, 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();  // no DMA write may land after the ring is reused
  __syncthreads();

  // scores -> LDS tile [BM][P]: lane holds token frow, columns
  // wave * 32 + 8 * (r / 4) + 4 * fhalf + r % 4
  float* tile_s = reinterpret_cast<float*>(smem);
  if (mma_wave) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v;
      v.x = acc[4 * q + 0];
      v.y = acc[4 * q + 1];
      v.z = acc[4 * q + 2];
      v.w = acc[4 * q + 3];
      *reinterpret_cast<float4*>(&tile_s[frow * P + wave * 32 + 8 * q + 4 * fhalf]) = v;
    }
  }
  __syncthreads();

  const int rows = min(BM, a.T - t0);
  if (a.KS > 1) {
    // partial scores of the live rows, then the tile's ticket
    float* mine = a.part + (static_cast<size_t>(tile) * a.KS + ks) * BM * NP;
    for (int i = tid * 4; i < rows * NP; i += NTHR * 4) {
      const int r = i / NP, c = i - r * NP;
      *reinterpret_cast<float4*>(mine + i) = *reinterpret_cast<const float4*>(&tile_s[r * P + c]);
    }
    __shared__ int s_last;
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      const unsigned prev = atomicInc(a.ticket + tile, static_cast<unsigned>(a.KS - 1));
      s_last = prev == static_cast<unsigned>(a.KS - 1);
      if (s_last) __threadfence();
    }
    __syncthreads();
    if (!s_last) return;
    const float* all = a.part + static_cast<size_t>(tile) * a.KS * BM * NP;
    for (int i = tid * 4; i < rows * NP; i += NTHR * 4) {
      const int r = i / NP, c = i - r * NP;
      float4 v = *reinterpret_cast<const float4*>(all + i);
      for (int q = 1; q < a.KS; ++q) {
        const float4 u = *reinterpret_cast<const float4*>(all + static_cast<size_t>(q) * BM * NP + i);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      *reinterpret_cast<float4*>(&tile_s[r * P + c]) = v;
    }
    __syncthreads();
  }
  finish_tile<keys_per_lane(NP)>(a, tile_s, t0, smem + BM * P * 4);
}

__global__ __launch_bounds__(NTHR) void router_f32_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* tile_s = reinterpret_cast<float*>(smem);
  const int P = pitch(a.NP);
  const int t0 = blockIdx.x * BM;
  const int rows = min(BM, a.T - t0);
  const float* x = static_cast<const float*>(a.x);
  const float* w = static_cast<const float*>(a.w);
  for (int i = threadIdx.x; i < rows * a.N; i += NTHR) {
    const int r = i / a.N, c = i - r * a.N;
    const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(t0 + r) * a.H);
    const float4* wr = reinterpret_cast<const float4*>(w + static_cast<size_t>(c) * a.H);
    float s = 0.f;
    for (int h = 0; h < a.H / 4; ++h) {
      const float4 u = xr[h], v = wr[h];
      s = fmaf(u.x, v.x, s);
      s = fmaf(u.y, v.y, s);
      s = fmaf(u.z, v.z, s);
      s = fmaf(u.w, v.w, s);
    }
    tile_s[r * P + c] = s;
  }
  __syncthreads();
  unsigned char* route_lds = smem + BM * P * 4;
  switch (a.NP) {
    case 32:
    case 64: finish_tile<1>(a, tile_s, t0, route_lds); break;
    case 128: finish_tile<2>(a, tile_s, t0, route_lds); break;
    default: finish_tile<4>(a, tile_s, t0, route_lds); break;
  }
}

// ------------------------------------------------------------------ host
inline int np_of(int N) { return N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256; }

struct Plan {
  int tiles, KS, kc, NP;
  size_t part_off, bytes;
};

// The split is a function of the shape only (never of the device), so the
// scores of a given shape are the same bits on every device.
inline Plan plan(int T, int N, int H, int dtype) {
  Plan p{};
  p.tiles = (T + BM - 1) / BM;
  p.NP = np_of(N);
  p.KS = 1;
  p.kc = H / BK;
  if (dtype == MOE_BF16 && p.tiles > 0) {
    const int nk = H / BK;
    int ks = std::min(MAX_SPLIT, std::max(1, FILL / p.tiles));
    ks = std::min(ks, nk);
    p.kc = (nk + ks - 1) / ks;
    p.KS = (nk + p.kc - 1) / p.kc;  // every split has at least one slice
  }
  const size_t tickets = (static_cast<size_t>(p.tiles) * 4 + 255) & ~size_t(255);
  p.part_off = tickets;
  p.bytes = tickets;
  if (p.KS > 1)
    p.bytes += static_cast<size_t>(p.tiles) * p.KS * BM * p.NP * 4;
  return p;
}

inline size_t epilogue_lds(int NP) {
  return static_cast<size_t>(BM) * pitch(NP) * 4 +
         (NTHR / MOE_WAVE) * static_cast<size_t>(cand_slots(NP)) * 8;
}

inline size_t ring_lds(int NP) {
  return static_cast<size_t>(SA) * BM * BK * 2 + static_cast<size_t>(stages_b(NP)) * NP * BK * 2;
}

template <int NP>
int launch_bf16(const Args& a, int grid, hipStream_t s) {
  const size_t lds = std::max(ring_lds(NP), epilogue_lds(NP));
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(router_bf16_kernel<NP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  hipLaunchKernelGGL(router_bf16_kernel<NP>, dim3(grid), dim3(NTHR), lds, s, a);
  return launch_status();
}

}  // namespace rtr
}  // namespace moe

using namespace moe;
using namespace moe::rtr;

extern "C" size_t moe_router_workspace_size(int T, int N, int H, int dtype) {
  if (T < 0 || N < 1 || H < 1 || (dtype != MOE_BF16 && dtype != MOE_F32)) return 0;
  if (dtype == MOE_BF16 && H % BK != 0) return 0;
  return plan(T, N, H, dtype).bytes;
}

extern "C" int moe_router_topk(const void* x, const void* w_gate, int T, int N,
                               int H, int k, int R, int dtype, float* logits,
                               int32_t* topk_ids, float* topk_gates,
                               int32_t* fallback_ids, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N || R < 0 ||
      R > N - k || H < 1)
    return MOE_EINVAL;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_EUNSUP;
  if (N > 256) return MOE_EUNSUP;
  if (dtype == MOE_BF16 &&
      (H % BK != 0 || static_cast<int64_t>(T) * H * 2 > (int64_t(1) << 31) ||
       static_cast<int64_t>(N) * H * 2 > (int64_t(1) << 31)))
    return MOE_EUNSUP;
  if (dtype == MOE_F32 && H % 4 != 0) return MOE_EUNSUP;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !topk_ids || !topk_gates || (R > 0 && !fallback_ids) || !workspace)
    return MOE_EINVAL;
  const Plan p = plan(T, N, H, dtype);
  if (workspace_bytes < p.bytes) return MOE_EINVAL;
  Args a{};
  a.x = x;
  a.w = w_gate;
  a.T = T;
  a.N = N;
  a.H = H;
  a.k = k;
  a.R = R;
  a.logits = logits;
  a.topk_ids = topk_ids;
  a.topk_gates = topk_gates;
  a.fallback_ids = fallback_ids;
  char* ws = static_cast<char*>(workspace);
  a.ticket = reinterpret_cast<unsigned*>(ws);
  a.part = reinterpret_cast<float*>(ws + p.part_off);
  a.KS = p.KS;
  a.kc = p.kc;
  a.NP = p.NP;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_F32) {
    const size_t lds = epilogue_lds(p.NP);
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(router_f32_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return MOE_EHIP;
    hipLaunchKernelGGL(router_f32_kernel, dim3(p.tiles), dim3(NTHR), lds, s, a);
    return launch_status();
  }
  const int grid = p.tiles * p.KS;
  switch (p.NP) {
    case 32: return launch_bf16<32>(a, grid, s);
    case 64: return launch_bf16<64>(a, grid, s);
    case 128: return launch_bf16<128>(a, grid, s);
    default: return launch_bf16<256>(a, grid, s);
  }
}
