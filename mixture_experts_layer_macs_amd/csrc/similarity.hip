// moe_expert_similarity: the SERE similarity calibration (multi-image QA
// write-up, §4.2: expert activations on a small generic calibration set
// give, once and offline, a per-layer matrix of Frobenius similarities).
//
//   S[i][j] = <A_i, A_j>_F / (||A_i||_F ||A_j||_F),   S[j][j] = 1,
//
// for N matrices A_j given flattened as the rows of acts [N, D] (e.g. the
// out rows of an FFN pass that sends every calibration token to every
// expert, which are expert-major and hence exactly this layout).  The Gram
// matrix G = V V^T over the rows is the whole cost: N^2 D MACs over N D
// elements, HBM-bound at N = 128.
//
// bf16 path, three launches:
//   1. gram: up to 256 workgroups of 8 waves, each over one contiguous range
//      of the D axis.  The NP x 64 slices of V (N rounded up to NP = 32, 64
//      or 128 rows) travel global -> LDS by direct-to-LDS loads through an
//      8-stage ring; one slice serves as both MFMA operands
//      (v_mfma_f32_32x32x16_bf16, fp32 accumulation), each wave owning up to
//      two 32 x 32 blocks of the upper triangle of G (G is symmetric).  Every 64 slices the fp32 accumulators are
//      added into fp64 registers and cleared, so fp32 only ever sums 4096
//      products.  Each workgroup writes its partial G in fp32.
//   2. reduce: G[i][j] = the fp64 sum of the partials, in a fixed order.
//   3. normalise: S from G in fp64, rounded once to fp32.
// Every sum has a fixed order: the result is deterministic.
// fp32 path: the same three launches; the partials are plain fp64 sums of
// the exact products over each workgroup's range.
#include <algorithm>
#include <cmath>

#include "dma.h"

namespace moe {
namespace sim {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;            // D slice: 128 bytes of every row
constexpr int NTHR = 512;         // 8 waves
constexpr int S = 8;              // ring stages
constexpr int FLUSH = 64;         // slices per fp32 accumulation run
constexpr int MAX_WG = 256;
constexpr int F32_KC = 32;        // fp32 path: D elements per LDS chunk

struct Args {
  const void* v;       // [N, D]
  int N, NP;
  long long D;
  long long s_per_wg;  // D slices (bf16) or elements (fp32) per workgroup
  int nwg;
  float* part;         // [nwg][NP][NP]
  double* gram;        // [N][N]
  float* sim;          // [N][N]
};

template <int NP>
__global__ __launch_bounds__(NTHR) void gram_bf16_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int SLICE = NP * BK * 2;          // bytes per slice
  constexpr int NL = NP / 8;                  // DMA instructions per slice
  constexpr int LW = NL < 8 ? NL : 8;         // loading waves
  constexpr int QL = NL / LW;                 // loads per loading wave
  constexpr int NB = NP / 32;                 // 32-row blocks
  constexpr int NF = NB * (NB + 1) / 2;       // blocks (bi <= bj) of G
  constexpr int FPW = (NF + 7) / 8;           // blocks per wave
  static_assert(S * SLICE <= 160 * 1024, "LDS");

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const long long nsl = a.D / BK;
  const long long sb = static_cast<long long>(blockIdx.x) * a.s_per_wg;
  const int ns = static_cast<int>(max(0LL, min(nsl, sb + a.s_per_wg) - sb));
  const uint32_t row_bytes = static_cast<uint32_t>(a.D * 2);

  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));
  // loading wave w < LW fills rows [(w * QL + q) * 8, +8) of every slice;
  // the lane filling LDS slot s of row r fetches chunk s ^ ((r >> 1) & 7)
  const i32x4 rsrc = buffer_rsrc(a.v, static_cast<uint32_t>(a.N) * row_bytes);
  const int lrow = lane / 8, lslot = lane % 8;
  uint32_t voff[QL];
#pragma unroll
  for (int q = 0; q < QL; ++q) {
    const int r = (wave * QL + q) * 8 + lrow;
    const int ch = lslot ^ ((r >> 1) & 7);
    voff[q] = r < a.N ? static_cast<uint32_t>(r) * row_bytes + ch * 16 : OOB_OFF;
  }
  // slices past the range re-fetch its last slice into a stage that is
  // never read again
  auto issue = [&](int s) {
    if (wave < LW) {
      const uint32_t koff = static_cast<uint32_t>((sb + min(s, ns - 1)) * BK * 2);
#pragma unroll
      for (int q = 0; q < QL; ++q)
        lds_dma16(rsrc, voff[q], koff, lds_base + (s % S) * SLICE + (wave * QL + q) * 1024);
    }
  };

  f32x16 acc[FPW];
  double acc64[FPW][16];
#pragma unroll
  for (int f = 0; f < FPW; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[f][r] = 0.f;
      acc64[f][r] = 0.0;
    }
  typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) const unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  const int frow = lane & 31, fhalf = lane >> 5;
  // G is symmetric: wave w owns the blocks w and w + 8 of the upper
  // triangle in row-major order (bi <= bj)
  int bi_[FPW], bj_[FPW];
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    int idx = wave + 8 * f, bi = 0;
    while (bi < NB - 1 && idx >= NB - bi) {
      idx -= NB - bi;
      ++bi;
    }
    bi_[f] = bi;
    bj_[f] = bi + idx;
  }

  if (ns > 0) {
    for (int s = 0; s + 1 < S; ++s) issue(s);
    for (int s = 0; s < ns; ++s) {
      // this wave's loads of slice s have landed; the barrier publishes
      // everyone's, and slice s + S - 1 goes to the stage of slice s - 1
      wait_vmcnt<(S - 2) * QL>();
      wg_barrier();
      issue(s + S - 1);
      lds_byte* L = lds0 + (s % S) * SLICE;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int sw = ((kk * 2 + fhalf) ^ ((frow >> 1) & 7)) << 4;
#pragma unroll
        for (int f = 0; f < FPW; ++f) {
          const int blk = wave + 8 * f;
          if (blk < NF) {
            const int bi = bi_[f], bj = bj_[f];
            const bf16x8 fa = *(lds_frag*)(L + (bi * 32 + frow) * (BK * 2) + sw);
            const bf16x8 fb = *(lds_frag*)(L + (bj * 32 + frow) * (BK * 2) + sw);
            acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb, fa, acc[f], 0, 0, 0);
          }
        }
      }
      if ((s + 1) % FLUSH == 0 || s + 1 == ns) {
#pragma unroll
        for (int f = 0; f < FPW; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc64[f][r] += static_cast<double>(acc[f][r]);
            acc[f][r] = 0.f;
          }
      }
    }
    wait_vmcnt<0>();
  }
  // partial G of this range: lane holds G[bi*32 + frow][bj*32 + 8*(r/4) +
  // 4*fhalf + r%4]
  float* P = a.part + static_cast<size_t>(blockIdx.x) * NP * NP;
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    const int blk = wave + 8 * f;
    if (blk < NF) {
      const int bi = bi_[f], bj = bj_[f];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v;
        v.x = static_cast<float>(acc64[f][4 * q + 0]);
        v.y = static_cast<float>(acc64[f][4 * q + 1]);
        v.z = static_cast<float>(acc64[f][4 * q + 2]);
        v.w = static_cast<float>(acc64[f][4 * q + 3]);
        *reinterpret_cast<float4*>(
            &P[(bi * 32 + frow) * NP + bj * 32 + 8 * q + 4 * fhalf]) = v;
        if (bi != bj) {  // the mirror block, from the same values
          const int c0 = bj * 32 + 8 * q + 4 * fhalf;
          P[(c0 + 0) * NP + bi * 32 + frow] = v.x;
          P[(c0 + 1) * NP + bi * 32 + frow] = v.y;
          P[(c0 + 2) * NP + bi * 32 + frow] = v.z;
          P[(c0 + 3) * NP + bi * 32 + frow] = v.w;
        }
      }
    }
  }
}

// fp32: each workgroup sums the exact products of its D range in fp64;
// LDS chunks of F32_KC columns of every row, one thread per (i, j) pair.
__global__ __launch_bounds__(256) void gram_f32_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* tile = reinterpret_cast<float*>(smem);  // [N][F32_KC]
  const int tid = threadIdx.x, N = a.N;
  const long long k0 = static_cast<long long>(blockIdx.x) * a.s_per_wg;
  const long long k1 = min(a.D, k0 + a.s_per_wg);
  const float* v = static_cast<const float*>(a.v);
  const int pairs = N * N;
  double acc[64];  // pairs per thread: N <= 128
#pragma unroll
  for (int u = 0; u < 64; ++u) acc[u] = 0.0;
  for (long long kc = k0; kc < k1; kc += F32_KC) {
    const int w = static_cast<int>(min(static_cast<long long>(F32_KC), k1 - kc));
    __syncthreads();
    for (int i = tid; i < N * F32_KC; i += 256) {
      const int r = i / F32_KC, c = i % F32_KC;
      tile[i] = c < w ? v[static_cast<size_t>(r) * a.D + kc + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      const int p = tid + 256 * u;
      if (p < pairs) {
        const float* ri = tile + (p / N) * F32_KC;
        const float* rj = tile + (p % N) * F32_KC;
        double s = 0.0;
        for (int c = 0; c < F32_KC; ++c)
          s += static_cast<double>(ri[c]) * static_cast<double>(rj[c]);
        acc[u] += s;
      }
    }
  }
  float* P = a.part + static_cast<size_t>(blockIdx.x) * a.NP * a.NP;
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const int p = tid + 256 * u;
    if (p < pairs) P[(p / N) * a.NP + p % N] = static_cast<float>(acc[u]);
  }
}

// G[i][j] = the fp64 sum over the workgroups of their partials (full
// NP x NP matrices; the bf16 partials carry each off-diagonal block and its
// mirror from the same values, so S comes out exactly symmetric).  A block
// of 256 threads serves 64 consecutive entries of the NP x NP layout (so
// that the 16 MB of partials at N = 128 spread over 256 workgroups):
// thread (part, q) loads entries 4q .. 4q+3 (16-byte loads) of the
// partials of workgroups part, part + 16, ... in order, 16 independent
// loads at a time; the sixteen sums are then added in part order.
constexpr int RPARTS = 16;
constexpr int REDUCE_ENTRIES = 64;
__global__ __launch_bounds__(256) void gram_reduce_kernel(Args a) {
  __shared__ double red[RPARTS][REDUCE_ENTRIES];
  const int q = threadIdx.x % 16, part = threadIdx.x / 16;
  const size_t base = static_cast<size_t>(blockIdx.x) * REDUCE_ENTRIES + 4 * q;
  const size_t stride = static_cast<size_t>(a.NP) * a.NP;
  double g[4] = {0.0, 0.0, 0.0, 0.0};
  for (int w0 = part; w0 < a.nwg; w0 += 16 * RPARTS) {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int w = w0 + RPARTS * u;
      v[u] = w < a.nwg ? *reinterpret_cast<const float4*>(a.part + w * stride + base)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (w0 + RPARTS * u < a.nwg) {
        g[0] += static_cast<double>(v[u].x);
        g[1] += static_cast<double>(v[u].y);
        g[2] += static_cast<double>(v[u].z);
        g[3] += static_cast<double>(v[u].w);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[part][4 * q + c] = g[c];
  __syncthreads();
  if (threadIdx.x < REDUCE_ENTRIES) {
    const int o = threadIdx.x;
    const size_t e = static_cast<size_t>(blockIdx.x) * REDUCE_ENTRIES + o;
    const int i = static_cast<int>(e / a.NP), j = static_cast<int>(e % a.NP);
    double t = red[0][o];
#pragma unroll
    for (int pp = 1; pp < RPARTS; ++pp) t += red[pp][o];
    if (i < a.N && j < a.N) a.gram[i * a.N + j] = t;
  }
}

__global__ __launch_bounds__(256) void normalise_kernel(Args a) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= a.N * a.N) return;
  const int i = p / a.N, j = p % a.N;
  const double gii = a.gram[i * a.N + i], gjj = a.gram[j * a.N + j];
  double s = 0.0;
  if (i == j)
    s = 1.0;
  else if (gii > 0.0 && gjj > 0.0)
    s = a.gram[p] / sqrt(gii * gjj);
  a.sim[p] = static_cast<float>(s);
}

// ------------------------------------------------------------------ host
struct Plan {
  int NP, nwg;
  long long per;
  size_t part_off, gram_off, bytes;
};

inline int np_of(int N) { return N <= 32 ? 32 : N <= 64 ? 64 : 128; }

inline Plan plan(int N, long long D, int dtype) {
  Plan p{};
  p.NP = np_of(N);
  const long long units = dtype == MOE_BF16 ? D / BK : D;  // slices or elements
  const long long cap = dtype == MOE_BF16 ? MAX_WG : 64;
  p.nwg = static_cast<int>(std::max(1LL, std::min(cap, units)));
  p.per = (units + p.nwg - 1) / p.nwg;
  if (dtype == MOE_F32) p.per = (p.per + F32_KC - 1) / F32_KC * F32_KC;
  p.nwg = static_cast<int>(std::max(1LL, (units + p.per - 1) / p.per));
  p.gram_off = 0;
  p.part_off = (static_cast<size_t>(N) * N * 8 + 255) & ~size_t(255);
  p.bytes = p.part_off + static_cast<size_t>(p.nwg) * p.NP * p.NP * 4;
  return p;
}

template <int NP>
int launch_gram(const Args& a, hipStream_t s) {
  constexpr size_t lds = static_cast<size_t>(S) * NP * BK * 2;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(gram_bf16_kernel<NP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  hipLaunchKernelGGL(gram_bf16_kernel<NP>, dim3(a.nwg), dim3(NTHR), lds, s, a);
  return MOE_OK;
}

}  // namespace sim
}  // namespace moe

using namespace moe;
using namespace moe::sim;

static bool sim_shape_ok(int N, long long D, int dtype) {
  if (N > 128) return false;
  if (dtype == MOE_BF16)
    return D % BK == 0 && static_cast<long long>(N) * D * 2 <= (1LL << 31);
  return true;
}

extern "C" size_t moe_similarity_workspace_size(int N, long long D, int dtype) {
  if (N < 1 || N > 1024 || D < 1 || (dtype != MOE_BF16 && dtype != MOE_F32)) return 0;
  if (!sim_shape_ok(N, D, dtype)) return 0;
  return plan(N, D, dtype).bytes;
}

extern "C" int moe_expert_similarity(const void* acts, int N, long long D,
                                     int dtype, float* sim, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (N < 1 || N > 1024 || D < 1) return MOE_EINVAL;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_EUNSUP;
  if (!sim_shape_ok(N, D, dtype)) return MOE_EUNSUP;
  if (!acts || !sim || !workspace) return MOE_EINVAL;
  const Plan p = plan(N, D, dtype);
  if (workspace_bytes < p.bytes) return MOE_EINVAL;
  Args a{};
  a.v = acts;
  a.N = N;
  a.NP = p.NP;
  a.D = D;
  a.s_per_wg = p.per;
  a.nwg = p.nwg;
  char* ws = static_cast<char*>(workspace);
  a.gram = reinterpret_cast<double*>(ws + p.gram_off);
  a.part = reinterpret_cast<float*>(ws + p.part_off);
  a.sim = sim;
  hipStream_t s = as_stream(stream);
  int st = MOE_OK;
  if (dtype == MOE_F32) {
    const size_t lds = static_cast<size_t>(N) * F32_KC * 4;
    hipLaunchKernelGGL(gram_f32_kernel, dim3(p.nwg), dim3(256), lds, s, a);
  } else {
    switch (p.NP) {
      case 32: st = launch_gram<32>(a, s); break;
      case 64: st = launch_gram<64>(a, s); break;
      default: st = launch_gram<128>(a, s); break;
    }
  }
  if (st != MOE_OK) return st;
  const int nb = (N * N + 255) / 256;
  hipLaunchKernelGGL(gram_reduce_kernel, dim3(p.NP * p.NP / REDUCE_ENTRIES), dim3(256), 0, s, a);
  hipLaunchKernelGGL(normalise_kernel, dim3(nb), dim3(256), 0, s, a);
  return launch_status();
}
