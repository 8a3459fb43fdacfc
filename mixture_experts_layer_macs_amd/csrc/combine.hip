// moe_combine: gate-weighted combine ("MACS", §3.1 Eq. 1):
//   y[t] = sum_{s kept} G(x_t)_{rank s} * E(x_t)[row(t,s)]
// fp32 accumulation in slot order, one workgroup per token, 16-byte
// (8-element) vector loads of the expert output rows, which are contiguous
// rows of out_rows, several rows in flight per thread.  Dropped slots (row -1) contribute nothing; the kept
// gates are used as they are (no renormalisation, the router's values are
// unchanged by re-routing).
#include "common.h"

namespace moe {
namespace comb {

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua += 0x7fffu + ((ua >> 16) & 1u);
  ub += 0x7fffu + ((ub >> 16) & 1u);
  return (ua >> 16) | (ub & 0xffff0000u);
}

// The slot rows and gates of the token are staged in LDS first, then the k
// output-row loads of a thread are issued in batches of 8 independent loads
// (a dependent chain of k round trips otherwise sets the time of a decode
// batch); the accumulation order stays the slot order.
constexpr int CB = 8;  // row loads in flight per thread

__global__ __launch_bounds__(256) void combine_bf16(
    const uint16_t* __restrict__ rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gates, int k, int H, uint16_t* __restrict__ y) {
  __shared__ int s_row[64];
  __shared__ float s_g[64];
  const int t = blockIdx.x;
  const int nv = H / 8;
  for (int v0 = 0; v0 < nv; v0 += blockDim.x) {
    const int v = v0 + threadIdx.x;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < k; s0 += 64) {
      const int kb = min(64, k - s0);
      __syncthreads();
      if (threadIdx.x < kb) {
        s_row[threadIdx.x] = slot_row[static_cast<size_t>(t) * k + s0 + threadIdx.x];
        s_g[threadIdx.x] = gates[static_cast<size_t>(t) * k + s0 + threadIdx.x];
      }
      __syncthreads();
      for (int sb = 0; sb < kb; sb += CB) {
        uint4 q[CB];
        int r[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          r[u] = sb + u < kb ? s_row[sb + u] : -1;
          if (r[u] >= 0 && v < nv)
            q[u] = *reinterpret_cast<const uint4*>(rows + static_cast<size_t>(r[u]) * H + v * 8);
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
          if (r[u] < 0) continue;
          const float g = s_g[sb + u];
          const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += g * bf16_lo(w[i]);
            acc[2 * i + 1] += g * bf16_hi(w[i]);
          }
        }
      }
    }
    if (v < nv) {
      uint4 o;
      o.x = pack_bf16(acc[0], acc[1]);
      o.y = pack_bf16(acc[2], acc[3]);
      o.z = pack_bf16(acc[4], acc[5]);
      o.w = pack_bf16(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(y + static_cast<size_t>(t) * H + v * 8) = o;
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32(
    const float* __restrict__ rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gates, int k, int H, float* __restrict__ y) {
  const int t = blockIdx.x;
  const int nv = H / 4;
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; ++s) {
      const int r = slot_row[static_cast<size_t>(t) * k + s];
      if (r < 0) continue;
      const float g = gates[static_cast<size_t>(t) * k + s];
      const float4 q = *reinterpret_cast<const float4*>(rows + static_cast<size_t>(r) * H + v * 4);
      acc.x += g * q.x;
      acc.y += g * q.y;
      acc.z += g * q.z;
      acc.w += g * q.w;
    }
    *reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H + v * 4) = acc;
  }
}

}  // namespace comb
}  // namespace moe

using namespace moe;
using namespace moe::comb;

extern "C" int moe_combine(const void* out_rows, const int32_t* slot_row,
                           const float* topk_gates, int T, int k, int H,
                           int dtype, void* y, void* stream) {
  if (T < 0 || T > (1 << 20) || k < 1 || k > 1024 || H < 1) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EUNSUP;
  if (H % 8 != 0) return MOE_EUNSUP;
  if (T == 0) return MOE_OK;
  if (!out_rows || !slot_row || !topk_gates || !y) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bf16, dim3(T), dim3(256), 0, s,
                       static_cast<const uint16_t*>(out_rows), slot_row,
                       topk_gates, k, H, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(combine_f32, dim3(T), dim3(256), 0, s,
                       static_cast<const float*>(out_rows), slot_row,
                       topk_gates, k, H, static_cast<float*>(y));
  return launch_status();
}
