// moe_route: router softmax and top-k ("MACS", §3.1 Eq. 1).
//
// Workgroups of 256 threads.  Up to 256 experts, each wave owns one token
// and ranks it with every key in registers (route_impl.h, route_token_wave:
// a radix search for the (k+R)-th key, then ranks among the selected);
// beyond that, four waves own a token and count ranks over LDS keys
// (route_token).  Ranking compares the fp32 logits themselves, so two
// logits that round to the same exp() value still rank by value.
#include "route_impl.h"

namespace moe {

template <int GT>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, int T, int N, int k, int R,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_gates,
    int32_t* __restrict__ fallback_ids) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TPB = 256 / GT;
  const int grp = threadIdx.x / GT;
  const int t = blockIdx.x * TPB + grp;
  rt::route_token<GT>(logits + static_cast<size_t>(t) * N, N, k, R, t, t < T,
                      smem + grp * rt::token_lds_bytes(N, GT), topk_ids,
                      topk_gates, fallback_ids);
}

// N <= 64 * KPL: one wave per token, keys in registers.
template <int KPL>
__global__ __launch_bounds__(256) void route_wave_kernel(
    const float* __restrict__ logits, int T, int N, int k, int R,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_gates,
    int32_t* __restrict__ fallback_ids) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
  const int t = blockIdx.x * (256 / MOE_WAVE) + wave;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem) + wave * (k + R);
  rt::route_token_wave<KPL>(logits + static_cast<size_t>(t) * N, N, k, R, t, t < T,
                            cand, topk_ids, topk_gates, fallback_ids);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const float* logits, int T, int N, int k, int R,
                         int32_t* topk_ids, float* topk_gates,
                         int32_t* fallback_ids, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      R < 0 || R > N - k)
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_gates || (R > 0 && !fallback_ids))
    return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  if (N <= 256) {
    const dim3 grid((T + 3) / 4), block(256);
    const size_t lds = 4 * static_cast<size_t>(k + R) * 8;
    if (N <= 64)
      hipLaunchKernelGGL(route_wave_kernel<1>, grid, block, lds, s, logits, T, N, k, R,
                         topk_ids, topk_gates, fallback_ids);
    else if (N <= 128)
      hipLaunchKernelGGL(route_wave_kernel<2>, grid, block, lds, s, logits, T, N, k, R,
                         topk_ids, topk_gates, fallback_ids);
    else
      hipLaunchKernelGGL(route_wave_kernel<4>, grid, block, lds, s, logits, T, N, k, R,
                         topk_ids, topk_gates, fallback_ids);
  } else {
    const size_t lds = rt::token_lds_bytes(N, 256);
    hipLaunchKernelGGL(route_kernel<256>, dim3(T), dim3(256), lds, s, logits, T,
                       N, k, R, topk_ids, topk_gates, fallback_ids);
  }
  return launch_status();
}
