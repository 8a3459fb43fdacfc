// moe_route: router softmax and top-k ("MACS", §3.1 Eq. 1).
//
// One 64-lane wave per token.  The token's N logits are spread over the
// lanes (NPL = ceil(N/64) per lane, kept in registers).  The softmax
// statistics are a wave max and a wave sum of exp(l - max) in fp32; the
// ranking is k+R rounds of a wave-wide argmax over a 64-bit key (order-
// preserving image of the fp32 logit, then the inverted expert index so the
// lower index wins a tie).  Ranking compares the fp32 logits themselves, so
// two logits that round to the same exp() value still rank by value.
#include "common.h"

namespace moe {

template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, int T, int N, int k, int R,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_gates,
    int32_t* __restrict__ fallback_ids) {
  const int wave = threadIdx.x / MOE_WAVE;
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / MOE_WAVE) + wave;
  if (t >= T) return;
  const float* row = logits + static_cast<size_t>(t) * N;

  float v[NPL];
  uint64_t key[NPL];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + i * MOE_WAVE;
    v[i] = j < N ? row[j] : -INFINITY;
    key[i] = j < N ? rank_key(v[i], j) : 0ull;
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + i * MOE_WAVE;
    if (j < N) se += expf(v[i] - mx);
  }
  se = wave_sum(se);

  const int n_pick = k + R;
  for (int r = 0; r < n_pick; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = rank_key_index(best);
    // retire the winner (it lives in exactly one lane/register)
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (key[i] == best) key[i] = 0ull;
    if (lane == 0) {
      if (r < k) {
        topk_ids[static_cast<size_t>(t) * k + r] = e;
        // the winning logit is recovered from its key: no reload
        topk_gates[static_cast<size_t>(t) * k + r] =
            expf(rank_key_value(best) - mx) / se;
      } else {
        fallback_ids[static_cast<size_t>(t) * R + (r - k)] = e;
      }
    }
  }
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
  const int waves = 4;
  dim3 grid((T + waves - 1) / waves), block(waves * MOE_WAVE);
  hipStream_t s = as_stream(stream);
  const int npl = (N + MOE_WAVE - 1) / MOE_WAVE;
#define MOE_ROUTE(NP)                                                        \
  hipLaunchKernelGGL(route_kernel<NP>, grid, block, 0, s, logits, T, N, k, R, \
                     topk_ids, topk_gates, fallback_ids)
  if (npl <= 1) MOE_ROUTE(1);
  else if (npl <= 2) MOE_ROUTE(2);
  else if (npl <= 4) MOE_ROUTE(4);
  else if (npl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  return launch_status();
}
