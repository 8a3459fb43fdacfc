// moe_sere_reroute: SERE similarity-guided expert re-routing (multi-image QA
// inference write-up, §4.1 algorithm, §4.2 protection matrix, §4.3 fused
// operator): one fused workgroup of 1024 threads, no host round trip, no
// sort (sere_impl.h).
#include "sere_impl.h"

namespace moe {

__global__ __launch_bounds__(1024) void sere_kernel(
    const int32_t* __restrict__ topk, int T, int N, int k, int kprime,
    float rho, const float* __restrict__ sim, const uint8_t* __restrict__ prot,
    int32_t* __restrict__ slot_expert, uint8_t* __restrict__ flags) {
  __shared__ sr::SereLds lds;
  sr::sere_block(topk, T, N, k, kprime, rho, sim, prot, slot_expert, flags, lds);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_sere_reroute(const int32_t* topk_ids, int T, int N, int k,
                                int kprime, float rho, const float* sim,
                                const uint8_t* prot, int32_t* slot_expert,
                                uint8_t* flags, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      kprime < 1 || kprime > k)
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !sim || !prot || !slot_expert || !flags) return MOE_EINVAL;
  hipLaunchKernelGGL(sere_kernel, dim3(1), dim3(1024), 0, as_stream(stream),
                     topk_ids, T, N, k, kprime, rho, sim, prot, slot_expert,
                     flags);
  return launch_status();
}
