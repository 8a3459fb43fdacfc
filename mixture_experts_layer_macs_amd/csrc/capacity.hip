// moe_capacity_assign: MACS entropy-weighted load, modality-adaptive
// capacity and re-route-else-drop ("MACS", §3.1 Eq. 3, §3.2 Eq. 5-6,
// §3.3 Eq. 7, §1 and Fig. 1).  The phases live in capacity_impl.h; this
// file holds the kernels and the entry point.  When the whole batch fits
// one workgroup (decode) all rounds run in one launch; otherwise each round
// is one launch over the token blocks (up to 128 blocks with no serial
// step between launches, cap_rounds_dec).
#include "capacity_impl.h"

namespace moe {
namespace cap {

__global__ __launch_bounds__(1024) void cap_kernel(Args a, int r_first,
                                                   int r_last) {
  extern __shared__ __align__(16) unsigned char smem[];
  cap_rounds(a, blockIdx.x, r_first, r_last, smem);
}

__global__ __launch_bounds__(256) void cap_dec_kernel(Args a, int r) {
  extern __shared__ __align__(16) unsigned char smem[];
  cap_rounds_dec(a, blockIdx.x, r, smem);
}

__global__ __launch_bounds__(1024) void cap_off_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  cap_off(a, blockIdx.x, smem);
}

}  // namespace cap
}  // namespace moe

using namespace moe;
using namespace moe::cap;

extern "C" size_t moe_capacity_workspace_size(int T, int N, int k) {
  if (T < 0 || N < 1 || k < 1) return 0;
  return layout(T, N, k).bytes;
}

extern "C" int moe_capacity_assign(
    const int32_t* topk_ids, const int32_t* slot_in,
    const int32_t* fallback_ids, const uint8_t* is_visual,
    const float* entropy_w, const int8_t* modality, int T, int N, int k, int R,
    int group, double gamma, double lam, int32_t* slot_out, uint8_t* flags,
    int64_t* load_q, int64_t* cap_q, int64_t* stats, double* r_v,
    void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      R < 0 || R > N - k || group < 1 || group > N)
    return MOE_EINVAL;
  if (std::isnan(gamma) || gamma <= 0.0 || (!std::isinf(gamma) && gamma > 1e30) ||
      !std::isfinite(lam))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !slot_in || (R > 0 && !fallback_ids) || !is_visual ||
      !entropy_w || !modality || !slot_out || !flags || !load_q || !cap_q ||
      !stats || !r_v || !workspace)
    return MOE_EINVAL;
  const Layout L = layout(T, N, k);
  if (workspace_bytes < L.bytes) return MOE_EINVAL;
  const Args a = make_args(topk_ids, slot_in, fallback_ids, is_visual,
                           entropy_w, modality, T, N, k, R, group, gamma, lam,
                           slot_out, flags, load_q, cap_q, stats, r_v,
                           static_cast<char*>(workspace), L);
  hipStream_t s = as_stream(stream);
  const dim3 grid(L.G), block(L.threads);
  if (std::isinf(gamma)) {
    hipLaunchKernelGGL(cap_off_kernel, grid, block, off_lds_bytes(a), s, a);
    return launch_status();
  }
  if (a.dec) {
    const size_t lds = dec_lds_bytes(a);
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(cap_dec_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return MOE_EHIP;
    for (int r = 0; r <= R + 1; ++r)
      hipLaunchKernelGGL(cap_dec_kernel, grid, block, lds, s, a, r);
    return launch_status();
  }
  const size_t lds = rounds_lds_bytes(a);
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(cap_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  if (L.G == 1) {
    hipLaunchKernelGGL(cap_kernel, grid, block, lds, s, a, 0, R + 1);
  } else {
    for (int r = 0; r <= R + 1; ++r)
      hipLaunchKernelGGL(cap_kernel, grid, block, lds, s, a, r, r);
  }
  return launch_status();
}
