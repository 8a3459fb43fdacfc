// moe_dispatch: stable counting sort of the kept slots into expert-major
// rows, (token, slot) ascending inside each expert.  The rows feed the
// grouped expert GEMMs, which gather the token rows of x themselves, so no
// permuted copy of the activations is ever written.
//
// Same block decomposition as the capacity step: each workgroup ranks its
// own slots per expert (ordered per-key prefix with unit weights) and
// writes its per-expert counts; in a second launch every workgroup sums the
// counts into the expert offsets and its own bases and scatters the row
// maps.  Beyond 128 workgroups the last workgroup of the first launch (an
// atomic ticket) computes offsets and bases for all instead.  A batch that
// fits one workgroup does everything in a single launch.
#include "dispatch_impl.h"

namespace moe {
namespace disp {

// phase 0: count (+ offsets and bases by the last block beyond 128 blocks);
// phase 1: scatter (+ its own offsets and bases up to 128 blocks); single
// block: all of it
__global__ __launch_bounds__(1024) void dispatch_kernel(Args a, int phase_first,
                                                        int phase_last) {
  extern __shared__ __align__(16) unsigned char smem[];
  // [tot: N int32][run table / scan staging: lds_scan int32]
  int32_t* tot = reinterpret_cast<int32_t*>(smem);
  int32_t* run = tot + a.N;
  __shared__ int s_last;
  const int g = blockIdx.x;
  const int t0 = g * a.TB, t1 = min(a.T, t0 + a.TB);
  if (phase_first == 1 && a.G <= DEC_MAX_G) {  // after a count-only launch
    scatter_dec(a, g, smem);
    return;
  }
  if (phase_first == 0) {
    count_block(a, g, t0, t1, run);
    if (a.G > 1 && a.G <= DEC_MAX_G) return;  // the next launch does the rest
    if (a.G > 1) {  // one agent-scope fence per workgroup, not per wave
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0) {
        __threadfence();
        const unsigned prev = atomicInc(a.ticket, static_cast<unsigned>(a.G - 1));
        s_last = prev == static_cast<unsigned>(a.G - 1);
        if (s_last) __threadfence();
      }
      __syncthreads();
      if (!s_last) return;
    }
    scan_offsets(a, tot, run);
    __syncthreads();
  }
  if (phase_last == 1)
    scatter_block(a, t0, t1, a.offsets, a.base + static_cast<size_t>(g) * a.N);
}

}  // namespace disp
}  // namespace moe

using namespace moe;
using namespace moe::disp;

extern "C" size_t moe_dispatch_workspace_size(int T, int N, int k) {
  if (T < 0 || N < 1 || k < 1) return 0;
  return layout(T, N, k).bytes;
}

extern "C" int moe_dispatch(const int32_t* slot_expert, int T, int N, int k,
                            int32_t* expert_offsets, int32_t* row_token,
                            int32_t* row_slot, int32_t* slot_row,
                            void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N)
    return MOE_EINVAL;
  if (!expert_offsets) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  if (T == 0) return MOE_OK;
  if (!slot_expert || !row_token || !row_slot || !slot_row || !workspace)
    return MOE_EINVAL;
  const Layout L = layout(T, N, k);
  if (workspace_bytes < L.bytes) return MOE_EINVAL;
  const Args a = make_args(slot_expert, T, N, k, expert_offsets, row_token,
                           row_slot, slot_row, static_cast<char*>(workspace), L);
  const size_t lds = lds_bytes(a);
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(dispatch_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  if (L.G == 1) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(L.threads), lds, s, a, 0, 1);
  } else {
    hipLaunchKernelGGL(dispatch_kernel, dim3(L.G), dim3(L.threads), lds, s, a, 0, 0);
    hipLaunchKernelGGL(dispatch_kernel, dim3(L.G), dim3(L.threads), lds, s, a, 1, 1);
  }
  return launch_status();
}
