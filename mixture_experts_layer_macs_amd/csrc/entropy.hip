// moe_entropy_weights: semantic token weights from the softmax entropy of
// each visual token's features ("MACS", §3.2 Eq. 4-5).
//
//   H(x_t) = -sum_i p_i ln p_i,  p = softmax(x_t)      (natural log)
//          = ln Z - S / Z,  Z = sum_i e^(z_i - m), S = sum_i e^(z_i - m)(z_i - m)
//   H~ = (H - mu) / (sigma + eps),  mu, sigma over the batch's visual tokens
//   w = 1 / (1 + e^(delta H~)) for visual tokens, 1 for text tokens
//
// One wave per token: bf16 rows up to 4096 values are loaded into registers
// in one batch (one memory round trip), the lane maxima and then the sums Z
// and S are taken in fp32 and combined across the wave with DPP reductions;
// other rows take two passes over memory.  Each workgroup adds its visual
// tokens' H and H^2 in fp64 and writes the partial sums.  A second launch
// (the kernel boundary orders the memory: no fences, no atomics) reduces
// the partials into mu and the population sigma and writes every token's
// weight.  HBM-bound: the row is
// read once from HBM.
#include <cmath>

#include "common.h"

namespace moe {
namespace ent {

constexpr int NT = 256;  // 4 waves, one token each per step

struct Args {
  const void* x;
  const uint8_t* is_visual;
  int T, H, dtype;
  float delta, eps;
  float* w;
  float* ent;         // H per token (workspace or caller's buffer)
  double* partial;    // [G][2] per-workgroup sums of H and H^2 (visual)
  int* count;         // [G] visual tokens per workgroup
};

__device__ __forceinline__ float load_elem(const Args& a, size_t i) {
  if (a.dtype == MOE_BF16) {
    const uint16_t b = static_cast<const uint16_t*>(a.x)[i];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  return static_cast<const float*>(a.x)[i];
}

// Entropy of one bf16 row held in registers: NCH 16-byte chunks per lane
// (8 values each), all loaded before any is used.  Whole wave; result in
// every lane.
template <int NCH>
__device__ float row_entropy_regs(const Args& a, int t) {
  const uint4* r = reinterpret_cast<const uint4*>(
      static_cast<const uint16_t*>(a.x) + static_cast<size_t>(t) * a.H);
  const int lane = lane_id(), n8 = a.H / 8;
  uint4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = lane + c * MOE_WAVE;
    v[c] = i < n8 ? r[i] : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
  }
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t w4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, __uint_as_float(w4[i] << 16));
      m = fmaxf(m, __uint_as_float(w4[i] & 0xffff0000u));
    }
  }
  m = wave_max(m);
  float Z = 0.f, S = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane + c * MOE_WAVE < n8) {
      const uint32_t w4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d0 = __uint_as_float(w4[i] << 16) - m;
        const float d1 = __uint_as_float(w4[i] & 0xffff0000u) - m;
        const float e0 = expf(d0), e1 = expf(d1);
        Z += e0 + e1;
        S += e0 * d0 + e1 * d1;
      }
    }
  }
  Z = wave_sum(Z);
  S = wave_sum(S);
  return logf(Z) - S / Z;
}

// Any row: two passes (max, then sums; the row is in cache for the second).
__device__ float row_entropy(const Args& a, int t) {
  const size_t base = static_cast<size_t>(t) * a.H;
  const int lane = lane_id();
  float m = -INFINITY;
  for (int i = lane; i < a.H; i += MOE_WAVE) m = fmaxf(m, load_elem(a, base + i));
  m = wave_max(m);
  float Z = 0.f, S = 0.f;
  for (int i = lane; i < a.H; i += MOE_WAVE) {
    const float d = load_elem(a, base + i) - m;
    const float e = expf(d);
    Z += e;
    S += e * d;
  }
  Z = wave_sum(Z);
  S = wave_sum(S);
  return logf(Z) - S / Z;
}

// NCH > 0: bf16 rows of at most NCH*512 values held in registers.
template <int NCH>
__global__ __launch_bounds__(NT) void entropy_kernel(Args a, int tokens_per_block) {
  __shared__ double sh[NT / MOE_WAVE][2];
  __shared__ int sc[NT / MOE_WAVE];
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int t0 = blockIdx.x * tokens_per_block;
  const int t1 = min(a.T, t0 + tokens_per_block);
  double s1 = 0.0, s2 = 0.0;
  int cnt = 0;
  for (int t = t0 + wave; t < t1; t += NT / MOE_WAVE) {
    float h;
    if constexpr (NCH > 0)
      h = row_entropy_regs<NCH>(a, t);
    else
      h = row_entropy(a, t);
    if (lane == 0) {
      a.ent[t] = h;
      if (a.is_visual[t]) {
        s1 += h;
        s2 += static_cast<double>(h) * h;
        ++cnt;
      }
    }
  }
  if (lane == 0) {
    sh[wave][0] = s1;
    sh[wave][1] = s2;
    sc[wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double b1 = 0.0, b2 = 0.0;
    int bc = 0;
    for (int w = 0; w < NT / MOE_WAVE; ++w) {  // fixed order
      b1 += sh[w][0];
      b2 += sh[w][1];
      bc += sc[w];
    }
    a.partial[2 * blockIdx.x] = b1;
    a.partial[2 * blockIdx.x + 1] = b2;
    a.count[blockIdx.x] = bc;
  }
}

// Second launch: every workgroup reduces the first launch's per-workgroup
// partials in the same fixed order (so all of them obtain the same mu and
// sigma, deterministically), then writes the weights of its tokens.
__global__ __launch_bounds__(NT) void weight_kernel(Args a, int G1) {
  __shared__ double sh[NT / MOE_WAVE][2];
  __shared__ int sc[NT / MOE_WAVE];
  __shared__ float s_mu, s_den;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  double S1 = 0.0, S2 = 0.0;
  int n = 0;
  for (int g = threadIdx.x; g < G1; g += NT) {
    S1 += a.partial[2 * g];
    S2 += a.partial[2 * g + 1];
    n += a.count[g];
  }
  S1 = wave_sum_f64(S1);
  S2 = wave_sum_f64(S2);
  n = wave_sum(n);
  if (lane == 0) {
    sh[wave][0] = S1;
    sh[wave][1] = S2;
    sc[wave] = n;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    S1 = S2 = 0.0;
    n = 0;
    for (int w = 0; w < NT / MOE_WAVE; ++w) {
      S1 += sh[w][0];
      S2 += sh[w][1];
      n += sc[w];
    }
    double mu = 0.0, var = 0.0;
    if (n > 0) {
      mu = S1 / static_cast<double>(n);
      var = S2 / static_cast<double>(n) - mu * mu;
    }
    s_mu = static_cast<float>(mu);
    s_den = static_cast<float>(var > 0.0 ? sqrt(var) : 0.0) + a.eps;
  }
  __syncthreads();
  const int t = blockIdx.x * NT + threadIdx.x;
  if (t >= a.T) return;
  float w = 1.f;
  if (a.is_visual[t]) w = 1.f / (1.f + expf(a.delta * ((a.ent[t] - s_mu) / s_den)));
  a.w[t] = w;
}

struct Layout {
  int G, TPB;
  size_t ent, partial, count, bytes;
};

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout layout(int T) {
  Layout L{};
  L.TPB = NT / MOE_WAVE;  // tokens per workgroup: one per wave
  L.G = T > 0 ? (T + L.TPB - 1) / L.TPB : 1;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o = align_up(o + n);
    return at;
  };
  L.ent = take(sizeof(float) * static_cast<size_t>(T > 0 ? T : 1));
  L.partial = take(sizeof(double) * 2 * static_cast<size_t>(L.G));
  L.count = take(sizeof(int) * static_cast<size_t>(L.G));
  L.bytes = o;
  return L;
}

}  // namespace ent
}  // namespace moe

using namespace moe;

extern "C" size_t moe_entropy_workspace_size(int T) {
  if (T < 0) return 0;
  return ent::layout(T).bytes;
}

extern "C" int moe_entropy_weights(const void* x, const uint8_t* is_visual, int T,
                                   int H, int dtype, float delta, float eps,
                                   float* entropy_w, float* entropy,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (T < 0 || T > (1 << 20) || H < 1 || H > (1 << 20)) return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EUNSUP;
  if (!std::isfinite(delta) || !std::isfinite(eps) || eps < 0.f) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !is_visual || !entropy_w || !workspace) return MOE_EINVAL;
  const ent::Layout L = ent::layout(T);
  if (workspace_bytes < L.bytes) return MOE_EINVAL;
  char* ws = static_cast<char*>(workspace);
  ent::Args a{};
  a.x = x;
  a.is_visual = is_visual;
  a.T = T;
  a.H = H;
  a.dtype = dtype;
  a.delta = delta;
  a.eps = eps;
  a.w = entropy_w;
  a.ent = entropy ? entropy : reinterpret_cast<float*>(ws + L.ent);
  a.partial = reinterpret_cast<double*>(ws + L.partial);
  a.count = reinterpret_cast<int*>(ws + L.count);

  hipStream_t s = as_stream(stream);
  const bool regs = dtype == MOE_BF16 && H % 8 == 0 && H <= 4096 &&
                    (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  const int nch = (H / 8 + MOE_WAVE - 1) / MOE_WAVE;
#define MOE_ENT(NC) \
  hipLaunchKernelGGL(ent::entropy_kernel<NC>, dim3(L.G), dim3(ent::NT), 0, s, a, L.TPB)
  if (!regs) MOE_ENT(0);
  else if (nch <= 1) MOE_ENT(1);
  else if (nch <= 2) MOE_ENT(2);
  else if (nch <= 4) MOE_ENT(4);
  else MOE_ENT(8);
#undef MOE_ENT
  hipLaunchKernelGGL(ent::weight_kernel, dim3((T + ent::NT - 1) / ent::NT), dim3(ent::NT), 0,
                     s, a, L.G);
  return launch_status();
}
