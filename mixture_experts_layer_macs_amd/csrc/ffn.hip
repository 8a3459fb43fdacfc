// moe_expert_ffn: grouped SwiGLU expert FFN over the dispatched rows
// ("MACS", §3.1 Eq. 1: E_j(x) for every kept token-expert pair).
//
//   gate-up  h[r] = silu(x[tok(r)] W1_j^T) * (x[tok(r)] W3_j^T)   -> bf16
//   down     out[r] = h[r] W2_j^T                                 -> bf16
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.
// Each workgroup (4 waves) owns one (expert, row tile, column tile).  A and B
// tiles are staged through LDS in BK = 64 slices, double buffered, with the
// 16-byte chunks of each row XOR-swizzled by the row index so the 16-byte
// fragment reads of a wave spread over the banks.  The gate-up tile holds the
// gate rows and the matching up rows of the same h columns, so the SwiGLU
// epilogue pairs two accumulators held by the same lane.  The x rows are
// gathered through row_token inside the load; no permuted x is written.
//
// Tile order: tiles of one expert are contiguous (column tile major, row tile
// minor), and the workgroup id is remapped so that each of the 8 XCDs (which
// receive workgroups round-robin) walks one contiguous range of tiles: the
// row tiles that share an expert's weight panel run on one XCD and share its
// L2.  The grid is an upper bound sized on the host (no device read-back);
// surplus workgroups exit after reading the expert offsets.
#include "common.h"

namespace moe {
namespace ffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { GATEUP = 0, DOWN = 1 };
constexpr int BK = 64;
constexpr int NT = 256;

struct Args {
  const uint16_t* a;       // GATEUP: x [T,H]; DOWN: h [T*k, I]
  const int32_t* row_token;
  const int32_t* offsets;  // [N+1]
  const uint16_t* w;       // GATEUP: w13 [N,2I,H]; DOWN: w2 [N,H,I]
  uint16_t* out;           // GATEUP: h [T*k, I]; DOWN: out_rows [T*k, H]
  int N, K, NC, I;         // K: reduction length; NC: output columns
  long w_stride;           // weight elements per expert
  int n_tiles;
};

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// Locate the tile of this workgroup.  cum: LDS [N+1] cumulative tile counts.
// Returns false for surplus workgroups.
template <int BM>
__device__ bool find_tile(const Args& a, int* cum, int& j, int& m0, int& nt,
                          int& Mj, int& row0) {
  __shared__ int s_total;
  if (threadIdx.x < MOE_WAVE) {
    int acc = 0;
    for (int j0 = 0; j0 < a.N; j0 += MOE_WAVE) {
      const int e = j0 + lane_id();
      int cnt = 0;
      if (e < a.N) {
        const int m = a.offsets[e + 1] - a.offsets[e];
        cnt = ((m + BM - 1) / BM) * a.n_tiles;
      }
      const int inc = wave_incl_scan(cnt);
      if (e < a.N) cum[e + 1] = acc + inc;
      acc += __shfl(inc, MOE_WAVE - 1, MOE_WAVE);
    }
    if (threadIdx.x == 0) {
      cum[0] = 0;
      s_total = acc;
    }
  }
  __syncthreads();
  const int total = s_total;
  const int p = blockIdx.x;
  const int q = (total + 7) / 8;  // tiles per XCD
  const int slot = p / 8;
  if (slot >= q) return false;
  const int L = (p % 8) * q + slot;
  if (L >= total) return false;
  int lo = 0, hi = a.N - 1;  // last expert with cum[e] <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cum[mid] <= L) lo = mid; else hi = mid - 1;
  }
  j = lo;
  row0 = a.offsets[j];
  Mj = a.offsets[j + 1] - row0;
  const int mt = (Mj + BM - 1) / BM;
  const int r = L - cum[j];
  nt = r / mt;
  m0 = (r % mt) * BM;
  return true;
}

template <int MODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(NT) void gemm_kernel(Args a) {
  static_assert(WM * WN == NT / MOE_WAVE, "4 waves");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1, "fragment grid");
  static_assert(MODE == DOWN || FN % 2 == 0, "gate/up pairs");
  constexpr int CPR = BK / 8;               // 16-byte chunks per tile row
  constexpr int A_CH = BM * CPR / NT;       // A chunks per thread per stage
  constexpr int B_CH = BN * CPR / NT;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  __shared__ __align__(16) uint16_t sa[2][BM * BK];
  __shared__ __align__(16) uint16_t sb[2][BN * BK];
  __shared__ int cum[1025];

  int j, m0, nt, Mj, row0;
  if (!find_tile<BM>(a, cum, j, m0, nt, Mj, row0)) return;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / MOE_WAVE;
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K;

  // global source pointers of this thread's chunks
  const uint16_t* ga[A_CH];
  const uint16_t* gb[B_CH];
  int la[A_CH], lb[B_CH];  // LDS element offsets (swizzled)
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT, r = c / CPR, ch = c % CPR;
    const int rr = min(m0 + r, Mj - 1);
    size_t src_row;
    if (MODE == GATEUP)
      src_row = static_cast<size_t>(a.row_token[row0 + rr]);
    else
      src_row = static_cast<size_t>(row0 + rr);
    ga[i] = a.a + src_row * K + ch * 8;
    la[i] = r * BK + ((ch ^ (r & 7)) << 3);
  }
  const uint16_t* wj = a.w + static_cast<size_t>(j) * a.w_stride;
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT, r = c / CPR, ch = c % CPR;
    size_t wrow;
    if (MODE == GATEUP) {
      const int nh0 = nt * (BN / 2);
      wrow = r < BN / 2 ? static_cast<size_t>(nh0 + r)
                        : static_cast<size_t>(a.I + nh0 + (r - BN / 2));
    } else {
      wrow = static_cast<size_t>(nt * BN + r);
    }
    gb[i] = wj + wrow * K + ch * 8;
    lb[i] = r * BK + ((ch ^ (r & 7)) << 3);
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int y = 0; y < FN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  u32x4 ra[A_CH], rb[B_CH];

  const int nk = K / BK;
  {
#pragma unroll
      for (int i = 0; i < A_CH; ++i)
        ra[i] = *(reinterpret_cast<const u32x4*>(ga[i] + 0));
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        rb[i] = *(reinterpret_cast<const u32x4*>(gb[i] + 0));
    }
  {
#pragma unroll
      for (int i = 0; i < A_CH; ++i)
        *reinterpret_cast<u32x4*>(&sa[0][la[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        *reinterpret_cast<u32x4*>(&sb[0][lb[i]]) = rb[i];
    }
  __syncthreads();
  const int frow = lane & 31, fhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i)
        ra[i] = *(reinterpret_cast<const u32x4*>(ga[i] + (kt + 1) * BK));
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        rb[i] = *(reinterpret_cast<const u32x4*>(gb[i] + (kt + 1) * BK));
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + fhalf;
      bf16x8 fa[FM], fb[FN];
#pragma unroll
      for (int x = 0; x < FM; ++x) {
        const int r = wm * TM + x * 32 + frow;
        fa[x] = *reinterpret_cast<const bf16x8*>(&sa[buf][r * BK + ((ch ^ (r & 7)) << 3)]);
      }
#pragma unroll
      for (int y = 0; y < FN; ++y) {
        int r;
        if (MODE == GATEUP)
          r = (y < FN / 2) ? (wn * (TN / 2) + y * 32 + frow)
                           : (BN / 2 + wn * (TN / 2) + (y - FN / 2) * 32 + frow);
        else
          r = wn * TN + y * 32 + frow;
        fb[y] = *reinterpret_cast<const bf16x8*>(&sb[buf][r * BK + ((ch ^ (r & 7)) << 3)]);
      }
#pragma unroll
      for (int x = 0; x < FM; ++x)
#pragma unroll
        for (int y = 0; y < FN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y],
                                                              acc[x][y], 0, 0, 0);
    }
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < A_CH; ++i)
        *reinterpret_cast<u32x4*>(&sa[(buf ^ 1)][la[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < B_CH; ++i)
        *reinterpret_cast<u32x4*>(&sb[(buf ^ 1)][lb[i]]) = rb[i];
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
  const int col = lane & 31;
#pragma unroll
  for (int x = 0; x < FM; ++x) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * TM + x * 32 + 8 * (r / 4) + 4 * fhalf + (r % 4);
      if (m0 + row >= Mj) continue;
      const size_t orow = static_cast<size_t>(row0 + m0 + row);
      if (MODE == GATEUP) {
#pragma unroll
        for (int y = 0; y < FN / 2; ++y) {
          const float g = acc[x][y][r], u = acc[x][y + FN / 2][r];
          const int hc = nt * (BN / 2) + wn * (TN / 2) + y * 32 + col;
          a.out[orow * a.NC + hc] = f32_to_bf16(silu(g) * u);
        }
      } else {
#pragma unroll
        for (int y = 0; y < FN; ++y) {
          const int c = nt * BN + wn * TN + y * 32 + col;
          a.out[orow * a.NC + c] = f32_to_bf16(acc[x][y][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------- fp32 path
// Plain fp32 FMA kernels (small fp32 layers); one thread per output value.
__device__ __forceinline__ int expert_of_row(const int32_t* off, int N, int row) {
  int lo = 0, hi = N - 1;  // last expert with off[e] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gateup_f32(
    const float* __restrict__ x, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ off, const float* __restrict__ w13, int N,
    int H, int I, int rows_cap, float* __restrict__ h) {
  const long gid = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int row = static_cast<int>(gid / I), c = static_cast<int>(gid % I);
  if (row >= rows_cap || row >= off[N]) return;
  const int j = expert_of_row(off, N, row);
  const float* xr = x + static_cast<size_t>(row_token[row]) * H;
  const float* w1 = w13 + (static_cast<size_t>(j) * 2 * I + c) * H;
  const float* w3 = w1 + static_cast<size_t>(I) * H;
  float g = 0.f, u = 0.f;
  for (int kk = 0; kk < H; ++kk) {
    g = fmaf(xr[kk], w1[kk], g);
    u = fmaf(xr[kk], w3[kk], u);
  }
  h[static_cast<size_t>(row) * I + c] = (g / (1.f + expf(-g))) * u;
}

__global__ __launch_bounds__(256) void down_f32(
    const float* __restrict__ h, const int32_t* __restrict__ off,
    const float* __restrict__ w2, int N, int H, int I, int rows_cap,
    float* __restrict__ out) {
  const long gid = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int row = static_cast<int>(gid / H), c = static_cast<int>(gid % H);
  if (row >= rows_cap || row >= off[N]) return;
  const int j = expert_of_row(off, N, row);
  const float* hr = h + static_cast<size_t>(row) * I;
  const float* wr = w2 + (static_cast<size_t>(j) * H + c) * I;
  float acc = 0.f;
  for (int kk = 0; kk < I; ++kk) acc = fmaf(hr[kk], wr[kk], acc);
  out[static_cast<size_t>(row) * H + c] = acc;
}

// ------------------------------------------------------------------ host
template <int MODE, int BM, int BN, int WM, int WN>
static void launch_gemm(const Args& a, int rows_cap, hipStream_t s) {
  const int mt_ub = (rows_cap + BM - 1) / BM + a.N;
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<MODE, BM, BN, WM, WN>), dim3(grid), dim3(NT),
                     0, s, a);
}

}  // namespace ffn
}  // namespace moe

using namespace moe;
using namespace moe::ffn;

// Tile shapes: decode-sized batches (at most 32 rows per expert on average)
// use 32-row tiles so the weight panels stream with little padding work;
// larger batches use 128 x 128 tiles.
static bool decode_tiles(int T, int N, int k) {
  return static_cast<long>(T) * k <= 32L * N;
}

static int check_ffn_shape(int T, int N, int k, int H, int I, int dtype) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      H < 1 || I < 1)
    return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EUNSUP;
  if (dtype == MOE_BF16 && (H % 256 != 0 || I % 128 != 0)) return MOE_EUNSUP;
  if (dtype == MOE_F32 && (H % 4 != 0 || I % 4 != 0)) return MOE_EUNSUP;
  return MOE_OK;
}

extern "C" size_t moe_ffn_workspace_size(int T, int N, int k, int H, int I,
                                         int dtype) {
  (void)N;
  (void)H;
  if (T < 0 || k < 1 || I < 1) return 0;
  const size_t el = dtype == MOE_F32 ? 4 : 2;
  return ((static_cast<size_t>(T) * k * I * el) + 255) & ~size_t(255);
}

extern "C" int moe_ffn_gate_up(const void* x, const int32_t* row_token,
                               const int32_t* expert_offsets, const void* w13,
                               int T, int N, int k, int H, int I, int dtype,
                               void* h, void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !row_token || !expert_offsets || !w13 || !h) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  const int rows_cap = T * k;
  if (dtype == MOE_F32) {
    const long n1 = static_cast<long>(rows_cap) * I;
    hipLaunchKernelGGL(gateup_f32, dim3((n1 + 255) / 256), dim3(256), 0, s,
                       static_cast<const float*>(x), row_token, expert_offsets,
                       static_cast<const float*>(w13), N, H, I, rows_cap,
                       static_cast<float*>(h));
    return launch_status();
  }
  Args g{};
  g.a = static_cast<const uint16_t*>(x);
  g.row_token = row_token;
  g.offsets = expert_offsets;
  g.w = static_cast<const uint16_t*>(w13);
  g.out = static_cast<uint16_t*>(h);
  g.N = N;
  g.K = H;
  g.NC = I;
  g.I = I;
  g.w_stride = 2L * I * H;
  if (decode_tiles(T, N, k)) {
    g.n_tiles = I / 128;
    launch_gemm<GATEUP, 32, 256, 1, 4>(g, rows_cap, s);
  } else {
    g.n_tiles = I / 64;
    launch_gemm<GATEUP, 128, 128, 2, 2>(g, rows_cap, s);
  }
  return launch_status();
}

extern "C" int moe_ffn_down(const void* h, const int32_t* expert_offsets,
                            const void* w2, int T, int N, int k, int H, int I,
                            int dtype, void* out_rows, void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!h || !expert_offsets || !w2 || !out_rows) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  const int rows_cap = T * k;
  if (dtype == MOE_F32) {
    const long n2 = static_cast<long>(rows_cap) * H;
    hipLaunchKernelGGL(down_f32, dim3((n2 + 255) / 256), dim3(256), 0, s,
                       static_cast<const float*>(h), expert_offsets,
                       static_cast<const float*>(w2), N, H, I, rows_cap,
                       static_cast<float*>(out_rows));
    return launch_status();
  }
  Args d{};
  d.a = static_cast<const uint16_t*>(h);
  d.row_token = nullptr;
  d.offsets = expert_offsets;
  d.w = static_cast<const uint16_t*>(w2);
  d.out = static_cast<uint16_t*>(out_rows);
  d.N = N;
  d.K = I;
  d.NC = H;
  d.I = I;
  d.w_stride = static_cast<long>(H) * I;
  if (decode_tiles(T, N, k)) {
    d.n_tiles = H / 256;
    launch_gemm<DOWN, 32, 256, 1, 4>(d, rows_cap, s);
  } else {
    d.n_tiles = H / 128;
    launch_gemm<DOWN, 128, 128, 2, 2>(d, rows_cap, s);
  }
  return launch_status();
}

extern "C" int moe_expert_ffn(const void* x, const int32_t* row_token,
                              const int32_t* expert_offsets, const void* w13,
                              const void* w2, int T, int N, int k, int H,
                              int I, int dtype, void* out_rows,
                              void* workspace, size_t workspace_bytes,
                              void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_ffn_workspace_size(T, N, k, H, I, dtype))
    return MOE_EINVAL;
  const int r = moe_ffn_gate_up(x, row_token, expert_offsets, w13, T, N, k, H,
                                I, dtype, workspace, stream);
  if (r != MOE_OK) return r;
  return moe_ffn_down(workspace, expert_offsets, w2, T, N, k, H, I, dtype,
                      out_rows, stream);
}
