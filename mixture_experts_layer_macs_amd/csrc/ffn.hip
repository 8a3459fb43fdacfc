// moe_expert_ffn: grouped SwiGLU expert FFN over the dispatched rows
// ("MACS", §3.1 Eq. 1: E_j(x) for every kept token-expert pair).
//
//   gate-up  h[r] = silu(x[tok(r)] W1_j^T) * (x[tok(r)] W3_j^T)   -> bf16
//   down     out[r] = h[r] W2_j^T                                 -> bf16
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation.
// Each workgroup (4 waves) owns one (expert, row tile, column tile).  A and B
// tiles travel global -> LDS by direct-to-LDS loads through a ring of S
// stages, with the 16-byte chunks of each row XOR-swizzled so that fragment
// reads of a wave are bank-conflict free.  The gate-up tile holds the gate
// rows and the matching up rows of the same h columns, so the SwiGLU
// epilogue pairs two accumulators held by the same lane.  The x rows are
// gathered through row_token inside the load; no permuted x is written.
//
// Tile order: tiles of one expert are contiguous (column tile major, row tile
// minor), and the workgroup id is remapped so that each of the 8 XCDs (which
// receive workgroups round-robin) walks one contiguous range of tiles: the
// row tiles that share an expert's weight panel run on one XCD and share its
// L2.  The grid is an upper bound sized on the host (no device read-back);
// surplus workgroups exit after reading the expert offsets.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "dma.h"

namespace moe {
namespace ffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { GATEUP = 0, DOWN = 1 };

struct Args {
  const uint16_t* a;       // GATEUP: x [T,H]; DOWN: h [T*k, I]
  int a_rows;              // rows of a (GATEUP: T; DOWN: T*k)
  const int32_t* row_token;
  const int32_t* offsets;  // [N+1]
  const uint16_t* w;       // GATEUP: w13 [N,2I,H]; DOWN: w2 [N,H,I]
  uint16_t* out;           // GATEUP: h [T*k, I]; DOWN: out_rows [T*k, H]
  int N, K, NC, I;         // K: reduction length; NC: output columns
  long w_stride;           // weight elements per expert
  int n_tiles;
  int dual_limit;          // gemm_dual_kernel: most tiles of the first height
  int panels;              // 1: w in the panel layout (moe_pack_weights)
};

// The gate-weighted combine folded into the down GEMV (moe_expert_ffn_combine).
struct Comb {
  const int32_t* slot_row;  // [T,k] dispatch row of each slot, -1 = dropped
  const float* gates;       // [T,k]
  uint16_t* y;              // [T,H] bf16
  unsigned* ticket;         // [H/32] arrivals per output column group (zero between calls)
  int T, k;
};

// Two fp32 values to a packed bf16 pair (round to nearest even), one
// v_cvt_pk_bf16_f32 on gfx950; the first value lands in the low half.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  const bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// silu(g) = g / (1 + e^-g), with the hardware exponential and reciprocal
// (about 1 ulp each; the result is rounded to bf16 afterwards).
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// ------------------------------------------------------------ panel layout
// moe_pack_weights stores each expert's weight matrix for the MFMA operand
// order.  Rows, in tile order, form panels of 128; a panel is stored as K/64
// consecutive blocks of 16 KB (128 rows x 64 K elements), and inside a block
// the bytes follow the 32 x 32 x 16 MFMA operand: for row group G (32 rows)
// and K step kk (16 elements), 1 KB holding, for lane l, the 8 elements
// 8 (l / 32) .. +7 of step kk of row l % 32 of the group.  A wave's operand
// for one K step is then one contiguous 1 KB load, and one 64-wide K slice
// of a 128-row panel one contiguous 16 KB block.
//
// Tile order of w13: panel P holds h columns 64P .. 64P+63 as four groups of
// 32 rows, group G = 16 gate rows (columns 64P+16G .. +15) followed by the
// 16 up rows of the same columns, so that the gate and up value of one h
// column meet in one lane's accumulators.  Tile order of w2: its rows.
constexpr uint32_t PANEL_ROWS = 128, PANEL_K = 64, PANEL_BLOCK = PANEL_ROWS * PANEL_K * 2;

// Tile-order row of w13 row wrow (gate rows 0 .. I-1, then the up rows).
__host__ __device__ __forceinline__ uint32_t w13_tile_row(uint32_t wrow, uint32_t I) {
  const uint32_t up = wrow >= I, c = up ? wrow - I : wrow;
  return (c / 64) * PANEL_ROWS + ((c % 64) / 16) * 32 + up * 16 + c % 16;
}

// Byte offset, from the start of one expert's packed block, of the 16-byte
// chunk of tile-order row t that starts at element k (k % 8 == 0), K being
// the reduction length.
__host__ __device__ __forceinline__ uint32_t panel_off(uint32_t t, uint32_t k, uint32_t K) {
  const uint32_t blk = (t / PANEL_ROWS) * (K / PANEL_K) + k / PANEL_K;
  const uint32_t G = (t % PANEL_ROWS) / 32, kk = (k % PANEL_K) / 16, half = (k % 16) / 8;
  return blk * PANEL_BLOCK + ((G * 4 + kk) * 64 + half * 32 + t % 32) * 16;
}

// Byte offset, inside one expert's weight block, of the 16-byte chunk at
// element kelem (a multiple of 8 below the slice width) of weight row wrow
// in a K slice starting at element 0; weight_k0 adds the slice start.
template <int MODE>
__device__ __forceinline__ uint32_t weight_off(const Args& a, uint32_t wrow, uint32_t kelem) {
  if (!a.panels) return wrow * static_cast<uint32_t>(a.K) * 2 + kelem * 2;
  const uint32_t t = MODE == GATEUP ? w13_tile_row(wrow, a.I) : wrow;
  return panel_off(t, kelem, static_cast<uint32_t>(a.K));
}

// Byte offset of K slice start kelem (a multiple of the slice width, 16 or
// more), added to every weight_off of that slice: whole blocks, then whole
// K steps inside the block (each step's 1 KB groups sit 1 KB apart).
__device__ __forceinline__ uint32_t weight_k0(const Args& a, uint32_t kelem) {
  return a.panels ? (kelem / PANEL_K) * PANEL_BLOCK + ((kelem % PANEL_K) / 16) * 1024 : kelem * 2;
}

// Tile table: cum (LDS [N+2]) receives the cumulative tile counts of the
// experts (BM-row tiles times a.n_tiles column tiles) and then the total,
// which is returned (after a barrier) to every thread.
template <int BM>
__device__ int tile_table(const Args& a, int* cum) {
  int* s_total = cum + a.N + 1;
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
      acc += read_lane(inc, MOE_WAVE - 1);
    }
    if (threadIdx.x == 0) {
      cum[0] = 0;
      *s_total = acc;
    }
  }
  __syncthreads();
  return *s_total;
}

// Tile L of the table: expert j (rows row0 .. row0 + Mj - 1), token rows
// m0 .. m0 + BM - 1 of it, column tile nt.
template <int BM>
__device__ __forceinline__ void locate_tile(const Args& a, const int* cum, int L, int& j,
                                            int& m0, int& nt, int& Mj, int& row0) {
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
}

// Locate the tile of this workgroup.  cum: LDS [N+2], the cumulative tile
// counts and then the total.  Returns false for surplus workgroups.
template <int BM>
__device__ bool find_tile(const Args& a, int* cum, int& j, int& m0, int& nt,
                          int& Mj, int& row0) {
  const int total = tile_table<BM>(a, cum);
  const int p = blockIdx.x;
  const int q = (total + 7) / 8;  // tiles per XCD
  const int slot = p / 8;
  if (slot >= q) return false;
  const int L = (p % 8) * q + slot;
  if (L >= total) return false;
  locate_tile<BM>(a, cum, L, j, m0, nt, Mj, row0);
  return true;
}

// The same search held in registers, for N < 64 * REG_CHUNKS experts: each
// wave reads the expert offsets itself in one batch of loads, counts tiles
// with a prefix scan, and finds the expert of tile L by a ballot (the
// number of experts whose inclusive tile count is at most L), so no LDS
// table, no workgroup barrier and no chain of dependent reads comes before
// the first weight request.  Lane l of chunk c stands for expert l + 64 c.
constexpr int REG_CHUNKS = 5;
struct TileRegs {
  int cum[REG_CHUNKS];  // inclusive tile counts
  int o0[REG_CHUNKS];   // offsets[e]
  int o1[REG_CHUNKS];   // offsets[e + 1]
  int total;
};

template <int BM>
__device__ __forceinline__ void tile_regs(const Args& a, TileRegs& tr) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < REG_CHUNKS; ++c) {
    const int e = lane + 64 * c;
    tr.o0[c] = a.offsets[min(e, a.N)];
    tr.o1[c] = a.offsets[min(e + 1, a.N)];
  }
  int carry = 0;
#pragma unroll
  for (int c = 0; c < REG_CHUNKS; ++c) {
    const int e = lane + 64 * c;
    const int m = e < a.N ? tr.o1[c] - tr.o0[c] : 0;
    const int inc = wave_incl_scan(((m + BM - 1) / BM) * a.n_tiles);
    tr.cum[c] = carry + inc;
    carry += read_lane(inc, MOE_WAVE - 1);
  }
  tr.total = __builtin_amdgcn_readfirstlane(carry);
}

template <int BM>
__device__ __forceinline__ void locate_regs(const Args& a, const TileRegs& tr, int L, int& j,
                                            int& m0, int& nt, int& Mj, int& row0) {
  const int lane = lane_id();
  int jj = 0;
#pragma unroll
  for (int c = 0; c < REG_CHUNKS; ++c)
    jj += __popcll(__ballot(lane + 64 * c < a.N && tr.cum[c] <= L));
  j = jj;  // L < total, so j < N
  const int cj = j / 64, lj = j % 64;
  int cum = 0, o0 = 0, o1 = 0;
#pragma unroll
  for (int c = 0; c < REG_CHUNKS; ++c)
    if (c == cj) {
      cum = read_lane(tr.cum[c], lj);
      o0 = read_lane(tr.o0[c], lj);
      o1 = read_lane(tr.o1[c], lj);
    }
  row0 = o0;
  Mj = o1 - o0;
  const int mt = (Mj + BM - 1) / BM;
  const int r = L - (cum - mt * a.n_tiles);
  nt = r / mt;
  m0 = (r % mt) * BM;
}

// ------------------------------------------------- direct-to-LDS pipeline
// Prefill variant: A and B slices travel global -> LDS with
// global_load_lds_dwordx4 (16 bytes per lane, 1 KB per wave instruction,
// written at consecutive LDS addresses), so no VGPRs hold staged tiles and
// the whole register file serves the accumulators and fragments.  S LDS
// stages form a ring; slice kt+S-1 is requested while slice kt is consumed.
// The swizzle is applied on the global side: the lane that fills LDS slot
// (row, s) fetches chunk s ^ ((row >> SWS) & SWZ) of that row.

// The DMA helpers (buffer resource, direct-to-LDS load, counted waits) are
// in dma.h.

// Scheduling groups of one sub-slice: its NMF MFMAs split as evenly as
// possible over its NFR fragment reads, one read after each group.
template <int NMF, int NFR, int I = 0>
__device__ __forceinline__ void interleave_groups() {
  if constexpr (I < NFR) {
    __builtin_amdgcn_sched_group_barrier(0x0008, NMF / NFR + (I < NMF % NFR ? 1 : 0), 0);
    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // DS read
    interleave_groups<NMF, NFR, I + 1>();
  }
}

// The tile of expert j, rows m0 .. m0 + BM - 1 of its Mj rows (dispatch rows
// from row0), column tile nt, computed by WM x WN waves (4 or 8) with an
// S-stage ring in smem (the dynamic LDS block).  All five values are the
// same in every lane.
template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int SB = S>
__device__ __forceinline__ void gemm_body(const Args& a, unsigned char* smem, int j, int m0,
                                          int nt, int Mj, int row0) {
  static_assert(S >= 2 && S <= 8, "pipeline depth");
  constexpr int W = WM * WN, NTH = W * MOE_WAVE;  // waves, threads
  static_assert(W == 4 || W == 8, "4 or 8 waves");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  // Gate-up pairing: with an even number of fragment columns per wave, the
  // first half holds gate rows and the second half the matching up rows;
  // with a single fragment column (MIX) each 32-row fragment holds 16 gate
  // rows and then the 16 matching up rows, so gate row i and up row i sit in
  // accumulator registers r and r + 8 of the same lane.
  constexpr bool MIX = MODE == GATEUP && FN == 1;
  static_assert(MODE == DOWN || MIX || FN % 2 == 0, "gate/up pairs");
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  constexpr int SWZ = CPR - 1;
  constexpr int SWS = BK == 64 ? 1 : (BK == 32 ? 2 : 0);  // 256-byte bank rows
  constexpr int RPJ = MOE_WAVE / CPR;         // rows per DMA instruction
  constexpr int NA = BM / RPJ, NB = BN / RPJ; // instructions per stage
  static_assert(NA % W == 0 && NB % W == 0, "split over the waves");
  constexpr int QA = NA / W, QB = NB / W;     // per wave
  constexpr int LPW = QA + QB;                // DMA loads per wave per stage
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  // Ring layout.  Symmetric (SB == S): stage s holds slice A then slice B.
  // Asymmetric: S stages of A, then SB stages of B, so the weights can be
  // requested further ahead than the token rows (or, with 3 and 2, the
  // token rows further ahead).
  constexpr bool ASYM = SB != S;
  static_assert(!ASYM || (S == 2 && SB >= 3) || (S == 3 && SB == 2),
                "asymmetric ring: 2 A stages and 3 or more B stages, or 3 and 2");
  constexpr int A_STRIDE = ASYM ? A_BYTES : STAGE;
  constexpr int B_BASE = ASYM ? S * A_BYTES : A_BYTES;
  constexpr int B_STRIDE = ASYM ? B_BYTES : STAGE;

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2;

  // A: gate-up gathers x rows by token (resource over all of x); down reads
  // the tile's own rows of h (resource from the tile's first row).  B: the
  // expert's weight block.  Byte offsets fit 32 bits (checked on the host).
  const int tile_rows = min(BM, Mj - m0);
  const i32x4 rsrc_a =
      MODE == GATEUP
          ? buffer_rsrc(a.a, static_cast<uint32_t>(a.a_rows) * row_bytes)
          : buffer_rsrc(a.a + static_cast<size_t>(row0 + m0) * K,
                        static_cast<uint32_t>(tile_rows) * row_bytes);
  const i32x4 rsrc_b = buffer_rsrc(a.w + static_cast<size_t>(j) * a.w_stride,
                                   static_cast<uint32_t>(a.w_stride) * 2);

  // per-lane byte offsets of this wave's loads (fixed over the K loop).
  // Rows past the tile's last row get an offset outside their resource's
  // range, so their loads fill LDS with zeros and fetch nothing: for down
  // that is any offset past the tile's rows, for gate-up OOB_OFF (x spans
  // at most 2^31 bytes, checked on the host).
  const int lrow = lane / CPR, lslot = lane % CPR;
  uint32_t va[QA], vb[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int row = (wave * QA + q) * RPJ + lrow;
    const int ch = lslot ^ ((row >> SWS) & SWZ);
    if (MODE == GATEUP)
      va[q] = row < tile_rows
                  ? static_cast<uint32_t>(a.row_token[row0 + m0 + row]) * row_bytes + ch * 16
                  : OOB_OFF;
    else
      va[q] = static_cast<uint32_t>(row) * row_bytes + ch * 16;
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int row = (wave * QB + q) * RPJ + lrow;
    const int ch = lslot ^ ((row >> SWS) & SWZ);
    uint32_t wrow;
    if (MIX) {
      const int hc = nt * (BN / 2) + (row / 32) * 16 + (row % 16);
      wrow = (row % 32) < 16 ? hc : a.I + hc;
    } else if (MODE == GATEUP) {
      wrow = row < BN / 2 ? nt * (BN / 2) + row : a.I + nt * (BN / 2) + (row - BN / 2);
    } else {
      wrow = nt * BN + row;
    }
    vb[q] = weight_off<MODE>(a, wrow, ch * 8);
  }
  // LDS byte address of the dynamic LDS block (M0 wants it as 32 bits)
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));
  // Slice kslice goes to ring stage kslice % S.  Requests past the last
  // slice re-fetch the last slice into a stage that is never read again, so
  // every iteration issues the same number of loads.  Load d < QA of a
  // slice is the wave's A row group d, the rest its B row groups.
  const int nk = K / BK;
  auto dma = [&](int kslice, int d) {
    const uint32_t ke = static_cast<uint32_t>(min(kslice, nk - 1) * BK);
    if (d < QA)
      lds_dma16(rsrc_a, va[d], ke * 2,
                lds_base + (kslice % S) * A_STRIDE + (wave * QA + d) * 1024);
    else
      lds_dma16(rsrc_b, vb[d - QA], weight_k0(a, ke),
                lds_base + B_BASE + (kslice % SB) * B_STRIDE + (wave * QB + d - QA) * 1024);
  };
  auto issue = [&](int kslice) {
#pragma unroll
    for (int d = 0; d < LPW; ++d) dma(kslice, d);
  };
  auto issue_a = [&](int kslice) {
#pragma unroll
    for (int d = 0; d < QA; ++d) dma(kslice, d);
  };
  auto issue_b = [&](int kslice) {
#pragma unroll
    for (int d = QA; d < LPW; ++d) dma(kslice, d);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int y = 0; y < FN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int frow = lane & 31, fhalf = lane >> 5;
  const int a_lane = (wm * TM + frow) * BK;
  const int b_lane = (MODE == GATEUP && !MIX ? wn * (TN / 2) + frow : wn * TN + frow) * BK;
  auto brow_rel = [](int y) {
    if (MODE == GATEUP && !MIX)
      return (y < FN / 2) ? y * 32 : BN / 2 + (y - FN / 2) * 32;
    return y * 32;
  };

  // Ring protocol (slice t in stage t % S, D = S - 2 slices requested ahead):
  //  - before the last sub-slice of slice kt: wait for this wave's loads of
  //    slice kt+1, barrier (everyone's slice kt+1 landed; everyone's reads of
  //    slice kt-1 are long consumed), request slice kt+1+D into the stage of
  //    slice kt-1;
  //  - the last sub-slice's MFMAs overlap the reads of slice kt+1's first
  //    fragments, so no LDS latency is exposed at slice boundaries.
  constexpr int D = S > 2 ? S - 2 : 1;
  constexpr int KK = BK / 16;
  constexpr int NFR = FM + FN, NMF = FM * FN;
  // fragment reads go through an LDS-typed pointer so they stay ds_read
  typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) const unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](int kslice, int kk, bf16x8* pa, bf16x8* pb) {
    lds_byte* A_ = lds0 + (kslice % S) * A_STRIDE;
    lds_byte* B_ = lds0 + B_BASE + (kslice % SB) * B_STRIDE;
    const int sw = ((kk * 2 + fhalf) ^ ((frow >> SWS) & SWZ)) << 4;  // bytes
#pragma unroll
    for (int x = 0; x < FM; ++x)
      pa[x] = *(lds_frag*)(A_ + (a_lane + x * 32 * BK) * 2 + sw);
#pragma unroll
    for (int y = 0; y < FN; ++y)
      pb[y] = *(lds_frag*)(B_ + (b_lane + brow_rel(y) * BK) * 2 + sw);
  };
  // The same reads, with the DMA requests of slice kslice spread over them
  // (load d after fragment read d * NFR / LPW), so that no run of requests
  // holds up the MFMAs that the scheduler places between the reads.
  auto read_frags_dma = [&](int rslice, int kk, bf16x8* pa, bf16x8* pb, int kslice) {
    lds_byte* A_ = lds0 + (rslice % S) * A_STRIDE;
    lds_byte* B_ = lds0 + B_BASE + (rslice % SB) * B_STRIDE;
    const int sw = ((kk * 2 + fhalf) ^ ((frow >> SWS) & SWZ)) << 4;  // bytes
#pragma unroll
    for (int f = 0; f < NFR; ++f) {
      if (f < FM)
        pa[f] = *(lds_frag*)(A_ + (a_lane + f * 32 * BK) * 2 + sw);
      else
        pb[f - FM] = *(lds_frag*)(B_ + (b_lane + brow_rel(f - FM) * BK) * 2 + sw);
#pragma unroll
      for (int d = f * LPW / NFR; d < (f + 1) * LPW / NFR; ++d) dma(kslice, d);
    }
  };
  auto mma = [&](const bf16x8* pa, const bf16x8* pb) {
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
      for (int y = 0; y < FN; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[y], pa[x], acc[x][y], 0, 0, 0);
  };
  auto interleave = [&]() { interleave_groups<NMF, NFR>(); };

  if constexpr (BM < 256 || S == 2) {
    // Streaming ring (decode tiles, and prefill tiles with two stages): S - 1
    // slices are requested ahead.  At the top of iteration kt a wave waits
    // until its loads of slice kt have landed (the S - 2 newer slices stay
    // in flight), the barrier publishes everyone's, and slice kt + S - 1 is
    // requested into the stage of slice kt - 1, which every wave finished
    // reading before the barrier.
    //
    // A short last tile of an expert leaves some of a wave's 32-row
    // fragments without tile rows; such a wave runs a copy of the loop that
    // skips their MFMAs (same loads and barriers), so the tile costs MFMA
    // time in proportion to its rows.
    const int nfrag = min(FM, max(0, (tile_rows - wm * TM + 31) / 32));
    auto stream = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      auto mma_rows = [&](const bf16x8* pa, const bf16x8* pb) {
        if constexpr (FULL) {
          mma(pa, pb);
        } else {
#pragma unroll
          for (int x = 0; x < FM; ++x)
            if (x < nfrag)
#pragma unroll
              for (int y = 0; y < FN; ++y)
                acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[y], pa[x], acc[x][y],
                                                                   0, 0, 0);
        }
      };
      if constexpr (ASYM && SB >= 3) {
        // A(0), B(0) .. B(SB-2) ahead; iteration kt requests A(kt+1) then
        // B(kt+SB-1), so A(kt) has landed once at most the last group's B
        // loads are outstanding, and B(kt), requested before it, too
        issue_a(0);
#pragma unroll
        for (int t = 0; t + 1 < SB; ++t) issue_b(t);
      } else if constexpr (ASYM) {  // the same with A and B exchanged
        issue_b(0);
        issue_a(0);
        issue_a(1);
      } else {
#pragma unroll
        for (int t = 0; t + 1 < S; ++t) issue(t);
      }
      for (int kt = 0; kt < nk; ++kt) {
        if constexpr (ASYM && SB >= 3) {
          wait_vmcnt<QB>();
          wg_barrier();
          issue_a(kt + 1);
          issue_b(kt + SB - 1);
        } else if constexpr (ASYM) {
          wait_vmcnt<QA>();
          wg_barrier();
          issue_b(kt + 1);
          issue_a(kt + 2);
        } else {
          wait_vmcnt<(S - 2) * LPW>();
          wg_barrier();
          issue(kt + S - 1);
        }
        read_frags(kt, 0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 1 < KK) read_frags(kt, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
          mma_rows(fa[kk & 1], fb[kk & 1]);
          if (kk == 0) {
            __builtin_amdgcn_sched_group_barrier(0x0020, LPW, 0);  // VMEM (DMA)
            __builtin_amdgcn_sched_group_barrier(0x0100, NFR, 0);  // first reads
          }
          if (kk + 1 < KK) interleave();
          else __builtin_amdgcn_sched_group_barrier(0x0008, NMF, 0);
        }
      }
    };
    if (nfrag == FM)
      stream(std::true_type{});
    else
      stream(std::false_type{});
  } else {
  #pragma unroll
    for (int t = 0; t <= D; ++t) issue(t);
    wait_vmcnt<D * LPW>();
    wg_barrier();
    read_frags(0, 0, fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      // sub-slices 0 .. KK-2 of slice kt (fragment set kk & 1)
  #pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
        read_frags(kt, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        mma(fa[kk & 1], fb[kk & 1]);
        interleave();
      }
      wait_vmcnt<(D - 1) * LPW>();
      wg_barrier();
      // last sub-slice of kt, reading slice kt+1's first fragments and
      // requesting slice kt+1+D meanwhile (on the last slice those reads
      // fetch stale data that nobody uses)
      read_frags_dma(kt + 1, 0, fa[KK & 1], fb[KK & 1], kt + 1 + D);
      mma(fa[(KK - 1) & 1], fb[(KK - 1) & 1]);
      interleave();
      if (KK & 1) {  // keep set 0 as "current" at the top of the loop
  #pragma unroll
        for (int x = 0; x < FM; ++x) fa[0][x] = fa[1][x];
  #pragma unroll
        for (int y = 0; y < FN; ++y) fb[0][y] = fb[1][y];
      }
    }
  }
  wait_vmcnt<0>();  // no DMA write may land after the workgroup ends

  const int fr = lane & 31;
  if constexpr (MIX) {  // h columns 8*(r/4) + 4*fhalf + r%4 of the wave's 16
#pragma unroll
    for (int x = 0; x < FM; ++x) {
      const int row = wm * TM + x * 32 + fr;
      const size_t orow = static_cast<size_t>(row0 + m0 + row) * a.NC;
      const int c0 = nt * (BN / 2) + wn * 16;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = silu(acc[x][0][4 * q + i]) * acc[x][0][4 * q + i + 8];
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        if (m0 + row < Mj)
          *reinterpret_cast<uint2*>(&a.out[orow + c0 + 8 * q + 4 * fhalf]) = pk;
      }
    }
    return;
  }
  constexpr int OUT_FN = MODE == GATEUP ? FN / 2 : FN;
  if constexpr (MODE == GATEUP) {
    // gate-up: 128 h columns per tile row; each lane stores its 4-column
    // groups directly (8-byte stores), which measured slightly faster than
    // staging these narrow rows through LDS
#pragma unroll
    for (int x = 0; x < FM; ++x) {
      const int row = wm * TM + x * 32 + fr;
      const bool live = m0 + row < Mj;
      const size_t orow = static_cast<size_t>(row0 + m0 + row) * a.NC;
#pragma unroll
      for (int y = 0; y < OUT_FN; ++y) {
        const int c0 = nt * (BN / 2) + wn * (TN / 2) + y * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = silu(acc[x][y][4 * q + i]) * acc[x][y + FN / 2][4 * q + i];
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          if (live)
            *reinterpret_cast<uint2*>(&a.out[orow + c0 + 8 * q + 4 * fhalf]) = pk;
        }
      }
    }
  } else {
    // down: the output tile is staged through LDS (the ring is free once
    // every wave has passed the barrier): each lane writes its 4-column groups
    // of bf16 results into a [BM][OUTC] tile whose row pitch is padded by 16
    // bytes (rows start 16 banks apart), then the workgroup stores whole tile
    // rows with 16-byte vector stores, consecutive lanes on consecutive
    // addresses.
    constexpr int OUTC = BN;  // output columns of the tile
    constexpr int PITCH = OUTC * 2 + 16;  // bytes per LDS row
    __syncthreads();
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) u32x2 lds_u2;
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    typedef __attribute__((address_space(3))) unsigned char lds_wbyte;
    lds_wbyte* ot = (lds_wbyte*)(smem);
#pragma unroll
    for (int x = 0; x < FM; ++x) {
      const int row = wm * TM + x * 32 + fr;
#pragma unroll
      for (int y = 0; y < OUT_FN; ++y) {
        const int c0 = wn * TN + y * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * q + i;
            v[i] = acc[x][y][r];
          }
          u32x2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *(lds_u2*)(ot + row * PITCH + (c0 + 8 * q + 4 * fhalf) * 2) = pk;
        }
      }
    }
    __syncthreads();
    constexpr int CH = OUTC / 8;  // 16-byte chunks per tile row
    const int col0 = nt * BN;
    const int rows = min(BM, Mj - m0);
    for (int i = tid; i < rows * CH; i += NTH) {
      const int r = i / CH, c = i % CH;
      const u32x4 v = *(lds_u4*)(ot + r * PITCH + c * 16);
      *reinterpret_cast<u32x4*>(
          &a.out[static_cast<size_t>(row0 + m0 + r) * a.NC + col0 + c * 8]) = v;
    }
  }
}

// Tile search (BM-row tiles) into scalar registers; false for surplus
// workgroups.  cum: LDS [N + 1].
template <int BM>
__device__ __forceinline__ bool find_tile_s(const Args& a, int* cum, int& j, int& m0, int& nt,
                                            int& Mj, int& row0, int* total = nullptr) {
  if (a.N < 64 * REG_CHUNKS) {  // registers only, every wave on its own
    TileRegs tr;
    tile_regs<BM>(a, tr);
    if (total) *total = tr.total;
    const int p = blockIdx.x;
    const int q = (tr.total + 7) / 8;  // tiles per XCD, as find_tile
    const int L = (p % 8) * q + p / 8;
    if (p / 8 >= q || L >= tr.total) return false;
    locate_regs<BM>(a, tr, L, j, m0, nt, Mj, row0);
    j = __builtin_amdgcn_readfirstlane(j);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    nt = __builtin_amdgcn_readfirstlane(nt);
    Mj = __builtin_amdgcn_readfirstlane(Mj);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    return true;
  }
  const bool live = find_tile<BM>(a, cum, j, m0, nt, Mj, row0);
  if (total) *total = cum[a.N + 1];
  // cum lives at the start of the ring, which the first loads overwrite:
  // every wave must be done with the search first (surplus workgroups
  // return together, all their waves having found no tile)
  __syncthreads();
  if (!live) return false;
  j = __builtin_amdgcn_readfirstlane(j);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  nt = __builtin_amdgcn_readfirstlane(nt);
  Mj = __builtin_amdgcn_readfirstlane(Mj);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  return true;
}

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int SB = S>
__device__ __forceinline__ void gemm_tile(const Args& a, unsigned char* smem, int* cum) {
  int j, m0, nt, Mj, row0;
  if (find_tile_s<BM>(a, cum, j, m0, nt, Mj, row0))
    gemm_body<MODE, BM, BN, BK, WM, WN, S, SB>(a, smem, j, m0, nt, Mj, row0);
}

// WM x WN waves per workgroup; WPE workgroups per CU; S stages of A and SB
// of B.
template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WPE, int SB>
__global__ __launch_bounds__(WM * WN * MOE_WAVE)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, WPE * WM * WN / 4)))
void gemm_dma_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  // the tile search table shares the dynamic block with the ring, so the
  // kernel has no static LDS and workgroups pack the CU's 160 KB exactly
  gemm_tile<MODE, BM, BN, BK, WM, WN, S, SB>(a, smem, reinterpret_cast<int*>(smem));
}

// ------------------------------------------------ persistent prefill down
// One workgroup per CU walks a fixed list of 256 x 256 tiles, and the ring
// runs on across tile boundaries: slice g of the workgroup's whole sequence
// (tile g / nk, K slice g % nk) lands in A stage g % SA and B stage g % SB,
// the token rows one slice ahead and the weights two, whatever tile they
// belong to.  The next tile's first slices are therefore in flight while
// the current tile's last slices are multiplied and its results stored,
// where a workgroup per tile pays a launch slot, the ring fill and the
// output store back to back.  The down reduction (K = I, e.g. 12 slices of
// 64 for I = 768) is short enough for that to matter.
//
// Tiles: the table of find_tile (experts' row tiles times column tiles), XCD
// x owning the contiguous range [x q, x q + q), q = ceil(total / 8); slot s
// of an XCD (workgroup p = 8 s + x) takes tiles x q + s, x q + s + G / 8,
// ..., so tiles of one expert run side by side on one XCD and share its L2.
// The grid G is a multiple of 8; every (slot, XCD) pair is one workgroup,
// so the lists partition the tiles.
//
// Output: when a tile's last slice has been multiplied, the A and B stages
// of that slice are free until the next iteration requests into them (the
// requests in flight target the other stages).  The tile leaves through
// them in two halves of 128 rows: the waves of that half write their bf16
// results (rows 0-63 of the half in the A stage, 64-127 in the B stage, 16-
// byte chunks XOR-swizzled by row), then every wave stores whole rows with
// 16-byte stores through a buffer resource over the tile's rows, so rows
// past the tile's end are dropped without a branch and every lane issues
// exactly NST stores per tile.  The wait after a tile's stores counts them:
// A(g + 1), issued before B(g + SB - 1) and the stores, has landed once at
// most QB + NST of the wave's vector-memory instructions are outstanding
// (gfx9 retires vector loads and stores in issue order).  Spreading the
// output over whole 512-byte rows matters: every CU reaches a tile's end at
// about the same time, and per-lane 8-byte stores of the MFMA layout (32
// rows per instruction) made the stores alone cost about a quarter of the
// kernel.
template <int BM, int BN, int BK, int WM, int WN, int SA, int SB>
__global__ __launch_bounds__(WM * WN * MOE_WAVE)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void gemm_persist_down_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int W = WM * WN;
  static_assert(W == 4 || W == 8, "4 or 8 waves");
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int CPR = BK / 8;
  constexpr int SWZ = CPR - 1;
  constexpr int SWS = BK == 64 ? 1 : (BK == 32 ? 2 : 0);
  constexpr int RPJ = MOE_WAVE / CPR;
  constexpr int NA = BM / RPJ, NB = BN / RPJ;
  static_assert(NA % W == 0 && NB % W == 0, "split over the waves");
  constexpr int QA = NA / W, QB = NB / W, LPW = QA + QB;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  constexpr int B_BASE = SA * A_BYTES;
  static_assert(SA == 2 && SB >= 3, "token rows one slice ahead, weights two or more");
  constexpr int NTH = W * MOE_WAVE;
  constexpr int NST = 2 * (BM / 2) * BN * 2 / (NTH * 16);  // 16-byte stores per lane per tile
  static_assert(QB + NST < 64, "vmcnt range");
  static_assert(BM == 256 && BN == 256 && BK == 64 && WM == 2 && A_BYTES == 32768 &&
                    B_BYTES == 32768,
                "output staging: half a tile (128 rows) in one free A and one free B stage");
  constexpr int KK = BK / 16;
  constexpr int NFR = FM + FN, NMF = FM * FN;

  TileRegs tr;
  tile_regs<BM>(a, tr);
  const int total = tr.total;
  const int p = blockIdx.x, nslot = gridDim.x / 8;
  const int q = (total + 7) / 8;
  const int lo = (p % 8) * q, hi = min(lo + q, total);
  const int first = lo + p / 8;
  if (first >= hi) return;
  const int ntile = (hi - first + nslot - 1) / nslot;
  const int nk = a.K / BK;

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int wm = wave / WN, wn = wave % WN;
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2;
  const int lrow = lane / CPR, lslot = lane % CPR;

  struct Tile {
    int j, m0, nt, Mj, row0;
  };
  auto tile_at = [&](int n, Tile& t) {
    locate_regs<BM>(a, tr, first + n * nslot, t.j, t.m0, t.nt, t.Mj, t.row0);
    t.j = __builtin_amdgcn_readfirstlane(t.j);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.nt = __builtin_amdgcn_readfirstlane(t.nt);
    t.Mj = __builtin_amdgcn_readfirstlane(t.Mj);
    t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  };

  // A: the tile's own rows of h; the per-lane offsets do not depend on the
  // tile (rows past its end fall outside the resource and read as zeros).
  uint32_t va[QA];
#pragma unroll
  for (int d = 0; d < QA; ++d) {
    const int row = (wave * QA + d) * RPJ + lrow;
    va[d] = static_cast<uint32_t>(row) * row_bytes + (lslot ^ ((row >> SWS) & SWZ)) * 16;
  }
  // B: rows of the tile's column block of w2.
  uint32_t vb[QB];
  i32x4 rsrc_a, rsrc_b;
  auto set_a = [&](const Tile& t) {
    rsrc_a = buffer_rsrc(a.a + static_cast<size_t>(t.row0 + t.m0) * a.K,
                         static_cast<uint32_t>(min(BM, t.Mj - t.m0)) * row_bytes);
  };
  auto set_b = [&](const Tile& t) {
    rsrc_b = buffer_rsrc(a.w + static_cast<size_t>(t.j) * a.w_stride,
                         static_cast<uint32_t>(a.w_stride) * 2);
#pragma unroll
    for (int d = 0; d < QB; ++d) {
      const int row = (wave * QB + d) * RPJ + lrow;
      vb[d] = weight_off<DOWN>(a, t.nt * BN + row, (lslot ^ ((row >> SWS) & SWZ)) * 8);
    }
  };
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));

  // Issue cursors: tile ordinal and K slice of the next A and B requests.
  // Past the last slice they stay on it, so the surplus requests at the end
  // re-fetch it into stages that are never read again and every iteration
  // issues the same number of loads.
  int na = 0, ka = 0, nb = 0, kb = 0;
  {
    Tile t0;
    tile_at(0, t0);
    set_a(t0);
    set_b(t0);
  }
  auto issue_a = [&](int g) {
#pragma unroll
    for (int d = 0; d < QA; ++d)
      lds_dma16(rsrc_a, va[d], static_cast<uint32_t>(ka * BK) * 2,
                lds_base + (g % SA) * A_BYTES + (wave * QA + d) * 1024);
  };
  auto issue_b = [&](int g) {
#pragma unroll
    for (int d = 0; d < QB; ++d)
      lds_dma16(rsrc_b, vb[d], weight_k0(a, static_cast<uint32_t>(kb * BK)),
                lds_base + B_BASE + (g % SB) * B_BYTES + (wave * QB + d) * 1024);
  };
  auto next_a = [&]() {
    if (++ka == nk) {
      if (na + 1 < ntile) {
        ka = 0;
        Tile t;
        tile_at(++na, t);
        set_a(t);
      } else {
        ka = nk - 1;
      }
    }
  };
  auto next_b = [&]() {
    if (++kb == nk) {
      if (nb + 1 < ntile) {
        kb = 0;
        Tile t;
        tile_at(++nb, t);
        set_b(t);
      } else {
        kb = nk - 1;
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int y = 0; y < FN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int frow = lane & 31, fhalf = lane >> 5;
  const int a_lane = (wm * TM + frow) * BK;
  const int b_lane = (wn * TN + frow) * BK;
  typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) const unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](int g, int kk, bf16x8* pa, bf16x8* pb) {
    lds_byte* A_ = lds0 + (g % SA) * A_BYTES;
    lds_byte* B_ = lds0 + B_BASE + (g % SB) * B_BYTES;
    const int sw = ((kk * 2 + fhalf) ^ ((frow >> SWS) & SWZ)) << 4;
#pragma unroll
    for (int x = 0; x < FM; ++x) pa[x] = *(lds_frag*)(A_ + (a_lane + x * 32 * BK) * 2 + sw);
#pragma unroll
    for (int y = 0; y < FN; ++y) pb[y] = *(lds_frag*)(B_ + (b_lane + y * 32 * BK) * 2 + sw);
  };

  int nfrag = FM;  // fragments of this wave with tile rows

  // One slice: the A and B requests of later slices, then the MFMAs of
  // slice g (all fragments, or only those with tile rows).
  auto slice = [&](int g, auto full) {
    constexpr bool FULL = decltype(full)::value;
    issue_a(g + 1);
    issue_b(g + SB - 1);
    read_frags(g, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) read_frags(g, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
      for (int x = 0; x < FM; ++x)
        if (FULL || x < nfrag)
#pragma unroll
          for (int y = 0; y < FN; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][y], fa[kk & 1][x],
                                                               acc[x][y], 0, 0, 0);
      if constexpr (FULL) {
        if (kk == 0) {
          __builtin_amdgcn_sched_group_barrier(0x0020, LPW, 0);  // VMEM (DMA)
          __builtin_amdgcn_sched_group_barrier(0x0100, NFR, 0);  // first reads
        }
        if (kk + 1 < KK) interleave_groups<NMF, NFR>();
        else __builtin_amdgcn_sched_group_barrier(0x0008, NMF, 0);
      }
    }
  };

  // prologue: A(0), B(0) .. B(SB - 2)
  issue_a(0);
  next_a();
#pragma unroll
  for (int t = 0; t + 1 < SB; ++t) {
    issue_b(t);
    next_b();
  }
  const int fr = lane & 31;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) u32x2 lds_u2;
  typedef __attribute__((address_space(3))) const u32x4_t lds_u4r;
  typedef __attribute__((address_space(3))) unsigned char lds_wbyte;
  int g = 0;  // slice of the whole sequence
  for (int nc = 0; nc < ntile; ++nc) {
    Tile tc;
    tile_at(nc, tc);
    const int rows = min(BM, tc.Mj - tc.m0);
    nfrag = min(FM, max(0, (rows - wm * TM + 31) / 32));
    // the K loop of one tile, all fragments or only those with tile rows
    auto run = [&](auto full) {
      for (int kc = 0; kc < nk; ++kc, ++g) {
        // A(g) was issued before the newest QB requests (B(g + SB - 2))
        // and, in a tile's first slice, the previous tile's NST stores;
        // B(g) before A(g)
        if (kc == 0 && nc > 0) wait_vmcnt<QB + NST>();
        else wait_vmcnt<QB>();
        wg_barrier();
        slice(g, full);
        next_a();
        next_b();
      }
    };
    if (nfrag == FM) run(std::true_type{});
    else run(std::false_type{});
    // the tile's results through the stages of its last slice, g - 1
    const __amdgpu_buffer_rsrc_t rsrc_o =
        store_rsrc(a.out + static_cast<size_t>(tc.row0 + tc.m0) * a.NC + tc.nt * BN,
                   static_cast<uint32_t>(rows) * static_cast<uint32_t>(a.NC) * 2);
    lds_wbyte* st0 = (lds_wbyte*)(smem) + ((g - 1) % SA) * A_BYTES;
    lds_wbyte* st1 = (lds_wbyte*)(smem) + B_BASE + ((g - 1) % SB) * B_BYTES;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      wg_barrier();  // slice g - 1's fragments, or the previous half, consumed
      if (wm == half) {
#pragma unroll
        for (int x = 0; x < FM; ++x) {
          const int r = (x % 2) * 32 + fr;  // row in its stage
          lds_wbyte* st = x < 2 ? st0 : st1;
#pragma unroll
          for (int y = 0; y < FN; ++y)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int ch = wn * (TN / 8) + y * 4 + qq;  // 16-byte chunk of the row
              u32x2 pk;
              pk.x = pack_bf16x2(acc[x][y][4 * qq], acc[x][y][4 * qq + 1]);
              pk.y = pack_bf16x2(acc[x][y][4 * qq + 2], acc[x][y][4 * qq + 3]);
              *(lds_u2*)(st + r * (BN * 2) + ((ch ^ (r & 31)) << 4) + fhalf * 8) = pk;
            }
        }
      }
      // this wave's LDS writes done, then everyone's
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < NST / 2; ++i) {
        const int e = i * NTH + tid;           // 16-byte chunk of the half
        const int r = e / (BN / 8), ch = e % (BN / 8);
        lds_wbyte* st = r < 64 ? st0 : st1;
        const int rr = r % 64;
        const u32x4_t v = *(lds_u4r*)(st + rr * (BN * 2) + ((ch ^ (rr & 31)) << 4));
        buf_store16(rsrc_o,
                    static_cast<uint32_t>(half * 128 + r) * static_cast<uint32_t>(a.NC) * 2 +
                        ch * 16,
                    v);
      }
    }
#pragma unroll
    for (int x = 0; x < FM; ++x)
#pragma unroll
      for (int y = 0; y < FN; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;
  }
  wait_vmcnt<0>();  // no DMA write may land after the workgroup ends
}

// Decode gate-up with the tile height chosen on the device: tiles of BMA
// token rows (SA token-row stages, SAB weight stages) when they number at
// most a.dual_limit, i.e. when every tile gets a workgroup slot at once,
// else tiles of BMB rows (SB and SBB stages).  Every workgroup reads the
// same offsets, so all take the same branch; the grid covers the larger
// tile count.
template <int MODE, int BN, int BK, int BMA, int SA, int SAB, int BMB, int SB, int SBB,
          int WPE>
__global__ __launch_bounds__(4 * MOE_WAVE)
__attribute__((amdgpu_waves_per_eu(1, WPE)))
void gemm_dual_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* cum = reinterpret_cast<int*>(smem);  // [N + 2], then the tile count
  int* s_stat = cum + a.N + 2;               // tiles of BMA rows, most rows
  if (threadIdx.x < MOE_WAVE) {
    int acc = 0, mx = 0;
    for (int j0 = 0; j0 < a.N; j0 += MOE_WAVE) {
      const int e = j0 + lane_id();
      const int m = e < a.N ? a.offsets[e + 1] - a.offsets[e] : 0;
      acc += wave_sum((m + BMA - 1) / BMA);
      mx = max(mx, wave_max(m));
    }
    if (threadIdx.x == 0) {
      s_stat[0] = acc * a.n_tiles;
      s_stat[1] = mx;
    }
  }
  __syncthreads();
  const bool one_wave = s_stat[0] <= a.dual_limit;
  const int most_rows = s_stat[1];
  __syncthreads();  // the tile search below rewrites the table
  if (one_wave) {
    // One tile per expert and weight panel.  When no expert has more than
    // 32 (64) rows, every tile runs with a 32 (64)-row A block, which
    // leaves LDS for more ring stages: more weight bytes in flight for the
    // same weight stream.  (Deepening only the small tiles of a launch that
    // also has large ones made the large ones finish later.)
    constexpr int RING = (SA * BMA + SAB * BN) * BK * 2;  // the LDS of the launch
    if constexpr (SA == SAB) {
      constexpr int S32 = RING / ((32 + BN) * BK * 2), S64 = RING / ((64 + BN) * BK * 2);
      if constexpr (BMA > 64 && S32 > SA && S64 >= SA) {
        if (most_rows <= 32) {
          gemm_tile<MODE, 32, BN, BK, 1, 4, (S32 < 8 ? S32 : 8)>(a, smem, cum);
          return;
        }
        if (most_rows <= 64) {
          gemm_tile<MODE, 64, BN, BK, 1, 4, (S64 < 8 ? S64 : 8)>(a, smem, cum);
          return;
        }
      }
    } else {
      // the same with 2 token-row stages and the rest of the ring as weights
      constexpr int B32 = (RING - 2 * 32 * BK * 2) / (BN * BK * 2);
      constexpr int B64 = (RING - 2 * 64 * BK * 2) / (BN * BK * 2);
      if constexpr (BMA > 64 && B64 > SAB) {
        if (most_rows <= 32) {
          gemm_tile<MODE, 32, BN, BK, 1, 4, 2, (B32 < 8 ? B32 : 8)>(a, smem, cum);
          return;
        }
        if (most_rows <= 64) {
          gemm_tile<MODE, 64, BN, BK, 1, 4, 2, (B64 < 8 ? B64 : 8)>(a, smem, cum);
          return;
        }
      }
    }
    gemm_tile<MODE, BMA, BN, BK, 1, 4, SA, SAB>(a, smem, cum);
  } else {
    gemm_tile<MODE, BMB, BN, BK, 1, 4, SB, SBB>(a, smem, cum);
  }
}

// Small-batch decode: with a handful of active experts, tiles of 128 weight
// rows give only a few hundred workgroups, and each streams its panel at the
// rate of one CU.  This kernel streams panels of 16 weight rows instead, for
// token tiles of 16 rows (the 16 x 16 x 32 MFMA): eight times the
// workgroups for the same bytes, each over the whole reduction, several per
// CU with a shallow ring.  The 4 waves split each 128-wide K slice: wave w
// runs the MFMA of K sub-step w into its own accumulator and loads rows
// [4 w, 4 w + 4) of both operands, and the four partial accumulators are
// added in LDS in wave order before the epilogue.
//
// Gate-up panel row p is gate column 2 * (p / 4) + p % 4 of the panel when
// p % 4 < 2, else the up row of column 2 * (p / 4) + p % 4 - 2, so each
// lane's four accumulator rows (panel rows 4 * (lane / 16) + i) hold two
// gate rows and their up rows.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int MODE, int S>
__global__ __launch_bounds__(4 * MOE_WAVE) void gemm_skinny_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int BM = 16, BN = 16, BK = 128;
  constexpr int SLICE_A = BM * BK * 2, SLICE_B = BN * BK * 2;  // 4 KB each
  constexpr int STAGE = SLICE_A + SLICE_B;
  static_assert(S >= 2 && S * STAGE >= 4 * MOE_WAVE * 4 * 4, "LDS for the partials");
  int j, m0, nt, Mj, row0;
  if (!find_tile_s<BM>(a, reinterpret_cast<int*>(smem), j, m0, nt, Mj, row0)) return;

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int K = a.K;
  const uint32_t row_bytes = static_cast<uint32_t>(K) * 2;
  const int tile_rows = min(BM, Mj - m0);
  const i32x4 rsrc_a =
      MODE == GATEUP ? buffer_rsrc(a.a, static_cast<uint32_t>(a.a_rows) * row_bytes)
                     : buffer_rsrc(a.a + static_cast<size_t>(row0 + m0) * K,
                                   static_cast<uint32_t>(tile_rows) * row_bytes);
  const i32x4 rsrc_b = buffer_rsrc(a.w + static_cast<size_t>(j) * a.w_stride,
                                   static_cast<uint32_t>(a.w_stride) * 2);
  // wave w fills rows [4 w, 4 w + 4) of both operands (one load each: 4
  // rows of 256 bytes); the lane filling LDS slot s of row r fetches chunk
  // s ^ r
  const int row = wave * 4 + lane / 16, ch = (lane % 16) ^ row;
  uint32_t va, vb;
  if (MODE == GATEUP)
    va = row < tile_rows
             ? static_cast<uint32_t>(a.row_token[row0 + m0 + row]) * row_bytes + ch * 16
             : OOB_OFF;
  else
    va = static_cast<uint32_t>(row) * row_bytes + ch * 16;  // past the tile: outside
  {
    uint32_t wrow;
    if (MODE == GATEUP) {
      const int c = nt * 8 + 2 * (row / 4) + row % 2;
      wrow = row % 4 < 2 ? c : a.I + c;
    } else {
      wrow = nt * BN + row;
    }
    vb = weight_off<MODE>(a, wrow, ch * 8);
  }
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)(smem))));
  const int nk = K / BK;
  auto issue = [&](int s) {
    const uint32_t ke = static_cast<uint32_t>(min(s, nk - 1) * BK);
    const uint32_t st = lds_base + (s % S) * STAGE + wave * 1024;
    lds_dma16(rsrc_a, va, ke * 2, st);
    lds_dma16(rsrc_b, vb, weight_k0(a, ke), st + SLICE_A);
  };
  typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
  typedef __attribute__((address_space(3))) const unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  const int frow = lane % 16;
  const int sw = ((wave * 4 + lane / 16) ^ frow) << 4;  // K sub-step = wave
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 + 1 < S; ++s0) issue(s0);
  for (int s0 = 0; s0 < nk; ++s0) {
    wait_vmcnt<(S - 2) * 2>();
    wg_barrier();
    issue(s0 + S - 1);
    lds_byte* st = lds0 + (s0 % S) * STAGE;
    const bf16x8 fa = *(lds_frag*)(st + frow * (BK * 2) + sw);
    const bf16x8 fb = *(lds_frag*)(st + SLICE_A + frow * (BK * 2) + sw);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa, acc, 0, 0, 0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [wave][lane][4]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * MOE_WAVE + lane) * 4 + r] = acc[r];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = red[lane * 4 + r];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[(w * MOE_WAVE + lane) * 4 + r];
    acc[r] = v;
  }
  // lane holds token row lane % 16 and panel rows 4 * (lane / 16) + r
  const bool live = m0 + frow < Mj;
  const size_t orow = static_cast<size_t>(row0 + m0 + frow) * a.NC;
  const int g4 = lane / 16;
  if constexpr (MODE == GATEUP) {
    const uint32_t pk = pack_bf16x2(silu(acc[0]) * acc[2], silu(acc[1]) * acc[3]);
    if (live) *reinterpret_cast<uint32_t*>(&a.out[orow + nt * 8 + 2 * g4]) = pk;
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(acc[0], acc[1]);
    pk.y = pack_bf16x2(acc[2], acc[3]);
    if (live) *reinterpret_cast<uint2*>(&a.out[orow + nt * BN + 4 * g4]) = pk;
  }
}

// ------------------------------------------- decode GEMV on packed panels
// With a few token rows per active expert (a decode batch of a few tokens)
// the product is a matrix-vector product per expert: the weight bytes are
// everything and a 32 x 32 MFMA tile would be mostly empty.  In the panel
// layout a 32-row group of a 64-wide K slice is 4 KB of contiguous bytes,
// four 1 KB loads of one wave (lane l: row l % 32, elements 8 (l / 32) ..
// +7 of each 16-wide K step), so a wave that owns a row group streams long
// contiguous runs, and holds every load of its share in registers at once.
//
// Workgroup: one (expert, chunk of up to MR token rows, 32-row group); its
// 4 waves split the K slices into quarters.  The token operand is staged in
// LDS: for gate-up every token of the batch (at most GEMV_MAX_T, so that no
// load waits for row_token), for down the tile's rows of h.  Its loads are
// issued first and the weight loads right after; the workgroup waits for
// the token rows only, so it crosses the barrier with every weight load in
// flight and the multiply of a K slice waits for that slice alone.  Each
// lane accumulates, per token row, its row's dot product over its half of
// every K step in fp32 (v_dot2 on bf16 pairs); the two halves are added
// across lanes l and l + 32, the four quarters in LDS in wave order, and
// wave 0 writes the outputs: for gate-up the group's 16 gate rows and 16 up
// rows give 16 h columns (silu(gate) * up), for down 32 output columns.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
constexpr int GEMV_MAX_K = 2048;  // K <= 2048: a wave's K slices fit its registers
constexpr int GEMV_MAX_T = 8;     // gate-up: tokens staged whole

// 8 bf16 products added to acc in element order (pairs by v_dot2).  The
// words are copied out of the vectors first: a bit cast of a subscripted
// vector element compiles to a read of element 0.
__device__ __forceinline__ float dot8(const u32x4 w, const u32x4 x, float acc) {
  const uint32_t wa[4] = {w.x, w.y, w.z, w.w}, xa[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, wa[i]),
                                          __builtin_bit_cast(bf16x2v, xa[i]), acc, false);
  return acc;
}

// NBW = K / 256: the K slices of one wave (a compile-time count, so that
// the compiler's wait for the token rows leaves every weight load alone).
template <int MODE, int MR, int NBW, bool COMB = false>
__global__ __launch_bounds__(4 * MOE_WAVE) void gemv_kernel(Args a, Comb c) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int XR = MODE == GATEUP ? GEMV_MAX_T : MR;  // staged token rows
  const int K = a.K;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  unsigned char* xs = smem;                                                       // [XR][K] bf16
  float* red = reinterpret_cast<float*>(smem + static_cast<size_t>(XR) * K * 2);  // [4][MR][32]
  int* cum = reinterpret_cast<int*>(red + 4 * MR * 32);                          // [N + 2]
  int j, m0, gi, Mj, row0, total;
  if (!find_tile_s<MR>(a, cum, j, m0, gi, Mj, row0, &total)) {
    // every slot dropped: no workgroup has a tile, and y is zero
    if constexpr (COMB)
      if (total == 0 && static_cast<int>(blockIdx.x) < a.n_tiles && tid < 64)
        for (int t = tid / 32; t < c.T; t += 2)
          c.y[static_cast<size_t>(t) * a.NC + blockIdx.x * 32 + tid % 32] = 0;
    return;
  }
  const int rows = min(MR, Mj - m0);
  const int nstage = MODE == GATEUP ? a.a_rows : rows;
  // combine: the slots' rows and gates (at most 64 slots, one per lane),
  // requested before the weight stream and used after it
  int slot_r = 0;
  float slot_g = 0.f;
  if constexpr (COMB) {
    const int q = min(lane, c.T * c.k - 1);
    slot_r = c.slot_row[q];
    slot_g = c.gates[q];
  }

  // token rows: thread i stages 16-byte chunk i of every row (K <= 2048:
  // at most 256 chunks a row; clamped loads, the extra ones unused)
  const int cpr = K / 8;  // chunks per row
  const int ch = min(tid, cpr - 1);
  u32x4 xv[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int rr = min(r, nstage - 1);
    const int src = MODE == GATEUP ? rr : row0 + m0 + rr;
    xv[r] = *reinterpret_cast<const u32x4*>(a.a + static_cast<size_t>(src) * K + ch * 8);
  }
  // this wave's K slices
  const int nb = 4 * NBW, b0 = wave * NBW;
  const unsigned char* wb =
      reinterpret_cast<const unsigned char*>(a.w + static_cast<size_t>(j) * a.w_stride) +
      (static_cast<size_t>(gi / 4) * nb + b0) * PANEL_BLOCK + ((gi % 4) * 4 * 64 + lane) * 16;
  u32x4 wv[NBW][4];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      wv[i][kk] = *reinterpret_cast<const u32x4*>(wb + static_cast<size_t>(i) * PANEL_BLOCK + kk * 1024);
  __builtin_amdgcn_sched_barrier(0);  // keep every weight request ahead of the waits
  // gate-up: the staged row of each tile row (scalar loads)
  int xrow[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r)
    xrow[r] = MODE == GATEUP ? min(max(a.row_token[row0 + m0 + min(r, rows - 1)], 0), nstage - 1)
                             : r;
#pragma unroll
  for (int r = 0; r < XR; ++r)
    if (r < nstage && tid < cpr)
      *reinterpret_cast<u32x4*>(xs + (static_cast<size_t>(r) * cpr + tid) * 16) = xv[r];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this thread's LDS stores (lgkmcnt 0)
  wg_barrier();                        // the weight loads stay in flight

  typedef __attribute__((address_space(3))) const u32x4 lds_u4;
  typedef __attribute__((address_space(3))) const unsigned char lds_b;
  const int half = lane / 32;
  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int kb = (b0 + i) * 64 + half * 8;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < MR; ++r)
        if (r < rows) {
          const u32x4 x = *(lds_u4*)((lds_b*)(xs) + (static_cast<size_t>(xrow[r]) * K + kb + kk * 16) * 2);
          acc[r] = dot8(wv[i][kk], x, acc[r]);
        }
  }
  // halves (lanes l, l + 32), then the quarters in wave order
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] += __shfl_xor(acc[r], 32);
  if (lane < 32)
#pragma unroll
    for (int r = 0; r < MR; ++r) red[(wave * MR + r) * 32 + lane] = acc[r];
  __syncthreads();
  if (wave != 0) return;
  const int t = lane % 32;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (r >= rows) break;
    float v = red[r * 32 + t];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[(w * MR + r) * 32 + t];
    const size_t orow = static_cast<size_t>(row0 + m0 + r) * a.NC;
    if constexpr (MODE == GATEUP) {
      // tile rows 0..15 of the group: gate of h columns 64 P + 16 G + t, 16..31: up
      const float up = __shfl(v, (lane & 15) + 16);
      if (lane < 16) {
        const uint32_t hv = pack_bf16x2(silu(v) * up, 0.f);
        a.out[orow + (gi / 4) * 64 + (gi % 4) * 16 + lane] = static_cast<uint16_t>(hv);
      }
    } else if (lane < 32) {
      const uint16_t o = static_cast<uint16_t>(pack_bf16x2(v, 0.f));
      if constexpr (COMB)  // written through to the device-coherent level
        __hip_atomic_store(&a.out[orow + gi * 32 + lane], o, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        a.out[orow + gi * 32 + lane] = o;
    }
  }
  if constexpr (COMB) {
    // The last of the workgroups that write output columns 32 gi .. +31
    // (one per expert tile; an arrival ticket that wraps back to zero)
    // combines those columns of every token: y[t] = sum over the kept slots,
    // in slot order, of gate * out_rows[row], fp32 fused multiply-adds from
    // zero, rounded to bf16 to nearest even -- the arithmetic of moe_combine.
    // The rows travel as device-scope atomic stores and loads, which the L2
    // of each XCD keeps coherent by themselves; the ticket is taken once
    // this wave's stores have completed (vmcnt 0) and the loads are issued
    // after its value has returned, so no L2 writeback or invalidation (a
    // device-scope fence) is needed in any of the workgroups.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the row stores are done
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const unsigned live = static_cast<unsigned>(total / a.n_tiles);
    unsigned prev = 0;
    if (lane == 0) prev = atomicInc(c.ticket + gi, live - 1);
    if (__builtin_amdgcn_readfirstlane(prev) != live - 1) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int col = gi * 32 + lane % 32;
    for (int t0 = 0; t0 < c.T; t0 += 2) {
      const int t = min(t0 + lane / 32, c.T - 1);
      float acc = 0.f;
      for (int s0 = 0; s0 < c.k; s0 += 8) {
        // the shuffles run in every lane: a lane reads the slot data of
        // its own token from lanes that hold it, which must be active
        int r[8];
        float g[8];
        uint32_t q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int src = t * c.k + min(s0 + u, c.k - 1);
          r[u] = __shfl(slot_r, src);
          g[u] = __shfl(slot_g, src);
          q[u] = __hip_atomic_load(&a.out[static_cast<size_t>(max(r[u], 0)) * a.NC + col],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < c.k && r[u] >= 0) acc = __builtin_fmaf(g[u], __uint_as_float(q[u] << 16), acc);
      }
      uint32_t ua = __float_as_uint(acc);
      ua += 0x7fffu + ((ua >> 16) & 1u);
      if (t0 + lane / 32 < c.T) c.y[static_cast<size_t>(t) * a.NC + col] = static_cast<uint16_t>(ua >> 16);
    }
  }
}

// ----------------------------------------------- decode tiles on panels
// Decode batches are bound by the weight stream: each active expert's
// panel is read once, and the rate at which those bytes arrive is the rate
// of the layer.  With packed weights (the panel layout) each wave reads its
// 32 weight rows of a K slice as NPW x 4 contiguous 1 KB loads straight into
// its MFMA operand registers, L slices ahead of the slice it multiplies, so
// the weight requests of a workgroup stay in flight across its barriers.
// The token rows (x gathered by row_token for gate-up, h for down) are the
// small operand: each thread loads its share of the next slice into
// registers one slice ahead, and the workgroup stores it into a two-stage
// LDS ring (rows of 128 bytes, 16-byte chunks XOR-swizzled) that every wave
// reads its fragments from.  All loads are ordinary loads, so the compiler
// places every wait.
//
// Workgroup: 4 waves, BN = 128 NPW weight rows (NPW panels), BM token rows
// (32, 64 or 128, chosen on the device from the largest expert: one tile
// per expert and panel when it fits), wave w owning weight rows
// [32 w NPW, 32 (w+1) NPW) of the tile and every token row.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

template <int MODE, int BM, int NPW, int L>
__device__ __forceinline__ void stream_body(const Args& a, unsigned char* smem, int j, int m0,
                                            int nt, int Mj, int row0) {
  constexpr int BK = 64, BN = 128 * NPW, FM = BM / 32, S = L + 1;
  constexpr int CH = BM * BK * 2 / 16 / 256;  // 16-byte chunks of A per thread per slice
  static_assert(CH >= 1 && FM >= 1, "token-row tile of 32, 64 or 128");
  constexpr int A_STAGE = BM * BK * 2;
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
  const int K = a.K, nk = K / BK;
  const int tile_rows = min(BM, Mj - m0);

  // A: thread tid fills chunk c = idx % 8 of row idx / 8 of each stage,
  // idx = q * 256 + tid.  Rows past the tile load the tile's first row (so
  // that every load is issued by every lane and the compiler can count
  // them) and store zeros.
  const uint16_t* asrc[CH];
  uint32_t alds[CH];
  bool alive[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int idx = q * 256 + tid, row = idx / 8, c = idx % 8;
    alive[q] = row < tile_rows;
    const int rr = alive[q] ? row : 0;
    const size_t r = MODE == GATEUP ? static_cast<size_t>(a.row_token[row0 + m0 + rr])
                                    : static_cast<size_t>(row0 + m0 + rr);
    asrc[q] = a.a + r * K + c * 8;
    alds[q] = row * (BK * 2) + ((c ^ ((row >> 1) & 7)) << 4);
  }
  // B: fragment column f of this wave is tile-order rows t0 .. t0 + 31,
  // t0 = nt * BN + (wave * NPW + f) * 32: block row group G of panel P
  const unsigned char* wbase =
      reinterpret_cast<const unsigned char*>(a.w + static_cast<size_t>(j) * a.w_stride);
  const unsigned char* bsrc[NPW];
#pragma unroll
  for (int f = 0; f < NPW; ++f) {
    const uint32_t t0 = nt * BN + (wave * NPW + f) * 32;
    bsrc[f] = wbase + static_cast<size_t>(t0 / PANEL_ROWS) * (K / PANEL_K) * PANEL_BLOCK +
              ((t0 % PANEL_ROWS) / 32) * 4 * 1024 + lane * 16;
  }

  u32x4v breg[S][NPW][4];
  u32x4v areg[S][CH];
  auto load_b = [&](int kt, auto slot) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int f = 0; f < NPW; ++f)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        breg[SL][f][kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(
            bsrc[f] + static_cast<size_t>(kt) * PANEL_BLOCK + kk * 1024));
  };
  auto load_a = [&](int kt, auto slot) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int q = 0; q < CH; ++q)
      areg[SL][q] = *reinterpret_cast<const u32x4v*>(asrc[q] + kt * BK);
  };
  typedef __attribute__((address_space(3))) u32x4v lds_u4;
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  lds_byte* lds0 = (lds_byte*)(smem);
  auto store_a = [&](int kt, auto slot) {
    constexpr int SL = decltype(slot)::value;
    lds_byte* st = lds0 + (kt & 1) * A_STAGE;
#pragma unroll
    for (int q = 0; q < CH; ++q)
      *(lds_u4*)(st + alds[q]) = alive[q] ? areg[SL][q] : u32x4v{0u, 0u, 0u, 0u};
  };

  f32x16 acc[FM][NPW];
#pragma unroll
  for (int x = 0; x < FM; ++x)
#pragma unroll
    for (int f = 0; f < NPW; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][f][r] = 0.f;
  const int nfrag = min(FM, (tile_rows + 31) / 32);
  const int frow = lane & 31, fhalf = lane >> 5;
  auto mma_slice = [&](int kt, auto slot) {
    constexpr int SL = decltype(slot)::value;
    typedef __attribute__((address_space(3))) const bf16x8 lds_frag;
    const lds_byte* st = lds0 + (kt & 1) * A_STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int sw = ((kk * 2 + fhalf) ^ ((frow >> 1) & 7)) << 4;
      bf16x8 fa[FM];
#pragma unroll
      for (int x = 0; x < FM; ++x) fa[x] = *(lds_frag*)(st + (x * 32 + frow) * (BK * 2) + sw);
#pragma unroll
      for (int x = 0; x < FM; ++x)
        if (x < nfrag)
#pragma unroll
          for (int f = 0; f < NPW; ++f)
            acc[x][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, breg[SL][f][kk]), fa[x], acc[x][f], 0, 0, 0);
    }
  };

  // Both operands are requested L slices ahead, the token rows of a slice
  // just before its weights: a wait for the token rows of slice kt + 1
  // (in-order completion) then leaves the weights of slices kt + 1 ..
  // kt + L in flight.  Prologue: slices 0 .. L-1 (the weights of slice 0
  // first: they need no row_token read), and slice 0's token rows in LDS
  // (nk >= 2: K is a multiple of 128).
  load_b(0, std::integral_constant<int, 0>{});
  load_a(0, std::integral_constant<int, 0>{});
  static_for<L - 1>([&](auto i) {
    constexpr int I1 = decltype(i)::value + 1;
    if (I1 < nk) {
      load_b(I1, std::integral_constant<int, I1>{});
      load_a(I1, std::integral_constant<int, I1>{});
    }
  });
  store_a(0, std::integral_constant<int, 0>{});
  __syncthreads();
  // iteration kt: request slice kt + L, multiply slice kt, store the token
  // rows of slice kt + 1 into the LDS stage of slice kt - 1 (read by every
  // wave before the last barrier), barrier; unrolled by S so that every ring
  // slot is a compile-time register set.  The main loop runs while every
  // request of its S iterations is in range, with no branch around a load,
  // so the compiler's waits count exactly the loads still needed; the last
  // slices follow with guarded requests.
  int k0 = 0;
  for (; k0 + S - 1 + L < nk; k0 += S) {
    static_for<S>([&](auto u) {
      constexpr int U = decltype(u)::value;
      const int kt = k0 + U;
      load_a(kt + L, std::integral_constant<int, (U + L) % S>{});
      load_b(kt + L, std::integral_constant<int, (U + L) % S>{});
      mma_slice(kt, u);
      store_a(kt + 1, std::integral_constant<int, (U + 1) % S>{});
      __syncthreads();
    });
  }
  for (; k0 < nk; k0 += S) {
    static_for<S>([&](auto u) {
      constexpr int U = decltype(u)::value;
      const int kt = k0 + U;
      if (kt < nk) {
        if (kt + L < nk) {
          load_a(kt + L, std::integral_constant<int, (U + L) % S>{});
          load_b(kt + L, std::integral_constant<int, (U + L) % S>{});
        }
        mma_slice(kt, u);
        if (kt + 1 < nk) store_a(kt + 1, std::integral_constant<int, (U + 1) % S>{});
        __syncthreads();
      }
    });
  }

  const int fr = lane & 31;
#pragma unroll
  for (int x = 0; x < FM; ++x) {
    const int row = x * 32 + fr;
    const bool live = row < tile_rows;
    const size_t orow = static_cast<size_t>(row0 + m0 + row) * a.NC;
#pragma unroll
    for (int f = 0; f < NPW; ++f) {
      const int g = wave * NPW + f;  // fragment column of the tile
      if constexpr (MODE == GATEUP) {
        // gate rows in registers 0..7, the matching up rows in 8..15
        const int c0 = nt * (BN / 2) + g * 16;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu(acc[x][f][4 * q + i]) * acc[x][f][4 * q + i + 8];
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          if (live) *reinterpret_cast<uint2*>(&a.out[orow + c0 + 8 * q + 4 * fhalf]) = pk;
        }
      } else {
        const int c0 = nt * BN + g * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[x][f][4 * q], acc[x][f][4 * q + 1]);
          pk.y = pack_bf16x2(acc[x][f][4 * q + 2], acc[x][f][4 * q + 3]);
          if (live) *reinterpret_cast<uint2*>(&a.out[orow + c0 + 8 * q + 4 * fhalf]) = pk;
        }
      }
    }
  }
}

// Experts are cut into tiles of up to BMX token rows; each tile runs the
// body of the smallest height (32, 64 or 128) that holds its rows.  The
// grid is at most the number of workgroups the CUs hold at once, and each
// workgroup walks its XCD's range of tiles (the tiles of one expert and
// panel stay on one XCD and share its L2), so no workgroup is launched
// only to find that it has no tile.
template <int MODE, int NPW, int L, int BMX>
__global__ __launch_bounds__(4 * MOE_WAVE) void gemm_stream_kernel(Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* cum = reinterpret_cast<int*>(smem + 2 * BMX * 64 * 2);  // after the A stages
  // The first tile is located from the table in registers (no barrier or
  // LDS round trips before its loads), which wave 0 also leaves in LDS for
  // the later tiles; past 64 * REG_CHUNKS experts the LDS table serves all.
  const bool regs = a.N < 64 * REG_CHUNKS;
  int total, j1 = 0, m01 = 0, nt1 = 0, Mj1 = 0, r01 = 0;
  const int p = blockIdx.x;
  if (regs) {
    TileRegs tr;
    tile_regs<BMX>(a, tr);
    total = tr.total;
    if (threadIdx.x < MOE_WAVE) {
#pragma unroll
      for (int c = 0; c < REG_CHUNKS; ++c)
        if (lane_id() + 64 * c < a.N) cum[lane_id() + 64 * c + 1] = tr.cum[c];
      if (threadIdx.x == 0) cum[0] = 0;
    }
    const int q1 = (total + 7) / 8, L1 = (p % 8) * q1 + p / 8;
    if (p / 8 < q1 && L1 < total) locate_regs<BMX>(a, tr, L1, j1, m01, nt1, Mj1, r01);
  } else {
    total = tile_table<BMX>(a, cum);
  }
  const int q = (total + 7) / 8;  // tiles per XCD
  const int step = gridDim.x / 8;
  for (int slot = p / 8; slot < q; slot += step) {
    const int Lt = (p % 8) * q + slot;
    if (Lt >= total) break;
    int j, m0, nt, Mj, row0;
    if (regs && slot == p / 8) {
      j = j1;
      m0 = m01;
      nt = nt1;
      Mj = Mj1;
      row0 = r01;
    } else {
      locate_tile<BMX>(a, cum, Lt, j, m0, nt, Mj, row0);  // after a workgroup barrier
    }
    j = __builtin_amdgcn_readfirstlane(j);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    nt = __builtin_amdgcn_readfirstlane(nt);
    Mj = __builtin_amdgcn_readfirstlane(Mj);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    const int rows = min(BMX, Mj - m0);
    if (BMX >= 128 && rows > 64) {
      if constexpr (BMX >= 128) stream_body<MODE, 128, NPW, L>(a, smem, j, m0, nt, Mj, row0);
    } else if (BMX >= 64 && rows > 32) {
      if constexpr (BMX >= 64) stream_body<MODE, 64, NPW, L>(a, smem, j, m0, nt, Mj, row0);
    } else {
      stream_body<MODE, 32, NPW, L>(a, smem, j, m0, nt, Mj, row0);
    }
    __syncthreads();  // the next tile's prologue rewrites the A stages
  }
}

// ------------------------------------------------------------- fp32 path
// Small fp32 layers: one workgroup of 256 threads per (expert, 16-row tile,
// 32-column tile), K in chunks of 64 staged through LDS; each thread owns a
// 1 x 2 block of outputs (gate-up: of both the gate and the up columns).
// Small tiles spread a tiny layer over many CUs.  fp32 accumulation in
// ascending K order.
constexpr int F32_BM = 16, F32_BN = 32, F32_BK = 64;

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(Args a, const float* __restrict__ x,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ out) {
  __shared__ int cum[1024 + 2];
  __shared__ float sa[F32_BM][F32_BK + 1];
  __shared__ float sb[MODE == GATEUP ? 2 : 1][F32_BN][F32_BK + 1];
  int j, m0, nt, Mj, row0;
  const bool live = find_tile<F32_BM>(a, cum, j, m0, nt, Mj, row0);
  if (!live) return;
  const int tid = threadIdx.x;
  const int K = a.K, I = a.I;
  const int tr = tid / 16, tc = tid % 16;  // row tr; columns 2 tc, 2 tc + 1
  const int rows = min(F32_BM, Mj - m0);
  const float* wbase = w + static_cast<size_t>(j) * a.w_stride;
  constexpr int NB = MODE == GATEUP ? 2 : 1;
  float acc[NB][2] = {};
  // the row tile (gathered by token for gate-up) and the weight rows of one
  // K chunk go through registers: chunk k0 + BK is requested before chunk k0
  // is multiplied, so its memory latency overlaps the FMAs
  constexpr int UA = F32_BM * F32_BK / 256, UB = NB * F32_BN * F32_BK / 256;
  float va[UA], vb[UB];
  size_t asrc[UA];
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    const int r = (tid + u * 256) / F32_BK;
    asrc[u] = r >= rows ? ~size_t(0)
              : MODE == GATEUP ? static_cast<size_t>(a.row_token[row0 + m0 + r]) * K
                               : static_cast<size_t>(row0 + m0 + r) * K;
  }
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int c = (tid + u * 256) % F32_BK;
      va[u] = asrc[u] != ~size_t(0) && k0 + c < K ? x[asrc[u] + k0 + c] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = tid + u * 256;
      const int b = i / (F32_BN * F32_BK), r = (i / F32_BK) % F32_BN, c = i % F32_BK;
      const int col = nt * F32_BN + r;  // h column (gate-up) or output column (down)
      const size_t wrow = MODE == GATEUP ? static_cast<size_t>(b * I + col) : col;
      vb[u] = col < a.NC && k0 + c < K ? wbase[wrow * K + k0 + c] : 0.f;
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += F32_BK) {
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int i = tid + u * 256;
      sa[i / F32_BK][i % F32_BK] = va[u];
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = tid + u * 256;
      sb[i / (F32_BN * F32_BK)][(i / F32_BK) % F32_BN][i % F32_BK] = vb[u];
    }
    __syncthreads();
    if (k0 + F32_BK < K) fetch(k0 + F32_BK);
#pragma unroll 8
    for (int kk = 0; kk < F32_BK; ++kk) {
      const float x0 = sa[tr][kk];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[b][q] = fmaf(x0, sb[b][2 * tc + q][kk], acc[b][q]);
    }
    __syncthreads();
  }
  if (tr < rows) {
    float* orow = out + static_cast<size_t>(row0 + m0 + tr) * a.NC;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int col = nt * F32_BN + 2 * tc + q;
      if (col >= a.NC) continue;
      if constexpr (MODE == GATEUP) {
        const float g = acc[0][q], u = acc[1][q];
        orow[col] = (g / (1.f + expf(-g))) * u;
      } else {
        orow[col] = acc[0][q];
      }
    }
  }
}

template <int MODE>
static int launch_gemm_f32(Args a, const float* x, const float* w, float* out, int rows_cap,
                           hipStream_t s) {
  if (a.N > 1024) return MOE_EUNSUP;
  a.n_tiles = (a.NC + F32_BN - 1) / F32_BN;
  const int mt_ub = (rows_cap + F32_BM - 1) / F32_BM + std::min(a.N, rows_cap);
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(gemm_f32_kernel<MODE>, dim3(grid), dim3(256), 0, s, a, x, w, out);
  return launch_status();
}

// ------------------------------------------------------------------ host
template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WPE = 1, int SB = S>
static int launch_gemm_dma(const Args& a, int rows_cap, hipStream_t s) {
  constexpr size_t ring = (static_cast<size_t>(S) * BM + static_cast<size_t>(SB) * BN) * BK * 2;
  constexpr size_t epi = MODE == DOWN ? static_cast<size_t>(BM) * (BN * 2 + 16) : 0;
  constexpr size_t lds = ring > epi ? ring : epi;
  // the LDS limit is a per-device function attribute: set once per device
  static std::atomic<bool> attr_set[64];
  const int dev = current_device();
  if (dev < 0 || !attr_set[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemm_dma_kernel<MODE, BM, BN, BK, WM, WN, S, WPE, SB>),
            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess)
      return MOE_EHIP;
    if (dev >= 0) attr_set[dev].store(true, std::memory_order_release);
  }
  // tiles <= sum over active experts of (rows / BM + 1), and at most
  // min(N, rows) experts are active
  const int mt_ub = (rows_cap + BM - 1) / BM + std::min(a.N, rows_cap);
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_dma_kernel<MODE, BM, BN, BK, WM, WN, S, WPE, SB>), dim3(grid),
                     dim3(WM * WN * MOE_WAVE), lds, s, a);
  return MOE_OK;
}

// Persistent prefill down GEMM: one workgroup per CU (a multiple of 8, so
// that every XCD has the same number of tile lists).
template <int BM, int BN, int BK, int WM, int WN, int SA, int SB>
static int launch_gemm_persist_down(const Args& a, hipStream_t s) {
  constexpr size_t lds = (static_cast<size_t>(SA) * BM + static_cast<size_t>(SB) * BN) * BK * 2;
  static std::atomic<bool> attr_set[64];
  const void* fn = reinterpret_cast<const void*>(gemm_persist_down_kernel<BM, BN, BK, WM, WN, SA, SB>);
  const int dev = current_device();
  if (dev < 0 || !attr_set[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return MOE_EHIP;
    if (dev >= 0) attr_set[dev].store(true, std::memory_order_release);
  }
  const int grid = std::max(8, cu_count() / 8 * 8);
  hipLaunchKernelGGL((gemm_persist_down_kernel<BM, BN, BK, WM, WN, SA, SB>), dim3(grid),
                     dim3(WM * WN * MOE_WAVE), lds, s, a);
  return MOE_OK;
}

template <int MODE, int BN, int BK, int BMA, int SA, int SAB, int BMB, int SB, int SBB,
          int WPE>
static int launch_gemm_dual(Args a, int rows_cap, hipStream_t s) {
  constexpr size_t la = (static_cast<size_t>(SA) * BMA + static_cast<size_t>(SAB) * BN) * BK * 2;
  constexpr size_t lb = (static_cast<size_t>(SB) * BMB + static_cast<size_t>(SBB) * BN) * BK * 2;
  constexpr size_t lds = la > lb ? la : lb;
  static std::atomic<bool> attr_set[64];
  const void* fn =
      reinterpret_cast<const void*>(gemm_dual_kernel<MODE, BN, BK, BMA, SA, SAB, BMB, SB, SBB, WPE>);
  const int dev = current_device();
  if (dev < 0 || !attr_set[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds)) != hipSuccess)
      return MOE_EHIP;
    if (dev >= 0) attr_set[dev].store(true, std::memory_order_release);
  }
  a.dual_limit = WPE * cu_count();
  constexpr int BMIN = BMA < BMB ? BMA : BMB;
  const int mt_ub = (rows_cap + BMIN - 1) / BMIN + std::min(a.N, rows_cap);
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_dual_kernel<MODE, BN, BK, BMA, SA, SAB, BMB, SB, SBB, WPE>), dim3(grid),
                     dim3(4 * MOE_WAVE), lds, s, a);
  return MOE_OK;
}

// Small-batch decode: panels of 16 weight rows (see gemm_skinny_kernel).
#ifndef MOE_SKINNY_S
#define MOE_SKINNY_S 3
#endif
constexpr int SKINNY_S = MOE_SKINNY_S;
template <int MODE>
static int launch_gemm_skinny(Args a, int rows_cap, hipStream_t s) {
  constexpr int BM = 16, BN = 16, BK = 128;
  constexpr size_t lds = static_cast<size_t>(SKINNY_S) * (BM + BN) * BK * 2;
  static_assert(lds <= 65536, "default LDS limit");
  a.n_tiles = MODE == GATEUP ? a.I / (BN / 2) : a.NC / BN;
  const int mt_ub = (rows_cap + BM - 1) / BM + std::min(a.N, rows_cap);
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_skinny_kernel<MODE, SKINNY_S>), dim3(grid), dim3(4 * MOE_WAVE), lds,
                     s, a);
  return MOE_OK;
}

// Decode GEMV on packed panels (see gemv_kernel): one workgroup per
// (expert, MR token rows, 32-row group).
template <int MODE, int MR, int NBW, bool COMB>
static int launch_gemv(Args a, const Comb& c, int rows_cap, hipStream_t s) {
  a.n_tiles = (MODE == GATEUP ? 2 * a.I : a.NC) / 32;
  constexpr int XR = MODE == GATEUP ? GEMV_MAX_T : MR;
  const size_t lds = static_cast<size_t>(XR) * a.K * 2 + 4 * MR * 32 * 4 +
                     static_cast<size_t>(a.N + 2) * 4;
  const void* fn = reinterpret_cast<const void*>(gemv_kernel<MODE, MR, NBW, COMB>);
  if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds)) != hipSuccess)
    return MOE_EHIP;
  const int mt_ub = (rows_cap + MR - 1) / MR + std::min(a.N, rows_cap);
  long grid = static_cast<long>(mt_ub) * a.n_tiles;
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemv_kernel<MODE, MR, NBW, COMB>), dim3(grid), dim3(4 * MOE_WAVE), lds, s,
                     a, c);
  return MOE_OK;
}

// GEMV for decode batches of at most MOE_GEMV_ROWS dispatch rows (and, for
// gate-up, at most GEMV_MAX_T tokens) on packed weights whose reduction
// length is a multiple of 256 up to GEMV_MAX_K.  Each workgroup makes one
// pass over its weights, so the path pays off while its workgroups fit the
// CUs at once: measured on the qwen3 shape in a chain of layers, batch 1
// (8 rows) 33.6 -> 32.5 us per layer, batch 2 (16 rows) 47.1 -> 41.7 us,
// but batch 8 (64 rows, ~1400 workgroups) 69.7 -> 78.1 us.
#ifndef MOE_GEMV_ROWS
#define MOE_GEMV_ROWS 16
#endif
static bool gemv_nbw_ok(int K) {
  const int nbw = K / 256;
  return K % 256 == 0 && (nbw == 1 || nbw == 2 || nbw == 3 || nbw == 4 || nbw == 8);
}
static bool gemv_ok(int mode, int T, int k, int K, bool panels) {
  return panels && static_cast<long>(T) * k <= MOE_GEMV_ROWS && gemv_nbw_ok(K) &&
         (mode == DOWN || T <= GEMV_MAX_T);
}
template <int MODE, int MR, bool COMB>
static int launch_gemv_k(const Args& a, const Comb& c, int rows_cap, hipStream_t s) {
  switch (a.K / 256) {
    case 1: return launch_gemv<MODE, MR, 1, COMB>(a, c, rows_cap, s);
    case 2: return launch_gemv<MODE, MR, 2, COMB>(a, c, rows_cap, s);
    case 3: return launch_gemv<MODE, MR, 3, COMB>(a, c, rows_cap, s);
    case 4: return launch_gemv<MODE, MR, 4, COMB>(a, c, rows_cap, s);
    default: return launch_gemv<MODE, MR, 8, COMB>(a, c, rows_cap, s);
  }
}
// COMB (down only): the combine folded in; needs T * k <= 64 (one slot per
// lane) -- every GEMV batch.
template <int MODE, bool COMB = false>
static int launch_gemv_rows(const Args& a, int rows_cap, hipStream_t s, const Comb& c = Comb{}) {
  static_assert(MOE_GEMV_ROWS <= 64, "token-row chunks of 4 or 16; a slot per lane");
  static_assert(!COMB || MODE == DOWN, "the combine follows the down projection");
  return rows_cap <= 16 ? launch_gemv_k<MODE, 4, COMB>(a, c, rows_cap, s)
                        : launch_gemv_k<MODE, 16, COMB>(a, c, rows_cap, s);
}

// ------------------------------------------------------- weight packing
// One thread per 16-byte chunk (8 elements) of the packed matrix: chunk q of
// an expert's block is (block, group G, K step kk, lane l), holding elements
// 64 b + 16 kk + 8 (l / 32) .. +7 of tile-order row 128 P + 32 G + l % 32
// (block P * K/64 + b), read from the source row that tile-order row stands
// for.
template <int MODE>
__global__ __launch_bounds__(256) void pack_panels_kernel(const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst, long chunks,
                                                          uint32_t rows, uint32_t K, uint32_t I) {
  const long o = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (o >= chunks) return;
  constexpr uint32_t CPB = PANEL_BLOCK / 16;             // chunks per block
  const long per_expert = static_cast<long>(rows) * K / 8;
  const long e = o / per_expert;
  const uint32_t q = static_cast<uint32_t>(o % per_expert);
  const uint32_t blk = q / CPB, w = q % CPB;
  const uint32_t P = blk / (K / PANEL_K), b = blk % (K / PANEL_K);
  const uint32_t G = w / 256, kk = (w / 64) % 4, l = w % 64;
  const uint32_t t = P * PANEL_ROWS + G * 32 + l % 32;   // tile-order row
  const uint32_t k = b * PANEL_K + kk * 16 + (l / 32) * 8;
  uint32_t wrow = t;
  if (MODE == GATEUP) {                                  // inverse of w13_tile_row
    const uint32_t r = t % 32, c = (t / PANEL_ROWS) * 64 + ((t % PANEL_ROWS) / 32) * 16 + r % 16;
    wrow = r < 16 ? c : I + c;
  }
  dst[o] = src[e * per_expert + (static_cast<long>(wrow) * K + k) / 8];
}

// Decode tiles on packed weights (gemm_stream_kernel), measured on MI355X
// (qwen3 and Mixtral decode shapes and the 48-layer sweep layer at batches
// 32, 128 and 256): operands requested 2 slices ahead (3 needs more than
// 256 registers with the 128-row tiles, halving the workgroups per CU, and
// is no faster where it fits); gate-up with token-row tiles up to 128 (one
// tile per expert and panel: the large experts after SERE read their panel
// once), down with tiles of 32 token rows (more workgroups per CU) and two
// panels per workgroup when the panels of the experts that may be active
// number at least twice the workgroup slots (4 per CU), else one.
#ifndef MOE_STREAM_L
#define MOE_STREAM_L 2
#endif
#ifndef MOE_STREAM_NPW_GU
#define MOE_STREAM_NPW_GU 1
#endif
#ifndef MOE_STREAM_GU
#define MOE_STREAM_GU 1
#endif
#ifndef MOE_STREAM_BMX_GU
#define MOE_STREAM_BMX_GU 128
#endif
#ifndef MOE_STREAM_BMX_DN
#define MOE_STREAM_BMX_DN 32
#endif
#ifndef MOE_STREAM_DN
#define MOE_STREAM_DN 1
#endif
template <int MODE, int NPW, int L, int BMX>
static int launch_gemm_stream(Args a, int rows_cap, hipStream_t s) {
  constexpr int BN = 128 * NPW;
  // two stages of the tallest token-row tile, then the tile table
  const size_t lds = 2 * BMX * 64 * 2 + (static_cast<size_t>(a.N) + 2) * 4;
  const void* fn = reinterpret_cast<const void*>(gemm_stream_kernel<MODE, NPW, L, BMX>);
  // workgroups one CU holds at once, per device (at most 4 with the
  // smallest tiles' registers)
  static std::atomic<int> per_cu[64];
  const int dev = current_device();
  int wpc = dev >= 0 ? per_cu[dev].load(std::memory_order_acquire) : 0;
  if (wpc == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&wpc, fn, 4 * MOE_WAVE, lds) !=
            hipSuccess ||
        wpc < 1)
      wpc = 1;
    if (dev >= 0) per_cu[dev].store(wpc, std::memory_order_release);
  }
  a.n_tiles = (MODE == GATEUP ? 2 * a.I : a.NC) / BN;
  const int mt_ub = (rows_cap + BMX - 1) / BMX + std::min(a.N, rows_cap);
  long grid = std::min(static_cast<long>(mt_ub) * a.n_tiles, static_cast<long>(wpc) * cu_count());
  grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_stream_kernel<MODE, NPW, L, BMX>), dim3(grid), dim3(4 * MOE_WAVE), lds,
                     s, a);
  return MOE_OK;
}

}  // namespace ffn
}  // namespace moe

using namespace moe;
using namespace moe::ffn;

// Prefill tiles: 256 rows x 256 columns of C per workgroup of 8 waves (2 x
// 4, each a 128 x 64 block of 4 x 2 fragments, two waves per SIMD), K slices
// of 64 (whole 128-byte row segments per load) through a direct-to-LDS ring
// of 2 token-row stages and 3 weight stages.  The gate-up tile covers 128 h columns (128 gate rows
// + 128 up rows of W13), the down tile 256 output columns.  Measured on
// MI355X against 4 waves with K slices of 32 in 4 stages: 3-6 % faster on
// the multimodal and Mixtral prefill shapes.
#ifndef MOE_GU_CFG
#define MOE_GU_CFG 256, 256, 64, 2, 4
#endif
#ifndef MOE_DN_CFG
#define MOE_DN_CFG 256, 256, 64, 2, 4
#endif
#ifndef MOE_DN_STAGES
#define MOE_DN_STAGES 2
#endif
#ifndef MOE_DN_WPE
#define MOE_DN_WPE 1
#endif
#ifndef MOE_STAGES
#define MOE_STAGES 2
#endif
// B (weight) ring depth of the prefill tiles: 3 stages of weights beside the
// 2 of token rows fill the 160 KB exactly (down 5 % faster on the multimodal
// prefill shape, the rest unchanged; 3 stages of token rows instead were
// slower)
#ifndef MOE_STAGES_B
#define MOE_STAGES_B 3
#endif
#ifndef MOE_DN_STAGES_B
#define MOE_DN_STAGES_B 3
#endif
// Prefill down tiles walked by one persistent workgroup per CU (below 320
// experts, the register tile search) instead of a workgroup per tile.
#ifndef MOE_PERSIST_DN
#define MOE_PERSIST_DN 1
#endif
// Decode tiles: 32 or 128 token rows x 128 or 256 weight rows (1 x 4
// waves), K through a streaming ring.  Measured on MI355X (qwen3 and
// Mixtral decode shapes, weights rotated so HBM is read every step;
// interleaved repeats, medians):
//   gate-up: 128-row weight tiles; reductions under 4096: 128 token rows
//            (one tile streams an expert's weight panel once for all its
//            rows), K slices of 64, 2 stages; reductions of 4096 or more:
//            32 token rows, K slices of 128, 3 stages;
//   down:    256-row weight tiles unless that leaves CUs idle (few experts),
//            then 128-row ones; 32 token rows; K slices of 64 with 2 stages,
//            or of 128 with 3 stages for reductions of 4096 or more.
//   K slices of 32 (64-byte row segments) stream worse than 64 or 128.
// Decode tile configurations {token rows, K slice, token-row stages,
// weight stages (0: as many as token-row stages)}; the _WIDE
// ones serve reductions of 4096 or more.  Gate-up below that picks on the
// device between DEC_GU (one tile per expert and weight panel, when those
// tiles fit the workgroup slots at once) and DEC_GU_MANY (32-row tiles and
// a deeper ring, when many experts are active).
#ifndef MOE_DEC_GU
#define MOE_DEC_GU 128, 64, 2
#endif
#ifndef MOE_DEC_GU_MANY
#define MOE_DEC_GU_MANY 32, 64, 3
#endif
#ifndef MOE_DEC_GU_WIDE
#define MOE_DEC_GU_WIDE 32, 128, 3
#endif
#ifndef MOE_DEC_DN
#define MOE_DEC_DN 32, 64, 2
#endif
#ifndef MOE_DEC_DN_WIDE
#define MOE_DEC_DN_WIDE 32, 128, 3
#endif
struct DecCfg {
  int bm, bk, s, sb0;
  constexpr int sb() const { return sb0 ? sb0 : s; }
};
constexpr DecCfg DEC_GU = {MOE_DEC_GU}, DEC_GU_MANY = {MOE_DEC_GU_MANY},
                 DEC_GU_WIDE = {MOE_DEC_GU_WIDE},
                 DEC_DN = {MOE_DEC_DN}, DEC_DN_WIDE = {MOE_DEC_DN_WIDE};
// LDS of a decode workgroup with bn weight rows: the ring (the tile-count
// table shares it)
constexpr int dec_lds(DecCfg c, int bn) { return (c.s * c.bm + c.sb() * bn) * c.bk * 2; }
// workgroups per CU that the LDS allows (160 KB per CU), at most 4
constexpr int dec_wpe(DecCfg c, int bn) {
  return (160 * 1024) / dec_lds(c, bn) < 4 ? (160 * 1024) / dec_lds(c, bn) : 4;
}
static_assert(dec_wpe(DEC_GU, 128) >= 1 && dec_wpe(DEC_GU_WIDE, 128) >= 1 &&
                  dec_wpe(DEC_DN, 128) >= 1 && dec_wpe(DEC_DN_WIDE, 128) >= 1,
              "decode tiles fit the LDS");
// 256-row down tiles only where their ring fits
constexpr bool DN_256 = dec_wpe(DEC_DN, 256) >= 1, DN_256_WIDE = dec_wpe(DEC_DN_WIDE, 256) >= 1;
constexpr int GU_CFG[] = {MOE_GU_CFG};
constexpr int DN_CFG[] = {MOE_DN_CFG};
constexpr int GU_BM = GU_CFG[0], GU_BN = GU_CFG[1], GU_BK = GU_CFG[2],
              GU_WM = GU_CFG[3], GU_WN = GU_CFG[4];
constexpr int DN_BM = DN_CFG[0], DN_BN = DN_CFG[1], DN_BK = DN_CFG[2],
              DN_WM = DN_CFG[3], DN_WN = DN_CFG[4];
// every bf16 shape the entry points accept (H % 256 == 0, I % 128 == 0)
// splits into whole column tiles and whole K slices
static_assert(128 % (GU_BN / 2) == 0, "h column tiles");
static_assert(256 % DN_BN == 0, "output column tiles");
static_assert(256 % GU_BK == 0, "gate-up K slices");
static_assert(128 % DN_BK == 0, "down K slices");

// Decode-sized batches (at most 32 rows per expert on average) use the
// weight-streaming decode tiles; larger batches use the 256 x 256 prefill
// tiles.
static bool decode_tiles(int T, int N, int k) {
  return static_cast<long>(T) * k <= 32L * N;
}


// The smallest batches (a few dispatch rows) stream 16-row weight panels:
// gate-up up to 64 dispatch rows, down up to 16 (measured on the 2048 x 768
// expert shape at 8, 16, 32, 48, 64 and 128 rows, with and without SERE).
#ifndef MOE_SKINNY_ROWS_GU
#define MOE_SKINNY_ROWS_GU 64
#endif
#ifndef MOE_SKINNY_ROWS_DN
#define MOE_SKINNY_ROWS_DN 16
#endif
static bool skinny_tiles(int T, int k, int mode) {
  return static_cast<long>(T) * k <= (mode == GATEUP ? MOE_SKINNY_ROWS_GU : MOE_SKINNY_ROWS_DN);
}

// Decode weight-tile height: 256 rows unless that gives fewer tiles than
// two per CU (the number of experts with rows is at most min(N, T*k)).
#ifndef MOE_DEC_DN_NARROW
#define MOE_DEC_DN_NARROW 0
#endif
static bool narrow_decode_tiles(int T, int N, int k, int cols_per_256) {
  if (MOE_DEC_DN_NARROW) return true;
  const long experts = std::min(static_cast<long>(N), static_cast<long>(T) * k);
  return experts * cols_per_256 < 2L * cu_count();
}

static int check_ffn_shape(int T, int N, int k, int H, int I, int dtype) {
  if (T < 0 || T > (1 << 20) || N < 1 || N > 1024 || k < 1 || k > N ||
      H < 1 || I < 1)
    return MOE_EINVAL;
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_BF16_PANELS) return MOE_EUNSUP;
  if (dtype != MOE_F32 && (H % 256 != 0 || I % 128 != 0)) return MOE_EUNSUP;
  // bf16 loads address x and one expert's weight block with 32-bit byte
  // offsets; x stays under 2^31 bytes so that OOB_OFF lies outside it
  if (dtype != MOE_F32 && (static_cast<uint64_t>(T) * H * 2 > (1ull << 31) ||
                            static_cast<uint64_t>(I) * H * 4 >= (1ull << 32)))
    return MOE_EUNSUP;
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
    Args g{};
    g.row_token = row_token;
    g.offsets = expert_offsets;
    g.N = N;
    g.K = H;
    g.NC = I;
    g.I = I;
    g.w_stride = 2L * I * H;
    return launch_gemm_f32<GATEUP>(g, static_cast<const float*>(x),
                                   static_cast<const float*>(w13), static_cast<float*>(h),
                                   rows_cap, s);
  }
  Args g{};
  g.a = static_cast<const uint16_t*>(x);
  g.a_rows = T;
  g.row_token = row_token;
  g.offsets = expert_offsets;
  g.w = static_cast<const uint16_t*>(w13);
  g.out = static_cast<uint16_t*>(h);
  g.N = N;
  g.K = H;
  g.NC = I;
  g.I = I;
  g.w_stride = 2L * I * H;
  g.panels = dtype == MOE_BF16_PANELS;
  if (decode_tiles(T, N, k)) {
    int st;
    g.n_tiles = I / 64;
    if (gemv_ok(GATEUP, T, k, H, g.panels)) {
      st = launch_gemv_rows<GATEUP>(g, rows_cap, s);
    } else if (MOE_STREAM_GU && g.panels && !skinny_tiles(T, k, GATEUP)) {
      st = launch_gemm_stream<GATEUP, MOE_STREAM_NPW_GU, MOE_STREAM_L, MOE_STREAM_BMX_GU>(g, rows_cap, s);
    } else if (skinny_tiles(T, k, GATEUP)) {
      st = launch_gemm_skinny<GATEUP>(g, rows_cap, s);
    } else if (H >= 4096) {
      constexpr DecCfg c = DEC_GU_WIDE;
      st = launch_gemm_dma<GATEUP, c.bm, 128, c.bk, 1, 4, c.s, dec_wpe(c, 128), c.sb()>(g, rows_cap, s);
    } else {
      // one wave of DEC_GU tiles when they fit the workgroup slots (few
      // active experts, e.g. after SERE), else the DEC_GU_MANY tiles
      constexpr DecCfg c = DEC_GU, m = DEC_GU_MANY;
      static_assert(c.bk == m.bk, "one K slice for both tile heights");
      constexpr int wpe = dec_wpe(c, 128) < dec_wpe(m, 128) ? dec_wpe(c, 128) : dec_wpe(m, 128);
      st = launch_gemm_dual<GATEUP, 128, c.bk, c.bm, c.s, c.sb(), m.bm, m.s, m.sb(), wpe>(g, rows_cap, s);
    }
    if (st != MOE_OK) return MOE_EHIP;
  } else {
    g.n_tiles = I / (GU_BN / 2);
    if (launch_gemm_dma<GATEUP, GU_BM, GU_BN, GU_BK, GU_WM, GU_WN, MOE_STAGES, 1,
                        MOE_STAGES_B>(g, rows_cap, s) != MOE_OK)
      return MOE_EHIP;
  }
  return launch_status();
}

// bf16 down-projection arguments (row or panel layout)
static Args down_args(const void* h, const int32_t* expert_offsets, const void* w2, int T,
                      int N, int k, int H, int I, int dtype, void* out_rows) {
  Args d{};
  d.a = static_cast<const uint16_t*>(h);
  d.a_rows = T * k;
  d.row_token = nullptr;
  d.offsets = expert_offsets;
  d.w = static_cast<const uint16_t*>(w2);
  d.out = static_cast<uint16_t*>(out_rows);
  d.N = N;
  d.K = I;
  d.NC = H;
  d.I = I;
  d.w_stride = static_cast<long>(H) * I;
  d.panels = dtype == MOE_BF16_PANELS;
  return d;
}

// The down GEMV with the combine folded in applies (see gemv_kernel).
static bool down_combine_fused(int T, int N, int k, int I, int dtype) {
  return dtype == MOE_BF16_PANELS && decode_tiles(T, N, k) && gemv_ok(DOWN, T, k, I, true);
}

// Down tiles streamed from packed weights (decode batches past the GEMV and
// the 16-row tiles): 256 output columns a tile when the tiles fill the CUs
// 8 times over, else 128.
static int launch_down_stream(const Args& d, int T, int N, int k, int H, hipStream_t s) {
  const long experts = std::min(static_cast<long>(N), static_cast<long>(T) * k);
  return experts * (H / 128) >= 8L * cu_count()
             ? launch_gemm_stream<DOWN, 2, MOE_STREAM_L, MOE_STREAM_BMX_DN>(d, T * k, s)
             : launch_gemm_stream<DOWN, 1, MOE_STREAM_L, MOE_STREAM_BMX_DN>(d, T * k, s);
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
    Args d{};
    d.offsets = expert_offsets;
    d.N = N;
    d.K = I;
    d.NC = H;
    d.I = I;
    d.w_stride = static_cast<long>(H) * I;
    return launch_gemm_f32<DOWN>(d, static_cast<const float*>(h),
                                 static_cast<const float*>(w2), static_cast<float*>(out_rows),
                                 rows_cap, s);
  }
  Args d = down_args(h, expert_offsets, w2, T, N, k, H, I, dtype, out_rows);
  if (decode_tiles(T, N, k)) {
    int st;
    const bool narrow = narrow_decode_tiles(T, N, k, H / 256);
    if (gemv_ok(DOWN, T, k, I, d.panels)) {
      st = launch_gemv_rows<DOWN>(d, rows_cap, s);
    } else if (MOE_STREAM_DN && d.panels && !skinny_tiles(T, k, DOWN)) {
      st = launch_down_stream(d, T, N, k, H, s);
    } else if (skinny_tiles(T, k, DOWN)) {
      st = launch_gemm_skinny<DOWN>(d, rows_cap, s);
    } else if (I >= 4096) {
      constexpr DecCfg c = DEC_DN_WIDE;
      const bool nar = narrow || !DN_256_WIDE;
      d.n_tiles = nar ? H / 128 : H / 256;
      if constexpr (DN_256_WIDE) {
        st = nar ? launch_gemm_dma<DOWN, c.bm, 128, c.bk, 1, 4, c.s, dec_wpe(c, 128), c.sb()>(d, rows_cap, s)
                 : launch_gemm_dma<DOWN, c.bm, 256, c.bk, 1, 4, c.s, dec_wpe(c, 256), c.sb()>(d, rows_cap, s);
      } else {
        st = launch_gemm_dma<DOWN, c.bm, 128, c.bk, 1, 4, c.s, dec_wpe(c, 128), c.sb()>(d, rows_cap, s);
      }
    } else {
      constexpr DecCfg c = DEC_DN;
      const bool nar = narrow || !DN_256;
      d.n_tiles = nar ? H / 128 : H / 256;
      if constexpr (DN_256) {
        st = nar ? launch_gemm_dma<DOWN, c.bm, 128, c.bk, 1, 4, c.s, dec_wpe(c, 128), c.sb()>(d, rows_cap, s)
                 : launch_gemm_dma<DOWN, c.bm, 256, c.bk, 1, 4, c.s, dec_wpe(c, 256), c.sb()>(d, rows_cap, s);
      } else {
        st = launch_gemm_dma<DOWN, c.bm, 128, c.bk, 1, 4, c.s, dec_wpe(c, 128), c.sb()>(d, rows_cap, s);
      }
    }
    if (st != MOE_OK) return MOE_EHIP;
  } else {
    d.n_tiles = H / DN_BN;
    const int st = MOE_PERSIST_DN && N < 64 * REG_CHUNKS
                       ? launch_gemm_persist_down<DN_BM, DN_BN, DN_BK, DN_WM, DN_WN, MOE_DN_STAGES,
                                                  MOE_DN_STAGES_B>(d, s)
                       : launch_gemm_dma<DOWN, DN_BM, DN_BN, DN_BK, DN_WM, DN_WN, MOE_DN_STAGES,
                                         MOE_DN_WPE, MOE_DN_STAGES_B>(d, rows_cap, s);
    if (st != MOE_OK) return MOE_EHIP;
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

// Arrival tickets of the fused combine at the start of its workspace, one
// per 32 output columns, then h.
static size_t ticket_bytes(int H) {
  return ((static_cast<size_t>(H) + 31) / 32 * 4 + 255) & ~size_t(255);
}

extern "C" size_t moe_ffn_combine_workspace_size(int T, int N, int k, int H, int I,
                                                 int dtype) {
  if (T < 0 || k < 1 || H < 1 || I < 1) return 0;
  return ticket_bytes(H) + moe_ffn_workspace_size(T, N, k, H, I, dtype);
}

extern "C" int moe_ffn_down_combine(const void* h, const int32_t* row_token,
                                    const int32_t* expert_offsets, const void* w2,
                                    const int32_t* slot_row, const float* topk_gates, int T,
                                    int N, int k, int H, int I, int dtype, void* out_rows,
                                    void* y, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (H % 8 != 0) return MOE_EUNSUP;  // the combine's row vectors
  if (T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < ticket_bytes(H)) return MOE_EINVAL;
  if (!h || !row_token || !expert_offsets || !w2 || !slot_row || !topk_gates || !out_rows || !y)
    return MOE_EINVAL;
  if (down_combine_fused(T, N, k, I, dtype)) {
    const Args d = down_args(h, expert_offsets, w2, T, N, k, H, I, dtype, out_rows);
    const Comb c{slot_row, topk_gates, static_cast<uint16_t*>(y),
                 static_cast<unsigned*>(workspace), T, k};
    if (launch_gemv_rows<DOWN, true>(d, T * k, as_stream(stream), c) != MOE_OK) return MOE_EHIP;
    return launch_status();
  }
  const int r = moe_ffn_down(h, expert_offsets, w2, T, N, k, H, I, dtype, out_rows, stream);
  if (r != MOE_OK) return r;
  return moe_combine(out_rows, slot_row, topk_gates, T, k, H,
                     dtype == MOE_F32 ? MOE_F32 : MOE_BF16, y, stream);
}

extern "C" int moe_expert_ffn_combine(const void* x, const int32_t* row_token,
                                      const int32_t* expert_offsets, const void* w13,
                                      const void* w2, const int32_t* slot_row,
                                      const float* topk_gates, int T, int N, int k, int H,
                                      int I, int dtype, void* out_rows, void* y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (H % 8 != 0) return MOE_EUNSUP;  // the combine's row vectors
  if (T == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_ffn_combine_workspace_size(T, N, k, H, I, dtype))
    return MOE_EINVAL;
  if (!x || !row_token || !expert_offsets || !w13 || !w2 || !slot_row || !topk_gates ||
      !out_rows || !y)
    return MOE_EINVAL;
  const size_t tb = ticket_bytes(H);
  void* h = static_cast<unsigned char*>(workspace) + tb;
  const int r = moe_ffn_gate_up(x, row_token, expert_offsets, w13, T, N, k, H, I, dtype, h,
                                stream);
  if (r != MOE_OK) return r;
  return moe_ffn_down_combine(h, row_token, expert_offsets, w2, slot_row, topk_gates, T, N, k,
                              H, I, dtype, out_rows, y, workspace, tb, stream);
}

extern "C" int moe_pack_weights(const void* w13, const void* w2, int N, int H, int I,
                                int dtype, void* w13_panels, void* w2_panels, void* stream) {
  if (dtype == MOE_F32 || dtype == MOE_BF16_PANELS) return MOE_EUNSUP;
  const int st = check_ffn_shape(0, N, 1, H, I, dtype);
  if (st != MOE_OK) return st;
  if ((w13 == nullptr) != (w13_panels == nullptr) || (w2 == nullptr) != (w2_panels == nullptr))
    return MOE_EINVAL;
  if ((w13 && w13 == w13_panels) || (w2 && w2 == w2_panels)) return MOE_EINVAL;
  hipStream_t s = as_stream(stream);
  if (w13) {
    const long chunks = static_cast<long>(N) * 2 * I * H / 8;
    hipLaunchKernelGGL(pack_panels_kernel<GATEUP>, dim3((chunks + 255) / 256), dim3(256), 0, s,
                       static_cast<const uint4*>(w13), static_cast<uint4*>(w13_panels), chunks,
                       static_cast<uint32_t>(2 * I), static_cast<uint32_t>(H),
                       static_cast<uint32_t>(I));
  }
  if (w2) {
    const long chunks = static_cast<long>(N) * H * I / 8;
    hipLaunchKernelGGL(pack_panels_kernel<DOWN>, dim3((chunks + 255) / 256), dim3(256), 0, s,
                       static_cast<const uint4*>(w2), static_cast<uint4*>(w2_panels), chunks,
                       static_cast<uint32_t>(H), static_cast<uint32_t>(I),
                       static_cast<uint32_t>(I));
  }
  return launch_status();
}

// ------------------------------------------------------- no allocation
// h of moe_expert_ffn_noalloc lives in this file-scope device array: each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol); it asks the runtime once per device for the array's
// device address and passes that, as moe_expert_ffn passes its workspace.
static __device__ __align__(256) unsigned char scratch[MOE_FFN_NOALLOC_MAX_BYTES];

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current; nullptr if the lookup fails.
static void* scratch_on_current_device() {
  static std::atomic<void*> addr[64];
  static std::mutex lookup;
  const int dev = current_device();
  if (dev < 0) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> g(lookup);
  p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  addr[dev].store(p, std::memory_order_release);
  return p;
}

extern "C" int moe_expert_ffn_noalloc(const void* x, const int32_t* row_token,
                                      const int32_t* expert_offsets, const void* w13,
                                      const void* w2, int T, int N, int k, int H, int I,
                                      int dtype, void* out_rows, void* stream) {
  const int st = check_ffn_shape(T, N, k, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (moe_ffn_workspace_size(T, N, k, H, I, dtype) > MOE_FFN_NOALLOC_MAX_BYTES)
    return MOE_ESCRATCH;
  void* h = scratch_on_current_device();
  if (!h) return MOE_EHIP;
  // h needs no clearing: the gate-up GEMM writes every row the down GEMM reads
  const int r = moe_ffn_gate_up(x, row_token, expert_offsets, w13, T, N, k, H,
                                I, dtype, h, stream);
  if (r != MOE_OK) return r;
  return moe_ffn_down(h, expert_offsets, w2, T, N, k, H, I, dtype, out_rows,
                      stream);
}
