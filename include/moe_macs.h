/*
 * moe_macs.h -- C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * One mixture-of-experts layer, y(x) = sum_{j in Top-k(G(x))} G(x)_j E_j(x)
 * ("MACS: Modality-Aware Capacity Scaling for Efficient Multimodal MoE
 * Inference", §3.1 Eq. 1), wrapped in
 *   - MACS capacity routing: entropy-weighted expert load (§3.2 Eq. 5-6),
 *     modality-adaptive capacity from the effective visual ratio (§3.3
 *     Eq. 7 and the expert modality indicator m_j), and re-route-else-drop
 *     of overflowing tokens (§1 and Fig. 1);
 *   - SERE re-routing (multi-image QA inference write-up, §4.1-§4.3): the
 *     batch union of every token's top-K' primaries, secondary experts moved
 *     onto the most similar primary above a threshold, gated by a per-layer
 *     0/1 protection matrix.
 *
 * Call order on one stream (prefill skips moe_sere_reroute, since prefill
 * keeps the original top-K):
 *   moe_route -> moe_sere_reroute -> moe_capacity_assign -> moe_dispatch
 *   -> moe_expert_ffn -> moe_combine
 * Decode-sized batches can replace the first four calls by one
 * moe_routing_fused launch, and moe_expert_ffn_combine makes the last two
 * one call.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps pointers after returning.
 *     The only state it keeps is per device and set on first use: the
 *     compute-unit count, whether a GEMM kernel's LDS limit has been set,
 *     and the device address of moe_expert_ffn_noalloc's fixed buffer.
 *   - Arrays are dense and row-major; "[T,k]" means T rows of k elements.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  No entry point synchronises with
 *     the host or reads device memory from the host, so the sequence can be
 *     captured in a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued.  On an
 *     error nothing is enqueued and the call returns:
 *        MOE_EINVAL  a required pointer is NULL or a size is out of range,
 *        MOE_EUNSUP  unsupported element type,
 *        MOE_EHIP    the HIP runtime reported a launch error,
 *        MOE_ESCRATCH  the no-allocation variant's fixed buffer is too
 *                    small for the call.
 *   - T == 0 is valid and enqueues nothing.
 *   - Limits: 1 <= N <= 1024 experts, 1 <= k <= N, 0 <= R <= N - k,
 *     T <= 2^20 tokens.
 *   - Device data are not validated: router logits must be finite, expert
 *     ids must lie in [0, N).
 *   - Results are deterministic: no floating-point atomics; integer
 *     reductions only where order cannot matter.
 *
 * Workspaces
 *   moe_router_topk, moe_capacity_assign, moe_dispatch, moe_routing_fused,
 *   moe_expert_ffn and moe_expert_ffn_combine take a workspace of at least
 *   the size their *_workspace_size() query returns.  The router, capacity,
 *   dispatch, fused-routing and FFN-combine workspaces hold a few control
 *   words: they must be filled with zero bytes once, before their first use
 *   (e.g. allocated zeroed); every call leaves those words zero again.  A workspace must not be
 *   shared by calls that may run concurrently.
 */
#ifndef MOE_MACS_H
#define MOE_MACS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_OK = 0, MOE_EINVAL = -1, MOE_EUNSUP = -2, MOE_EHIP = -3,
       MOE_ESCRATCH = -4 };

/* element type of x, expert weights, intermediates, out_rows and y;
 * MOE_BF16_PANELS (expert FFN calls only) is bf16 with the expert weights in
 * the panel layout written by moe_pack_weights */
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_BF16_PANELS = 2 };

/* flags[t,s] bits written by moe_sere_reroute / moe_capacity_assign */
enum { MOE_FLAG_SERE = 1, MOE_FLAG_MACS = 2, MOE_FLAG_DROP = 4 };

/* Fixed-point unit of token weights, loads and capacities: one full token. */
#define MOE_WEIGHT_ONE 65536

/*
 * moe_route -- router softmax and top-k (MACS §3.1 Eq. 1).
 *
 * logits        f32[T,N]  router scores.
 * topk_ids      i32[T,k]  out: experts ranked by logit descending; equal
 *                         logits rank the lower expert index first, and
 *                         -0.0 equals +0.0.
 * topk_gates    f32[T,k]  out: G(x)_j = softmax over all N logits of the
 *                         ranked expert (no renormalisation over the top-k).
 * fallback_ids  i32[T,R]  out: ranks k+1..k+R, the overflow re-route
 *                         candidates of moe_capacity_assign; may be NULL
 *                         when R == 0.
 */
int moe_route(const float* logits, int T, int N, int k, int R,
              int32_t* topk_ids, float* topk_gates, int32_t* fallback_ids,
              void* stream);

/*
 * moe_router_topk -- the router network's scores and moe_route over them in
 * one launch (MACS §3.1: the router G scores every expert and Eq. 1 takes
 * the top k; the form of G is not given there: a bias-free linear map).
 *
 *   logits[t][j] = sum_h w_gate[j][h] * x[t][h]
 *
 * x             [T,H]  token features (dtype).
 * w_gate        [N,H]  router weights (dtype), one row of H per expert.
 * dtype         MOE_BF16: bf16 MFMA with fp32 accumulation; H must be a
 *               multiple of 64 and x and w_gate under 2^31 bytes each.
 *               MOE_F32: fp32 fused multiply-add in increasing h; H must be
 *               a multiple of 4.  Otherwise, and for N > 256, MOE_EUNSUP.
 * logits        f32[T,N]  out: the scores; may be NULL.
 * topk_ids, topk_gates, fallback_ids: as moe_route, and bit for bit what
 *               moe_route returns when given these scores.
 * Workspace of moe_router_workspace_size(T, N, H, dtype) bytes: holds one
 * control word per 32-token tile, which must be zero before the first use
 * (e.g. allocated zeroed); every call leaves them zero again.  For short
 * batches the H axis is split over several workgroups whose partial scores
 * are added in a fixed order; the split depends on the shape only, so the
 * scores are deterministic for a given shape, and may differ in the last
 * bits between batch sizes.
 * One launch on `stream`.
 */
size_t moe_router_workspace_size(int T, int N, int H, int dtype);
int moe_router_topk(const void* x, const void* w_gate, int T, int N, int H,
                    int k, int R, int dtype, float* logits, int32_t* topk_ids,
                    float* topk_gates, int32_t* fallback_ids, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * moe_expert_similarity -- the SERE similarity calibration (multi-image QA
 * write-up §4.2: expert activations on a small generic calibration set give,
 * once and offline, the per-layer matrix of Frobenius similarities that
 * moe_sere_reroute takes as `sim`).
 *
 *   sim[i][j] = <A_i, A_j>_F / (||A_i||_F ||A_j||_F),   sim[j][j] = 1,
 *
 * where A_j is row j of acts, i.e. the D values of expert j's matrix
 * flattened; a matrix of zeros has similarity 0 with every other one.  The
 * out_rows of an FFN pass that sends every calibration token to every
 * expert (expert_offsets = 0, T, 2T, ...; row_token = 0..T-1 for each
 * expert; k = N) are exactly acts [N, T*H].
 *
 * acts   [N, D]  dtype MOE_BF16 (bf16 MFMA; D a multiple of 64 and acts at
 *                most 2^31 bytes) or MOE_F32 (exact products summed in
 *                fp64; meant for small inputs).  N <= 128, else MOE_EUNSUP.
 * sim    f32[N, N]  out.
 * Workspace of moe_similarity_workspace_size(N, D, dtype) bytes (scratch
 * only; no initialisation).  The Gram matrix is accumulated in fp32 over
 * runs of at most 4096 products (bf16), then in fp64 in a fixed order:
 * deterministic.  Three launches on `stream`.
 */
size_t moe_similarity_workspace_size(int N, long long D, int dtype);
int moe_expert_similarity(const void* acts, int N, long long D, int dtype,
                          float* sim, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * moe_sere_reroute -- SERE similarity-guided re-routing (multi-image QA
 * write-up §4.1-§4.3), for decode batches.
 *
 * P is the union over the whole batch of every token's ranks 1..kprime.
 * For each secondary slot (rank > kprime) whose expert e is not in P, let
 * p* be the expert of P with the largest sim[e][p] (ties: lowest index).
 * The slot moves to p* iff sim[e][p*] > rho (fp32 compare) and
 * prot[e][p*] == 0; otherwise it keeps e.  Experts already in P never move.
 * Gates are not touched: a moved slot keeps its original rank's gate.
 *
 * topk_ids     i32[T,k]  moe_route's output.
 * sim          f32[N,N]  per-layer expert similarity, row = source expert.
 * prot         u8[N,N]   per-layer protection, same layout as sim; nonzero
 *                        forbids moving source e to target p.  A protected
 *                        expert has an all-ones row.  Must be non-NULL (pass
 *                        zeros for no protection).
 * slot_expert  i32[T,k]  out: expert of every slot after re-routing.
 * flags        u8[T,k]   out: MOE_FLAG_SERE on moved slots, else 0.
 * Requires 1 <= kprime <= k.  One workgroup; the union bitset and the
 * per-expert targets live in LDS.
 */
int moe_sere_reroute(const int32_t* topk_ids, int T, int N, int k, int kprime,
                     float rho, const float* sim, const uint8_t* prot,
                     int32_t* slot_expert, uint8_t* flags, void* stream);

/*
 * moe_capacity_assign -- MACS weighted load, modality-adaptive capacity and
 * re-route-else-drop (MACS §3.1 Eq. 3, §3.2 Eq. 5-6, §3.3 Eq. 7, §1 Fig. 1).
 *
 * Token weight (fixed point, MOE_WEIGHT_ONE = 1.0): text tokens 1; visual
 * tokens clamp(entropy_w, 0, 1) (NaN counts as 1), rounded half-to-even.
 * R_v = (sum of visual weights) / (sum of all weights), or 1/2 if the sum
 * is 0.  Capacity of expert j, each step one IEEE double operation:
 *   C_j = max(((gamma*T)*k)/N * (1 + (lam*m_j)*(R_v - 0.5)), 1.0)
 *   cap_q[j] = floor(C_j * MOE_WEIGHT_ONE)      (clamped at 2^62)
 * Round 0: each expert keeps its proposers, in increasing (token, slot)
 * order, while the inclusive running weight of all its proposers so far is
 * <= cap_q.  Rounds r = 1..R: a token with an unplaced overflowed slot
 * offers its lowest such slot to its rank k+r expert c when c had a
 * round-0 proposer, c/group == e/group for the slot's expert e, and the
 * token holds c in no slot; each expert admits the round's offers in token
 * order by the same prefix rule against its remaining capacity.  Slots
 * still unplaced after round R are dropped.  gamma = +inf disables
 * capacity (everything kept).
 *
 * topk_ids      i32[T,k]  router ranking (for MOE_FLAG_SERE).
 * slot_in       i32[T,k]  experts after SERE (or topk_ids when SERE is off);
 *                         may equal slot_out (in place).
 * fallback_ids  i32[T,R]  router ranks k+1..k+R; NULL allowed when R == 0.
 * is_visual     u8[T]     nonzero = visual token.
 * entropy_w     f32[T]    semantic weight of visual tokens (ignored for text).
 * modality      i8[N]     m_j in {+1 visual, -1 text, 0 shared}.
 * group         locality group size g (N = no restriction), 1 <= g <= N.
 * slot_out      i32[T,k]  out: final expert, -1 = dropped.
 * flags         u8[T,k]   out: MOE_FLAG_SERE | MOE_FLAG_MACS | MOE_FLAG_DROP.
 * load_q        i64[N]    out: admitted weight per expert.
 * cap_q         i64[N]    out: capacity per expert (INT64_MAX when off).
 * stats         i64[4]    out: {sum of weights, sum of visual weights,
 *                         dropped slots, MACS re-routed slots}.
 * r_v           f64[1]    out: effective visual ratio R_v.
 */
size_t moe_capacity_workspace_size(int T, int N, int k);
int moe_capacity_assign(const int32_t* topk_ids, const int32_t* slot_in,
                        const int32_t* fallback_ids, const uint8_t* is_visual,
                        const float* entropy_w, const int8_t* modality,
                        int T, int N, int k, int R, int group,
                        double gamma, double lam,
                        int32_t* slot_out, uint8_t* flags, int64_t* load_q,
                        int64_t* cap_q, int64_t* stats, double* r_v,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * moe_dispatch -- permutation of the kept slots into expert-major rows,
 * ordered by (token, slot) inside each expert; feeds the grouped FFN.
 * This is the hand-off of the multi-image QA write-up §4.2 (online
 * execution): the re-routed slots go straight to the fused expert FFN, the
 * grouping done by a counting scan rather than a sort; dropped slots
 * (MACS §1, Fig. 1) take no row.
 *
 * slot_expert     i32[T,k]   final experts, -1 = dropped.
 * expert_offsets  i32[N+1]   out: rows of expert j are
 *                            [expert_offsets[j], expert_offsets[j+1]);
 *                            expert_offsets[N] = M, the number of kept slots.
 * row_token       i32[T*k]   out: token of each row (first M valid).
 * row_slot        i32[T*k]   out: slot of each row (first M valid).
 * slot_row        i32[T,k]   out: row of each slot, -1 when dropped.
 */
size_t moe_dispatch_workspace_size(int T, int N, int k);
int moe_dispatch(const int32_t* slot_expert, int T, int N, int k,
                 int32_t* expert_offsets, int32_t* row_token,
                 int32_t* row_slot, int32_t* slot_row,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_entropy_weights -- semantic token weights from the entropy of each
 * visual token's features (MACS §3.2 Eq. 4-5): H(x_t) = Shannon entropy
 * (natural log) of softmax(x_t); H~ = (H - mu) / (sigma + eps) with mu and
 * the population standard deviation sigma of H over the batch's visual
 * tokens; w = 1 / (1 + exp(delta * H~)) for visual tokens, 1 for text
 * tokens.  The result is the entropy_w input of moe_capacity_assign.
 *
 * x          [T,H] element type `dtype` (the token features, e.g. the
 *            layer input).
 * is_visual  u8[T]   nonzero = visual token.
 * delta, eps finite, eps >= 0 (the page leaves both open).
 * entropy_w  f32[T]  out: w.
 * entropy    f32[T]  out: H per token; may be NULL.
 * Workspace of moe_entropy_workspace_size(T) bytes (scratch only; no
 * initialisation needed).  Two launches on `stream`.  Sums over tokens are
 * taken in a fixed order: results are deterministic.
 */
size_t moe_entropy_workspace_size(int T);
int moe_entropy_weights(const void* x, const uint8_t* is_visual, int T, int H,
                        int dtype, float delta, float eps, float* entropy_w,
                        float* entropy, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * moe_routing_fused -- moe_route, moe_sere_reroute (when kprime > 0),
 * moe_capacity_assign and moe_dispatch in ONE launch, for decode-sized
 * batches.  SERE write-up §4.3: the re-route operator is a
 * single fused kernel with no host round trip that feeds the fused MoE
 * directly; here the router and the capacity step join it.
 *
 * Every output has the meaning, layout and value that the four separate
 * calls give when run in order on the same inputs:
 *   topk_ids, topk_gates, fallback_ids      as moe_route;
 *   slot_sere  i32[T,k]  as moe_sere_reroute's slot_expert (required when
 *                        kprime > 0, unused and may be NULL when kprime == 0);
 *   slot_expert, flags, load_q, cap_q, stats, r_v
 *                        as moe_capacity_assign (flags carry MOE_FLAG_SERE);
 *   expert_offsets, row_token, row_slot, slot_row
 *                        as moe_dispatch.
 * kprime == 0 turns SERE off (sim and prot may then be NULL); gamma = +inf
 * turns capacity off.  The workspace holds control words: fill it with
 * zero bytes once before its first use; every call leaves it zero again.
 * The batch-wide steps run in one workgroup with every array in LDS, which
 * bounds the batch: moe_routing_workspace_size returns 0 for shapes the
 * fused launch does not cover (about T*k <= 4096 at N = 128, k = R = 8),
 * and moe_routing_fused returns MOE_EUNSUP for them; the separate calls
 * cover every shape.  A batch of at most 8 tokens and 64 slots (k <= 8,
 * R <= 8, N <= 256) is routed by a single workgroup from start to end; the
 * outputs are the same.
 * Errors: as the separate calls, plus MOE_EUNSUP as above.
 */
size_t moe_routing_workspace_size(int T, int N, int k, int R);
int moe_routing_fused(const float* logits, const uint8_t* is_visual,
                      const float* entropy_w, const int8_t* modality,
                      const float* sim, const uint8_t* prot,
                      int T, int N, int k, int R, int kprime, float rho,
                      int group, double gamma, double lam,
                      int32_t* topk_ids, float* topk_gates,
                      int32_t* fallback_ids, int32_t* slot_sere,
                      int32_t* slot_expert, uint8_t* flags, int64_t* load_q,
                      int64_t* cap_q, int64_t* stats, double* r_v,
                      int32_t* expert_offsets, int32_t* row_token,
                      int32_t* row_slot, int32_t* slot_row,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_ffn -- grouped SwiGLU expert FFN over the dispatched rows
 * (MACS §3.1 Eq. 1, E_j(x) of every kept token-expert pair): for row r of
 * expert j with token t = row_token[r],
 *   h[r]        = silu(W1_j x_t) * (W3_j x_t),   silu(a) = a / (1 + e^-a)
 *   out_rows[r] = W2_j h[r]
 * The rows of x are gathered inside the GEMM; no permuted copy of x is made.
 * M = expert_offsets[N] rows are computed; M is read on the device.
 *
 * x               [T,H]      activations (dtype).
 * row_token       i32[T*k], expert_offsets i32[N+1]: moe_dispatch output.
 * w13             [N,2I,H]   per expert: gate rows W1 (0..I-1), then up
 *                            rows W3 (I..2I-1); each row H contiguous.
 * w2              [N,H,I]    per expert down projection, each row I
 *                            contiguous.
 * out_rows        [T*k,H]    out: un-gated expert outputs, first M rows.
 * dtype           MOE_F32 (fp32 FMA) or MOE_BF16 (bf16 MFMA with fp32
 *                 accumulation; h and out_rows are rounded to bf16), or
 *                 MOE_BF16_PANELS: MOE_BF16 arithmetic, with w13 and w2 as
 *                 moe_pack_weights wrote them; the results equal those of
 *                 MOE_BF16 on the unpacked weights bit for bit, except for
 *                 decode batches of at most 16 dispatch rows (T*k <= 16)
 *                 whose reduction length (H for the gate-up half, I for the
 *                 down half) is 256, 512, 768, 1024 or 2048 (gate-up also
 *                 T <= 8): those run as GEMVs with fp32 dot products of bf16
 *                 pairs summed in another order, within the bf16 rounding
 *                 of the row layout's results (deterministic run to run).
 * The workspace holds h ([T*k, I] of dtype).
 * Shapes: the bf16 formats need H % 256 == 0, I % 128 == 0, x of at most 2 GiB
 * (T*H*2 <= 2^31 bytes) and one expert's w13 under 4 GiB (I*H*4 < 2^32
 * bytes); MOE_F32 needs H % 4 == 0 and I % 4 == 0; otherwise MOE_EUNSUP.
 *
 * moe_ffn_gate_up and moe_ffn_down are the two halves of moe_expert_ffn
 * (same arguments, h passed explicitly, [T*k, I] of dtype), for callers that
 * schedule or time them separately.
 */
size_t moe_ffn_workspace_size(int T, int N, int k, int H, int I, int dtype);
int moe_expert_ffn(const void* x, const int32_t* row_token,
                   const int32_t* expert_offsets, const void* w13,
                   const void* w2, int T, int N, int k, int H, int I,
                   int dtype, void* out_rows,
                   void* workspace, size_t workspace_bytes, void* stream);
int moe_ffn_gate_up(const void* x, const int32_t* row_token,
                    const int32_t* expert_offsets, const void* w13,
                    int T, int N, int k, int H, int I, int dtype, void* h,
                    void* stream);
int moe_ffn_down(const void* h, const int32_t* expert_offsets, const void* w2,
                 int T, int N, int k, int H, int I, int dtype, void* out_rows,
                 void* stream);

/*
 * moe_expert_ffn_combine -- moe_expert_ffn followed by moe_combine (MACS
 * §3.1 Eq. 1, the whole sum over the kept experts) in one call: out_rows
 * and y equal those of the two calls bit for bit.  For decode batches on
 * packed weights whose down half runs as a GEMV (dtype MOE_BF16_PANELS,
 * T*k <= 16, I as listed above) the combine is folded into that GEMV: the
 * last workgroup to finish a group of 32 output columns, told by a ticket
 * in the workspace, combines those columns of every token, which saves a
 * launch and a pass over out_rows; other calls enqueue the two.
 *
 * Arguments: those of moe_expert_ffn, plus slot_row i32[T,k] (moe_dispatch
 * output) and topk_gates f32[T,k] as for moe_combine, and y [T,H] out
 * (dtype; bf16 for the packed formats).  The workspace holds the tickets
 * (H/32 words, rounded up to 256 bytes) and then h; its size is
 * moe_ffn_combine_workspace_size(), and the ticket words must be filled
 * with zero bytes once before the first use (every call leaves them zero).
 * Shapes as moe_expert_ffn, and H % 8 == 0; errors as moe_expert_ffn.
 *
 * moe_ffn_down_combine is the second half (moe_ffn_down then moe_combine,
 * h passed explicitly, [T*k, I] of dtype, with the tickets at the start of
 * its workspace: moe_ffn_combine_workspace_size() bytes suffice), for
 * callers that schedule or time the halves separately.
 */
size_t moe_ffn_combine_workspace_size(int T, int N, int k, int H, int I, int dtype);
int moe_expert_ffn_combine(const void* x, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* w13,
                           const void* w2, const int32_t* slot_row,
                           const float* topk_gates, int T, int N, int k, int H,
                           int I, int dtype, void* out_rows, void* y,
                           void* workspace, size_t workspace_bytes,
                           void* stream);
int moe_ffn_down_combine(const void* h, const int32_t* row_token,
                         const int32_t* expert_offsets, const void* w2,
                         const int32_t* slot_row, const float* topk_gates, int T,
                         int N, int k, int H, int I, int dtype, void* out_rows,
                         void* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * moe_pack_weights -- the expert weights in the panel layout that the
 * expert FFN streams from HBM in whole 16 KB blocks, each wave's share of a
 * block loaded straight into its MFMA operand registers (dtype
 * MOE_BF16_PANELS), written once when the weights are loaded.  The FFN of a
 * decode step reads every active expert's weights once (MACS §3.1 Eq. 1,
 * E_j), so its speed is the rate at which those blocks stream.
 *
 * Layout, per expert (K = H for w13, I for w2): the rows of the matrix in
 * tile order -- w13: for each 16 h columns c0 .. c0+15 (c0 = 0, 16, ...)
 * the 16 gate rows c0 .. c0+15, then the 16 up rows I+c0 .. I+c0+15; w2:
 * rows 0 .. H-1 -- are cut into panels of 128 rows, and panel P is stored
 * as K/64 consecutive 16 KB blocks, block b holding elements 64b .. 64b+63
 * of the panel's rows in the operand order of the 32x32x16 bf16 MFMA: for
 * each row group G = 0..3 (32 rows) and K step s = 0..3 (16 elements), 64
 * chunks of 8 elements, chunk l being elements 64b + 16s + 8(l/32) .. +7 of
 * group row l % 32.  So element (t, kk) of the tile-order matrix (kk % 8 ==
 * 0 starts a chunk) is at byte
 *   (P * K/64 + kk/64) * 16384
 *     + ((G * 4 + (kk % 64)/16) * 64 + ((kk % 16)/8) * 32 + t % 32) * 16,
 * P = t / 128, G = (t % 128) / 32, from the start of the expert's block,
 * whose size and position are those of the row layout.
 *
 * w13, w2           [N,2I,H], [N,H,I] bf16 in the row layout (device).
 * w13_panels,       out: the same sizes, packed (device; must not alias
 * w2_panels         the inputs).  Either pair may be NULL to skip it.
 * dtype             MOE_BF16 (the element type); MOE_F32 and
 *                   MOE_BF16_PANELS give MOE_EUNSUP.
 * Shapes as the bf16 expert FFN (H % 256 == 0, I % 128 == 0); errors:
 * MOE_EINVAL for bad sizes, a pointer given without its partner, or
 * aliasing; MOE_EUNSUP for other shapes; MOE_EHIP for launch failures.
 */
int moe_pack_weights(const void* w13, const void* w2, int N, int H, int I,
                     int dtype, void* w13_panels, void* w2_panels, void* stream);

/*
 * moe_expert_ffn_noalloc -- moe_expert_ffn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, same kernels and the
 * same results bit for bit, minus the workspace.  h is kept in a fixed
 * device-resident buffer of MOE_FFN_NOALLOC_MAX_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * allocates and frees nothing.
 * Limit: moe_ffn_workspace_size(T, N, k, H, I, dtype) must not exceed
 * MOE_FFN_NOALLOC_MAX_BYTES (32 MiB: every decode batch of the shapes
 * above, e.g. T*k*I*2 bytes of bf16 h up to 16 Mi elements), else the call
 * returns MOE_ESCRATCH and enqueues nothing.
 * Every call on one GPU uses that GPU's one buffer: calls that may overlap
 * on one GPU (several streams, or several host threads) race and must be
 * serialised by the caller.  Nothing in the buffer needs to start at zero.
 * Errors: as moe_expert_ffn, plus MOE_ESCRATCH, and MOE_EHIP when the
 * runtime cannot report the buffer's device address.
 */
#define MOE_FFN_NOALLOC_MAX_BYTES (32u << 20)
int moe_expert_ffn_noalloc(const void* x, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* w13,
                           const void* w2, int T, int N, int k, int H, int I,
                           int dtype, void* out_rows, void* stream);

/*
 * moe_combine -- gate-weighted combine (MACS §3.1 Eq. 1):
 *   y[t] = sum over s = 0..k-1 with slot_row[t,s] >= 0 of
 *          topk_gates[t,s] * out_rows[slot_row[t,s]]
 * accumulated in fp32 in slot order, then stored in dtype.  Dropped slots
 * contribute nothing and the remaining gates are not renormalised.
 *
 * out_rows [T*k,H] (dtype), slot_row i32[T,k], topk_gates f32[T,k],
 * y [T,H] out (dtype).  Requires H % 8 == 0.
 */
int moe_combine(const void* out_rows, const int32_t* slot_row,
                const float* topk_gates, int T, int k, int H, int dtype,
                void* y, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MACS_H */
