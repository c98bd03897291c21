/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path: deterministic no-drop
 * top-k routing or routing replay, stable dispatch into expert-contiguous rows, grouped
 * SwiGLU expert GEMMs, the slot-order weighted combine, and per-expert load statistics.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers the caller owns (e.g. torch tensors). The
 *    library only borrows them until the work it enqueued has run. It never allocates,
 *    never frees, never synchronises the host, and enqueues everything on `stream`
 *    (a hipStream_t; NULL = the null stream).
 *  - Layouts are row-major and dense. bf16 tensors hold bfloat16 bit patterns (uint16).
 *    Weight layouts follow the Linear convention [out, in]: w_router[E,d],
 *    w13[E,2I,d] (gate rows 0..I-1 then up rows I..2I-1), w2[E,d,I].
 *  - Host-checkable errors (null required pointer, bad sizes or dtype, small workspace)
 *    return a status and enqueue nothing. Data errors found on the device (bad replay
 *    ids, non-finite logits/weights, bad cu_seqlens) are OR-ed into the caller's int32
 *    *d_err (device memory; the library never clears it, the caller zeroes it before the
 *    first call). When *d_err != 0 the outputs are unspecified, but every kernel stays
 *    inside its buffers. d_err may be NULL (no report).
 *  - Determinism: every output is bitwise identical from run to run. Every per-token
 *    output row (topk_idx, topk_w, x_perm/h/y rows reached through inv, out) is bitwise
 *    independent of T, of the other tokens and of the launch shape (tile_m), because
 *    every reduction has one fixed order that nothing but the reduced length decides.
 *  - Reentrant; no global mutable state. No C++ exception crosses this boundary.
 *
 * Sources (page title, section):
 *  [MM]  "0 train-infer mismatch for Open-weight MoE RL in Open-source code",
 *        "Matrix multiplication: the same reduction along K" (fixed-K products).
 *  [SW]  same page, "SwiGLU: rounding after the multiply".
 *  [RT]  same page, "The router: matching expert ids and weights".
 *  [EX]  same page, "The experts: keeping the route weight inside the accumulator" and
 *        "Sharding the experts".
 *  [TRR] same page, "Total Router Recall"; "Hash and learned expert routing".
 *  [SEL] same page, "Selecting sparse-attention positions" (lower position wins ties).
 *  [GLM] same page, "Choosing GLM's eight experts" (sigmoid scores, FP32 correction bias
 *        for the choice only, weights from the pre-bias scores normalised in FP32, the
 *        factor 2.5 applied inside the expert kernel).
 *  [HL]  same page, "Hash and learned expert routing" (frozen token-id -> experts table;
 *        sqrt-softplus scores with the correction bias in the learned layers).
 *  [RP]  "RoutePack: Expert Placement and Attention-Aware Data Packing for MoE
 *        Reinforcement Learning", Sec. 2.1 eq. (1), Sec. 3.3.
 *  [HA]  "HARTS: Efficient Agentic Reinforcement Learning for Hybrid-Attention Models
 *        over Arbitrary Rollout Trees", eq. (20) and "MoE execution and objectives".
 */
#ifndef MOE_LAYER_ROUTING_AMD_MOE_H
#define MOE_LAYER_ROUTING_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_E_NULLPTR = 1,   /* a required pointer is NULL */
    MOE_E_SHAPE = 2,     /* a size is outside the supported range */
    MOE_E_DTYPE = 3,     /* dtype is not MOE_F32 or MOE_BF16 */
    MOE_E_WORKSPACE = 4, /* workspace NULL or smaller than moe_workspace_size() */
    MOE_E_LAUNCH = 5,    /* the HIP runtime rejected a launch or an event record */
    MOE_E_SCRATCH = 6    /* moe_forward_noalloc: the layer needs more than the static scratch */
} moe_status;

/* bits OR-ed into *d_err by device-side checks */
enum {
    MOE_DERR_IDX_RANGE = 1, /* an expert id outside [0, E) */
    MOE_DERR_IDX_DUP = 2,   /* the same expert twice in one token's replayed row */
    MOE_DERR_NONFINITE = 4, /* a NaN/Inf router logit or replayed weight */
    MOE_DERR_SEQLENS = 8,   /* cu_seqlens not 0 = c_0 <= c_1 <= ... <= c_S = T */
    MOE_DERR_SLOTMAP = 16   /* slot_of_expert is not a permutation of 0..E-1 */
};

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Problem sizes. Supported: 0 <= T, T*k < 2^31; 1 <= E <= 256; 1 <= k <= min(E, 8);
 * 64 <= d <= 16384 and 64 <= inter <= 16384, both multiples of 64.
 * dtype is the storage type of x, w_router, w13, w2, x_perm, h and out; logits,
 * probabilities, routing weights, y and all accumulators are FP32.
 * tile_m: 0 selects the grouped-GEMM token-tile height automatically; 16, 32, 64, 128 or
 * 256 forces it. Results are bitwise identical for every value (launch shape only). */
typedef struct moe_dims {
    int64_t T;
    int32_t d;
    int32_t E;
    int32_t k;
    int32_t inter;
    int32_t dtype;
    int32_t tile_m;
} moe_dims;

/* Bytes of device workspace any entry point needs for `dims` (the largest of them; it
 * serves moe_forward as well). Pure host function; returns 0 for invalid dims. The
 * workspace holds small per-block partials and tile lists, never a full activation. */
size_t moe_workspace_size(const moe_dims *dims);

/* Token-tile height (rows of the permuted activation per GEMM block) that every grouped
 * GEMM of `dims` uses: dims->tile_m when it is nonzero, else the automatic choice. The
 * automatic choice is 256 from 128 mean rows per expert (T*k/E, rounded down) on; below
 * that it is the smallest of 16, 32, 64, 128 that holds min(T, ceil(1.5 T*k/E)) rows, so
 * that most active experts take a single token tile. Results do not depend on it (launch
 * shape only). Pure host function; returns 0 for invalid dims. */
int32_t moe_tile_height(const moe_dims *dims);

/* Human-readable name of a status code (static string). */
const char *moe_status_string(moe_status s);

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/* Router [MM][RT][SEL][HA].
 *   logits[t,e] = sum_c x[t,c] w_router[e,c] (+ logit_bias[e]): FP32 accumulation over c
 *     in one fixed order for every T (no M-dependent split of K);
 *   probabilities p[t,:] = FP32 softmax over all E logits (shifted by the largest);
 *   slots: the k experts first in the order (logit desc, id asc), slot 0 = largest;
 *   topk_w[t,j] = p[t,idx_j] / s with s = ((p_idx0 + p_idx1) + ...) left to right;
 *   prob_mass[e] = sum_t q_t p[t,e] (q_t = token_mult[t], or 1 when token_mult is NULL),
 *     summed in a fixed order.
 * x [T,d] (dtype), w_router [E,d] (dtype), logit_bias [E] f32 or NULL,
 * topk_idx [T,k] i32 and topk_w [T,k] f32 (outputs, required),
 * logits [T,E] f32 output or NULL (then held in the workspace),
 * prob_mass [E] f32 output or NULL, token_mult [T] i32 or NULL.
 * Non-finite logits set MOE_DERR_NONFINITE. */
moe_status moe_route(const moe_dims *dims, const void *x, const void *w_router,
                     const float *logit_bias, int32_t *topk_idx, float *topk_w,
                     float *logits, float *prob_mass, const int32_t *token_mult,
                     int32_t *d_err, void *workspace, size_t workspace_bytes, void *stream);

/* Score function of a router [RT][GLM][HL]. */
typedef enum moe_score_fn {
    MOE_SCORE_SOFTMAX = 0,      /* p = FP32 softmax over the E logits (as moe_route) */
    MOE_SCORE_SIGMOID = 1,      /* s = 1 / (1 + exp(-l)) */
    MOE_SCORE_SQRT_SOFTPLUS = 2 /* s = sqrt(log(1 + exp(l))) */
} moe_score_fn;

/* Router variant options (all device pointers; NULL = absent).
 *  score_fn   moe_score_fn. The sigmoid and sqrt-softplus scores are the functions
 *             evaluated in FP64 and rounded once to FP32, so that any two correct
 *             implementations agree on the score (and on the choice) bit for bit except
 *             where the FP64 value lies within an FP64 rounding error of a point halfway
 *             between two FP32 numbers.
 *  corr_bias  [E] f32: correction bias, added in FP32 to each score to choose the
 *             experts and nowhere else [GLM]. Only with SIGMOID / SQRT_SOFTPLUS
 *             (MOE_E_SHAPE with SOFTMAX, whose choice keys on the logits).
 *  hash_table [vocab, k] i32: frozen token-id -> expert table [HL]; with it, slot j of
 *             token t is hash_table[token_ids[t] * k + j] (the table's order; the bias
 *             is not used) and the logits only set the weights. token_ids [T] i32 is then
 *             required and vocab >= 1. A token id outside [0, vocab) sets
 *             MOE_DERR_IDX_RANGE and gives the row ids -1 and weights 0; a table id
 *             outside [0, E) or repeated within the row sets MOE_DERR_IDX_RANGE /
 *             MOE_DERR_IDX_DUP and gives the row weights 0 (the ids pass through).
 *  lse        [T] f32 output: log-sum-exp of each token's logits, max + log(sum exp(l -
 *             max)), FP32 (the router z-loss input of moe_objectives). */
typedef struct moe_router_opts {
    int32_t score_fn;
    const float *corr_bias;
    const int32_t *hash_table;
    const int32_t *token_ids;
    int32_t vocab;
    float *lse;
} moe_router_opts;

/* Router variants [RT][GLM][HL][HA]: logits as moe_route (same kernel, same bits), then
 * per token, with v[e] = softmax probability (SOFTMAX) or score s[e] (otherwise):
 *   choice: SOFTMAX without a table: as moe_route (logit desc, id asc); SIGMOID /
 *     SQRT_SOFTPLUS without a table: the k experts first in the order (s[e] +
 *     corr_bias[e] desc, id asc), slot 0 = largest; with a table: the table's row;
 *   topk_w[t,j] = v[idx_j] / ((v[idx_0] + v[idx_1]) + ...), FP32, left to right: the
 *     bias never enters a weight;
 *   prob_mass[e] = sum_t q_t prob[t,e], prob = p (SOFTMAX) or s[e] / sum_e' s[e']
 *     (the scores normalised over all E experts), summed in a fixed order.
 * With score_fn SOFTMAX and neither bias nor table, every output is bitwise moe_route's.
 * opts NULL = SOFTMAX with no options. Other arguments as moe_route. */
moe_status moe_route_scored(const moe_dims *dims, const moe_router_opts *opts, const void *x,
                            const void *w_router, const float *logit_bias, int32_t *topk_idx,
                            float *topk_w, float *logits, float *prob_mass,
                            const int32_t *token_mult, int32_t *d_err, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Routing replay [TRR][RP]: the caller's expert ids (int32) and normalised FP32 weights,
 * one per token per slot, are validated and passed through unchanged: no
 * renormalisation, no reordering. idx_in/w_in [T,k] -> topk_idx/topk_w [T,k]; the output
 * may alias the input. Ids outside [0,E) set MOE_DERR_IDX_RANGE, an id repeated within a
 * row sets MOE_DERR_IDX_DUP, a non-finite weight sets MOE_DERR_NONFINITE. */
moe_status moe_route_replay(const moe_dims *dims, const int32_t *idx_in, const float *w_in,
                            int32_t *topk_idx, float *topk_w, int32_t *d_err, void *stream);

/* Dispatch and load statistics [RP][HA]. Flat assignments a = t*k + j are
 * counting-sorted by expert, stably (increasing a inside each expert's segment):
 *   counts[e] = #{a : topk_idx[a] == e};  offsets[0] = 0, offsets[e+1] = offsets[e] +
 *   counts[e];  perm[p] = a and inv[a] = p for the sorted position p;
 *   x_perm[p,:] = x[perm[p] / k, :] (exact copy; NULL skips the gather);
 *   seq_counts[s,e] = assignments to e from tokens [cu_seqlens[s], cu_seqlens[s+1])
 *     (cu_seqlens [S+1] i32 and seq_counts [S,E] i32, both NULL or both given);
 *   weighted_counts[e] = sum_t q_t [e in topk_idx[t]] (int64; q_t = 1 if token_mult is
 *     NULL).
 * topk_idx [T,k] i32, x [T,d] dtype, x_perm [T*k,d] dtype, perm/inv [T*k] i32,
 * counts [E] i32, offsets [E+1] i32 (all outputs except topk_idx/x/token_mult/cu).
 * Ids outside [0,E) set MOE_DERR_IDX_RANGE and are left out (their inv is -1). */
moe_status moe_permute(const moe_dims *dims, const int32_t *topk_idx, const void *x,
                       void *x_perm, int32_t *perm, int32_t *inv, int32_t *counts,
                       int32_t *offsets, const int32_t *cu_seqlens, int32_t num_seqs,
                       int32_t *seq_counts, const int32_t *token_mult,
                       int64_t *weighted_counts, int32_t *d_err, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Dispatch with a logical->physical expert placement [RP] (RoutePack, Sec. 3 "State-
 * consistent materialization": routing stays in logical expert ids; the dispatcher sends
 * logical expert e to physical slot slot_of_expert[e]). The same as moe_permute with
 * every id e replaced by its slot: counts, offsets, seq_counts and weighted_counts are
 * per physical slot, segments are in slot order, and x_perm rows of slot v are the rows
 * routed to the expert placed there; the expert weights handed to moe_grouped_ffn must
 * be stored in slot order (slot v holds the weights of the expert e with
 * slot_of_expert[e] == v). slot_of_expert [E] i32, device. A map that is not a
 * permutation of 0..E-1 sets MOE_DERR_SLOTMAP (an entry outside [0,E) also drops the
 * expert's rows, like an invalid id). Every output row of the layer is then bitwise the
 * one of the identity placement. */
moe_status moe_permute_placed(const moe_dims *dims, const int32_t *topk_idx,
                              const int32_t *slot_of_expert, const void *x, void *x_perm,
                              int32_t *perm, int32_t *inv, int32_t *counts, int32_t *offsets,
                              const int32_t *cu_seqlens, int32_t num_seqs, int32_t *seq_counts,
                              const int32_t *token_mult, int64_t *weighted_counts,
                              int32_t *d_err, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Layer-local LPT expert placement [RP] (RoutePack, Sec. 3, Algorithm 1): host function,
 * host pointers, no GPU work. loads [E] int64 >= 0 (aggregate routed assignments per
 * logical expert, e.g. counts summed over an optimizer step), P ranks of H = E / P slots
 * each (slot v belongs to rank v / H). Experts are taken in order of (load descending, id
 * ascending); each goes to the rank with the least assigned load among the ranks that
 * still have a free slot (equal loads: the lower rank), into that rank's next free slot
 * (rank p's slots fill in order p*H, p*H+1, ...). Writes slot_of_expert [E] (a
 * permutation of 0..E-1); rank_load [P] (NULL: not written) = sum of the loads placed on
 * each rank; cv (NULL: not written) = population standard deviation of rank_load over its
 * mean (0 when the mean is 0). MOE_E_SHAPE: E < 1, P < 1, E % P != 0, E > 256 or a
 * negative load; MOE_E_NULLPTR: loads or slot_of_expert NULL. */
moe_status moe_place_lpt(const int64_t *loads, int32_t E, int32_t P, int32_t *slot_of_expert,
                         int64_t *rank_load, double *cv);

/* Grouped SwiGLU experts [MM][SW][EX]. For every expert e and row p in
 * [offsets[e], offsets[e+1]):
 *   g_i = sum_c x_perm[p,c] w13[e,i,c],  u_i = sum_c x_perm[p,c] w13[e,I+i,c]   (FP32)
 *   h[p,i] = round_dtype( silu(g_i) * u_i ),  silu(g) = g / (1 + exp(-g)), in FP32,
 *            rounded once (bf16 round-to-nearest-even; identity for f32);
 *   y[p,o] = sum_i h[p,i] w2[e,o,i]   (FP32, stored FP32).
 * Each sum runs over its K in one fixed order (bf16: 16x16x32 MFMA steps in increasing
 * K; f32: 16x16x4 steps) whatever the segment lengths or tile_m.
 * x_perm [T*k,d], w13 [E,2I,d], w2 [E,d,I], h [T*k,I] (all dtype), y [T*k,d] f32,
 * offsets [E+1] i32 (device; read on the device only). Rows past offsets[E] are
 * untouched. */
moe_status moe_grouped_ffn(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                           const void *w13, const void *w2, void *h, float *y,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Weighted combine [EX][RT]:
 *   out[t,o] = round_dtype( ((0 + w_0 y_0) + w_1 y_1) + ... )  over slots j = 0..k-1,
 * where w_j = topk_w[t,j] and y_j = y[inv[t*k+j], o]; each product and sum in FP32, in
 * slot order, one final rounding. y [T*k,d] f32, inv [T*k] i32, topk_w [T,k] f32,
 * out [T,d] dtype. */
moe_status moe_combine(const moe_dims *dims, const float *y, const int32_t *inv,
                       const float *topk_w, void *out, void *stream);

/* Weighted combine with a routed scaling factor [GLM]: the factor multiplies the FP32
 * slot-order sum before the one rounding,
 *   out[t,o] = round_dtype( routed_scale * (((0 + w_0 y_0) + w_1 y_1) + ...) ).
 * routed_scale 1 gives moe_combine's bits (a multiplication by 1 is exact); it must be
 * finite (else MOE_E_SHAPE). */
moe_status moe_combine_scaled(const moe_dims *dims, const float *y, const int32_t *inv,
                              const float *topk_w, float routed_scale, void *out,
                              void *stream);

/* Objective statistics of one routed batch [HA] (HARTS, eq. (20) and "MoE execution and
 * objectives": the multiplicity q_t of a compact token weights its router z-loss term, the
 * probability mass and assignment counts of the load-balancing loss, and the counts of
 * the expert-bias update). Device inputs, written by moe_route_scored / moe_permute:
 *   lse [T] f32 or NULL, token_mult [T] i32 or NULL (q_t = 1), weighted_counts [E] i64 or
 *   NULL, prob_mass [E] f32 or NULL; slot_of_expert [E] i32 or NULL: when the counts
 *   came from moe_permute_placed, the map that placed them (the mass and the bias are in
 *   logical expert order; the counts are read as C_e = weighted_counts[slot_of_expert[e]]).
 * Writes out [3] f64 (device):
 *   out[0] = z_loss = (1/S) sum_t q_t lse_t^2 (0 if lse is NULL or S = 0), where
 *            S = sum_t q_t is the number of semantic token positions;
 *   out[1] = aux_loss = E / (k S^2) sum_e C_e M_e, i.e. E sum_e (C_e / (k S)) (M_e / S)
 *            (0 if weighted_counts or prob_mass is NULL, or S = 0);
 *   out[2] = S.
 * Every sum is FP64 in a fixed order. Unscaled: the caller multiplies by its coefficients.
 * corr_bias [E] f32 (NULL: not touched) is updated in place with the sign rule: with the
 * mean load Cbar = sum_e C_e / E, bias[e] += bias_rate if C_e < Cbar, -= bias_rate if
 * C_e > Cbar, unchanged if equal (compared exactly in integers; requires
 * weighted_counts). A slot_of_expert entry outside [0, E) sets MOE_DERR_SLOTMAP. */
moe_status moe_objectives(const moe_dims *dims, const float *lse, const int32_t *token_mult,
                          const int64_t *weighted_counts, const float *prob_mass,
                          const int32_t *slot_of_expert, float bias_rate, float *corr_bias,
                          double *out, int32_t *d_err, void *stream);

/* Expert-parallel output of the layer, emulated on one device [EX] ("Sharding the
 * experts"; the shared-expert passage of "The experts: keeping the route weight inside the
 * accumulator"). R = ranks (1 <= R <= 16, R divides E) each own E/R consecutive physical
 * slots; the physical slot of routed id e is slot_of_expert[e] (identity when NULL).
 *  partial_r[t,o] = round_dtype( routed_scale * acc_r + y_shared[r,t,o] ), where
 *    acc_r = ((0 + c_0) + c_1) + ... over the slots j = 0..k-1 in slot order, FP32, with
 *    c_j = w_j y[inv[t*k+j], o] when slot j's expert lives on rank r and an exact 0
 *    otherwise (y_shared NULL: no shared expert; routed_scale 0 means 1);
 *  out[t,o] = round_dtype( pairwise FP64 tree over partial_0 .. partial_{R-1} ): adjacent
 *    pairs added in FP64, an odd last contributor carried to the next level unchanged,
 *    until one value remains (8 ranks: three levels; 16: four), rounded once (bf16 round
 *    to nearest even, directly from FP64).
 * y [T*k,d] f32, inv [T*k] i32, topk_w [T,k] f32, topk_idx [T,k] i32 (logical ids; an id
 * outside [0,E) belongs to no rank), slot_of_expert [E] i32 or NULL, y_shared [R,T,d] f32
 * or NULL, partials [R,T,d] dtype output or NULL, out [T,d] dtype. With R = 1 and no shared
 * expert, out is moe_combine_scaled's, bit for bit. MOE_E_SHAPE for a bad R or a
 * non-finite routed_scale. */
moe_status moe_combine_ranks(const moe_dims *dims, int32_t ranks, const float *y,
                             const int32_t *inv, const float *topk_w, const int32_t *topk_idx,
                             const int32_t *slot_of_expert, const float *y_shared,
                             float routed_scale, void *partials, void *out, void *stream);

/* The shared expert sharded over R ranks along its inter dimension [MM][SW][EX]: rank r
 * holds gate/up rows w13_shared[r] = [2*Is/R, d] (its gate rows, then its up rows) and
 * down columns w2_shared[r] = [d, Is/R] (Is = inter_shared), and computes for every token
 *   h_shared[r,t,i] = round_dtype( silu(g_i) * u_i ),  g, u = fixed-K FP32 dot products of
 *                     x[t] with its gate / up rows;
 *   y_shared[r,t,o] = sum_i h_shared[r,t,i] w2_shared[r,o,i]   (FP32, fixed K order),
 * the same fixed-K grouped GEMMs as the routed experts (every row is bitwise independent of
 * T). x [T,d] dtype (< 4 GiB), h_shared [R,T,Is/R] dtype, y_shared [R,T,d] f32.
 * Supported: 1 <= R <= 16, Is % R == 0, Is/R a multiple of 64 in [64, 16384], T*R < 2^31.
 * Workspace: moe_shared_workspace_size() bytes (0 for invalid arguments). */
size_t moe_shared_workspace_size(const moe_dims *dims, int32_t ranks, int32_t inter_shared);
moe_status moe_shared_ffn(const moe_dims *dims, int32_t ranks, int32_t inter_shared,
                          const void *x, const void *w13_shared, const void *w2_shared,
                          void *h_shared, float *y_shared, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Everything moe_forward needs. Replay mode iff idx_in != NULL (then w_in is required
 * and w_router/logit_bias/logits/prob_mass are ignored); router mode otherwise.
 * Required: x, w13, w2, out, topk_idx, topk_w, counts, offsets, perm, inv, h, y,
 * workspace. Optional (NULL = not produced / not used): logit_bias, logits, prob_mass,
 * token_mult, cu_seqlens + seq_counts, weighted_counts, d_err, prof_events, x_perm.
 * x_perm NULL: the dispatch gather is fused into the gate/up GEMM, which reads token rows
 * of x through perm (identical results; x must then be smaller than 4 GiB, else
 * MOE_E_SHAPE).
 * prof_events: NULL, or three hipEvent_t handles recorded on `stream` before the
 * gate/up GEMM, between the two GEMMs and after the down GEMM (for timing). A bf16 layer
 * with at most 16 expert rows (T*k <= 16), d/16 >= 256 and inter a multiple of 768 runs
 * the down GEMM and the plain combine as one launch (same outputs, y included); the third
 * event then follows that launch. When such a layer also has T <= 2, E <= 128, the plain
 * softmax router (router NULL or softmax, no hash table), no placement map and x_perm NULL,
 * the gate/up launch routes the tokens itself (every output as from the separate routing
 * steps, bit for bit), so the first two events bracket routing and gate/up together.
 * Events recorded between the launches delay each following launch by a few
 * microseconds; decode-sized steps are best timed without them.
 * slot_of_expert: NULL, or a device placement map as in moe_permute_placed (w13 and w2
 * then hold the experts in slot order; counts/offsets/statistics are per slot; topk_idx
 * stays in logical ids).
 * router: NULL, or the router variant of moe_route_scored (router mode only).
 * routed_scale: the combine's routed scaling factor as in moe_combine_scaled; 0 means 1
 * (no factor), so a zero-initialised struct keeps moe_combine's bits.
 * ranks: 0 = the plain combine; R >= 1 = the output is moe_combine_ranks' (partials
 * optional), with the shared expert of moe_shared_ffn when w13_shared is not NULL (then
 * w2_shared, h_shared, y_shared and a shared_workspace of moe_shared_workspace_size()
 * bytes are required). */
typedef struct moe_forward_args {
    const void *x;
    const void *w_router;
    const float *logit_bias;
    const int32_t *idx_in;
    const float *w_in;
    const void *w13;
    const void *w2;
    const int32_t *token_mult;
    const int32_t *cu_seqlens;
    int32_t num_seqs;
    void *out;
    int32_t *topk_idx;
    float *topk_w;
    float *logits;
    float *prob_mass;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv;
    int32_t *seq_counts;
    int64_t *weighted_counts;
    void *x_perm;
    void *h;
    float *y;
    int32_t *d_err;
    void *workspace;
    size_t workspace_bytes;
    void *const *prof_events;
    const int32_t *slot_of_expert; /* NULL: identity placement; else as moe_permute_placed */
    const moe_router_opts *router; /* host pointer; NULL: softmax router as moe_route */
    float routed_scale;            /* 0 or 1: no factor */
    int32_t ranks;                 /* 0: plain combine; R: rank partials + FP64 tree */
    void *partials;                /* [R,T,d] dtype or NULL */
    const void *w13_shared;        /* [R, 2*inter_shared/R, d] or NULL: no shared expert */
    const void *w2_shared;         /* [R, d, inter_shared/R] */
    int32_t inter_shared;
    void *h_shared;                /* [R, T, inter_shared/R] dtype */
    float *y_shared;               /* [R, T, d] f32 */
    void *shared_workspace;
    size_t shared_workspace_bytes;
    /* NULL, or FP32 [T*k, 2*inter]: the gate/up GEMM also stores its pre-activations for
     * a later moe_backward (gu_saved = 1), which then skips their recomputation: row p
     * (expert row order, as h) holds g at columns [0, inter) and u at [inter, 2*inter),
     * the FP32 values h[p,:] = round(silu(g) * u) is formed from ("SwiGLU: rounding
     * after the multiply"). Memory for compute: 8*T*k*inter bytes kept between the
     * forward and the backward. */
    float *gu;
} moe_forward_args;

/* The whole layer: route (or replay) -> permute -> grouped FFN -> combine, each step as
 * the entry point above defines it, enqueued on `stream` with no host synchronisation
 * (graph-capturable). */
moe_status moe_forward(const moe_dims *dims, const moe_forward_args *args, void *stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same layer, bitwise
 * the same outputs, with the workspace (and the shared expert's, after it at a 256-byte
 * boundary) taken from a static device array of MOE_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends; args->workspace,
 * workspace_bytes, shared_workspace and shared_workspace_bytes are ignored. The caller
 * still passes every input and output. No hipMalloc, hipFree or allocating library call.
 * The array of the current device is used (the stream must belong to that device); its
 * address is looked up on the first call on each device. Every call on one GPU shares the
 * one array, which keeps the last call's contents (no step needs it cleared): calls that
 * overlap on one GPU (other streams, other threads) race, and the caller must serialise
 * them. Returns MOE_E_SCRATCH, enqueuing nothing, when moe_workspace_size(dims) (plus the
 * shared expert's workspace) exceeds MOE_NOALLOC_SCRATCH_BYTES; otherwise as moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_dims *dims, const moe_forward_args *args,
                               void *stream);

/* Backward of the layer [EX][SW][RT][TRR]: the derivative of the forward definitions,
 * every reduction in one fixed order (results bitwise identical run to run; every per-token
 * row of d_x, d_y, d_h, d_gu, d_xp and d_topk_w is bitwise independent of T). With
 * s = routed_scale (0 means 1), for assignment (t,j) at row p = inv[t*k+j] of expert e:
 *   d_y[p,:]    = (s topk_w[t,j]) d_out[t,:]                                  (FP32)
 *   d_topk_w[t,j] = s <d_out[t,:], y[p,:]>
 *   gu[p,:]     = the forward's gate (n < I) and up (n >= I) pre-activations, recomputed by
 *                 the forward's own GEMM (bit for bit the values the forward used)
 *   d_h[p,i]    = sum_o d_y[p,o] w2[e,o,i]
 *   d_gu[p,i]   = (d_h u) silu'(g),  d_gu[p,I+i] = d_h silu(g)   (g, u = gu[p,i], gu[p,I+i])
 *   d_xp[p,c]   = sum_n d_gu[p,n] w13[e,n,c]
 *   d_w2[e,o,i] = sum over the segment's rows p (ascending) of d_y[p,o] h[p,i]
 *   d_w13[e,n,c]= sum over the segment's rows p (ascending) of d_gu[p,n] x[perm[p]/k,c]
 *   router (w_router not NULL): its own top-k from the logits (saved, or recomputed from
 *     x, w_router and logit_bias when logits is NULL), p = softmax, s' = sum of the chosen
 *     p left to right; a = sum_j d_topk_w[t,j] p_j / s', dp_j = (d_topk_w[t,j] - a) / s',
 *     c = sum_j dp_j p_j; d_logits[t,e] = p_e (dp_e - c) (dp_e = 0 for experts not chosen);
 *     d_w_router = d_logits^T x; d_x_router = d_logits w_router. For T >= 512 and E, d
 *     multiples of 4, d_w_router's sum over t runs as S = min(8, T/256) segments of
 *     ceil(T/S) ascending rows, each its own ascending sum, the S partials then added in
 *     segment order (the partials are staged in d_x, which the call writes last).
 *     Under routing replay this is the gradient of w - sg[w] + w* ("Total Router Recall"):
 *     the forward value is the replayed w*, the router's gradient flows through its own
 *     weights at its own choice, slot by slot.
 *   d_x[t,:]    = ((0 + d_xp[inv[t*k]]) + d_xp[inv[t*k+1]] + ...) + d_x_router[t,:].
 * The gradient GEMMs run FP32 MFMA on FP32 operands (bf16 storage widened exactly).
 * Placement: with slot-ordered w13/w2 and the forward's per-slot offsets, d_w13/d_w2 come
 * out in slot order; the router's gradients are in logical order.
 * Buffers: inputs as moe_forward wrote them (offsets [E+1], perm/inv [T*k], topk_w [T,k],
 * h [T*k,I] dtype, y [T*k,d] f32), d_out [T,d] dtype; outputs FP32: d_x [T,d],
 * d_w13 [E,2I,d], d_w2 [E,d,I], d_topk_w [T,k], and with w_router: d_logits [T,E],
 * d_w_router [E,d] (optional), d_x_router [T,d]; FP32 intermediates d_y [T*k,d],
 * gu [T*k,2I] (may be NULL for a bf16 layer: the recomputation then runs after d_h and
 * forms d_gu in its epilogue with the same arithmetic, so every gradient has the same bits
 * and gu is not written), d_h [T*k,I], d_gu [T*k,2I], d_xp [T*k,d]; x_perm [T*k,d] or NULL (the
 * recomputation gathers x through perm; x must then be under 4 GiB); workspace of
 * moe_workspace_size() bytes. No output or intermediate may overlap an input. */
typedef struct moe_backward_args {
    const void *x;
    const void *x_perm;
    const void *w13;
    const void *w2;
    const void *w_router;
    const float *logit_bias;
    const float *logits;
    const int32_t *offsets;
    const int32_t *perm;
    const int32_t *inv;
    const float *topk_w;
    const void *h;
    const float *y;
    const void *d_out;
    float routed_scale;
    float *d_x;
    float *d_w13;
    float *d_w2;
    float *d_topk_w;
    float *d_logits;
    float *d_w_router;
    float *d_x_router;
    float *d_y;
    float *gu;
    float *d_h;
    float *d_gu;
    float *d_xp;
    void *workspace;
    size_t workspace_bytes;
    /* MOE_F32 (0): the gradient GEMMs take FP32 operands, as above. MOE_BF16 (bf16 layers
     * only): d_y and d_gu are rounded once to bf16 where they are formed (RNE; the buffers
     * then hold bf16 [T*k,d] and [T*k,2I]), and every gradient GEMM consumes the rounded
     * values on bf16 MFMA: dh and d_xp through the forward's grouped GEMM reading w2 and
     * w13 as stored (K-major for these products), d_w2 and d_w13 on a bf16 weight-gradient
     * kernel. */
    int32_t grad_dtype;
    /* 1: gu holds the forward's pre-activations (moe_forward_args.gu of the same step):
     * the recomputation is skipped and the SwiGLU derivative reads them, so every
     * gradient is bitwise the one of the recomputing call. 0: gu (if given) is written by
     * the recomputation. */
    int32_t gu_saved;
} moe_backward_args;
moe_status moe_backward(const moe_dims *dims, const moe_backward_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_ROUTING_AMD_MOE_H */
