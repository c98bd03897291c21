/*
 * moe_oracle.c -- plain, slow, CPU reference for one MoE layer's routing, dispatch,
 * grouped SwiGLU experts, combine and load statistics.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or calls this
 * file; only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every floating-point step is FP32 (the precision the pages fix for router softmax,
 * routing weights and the expert accumulators) except two: the sigmoid / sqrt-softplus
 * router scores are evaluated in FP64 and rounded once to FP32, and the objective
 * statistics accumulate in FP64. Each is evaluated in one written-out sequential
 * order, built with -ffp-contract=off and without fast-math so no step is fused or
 * reordered. OpenMP is used only across independent rows: each result is computed by
 * one thread in the same order whatever the thread count.
 *
 * Sources (page title, section):
 *  [MM]  "0 train-infer mismatch for Open-weight MoE RL in Open-source code",
 *        "Matrix multiplication: the same reduction along K".
 *  [SW]  same page, "SwiGLU: rounding after the multiply".
 *  [RT]  same page, "Mixture-of-experts layers" / "The router: matching expert ids and
 *        weights" / "Choosing GLM's eight experts" (sigmoid scores, FP32 correction bias
 *        for the choice only, FP32-normalised pre-bias weights, factor 2.5 applied by the
 *        expert kernel).
 *  [EX]  same page, "The experts: keeping the route weight inside the accumulator" and
 *        "Sharding the experts" (slot-order FP32 accumulation, rounded once).
 *  [TRR] same page, "Total Router Recall" (replayed ids as ints + normalized FP32
 *        weights, used as given) and "Hash and learned expert routing" (frozen token-id
 *        table, sqrt-softplus scores; weights, ids and slot order preserved through the
 *        expert forward).
 *  [SEL] same page, "Selecting sparse-attention positions" (lower position wins ties;
 *        adopted for expert ties).
 *  [RP]  "RoutePack: Expert Placement and Attention-Aware Data Packing for MoE
 *        Reinforcement Learning", Sec. 2.1 "Routing replay" eq. (1) (per-sample
 *        per-expert assignment counts) and Sec. 3.3 (aggregate expert load L_e).
 *  [HA]  "HARTS: Efficient Agentic Reinforcement Learning for Hybrid-Attention Models
 *        over Arbitrary Rollout Trees", Sec. 3 "MoE semantics without expert expansion"
 *        eq. (20) (multiplicity q_c weights mass and counts) and Sec. 4 "MoE execution
 *        and objectives" (no-token-drop: each row routed, dispatched, computed and
 *        combined once).
 *
 * Data types: dt = 0 means float32 arrays, dt = 1 means bfloat16 stored as uint16.
 * All pins of these functions live in the CPU test suite; no function is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ERR_IDX_RANGE 1
#define ORC_ERR_IDX_DUP 2
#define ORC_ERR_NONFINITE 4
#define ORC_ERR_SEQLENS 8

#define ORC_SCORE_SOFTMAX 0
#define ORC_SCORE_SIGMOID 1
#define ORC_SCORE_SQRT_SOFTPLUS 2

/* bfloat16 <-> float32. Widening is exact; narrowing rounds to nearest, ties to even. */
static float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN */
    uint32_t keep_lsb = (u >> 16) & 1u;
    u = u + 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

static float orc_load(const void *p, int64_t i, int dt) {
    return dt ? orc_bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

static void orc_store(void *p, int64_t i, float v, int dt) {
    if (dt) ((uint16_t *)p)[i] = orc_f32_to_bf16(v);
    else ((float *)p)[i] = v;
}

int orc_version(void) { return 1; }

/* Exposed for the test suite: the bf16 narrowing used at every rounding point. */
void orc_round_bf16(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

/* [MM], [RT]: router logits l[t,e] = sum_c x[t,c] * w_router[e,c] (+ bias[e]).
 * One FP32 accumulator per logit, c increasing: the K order never depends on T. */
void orc_router_logits(const void *x, const void *w_router, const float *bias, int64_t T,
                       int d, int E, int dt, float *logits) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            float acc = 0.0f;
            for (int c = 0; c < d; ++c) {
                float prod = orc_load(x, t * (int64_t)d + c, dt) *
                             orc_load(w_router, (int64_t)e * d + c, dt);
                acc = acc + prod;
            }
            logits[t * (int64_t)E + e] = bias ? acc + bias[e] : acc;
        }
    }
}

/* Does expert a rank before expert b? Larger logit first; equal logits: lower id [SEL]. */
static int orc_ranks_before(float la, int a, float lb, int b) {
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

/* [RT] + [HA]: FP32 softmax over all E logits, top-k, left-to-right renormalisation.
 *  - selection: the k experts that come first in the order (logit desc, id asc); slot j
 *    holds the j-th of them ("sorted by probability"; selection keyed on the FP32 logit,
 *    which orders the probabilities the same way);
 *  - p_e = exp(l_e - m) / Z with m = the largest logit and Z = sum over e ascending;
 *  - s = ((p_0 + p_1) + ...) over the selected slots, w_j = p_j / s;
 *  - prob_mass[e] = sum over t ascending of q_t * p[t,e] (q_t = 1 when q is NULL).
 * probs (optional, [T,E]) receives p. Returns error bits (non-finite logit). */
int orc_route_from_logits(const float *logits, const int32_t *q, int64_t T, int E, int k,
                          int32_t *idx, float *w, float *probs, float *prob_mass) {
    int err = 0;
    if (E > 256 || k < 1 || k > E) return -1;
    float *p_all = probs;
    int own = 0;
    if (prob_mass && !p_all) {
        p_all = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
        own = 1;
    }
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * (int64_t)E;
        int32_t sel[256];
        unsigned char taken[256];
        memset(taken, 0, sizeof(taken));
        for (int e = 0; e < E; ++e)
            if (!isfinite(l[e])) err |= ORC_ERR_NONFINITE;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || orc_ranks_before(l[e], e, l[best], best)) best = e;
            }
            sel[j] = best;
            taken[best] = 1;
        }
        float m = l[sel[0]];
        float z[256];
        float Z = 0.0f;
        for (int e = 0; e < E; ++e) {
            z[e] = expf(l[e] - m);
            Z = Z + z[e];
        }
        float p[256];
        for (int e = 0; e < E; ++e) p[e] = z[e] / Z;
        float s = p[sel[0]];
        for (int j = 1; j < k; ++j) s = s + p[sel[j]];
        for (int j = 0; j < k; ++j) {
            idx[t * k + j] = sel[j];
            w[t * k + j] = p[sel[j]] / s;
        }
        if (p_all)
            for (int e = 0; e < E; ++e) p_all[t * (int64_t)E + e] = p[e];
    }
    if (prob_mass) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e) {
            float acc = 0.0f;
            for (int64_t t = 0; t < T; ++t) {
                float qt = q ? (float)q[t] : 1.0f;
                acc = acc + qt * p_all[t * (int64_t)E + e];
            }
            prob_mass[e] = acc;
        }
    }
    if (own) free(p_all);
    return err;
}

/* [TRR]: replayed ids and weights are used as given. The only work is validation:
 * every id in [0,E), no id twice in a row, every weight finite. Returns error bits. */
int orc_replay_check(const int32_t *idx, const float *w, int64_t T, int E, int k) {
    int err = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E) err |= ORC_ERR_IDX_RANGE;
            if (!isfinite(w[t * k + j])) err |= ORC_ERR_NONFINITE;
            for (int i = 0; i < j; ++i)
                if (idx[t * k + i] == e) err |= ORC_ERR_IDX_DUP;
        }
    }
    return err;
}

/* [RP] eq. (1) / Sec. 3.3 and [HA] Sec. 4: expert histogram, exclusive offsets and a
 * stable counting sort of the flat assignments a = t*k + j by expert.
 *   counts[e]    = #{a : idx[a] == e}
 *   offsets[0]=0, offsets[e+1] = offsets[e] + counts[e]
 *   perm[p] = a, inv[a] = p, where segment e holds its assignments in increasing a.
 * Out-of-range ids raise ORC_ERR_IDX_RANGE and are left out. Returns error bits. */
int orc_permute(const int32_t *idx, int64_t T, int k, int E, int32_t *counts,
                int32_t *offsets, int32_t *perm, int32_t *inv) {
    int err = 0;
    int64_t A = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = idx[a];
        if (e < 0 || e >= E) { err |= ORC_ERR_IDX_RANGE; continue; }
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = idx[a];
        if (e < 0 || e >= E) { inv[a] = -1; continue; }
        int32_t p = cursor[e]++;
        perm[p] = (int32_t)a;
        inv[a] = p;
    }
    free(cursor);
    return err;
}

/* [RP] eq. (1): per-sequence counts a_{s,e} over the tokens [cu[s], cu[s+1]) of a packed
 * microbatch. cu must start at 0, end at T and never decrease (else ORC_ERR_SEQLENS). */
int orc_seq_counts(const int32_t *idx, int64_t T, int k, int E, const int32_t *cu, int S,
                   int32_t *seq_counts) {
    if (cu[0] != 0 || cu[S] != T) return ORC_ERR_SEQLENS;
    for (int s = 0; s < S; ++s)
        if (cu[s + 1] < cu[s]) return ORC_ERR_SEQLENS;
    memset(seq_counts, 0, sizeof(int32_t) * (size_t)S * (size_t)E);
    int err = 0;
    for (int s = 0; s < S; ++s) {
        for (int64_t t = cu[s]; t < cu[s + 1]; ++t) {
            for (int j = 0; j < k; ++j) {
                int32_t e = idx[t * k + j];
                if (e < 0 || e >= E) { err |= ORC_ERR_IDX_RANGE; continue; }
                seq_counts[(int64_t)s * E + e] += 1;
            }
        }
    }
    return err;
}

/* [HA] eq. (20): multiplicity-weighted assignment counts sum_t q_t [e in idx[t]]. */
int orc_weighted_counts(const int32_t *idx, const int32_t *q, int64_t T, int k, int E,
                        int64_t *wc) {
    int err = 0;
    for (int e = 0; e < E; ++e) wc[e] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E) { err |= ORC_ERR_IDX_RANGE; continue; }
            wc[e] += q ? (int64_t)q[t] : 1;
        }
    }
    return err;
}

/* [RP] Introduction (dispatch): x_perm[p,:] = x[perm[p] / k, :], an exact copy. */
void orc_gather(const void *x, const int32_t *perm, int64_t n_rows, int k, int d, int dt,
                void *x_perm) {
    size_t es = dt ? 2 : 4;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < n_rows; ++p) {
        int64_t t = perm[p] / k;
        memcpy((char *)x_perm + (size_t)p * d * es, (const char *)x + (size_t)t * d * es,
               (size_t)d * es);
    }
}

/* [MM], [SW], [EX]: one expert's SwiGLU FFN for each row r with its expert rowexp[r]:
 *   g_i = sum_c xr[c] w13[e,i,c],  u_i = sum_c xr[c] w13[e,I+i,c]  (FP32, c ascending)
 *   h_i = silu(g_i) * u_i in FP32, silu(g) = g / (1 + exp(-g)); rounded once to the
 *         storage dtype (bf16 for dt=1, unchanged for dt=0)
 *   y_o = sum_i h_i w2[e,o,i] (FP32, i ascending), kept in FP32.
 * h (dtype dt, [n,I]) and y (float, [n,d]) are outputs. */
void orc_expert_ffn(const void *xr, const int32_t *rowexp, int64_t n, int d, int I,
                    const void *w13, const void *w2, int dt, void *h, float *y) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        int64_t e = rowexp[r];
        float *hr = (float *)malloc(sizeof(float) * (size_t)I);
        for (int i = 0; i < I; ++i) {
            float g = 0.0f, u = 0.0f;
            for (int c = 0; c < d; ++c) {
                float xv = orc_load(xr, r * (int64_t)d + c, dt);
                g = g + xv * orc_load(w13, (e * 2 * I + i) * (int64_t)d + c, dt);
                u = u + xv * orc_load(w13, (e * 2 * I + I + i) * (int64_t)d + c, dt);
            }
            float silu = g / (1.0f + expf(-g));
            float hv = silu * u;
            orc_store(h, r * (int64_t)I + i, hv, dt);
            hr[i] = orc_load(h, r * (int64_t)I + i, dt);
        }
        for (int o = 0; o < d; ++o) {
            float acc = 0.0f;
            for (int i = 0; i < I; ++i)
                acc = acc + hr[i] * orc_load(w2, (e * d + o) * (int64_t)I + i, dt);
            y[r * (int64_t)d + o] = acc;
        }
        free(hr);
    }
}

/* [EX], [RT]: out[t,o] = round_out( ((0 + w_0 Y_0) + w_1 Y_1) + ... ) over the slots in
 * slot order, every product and sum in FP32, one final rounding (bf16 for dt=1). Y_j is
 * row inv[t*k+j] of y (the expert output of assignment (t,j)). */
/* [EX], [RT]: out[t,o] = round_out( scale * ( ((0 + w_0 Y_0) + w_1 Y_1) + ... ) ) over
 * the slots in slot order, every product and sum in FP32, one final rounding (bf16 for
 * dt=1). Y_j is row inv[t*k+j] of y (the expert output of assignment (t,j)). scale is the
 * routed scaling factor the expert kernel applies to the weighted sum ("Choosing GLM's
 * eight experts": the factor is applied inside the expert kernel to FP32 weights); 1 for
 * routers without one (a multiplication by 1 is exact). */
void orc_combine_scaled(const float *y, const int32_t *inv, const float *w, int64_t T,
                        int k, int d, int dt, float scale, void *out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int o = 0; o < d; ++o) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                float prod = w[t * k + j] * y[(int64_t)inv[t * k + j] * d + o];
                acc = acc + prod;
            }
            orc_store(out, t * (int64_t)d + o, scale * acc, dt);
        }
    }
}

void orc_combine(const float *y, const int32_t *inv, const float *w, int64_t T, int k,
                 int d, int dt, void *out) {
    orc_combine_scaled(y, inv, w, T, k, d, dt, 1.0f, out);
}

int orc_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Layer-local LPT placement ("RoutePack ...", Sec. 3, Algorithm 1). P ranks of H = E/P
 * slots; slot v belongs to rank v / H. Experts are visited in order of decreasing load,
 * equal loads by increasing id (picked by a plain selection scan over the unvisited
 * experts); each goes to the rank with the smallest accumulated load among the ranks
 * with a free slot, equal loads to the lower rank, and takes that rank's next slot.
 * rank_load [P] receives the accumulated loads. Returns 0, or 1 for bad arguments. */
int orc_place_lpt(const int64_t *loads, int E, int P, int32_t *slot_of_expert,
                  int64_t *rank_load) {
    if (E < 1 || P < 1 || E % P != 0) return 1;
    const int H = E / P;
    unsigned char *done = (unsigned char *)calloc((size_t)E, 1);
    int32_t *filled = (int32_t *)calloc((size_t)P, sizeof(int32_t));
    for (int p = 0; p < P; ++p) rank_load[p] = 0;
    for (int step = 0; step < E; ++step) {
        int pick = -1;
        for (int e = 0; e < E; ++e) {
            if (done[e]) continue;
            if (pick < 0 || loads[e] > loads[pick]) pick = e;  /* first max = lowest id */
        }
        int rank = -1;
        for (int p = 0; p < P; ++p) {
            if (filled[p] >= H) continue;
            if (rank < 0 || rank_load[p] < rank_load[rank]) rank = p; /* first min = lowest */
        }
        slot_of_expert[pick] = rank * H + filled[rank];
        filled[rank] += 1;
        rank_load[rank] += loads[pick];
        done[pick] = 1;
    }
    free(done);
    free(filled);
    return 0;
}

/* Scores of the learned routers, each the real function evaluated in FP64 and rounded
 * once to FP32 (so that two correct implementations agree on the FP32 score, and with it
 * on the selection, except where the FP64 value falls within an FP64 rounding error of a
 * point halfway between two FP32 numbers):
 *   ORC_SCORE_SIGMOID        s = 1 / (1 + e^-l)   ("Choosing GLM's eight experts");
 *   ORC_SCORE_SQRT_SOFTPLUS  s = sqrt(log(1 + e^l))   ("Hash and learned expert routing"),
 *                            with log(1 + e^l) written as max(l, 0) + log1p(e^-|l|). */
static float orc_score(float l, int fn) {
    double x = (double)l;
    if (fn == ORC_SCORE_SIGMOID) return (float)(1.0 / (1.0 + exp(-x)));
    double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
    return (float)sqrt(sp);
}

/* Does expert a rank before expert b under selection key values ka, kb? */
static int orc_key_before(float ka, int a, float kb, int b) {
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return a < b;
}

/* Router variants, from the logits, token by token:
 *  - per-expert value v[t,e]: fn ORC_SCORE_SOFTMAX: p = exp(l - m) / Z (m = the largest
 *    logit, Z summed over e ascending) [RT]; fn SIGMOID / SQRT_SOFTPLUS: s = score(l);
 *  - selection, when hash_table is NULL: fn SOFTMAX keys on the logit as
 *    orc_route_from_logits does (corr_bias must then be NULL); the scored routers key on
 *    s + corr_bias[e] (FP32 add; bias 0 when corr_bias is NULL): the k experts first in
 *    the order (key desc, id asc), slot 0 = largest. The bias chooses the experts only
 *    ("Choosing GLM's eight experts": FP32 correction bias added before choosing the top
 *    eight);
 *  - hash routing ("Hash and learned expert routing": a frozen table maps each token id to
 *    its experts, the logits only set the weights): slot j holds
 *    hash_table[token_ids[t] * k + j], in the table's order. A token id outside [0, V)
 *    sets ORC_ERR_IDX_RANGE and the row gets ids -1 and weights 0; a table id outside
 *    [0, E) or repeated within the row sets ORC_ERR_IDX_RANGE / ORC_ERR_IDX_DUP, the ids
 *    pass through and the row's weights are 0;
 *  - weights: w_j = v[sel_j] / ((v[sel_0] + v[sel_1]) + ...), the values before the bias
 *    normalised in FP32, left to right in slot order;
 *  - routing probabilities for the mass: fn SOFTMAX: p; the scored routers: s_e / sum_e s_e
 *    (e ascending); prob_mass[e] = sum over t ascending of q_t * prob[t,e] [HA];
 *  - lse[t] = m + log(Z), the log-sum-exp of the token's logits in FP32 (z-loss input).
 * scores (optional [T,E]) receives v. Non-finite logits set ORC_ERR_NONFINITE.
 * Returns the error bits, or -1 for bad dimensions or a bias with the softmax router. */
int orc_route_scored(const float *logits, const int32_t *q, int64_t T, int E, int k, int fn,
                     const float *corr_bias, const int32_t *hash_table,
                     const int32_t *token_ids, int V, int32_t *idx, float *w, float *scores,
                     float *prob_mass, float *lse) {
    int err = 0;
    if (E > 256 || k < 1 || k > E || fn < 0 || fn > 2) return -1;
    if (fn == ORC_SCORE_SOFTMAX && corr_bias && !hash_table) return -1;
    if (hash_table && (!token_ids || V < 1)) return -1;
    float *pr = NULL;
    if (prob_mass) pr = (float *)malloc(sizeof(float) * (size_t)(T > 0 ? T : 1) * (size_t)E);
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * (int64_t)E;
        float v[256], key[256];
        int32_t sel[256];
        for (int e = 0; e < E; ++e)
            if (!isfinite(l[e])) err |= ORC_ERR_NONFINITE;
        float m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        float Z = 0.0f;
        for (int e = 0; e < E; ++e) Z = Z + expf(l[e] - m);
        if (lse) lse[t] = m + logf(Z);
        if (fn == ORC_SCORE_SOFTMAX) {
            for (int e = 0; e < E; ++e) v[e] = expf(l[e] - m) / Z;
        } else {
            for (int e = 0; e < E; ++e) v[e] = orc_score(l[e], fn);
        }
        int zero_w = 0;
        if (hash_table) {
            const int32_t tok = token_ids[t];
            if (tok < 0 || tok >= V) {
                err |= ORC_ERR_IDX_RANGE;
                for (int j = 0; j < k; ++j) sel[j] = -1;
                zero_w = 1;
            } else {
                for (int j = 0; j < k; ++j) {
                    sel[j] = hash_table[(int64_t)tok * k + j];
                    if (sel[j] < 0 || sel[j] >= E) {
                        err |= ORC_ERR_IDX_RANGE;
                        zero_w = 1;
                    }
                    for (int i = 0; i < j; ++i)
                        if (sel[i] == sel[j]) {
                            err |= ORC_ERR_IDX_DUP;
                            zero_w = 1;
                        }
                }
            }
        } else {
            for (int e = 0; e < E; ++e) {
                if (fn == ORC_SCORE_SOFTMAX) key[e] = l[e];
                else key[e] = v[e] + (corr_bias ? corr_bias[e] : 0.0f);
            }
            unsigned char taken[256];
            memset(taken, 0, sizeof(taken));
            for (int j = 0; j < k; ++j) {
                int best = -1;
                for (int e = 0; e < E; ++e) {
                    if (taken[e]) continue;
                    if (best < 0 || orc_key_before(key[e], e, key[best], best)) best = e;
                }
                sel[j] = best;
                taken[best] = 1;
            }
        }
        if (zero_w) {
            for (int j = 0; j < k; ++j) w[t * k + j] = 0.0f;
        } else {
            float s = v[sel[0]];
            for (int j = 1; j < k; ++j) s = s + v[sel[j]];
            for (int j = 0; j < k; ++j) w[t * k + j] = v[sel[j]] / s;
        }
        for (int j = 0; j < k; ++j) idx[t * k + j] = sel[j];
        if (scores)
            for (int e = 0; e < E; ++e) scores[t * (int64_t)E + e] = v[e];
        if (pr) {
            if (fn == ORC_SCORE_SOFTMAX) {
                for (int e = 0; e < E; ++e) pr[t * (int64_t)E + e] = v[e];
            } else {
                float ssum = 0.0f;
                for (int e = 0; e < E; ++e) ssum = ssum + v[e];
                for (int e = 0; e < E; ++e) pr[t * (int64_t)E + e] = v[e] / ssum;
            }
        }
    }
    if (prob_mass) {
#pragma omp parallel for schedule(static)
        for (int e = 0; e < E; ++e) {
            float acc = 0.0f;
            for (int64_t t = 0; t < T; ++t) {
                float qt = q ? (float)q[t] : 1.0f;
                acc = acc + qt * pr[t * (int64_t)E + e];
            }
            prob_mass[e] = acc;
        }
        free(pr);
    }
    return err;
}

/* [HA] eq. (20) and "MoE execution and objectives": the multiplicity q_t of a compact
 * token weights its router z-loss term, and the probability mass and assignment counts of
 * the load-balancing loss; the expert-bias update uses the same weighted counts.
 *   S = sum_t q_t (q_t = 1 when q is NULL): the number of semantic token positions;
 *   z_loss = (1/S) sum_t q_t lse_t^2, accumulated in FP64, t ascending (0 when lse is
 *     NULL or S = 0);
 *   aux_loss = E * sum_e (C_e / (k S)) * (M_e / S) = E / (k S^2) * sum_e C_e M_e, with
 *     C = weighted assignment counts and M = probability mass, both in logical expert
 *     order, FP64, e ascending (0 when M or C is NULL or S = 0);
 *   bias update (bias not NULL): mean load Cbar = sum_e C_e / E; bias[e] + rate when
 *     C_e < Cbar, bias[e] - rate when C_e > Cbar, unchanged when equal (one FP32 add).
 * out[0] = z_loss, out[1] = aux_loss, out[2] = S. */
void orc_objectives(const float *lse, const int32_t *q, int64_t T, const int64_t *C,
                    const float *M, int E, int k, float rate, float *bias, double *out) {
    int64_t S = 0;
    double z = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t qt = q ? q[t] : 1;
        S += qt;
        if (lse) z += (double)qt * ((double)lse[t] * (double)lse[t]);
    }
    out[0] = (lse && S > 0) ? z / (double)S : 0.0;
    double a = 0.0;
    if (C && M && S > 0) {
        for (int e = 0; e < E; ++e) a += (double)C[e] * (double)M[e];
        out[1] = a * (double)E / ((double)k * (double)S * (double)S);
    } else {
        out[1] = 0.0;
    }
    out[2] = (double)S;
    if (bias && C) {
        int64_t tot = 0;
        for (int e = 0; e < E; ++e) tot += C[e];
        for (int e = 0; e < E; ++e) {
            /* C_e < tot / E  <=>  E * C_e < tot, in exact integers */
            const int64_t ec = (int64_t)E * C[e];
            if (ec < tot) bias[e] = bias[e] + rate;
            else if (ec > tot) bias[e] = bias[e] + (-rate);
        }
    }
}

/* Round a double to bfloat16, to nearest with ties to even, in one step (no intermediate
 * FP32 rounding): |x| = m 2^e with m in [1/2, 1) has 8 significant bits in bf16, so its
 * quantum is 2^(e-8), and never below the smallest subnormal 2^-133; scale by the quantum
 * (exact), round to an integer with rint (ties to even in the default mode), scale back. */
static uint16_t orc_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isinf(x)) return (uint16_t)(sign | 0x7f80);
    if (x == 0.0) return sign;
    int e;
    frexp(fabs(x), &e);
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    const double r = ldexp(rint(ldexp(fabs(x), -qexp)), qexp);
    if (r > 3.3895313892515355e38) return (uint16_t)(sign | 0x7f80); /* above bf16 max */
    const float f = (float)r;                                         /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

void orc_round_f64_bf16(const double *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(in[i]);
}

/* Expert-parallel output of one token, emulated on one device ("0 train-infer mismatch
 * ...", "Sharding the experts", and the shared-expert passage of "The experts: keeping the
 * route weight inside the accumulator"):
 *  - R ranks; rank r owns physical slots [r E/R, (r+1) E/R); the slot of routed id e is
 *    slot_map[e] (identity when NULL); an id outside [0, E) belongs to no rank;
 *  - rank r's partial: acc = 0; for j = 0..k-1 in slot order acc = acc + (the slot's rank
 *    is r ? w_j Y_j : 0) (other ranks' slots add exact zeros), all FP32; then
 *    acc = scale * acc (the routed scaling factor, 1 for none), plus the rank's shard of
 *    the shared expert ys[r, t, o] when ys is given; rounded once to the output type
 *    (bf16 for dt = 1; FP32 stays);
 *  - the R partials, in rank order, reduced by a pairwise tree: adjacent pairs added in
 *    FP64, an odd last contributor carried to the next level unchanged, repeated until one
 *    value remains, which is rounded once to the output type.
 * partials (optional, [R, T, d], output type) receives the rank partials. */
int orc_combine_ranks(const float *y, const int32_t *inv, const float *w, const int32_t *idx,
                      const int32_t *slot_map, int64_t T, int k, int d, int E, int R,
                      const float *ys, float scale, int dt, void *partials, void *out) {
    if (E < 1 || E > 256 || k < 1 || k > E || d < 1 || R < 1 || R > E || E % R) return -1;
    const int H = E / R;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int owner[256];
        for (int j = 0; j < k; ++j) {
            int e = idx[t * k + j];
            int v = (e >= 0 && e < E) ? (slot_map ? slot_map[e] : e) : -1;
            owner[j] = (v >= 0 && v < E) ? v / H : -1;
        }
        for (int o = 0; o < d; ++o) {
            double lvl[256];
            for (int r = 0; r < R; ++r) {
                float acc = 0.0f;
                for (int j = 0; j < k; ++j) {
                    float prod = (owner[j] == r) ? w[t * k + j] * y[(int64_t)inv[t * k + j] * d + o]
                                                 : 0.0f;
                    acc = acc + prod;
                }
                acc = scale * acc;
                if (ys) acc = acc + ys[((int64_t)r * T + t) * d + o];
                float part;
                if (dt == 1) {
                    uint16_t b = orc_f32_to_bf16(acc);
                    part = orc_bf16_to_f32(b);
                } else {
                    part = acc;
                }
                if (partials) orc_store(partials, ((int64_t)r * T + t) * d + o, part, dt);
                lvl[r] = (double)part;
            }
            int n = R;
            while (n > 1) {
                int m = 0;
                for (int i = 0; i + 1 < n; i += 2) lvl[m++] = lvl[i] + lvl[i + 1];
                if (n & 1) lvl[m++] = lvl[n - 1];
                n = m;
            }
            if (dt == 1) ((uint16_t *)out)[t * (int64_t)d + o] = orc_f64_to_bf16(lvl[0]);
            else ((float *)out)[t * (int64_t)d + o] = (float)lvl[0];
        }
    }
    return 0;
}

/* Backward of the expert path of the layer (the derivative of the forward definitions
 * above; "0 train-infer mismatch ...", "The experts: keeping the route weight inside the
 * accumulator" and "SwiGLU: rounding after the multiply" fix the forward). Given the
 * upstream gradient dout [T,d] of out, with the forward's saved h [A,I] (dt) and y [A,d]
 * (FP32) and the routing (perm, inv, segments, weights w [T,k], routed scaling factor s):
 *   dy[p,:]  = (s * w[t,j]) * dout[t,:]            for p = inv[t*k+j]   (FP32)
 *   dw[t,j]  = s * (sum over o ascending of dout[t,o] * y[p,o])
 *   gu[p,n]  = sum over c ascending of xr[p,c] * w13[e,n,c]   (xr = x[perm[p] / k]; the
 *              forward's gate (n < I) and up (n >= I) pre-activations, recomputed)
 *   dh[p,i]  = sum over o ascending of dy[p,o] * w2[e,o,i]
 *   with g = gu[p,i], u = gu[p,I+i], sg = 1 / (1 + exp(-g)), silu = g / (1 + exp(-g)),
 *        dsilu = sg * (1 + g * (1 - sg)):
 *   dgu[p,i] = (dh * u) * dsilu,  dgu[p,I+i] = dh * silu
 *   dxp[p,c] = sum over n ascending of dgu[p,n] * w13[e,n,c]
 *   dx[t,c]  = ((0 + dxp[inv[t*k],c]) + dxp[inv[t*k+1],c]) + ...   (slot order)
 *   dw2[e,o,i]  = sum over the segment's rows p ascending of dy[p,o] * h[p,i]
 *   dw13[e,n,c] = sum over the segment's rows p ascending of dgu[p,n] * xr[p,c]
 * All FP32, each sum sequential; rowexp [A] gives each row's expert. */
static float orc_round_to_bf16_value(float v) { return orc_bf16_to_f32(orc_f32_to_bf16(v)); }

/* With round_grads = 1 the two upstream gradients that feed the gradient GEMMs, dy and
 * dgu, are rounded once to bf16 (round to nearest even) where they are formed, as the
 * forward rounds h once: every later use (dh, dw2, dxp, dw13) takes the rounded values.
 * With 0 they stay FP32. */
void orc_backward_experts_r(const void *x, const int32_t *perm, const int32_t *inv,
                            const int32_t *rowexp, const float *w, const void *w13,
                            const void *w2, const void *h, const float *y, const void *dout,
                            float s, int64_t T, int k, int d, int I, int E, int dt,
                            int round_grads, float *dw, float *dy, float *gu, float *dh,
                            float *dgu, float *dxp, float *dx, float *dw13, float *dw2);

void orc_backward_experts(const void *x, const int32_t *perm, const int32_t *inv,
                          const int32_t *rowexp, const float *w, const void *w13,
                          const void *w2, const void *h, const float *y, const void *dout,
                          float s, int64_t T, int k, int d, int I, int E, int dt, float *dw,
                          float *dy, float *gu, float *dh, float *dgu, float *dxp, float *dx,
                          float *dw13, float *dw2) {
    orc_backward_experts_r(x, perm, inv, rowexp, w, w13, w2, h, y, dout, s, T, k, d, I, E, dt,
                           0, dw, dy, gu, dh, dgu, dxp, dx, dw13, dw2);
}

void orc_backward_experts_r(const void *x, const int32_t *perm, const int32_t *inv,
                            const int32_t *rowexp, const float *w, const void *w13,
                            const void *w2, const void *h, const float *y, const void *dout,
                            float s, int64_t T, int k, int d, int I, int E, int dt,
                            int round_grads, float *dw, float *dy, float *gu, float *dh,
                            float *dgu, float *dxp, float *dx, float *dw13, float *dw2) {
    const int64_t A = T * k;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            const int64_t p = inv[t * k + j];
            const float ws = s * w[t * k + j];
            float acc = 0.0f;
            for (int o = 0; o < d; ++o) {
                const float g = orc_load(dout, t * (int64_t)d + o, dt);
                dy[p * d + o] = round_grads ? orc_round_to_bf16_value(ws * g) : ws * g;
                acc = acc + g * y[p * d + o];
            }
            dw[t * k + j] = s * acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < A; ++p) {
        const int e = rowexp[p];
        const int64_t xt = perm[p] / k;
        const int64_t wb13 = (int64_t)e * 2 * I * d, wb2 = (int64_t)e * d * I;
        for (int n = 0; n < 2 * I; ++n) {
            float acc = 0.0f;
            for (int c = 0; c < d; ++c)
                acc = acc + orc_load(x, xt * d + c, dt) * orc_load(w13, wb13 + (int64_t)n * d + c, dt);
            gu[p * 2 * I + n] = acc;
        }
        for (int i = 0; i < I; ++i) {
            float acc = 0.0f;
            for (int o = 0; o < d; ++o)
                acc = acc + dy[p * d + o] * orc_load(w2, wb2 + (int64_t)o * I + i, dt);
            dh[p * I + i] = acc;
            const float g = gu[p * 2 * I + i], u = gu[p * 2 * I + I + i];
            const float sg = 1.0f / (1.0f + expf(-g));
            const float silu = g / (1.0f + expf(-g));
            const float dsilu = sg * (1.0f + g * (1.0f - sg));
            dgu[p * 2 * I + i] = (acc * u) * dsilu;
            dgu[p * 2 * I + I + i] = acc * silu;
            if (round_grads) {
                dgu[p * 2 * I + i] = orc_round_to_bf16_value(dgu[p * 2 * I + i]);
                dgu[p * 2 * I + I + i] = orc_round_to_bf16_value(dgu[p * 2 * I + I + i]);
            }
        }
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int n = 0; n < 2 * I; ++n)
                acc = acc + dgu[p * 2 * I + n] * orc_load(w13, wb13 + (int64_t)n * d + c, dt);
            dxp[p * d + c] = acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) acc = acc + dxp[(int64_t)inv[t * k + j] * d + c];
            dx[t * d + c] = acc;
        }
    /* segments: rows of expert e are contiguous; find each segment's bounds */
#pragma omp parallel for schedule(dynamic)
    for (int e = 0; e < E; ++e) {
        int64_t p0 = 0;
        while (p0 < A && rowexp[p0] != e) ++p0;
        int64_t p1 = p0;
        while (p1 < A && rowexp[p1] == e) ++p1;
        for (int o = 0; o < d; ++o)
            for (int i = 0; i < I; ++i) {
                float acc = 0.0f;
                for (int64_t p = p0; p < p1; ++p)
                    acc = acc + dy[p * d + o] * orc_load(h, p * (int64_t)I + i, dt);
                dw2[(int64_t)e * d * I + (int64_t)o * I + i] = acc;
            }
        for (int n = 0; n < 2 * I; ++n)
            for (int c = 0; c < d; ++c) {
                float acc = 0.0f;
                for (int64_t p = p0; p < p1; ++p)
                    acc = acc + dgu[p * 2 * I + n] * orc_load(x, (int64_t)(perm[p] / k) * d + c, dt);
                dw13[(int64_t)e * 2 * I * d + (int64_t)n * d + c] = acc;
            }
    }
}

/* Backward of the softmax router ("The router: matching expert ids and weights"), given
 * the gradient dw [T,k] of the routing weights by slot. The router's own choice is
 * recomputed from the logits (the k experts first in (logit desc, id asc)); with
 * p = softmax(l) (Z summed over e ascending), s = ((p_sel0 + p_sel1) + ...), w_j = p_selj / s:
 *   a = sum_j dw_j w_j,  dp_j = (dw_j - a) / s,  c = sum_j dp_j p_selj   (j ascending)
 *   dl[t,e] = p_e * (dp_e - c),  dp_e = dp_j for e = sel_j, 0 for an expert not chosen.
 * Under routing replay the weights the layer used are the sampler's w*, passed forward
 * as w - sg[w] + w* ("Total Router Recall"): the value is w*, the gradient reaches the
 * router through w, the router's own weights at its own choice, slot by slot; this
 * function is that gradient in both modes.
 *   dw_router[e,c] = sum over t ascending of dl[t,e] * x[t,c];
 *   dx_r[t,c]      = sum over e ascending of dl[t,e] * w_router[e,c]. */
int orc_backward_router(const float *logits, const float *dw, const void *x,
                        const void *w_router, int64_t T, int E, int k, int d, int dt,
                        float *dl, float *dw_router, float *dx_r) {
    if (E < 1 || E > 256 || k < 1 || k > E || d < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * (int64_t)E;
        int sel[256];
        unsigned char taken[256];
        memset(taken, 0, sizeof(taken));
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || orc_ranks_before(l[e], e, l[best], best)) best = e;
            }
            sel[j] = best;
            taken[best] = 1;
        }
        const float m = l[sel[0]];
        float p[256], Z = 0.0f;
        for (int e = 0; e < E; ++e) {
            p[e] = expf(l[e] - m);
            Z = Z + p[e];
        }
        for (int e = 0; e < E; ++e) p[e] = p[e] / Z;
        float s = p[sel[0]];
        for (int j = 1; j < k; ++j) s = s + p[sel[j]];
        float a = 0.0f;
        for (int j = 0; j < k; ++j) a = a + dw[t * k + j] * (p[sel[j]] / s);
        float dp[256], c = 0.0f;
        for (int j = 0; j < k; ++j) {
            dp[j] = (dw[t * k + j] - a) / s;
            c = c + dp[j] * p[sel[j]];
        }
        for (int e = 0; e < E; ++e) {
            float dpe = 0.0f;
            for (int j = 0; j < k; ++j)
                if (sel[j] == e) dpe = dp[j];
            dl[t * E + e] = p[e] * (dpe - c);
        }
    }
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e)
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int64_t t = 0; t < T; ++t) acc = acc + dl[t * E + e] * orc_load(x, t * (int64_t)d + c, dt);
            dw_router[(int64_t)e * d + c] = acc;
        }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int e = 0; e < E; ++e)
                acc = acc + dl[t * E + e] * orc_load(w_router, (int64_t)e * d + c, dt);
            dx_r[t * d + c] = acc;
        }
    return 0;
}
