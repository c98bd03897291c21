// moe_api.hip -- the C ABI: argument checks, workspace carving, launches.
// Nothing here allocates, synchronises the host or throws.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "moe_internal.h"

namespace moe {

int64_t perm_chunks(int64_t A) { return (A + kPermChunk - 1) / kPermChunk; }

static bool dims_ok(const moe_dims *d) {
    if (!d) return false;
    if (d->T < 0 || d->E < 1 || d->E > kMaxE || d->k < 1 || d->k > kMaxK || d->k > d->E)
        return false;
    if (d->T * (int64_t)d->k >= (int64_t(1) << 31)) return false;
    if (d->d < 64 || d->d > 16384 || d->d % 64) return false;
    if (d->inter < 64 || d->inter > 16384 || d->inter % 64) return false;
    if (d->tile_m != 0 && d->tile_m != 16 && d->tile_m != 32 && d->tile_m != 64 &&
        d->tile_m != 128 && d->tile_m != 256)
        return false;
    return true;
}

static bool dtype_ok(const moe_dims *d) { return d->dtype == MOE_F32 || d->dtype == MOE_BF16; }

Workspace carve_workspace(const moe_dims &d, void *base) {
    Workspace w{};
    const int64_t T = d.T, E = d.E, A = d.T * d.k;
    const int64_t nchunks = perm_chunks(A);
    const int64_t tblk = (T + kTopkTokPerBlock - 1) / kTopkTokPerBlock;
    // the tile list must hold the smallest tile height any launch may use
    const int64_t tiles = max_m_tiles(A, d.E, 16);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return base ? static_cast<char *>(base) + o : nullptr;
    };
    w.logits = reinterpret_cast<float *>(take(sizeof(float) * T * E));
    w.mass_part = reinterpret_cast<float *>(take(sizeof(float) * std::max<int64_t>(tblk, 1) * E));
    w.blk_hist = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * std::max<int64_t>(nchunks, 1) * E));
    w.blk_whist = reinterpret_cast<uint64_t *>(take(sizeof(uint64_t) * std::max<int64_t>(nchunks, 1) * E));
    w.tiles = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (1 + 3 * tiles)));
    w.logit_part = reinterpret_cast<float *>(
        take(T * E <= kChainSumMax ? sizeof(float) * kLogitChains * T * E : 1));
    w.total = off;
    return w;
}

}  // namespace moe

using namespace moe;

#define MOE_REQUIRE(cond, code) \
    do {                        \
        if (!(cond)) return (code); \
    } while (0)

extern "C" {

int moe_version(void) { return 100; }

const char *moe_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULLPTR: return "required pointer is NULL";
    case MOE_E_SHAPE: return "size outside the supported range";
    case MOE_E_DTYPE: return "unsupported dtype";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_LAUNCH: return "HIP launch failed";
    case MOE_E_SCRATCH: return "layer needs more workspace than the static scratch holds";
    }
    return "unknown status";
}

size_t moe_workspace_size(const moe_dims *dims) {
    if (!dims_ok(dims) || !dtype_ok(dims)) return 0;
    return carve_workspace(*dims, nullptr).total;
}

int32_t moe_tile_height(const moe_dims *dims) {
    if (!dims_ok(dims) || !dtype_ok(dims)) return 0;
    return select_tile_m(*dims);
}

static moe_status check_common(const moe_dims *dims) {
    if (!dims) return MOE_E_NULLPTR;
    if (!dtype_ok(dims)) return MOE_E_DTYPE;
    if (!dims_ok(dims)) return MOE_E_SHAPE;
    return MOE_OK;
}

static moe_status check_ws(const moe_dims *dims, void *ws, size_t bytes) {
    if (!ws) return MOE_E_WORKSPACE;
    if (bytes < carve_workspace(*dims, nullptr).total) return MOE_E_WORKSPACE;
    return MOE_OK;
}

static moe_status to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_LAUNCH; }

moe_status moe_route(const moe_dims *dims, const void *x, const void *w_router,
                     const float *logit_bias, int32_t *topk_idx, float *topk_w, float *logits,
                     float *prob_mass, const int32_t *token_mult, int32_t *d_err,
                     void *workspace, size_t workspace_bytes, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(x && w_router && topk_idx && topk_w, MOE_E_NULLPTR);
    st = check_ws(dims, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, workspace);
    return to_status(launch_route(*dims, x, w_router, logit_bias, logits ? logits : ws.logits,
                                  topk_idx, topk_w, ws.mass_part, prob_mass, token_mult, d_err,
                                  static_cast<hipStream_t>(stream)));
}

// Router options as the kernels take them; MOE_OK or the status of the first bad field.
static moe_status router_opts(const moe_dims *dims, const moe_router_opts *o, RouteOpts *r) {
    *r = RouteOpts();
    if (!o) return MOE_OK;
    if (o->score_fn < MOE_SCORE_SOFTMAX || o->score_fn > MOE_SCORE_SQRT_SOFTPLUS)
        return MOE_E_SHAPE;
    if (o->hash_table) {
        if (!o->token_ids) return MOE_E_NULLPTR;
        if (o->vocab < 1) return MOE_E_SHAPE;
        if ((int64_t)o->vocab * dims->k >= (int64_t(1) << 31)) return MOE_E_SHAPE;
    } else if (o->score_fn == MOE_SCORE_SOFTMAX && o->corr_bias) {
        return MOE_E_SHAPE;   // the softmax router chooses on the logits
    }
    r->fn = o->score_fn;
    r->corr_bias = o->hash_table ? nullptr : o->corr_bias;
    r->hash_table = o->hash_table;
    r->token_ids = o->hash_table ? o->token_ids : nullptr;
    r->vocab = o->hash_table ? o->vocab : 0;
    r->lse = o->lse;
    return MOE_OK;
}

moe_status moe_route_scored(const moe_dims *dims, const moe_router_opts *opts, const void *x,
                            const void *w_router, const float *logit_bias, int32_t *topk_idx,
                            float *topk_w, float *logits, float *prob_mass,
                            const int32_t *token_mult, int32_t *d_err, void *workspace,
                            size_t workspace_bytes, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(x && w_router && topk_idx && topk_w, MOE_E_NULLPTR);
    RouteOpts ro;
    st = router_opts(dims, opts, &ro);
    if (st != MOE_OK) return st;
    st = check_ws(dims, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, workspace);
    return to_status(launch_route(*dims, x, w_router, logit_bias, logits ? logits : ws.logits,
                                  topk_idx, topk_w, ws.mass_part, prob_mass, token_mult, d_err,
                                  static_cast<hipStream_t>(stream), ro));
}

moe_status moe_route_replay(const moe_dims *dims, const int32_t *idx_in, const float *w_in,
                            int32_t *topk_idx, float *topk_w, int32_t *d_err, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(idx_in && w_in && topk_idx && topk_w, MOE_E_NULLPTR);
    return to_status(launch_replay(*dims, idx_in, w_in, topk_idx, topk_w, d_err,
                                   static_cast<hipStream_t>(stream)));
}

static moe_status permute_impl(const moe_dims *dims, const int32_t *topk_idx,
                               const int32_t *slot_map, const void *x, void *x_perm,
                               int32_t *perm, int32_t *inv, int32_t *counts, int32_t *offsets,
                               const int32_t *cu_seqlens, int32_t num_seqs,
                               int32_t *seq_counts, const int32_t *token_mult,
                               int64_t *weighted_counts, int32_t *d_err, void *workspace,
                               size_t workspace_bytes, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(counts && offsets, MOE_E_NULLPTR);
    if (dims->T > 0) MOE_REQUIRE(topk_idx && perm && inv, MOE_E_NULLPTR);
    if (dims->T > 0 && x_perm) MOE_REQUIRE(x, MOE_E_NULLPTR);
    MOE_REQUIRE((cu_seqlens == nullptr) == (seq_counts == nullptr), MOE_E_NULLPTR);
    if (seq_counts) MOE_REQUIRE(num_seqs >= 1 && num_seqs <= dims->T + 1, MOE_E_SHAPE);
    st = check_ws(dims, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, workspace);
    return to_status(launch_permute(*dims, topk_idx, x, x_perm, perm, inv, counts, offsets,
                                    cu_seqlens, seq_counts ? num_seqs : 0, seq_counts,
                                    token_mult, weighted_counts, d_err, ws,
                                    static_cast<hipStream_t>(stream), slot_map));
}

moe_status moe_permute(const moe_dims *dims, const int32_t *topk_idx, const void *x,
                       void *x_perm, int32_t *perm, int32_t *inv, int32_t *counts,
                       int32_t *offsets, const int32_t *cu_seqlens, int32_t num_seqs,
                       int32_t *seq_counts, const int32_t *token_mult,
                       int64_t *weighted_counts, int32_t *d_err, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return permute_impl(dims, topk_idx, nullptr, x, x_perm, perm, inv, counts, offsets,
                        cu_seqlens, num_seqs, seq_counts, token_mult, weighted_counts, d_err,
                        workspace, workspace_bytes, stream);
}

moe_status moe_permute_placed(const moe_dims *dims, const int32_t *topk_idx,
                              const int32_t *slot_of_expert, const void *x, void *x_perm,
                              int32_t *perm, int32_t *inv, int32_t *counts, int32_t *offsets,
                              const int32_t *cu_seqlens, int32_t num_seqs, int32_t *seq_counts,
                              const int32_t *token_mult, int64_t *weighted_counts,
                              int32_t *d_err, void *workspace, size_t workspace_bytes,
                              void *stream) {
    MOE_REQUIRE(slot_of_expert, MOE_E_NULLPTR);
    return permute_impl(dims, topk_idx, slot_of_expert, x, x_perm, perm, inv, counts, offsets,
                        cu_seqlens, num_seqs, seq_counts, token_mult, weighted_counts, d_err,
                        workspace, workspace_bytes, stream);
}

// RoutePack, Sec. 3, Algorithm 1 ("Layer-local LPT expert placement"): experts in order of
// (load desc, id asc), each onto the least-loaded rank that still has a free slot (ties to
// the lower rank), into that rank's next free slot. Host code; E <= 256, so the
// O(E log E + E P) cost is negligible.
moe_status moe_place_lpt(const int64_t *loads, int32_t E, int32_t P, int32_t *slot_of_expert,
                         int64_t *rank_load, double *cv) {
    MOE_REQUIRE(loads && slot_of_expert, MOE_E_NULLPTR);
    MOE_REQUIRE(E >= 1 && E <= kMaxE && P >= 1 && E % P == 0, MOE_E_SHAPE);
    for (int32_t e = 0; e < E; ++e) MOE_REQUIRE(loads[e] >= 0, MOE_E_SHAPE);
    const int32_t H = E / P;
    int32_t order[kMaxE];
    for (int32_t e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order, order + E, [&](int32_t a, int32_t b) {
        return loads[a] > loads[b];  // stable: equal loads keep increasing id
    });
    int64_t G[kMaxE] = {0};
    int32_t n[kMaxE] = {0};
    for (int32_t i = 0; i < E; ++i) {
        const int32_t e = order[i];
        int32_t best = -1;
        for (int32_t p = 0; p < P; ++p)
            if (n[p] < H && (best < 0 || G[p] < G[best])) best = p;
        slot_of_expert[e] = best * H + n[best];
        G[best] += loads[e];
        n[best] += 1;
    }
    if (rank_load)
        for (int32_t p = 0; p < P; ++p) rank_load[p] = G[p];
    if (cv) {
        double mean = 0.0;
        for (int32_t p = 0; p < P; ++p) mean += (double)G[p];
        mean /= P;
        double var = 0.0;
        for (int32_t p = 0; p < P; ++p) var += ((double)G[p] - mean) * ((double)G[p] - mean);
        var /= P;
        *cv = mean > 0.0 ? std::sqrt(var) / mean : 0.0;
    }
    return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_dims *dims, const void *x_perm, const int32_t *offsets,
                           const void *w13, const void *w2, void *h, float *y, void *workspace,
                           size_t workspace_bytes, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(x_perm && offsets && w13 && w2 && h && y, MOE_E_NULLPTR);
    st = check_ws(dims, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, workspace);
    return to_status(launch_grouped_ffn(*dims, x_perm, offsets, w13, w2, h, y, ws, nullptr,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_dims *dims, const float *y, const int32_t *inv,
                       const float *topk_w, void *out, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(y && inv && topk_w && out, MOE_E_NULLPTR);
    return to_status(launch_combine(*dims, y, inv, topk_w, out, static_cast<hipStream_t>(stream)));
}

moe_status moe_combine_scaled(const moe_dims *dims, const float *y, const int32_t *inv,
                              const float *topk_w, float routed_scale, void *out,
                              void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    if (dims->T > 0) MOE_REQUIRE(y && inv && topk_w && out, MOE_E_NULLPTR);
    MOE_REQUIRE(std::isfinite(routed_scale), MOE_E_SHAPE);
    return to_status(launch_combine(*dims, y, inv, topk_w, out,
                                    static_cast<hipStream_t>(stream), routed_scale));
}

moe_status moe_objectives(const moe_dims *dims, const float *lse, const int32_t *token_mult,
                          const int64_t *weighted_counts, const float *prob_mass,
                          const int32_t *slot_of_expert, float bias_rate, float *corr_bias,
                          double *out, int32_t *d_err, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(out, MOE_E_NULLPTR);
    if (corr_bias) {
        MOE_REQUIRE(weighted_counts, MOE_E_NULLPTR);
        MOE_REQUIRE(std::isfinite(bias_rate), MOE_E_SHAPE);
    }
    return to_status(launch_objectives(*dims, lse, token_mult, weighted_counts, prob_mass,
                                       slot_of_expert, bias_rate, corr_bias, out, d_err,
                                       static_cast<hipStream_t>(stream)));
}

static bool ranks_ok(const moe_dims *dims, int32_t R) {
    return R >= 1 && R <= kMaxRanks && dims->E % R == 0;
}

// The shared expert alone needs no relation between R and E (the rank combine does).
static bool shared_ok(const moe_dims *dims, int32_t R, int32_t Is) {
    if (R < 1 || R > kMaxRanks || Is < 1 || Is % R) return false;
    const int32_t s = Is / R;
    if (s < 64 || s > 16384 || s % 64) return false;
    if (dims->T * (int64_t)R >= (int64_t(1) << 31)) return false;
    const int64_t x_bytes = dims->T * (int64_t)dims->d * (dims->dtype == MOE_BF16 ? 2 : 4);
    return x_bytes < (int64_t(1) << 32);   // rows are gathered with 32-bit byte offsets
}

moe_status moe_combine_ranks(const moe_dims *dims, int32_t ranks, const float *y,
                             const int32_t *inv, const float *topk_w, const int32_t *topk_idx,
                             const int32_t *slot_of_expert, const float *y_shared,
                             float routed_scale, void *partials, void *out, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(ranks_ok(dims, ranks), MOE_E_SHAPE);
    MOE_REQUIRE(std::isfinite(routed_scale), MOE_E_SHAPE);
    if (dims->T > 0) MOE_REQUIRE(y && inv && topk_w && topk_idx && out, MOE_E_NULLPTR);
    const float scale = routed_scale == 0.0f ? 1.0f : routed_scale;
    return to_status(launch_combine_ranks(*dims, ranks, y, inv, topk_w, topk_idx,
                                          slot_of_expert, scale, y_shared, partials, out,
                                          static_cast<hipStream_t>(stream)));
}

size_t moe_shared_workspace_size(const moe_dims *dims, int32_t ranks, int32_t inter_shared) {
    if (!dims_ok(dims) || !dtype_ok(dims) || !shared_ok(dims, ranks, inter_shared)) return 0;
    return shared_workspace_bytes(*dims, ranks, inter_shared);
}

moe_status moe_shared_ffn(const moe_dims *dims, int32_t ranks, int32_t inter_shared,
                          const void *x, const void *w13_shared, const void *w2_shared,
                          void *h_shared, float *y_shared, void *workspace,
                          size_t workspace_bytes, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(shared_ok(dims, ranks, inter_shared), MOE_E_SHAPE);
    if (dims->T > 0)
        MOE_REQUIRE(x && w13_shared && w2_shared && h_shared && y_shared, MOE_E_NULLPTR);
    MOE_REQUIRE(workspace, MOE_E_WORKSPACE);
    MOE_REQUIRE(workspace_bytes >= shared_workspace_bytes(*dims, ranks, inter_shared),
                MOE_E_WORKSPACE);
    return to_status(launch_shared_ffn(*dims, ranks, inter_shared, x, w13_shared, w2_shared,
                                       h_shared, y_shared, workspace,
                                       static_cast<hipStream_t>(stream)));
}

// The layer's output step: the plain combine, or (ranks >= 1) the shared expert's shards
// and the rank partials with their FP64 tree.
static hipError_t finish_layer(const moe_dims *dims, const moe_forward_args *a, float scale,
                               void *shared_work, hipStream_t s) {
    if (!a->ranks) return launch_combine(*dims, a->y, a->inv, a->topk_w, a->out, s, scale);
    if (a->w13_shared) {
        const hipError_t e = launch_shared_ffn(*dims, a->ranks, a->inter_shared, a->x,
                                               a->w13_shared, a->w2_shared, a->h_shared,
                                               a->y_shared, shared_work, s);
        if (e != hipSuccess) return e;
    }
    return launch_combine_ranks(*dims, a->ranks, a->y, a->inv, a->topk_w, a->topk_idx,
                                a->slot_of_expert, scale, a->w13_shared ? a->y_shared : nullptr,
                                a->partials, a->out, s);
}

// moe_forward with the workspace (and the shared expert's) given explicitly.
static moe_status forward_impl(const moe_dims *dims, const moe_forward_args *a, void *work,
                               size_t work_bytes, void *shared_work, size_t shared_bytes,
                               void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(a, MOE_E_NULLPTR);
    MOE_REQUIRE(a->counts && a->offsets, MOE_E_NULLPTR);
    const bool replay = a->idx_in != nullptr;
    if (dims->T > 0) {
        MOE_REQUIRE(a->x && a->w13 && a->w2 && a->out && a->topk_idx && a->topk_w && a->perm &&
                        a->inv && a->h && a->y,
                    MOE_E_NULLPTR);
        // the fused gather addresses token rows of x with 32-bit byte offsets
        const int64_t x_bytes = dims->T * (int64_t)dims->d * (dims->dtype == MOE_BF16 ? 2 : 4);
        if (!a->x_perm) MOE_REQUIRE(x_bytes < (int64_t(1) << 32), MOE_E_SHAPE);
        MOE_REQUIRE(replay ? (a->w_in != nullptr) : (a->w_router != nullptr), MOE_E_NULLPTR);
    }
    MOE_REQUIRE((a->cu_seqlens == nullptr) == (a->seq_counts == nullptr), MOE_E_NULLPTR);
    if (a->seq_counts) MOE_REQUIRE(a->num_seqs >= 1 && a->num_seqs <= dims->T + 1, MOE_E_SHAPE);
    RouteOpts ro;
    if (!replay) {
        st = router_opts(dims, a->router, &ro);
        if (st != MOE_OK) return st;
    }
    MOE_REQUIRE(std::isfinite(a->routed_scale), MOE_E_SHAPE);
    const float scale = a->routed_scale == 0.0f ? 1.0f : a->routed_scale;
    if (a->ranks) MOE_REQUIRE(ranks_ok(dims, a->ranks), MOE_E_SHAPE);
    if (a->w13_shared) {
        MOE_REQUIRE(a->ranks >= 1 && shared_ok(dims, a->ranks, a->inter_shared), MOE_E_SHAPE);
        MOE_REQUIRE(a->w2_shared && a->h_shared && a->y_shared, MOE_E_NULLPTR);
        MOE_REQUIRE(shared_work && shared_bytes >= shared_workspace_bytes(*dims, a->ranks,
                                                                         a->inter_shared),
                    MOE_E_WORKSPACE);
    }
    st = check_ws(dims, work, work_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, work);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dims->T >= 1 && dims->T <= kSmallT && !a->seq_counts) {
        // small batch: router logits, then the whole routing tail (top-k, statistics,
        // permutation, tile list) in one block. For the smallest batches the logits' 16
        // K-chains run as separate waves (the router weights then stream through 4x as many
        // CUs) and the tail adds the partials; past kChainSumMax partial values per chain
        // that sum costs the single block more than the wider logits launch saves.
        float *logits = a->logits ? a->logits : ws.logits;
        const bool chains = !replay && dims->T * dims->E <= kChainSumMax;
        // the smallest batches run the down GEMM and the plain combine as one launch
        const bool dc = !a->ranks && down_combine_small_ok(*dims);
        if (chains) {
            e = launch_router_logit_chains(*dims, a->x, a->w_router, ws.logit_part, s);
            if (e != hipSuccess) return MOE_E_LAUNCH;
            // one or two tokens, plain softmax router: the gate/up launch routes them (no
            // tail launch)
            if (dc && ro.plain() && !a->slot_of_expert && !a->x_perm &&
                decode_self_route_ok(*dims)) {
                DecodeRoute r;
                r.part = ws.logit_part;
                r.bias = a->logit_bias;
                r.q = a->token_mult;
                r.logits = logits;
                r.topk_w = a->topk_w;
                r.prob_mass = a->prob_mass;
                r.lse = ro.lse;
                r.topk_idx = a->topk_idx;
                r.counts = a->counts;
                r.offsets = a->offsets;
                r.perm = a->perm;
                r.inv = a->inv;
                r.tiles = ws.tiles;
                r.d_err = a->d_err;
                r.weighted_counts = a->weighted_counts;
                e = launch_decode_self_route(*dims, r, a->x, a->w13, a->h, a->gu,
                                             a->prof_events, s);
                if (e != hipSuccess) return MOE_E_LAUNCH;
                return to_status(launch_down_combine_small(*dims, a->h, a->w2, a->y, ws.tiles,
                                                           a->inv, a->topk_w, scale, a->out,
                                                           a->prof_events, s));
            }
        } else if (!replay) {
            e = launch_router_logits(*dims, a->x, a->w_router, a->logit_bias, logits, s);
            if (e != hipSuccess) return MOE_E_LAUNCH;
        }
        e = launch_small_tail(*dims, logits, a->token_mult, a->idx_in, a->w_in, a->topk_idx,
                              a->topk_w, a->prob_mass, a->counts, a->offsets, a->perm, a->inv,
                              a->weighted_counts, ws.tiles, a->d_err, s, a->slot_of_expert,
                              ro, chains ? ws.logit_part : nullptr, a->logit_bias);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        if (a->x_perm) {
            e = launch_gather(*dims, a->x, a->inv, a->x_perm, s);
            if (e != hipSuccess) return MOE_E_LAUNCH;
        }
        e = launch_grouped_ffn(*dims, a->x_perm, a->offsets, a->w13, a->w2, a->h, a->y, ws,
                               a->prof_events, s, a->x, a->perm, /*tiles_ready=*/true, a->gu,
                               /*gate_up_only=*/dc);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        if (dc)
            return to_status(launch_down_combine_small(*dims, a->h, a->w2, a->y, ws.tiles, a->inv,
                                                       a->topk_w, scale, a->out, a->prof_events,
                                                       s));
        return to_status(finish_layer(dims, a, scale, shared_work, s));
    }
    if (replay)
        e = launch_replay(*dims, a->idx_in, a->w_in, a->topk_idx, a->topk_w, a->d_err, s);
    else
        // the probability mass is reduced by the permutation's histogram launch
        e = launch_route(*dims, a->x, a->w_router, a->logit_bias,
                         a->logits ? a->logits : ws.logits, a->topk_idx, a->topk_w,
                         ws.mass_part, a->prob_mass, a->token_mult, a->d_err, s, ro,
                         /*defer_mass=*/dims->T > 0);
    if (e != hipSuccess) return MOE_E_LAUNCH;
    const bool mass_here = !replay && a->prob_mass && dims->T > 0;
    e = launch_permute(*dims, a->topk_idx, a->x, a->x_perm, a->perm, a->inv, a->counts,
                       a->offsets, a->cu_seqlens, a->seq_counts ? a->num_seqs : 0,
                       a->seq_counts, a->token_mult, a->weighted_counts, a->d_err, ws, s,
                       a->slot_of_expert, select_tile_m(*dims),   // tile list with the scan
                       mass_here ? ws.mass_part : nullptr,
                       (dims->T + kTopkTokPerBlock - 1) / kTopkTokPerBlock,
                       mass_here ? a->prob_mass : nullptr);
    if (e != hipSuccess) return MOE_E_LAUNCH;
    e = launch_grouped_ffn(*dims, a->x_perm, a->offsets, a->w13, a->w2, a->h, a->y, ws,
                           a->prof_events, s, a->x, a->perm, /*tiles_ready=*/true, a->gu);
    if (e != hipSuccess) return MOE_E_LAUNCH;
    return to_status(finish_layer(dims, a, scale, shared_work, s));
}

moe_status moe_forward(const moe_dims *dims, const moe_forward_args *a, void *stream) {
    if (!a) return check_common(dims) != MOE_OK ? check_common(dims) : MOE_E_NULLPTR;
    return forward_impl(dims, a, a->workspace, a->workspace_bytes, a->shared_workspace,
                        a->shared_workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free forward
// The workspace of moe_forward_noalloc: one array per GPU, held from the code object's load
// until the process ends. Host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or nullptr when it cannot be had.
void *scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    // a concurrent first call stores the same address
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}
}  // namespace

extern "C" {

moe_status moe_forward_noalloc(const moe_dims *dims, const moe_forward_args *a, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(a, MOE_E_NULLPTR);
    // the layer's workspace, then the shared expert's, carved from the one array
    const size_t work = carve_workspace(*dims, nullptr).total;
    size_t shared = 0;
    if (a->w13_shared) {
        MOE_REQUIRE(a->ranks >= 1 && shared_ok(dims, a->ranks, a->inter_shared), MOE_E_SHAPE);
        shared = shared_workspace_bytes(*dims, a->ranks, a->inter_shared);
    }
    const size_t shared_off = align_up(work, 256);
    MOE_REQUIRE(shared_off + shared <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_E_SCRATCH);
    uint8_t *base = static_cast<uint8_t *>(scratch_ptr());
    MOE_REQUIRE(base != nullptr, MOE_E_LAUNCH);
    return forward_impl(dims, a, base, work, shared ? base + shared_off : nullptr, shared,
                        stream);
}

moe_status moe_backward(const moe_dims *dims, const moe_backward_args *a, void *stream) {
    moe_status st = check_common(dims);
    if (st != MOE_OK) return st;
    MOE_REQUIRE(a, MOE_E_NULLPTR);
    MOE_REQUIRE(std::isfinite(a->routed_scale), MOE_E_SHAPE);
    if (dims->T == 0) return MOE_OK;
    MOE_REQUIRE(a->x && a->w13 && a->w2 && a->offsets && a->perm && a->inv && a->topk_w &&
                    a->h && a->y && a->d_out && a->d_x && a->d_w13 && a->d_w2 &&
                    a->d_topk_w && a->d_y && a->d_h && a->d_gu && a->d_xp,
                MOE_E_NULLPTR);
    // gu may be omitted on bf16 layers: the recomputation then forms d_gu in its epilogue
    MOE_REQUIRE(a->gu || dims->dtype == MOE_BF16, MOE_E_NULLPTR);
    if (a->w_router) MOE_REQUIRE(a->d_logits && a->d_x_router, MOE_E_NULLPTR);
    MOE_REQUIRE(a->grad_dtype == MOE_F32 || a->grad_dtype == MOE_BF16, MOE_E_DTYPE);
    MOE_REQUIRE(a->gu_saved == 0 || a->gu_saved == 1, MOE_E_SHAPE);
    if (a->gu_saved) MOE_REQUIRE(a->gu != nullptr, MOE_E_NULLPTR);
    const bool g16 = a->grad_dtype == MOE_BF16;
    if (g16) MOE_REQUIRE(dims->dtype == MOE_BF16, MOE_E_DTYPE);
    if (!a->x_perm) {
        const int64_t x_bytes = dims->T * (int64_t)dims->d * (dims->dtype == MOE_BF16 ? 2 : 4);
        MOE_REQUIRE(x_bytes < (int64_t(1) << 32), MOE_E_SHAPE);
    }
    st = check_ws(dims, a->workspace, a->workspace_bytes);
    if (st != MOE_OK) return st;
    const Workspace ws = carve_workspace(*dims, a->workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const float scale = a->routed_scale == 0.0f ? 1.0f : a->routed_scale;
    const bool bf16 = dims->dtype == MOE_BF16;
    const int64_t A = dims->T * dims->k;
    const int I = dims->inter, d = dims->d;
    hipError_t e = launch_combine_bwd(*dims, a->d_out, a->y, a->inv, a->topk_w, scale, a->d_y,
                                      a->d_topk_w, g16, s);
    if (e != hipSuccess) return MOE_E_LAUNCH;
    const void *xb = a->x_perm ? a->x_perm : a->x;
    const int32_t *xperm = a->x_perm ? nullptr : a->perm;
    const int64_t xrows = a->x_perm ? A : dims->T;
    // with gu, the gate/up pre-activations are recomputed into it and the SwiGLU derivative
    // is its own kernel; without, the recomputation runs after dh and forms d_gu itself
    // with gu saved by the forward, the SwiGLU derivative reads it as it stands
    const bool fused = a->gu == nullptr;
    if (!fused && !a->gu_saved) {
        e = launch_plain_gemm(*dims, xb, xperm, a->w13, a->gu, 2 * I, a->offsets, ws, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
    }
    auto swiglu_grad = [&](bool out_bf16) {
        return fused ? launch_gate_up_grad(*dims, xb, xperm, a->w13, a->d_h, a->d_gu, out_bf16,
                                           a->offsets, ws, s)
                     : launch_swiglu_bwd(*dims, a->gu, a->d_h, a->d_gu, out_bf16, s);
    };
    if (g16) {
        // data gradients on the forward's DMA GEMM with the weights read K-major as stored:
        // dh = dy w2[e] (K = d rows of w2), dxp = dgu w13[e] (K = 2I rows of w13)
        e = launch_plain_gemm(*dims, a->d_y, nullptr, a->w2, a->d_h, I, a->offsets, ws, s, d,
                              /*kmajor=*/true);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = swiglu_grad(true);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_plain_gemm(*dims, a->d_gu, nullptr, a->w13, a->d_xp, d, a->offsets, ws, s,
                              2 * I, /*kmajor=*/true);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_wgrad_bf16(dims->E, a->d_y, a->h, nullptr, 1, A, a->offsets, A, d, I,
                              a->d_w2, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_wgrad_bf16(dims->E, a->d_gu, xb, xperm, dims->k, xrows, a->offsets, A,
                              2 * I, d, a->d_w13, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
    } else {
        e = launch_dgrad(*dims, a->d_y, a->w2, bf16, d, I, a->offsets, a->d_h, ws, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = swiglu_grad(false);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_dgrad(*dims, a->d_gu, a->w13, bf16, 2 * I, d, a->offsets, a->d_xp, ws, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_wgrad(dims->E, a->d_y, a->h, bf16, nullptr, 1, A, a->offsets, A, d, I,
                         a->d_w2, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        e = launch_wgrad(dims->E, a->d_gu, xb, bf16, xperm, dims->k, xrows, a->offsets, A,
                         2 * I, d, a->d_w13, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
    }
    const float *dxr = nullptr;
    if (a->w_router) {
        const float *logits = a->logits;
        if (!logits) {
            e = launch_router_logits(*dims, a->x, a->w_router, a->logit_bias, ws.logits, s);
            if (e != hipSuccess) return MOE_E_LAUNCH;
            logits = ws.logits;
        }
        e = launch_router_bwd(*dims, logits, a->d_topk_w, a->d_logits, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        if (a->d_w_router) {
            // d_x is written last (the slot-order sum below): its T x d floats serve as
            // the scratch of the router weight gradient's row segments
            e = launch_router_wgrad(*dims, a->d_logits, a->x, a->d_w_router, a->d_x,
                                    dims->T * (int64_t)dims->d, s);
            if (e != hipSuccess) return MOE_E_LAUNCH;
        }
        e = launch_router_dx(*dims, a->d_logits, a->w_router, a->d_x_router, s);
        if (e != hipSuccess) return MOE_E_LAUNCH;
        dxr = a->d_x_router;
    }
    e = launch_dx_sum(*dims, a->d_xp, a->inv, dxr, a->d_x, s);
    return to_status(e);
}

}  // extern "C"
