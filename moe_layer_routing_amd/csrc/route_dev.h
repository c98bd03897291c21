// route_dev.h -- device routines shared by the routing kernels: the total order used for
// expert selection, DPP wave reductions, and softmax + top-k + renormalisation of the
// tokens of one wave. Every per-token result depends only on that token's E logits.
#pragma once
#include "moe_internal.h"

#include <type_traits>

namespace moe {

// Total order used for expert selection: larger logit first, equal logits -> lower id.
// The logit maps to an unsigned key that orders like the real number (-0 == +0); among
// lanes holding the maximal key the lowest expert id is taken (see route_rows4).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Wave-wide maximum through DPP lane moves (no LDS round trip): within quads (xor 1, 2),
// half-rows and rows (mirrors), then across rows (broadcast of lane 15 / lane 31); lane 63
// ends with the maximum of all 64 lanes, which readlane makes uniform.
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v, uint32_t o) { return o > v ? o : v; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide sum in a fixed DPP tree: quads (xor 1, xor 2), half-rows and rows
// (mirrors), then rows 1 and 3 add rows 0 and 2, and rows 2 and 3 add the first
// 32-lane sum; lane 63 ends with the total, which readlane makes uniform. Lanes a DPP
// move leaves out add 0, which is exact for the non-negative sums taken here.
__device__ __forceinline__ float dpp_add(float v, int ctrl_out) {
    return v + __int_as_float(ctrl_out);
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Row-wide (16-lane) reductions through DPP lane moves (quad xor 1 and 2, half-row and
// row mirrors): every lane of the row ends with the same result. For the sum, every level
// adds the same two operands in every lane (only commuted), so all lanes hold equal bits.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
}
__device__ __forceinline__ int row_min_i32(int v) {
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
    return v;
}
__device__ __forceinline__ float row_sum(float v) {
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// The k selection rounds of route_rows4 over one 16-lane row: lane c holds the keys hi[i]
// of experts c + 16 i (0 = absent; a present expert's key is >= 1). Lane j < k receives
// round j's id and key.
template <int NV>
__device__ __forceinline__ void topk_rounds(uint32_t (&hi)[NV], int c, int k, int &my_sel,
                                            uint32_t &my_key) {
    if constexpr (NV <= 8) {
        uint64_t kv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
            kv[i] = ((uint64_t)hi[i] << 32) | (uint32_t)~(uint32_t)(c + 16 * i);
#pragma unroll
        for (int pw = 1; pw < NV; pw <<= 1)
#pragma unroll
            for (int kk = pw; kk >= 1; kk >>= 1)
#pragma unroll
                for (int j = kk % pw; j + kk < NV; j += 2 * kk)
#pragma unroll
                    for (int i = 0; i < kk; ++i)
                        if ((i + j) / (2 * pw) == (i + j + kk) / (2 * pw)) {
                            const uint64_t a = kv[i + j], b = kv[i + j + kk];
                            kv[i + j] = b > a ? b : a;
                            kv[i + j + kk] = b > a ? a : b;
                        }
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            const uint32_t head = (uint32_t)(kv[0] >> 32);
            const uint32_t m = row_max_u32(head);
            const int e = row_min_i32(head == m ? (int)~(uint32_t)kv[0] : 0x7fffffff);
            if (c == j) {
                my_sel = e;
                my_key = m;
            }
            if ((e & 15) == c) {   // the owner drops its head
#pragma unroll
                for (int i = 0; i + 1 < NV; ++i) kv[i] = kv[i + 1];
                kv[NV - 1] = 0;
            }
        }
    } else {
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            uint32_t best = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) best = max(best, hi[i]);
            const uint32_t m = row_max_u32(best);
            int cand = 0x7fffffff;
#pragma unroll
            for (int i = NV - 1; i >= 0; --i)
                if (hi[i] == m) cand = c + 16 * i;
            const int e = row_min_i32(cand);
            if (c == j) {
                my_sel = e;
                my_key = m;
            }
            const bool own = (e & 15) == c;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (own && i == (e >> 4)) hi[i] = 0u;
        }
    }
}

// Softmax + top-k + renormalisation ("0 train-infer mismatch ...", "The router: matching
// expert ids and weights") of four consecutive tokens t0 .. t0+3, one per 16-lane row of
// the calling wave: lane c of row r holds token t0+r's logits of experts c, c+16, c+32, ...
// Each of the k rounds takes the row's largest remaining logit (row max of order-preserving
// keys), ties to the lowest expert id (row min over the lanes holding that key); the
// probabilities are exp(l - max) / Z with Z summed per lane in expert order and then in a
// fixed row tree; the k selected probabilities (recomputed from the selected logit, the
// same expression) are renormalised by their left-to-right sum. Writes topk_idx / topk_w
// (and the ids to lds_ids when given) for rows with t < T, returns q[t]·p for the lane's
// experts in qp (0 for rows past T) and ORs MOE_DERR_NONFINITE into err for a non-finite
// logit of an existing token. lse (optional) receives max + log(Z) per token.
constexpr int kRowVals = kMaxE / 16;   // logits per lane

template <int NV>
__device__ __forceinline__ void route_rows4(const float *__restrict__ logits,
                                            const int32_t *__restrict__ q, int64_t t0,
                                            int64_t T, int E, int k,
                                            int32_t *__restrict__ topk_idx,
                                            float *__restrict__ topk_w, int32_t *lds_ids,
                                            float (&qp)[kRowVals], int &err,
                                            float *__restrict__ lse = nullptr,
                                            int64_t row0 = 0) {
    const int lane = threadIdx.x & 63, c = lane & 15;
    const int64_t t = t0 + (lane >> 4);
    const bool tv = t < T;
    const int nv = (E + 15) >> 4;     // logits per lane actually used (uniform)
    float lv[NV];
    uint32_t hi[NV];                  // selection keys; 0 = absent or already taken
    bool valid[NV];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        valid[i] = c + 16 * i < E;
        lv[i] = (tv && valid[i]) ? logits[(t - row0) * E + c + 16 * i] : 0.f;
        if (tv && valid[i] && !__builtin_isfinite(lv[i])) err |= MOE_DERR_NONFINITE;
        // a present expert's key is at least 1 (only the NaN with all bits set maps to 0)
        hi[i] = valid[i] ? max(ordered_bits(lv[i]), 1u) : 0u;
        lmax = max(lmax, hi[i]);
    }
    // softmax over all E: shift by the row maximum (the first round's logit)
    const float mx = from_ordered_bits(row_max_u32(lmax));
    float z[NV];
    float zl = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        z[i] = valid[i] ? expf(lv[i] - mx) : 0.f;
        if (i < nv) zl = (i == 0) ? z[0] : zl + z[i];
    }
    const float Z = row_sum(zl);
    if (lse && tv && c == 0) lse[t] = mx + logf(Z);
    const float qt = (q && tv) ? static_cast<float>(q[t]) : 1.0f;
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) qp[i] = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) qp[i] = (tv && valid[i]) ? qt * (z[i] / Z) : 0.f;
    // Selection: k rounds, as a loop (decode-sized launches fetch this code cold, so its
    // size counts), each taking the row's largest remaining key with ties to the lowest id.
    // With 4 or 8 keys per lane, each lane first sorts its own (key, id) pairs, largest key
    // first and equal keys by ascending id (Batcher's odd-even merge network on the 64-bit
    // composite key << 32 | ~id); a round then takes the row maximum m of the lanes' head
    // keys and the lowest id among the heads equal to m (a lane's head is its lowest id of
    // its largest key), and the owning lane drops its head. With 16 keys per lane (E > 128)
    // the sorted lists do not fit the 1024-thread tail's registers, so a round takes the
    // maximum over all of the lane's keys and the owner clears the taken key in place (a
    // present expert's key is >= 1). Lane c of the row keeps round c's key and id; the
    // probabilities are formed after the loop, one per lane, and added left to right.
    int my_sel = 0;
    uint32_t my_key = 0;
    topk_rounds<NV>(hi, c, k, my_sel, my_key);
    // round c's probability (lanes c < k), then the left-to-right sum over the row's rounds
    const float my_p = expf(from_ordered_bits(my_key) - mx) / Z;
    const int rbase = lane & ~15;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
            const float pj = __shfl(my_p, rbase + j, 64);
            sum = (j == 0) ? pj : sum + pj;
        }
    }
    if (tv && c < k) {
        topk_idx[t * k + c] = my_sel;
        topk_w[t * k + c] = my_p / sum;
        if (lds_ids) lds_ids[t * k + c] = my_sel;
    }
}

// The ids route_rows4 selects for the one token whose E logits are at `logits` (every
// 16-lane row of the calling wave forms the same keys; lane j < k of each row returns
// round j's id): the selection alone, without the softmax, the weights or the mass.
template <int NV>
__device__ __forceinline__ int select_row4(const float *__restrict__ logits, int E, int k) {
    const int c = threadIdx.x & 15;
    uint32_t hi[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const bool valid = c + 16 * i < E;
        hi[i] = valid ? max(ordered_bits(logits[c + 16 * i]), 1u) : 0u;
    }
    int my_sel = 0;
    uint32_t my_key = 0;
    topk_rounds<NV>(hi, c, k, my_sel, my_key);
    return my_sel;
}

// Scores of the learned routers: the function evaluated in FP64 and rounded once to FP32.
//   sigmoid:       1 / (1 + e^-x) for x >= 0 and e^x / (1 + e^x) for x < 0, i.e.
//                  (x >= 0 ? 1 : e) / (1 + e) with e = e^-|x| (one exponential, no overflow);
//   sqrt-softplus: sqrt(log(1 + e^x)) with log(1 + e^x) = max(x, 0) + log1p(e^-|x|).
template <int kFn>
__device__ __forceinline__ float router_score(float l) {
    const double x = static_cast<double>(l);
    const double e = exp(-fabs(x));
    if constexpr (kFn == kScoreSigmoid) {
        return static_cast<float>((x >= 0.0 ? 1.0 : e) / (1.0 + e));
    } else {
        return static_cast<float>(sqrt(fmax(x, 0.0) + log1p(e)));
    }
}

// Row-uniform value v[e] of the row's lane (e & 15), register e >> 4 (v >= 0 or NaN, so
// its bits order like the value; non-owning lanes offer +0). 0 for e outside [0, 16 * nv).
template <int NV>
__device__ __forceinline__ float row_pick(const float (&v)[NV], int e, int c, int nv) {
    const bool own = e >= 0 && (e & 15) == c && (e >> 4) < nv;
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (own && i == (e >> 4)) b = __float_as_uint(v[i]);
    return __uint_as_float(row_max_u32(b));
}

// Router variants of route_rows4 for the same row layout ("0 train-infer mismatch ...",
// "Choosing GLM's eight experts" and "Hash and learned expert routing"; the mass per
// "HARTS ...", eq. (20)). Per token, v[e] is the softmax probability (kFn = softmax) or the
// score s[e] = router_score(l[e]).
//  - kHash: slot j holds hash_table[token_ids[t] * k + j]; a token id outside [0, vocab)
//    gives ids -1 and weights 0 (MOE_DERR_IDX_RANGE); a table id outside [0, E) or
//    repeated in the row gives weights 0 (MOE_DERR_IDX_RANGE / MOE_DERR_IDX_DUP).
//  - otherwise (scored routers only): k rounds of the row maximum of the FP32 key
//    s[e] + corr_bias[e] (order-preserving bits), ties to the lowest id, as route_rows4.
//  - weights: v at the chosen ids (row_pick), summed left to right, each divided by the
//    sum: the bias never enters a weight.
//  - qp: q[t] * prob[e], prob = p (softmax) or s[e] / (row sum of s) for the scored
//    routers; lse: max logit + log(Z) with Z = row sum of exp(l - max).
template <int kFn, bool kHash, int NV>
__device__ __forceinline__ void route_rows4_scored(
    const float *__restrict__ logits, const int32_t *__restrict__ q, int64_t t0, int64_t T,
    int E, int k, const RouteOpts &o, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int32_t *lds_ids, float (&qp)[kRowVals], int &err) {
    const int lane = threadIdx.x & 63, c = lane & 15;
    const int64_t t = t0 + (lane >> 4);
    const bool tv = t < T;
    const int nv = (E + 15) >> 4;
    float lv[NV], v[NV];
    bool valid[NV];
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        valid[i] = c + 16 * i < E;
        lv[i] = (tv && valid[i]) ? logits[t * E + c + 16 * i] : 0.f;
        if (tv && valid[i] && !__builtin_isfinite(lv[i])) err |= MOE_DERR_NONFINITE;
        if (valid[i]) lmax = max(lmax, ordered_bits(lv[i]));
    }
    const float mx = from_ordered_bits(row_max_u32(lmax));
    float Z = 1.f;
    if (kFn == kScoreSoftmax || o.lse) {
        float zl = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float z = valid[i] ? expf(lv[i] - mx) : 0.f;
            if (i < nv) zl = (i == 0) ? z : zl + z;
            if constexpr (kFn == kScoreSoftmax) v[i] = z;
        }
        Z = row_sum(zl);
        if (o.lse && tv && c == 0) o.lse[t] = mx + logf(Z);
    }
    float norm;
    if constexpr (kFn == kScoreSoftmax) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = valid[i] ? v[i] / Z : 0.f;
        norm = 1.f;
    } else {
        float sl = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i] = valid[i] ? router_score<kFn>(lv[i]) : 0.f;
            if (i < nv) sl = (i == 0) ? v[0] : sl + v[i];
        }
        norm = row_sum(sl);
    }
    const float qt = (q && tv) ? static_cast<float>(q[t]) : 1.0f;
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) qp[i] = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if constexpr (kFn == kScoreSoftmax) qp[i] = (tv && valid[i]) ? qt * v[i] : 0.f;
        else qp[i] = (tv && valid[i]) ? qt * (v[i] / norm) : 0.f;
    }

    if constexpr (kHash) {
        int sel[kMaxK];
        const int32_t tok = tv ? o.token_ids[t] : 0;
        const bool bad_tok = tv && (tok < 0 || tok >= o.vocab);
        if (bad_tok) err |= MOE_DERR_IDX_RANGE;
        bool zero_w = bad_tok;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            sel[j] = -1;
            if (j < k && tv && !bad_tok) {
                sel[j] = o.hash_table[(int64_t)tok * k + j];
                if (sel[j] < 0 || sel[j] >= E) {
                    err |= MOE_DERR_IDX_RANGE;
                    zero_w = true;
                }
#pragma unroll
                for (int i = 0; i < kMaxK; ++i)
                    if (i < j && sel[i] == sel[j]) {
                        err |= MOE_DERR_IDX_DUP;
                        zero_w = true;
                    }
            }
        }
        float vs[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) vs[j] = (j < k) ? row_pick(v, sel[j], c, nv) : 0.f;
        float sum = vs[0];
#pragma unroll
        for (int j = 1; j < kMaxK; ++j)
            if (j < k) sum = sum + vs[j];
        if (tv) {
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k && c == j) {
                    topk_idx[t * k + j] = sel[j];
                    topk_w[t * k + j] = zero_w ? 0.f : vs[j] / sum;
                    if (lds_ids) lds_ids[t * k + j] = sel[j];
                }
            }
        }
    } else {
        uint32_t hi[NV];            // selection keys; 0 = absent or already taken
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float b = (o.corr_bias && valid[i]) ? o.corr_bias[c + 16 * i] : 0.f;
            hi[i] = valid[i] ? max(ordered_bits(v[i] + b), 1u) : 0u;
        }
        // rounds as a loop (compact code, as route_rows4); lane c keeps round c's id and
        // value, the weights' sum runs left to right over the rounds
        int my_sel = 0;
        float my_v = 0.f, sum = 0.f;
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            uint32_t best = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) best = max(best, hi[i]);
            const uint32_t m = row_max_u32(best);
            int cand = 0x7fffffff;
#pragma unroll
            for (int i = NV - 1; i >= 0; --i)
                if (hi[i] == m) cand = c + 16 * i;
            const int e = row_min_i32(cand);
            const float vj = row_pick(v, e, c, nv);
            sum = (j == 0) ? vj : sum + vj;
            if (c == j) {
                my_sel = e;
                my_v = vj;
            }
            const bool own = (e & 15) == c;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (own && i == (e >> 4)) hi[i] = 0u;
        }
        if (tv && c < k) {
            topk_idx[t * k + c] = my_sel;
            topk_w[t * k + c] = my_v / sum;
            if (lds_ids) lds_ids[t * k + c] = my_sel;
        }
    }
}

// The row routine of a router variant (the plain softmax router is route_rows4).
template <int kFn, bool kHash, int NV>
__device__ __forceinline__ void route_rows(const float *__restrict__ logits,
                                           const int32_t *__restrict__ q, int64_t t0,
                                           int64_t T, int E, int k, const RouteOpts &o,
                                           int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, int32_t *lds_ids,
                                           float (&qp)[kRowVals], int &err, int64_t row0 = 0) {
    // logits holds the rows of tokens row0 .. (the softmax router may read a block's own
    // copy of its rows; the scored variants always read the full array, row0 = 0)
    if constexpr (kFn == kScoreSoftmax && !kHash)
        route_rows4<NV>(logits, q, t0, T, E, k, topk_idx, topk_w, lds_ids, qp, err, o.lse,
                        row0);
    else
        route_rows4_scored<kFn, kHash, NV>(logits, q, t0, T, E, k, o, topk_idx, topk_w, lds_ids,
                                       qp, err);
}

// Logits per lane for E experts, as a template argument (4, 8 or 16 registers): the row
// routines then hold and scan only as many values as E needs.
template <class F>
inline void with_row_vals(int E, F &&f) {
    if (E <= 64) f(std::integral_constant<int, 4>{});
    else if (E <= 128) f(std::integral_constant<int, 8>{});
    else f(std::integral_constant<int, 16>{});
}

// OR a per-lane error mask over the wave and raise it once.
__device__ __forceinline__ void wave_raise(int err, int32_t *d_err) {
    if (__ballot(err != 0)) {
        int e_all = err;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) e_all |= __shfl_xor(e_all, off);
        if ((threadIdx.x & 63) == 0) raise_err(d_err, e_all);
    }
}

}  // namespace moe
