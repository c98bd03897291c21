// route_dev.h -- device routines shared by the routing kernels: the total order used for
// expert selection, DPP wave reductions, and softmax + top-k + renormalisation of the
// tokens of one wave. Every per-token result depends only on that token's E logits.
#pragma once
#include "moe_internal.h"

namespace moe {

// Total order used for expert selection: larger logit first, equal logits -> lower id.
// The logit maps to an unsigned key that orders like the real number (-0 == +0); among
// lanes holding the maximal key the lowest expert id is taken (see route_wave).
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

// Softmax + top-k + renormalisation ("0 train-infer mismatch ...", "The router: matching
// expert ids and weights") of the NTOK consecutive tokens t0 .. t0+NTOK-1 (those < T) of
// the calling wave. Lane l holds experts l, l+64, l+128, l+192. The k rounds each take
// the largest remaining logit (wave max of its ordered bits) with ties to the lowest
// expert id; probabilities are exp(l - max) / Z with Z summed in a fixed tree; the k
// selected probabilities are renormalised by their left-to-right sum. Writes topk_idx /
// topk_w (and the ids to lds_ids when given), adds q[t] * p to macc (lane's experts, in
// token order) and ORs MOE_DERR_NONFINITE into err for a non-finite logit.
//
// The NTOK tokens go through each round together (their reductions are independent and
// overlap); tokens past T are computed on zeros and their results dropped.
template <int NTOK>
__device__ __forceinline__ void route_tokens(const float *__restrict__ logits,
                                           const int32_t *__restrict__ q, int64_t t0,
                                           int64_t T, int E, int k,
                                           int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, int32_t *lds_ids,
                                           float (&macc)[4], int &err) {
    const int lane = threadIdx.x & 63;
    const int nlv = (E + 63) >> 6;    // logits per lane actually used
    float lv[NTOK][4];
    bool tv[NTOK];                    // token exists (uniform over the wave)
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) valid[i] = lane + 64 * i < E;
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
        tv[tt] = t0 + tt < T;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lv[tt][i] = (tv[tt] && valid[i]) ? logits[(t0 + tt) * E + lane + 64 * i] : 0.f;
    }
    uint32_t hi[NTOK][4];
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tv[tt] && valid[i] && !__builtin_isfinite(lv[tt][i])) err |= MOE_DERR_NONFINITE;
            hi[tt][i] = valid[i] ? ordered_bits(lv[tt][i]) : 0u;
        }
    // k rounds: per token the largest remaining logit, ties to the lowest expert id
    // (lowest lane of the lowest 64-expert group holding it)
    uint32_t taken[NTOK], top_hi[NTOK];
    int sel[NTOK][kMaxK];
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
        taken[tt] = 0;
        top_hi[tt] = 0;
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
            uint32_t m[NTOK];
#pragma unroll
            for (int tt = 0; tt < NTOK; ++tt) {
                uint32_t best = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i < nlv && valid[i] && !((taken[tt] >> i) & 1u) && hi[tt][i] > best)
                        best = hi[tt][i];
                m[tt] = wave_max_u32(best);
            }
#pragma unroll
            for (int tt = 0; tt < NTOK; ++tt) {
                int we = -1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint64_t mask = __ballot(i < nlv && valid[i] &&
                                                   !((taken[tt] >> i) & 1u) && hi[tt][i] == m[tt]);
                    if (we < 0 && mask) we = 64 * i + (int)__builtin_ctzll(mask);
                }
                sel[tt][j] = we;
                if (j == 0) top_hi[tt] = m[tt];
                if ((we & 63) == lane) taken[tt] |= 1u << (we >> 6);
            }
        } else {
#pragma unroll
            for (int tt = 0; tt < NTOK; ++tt) sel[tt][j] = 0;
        }
    }
    // softmax over all E, renormalisation of the k selected probabilities
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
        const int64_t t = t0 + tt;
        const float mx = from_ordered_bits(top_hi[tt]);
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = valid[i] ? expf(lv[tt][i] - mx) : 0.f;
        float zl = z[0] + z[1];
        zl = zl + z[2];
        zl = zl + z[3];
        const float Z = wave_sum(zl);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = z[i] / Z;
        if (tv[tt]) {
            const float qt = q ? static_cast<float>(q[t]) : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) macc[i] = macc[i] + qt * p[i];
        }
        float ps[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            ps[j] = 0.f;
            if (j < k) {
                const int e = sel[tt][j];          // uniform over the wave
                const int ri = e >> 6;
                const float mine = ri == 0 ? p[0] : ri == 1 ? p[1] : ri == 2 ? p[2] : p[3];
                ps[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63));
            }
        }
        float sum = ps[0];
#pragma unroll
        for (int j = 1; j < kMaxK; ++j)
            if (j < k) sum = sum + ps[j];
        if (tv[tt]) {
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k && lane == j) {
                    topk_idx[t * k + j] = sel[tt][j];
                    topk_w[t * k + j] = ps[j] / sum;
                    if (lds_ids) lds_ids[t * k + j] = sel[tt][j];
                }
            }
        }
    }
}

// The wave's tokens: all NTOK together when they all exist, else one at a time (the
// per-token arithmetic is the same either way; macc is added in token order).
template <int NTOK>
__device__ __forceinline__ void route_wave(const float *__restrict__ logits,
                                           const int32_t *__restrict__ q, int64_t t0,
                                           int64_t T, int E, int k,
                                           int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, int32_t *lds_ids,
                                           float (&macc)[4], int &err) {
    if (t0 + NTOK <= T) {
        route_tokens<NTOK>(logits, q, t0, T, E, k, topk_idx, topk_w, lds_ids, macc, err);
    } else {
        for (int64_t t = t0; t < T; ++t)
            route_tokens<1>(logits, q, t, T, E, k, topk_idx, topk_w, lds_ids, macc, err);
    }
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
