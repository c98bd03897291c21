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

// Butterfly sum: every lane ends with the same bits (each level adds the same two
// operands, only commuted), and the tree shape is fixed by the wave width alone.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off);
    return v;
}

// Softmax + top-k + renormalisation ("0 train-infer mismatch ...", "The router: matching
// expert ids and weights") of the NTOK consecutive tokens t0 .. t0+NTOK-1 (those < T) of
// the calling wave. Lane l holds experts l, l+64, l+128, l+192. The k rounds each take
// the largest remaining logit (wave max of its ordered bits) with ties to the lowest
// expert id; probabilities are exp(l - max) / Z with Z summed in a fixed tree; the k
// selected probabilities are renormalised by their left-to-right sum. Writes topk_idx /
// topk_w (and the ids to lds_ids when given), adds q[t] * p to macc (lane's experts) and
// ORs MOE_DERR_NONFINITE into err for a non-finite logit.
template <int NTOK>
__device__ __forceinline__ void route_wave(const float *__restrict__ logits,
                                           const int32_t *__restrict__ q, int64_t t0,
                                           int64_t T, int E, int k,
                                           int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w, int32_t *lds_ids,
                                           float (&macc)[4], int &err) {
    const int lane = threadIdx.x & 63;
    const int nlv = (E + 63) >> 6;    // logits per lane actually used
    float lv[NTOK][4];
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            const int64_t t = t0 + tt;
            lv[tt][i] = (t < T && e < E) ? logits[t * E + e] : 0.f;
        }
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
        const int64_t t = t0 + tt;
        if (t >= T) break;
        uint32_t hi[4];
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            valid[i] = e < E;
            if (valid[i] && !__builtin_isfinite(lv[tt][i])) err |= MOE_DERR_NONFINITE;
            hi[i] = valid[i] ? ordered_bits(lv[tt][i]) : 0u;
        }
        // k rounds: the largest remaining logit (wave max of its ordered bits), ties to
        // the lowest expert id (lowest lane of the lowest 64-expert group holding it)
        uint32_t taken = 0;
        int sel[kMaxK];
        uint32_t top_hi = 0;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            sel[j] = 0;
            if (j < k) {
                uint32_t best = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i < nlv && valid[i] && !((taken >> i) & 1u) && hi[i] > best) best = hi[i];
                const uint32_t m = wave_max_u32(best);
                int we = -1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint64_t mask =
                        __ballot(i < nlv && valid[i] && !((taken >> i) & 1u) && hi[i] == m);
                    if (we < 0 && mask) we = 64 * i + (int)__builtin_ctzll(mask);
                }
                sel[j] = we;
                if (j == 0) top_hi = m;
                if ((we & 63) == lane) taken |= 1u << (we >> 6);
            }
        }
        const float mx = from_ordered_bits(top_hi);
        float z[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = valid[i] ? expf(lv[tt][i] - mx) : 0.f;
        float zl = z[0] + z[1];
        zl = zl + z[2];
        zl = zl + z[3];
        const float Z = wave_sum(zl);
        float p[4];
        const float qt = q ? static_cast<float>(q[t]) : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = z[i] / Z;
            macc[i] = macc[i] + qt * p[i];
        }
        float ps[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            ps[j] = 0.f;
            if (j < k) {
                const int ri = sel[j] >> 6;
                const float mine = ri == 0 ? p[0] : ri == 1 ? p[1] : ri == 2 ? p[2] : p[3];
                ps[j] = __shfl(mine, sel[j] & 63);
            }
        }
        float sum = ps[0];
#pragma unroll
        for (int j = 1; j < kMaxK; ++j)
            if (j < k) sum = sum + ps[j];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k && lane == j) {
                topk_idx[t * k + j] = sel[j];
                topk_w[t * k + j] = ps[j] / sum;
                if (lds_ids) lds_ids[t * k + j] = sel[j];
            }
        }
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
