// route.hip -- router logits, FP32 softmax + top-k + renormalisation, probability mass,
// and routing-replay validation.
//
// Router ("0 train-infer mismatch for Open-weight MoE RL in Open-source code", "The
// router: matching expert ids and weights"): a fixed-K projection, FP32 softmax, the top
// k experts sorted by probability, weights renormalised by their left-to-right FP32 sum.
// Ties between equal logits go to the lower expert id (the same page's rule for equal
// sparse-attention scores, "Selecting sparse-attention positions"). Probability mass is
// weighted by token multiplicity ("HARTS ...", eq. (20)). Replay ("Total Router Recall")
// passes the sampler's ids and FP32 weights through untouched after validation.
#include "moe_internal.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ router logits
// One 256-thread block computes a 16-expert x 16-token tile of logits. The four waves
// split K statically: wave w takes K-steps w, w+4, w+8, ... and the four partial tiles
// are added in wave order. The split depends only on d, never on T, so every logit is
// the same sequence of MFMA steps and additions at any batch size.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4f32): the A operand
// rows are experts, the B operand columns are tokens; lane l feeds row/column l%16 and
// K-slice l/16; the result lane l holds column l%16 and rows 4*(l/16) + 0..3.
template <bool kBF16>
__global__ __launch_bounds__(256) void route_logits_kernel(const void *__restrict__ x_,
                                                           const void *__restrict__ wr_,
                                                           const float *__restrict__ bias,
                                                           float *__restrict__ logits,
                                                           int64_t T, int d, int E) {
    const int n_eb = (E + 15) >> 4;
    const int eb = (int)(blockIdx.x % n_eb) * 16;
    const int64_t tb = (int64_t)(blockIdx.x / n_eb) * 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int e_row = min(eb + r, E - 1);
    const int64_t t_row = min<int64_t>(tb + r, T - 1);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // K-steps w, w+4, w+8, ... of this wave, accumulated in that order; the operands of
    // up to 8 steps are loaded before their MFMAs so that the loads overlap.
    constexpr int kGroup = 8;
    if constexpr (kBF16) {
        const uint16_t *wp = static_cast<const uint16_t *>(wr_) + (int64_t)e_row * d + g * 8;
        const uint16_t *xp = static_cast<const uint16_t *>(x_) + t_row * d + g * 8;
        const int nsteps = d >> 5;
        for (int s0 = wave; s0 < nsteps; s0 += 4 * kGroup) {
            bf16x8_t a[kGroup], b[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int s = min(s0 + 4 * i, nsteps - 1);
                a[i] = *reinterpret_cast<const bf16x8_t *>(wp + s * 32);
                b[i] = *reinterpret_cast<const bf16x8_t *>(xp + s * 32);
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                if (s0 + 4 * i < nsteps)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[i], acc, 0, 0, 0);
        }
    } else {
        const float *wp = static_cast<const float *>(wr_) + (int64_t)e_row * d + g;
        const float *xp = static_cast<const float *>(x_) + t_row * d + g;
        const int nsteps = d >> 2;
        for (int s0 = wave; s0 < nsteps; s0 += 4 * kGroup) {
            float a[kGroup], b[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int s = min(s0 + 4 * i, nsteps - 1);
                a[i] = wp[s * 4];
                b[i] = xp[s * 4];
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                if (s0 + 4 * i < nsteps)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
        }
    }
    __shared__ float part[4][4][64];
    for (int i = 0; i < 4; ++i) part[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
        const int64_t t = tb + r;
        for (int i = 0; i < 4; ++i) {
            float v = part[0][i][lane];
            v = v + part[1][i][lane];
            v = v + part[2][i][lane];
            v = v + part[3][i][lane];
            const int e = eb + 4 * g + i;
            if (t < T && e < E) logits[t * E + e] = bias ? v + bias[e] : v;
        }
    }
}

// Total order used for expert selection: larger logit first, equal logits -> lower id.
// The logit maps to an unsigned key that orders like the real number (-0 == +0), and the
// low 32 bits hold ~id so that among equal logits the lower id has the larger key.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
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

// ------------------------------------------------------------- softmax + top-k
// One wave per token; a block of 4 waves handles kTopkTokPerBlock tokens, each wave
// kTopkTokPerBlock/4 of them with all their logits loaded up front. Lane l holds experts
// l, l+64, l+128, l+192. Every per-token result depends only on that token's E logits.
constexpr int kTokPerWave = kTopkTokPerBlock / 4;

__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         const int32_t *__restrict__ q,
                                                         int64_t T, int E, int k,
                                                         int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w,
                                                         float *__restrict__ mass_part,
                                                         int32_t *__restrict__ d_err) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t0 = (int64_t)blockIdx.x * kTopkTokPerBlock + wave * kTokPerWave;
    const int nlv = (E + 63) >> 6;    // logits per lane actually used
    float lv[kTokPerWave][4];
#pragma unroll
    for (int tt = 0; tt < kTokPerWave; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            const int64_t t = t0 + tt;
            lv[tt][i] = (t < T && e < E) ? logits[t * E + e] : 0.f;
        }
    float macc[4] = {0.f, 0.f, 0.f, 0.f};
    int err = 0;
#pragma unroll
    for (int tt = 0; tt < kTokPerWave; ++tt) {
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
            }
        }
    }
    if (__ballot(err != 0)) {
        int e_all = err;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) e_all |= __shfl_xor(e_all, off);
        if (lane == 0) raise_err(d_err, e_all);
    }
    if (mass_part) {
        __shared__ float mp[4][kMaxE];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < E) mp[wave][e] = macc[i];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += 256) {
            float v = mp[0][e];
            v = v + mp[1][e];
            v = v + mp[2][e];
            v = v + mp[3][e];
            mass_part[(int64_t)blockIdx.x * E + e] = v;
        }
    }
}

// prob_mass[e]: one block per expert; thread i adds the partials of blocks i, i+256, ...
// in order, then a fixed binary tree over the 256 threads. The order depends only on the
// number of partials (i.e. on T).
__global__ __launch_bounds__(256) void mass_reduce_kernel(const float *__restrict__ part,
                                                          int64_t nblk, int E,
                                                          float *__restrict__ mass) {
    __shared__ float red[256];
    const int e = blockIdx.x;
    float acc = 0.f;
    for (int64_t b = threadIdx.x; b < nblk; b += 256) acc = acc + part[b * E + e];
    red[threadIdx.x] = acc;
    __syncthreads();
#pragma unroll
    for (int s = 128; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) mass[e] = red[0];
}

// ------------------------------------------------------------------------ replay
__global__ __launch_bounds__(256) void replay_kernel(const int32_t *__restrict__ idx_in,
                                                     const float *__restrict__ w_in,
                                                     int64_t T, int E, int k,
                                                     int32_t *topk_idx, float *topk_w,
                                                     int32_t *__restrict__ d_err) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int err = 0;
    if (t < T) {
        int ids[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            ids[j] = -1;
            if (j < k) {
                const int e = idx_in[t * k + j];
                const float wv = w_in[t * k + j];
                ids[j] = e;
                if (e < 0 || e >= E) err |= MOE_DERR_IDX_RANGE;
                if (!__builtin_isfinite(wv)) err |= MOE_DERR_NONFINITE;
#pragma unroll
                for (int i = 0; i < kMaxK; ++i)
                    if (i < j && ids[i] == e) err |= MOE_DERR_IDX_DUP;
                topk_idx[t * k + j] = e;
                topk_w[t * k + j] = wv;
            }
        }
    }
    raise_err(d_err, err);
}

}  // namespace

hipError_t launch_route(const moe_dims &dm, const void *x, const void *w_router,
                        const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                        float *mass_part, float *prob_mass, const int32_t *token_mult,
                        int32_t *d_err, hipStream_t s) {
    const int64_t T = dm.T;
    const int E = dm.E;
    if (T > 0) {
        const int64_t nblk = ((E + 15) / 16) * ((T + 15) / 16);
        if (dm.dtype == MOE_BF16)
            route_logits_kernel<true><<<dim3((unsigned)nblk), dim3(256), 0, s>>>(
                x, w_router, bias, logits, T, dm.d, E);
        else
            route_logits_kernel<false><<<dim3((unsigned)nblk), dim3(256), 0, s>>>(
                x, w_router, bias, logits, T, dm.d, E);
        const int64_t tblk = (T + kTopkTokPerBlock - 1) / kTopkTokPerBlock;
        route_topk_kernel<<<dim3((unsigned)tblk), dim3(256), 0, s>>>(
            logits, token_mult, T, E, dm.k, topk_idx, topk_w, prob_mass ? mass_part : nullptr,
            d_err);
        if (prob_mass)
            mass_reduce_kernel<<<dim3(E), dim3(256), 0, s>>>(mass_part, tblk, E, prob_mass);
    } else if (prob_mass) {
        mass_reduce_kernel<<<dim3(E), dim3(256), 0, s>>>(mass_part, 0, E, prob_mass);
    }
    return hipGetLastError();
}

hipError_t launch_replay(const moe_dims &dm, const int32_t *idx_in, const float *w_in,
                         int32_t *topk_idx, float *topk_w, int32_t *d_err, hipStream_t s) {
    if (dm.T > 0)
        replay_kernel<<<dim3((unsigned)((dm.T + 255) / 256)), dim3(256), 0, s>>>(
            idx_in, w_in, dm.T, dm.E, dm.k, topk_idx, topk_w, d_err);
    return hipGetLastError();
}

}  // namespace moe
