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
// Router variants share the logits and the block layout: sigmoid or sqrt-softplus scores
// with a correction bias that only chooses ("Choosing GLM's eight experts"), and hash
// routing from a frozen token-id table ("Hash and learned expert routing").
#include "route_dev.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ router logits
// Logits come in 16-expert x 16-token MFMA tiles. Each logit is split statically over K
// into 16 partial chains: chain w takes K-steps w, w+16, w+32, ... (one MFMA each, in that
// order), and the 16 partials are added in chain order. The split depends only on d,
// never on T or on the launch shape, so every logit is the same sequence of MFMA steps and
// additions at any batch size.
//
// A 1024-thread block holds the 16 chains of EPB expert tiles of one token tile (wave w
// runs chain w of each): the token fragment of a K-step is loaded once and used for EPB
// expert tiles. EPB only groups tiles into blocks; it is chosen per launch so that small
// batches still spread over enough blocks.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4f32): the A operand
// rows are experts, the B operand columns are tokens; lane l feeds row/column l%16 and
// K-slice l/16; the result lane l holds column l%16 and rows 4*(l/16) + 0..3.
constexpr int kLogitSplit = kLogitChains;
static_assert(kLogitSplit == 16, "16 K-chains per logit");

// Chain `chain` of the logits of token tile tb (16 tokens) and expert tiles et0 .. et0+EPB-1:
// K-steps chain, chain+16, ... accumulated in that order into acc (one MFMA per step and
// tile). Every kernel that forms logits runs this routine, so a chain's partial is the
// same bits whichever launch computes it.
//
// Operand loads: a fragment is 16 rows x one K-step. Loaded in the MFMA layout (lane l:
// row l%16, K-slice l/16) every lane of a 4-lane group would touch a different row, and
// the memory pipeline serves such a load as 64 separate pieces; so lane l loads row l/4,
// K-slice l%4 (each 4-lane group reads one row's contiguous K-step) and a cross-lane
// permutation (ds_bpermute: lane l takes lane 4(l%16) + l/16's value) puts every value in
// the lane the MFMA reads it from. The MFMA operands are unchanged, value for value.
// Steps go in groups of kGroup whose loads are all issued before the first MFMA of the
// group; a chain's last steps that do not fill a group follow one at a time, in order.
__device__ __forceinline__ int to_mfma_lane(int v, int src) {
    return __builtin_amdgcn_ds_bpermute(src, v);
}

template <bool kBF16, int EPB>
__device__ __forceinline__ void logit_chain(const void *__restrict__ x_,
                                            const void *__restrict__ wr_, int64_t T, int d,
                                            int E, int64_t tb, int et0, int chain,
                                            f32x4_t (&acc)[EPB]) {
    const int lane = threadIdx.x & 63;
    const int rc = lane >> 2, gc = lane & 3;                  // the lane's load row / slice
    const int src = 4 * (4 * (lane & 15) + (lane >> 4));       // byte address of its source
    const int64_t t_row = min<int64_t>(tb + rc, T - 1);
#pragma unroll
    for (int j = 0; j < EPB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int kGroup = EPB >= 8 ? 2 : (EPB == 1 ? 8 : 4);
    constexpr int kStride = kLogitSplit;
    if constexpr (kBF16) {
        auto lay = [&](bf16x8_t v) {
            int4 q = __builtin_bit_cast(int4, v);
            q.x = to_mfma_lane(q.x, src);
            q.y = to_mfma_lane(q.y, src);
            q.z = to_mfma_lane(q.z, src);
            q.w = to_mfma_lane(q.w, src);
            return __builtin_bit_cast(bf16x8_t, q);
        };
        const uint16_t *wp[EPB];
#pragma unroll
        for (int j = 0; j < EPB; ++j)
            wp[j] = static_cast<const uint16_t *>(wr_) +
                    (int64_t)min((et0 + j) * 16 + rc, E - 1) * d + gc * 8;
        const uint16_t *xp = static_cast<const uint16_t *>(x_) + t_row * d + gc * 8;
        const int nsteps = d >> 5;
        int s0 = chain;
        for (; s0 + kStride * (kGroup - 1) < nsteps; s0 += kStride * kGroup) {
            bf16x8_t a[kGroup][EPB], b[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int st = s0 + kStride * i;
                b[i] = *reinterpret_cast<const bf16x8_t *>(xp + st * 32);
#pragma unroll
                for (int j = 0; j < EPB; ++j)
                    a[i][j] = *reinterpret_cast<const bf16x8_t *>(wp[j] + st * 32);
            }
            __builtin_amdgcn_sched_barrier(0);   // the group's loads are all in flight
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const bf16x8_t bi = lay(b[i]);
#pragma unroll
                for (int j = 0; j < EPB; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lay(a[i][j]), bi, acc[j],
                                                                     0, 0, 0);
            }
        }
        for (; s0 < nsteps; s0 += kStride) {
            const bf16x8_t bi = lay(*reinterpret_cast<const bf16x8_t *>(xp + s0 * 32));
#pragma unroll
            for (int j = 0; j < EPB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    lay(*reinterpret_cast<const bf16x8_t *>(wp[j] + s0 * 32)), bi, acc[j], 0,
                    0, 0);
        }
    } else {
        auto lay = [&](float v) {
            return __builtin_bit_cast(float, to_mfma_lane(__builtin_bit_cast(int, v), src));
        };
        const float *wp[EPB];
#pragma unroll
        for (int j = 0; j < EPB; ++j)
            wp[j] = static_cast<const float *>(wr_) +
                    (int64_t)min((et0 + j) * 16 + rc, E - 1) * d + gc;
        const float *xp = static_cast<const float *>(x_) + t_row * d + gc;
        const int nsteps = d >> 2;
        int s0 = chain;
        for (; s0 + kStride * (kGroup - 1) < nsteps; s0 += kStride * kGroup) {
            float a[kGroup][EPB], b[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const int st = s0 + kStride * i;
                b[i] = xp[st * 4];
#pragma unroll
                for (int j = 0; j < EPB; ++j) a[i][j] = wp[j][st * 4];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const float bi = lay(b[i]);
#pragma unroll
                for (int j = 0; j < EPB; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(lay(a[i][j]), bi, acc[j],
                                                                  0, 0, 0);
            }
        }
        for (; s0 < nsteps; s0 += kStride) {
            const float bi = lay(xp[s0 * 4]);
#pragma unroll
            for (int j = 0; j < EPB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(lay(wp[j][s0 * 4]), bi, acc[j],
                                                              0, 0, 0);
        }
    }
}

// The logits of block `blk` of a launch with n_eg expert-tile groups: the 16 chains of EPB
// expert tiles of one token tile, one chain per wave, added in chain order (then the bias).
template <bool kBF16, int EPB>
__device__ __forceinline__ void logits_block(const void *__restrict__ x_,
                                             const void *__restrict__ wr_,
                                             const float *__restrict__ bias,
                                             float *__restrict__ logits, int64_t T, int d,
                                             int E, int64_t blk,
                                             float (&part)[kLogitSplit][EPB][4][64],
                                             float *lds_rows = nullptr) {
    const int n_et = (E + 15) >> 4;
    const int n_eg = (n_et + EPB - 1) / EPB;
    const int et0 = (int)(blk % n_eg) * EPB;
    const int64_t tb = (blk / n_eg) * 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    f32x4_t acc[EPB];
    logit_chain<kBF16, EPB>(x_, wr_, T, d, E, tb, et0, wave, acc);
#pragma unroll
    for (int j = 0; j < EPB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[wave][j][i][lane] = acc[j][i];
    __syncthreads();
    // one thread per logit adds the 16 partials in chain order
    for (int o = threadIdx.x; o < EPB * 256; o += 64 * kLogitSplit) {
        const int j = o >> 8, i = (o >> 6) & 3, l = o & 63;
        float v = part[0][j][i][l];
#pragma unroll
        for (int w = 1; w < kLogitSplit; ++w) v = v + part[w][j][i][l];
        const int64_t t = tb + (l & 15);
        const int e = (et0 + j) * 16 + 4 * (l >> 4) + i;
        if (t < T && e < E && et0 + j < n_et) {
            const float lv = bias ? v + bias[e] : v;
            logits[t * E + e] = lv;
            if (lds_rows) lds_rows[(l & 15) * E + e] = lv;   // the block's own copy
        }
    }
}

template <bool kBF16, int EPB>
__global__ __launch_bounds__(64 * kLogitSplit) void route_logits_kernel(
    const void *__restrict__ x_, const void *__restrict__ wr_, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E) {
    __shared__ float part[kLogitSplit][EPB][4][64];
    logits_block<kBF16, EPB>(x_, wr_, bias, logits, T, d, E, blockIdx.x, part);
}

// Small batches: the 16 chains of every (token tile, expert tile) run as separate waves of
// kChainWaves-wave blocks (many more blocks than the single-block-per-tile kernel, so the
// router weights stream through many CUs) and each writes its partial to
// part[chain][t][e]; the routing tail then adds the 16 partials in chain order (and the
// bias) exactly as route_logits_kernel does, so the logits are the same bits.
constexpr int kChainWaves = 4;

template <bool kBF16>
__global__ __launch_bounds__(64 * kChainWaves) void route_logit_chains_kernel(
    const void *__restrict__ x_, const void *__restrict__ wr_, float *__restrict__ part,
    int64_t T, int d, int E) {
    constexpr int kGroups = kLogitSplit / kChainWaves;
    const int n_et = (E + 15) >> 4;
    const int cg = (int)(blockIdx.x % kGroups);
    const int tile = (int)(blockIdx.x / kGroups);
    const int et0 = tile % n_et;
    const int64_t tb = (int64_t)(tile / n_et) * 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int chain = cg * kChainWaves + wave;
    f32x4_t acc[1];
    logit_chain<kBF16, 1>(x_, wr_, T, d, E, tb, et0, chain, acc);
    // lane l holds token tb + l%16, experts 16 et0 + 4 (l/16) + 0..3
    const int64_t t = tb + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = et0 * 16 + 4 * (lane >> 4) + i;
        if (t < T && e < E) part[((int64_t)chain * T + t) * E + e] = acc[0][i];
    }
}

// ------------------------------------------------------------- softmax + top-k
// A block of 4 waves routes kTopkTokPerBlock = 16 tokens, 4 per wave (one per 16-lane
// row), and writes its per-expert probability-mass partial: per wave the sum of its four
// tokens' q·p in token order (starting from 0), then the four waves' sums in wave order.
static_assert(kTopkTokPerBlock == 16, "4 waves x 4 tokens");

// Top-k of the 16 tokens of group `grp` (waves 0..3 of the block, 4 tokens each) and the
// group's probability-mass partial; every thread of the block (nthr of them) reaches the
// one barrier.
template <int kFn, bool kHash, int NV>
__device__ __forceinline__ void topk_group(const float *__restrict__ logits,
                                           const int32_t *__restrict__ q, int64_t T, int E,
                                           int k, int32_t *__restrict__ topk_idx,
                                           float *__restrict__ topk_w,
                                           float *__restrict__ mass_part,
                                           int32_t *__restrict__ d_err, const RouteOpts &opts,
                                           int64_t grp, int nthr,
                                           float (&mpt)[kTopkTokPerBlock][kMaxE],
                                           const float *lds_rows = nullptr) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t0 = grp * kTopkTokPerBlock + wave * 4;
    float qp[kRowVals];
    int err = 0;
    if (wave < 4 && t0 < T) {   // wave-uniform; a wave past the batch only contributes zeros
        // lds_rows: the group's 16 logit rows as this block formed them (same values)
        if (lds_rows)
            route_rows<kFn, kHash, NV>(lds_rows, q, t0, T, E, k, opts, topk_idx, topk_w,
                                       nullptr, qp, err, grp * kTopkTokPerBlock);
        else
            route_rows<kFn, kHash, NV>(logits, q, t0, T, E, k, opts, topk_idx, topk_w, nullptr,
                                       qp, err);
    } else {
#pragma unroll
        for (int i = 0; i < kRowVals; ++i) qp[i] = 0.f;
    }
    wave_raise(err, d_err);
    if (mass_part) {
        const int row = wave * 4 + (lane >> 4), c = lane & 15;
        if (wave < 4) {
#pragma unroll
            for (int i = 0; i < kRowVals; ++i)
                if (c + 16 * i < E) mpt[row][c + 16 * i] = qp[i];
        }
        lds_barrier();   // (the top-k's stores to memory are not read back here)
        for (int e = threadIdx.x; e < E; e += nthr) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float m = 0.f + mpt[4 * w][e];
                m = m + mpt[4 * w + 1][e];
                m = m + mpt[4 * w + 2][e];
                m = m + mpt[4 * w + 3][e];
                v = (w == 0) ? m : v + m;
            }
            mass_part[grp * E + e] = v;
        }
    }
}

template <int kFn, bool kHash, int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         const int32_t *__restrict__ q,
                                                         int64_t T, int E, int k,
                                                         int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w,
                                                         float *__restrict__ mass_part,
                                                         int32_t *__restrict__ d_err,
                                                         RouteOpts opts) {
    __shared__ float mpt[kTopkTokPerBlock][kMaxE];
    topk_group<kFn, kHash, NV>(logits, q, T, E, k, topk_idx, topk_w, mass_part, d_err, opts,
                               blockIdx.x, 256, mpt);
}

// Logits and top-k in one launch, when one block holds every expert of its token tile
// (EPB >= E/16): block b forms the logits of tokens 16b .. 16b+15 (as route_logits_kernel
// does) and then routes the same 16 tokens (as route_topk_kernel's block b does), reading
// the logits from the copy it kept in LDS (the values it wrote to memory); every output is
// the bits of the two-kernel path.
template <bool kBF16, int EPB, int kFn, bool kHash, int NV>
__global__ __launch_bounds__(64 * kLogitSplit) void route_fused_kernel(
    const void *__restrict__ x_, const void *__restrict__ wr_, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E, const int32_t *__restrict__ q, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    float *__restrict__ mass_part, int32_t *__restrict__ d_err, RouteOpts opts) {
    static_assert(kFn == kScoreSoftmax && !kHash, "the fused launch routes the softmax router");
    __shared__ float part[kLogitSplit][EPB][4][64];
    __shared__ float mpt[kTopkTokPerBlock][kMaxE];
    __shared__ float rows[kTopkTokPerBlock * 16 * EPB];   // the block's logits (E <= 16 EPB)
    logits_block<kBF16, EPB>(x_, wr_, bias, logits, T, d, E, blockIdx.x, part, rows);
    lds_barrier();   // the top-k reads the LDS copy, not the logits just stored
    topk_group<kFn, kHash, NV>(logits, q, T, E, k, topk_idx, topk_w, mass_part, d_err, opts,
                               blockIdx.x, 64 * kLogitSplit, mpt, rows);
}

// prob_mass[e]: one wave per expert (mass_reduce_wave), four per block.
__global__ __launch_bounds__(256) void mass_reduce_kernel(const float *__restrict__ part,
                                                          int64_t nblk, int E,
                                                          float *__restrict__ mass) {
    const int e = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (e < E) mass_reduce_wave(part, nblk, E, e, mass);
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

// Expert tiles per block: as many as keep at least 256 blocks (the x fragment of a K-step
// then serves several expert tiles), at most 8.
static int logits_epb(int64_t T, int E) {
    const int64_t n_tt = (T + 15) / 16;
    const int n_et = (E + 15) / 16;
    int epb = 1;
    while (epb * 2 <= 8 && epb * 2 <= n_et && n_tt * ((n_et + epb * 2 - 1) / (epb * 2)) >= 256)
        epb *= 2;
    return epb;
}

template <bool kBF16>
static void launch_logits_t(const moe_dims &dm, const void *x, const void *w_router,
                            const float *bias, float *logits, hipStream_t s) {
    const int epb = logits_epb(dm.T, dm.E);
    const int n_eg = ((dm.E + 15) / 16 + epb - 1) / epb;
    const dim3 grid((unsigned)(((dm.T + 15) / 16) * n_eg)), block(64 * kLogitSplit);
    switch (epb) {
    case 1: route_logits_kernel<kBF16, 1><<<grid, block, 0, s>>>(x, w_router, bias, logits, dm.T, dm.d, dm.E); break;
    case 2: route_logits_kernel<kBF16, 2><<<grid, block, 0, s>>>(x, w_router, bias, logits, dm.T, dm.d, dm.E); break;
    case 4: route_logits_kernel<kBF16, 4><<<grid, block, 0, s>>>(x, w_router, bias, logits, dm.T, dm.d, dm.E); break;
    default: route_logits_kernel<kBF16, 8><<<grid, block, 0, s>>>(x, w_router, bias, logits, dm.T, dm.d, dm.E); break;
    }
}

hipError_t launch_router_logits(const moe_dims &dm, const void *x, const void *w_router,
                                const float *bias, float *logits, hipStream_t s) {
    if (dm.T > 0) {
        if (dm.dtype == MOE_BF16) launch_logits_t<true>(dm, x, w_router, bias, logits, s);
        else launch_logits_t<false>(dm, x, w_router, bias, logits, s);
    }
    return hipGetLastError();
}

hipError_t launch_router_logit_chains(const moe_dims &dm, const void *x, const void *w_router,
                                      float *part, hipStream_t s) {
    if (dm.T > 0) {
        const int64_t tiles = ((dm.T + 15) / 16) * (int64_t)((dm.E + 15) / 16);
        const dim3 grid((unsigned)(tiles * (kLogitSplit / kChainWaves))), block(64 * kChainWaves);
        if (dm.dtype == MOE_BF16)
            route_logit_chains_kernel<true><<<grid, block, 0, s>>>(x, w_router, part, dm.T, dm.d, dm.E);
        else
            route_logit_chains_kernel<false><<<grid, block, 0, s>>>(x, w_router, part, dm.T, dm.d, dm.E);
    }
    return hipGetLastError();
}

template <int kFn, bool kHash>
static void launch_topk_t(const moe_dims &dm, int64_t tblk, const float *logits,
                          const int32_t *q, int32_t *topk_idx, float *topk_w, float *mass_part,
                          int32_t *d_err, const RouteOpts &o, hipStream_t s) {
    with_row_vals(dm.E, [&](auto nv) {
        route_topk_kernel<kFn, kHash, decltype(nv)::value><<<dim3((unsigned)tblk), dim3(256), 0, s>>>(
            logits, q, dm.T, dm.E, dm.k, topk_idx, topk_w, mass_part, d_err, o);
    });
}

// Logits + top-k in one launch for the plain softmax router when the logits launch would
// give every block all expert tiles of its token tile anyway (EPB >= number of tiles).
template <bool kBF16>
static bool launch_fused_t(const moe_dims &dm, const void *x, const void *w_router,
                           const float *bias, float *logits, const int32_t *q,
                           int32_t *topk_idx, float *topk_w, float *mass_part, int32_t *d_err,
                           const RouteOpts &o, hipStream_t s) {
    const int n_et = (dm.E + 15) / 16;
    const int epb = logits_epb(dm.T, dm.E);
    if (!o.plain() || epb < n_et) return false;
    const dim3 grid((unsigned)((dm.T + 15) / 16)), block(64 * kLogitSplit);
#define MOE_FUSED(EPB, NV)                                                                    \
    route_fused_kernel<kBF16, EPB, kScoreSoftmax, false, NV><<<grid, block, 0, s>>>(          \
        x, w_router, bias, logits, dm.T, dm.d, dm.E, q, dm.k, topk_idx, topk_w, mass_part,   \
        d_err, o)
    switch (epb) {
    case 1: MOE_FUSED(1, 4); break;
    case 2: MOE_FUSED(2, 4); break;
    case 4: MOE_FUSED(4, 4); break;
    default: MOE_FUSED(8, 8); break;
    }
#undef MOE_FUSED
    return true;
}

hipError_t launch_route(const moe_dims &dm, const void *x, const void *w_router,
                        const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                        float *mass_part, float *prob_mass, const int32_t *token_mult,
                        int32_t *d_err, hipStream_t s, const RouteOpts &o, bool defer_mass) {
    const int64_t T = dm.T;
    const int E = dm.E;
    if (T > 0) {
        const int64_t tblk = (T + kTopkTokPerBlock - 1) / kTopkTokPerBlock;
        float *mp = prob_mass ? mass_part : nullptr;
        if (defer_mass) prob_mass = nullptr;   // the caller's next launch reduces mass_part
        const bool fused =
            dm.dtype == MOE_BF16
                ? launch_fused_t<true>(dm, x, w_router, bias, logits, token_mult, topk_idx,
                                       topk_w, mp, d_err, o, s)
                : launch_fused_t<false>(dm, x, w_router, bias, logits, token_mult, topk_idx,
                                        topk_w, mp, d_err, o, s);
        if (fused) {
            if (prob_mass)
                mass_reduce_kernel<<<dim3((E + 3) / 4), dim3(256), 0, s>>>(mass_part, tblk, E, prob_mass);
            return hipGetLastError();
        }
        const hipError_t le = launch_router_logits(dm, x, w_router, bias, logits, s);
        if (le != hipSuccess) return le;
        const bool h = o.hash_table != nullptr;
        switch (o.fn * 2 + (h ? 1 : 0)) {
        case 0: launch_topk_t<kScoreSoftmax, false>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        case 1: launch_topk_t<kScoreSoftmax, true>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        case 2: launch_topk_t<kScoreSigmoid, false>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        case 3: launch_topk_t<kScoreSigmoid, true>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        case 4: launch_topk_t<kScoreSqrtSoftplus, false>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        default: launch_topk_t<kScoreSqrtSoftplus, true>(dm, tblk, logits, token_mult, topk_idx, topk_w, mp, d_err, o, s); break;
        }
        if (prob_mass)
            mass_reduce_kernel<<<dim3((E + 3) / 4), dim3(256), 0, s>>>(mass_part, tblk, E, prob_mass);
    } else if (prob_mass) {
        mass_reduce_kernel<<<dim3((E + 3) / 4), dim3(256), 0, s>>>(mass_part, 0, E, prob_mass);
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
