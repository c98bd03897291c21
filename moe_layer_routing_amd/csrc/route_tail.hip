// route_tail.hip -- the routing tail of a small batch (1 <= T <= kSmallT) in one block.
//
// Decode-sized batches spend most of their routing time in kernel boundaries: every step
// of the multi-kernel path (top-k, probability-mass reduction, histogram, scan, stable
// scatter, tile list) is a launch plus a memory round trip for a few hundred bytes. This
// kernel runs those steps back to back in one 1024-thread block, with the logits, ids,
// counts and offsets kept in LDS; no step reads back what an earlier one stored to memory,
// so its barriers wait only for LDS traffic. It computes the same functions as the multi-kernel path, in the
// same floating-point order, so each output is bitwise the one that path gives for the
// same T:
//   * top-k: wave w routes tokens 4w .. 4w+3 (one per 16-lane row) with the routine the
//     multi-block kernel uses (for every router variant)
//     ("0 train-infer mismatch for Open-weight MoE RL in Open-source code", "The router:
//     matching expert ids and weights"); replay ("Total Router Recall") is validated and
//     passed through;
//   * probability mass ("HARTS ...", eq. (20)): a wave's partial is its four tokens' q·p
//     added in token order from 0; waves 4b .. 4b+3 form the 16-token group b of the
//     multi-block kernel; group partials are ((m0 + m1) + m2) + m3 and the groups
//     (at most four) are added as the 256-thread reduction tree adds them,
//     (P0 + P2) + (P1 + P3), absent groups being exact zeros;
//   * permutation ("RoutePack ...", Sec. 2.1): the stable counting sort by expert (by the
//     expert's physical slot under a placement map, Sec. 3), which has one result; wave w
//     ranks the flat assignments [64w, 64w + 64);
//   * token tiles: ceil(count_e / bt) tiles per expert in expert order.
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kTailWaves = 16;
constexpr int kTailTokPerWave = kTopkTokPerBlock / 4;
constexpr int kTailMaxA = kSmallT * kMaxK;
static_assert(kTailWaves * kTailTokPerWave == kSmallT, "one wave per 4 tokens");
static_assert(kTailMaxA / kWave <= kTailWaves, "one wave per 64 assignments");

template <bool kReplay, int kFn, bool kHash, int NV>
__global__ __launch_bounds__(64 * kTailWaves) void route_tail_kernel(
    float *__restrict__ logits, const int32_t *__restrict__ q,
    const int32_t *__restrict__ idx_in, const float *__restrict__ w_in, int T, int E, int k,
    int bt, int cap, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    float *__restrict__ prob_mass, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int64_t *__restrict__ weighted_counts, int32_t *__restrict__ tiles,
    int32_t *__restrict__ d_err, const int32_t *__restrict__ slot_map, RouteOpts opts,
    const float *__restrict__ part, const float *__restrict__ bias) {
    __shared__ int32_t ids[kTailMaxA];
    __shared__ int32_t wstart[kTailMaxA / kWave][kMaxE];  // per-wave counts -> run starts
    __shared__ int32_t eoff[kMaxE + 1];                    // counts -> exclusive offsets
    __shared__ int32_t toff[kMaxE + 1];                    // tile starts
    __shared__ unsigned long long wsum[kMaxE];
    __shared__ float mpt[kSmallT][kMaxE];                  // q·p per token, router mode
    __shared__ float lgl[kChainSumMax];                    // logits formed here (T*E <= 2048)
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int A = T * k;
    for (int i = tid; i < (kTailMaxA / kWave) * kMaxE; i += 64 * kTailWaves)
        (&wstart[0][0])[i] = 0;
    for (int i = tid; i < kMaxE; i += 64 * kTailWaves) wsum[i] = 0;
    if (!kReplay && part) {
        // router logits from the chain partials, in chain order, then the bias
        // (two logits per thread and pass: their 32 partial loads are in flight together)
        const int TE = T * E;
        constexpr int kNT = 64 * kTailWaves;
        for (int i0 = tid; i0 < TE; i0 += 2 * kNT) {
            const int i1 = min(i0 + kNT, TE - 1);
            float p0[kLogitChains], p1[kLogitChains];
#pragma unroll
            for (int c = 0; c < kLogitChains; ++c) {
                p0[c] = part[(int64_t)c * TE + i0];
                p1[c] = part[(int64_t)c * TE + i1];
            }
            float v0 = p0[0], v1 = p1[0];
#pragma unroll
            for (int c = 1; c < kLogitChains; ++c) {
                v0 = v0 + p0[c];
                v1 = v1 + p1[c];
            }
            const float l0 = bias ? v0 + bias[i0 % E] : v0;
            const float l1 = bias ? v1 + bias[i1 % E] : v1;
            logits[i0] = l0;
            lgl[i0] = l0;
            if (i0 + kNT < TE) {
                logits[i1] = l1;
                lgl[i1] = l1;
            }
        }
        lds_barrier();
    }

    // ---- top-k (or replay validation); ids also go to LDS
    int err = 0;
    if constexpr (kReplay) {
        if (tid < T) {
            int seen[kMaxK];
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                seen[j] = -1;
                if (j < k) {
                    const int e = idx_in[tid * k + j];
                    const float wv = w_in[tid * k + j];
                    seen[j] = e;
                    if (e < 0 || e >= E) err |= MOE_DERR_IDX_RANGE;
                    if (!__builtin_isfinite(wv)) err |= MOE_DERR_NONFINITE;
#pragma unroll
                    for (int i = 0; i < kMaxK; ++i)
                        if (i < j && seen[i] == e) err |= MOE_DERR_IDX_DUP;
                    topk_idx[tid * k + j] = e;
                    topk_w[tid * k + j] = wv;
                    ids[tid * k + j] = e;
                }
            }
        }
    } else {
        float qp[kRowVals];
        if (wave * kTailTokPerWave < T) {   // waves past the batch hold zeros
            // logits formed here are read from the LDS copy (the values stored to memory);
            // a separate call, so that its reads are LDS reads, which wait for nothing else
            if (part)
                route_rows<kFn, kHash, NV>(lgl, q, (int64_t)wave * kTailTokPerWave, T, E, k,
                                           opts, topk_idx, topk_w, ids, qp, err);
            else
                route_rows<kFn, kHash, NV>(logits, q, (int64_t)wave * kTailTokPerWave, T, E, k,
                                           opts, topk_idx, topk_w, ids, qp, err);
        } else {
#pragma unroll
            for (int i = 0; i < kRowVals; ++i) qp[i] = 0.f;
        }
        if (prob_mass) {
            const int row = wave * 4 + (lane >> 4), c = lane & 15;
#pragma unroll
            for (int i = 0; i < kRowVals; ++i)
                if (c + 16 * i < E) mpt[row][c + 16 * i] = qp[i];
        }
    }
    wave_raise(err, d_err);
    lds_barrier();

    // ---- per-wave expert counts and in-wave stable ranks
    const int nwv = (A + kWave - 1) / kWave;
    const int a = wave * kWave + lane;
    int e0 = -1, before = 0;
    bool valid = false;
    err = 0;
    if (wave < nwv) {  // uniform per wave
        e0 = a < A ? slot_of(slot_map, ids[a], E, err) : -1;   // physical slot
        valid = e0 >= 0;
        const uint64_t peers = wave_match9(valid ? (uint32_t)e0 : 0x1ffu);
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        before = __popcll(peers & lt_mask);
        if (valid && (peers >> lane) == 1ull) wstart[wave][e0] = __popcll(peers);
        if (valid && weighted_counts && q)
            atomicAdd(&wsum[e0], (unsigned long long)(uint32_t)q[a / k]);
    }
    wave_raise(err, d_err);
    lds_barrier();

    // ---- per expert: run starts of each wave, totals, weighted counts, probability mass
    if (tid < E) {
        int32_t run = 0;
        for (int w = 0; w < nwv; ++w) {
            const int32_t c = wstart[w][tid];
            wstart[w][tid] = run;
            run += c;
        }
        counts[tid] = run;
        eoff[tid] = run;
        if (weighted_counts) weighted_counts[tid] = q ? (int64_t)wsum[tid] : (int64_t)run;
        if (!kReplay && prob_mass) {
            float P[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float v = 0.f;
#pragma unroll
                for (int w = 4 * b; w < 4 * b + 4; ++w) {
                    float m = 0.f + mpt[4 * w][tid];
                    m = m + mpt[4 * w + 1][tid];
                    m = m + mpt[4 * w + 2][tid];
                    m = m + mpt[4 * w + 3][tid];
                    v = (w == 4 * b) ? m : v + m;
                }
                P[b] = v;
            }
            prob_mass[tid] = (P[0] + P[2]) + (P[1] + P[3]);
        }
    }
    lds_barrier();

    // ---- exclusive scans over experts (wave 0; lane l holds experts 4l .. 4l+3)
    if (wave == 0) {
        int32_t c[4], nt[4], cs = 0, ts = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            c[i] = e < E ? eoff[e] : 0;
            nt[i] = (c[i] + bt - 1) / bt;
            cs += c[i];
            ts += nt[i];
        }
        int32_t cx = wave_incl_scan(cs) - cs, tx = wave_incl_scan(ts) - ts;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) {
                eoff[e] = cx;
                toff[e] = tx;
            }
            cx += c[i];
            tx += nt[i];
        }
        if (lane == 63) {
            eoff[E] = cx;
            toff[E] = tx;
        }
    }
    lds_barrier();

    // ---- outputs: offsets, perm / inv, tile list
    if (tid <= E) offsets[tid] = eoff[tid];
    if (tid == 0) tiles[0] = min(toff[E], cap);
    if (wave < nwv) {
        if (valid) {
            const int32_t pos = eoff[e0] + wstart[wave][e0] + before;
            perm[pos] = a;
            inv[a] = pos;
        } else if (a < A) {
            inv[a] = -1;
        }
    }
    if (tid < E) {
        const int32_t cnt = eoff[tid + 1] - eoff[tid], p0 = eoff[tid];
        const int32_t nt = (cnt + bt - 1) / bt;
        for (int i = 0; i < nt; ++i) {
            const int32_t slot = toff[tid] + i;
            if (slot >= cap) break;
            int32_t *d = tiles + 1 + 3 * slot;
            d[0] = tid;
            d[1] = p0 + i * bt;
            d[2] = min(bt, cnt - i * bt);
        }
    }
}

}  // namespace

template <bool kReplay, int kFn, bool kHash>
static void launch_tail_t(const moe_dims &dm, int bt, int cap, float *logits,
                          const int32_t *q, const int32_t *idx_in, const float *w_in,
                          int32_t *topk_idx, float *topk_w, float *prob_mass, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv,
                          int64_t *weighted_counts, int32_t *tiles, int32_t *d_err,
                          const int32_t *slot_map, const RouteOpts &o, const float *part,
                          const float *bias, hipStream_t s) {
    auto go = [&](auto nv) {
        route_tail_kernel<kReplay, kFn, kHash, decltype(nv)::value>
            <<<dim3(1), dim3(64 * kTailWaves), 0, s>>>(
                logits, q, idx_in, w_in, (int)dm.T, dm.E, dm.k, bt, cap, topk_idx, topk_w,
                prob_mass, counts, offsets, perm, inv, weighted_counts, tiles, d_err, slot_map,
                o, part, bias);
    };
    if constexpr (kReplay) go(std::integral_constant<int, kRowVals>{});   // no top-k
    else with_row_vals(dm.E, go);
}

hipError_t launch_small_tail(const moe_dims &dm, const float *logits_in, const int32_t *q,
                             const int32_t *idx_in, const float *w_in, int32_t *topk_idx,
                             float *topk_w, float *prob_mass, int32_t *counts,
                             int32_t *offsets, int32_t *perm, int32_t *inv,
                             int64_t *weighted_counts, int32_t *tiles, int32_t *d_err,
                             hipStream_t s, const int32_t *slot_map, const RouteOpts &o,
                             const float *logit_part, const float *bias) {
    // the block writes the logits itself when it forms them from chain partials
    float *logits = const_cast<float *>(logits_in);
    if (dm.T < 1 || dm.T > kSmallT || dm.E > kMaxE || dm.k > kMaxK)
        return hipErrorInvalidValue;
    if (logit_part && dm.T * dm.E > kChainSumMax) return hipErrorInvalidValue;   // LDS copy
    if (slot_map) {
        const hipError_t me = launch_check_slot_map(slot_map, dm.E, d_err, s);
        if (me != hipSuccess) return me;
    }
    const int bt = select_tile_m(dm);
    const int cap = (int)max_m_tiles(dm.T * dm.k, dm.E, bt);
#define MOE_TAIL_ARGS dm, bt, cap, logits, q, idx_in, w_in, topk_idx, topk_w, prob_mass, \
        counts, offsets, perm, inv, weighted_counts, tiles, d_err, slot_map, o, logit_part, bias, s
    if (idx_in) {
        launch_tail_t<true, kScoreSoftmax, false>(MOE_TAIL_ARGS);
    } else {
        switch (o.fn * 2 + (o.hash_table ? 1 : 0)) {
        case 0: launch_tail_t<false, kScoreSoftmax, false>(MOE_TAIL_ARGS); break;
        case 1: launch_tail_t<false, kScoreSoftmax, true>(MOE_TAIL_ARGS); break;
        case 2: launch_tail_t<false, kScoreSigmoid, false>(MOE_TAIL_ARGS); break;
        case 3: launch_tail_t<false, kScoreSigmoid, true>(MOE_TAIL_ARGS); break;
        case 4: launch_tail_t<false, kScoreSqrtSoftplus, false>(MOE_TAIL_ARGS); break;
        default: launch_tail_t<false, kScoreSqrtSoftplus, true>(MOE_TAIL_ARGS); break;
        }
    }
#undef MOE_TAIL_ARGS
    return hipGetLastError();
}

}  // namespace moe
