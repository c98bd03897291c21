// grouped_ffn.hip -- grouped SwiGLU expert GEMMs over variable-length expert segments.
//
// Numerics ("0 train-infer mismatch for Open-weight MoE RL in Open-source code"):
//  * "Matrix multiplication: the same reduction along K": every output element is one
//    FP32 accumulator fed by the same MFMA instruction over the same K-steps in
//    increasing K, for every segment length, tile height and grid size (no split-K);
//  * "SwiGLU: rounding after the multiply": gate and up stay FP32, silu(g)*u is formed
//    in FP32 and rounded once to the storage type;
//  * "The experts: keeping the route weight inside the accumulator": the down
//    projection is kept in FP32 (y) so the combine can apply the route weight before the
//    single final rounding.
//
// Shape of the work ("RoutePack ...", Sec. 2.3: local experts run as one grouped
// operation): expert e owns rows [offsets[e], offsets[e+1]) of the permuted activations.
// A small kernel turns the device-resident offsets into a list of (expert, first row,
// rows) token tiles, so no count ever travels to the host. GEMM blocks beyond the list's
// length exit at once.
//
// Operand roles: the MFMA A operand is a 16-row slice of the expert's weight matrix
// (output features), the B operand a 16-token slice of activations. With the result
// layout of v_mfma_f32_16x16x{32bf16,4f32} (lane l holds token l%16 and features
// 4*(l/16)+0..3) every lane stores 4 consecutive features of one token row.
#include <type_traits>

#include "route_dev.h"

namespace moe {
namespace {


// tiles[0] = number of token tiles; tiles[1 + 3*i ..] = (expert, first row, rows).
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t *__restrict__ offsets,
                                                          int E, int64_t A, int bt,
                                                          int64_t capacity,
                                                          int32_t *__restrict__ tiles) {
    __shared__ int32_t pre[kMaxE + 1];
    const int e = threadIdx.x;
    int32_t p0 = 0, cnt = 0, nt = 0;
    if (e < E) {
        const int64_t lo = min<int64_t>(max<int64_t>(offsets[e], 0), A);
        const int64_t hi = min<int64_t>(max<int64_t>(offsets[e + 1], lo), A);
        p0 = (int32_t)lo;
        cnt = (int32_t)(hi - lo);
        nt = (cnt + bt - 1) / bt;
        pre[e] = nt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int i = 0; i < E; ++i) {
            const int32_t c = pre[i];
            pre[i] = acc;
            acc += c;
        }
        pre[E] = acc;
        tiles[0] = (int32_t)min<int64_t>(acc, capacity);
    }
    __syncthreads();
    if (e < E) {
        for (int i = 0; i < nt; ++i) {
            const int64_t slot = (int64_t)pre[e] + i;
            if (slot >= capacity) break;
            int32_t *d = tiles + 1 + 3 * slot;
            d[0] = e;
            d[1] = p0 + i * bt;
            d[2] = min(bt, cnt - i * bt);
        }
    }
}

// Row of the activation matrix that tile row rr reads: rr itself (segment-relative rows of
// x_perm / h), or, when the dispatch gather is fused, the token perm[p0+rr] / k of x
// (clamped into [0, gT) so that a corrupted permutation cannot read outside x).
__device__ __forceinline__ int64_t act_row(const int32_t *gperm, int gk, int64_t gT, int p0,
                                           int rr) {
    if (!gperm) return rr;
    const int64_t t = (int64_t)max(gperm[p0 + rr], 0) / gk;
    return t < gT ? t : gT - 1;
}

// Block -> (token tile, feature tile). The grid is sized for the most tiles any routing
// can produce, but only ntiles*nft blocks have work; the hardware deals consecutive block
// ids round-robin over the 8 XCDs, so the live blocks are ids 0..live-1 and the rest leave
// at once. Among the live ids, each XCD gets one contiguous range of logical tiles in
// (token tile, feature tile) order, so blocks that share a token slice or an expert's
// weights share that XCD's L2. Renumbering over the live count (not the grid) keeps all 8
// XCDs busy when few tiles are live (decode) and when padding leaves the grid's tail empty.
__device__ __forceinline__ bool block_tile(int ntiles, int nft, int &mt, int &ft) {
    const uint32_t live = (uint32_t)ntiles * (uint32_t)nft, bid = blockIdx.x;
    if (bid >= live) return false;
    const uint32_t xcd = bid & 7u, loc = bid >> 3, per = live >> 3, rem = live & 7u;
    const uint32_t L = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
    mt = (int)(L / (uint32_t)nft);
    ft = (int)(L % (uint32_t)nft);
    return true;
}

// kGateUp: out = h[A, I] = round(silu(x w_gate^T) * (x w_up^T)), K = d, N = I,
//          the weight tile stacks BW/2 gate rows over the matching BW/2 up rows.
// else:    out = y[A, d] (FP32) = h w2^T, K = I, N = d.
// Block tile: BW weight rows x BT tokens; WF x WT waves, each owning (BW/WF) x (BT/WT).
// K advances in stages of SRB bytes per row (64 or 128), double-buffered in LDS with a
// 16-byte pad per row; PF = 1 or 2 stages are in flight in registers ahead of the stage
// being computed. Every configuration walks K in the same MFMA steps, in the same order.
template <bool kBF16, bool kGateUp, int BW, int BT, int WF, int WT, int PF, int SRB, int WPE>
__global__ __launch_bounds__(64 * WF * WT)
__attribute__((amdgpu_waves_per_eu(WPE, WPE))) void grouped_gemm_kernel(
    const uint8_t *__restrict__ act, const uint8_t *__restrict__ wgt, void *__restrict__ out,
    const int32_t *__restrict__ tiles, int K, int N, int nft,
    const int32_t *__restrict__ gperm, int gk, int64_t gT, float *__restrict__ gu_out) {
    constexpr int NTHR = 64 * WF * WT;
    constexpr int kRowBytes = SRB;                     // K bytes of one row per stage
    constexpr int kLdsStride = kRowBytes + 16;         // padded LDS row (bank spread)
    constexpr int kVecPerRow = kRowBytes / 16;         // 16-byte vectors per staged row
    constexpr int kEB = kBF16 ? 2 : 4;                 // element bytes
    constexpr int kSubBytes = kBF16 ? 64 : 16;         // bytes of K per MFMA step
    constexpr int kSub = kRowBytes / kSubBytes;        // MFMA K-steps per stage
    constexpr int kFeat = kGateUp ? BW / 2 : BW;       // output features per block
    constexpr int kWaveRows = (kGateUp ? BW / 2 : BW) / WF;
    constexpr int NFh = kWaveRows / 16;                // fragments per half (gate/up)
    constexpr int NF = kGateUp ? 2 * NFh : NFh;
    constexpr int NT = BT / WT / 16;
    constexpr int RPI = NTHR / kVecPerRow;             // rows one load round covers
    constexpr int LW = (BW + RPI - 1) / RPI;
    constexpr int LT = (BT + RPI - 1) / RPI;
    static_assert(NFh >= 1 && NT >= 1 && (PF == 1 || PF == 2), "bad tile shape");
    static_assert((kGateUp ? BW / 2 : BW) % (16 * WF) == 0 && BT % (16 * WT) == 0, "tile");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BW + BT) * kLdsStride];

    int mt, ft;
    if (!block_tile(tiles[0], nft, mt, ft)) return;
    const int e = tiles[1 + 3 * mt], p0 = tiles[2 + 3 * mt], nrows = tiles[3 + 3 * mt];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wf = wv % WF, wt = wv / WF;
    const int n0 = ft * kFeat;
    const int64_t rows_per_expert = kGateUp ? 2 * (int64_t)N : (int64_t)N;
    const uint32_t krow = (uint32_t)K * kEB;
    const uint8_t *wbase = wgt + (int64_t)e * rows_per_expert * krow;
    // activation rows: the tile's segment rows, or (gathered) the token rows perm[p] / k
    const uint8_t *abase = gperm ? act : act + (int64_t)p0 * krow;

    // byte offsets of this thread's staged 16-byte vectors (chunk c of rows r0 + i*RPI)
    const int c = tid % kVecPerRow, r0 = tid / kVecPerRow;
    uint32_t wo[LW], to[LT];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int r = min(r0 + i * RPI, BW - 1);
        int grow;
        if (kGateUp) {
            const int half = r >= BW / 2;
            grow = min(n0 + (half ? r - BW / 2 : r), N - 1) + (half ? N : 0);
        } else {
            grow = min(n0 + r, N - 1);
        }
        wo[i] = (uint32_t)grow * krow + c * 16;
    }
#pragma unroll
    for (int i = 0; i < LT; ++i)
        to[i] = (uint32_t)act_row(gperm, gk, gT, p0, min(r0 + i * RPI, nrows - 1)) * krow + c * 16;

    u32x4_t rw[PF][LW], rt[PF][LT];
    auto load_global = [&](int kt, auto slot) {
        constexpr int S = decltype(slot)::value;
        const uint32_t ko = (uint32_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < LW; ++i)
            if (BW % RPI == 0 || r0 + i * RPI < BW)
                rw[S][i] = *reinterpret_cast<const u32x4_t *>(wbase + wo[i] + ko);
#pragma unroll
        for (int i = 0; i < LT; ++i)
            if (BT % RPI == 0 || r0 + i * RPI < BT)
                rt[S][i] = *reinterpret_cast<const u32x4_t *>(abase + to[i] + ko);
    };
    auto store_lds = [&](int b, auto slot) {
        constexpr int S = decltype(slot)::value;
        uint8_t *sb = smem[b] + r0 * kLdsStride + c * 16;
#pragma unroll
        for (int i = 0; i < LW; ++i)
            if (BW % RPI == 0 || r0 + i * RPI < BW)
                *reinterpret_cast<u32x4_t *>(sb + i * RPI * kLdsStride) = rw[S][i];
#pragma unroll
        for (int i = 0; i < LT; ++i)
            if (BT % RPI == 0 || r0 + i * RPI < BT)
                *reinterpret_cast<u32x4_t *>(sb + (BW + i * RPI) * kLdsStride) = rt[S][i];
    };

    // LDS byte offsets of this lane's fragment rows
    const int r16 = lane & 15, g4 = lane >> 4;
    const int frag_lane = r16 * kLdsStride + g4 * (kBF16 ? 16 : 4);
    auto wrow = [&](int f) {
        if (kGateUp) return (f < NFh ? 0 : BW / 2) + wf * kWaveRows + (f % NFh) * 16;
        return wf * kWaveRows + f * 16;
    };
    auto trow = [&](int t) { return BW + wt * (BT / WT) + t * 16; };

    f32x4_t acc[NF][NT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // One stage: kSub MFMA K-steps. Fragments are double-buffered across K-steps: all LDS
    // reads of step kk+1 are issued before the MFMAs of step kk, and scheduling barriers
    // keep the compiler from folding the two phases back into one serial chain.
    using FragT = typename std::conditional<kBF16, bf16x8_t, float>::type;
    auto read_frags = [&](const uint8_t *sb, int kk, FragT (&a)[NF], FragT (&bv)[NT]) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
            a[f] = *reinterpret_cast<const FragT *>(sb + wrow(f) * kLdsStride + kk * kSubBytes);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            bv[t] = *reinterpret_cast<const FragT *>(sb + trow(t) * kLdsStride + kk * kSubBytes);
    };
    auto mfmas = [&](const FragT (&a)[NF], const FragT (&bv)[NT]) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (kBF16)
                    acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], bv[t], acc[f][t],
                                                                        0, 0, 0);
                else
                    acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[f], bv[t], acc[f][t], 0,
                                                                     0, 0);
            }
    };
    auto compute = [&](int b) {
        const uint8_t *sb = smem[b] + frag_lane;
        FragT a0[NF], b0[NT], a1[NF], b1[NT];
        read_frags(sb, 0, a0, b0);
#pragma unroll
        for (int kk = 0; kk < kSub; kk += 2) {
            if (kk + 1 < kSub) read_frags(sb, kk + 1, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            if (kk + 1 < kSub) {
                if (kk + 2 < kSub) read_frags(sb, kk + 2, a0, b0);
                __builtin_amdgcn_sched_barrier(0);
                mfmas(a1, b1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int nk = K / (kRowBytes / kEB);
    if constexpr (PF == 1) {
        load_global(0, S0{});
        store_lds(0, S0{});
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) load_global(kt + 1, S0{});
            compute(kt & 1);
            if (kt + 1 < nk) store_lds((kt + 1) & 1, S0{});
            __syncthreads();
        }
    } else {
        // two register stages: stage kt+2 is fetched while stage kt is computed, so each
        // global load has two compute phases to arrive. Unrolled by two so every register
        // stage index is a compile-time constant.
        load_global(0, S0{});
        if (nk > 1) load_global(1, S1{});
        store_lds(0, S0{});
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            if (kt + 2 < nk) load_global(kt + 2, S0{});
            compute(0);
            if (kt + 1 < nk) store_lds(1, S1{});
            __syncthreads();
            if (kt + 1 >= nk) break;
            if (kt + 3 < nk) load_global(kt + 3, S1{});
            compute(1);
            if (kt + 2 < nk) store_lds(0, S0{});
            __syncthreads();
        }
    }

    // epilogue
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = wt * (BT / WT) + t * 16 + r16;
        if (m >= nrows) continue;
        const int64_t row = (int64_t)p0 + m;
        if constexpr (kGateUp) {
#pragma unroll
            for (int f = 0; f < NFh; ++f) {
                const int feat = n0 + wf * kWaveRows + f * 16 + g4 * 4;
                if (feat >= N) continue;
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gv = acc[f][t][i];
                    const float uv = acc[f + NFh][t][i];
                    const float silu = gv / (1.0f + expf(-gv));
                    hv[i] = silu * uv;
                }
                if constexpr (kBF16) {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
                    pk.y = (uint32_t)f32_to_bf16(hv[2]) | ((uint32_t)f32_to_bf16(hv[3]) << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + row * N + feat) = pk;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(out) + row * N + feat) =
                        make_float4(hv[0], hv[1], hv[2], hv[3]);
                }
                if (gu_out) {   // the pre-activations g and u, FP32 [rows][2N], as computed
                    store_nt(gu_out + row * 2 * N + feat,
                             make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]));
                    store_nt(gu_out + row * 2 * N + N + feat,
                             make_float4(acc[f + NFh][t][0], acc[f + NFh][t][1],
                                         acc[f + NFh][t][2], acc[f + NFh][t][3]));
                }
            }
        } else {
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int feat = n0 + wf * kWaveRows + f * 16 + g4 * 4;
                if (feat >= N) continue;
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + row * N + feat) =
                    make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]);
            }
        }
    }
}


// ------------------------------------------------------------------------------------
// Same GEMM with 128-byte K stages (64 bf16 per row): every DMA lane group of 8 covers one
// full 128-byte line of a row, which the global->LDS path moves at about 1.7x the rate of
// 64-byte halves. A stage is 8-row x 128-byte LDS blocks; lane l of a DMA instruction
// fetches chunk (l%8) ^ swz(row) of row l/8. With swz(row) = row % 8, the fragment reads
// (16 rows, one 16-byte chunk each) are free of LDS bank conflicts on gfx950 (measured
// with SQ_LDS_BANK_CONFLICT; also folding bit 3 of the row into the swizzle conflicts).
// Two slots: stage kt+1 is in flight while the two 32-deep MFMA K-steps of stage kt run;
// one wait + one s_barrier per stage.
__device__ __forceinline__ int chunk_swizzle8(int r) { return r & 7; }


template <int NBW, int NW, bool kWeightNT = false>
__device__ __forceinline__ void dma_stage128(uint8_t *slot, const uint8_t *wbase,
                                             const uint8_t *abase, const uint32_t (&off)[NBW],
                                             uint32_t is_act_mask, int kt, uint32_t wstride,
                                             int wv) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass never runs this; it cannot parse the builtin
    const uint32_t ako = (uint32_t)kt * 128u, wko = (uint32_t)kt * wstride;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const bool is_act = (is_act_mask >> i) & 1u;   // wave-uniform
        auto *dst = (__attribute__((address_space(3))) void *)(slot + (wv + i * NW) * 1024);
        if (kWeightNT && !is_act)   // weight rows read once: nontemporal (cache policy nt)
            __builtin_amdgcn_global_load_lds(wbase + off[i] + wko, dst, 16, 0, 2);
        else
            __builtin_amdgcn_global_load_lds(
                (is_act ? abase : wbase) + off[i] + (is_act ? ako : wko), dst, 16, 0, 0);
    }
#endif
}

// kKMajor (plain mode only): the weights are stored K-major, wgt[e][k][n] (n contiguous),
// as the data-gradient GEMMs of the backward read w2 and w13. A stage's 64 K-rows of the
// BW features are copied as stored (2 BW bytes per K-row, 16-byte chunks swizzled by
// kmajor_swz(k-row)), and the weight fragments come from gfx950's transposing LDS read
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives in slot j the element that
// lane 4j + i/4 named at position i%4, so lane s naming K-row 8g + s/4 (then + 4) at
// features f + 4(s%4) hands lane i feature f + i at K-rows 8g + 0..7 -- the operand a
// row-major weight tile gives, in the same K positions, hence the same bits.
//
// dma128_tile computes one block's tile: feature tile ft of expert e's weights against the
// output's token rows p0 .. p0 + nrows - 1, whose activation rows start at abase (or are
// gathered through gperm); ring is the block's LDS ring of NS stages.
template <bool kGateUp, int BW, int BT, int WF, int WT, int NS, bool kKMajor, int kGrad>
__device__ __forceinline__ void dma128_tile(uint8_t *ring, const uint8_t *__restrict__ abase,
                                            const uint8_t *__restrict__ wgt,
                                            void *__restrict__ out, int K, int N, int e, int p0,
                                            int nrows, int ft, const int32_t *__restrict__ gperm,
                                            int gk, int64_t gT, const float *__restrict__ dh,
                                            float *__restrict__ gu_out) {
    constexpr int NW = WF * WT;
    constexpr int NBLK = (BW + BT) / 8;                // 8-row LDS blocks per stage
    constexpr int NBW = NBLK / NW;                     // DMA instructions per wave per stage
    constexpr int kStageBytes = NBLK * 1024;
    constexpr int kFeat = kGateUp ? BW / 2 : BW;
    constexpr int kWaveRows = (kGateUp ? BW / 2 : BW) / WF;
    constexpr int NFh = kWaveRows / 16;
    constexpr int NF = kGateUp ? 2 * NFh : NFh;
    constexpr int NT = BT / WT / 16;
    static_assert(NBLK % NW == 0 && NBW <= 32 && NFh >= 1 && NT >= 1, "bad tile shape");
    static_assert(BW % 16 == 0 && (BW / 2) % 16 == 0, "16-row fragments");
    static_assert(NS >= 2 && NBW * (NS - 2) < 64, "ring depth");
    static_assert(!kKMajor || (!kGateUp && BW >= 64 && BW <= 512), "K-major: plain mode");
    constexpr int kCPR = BW / 8;                        // K-major: 16-byte chunks per K-row


    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wf = wv % WF, wt = wv / WF;
    const int n0 = ft * kFeat;
    const int64_t rows_per_expert = kGateUp ? 2 * (int64_t)N : (int64_t)N;
    const uint32_t krow = (uint32_t)K * 2u;
    const uint8_t *wbase = wgt + (int64_t)e * rows_per_expert * krow;

    // DMA sources (byte offsets from wbase / abase) of this lane's row in each block
    const int rb = lane >> 3;
    uint32_t off[NBW];
    uint32_t is_act = 0;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int row = (wv + i * NW) * 8 + rb;
        const int chunk = (lane & 7) ^ chunk_swizzle8(row);
        if (kKMajor && row < BW) {
            // instruction block bi moves K-rows bi * (64 / kCPR) + lane / kCPR of the stage;
            // lane chunk position p holds logical chunk p ^ kmajor_swz(k-row)
            const int bi = wv + i * NW;
            const int kr = bi * (64 / kCPR) + lane / kCPR;
            const int lc = (lane % kCPR) ^ kmajor_swz<kCPR>(kr);
            off[i] = (uint32_t)kr * (uint32_t)N * 2u + (uint32_t)min(n0 + 8 * lc, N - 8) * 2u;
        } else if (row < BW) {
            int grow;
            if (kGateUp) {
                const int half = row >= BW / 2;
                grow = min(n0 + (half ? row - BW / 2 : row), N - 1) + (half ? N : 0);
            } else {
                grow = min(n0 + row, N - 1);
            }
            off[i] = (uint32_t)grow * krow + chunk * 16;
        } else {
            off[i] = (uint32_t)act_row(gperm, gk, gT, p0, min(row - BW, nrows - 1)) * krow +
                     chunk * 16;
            is_act |= 1u << i;
        }
    }

    // fragment read offsets: row r16 of a 16-row fragment, K-chunk kk*4 + g4 of the stage
    const int r16 = lane & 15, g4 = lane >> 4;
    const int lane_off0 = (r16 >> 3) * 1024 + (r16 & 7) * 128 + ((g4 ^ chunk_swizzle8(r16)) << 4);
    const int lane_off1 = (r16 >> 3) * 1024 + (r16 & 7) * 128 +
                          (((4 + g4) ^ chunk_swizzle8(r16)) << 4);
    auto wrow = [&](int f) {
        if (kGateUp) return (f < NFh ? 0 : BW / 2) + wf * kWaveRows + (f % NFh) * 16;
        return wf * kWaveRows + f * 16;
    };
    auto trow = [&](int t) { return BW + wt * (BT / WT) + t * 16; };

    f32x4_t acc[NF][NT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // K-major weight fragment f of K-step kk: this lane names K-row 32 kk + 8 g4 + r16/4
    // (then + 4) at features wrow(f) + 4 (r16 % 4) .. + 3
    const int kmr = 8 * g4 + (r16 >> 2);
    const int kms = kmajor_swz<kCPR>(kmr);           // equal for K-rows kmr and kmr + 4
    auto kmajor_ptr = [&](const uint8_t *stage, int kk, int f) {
        const int byte = 2 * wrow(f) + 8 * (r16 & 3);
        const int pb = (((byte >> 4) ^ kms) << 4) | (byte & 15);
        return stage + (32 * kk + kmr) * (2 * BW) + pb;
    };
    auto kstep = [&](const uint8_t *sb, const uint8_t *stage, int kk) {
        bf16x8_t a[NF], b[NT];
        if constexpr (kKMajor) {
            // transposing reads from inline assembly (no compiler wait on the DMA ring),
            // the token fragments as usual, then one lgkmcnt(0) for both
            i32x2_t lo[NF], hi[NF];
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const uint8_t *p = kmajor_ptr(stage, kk, f);
                lo[f] = tr_read(p);
                hi[f] = tr_read(p + 4 * (2 * BW));
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
                b[t] = *reinterpret_cast<const bf16x8_t *>(sb + (trow(t) >> 3) * 1024);
            tr_fence();
#pragma unroll
            for (int f = 0; f < NF; ++f) a[f] = tr_take(lo[f], hi[f]);
        } else {
#pragma unroll
            for (int f = 0; f < NF; ++f)
                a[f] = *reinterpret_cast<const bf16x8_t *>(sb + (wrow(f) >> 3) * 1024);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                b[t] = *reinterpret_cast<const bf16x8_t *>(sb + (trow(t) >> 3) * 1024);
        }
        // the MFMA block at raised wave priority: while one wave of a SIMD issues MFMAs the
        // others' fragment reads and DMA issue wait (measured 0 to +1 %, same bytes)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], b[t], acc[f][t], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // NS-slot ring: stages kt+1 .. kt+NS-1 are in flight while stage kt is computed. At
    // iteration kt (after the barrier that made stage kt resident) stage kt+NS-1 goes into
    // the slot stage kt-1 has left; before the next barrier each wave waits for its own DMA
    // of stage kt+1 (the NS-2 newer stages may stay in flight) and its own LDS reads.
    // a wave whose features or tokens are all padding issues no MFMAs (loop-invariant)
    const bool active = (n0 + wf * kWaveRows < N) && (wt * (BT / WT) < nrows);
    const int nk = K >> 6;
    // bytes one stage advances in the weights: 64 K-values of a row, or 64 K-rows
    const uint32_t wstride = kKMajor ? 64u * (uint32_t)N * 2u : 128u;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nk)
            dma_stage128<NBW, NW, (BT < 128)>(ring + st * kStageBytes, wbase, abase, off, is_act, st, wstride,
                                  wv);
    if (NS - 2 < nk) wait_vm_lgkm0<NBW * (NS - 2)>();
    else wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    for (int kt = 0; kt < nk; ++kt) {
        uint8_t *cur = ring + (kt % NS) * kStageBytes;
        if (kt + NS - 1 < nk)
            dma_stage128<NBW, NW, (BT < 128)>(ring + ((kt + NS - 1) % NS) * kStageBytes, wbase, abase, off,
                                  is_act, kt + NS - 1, wstride, wv);
        if (active) {
            kstep(cur + lane_off0, cur, 0);
            kstep(cur + lane_off1, cur, 1);
        }
        if (kt + 1 < nk) {
            if (kt + NS - 1 < nk) wait_vm_lgkm0<NBW * (NS - 2)>();
            else wait_vm_lgkm0<0>();
            __builtin_amdgcn_s_barrier();
        }
    }

    if constexpr (!kGateUp && BT >= 128) {
        // plain FP32 output of the large tiles, staged through the ring: one wave row of
        // tokens (RP rows) per pass, row stride BW + 4 floats; then every thread stores
        // consecutive 16-byte pieces of whole output rows (instead of 64-byte row pieces
        // from the result lanes). The values are the accumulators, unchanged.
        constexpr int RP = BT / WT, kLd = BW + 4, kRow4 = BW / 4;
        static_assert(RP * kLd * 4 <= NS * kStageBytes, "staging fits the ring");
        float *stg = reinterpret_cast<float *>(ring);
        float *outf = static_cast<float *>(out);
        __syncthreads();   // every wave is past its last fragment read; no DMA is pending
#pragma unroll 1
        for (int q = 0; q < WT; ++q) {
            if (wt == q) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        *reinterpret_cast<float4 *>(stg + (t * 16 + r16) * kLd + wf * kWaveRows +
                                                    f * 16 + g4 * 4) =
                            make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]);
            }
            __syncthreads();
            for (int idx = tid; idx < RP * kRow4; idx += 64 * NW) {
                const int r = idx / kRow4, c = (idx % kRow4) * 4;
                const int m = q * RP + r;
                if (m < nrows && n0 + c < N)
                    store_nt(outf + ((int64_t)p0 + m) * N + n0 + c,
                             *reinterpret_cast<const float4 *>(stg + r * kLd + c));
            }
            __syncthreads();
        }
        return;
    }
    // epilogue (same arithmetic and layout as grouped_gemm_kernel)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = wt * (BT / WT) + t * 16 + r16;
        if (m >= nrows) continue;
        const int64_t row = (int64_t)p0 + m;
        if constexpr (kGateUp && kGrad != 0) {
            // backward: the SwiGLU derivative of the recomputed gate and up values with
            // dh [rows][N]; d_gu [rows][2N] (bf16 for kGrad 1, FP32 for kGrad 2)
#pragma unroll
            for (int f = 0; f < NFh; ++f) {
                const int feat = n0 + wf * kWaveRows + f * 16 + g4 * 4;
                if (feat >= N) continue;
                const float4 d4 = *reinterpret_cast<const float4 *>(dh + row * N + feat);
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
                float dg[4], du[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    swiglu_grad(acc[f][t][i], acc[f + NFh][t][i], dv[i], dg[i], du[i]);
                store_dgu4<kGrad == 1>(out, row * 2 * N + feat, N, dg, du);
            }
        } else if constexpr (kGateUp) {
#pragma unroll
            for (int f = 0; f < NFh; ++f) {
                const int feat = n0 + wf * kWaveRows + f * 16 + g4 * 4;
                if (feat >= N) continue;
                float hv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gv = acc[f][t][i];
                    const float uv = acc[f + NFh][t][i];
                    const float silu = gv / (1.0f + expf(-gv));
                    hv[i] = silu * uv;
                }
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
                pk.y = (uint32_t)f32_to_bf16(hv[2]) | ((uint32_t)f32_to_bf16(hv[3]) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + row * N + feat) = pk;
                if (gu_out) {   // the pre-activations g and u, FP32 [rows][2N], as computed
                    store_nt(gu_out + row * 2 * N + feat,
                             make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]));
                    store_nt(gu_out + row * 2 * N + N + feat,
                             make_float4(acc[f + NFh][t][0], acc[f + NFh][t][1],
                                         acc[f + NFh][t][2], acc[f + NFh][t][3]));
                }
            }
        } else {
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int feat = n0 + wf * kWaveRows + f * 16 + g4 * 4;
                if (feat >= N) continue;
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + row * N + feat) =
                    make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]);
            }
        }
    }
}

template <bool kGateUp, int BW, int BT, int WF, int WT, int WPE, int NS, bool kKMajor = false,
          int kGrad = 0>
__global__ __launch_bounds__(64 * WF * WT)
__attribute__((amdgpu_waves_per_eu(WPE, WPE))) void grouped_gemm_dma128_kernel(
    const uint8_t *__restrict__ act, const uint8_t *__restrict__ wgt, void *__restrict__ out,
    const int32_t *__restrict__ tiles, int K, int N, int nft,
    const int32_t *__restrict__ gperm, int gk, int64_t gT, const float *__restrict__ dh,
    float *__restrict__ gu_out = nullptr) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * ((BW + BT) / 8) * 1024];
    int mt, ft;
    if (!block_tile(tiles[0], nft, mt, ft)) return;
    const int e = tiles[1 + 3 * mt], p0 = tiles[2 + 3 * mt], nrows = tiles[3 + 3 * mt];
    const uint8_t *abase = gperm ? act : act + (int64_t)p0 * ((uint32_t)K * 2u);
    dma128_tile<kGateUp, BW, BT, WF, WT, NS, kKMajor, kGrad>(ring, abase, wgt, out, K, N, e, p0,
                                                              nrows, ft, gperm, gk, gT, dh,
                                                              gu_out);
}

// Decode steps of one or two tokens with the plain softmax router: the gate/up launch routes
// the tokens itself. Every block forms the T x E router logits from the K-chain partials
// (chain order, then the bias: the routing tail's sums). The last block runs the tail's
// softmax + top-k + renormalisation routine on them ("0 train-infer mismatch ...", "The
// router: matching expert ids and weights") and stores every output of the routing tail
// (logits, ids and weights, lse, probability mass, counts, offsets, perm / inv, weighted
// counts, tile list, error bits); it computes no GEMM tile. The GEMM blocks run only that
// routine's selection rounds on the same keys (select_row4), so they hold the same ids, and
// form in LDS the stable counting sort of the T k assignments by expert ("RoutePack ...",
// Sec. 2.1; at most 16 rows, so every active expert is one 16-row tile, in expert order).
// Block (mt, ft) computes feature tile ft of the mt-th active expert, gathering its rows'
// tokens through that LDS permutation; blocks past the active experts exit. The tail's
// launch and its boundary leave the step: the partials come straight from the logit-chain
// launch before this one.
constexpr int kSrMaxT = 2;   // tokens per self-routing launch

template <class C, int NV, int MT>   // MT: the most tokens the instantiation takes (1 or 2)
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE))) void gate_up_self_route_kernel(
    const uint8_t *__restrict__ x, const uint8_t *__restrict__ w13, void *__restrict__ h,
    int K, int N, int nft, int T, int E, int k, int cap, DecodeRoute r,
    float *__restrict__ gu_out) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[C::NS * ((C::BW + C::BT) / 8) * 1024];
    static_assert(MT >= 1 && MT <= kSrMaxT, "one or two tokens");
    __shared__ float lgl[MT * kMaxE / 2];
    __shared__ float mp[MT][kMaxE / 2];          // q p per token (routing block)
    __shared__ float selw[MT * kMaxK];
    __shared__ int32_t sel[MT * kMaxK], lperm[MT * kMaxK], first[MT * kMaxK], tinfo[4];
    const int tid = threadIdx.x;
    const int A = T * k, TE = T * E;
    const bool router = blockIdx.x == gridDim.x - 1;   // the block that writes the routing
    for (int t = 0; t < (MT == 1 ? 1 : T); ++t) {
        for (int e = tid; e < E; e += C::kThreads) {
            const int i = t * E + e;
            float p[kLogitChains];
#pragma unroll
            for (int c = 0; c < kLogitChains; ++c) p[c] = r.part[c * TE + i];
            float v = p[0];
#pragma unroll
            for (int c = 1; c < kLogitChains; ++c) v = v + p[c];
            const float l = r.bias ? v + r.bias[e] : v;
            lgl[i] = l;
            if (router) r.logits[i] = l;
        }
    }
    lds_barrier();
    if (MT == 1 && router) {   // one token: the k ids are distinct, row j of the sort is id j's rank
        if (tid < kWave) {
            float qp[kRowVals];
            int err = 0;
            route_rows4<NV>(lgl, r.q, 0, 1, E, k, sel, selw, nullptr, qp, err, r.lse);
            wave_raise(err, r.d_err);
            if (r.prob_mass && tid < 16) {
                // the tail's sum over one token reduces to 0 + q p (the other rows add zeros)
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (tid + 16 * i < E) r.prob_mass[tid + 16 * i] = 0.f + qp[i];
            }
        }
        lds_barrier();
        if (tid < k) {
            const int ej = sel[tid];
            int rank = 0;
            for (int i = 0; i < k; ++i) rank += sel[i] < ej;
            r.topk_idx[tid] = ej;
            r.topk_w[tid] = selw[tid];
            r.perm[rank] = tid;
            r.inv[tid] = rank;
            int32_t *d = r.tiles + 1 + 3 * rank;
            d[0] = ej;
            d[1] = rank;
            d[2] = 1;
        }
        if (tid == 0) {
            r.tiles[0] = k;
            r.offsets[E] = k;
        }
        for (int e = tid; e < E; e += C::kThreads) {
            int before = 0;
            bool chosen = false;
            for (int i = 0; i < k; ++i) {
                before += sel[i] < e;
                chosen |= sel[i] == e;
            }
            r.counts[e] = chosen;
            r.offsets[e] = before;
            if (r.weighted_counts)
                r.weighted_counts[e] = !chosen ? 0 : r.q ? (int64_t)(uint32_t)r.q[0] : 1;
        }
        return;
    }
    if (router) {
        if (tid < kWave) {
            float qp[kRowVals];
            int err = 0;
            route_rows4<NV>(lgl, r.q, 0, T, E, k, sel, selw, nullptr, qp, err, r.lse);
            wave_raise(err, r.d_err);
            const int row = tid >> 4, c = tid & 15;
            if (row < T) {
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    if (c + 16 * i < E) mp[row][c + 16 * i] = qp[i];
            }
        }
        lds_barrier();
        if (tid < A) {   // assignment a = t k + j: its place in the stable sort by expert
            const int ea = sel[tid];
            int before = 0, same = 0;
            for (int b = 0; b < A; ++b) {
                before += sel[b] < ea;
                same += (sel[b] == ea) & (b < tid);
            }
            r.topk_idx[tid] = ea;
            r.topk_w[tid] = selw[tid];
            r.perm[before + same] = tid;
            r.inv[tid] = before + same;
            first[tid] = same == 0;   // the expert's first assignment
        }
        if (tid == 0) r.offsets[E] = A;
        lds_barrier();
        for (int e = tid; e < E; e += C::kThreads) {
            int before = 0, cnt = 0, tile = 0;   // tile: active experts below e
            uint64_t wsum = 0;
            for (int b = 0; b < A; ++b) {
                const int eb = sel[b];
                before += eb < e;
                tile += first[b] & (eb < e);
                if (eb == e) {
                    ++cnt;
                    if (r.q) wsum += (uint64_t)(uint32_t)r.q[b / k];
                }
            }
            r.counts[e] = cnt;
            r.offsets[e] = before;
            if (r.weighted_counts) r.weighted_counts[e] = r.q ? (int64_t)wsum : (int64_t)cnt;
            if (r.prob_mass) {
                // the tail's sum for a batch of at most two tokens: its first wave's four
                // rows (rows past the batch add zeros), then the other waves' and groups'
                // zero sums
                float m = 0.f + mp[0][e];
                m = m + (MT > 1 && T > 1 ? mp[MT - 1][e] : 0.f);
                m = m + 0.f;
                m = m + 0.f;
                float v = m;
                v = v + 0.f;
                v = v + 0.f;
                v = v + 0.f;
                r.prob_mass[e] = (v + 0.f) + (0.f + 0.f);
            }
            if (cnt) {
                int32_t *d = r.tiles + 1 + 3 * tile;
                d[0] = e;
                d[1] = before;
                d[2] = cnt;
            }
            if (e == E - 1) r.tiles[0] = tile + (cnt ? 1 : 0);
        }
        return;
    }
    // the GEMM blocks need the ids only: the selection rounds without the softmax
    if (tid < kWave) {
        if constexpr (MT == 1) {
            const int e = select_row4<NV>(lgl, E, k);
            if (tid < k) sel[tid] = e;
        } else {   // row t of the wave selects token t's experts
            const int row = tid >> 4, c = tid & 15;
            const int e = select_row4<NV>(lgl + min(row, T - 1) * E, E, k);
            if (row < T && c < k) sel[row * k + c] = e;
        }
    }
    lds_barrier();
    int mt, ft;
    block_tile(cap, nft, mt, ft);   // blocks 0 .. cap nft - 1 are the GEMM's
    if constexpr (MT == 1) {
        // one token: k distinct experts, tile mt = the mt-th smallest id, row mt = token 0
        if (tid < k) {
            const int ej = sel[tid];
            int rank = 0;
            for (int i = 0; i < k; ++i) rank += sel[i] < ej;
            lperm[rank] = ej;
        }
        lds_barrier();
        dma128_tile<true, C::BW, C::BT, C::WF, C::WT, C::NS, false, 0>(
            ring, x, w13, h, K, N, lperm[mt], mt, 1, ft, nullptr, 1, 1, nullptr, gu_out);
        return;
    }
    if (tid < A) {
        const int ea = sel[tid];
        int before = 0, same = 0;
        for (int b = 0; b < A; ++b) {
            before += sel[b] < ea;
            same += (sel[b] == ea) & (b < tid);
        }
        lperm[before + same] = tid;
        first[tid] = same == 0;
    }
    lds_barrier();
    if (tid < A && first[tid]) {   // the active experts in id order: tile mt is this block's
        const int ea = sel[tid];
        int rank = 0, before = 0, cnt = 0;
        for (int b = 0; b < A; ++b) {
            rank += first[b] & (sel[b] < ea);
            before += sel[b] < ea;
            cnt += sel[b] == ea;
        }
        if (rank == mt) {
            tinfo[0] = ea;
            tinfo[1] = before;
            tinfo[2] = cnt;
        }
    }
    if (tid == 0) {
        int n = 0;
        for (int b = 0; b < A; ++b) n += first[b];
        tinfo[3] = n;
    }
    lds_barrier();
    if (mt >= tinfo[3]) return;   // fewer active experts than the grid allows for
    dma128_tile<true, C::BW, C::BT, C::WF, C::WT, C::NS, false, 0>(
        ring, x, w13, h, K, N, tinfo[0], tinfo[1], tinfo[2], ft, lperm, k, T, nullptr, gu_out);
}

// ------------------------------------------------------------------------------------
// Decode-sized layers (at most kDcRows expert rows, so one 16-row token tile per active
// expert): the down GEMM and the weighted combine in one launch. Block b owns output
// features 16b .. 16b+15 of every row; wave w runs tiles w, w + 8, ... (one expert each)
// through the whole K = I in the down GEMM's MFMA sequence (one 16x16x32 step per 32
// K-values in K order, the 16 weight rows as the A operand and the tile's token rows as B,
// the same operands as the tiled kernel), so y gets the down GEMM's bits. The weight rows
// are loaded 4 lanes per row (each 4-lane group one row's contiguous 64 bytes) and moved
// to the MFMA lanes with ds_bpermute; the token rows are read in the MFMA layout. Each
// wave keeps 2 x 12 K-steps of loads in flight (nontemporal weight loads measured slower
// here: T = 1 layer 77.6 vs 79.1 us). The rows go to y and to LDS; after a barrier each of
// the block's 16 features of each token is summed over the token's k slots in slot order
// with the combine kernel's arithmetic ("0 train-infer mismatch ...", "The experts:
// keeping the route weight inside the accumulator"), scaled and rounded once.
// (up to 64 rows measured the same at T = 4 and 8, where the tiled down GEMM and the
// combine kernel already stream well; the one-launch form pays off at T <= 2)
constexpr int kDcRows = 16, kDcTile = 16, kDcFeat = 16, kDcWaves = 8, kDcGroup = 12;
constexpr int kDcMaxTiles = kDcRows / kDcTile + kDcRows;   // max_m_tiles(kDcRows, E, 16)
constexpr int kDcMinBlocks = 256;   // d / 16 blocks must fill the 256 CUs

__device__ __forceinline__ bf16x8_t dc_lay(bf16x8_t v, int src) {
    int4 q = __builtin_bit_cast(int4, v);
    q.x = __builtin_amdgcn_ds_bpermute(src, q.x);
    q.y = __builtin_amdgcn_ds_bpermute(src, q.y);
    q.z = __builtin_amdgcn_ds_bpermute(src, q.z);
    q.w = __builtin_amdgcn_ds_bpermute(src, q.w);
    return __builtin_bit_cast(bf16x8_t, q);
}

// kDcGroup K-steps of weight and token fragments (16 bytes per lane each), in flight
// together (the launch requires I to be a multiple of 2 kDcGroup steps, so no step is
// conditional and the compiler's load counting keeps the next group in flight)
struct DcGroup {
    bf16x8_t a[kDcGroup], b[kDcGroup];
};
__device__ __forceinline__ void dc_load(DcGroup &g, const uint16_t *wp, const uint16_t *hp,
                                        int s0) {
#pragma unroll
    for (int i = 0; i < kDcGroup; ++i) {
        g.a[i] = *reinterpret_cast<const bf16x8_t *>(wp + (s0 + i) * 32);
        g.b[i] = *reinterpret_cast<const bf16x8_t *>(hp + (s0 + i) * 32);
    }
}
__device__ __forceinline__ void dc_mfma(f32x4_t &acc, const DcGroup &g, int src) {
#pragma unroll
    for (int i = 0; i < kDcGroup; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dc_lay(g.a[i], src), g.b[i], acc, 0, 0, 0);
}

__global__ __launch_bounds__(64 * kDcWaves) void down_combine_small_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ w2, float *__restrict__ y,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ inv,
    const float *__restrict__ topk_w, int T, int k, int d, int I, float scale,
    uint16_t *__restrict__ out) {
    __shared__ float yl[kDcRows][kDcFeat];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int f0 = blockIdx.x * kDcFeat;
    const int A = T * k;
    const int ntiles = min(tiles[0], kDcMaxTiles);
    const int rc = lane >> 2, gc = lane & 3;                   // the lane's load row / slice
    const int src = 4 * (4 * (lane & 15) + (lane >> 4));       // byte address of its source
    const int nsteps = I >> 5;
    for (int mt = wave; mt < ntiles; mt += kDcWaves) {
        const int e = tiles[1 + 3 * mt], p0 = tiles[2 + 3 * mt];
        const int nrows = min(tiles[3 + 3 * mt], A - p0);
        if (nrows <= 0 || p0 < 0) continue;   // (a valid tile list has neither)
        const uint16_t *wp = w2 + ((int64_t)e * d + f0 + rc) * I + gc * 8;
        // the token rows (a few KB, L2-resident) are loaded in the MFMA layout directly:
        // lane l reads row l % 16 (rows past the tile repeat its last row), K-slice l / 16
        const uint16_t *hp = h + (int64_t)(p0 + min(lane & 15, nrows - 1)) * I + (lane >> 4) * 8;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // two register sets: the loads of the next group are issued before this group's
        // MFMAs, so a wave has up to 2 x kDcGroup K-steps in flight
        DcGroup g0, g1;
        dc_load(g0, wp, hp, 0);
        for (int s0 = 0; s0 < nsteps; s0 += 2 * kDcGroup) {
            dc_load(g1, wp, hp, s0 + kDcGroup);
            dc_mfma(acc, g0, src);
            if (s0 + 2 * kDcGroup < nsteps) dc_load(g0, wp, hp, s0 + 2 * kDcGroup);
            dc_mfma(acc, g1, src);
        }
        // lane l holds token row l % 16 of the tile, features 4 (l / 16) + 0..3
        const int col = lane & 15, fr = 4 * (lane >> 4);
        if (col < nrows) {
            const int p = p0 + col;
            *reinterpret_cast<float4 *>(y + (int64_t)p * d + f0 + fr) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) yl[p][fr + i] = acc[i];
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < T * kDcFeat; o += 64 * kDcWaves) {
        const int t = o / kDcFeat, f = o % kDcFeat;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            int p = inv[t * k + j];
            p = (p < 0 || p >= A) ? 0 : p;   // invalid ids were reported by the routing step
            acc = acc + topk_w[t * k + j] * yl[p][f];
        }
        acc = scale * acc;
        out[(int64_t)t * d + f0 + f] = f32_to_bf16(acc);
    }
}

template <int BW_, int BT_, int WF_, int WT_, int NS_ = 2, int WPE_ = (WF_ * WT_ + 3) / 4>
struct Dma128Cfg {
    static constexpr int BW = BW_, BT = BT_, WF = WF_, WT = WT_, WPE = WPE_, NS = NS_;
    static constexpr int kThreads = 64 * WF_ * WT_;
    static constexpr bool kDma128 = true;
};

// Launch shape of one GEMM: block tile and waves. Any shape gives the same bits.
// WPE: waves per SIMD the kernel is compiled for (the register budget follows from it).
template <int BW_, int BT_, int WF_, int WT_, int PF_, int SRB_ = 128, int WPE_ = 1>
struct Cfg {
    static constexpr int BW = BW_, BT = BT_, WF = WF_, WT = WT_, PF = PF_, SRB = SRB_,
                         WPE = WPE_;
    static constexpr int kThreads = 64 * WF_ * WT_;
};

template <class C, class = void>
struct IsDma128 : std::false_type {};
template <class C>
struct IsDma128<C, std::void_t<decltype(C::kDma128)>> : std::true_type {};


// gperm != nullptr: activation rows are gathered (token perm[p] / gk of act, gT rows).
// kKMajor: weights stored wgt[e][k][n] (bf16 DMA kernel only).
template <bool kBF16, bool kGateUp, class C, bool kKMajor = false, int kGrad = 0>
hipError_t launch_gemm(const void *act, const void *wgt, void *out, const int32_t *tiles,
                       int64_t mtiles, int K, int N, hipStream_t s,
                       const int32_t *gperm = nullptr, int gk = 1, int64_t gT = 0,
                       const float *dh = nullptr, float *gu_out = nullptr) {
    constexpr int feat = kGateUp ? C::BW / 2 : C::BW;
    const int nft = (N + feat - 1) / feat;
    static_assert(!kKMajor || (IsDma128<C>::value && kBF16 && !kGateUp), "K-major weights");
    static_assert(kGrad == 0 || (IsDma128<C>::value && kBF16 && kGateUp), "fused SwiGLU grad");
    if constexpr (IsDma128<C>::value && kBF16) {
        grouped_gemm_dma128_kernel<kGateUp, C::BW, C::BT, C::WF, C::WT, C::WPE, C::NS, kKMajor,
                                   kGrad>
            <<<dim3((unsigned)(mtiles * nft)), dim3(C::kThreads), 0, s>>>(
                static_cast<const uint8_t *>(act), static_cast<const uint8_t *>(wgt), out, tiles,
                K, N, nft, gperm, gk, gT, dh, gu_out);
    } else if constexpr (IsDma128<C>::value) {
        // the DMA kernel is bf16-only: FP32 layers use the register-staged kernel with the
        // same token tiles (the 256-token gate/up tile takes 128 weight rows: with 256 its
        // gate and up accumulators do not fit the registers)
        using F = typename std::conditional<
            (C::BT <= 32), Cfg<128, C::BT, 4, 1, 1, 128, 3>,
            typename std::conditional<
                (C::BT == 64), Cfg<128, 64, 2, 2, 1, 128, 2>,
                typename std::conditional<(kGateUp && C::BT == 256),
                                          Cfg<128, 256, 2, 2, 1, 64, 1>,
                                          Cfg<256, C::BT, 2, 2, 1, 64, 1>>::type>::type>::type;
        return launch_gemm<kBF16, kGateUp, F>(act, wgt, out, tiles, mtiles, K, N, s, gperm, gk,
                                              gT, nullptr, gu_out);
    } else {
        grouped_gemm_kernel<kBF16, kGateUp, C::BW, C::BT, C::WF, C::WT, C::PF, C::SRB, C::WPE>
            <<<dim3((unsigned)(mtiles * nft)), dim3(C::kThreads), 0, s>>>(
                static_cast<const uint8_t *>(act), static_cast<const uint8_t *>(wgt), out, tiles,
                K, N, nft, gperm, gk, gT, gu_out);
    }
    return hipGetLastError();
}

// act13: x_perm (segment rows), or x with gperm = perm (gather fused into the gate/up GEMM)
template <bool kBF16, class C13, class C2>
hipError_t run_ffn(const moe_dims &dm, const void *act13, const int32_t *gperm, const void *w13,
                   const void *w2, void *h, float *y, const int32_t *tiles, int64_t mtiles,
                   void *const *ev, hipStream_t s, float *gu_out, bool gate_up_only) {
    static_assert(C13::BT == C2::BT, "both GEMMs walk the same token tiles");
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[0]), s) != hipSuccess)
        return hipErrorInvalidValue;
    hipError_t e = launch_gemm<kBF16, true, C13>(act13, w13, h, tiles, mtiles, dm.d, dm.inter, s,
                                                 gperm, dm.k, dm.T, nullptr, gu_out);
    if (e != hipSuccess) return e;
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[1]), s) != hipSuccess)
        return hipErrorInvalidValue;
    if (gate_up_only) return hipSuccess;
    e = launch_gemm<kBF16, false, C2>(h, w2, y, tiles, mtiles, dm.inter, dm.d, s);
    if (e != hipSuccess) return e;
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[2]), s) != hipSuccess)
        return hipErrorInvalidValue;
    return hipSuccess;
}

// Prefill-shaped launches: two 128-byte K stages in LDS. 128-token tiles stage 512 weight
// rows (256 output features of gate/up) on 16 waves (4 per SIMD, 64x64 per wave); 256-token
// tiles 256 weight rows, on 16 waves for gate/up and 8 (2 per SIMD, 128x64 per wave) for
// the down GEMM, which measured marginally faster there. Both rings fit the 160 KB of LDS.
#ifndef MOE_FFN_LARGE_CFG13
#define MOE_FFN_LARGE_CFG13 Dma128Cfg<512, 128, 8, 2, 2, 4>
#define MOE_FFN_LARGE_CFG2 Dma128Cfg<512, 128, 8, 2, 2, 4>
#endif
#ifndef MOE_FFN_HUGE_CFG13
#define MOE_FFN_HUGE_CFG13 Dma128Cfg<256, 256, 4, 4, 2, 4>
#define MOE_FFN_HUGE_CFG2 Dma128Cfg<256, 256, 2, 4>
#endif

#ifndef MOE_FFN_CFG16
#define MOE_FFN_CFG16 Dma128Cfg<64, 16, 2, 1, 5, 2>
#endif
using PLAIN_CFG16 = MOE_FFN_CFG16;
#ifndef MOE_FFN_DOWN_CFG16
#define MOE_FFN_DOWN_CFG16 Dma128Cfg<64, 16, 2, 1, 4, 2>
#endif
using DOWN_CFG16 = MOE_FFN_DOWN_CFG16;
#ifndef MOE_SELF_ROUTE_CFG
#define MOE_SELF_ROUTE_CFG Dma128Cfg<32, 16, 1, 1, 6>
#endif
using SELF_ROUTE_CFG = MOE_SELF_ROUTE_CFG;
#ifndef MOE_SELF_ROUTE_CFG2
#define MOE_SELF_ROUTE_CFG2 Dma128Cfg<64, 16, 2, 1, 5, 2>
#endif
using SELF_ROUTE_CFG2 = MOE_SELF_ROUTE_CFG2;   // two tokens: the 16-row gate/up shape
#ifndef MOE_FFN_CFG32
#define MOE_FFN_CFG32 Dma128Cfg<64, 32, 2, 1, 4, 2>
#endif
#ifndef MOE_FFN_CFG64
#define MOE_FFN_CFG64 Dma128Cfg<128, 64, 2, 2, 3, 2>
#endif
using PLAIN_CFG32 = MOE_FFN_CFG32;
using PLAIN_CFG64 = MOE_FFN_CFG64;
using PLAIN_LARGE = MOE_FFN_LARGE_CFG2;
using PLAIN_HUGE = MOE_FFN_HUGE_CFG2;

template <bool kBF16>
hipError_t dispatch_ffn(const moe_dims &dm, int bt, const void *x_perm, const int32_t *gperm,
                        const void *w13, const void *w2, void *h, float *y,
                        const int32_t *tiles, int64_t mtiles, void *const *ev, hipStream_t s,
                        float *gu_out, bool gate_up_only) {
    // Decode-shaped launches stream the weights: narrow 64-row weight slices (many blocks per
    // active expert). Their kernels are compiled for two waves per SIMD (WPE 2: compiled for
    // one, they declared over 256 registers and so held a CU to two 2-wave blocks whatever
    // the LDS), and the rings are sized so that several blocks share a CU: the 16-row
    // gate/up 5 slots (three blocks), its down GEMM 4 (four), the 32-row tiles 4 (three),
    // the 64-row tiles 3 (two). Measured on the decode-shaped layer against one wave per
    // SIMD and 6 / 6 / 4-slot rings: T = 2 0.122 -> 0.114 ms, T = 4 and 16 2 % and T = 64
    // 1 % faster; tiles forced to 32 / 64 rows at T = 64 3-4 % / 11 % faster.
    switch (bt) {
    case 16:
        return run_ffn<kBF16, PLAIN_CFG16, DOWN_CFG16>(dm, x_perm, gperm, w13, w2, h, y, tiles,
                                                       mtiles, ev, s, gu_out, gate_up_only);
    case 32: {
        using C = PLAIN_CFG32;
        return run_ffn<kBF16, C, C>(dm, x_perm, gperm, w13, w2, h, y, tiles, mtiles, ev, s, gu_out,
                                    gate_up_only);
    }
    case 64: {
        using C = PLAIN_CFG64;
        return run_ffn<kBF16, C, C>(dm, x_perm, gperm, w13, w2, h, y, tiles, mtiles, ev, s, gu_out,
                                    gate_up_only);
    }
    case 128:
        return run_ffn<kBF16, MOE_FFN_LARGE_CFG13, MOE_FFN_LARGE_CFG2>(dm, x_perm, gperm, w13, w2, h, y,
                                                                       tiles, mtiles, ev, s, gu_out,
                                                                       gate_up_only);
    default:
        return run_ffn<kBF16, MOE_FFN_HUGE_CFG13, MOE_FFN_HUGE_CFG2>(dm, x_perm, gperm, w13, w2, h, y,
                                                                     tiles, mtiles, ev, s, gu_out,
                                                                     gate_up_only);
    }
}

}  // namespace

// Automatic token-tile height. Below 128 mean rows per expert the GEMMs mostly stream the
// active experts' weights, once per token tile, so the tile is the smallest that holds
// 1.5x the mean rows (no expert has more than T): most experts then take a single tile.
// (Measured on a d=4096, E=128, top-8 layer: T = 256 and 512 went from 1.12 / 1.17 ms to
// 0.84 / 0.87 ms, T = 1024 and 1536 from 1.29 / 1.74 ms to 0.94 / 1.00 ms; a tile at the
// mean left about half the experts with a second tile.) From 128 mean rows on, 256-row
// tiles: half the weight passes of 128-row tiles outweigh their padding (uniform routing,
// d = 4096 / E = 128 and d = 2048 / E = 64, 128 to 768 rows per expert: 6-13 % faster; the
// skewed training-shaped layer 2.5 %; at 96 rows 128-row tiles were still 15 % faster).
int select_tile_m(const moe_dims &dm) {
    if (dm.tile_m) return dm.tile_m;
    const int64_t A = dm.T * dm.k;
    const int64_t avg = A / dm.E;          // mean rows per expert
    if (avg >= 128) return 256;
    const int64_t want = std::min<int64_t>(dm.T, (3 * A + 2 * dm.E - 1) / (2 * dm.E));
    if (want <= 16) return 16;
    if (want <= 32) return 32;
    if (want <= 64) return 64;
    return 128;
}

// Token tiles of any routing of A rows: sum over the active experts of ceil(c_e / tile_m)
// <= A / tile_m + (active experts), and at most min(E, A) experts are active. (The bound
// sizes the launch grids, so decode-sized batches do not launch blocks for 128 experts.)
int64_t max_m_tiles(int64_t A, int E, int tile_m) {
    return (A + tile_m - 1) / tile_m + std::min<int64_t>(E, A);
}

hipError_t launch_build_tiles(const int32_t *offsets, int E, int64_t A, int bt, int64_t cap,
                              int32_t *tiles, hipStream_t s) {
    build_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(offsets, E, A, bt, cap, tiles);
    return hipGetLastError();
}

// out[p, n] = sum_k act[p, k] wgt[e, n, k] for the rows p of every segment e (FP32 output,
// no activation): the down-GEMM launch with N output features and K (0: dm.d), gathered
// through gperm when given. Every output is the same sequence of MFMA steps over K as the
// gate/up GEMM's pre-activations for the same weight row, so with wgt = w13 and N = 2I it
// reproduces the forward's gate and up values bit for bit.
hipError_t launch_plain_gemm(const moe_dims &dm, const void *act, const int32_t *gperm,
                             const void *wgt, float *out, int N, const int32_t *offsets,
                             const Workspace &ws, hipStream_t s, int K, bool kmajor) {
    const int64_t A = dm.T * dm.k;
    if (A == 0) return hipGetLastError();
    if (K == 0) K = dm.d;
    if (kmajor && dm.dtype != MOE_BF16) return hipErrorInvalidValue;
    const int bt = select_tile_m(dm);
    const int64_t cap = max_m_tiles(A, dm.E, bt);
    build_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(offsets, dm.E, A, bt, cap, ws.tiles);
    const bool b = dm.dtype == MOE_BF16;
#define MOE_PLAIN(CFG)                                                                          \
    (kmajor ? launch_gemm<true, false, CFG, true>(act, wgt, out, ws.tiles, cap, K, N, s, gperm,  \
                                                  dm.k, dm.T)                                   \
     : b    ? launch_gemm<true, false, CFG>(act, wgt, out, ws.tiles, cap, K, N, s, gperm, dm.k,  \
                                            dm.T)                                               \
            : launch_gemm<false, false, CFG>(act, wgt, out, ws.tiles, cap, K, N, s, gperm, dm.k, \
                                             dm.T))
    hipError_t e;
    switch (bt) {
    case 16: e = MOE_PLAIN(PLAIN_CFG16); break;
    case 32: e = MOE_PLAIN(PLAIN_CFG32); break;
    case 64: e = MOE_PLAIN(PLAIN_CFG64); break;
    case 128: e = MOE_PLAIN(PLAIN_LARGE); break;
    default: e = MOE_PLAIN(PLAIN_HUGE); break;
    }
#undef MOE_PLAIN
    return e;
}

// The backward's gate/up recomputation fused with the SwiGLU derivative (bf16 layers): each
// (row, feature)'s gate and up values are the forward's (the forward's gate/up launch shape
// for the tile height, the same MFMA sequence), and the epilogue forms
// d_gu[p, n] = (dh u) silu'(g), d_gu[p, I + n] = dh silu(g) with the elementwise kernel's
// arithmetic, so g and u never reach memory. d_gu is bf16 (dgu_bf16) or FP32.
hipError_t launch_gate_up_grad(const moe_dims &dm, const void *act, const int32_t *gperm,
                               const void *w13, const float *dh, void *dgu, bool dgu_bf16,
                               const int32_t *offsets, const Workspace &ws, hipStream_t s) {
    const int64_t A = dm.T * dm.k;
    if (A == 0) return hipGetLastError();
    if (dm.dtype != MOE_BF16) return hipErrorInvalidValue;
    const int bt = select_tile_m(dm);
    const int64_t cap = max_m_tiles(A, dm.E, bt);
    build_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(offsets, dm.E, A, bt, cap, ws.tiles);
    using GugLarge = MOE_FFN_LARGE_CFG13;
    using GugHuge = MOE_FFN_HUGE_CFG13;
#define MOE_GUG(CFG)                                                                            \
    (dgu_bf16 ? launch_gemm<true, true, CFG, false, 1>(act, w13, dgu, ws.tiles, cap, dm.d,       \
                                                       dm.inter, s, gperm, dm.k, dm.T, dh)      \
              : launch_gemm<true, true, CFG, false, 2>(act, w13, dgu, ws.tiles, cap, dm.d,       \
                                                       dm.inter, s, gperm, dm.k, dm.T, dh))
    hipError_t e;
    switch (bt) {
    case 16: e = MOE_GUG(PLAIN_CFG16); break;
    case 32: e = MOE_GUG(PLAIN_CFG32); break;
    case 64: e = MOE_GUG(PLAIN_CFG64); break;
    case 128: e = MOE_GUG(GugLarge); break;
    default: e = MOE_GUG(GugHuge); break;
    }
#undef MOE_GUG
    return e;
}

hipError_t launch_grouped_ffn(const moe_dims &dm, const void *x_perm, const int32_t *offsets,
                              const void *w13, const void *w2, void *h, float *y,
                              const Workspace &ws, void *const *prof_events, hipStream_t s,
                              const void *x, const int32_t *perm, bool tiles_ready,
                              float *gu_out, bool gate_up_only) {
    const int64_t A = dm.T * dm.k;
    const int bt = select_tile_m(dm);
    const int64_t cap = max_m_tiles(A, dm.E, bt);
    if (A == 0) {
        if (prof_events)
            for (int i = 0; i < 3; ++i)
                if (hipEventRecord(static_cast<hipEvent_t>(prof_events[i]), s) != hipSuccess)
                    return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (!tiles_ready)
        build_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(offsets, dm.E, A, bt, cap, ws.tiles);
    // x_perm == nullptr: the gate/up GEMM gathers token rows of x through perm itself
    const void *act13 = x_perm ? x_perm : x;
    const int32_t *gperm = x_perm ? nullptr : perm;
    if (dm.dtype == MOE_BF16)
        return dispatch_ffn<true>(dm, bt, act13, gperm, w13, w2, h, y, ws.tiles, cap, prof_events,
                                  s, gu_out, gate_up_only);
    return dispatch_ffn<false>(dm, bt, act13, gperm, w13, w2, h, y, ws.tiles, cap, prof_events,
                               s, gu_out, gate_up_only);
}

bool decode_self_route_ok(const moe_dims &dm) {
    return dm.dtype == MOE_BF16 && dm.T >= 1 && dm.T <= kSrMaxT && dm.T * dm.k <= 16 &&
           dm.E >= dm.k && dm.E <= kMaxE / 2 && dm.k >= 1 && dm.k <= kMaxK &&
           select_tile_m(dm) == 16;
}

hipError_t launch_decode_self_route(const moe_dims &dm, const DecodeRoute &r, const void *x,
                                    const void *w13, void *h, float *gu_out,
                                    void *const *prof_events, hipStream_t s) {
    if (!decode_self_route_ok(dm)) return hipErrorInvalidValue;
    if (prof_events && hipEventRecord(static_cast<hipEvent_t>(prof_events[0]), s) != hipSuccess)
        return hipErrorInvalidValue;
    // at most one 16-row tile per active expert: min(E, T k) tiles
    const int cap = (int)std::min<int64_t>(dm.E, dm.T * dm.k);
    auto go = [&](auto nv, auto cfg, auto mt) {
        using C = decltype(cfg);
        const int nft = (dm.inter + C::BW / 2 - 1) / (C::BW / 2);
        gate_up_self_route_kernel<C, decltype(nv)::value, decltype(mt)::value>
            <<<dim3((unsigned)(cap * nft + 1)), dim3(C::kThreads), 0, s>>>(
                static_cast<const uint8_t *>(x), static_cast<const uint8_t *>(w13), h, dm.d,
                dm.inter, nft, (int)dm.T, dm.E, dm.k, cap, r, gu_out);
    };
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    using NV4 = std::integral_constant<int, 4>;
    using NV8 = std::integral_constant<int, 8>;
    if (dm.T == 1) {
        if (dm.E <= 64) go(NV4{}, SELF_ROUTE_CFG{}, One{});
        else go(NV8{}, SELF_ROUTE_CFG{}, One{});
    } else {
        if (dm.E <= 64) go(NV4{}, SELF_ROUTE_CFG2{}, Two{});
        else go(NV8{}, SELF_ROUTE_CFG2{}, Two{});
    }
    if (prof_events && hipEventRecord(static_cast<hipEvent_t>(prof_events[1]), s) != hipSuccess)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

bool down_combine_small_ok(const moe_dims &dm) {
    return dm.dtype == MOE_BF16 && dm.T >= 1 && dm.T * dm.k <= kDcRows &&
           select_tile_m(dm) == kDcTile && dm.d % kDcFeat == 0 &&
           dm.d / kDcFeat >= kDcMinBlocks && dm.inter % (64 * kDcGroup) == 0;
}

hipError_t launch_down_combine_small(const moe_dims &dm, const void *h, const void *w2, float *y,
                                     const int32_t *tiles, const int32_t *inv,
                                     const float *topk_w, float scale, void *out,
                                     void *const *prof_events, hipStream_t s) {
    if (!down_combine_small_ok(dm)) return hipErrorInvalidValue;
    down_combine_small_kernel<<<dim3((unsigned)(dm.d / kDcFeat)), dim3(64 * kDcWaves), 0, s>>>(
        static_cast<const uint16_t *>(h), static_cast<const uint16_t *>(w2), y, tiles, inv,
        topk_w, (int)dm.T, dm.k, dm.d, dm.inter, scale, static_cast<uint16_t *>(out));
    if (prof_events && hipEventRecord(static_cast<hipEvent_t>(prof_events[2]), s) != hipSuccess)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
