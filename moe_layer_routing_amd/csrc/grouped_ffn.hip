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
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowBytes = 128;                // one K-stage of a row: 64 bf16 or 32 f32
constexpr int kLdsStride = kRowBytes + 16;    // padded LDS row (bank spread)
constexpr int kVecPerRow = kRowBytes / 16;    // 16-byte vectors per staged row

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

template <bool kBF16>
struct Elem;
template <>
struct Elem<true> {
    static constexpr int kPerVec = 8;       // bf16 per 16 bytes
    static constexpr int kSub = 2;          // MFMA K-steps (32 each) per 128-byte stage
    static constexpr int kSubBytes = 64;
};
template <>
struct Elem<false> {
    static constexpr int kPerVec = 4;
    static constexpr int kSub = 8;          // K-steps of 4 floats
    static constexpr int kSubBytes = 16;
};

// kGateUp: out = h[A, I] = round(silu(x w_gate^T) * (x w_up^T)), K = d, N = I,
//          the weight tile stacks BW/2 gate rows over the matching BW/2 up rows.
// else:    out = y[A, d] (FP32) = h w2^T, K = I, N = d.
template <bool kBF16, bool kGateUp, int BW, int BT, int WF, int WT>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(const uint8_t *__restrict__ act,
                                                           const uint8_t *__restrict__ wgt,
                                                           void *__restrict__ out,
                                                           const int32_t *__restrict__ tiles,
                                                           int K, int N, int nft) {
    using EL = Elem<kBF16>;
    constexpr int kEB = kBF16 ? 2 : 4;                 // element bytes
    constexpr int kFeat = kGateUp ? BW / 2 : BW;       // output features per block
    constexpr int kWaveRows = (kGateUp ? BW / 2 : BW) / WF;
    constexpr int NFh = kWaveRows / 16;                // fragments per half (gate/up)
    constexpr int NF = kGateUp ? 2 * NFh : NFh;
    constexpr int NT = BT / WT / 16;
    constexpr int kVW = BW * kVecPerRow;               // 16-byte vectors per stage
    constexpr int kVT = BT * kVecPerRow;
    constexpr int kLW = (kVW + 255) / 256;
    constexpr int kLT = (kVT + 255) / 256;
    static_assert(NFh >= 1 && NT >= 1 && WF * WT == 4, "bad tile shape");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BW + BT) * kLdsStride];

    // XCD-aware order: the hardware deals consecutive block ids round-robin over the 8
    // XCDs; renumber so each XCD gets one contiguous range of logical tiles (tiles that
    // share a token slice or an expert's weights then share that XCD's L2).
    const uint32_t nwg = gridDim.x, bid = blockIdx.x;
    const uint32_t xcd = bid & 7u, loc = bid >> 3, per = nwg >> 3, rem = nwg & 7u;
    const uint32_t L = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
    const int mt = (int)(L / (uint32_t)nft), ft = (int)(L % (uint32_t)nft);
    if (mt >= tiles[0]) return;
    const int e = tiles[1 + 3 * mt], p0 = tiles[2 + 3 * mt], nrows = tiles[3 + 3 * mt];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wf = wv % WF, wt = wv / WF;
    const int n0 = ft * kFeat;
    const int64_t rows_per_expert = kGateUp ? 2 * (int64_t)N : (int64_t)N;
    const int64_t krow_bytes = (int64_t)K * kEB;

    // global row base pointers for this thread's staged vectors
    const uint8_t *gw[kLW];
    const uint8_t *gt[kLT];
#pragma unroll
    for (int i = 0; i < kLW; ++i) {
        const int v = tid + i * 256;
        const int r = v / kVecPerRow, c = v % kVecPerRow;
        int grow;
        if (kGateUp) {
            const int half = r >= BW / 2;
            const int rr = half ? r - BW / 2 : r;
            grow = min(n0 + rr, N - 1) + (half ? N : 0);
        } else {
            grow = min(n0 + r, N - 1);
        }
        gw[i] = wgt + ((int64_t)e * rows_per_expert + grow) * krow_bytes + c * 16;
    }
#pragma unroll
    for (int i = 0; i < kLT; ++i) {
        const int v = tid + i * 256;
        const int r = v / kVecPerRow, c = v % kVecPerRow;
        const int rr = min(r, nrows - 1);
        gt[i] = act + ((int64_t)p0 + rr) * krow_bytes + c * 16;
    }
    u32x4_t rw[kLW], rt[kLT];

    auto load_global = [&](int kt) {
        const int64_t ko = (int64_t)kt * kRowBytes;
#pragma unroll
        for (int i = 0; i < kLW; ++i)
            if (kVW % 256 == 0 || tid + i * 256 < kVW)
                rw[i] = *reinterpret_cast<const u32x4_t *>(gw[i] + ko);
#pragma unroll
        for (int i = 0; i < kLT; ++i)
            if (kVT % 256 == 0 || tid + i * 256 < kVT)
                rt[i] = *reinterpret_cast<const u32x4_t *>(gt[i] + ko);
    };
    auto store_lds = [&](int b) {
#pragma unroll
        for (int i = 0; i < kLW; ++i) {
            const int v = tid + i * 256;
            if (kVW % 256 == 0 || v < kVW)
                *reinterpret_cast<u32x4_t *>(&smem[b][(v / kVecPerRow) * kLdsStride +
                                                    (v % kVecPerRow) * 16]) = rw[i];
        }
#pragma unroll
        for (int i = 0; i < kLT; ++i) {
            const int v = tid + i * 256;
            if (kVT % 256 == 0 || v < kVT)
                *reinterpret_cast<u32x4_t *>(&smem[b][(BW + v / kVecPerRow) * kLdsStride +
                                                    (v % kVecPerRow) * 16]) = rt[i];
        }
    };

    // LDS row of weight fragment f (16 rows) and token fragment t for this wave
    auto wrow = [&](int f) {
        if (kGateUp)
            return (f < NFh ? 0 : BW / 2) + wf * kWaveRows + (f % NFh) * 16;
        return wf * kWaveRows + f * 16;
    };
    auto trow = [&](int t) { return BW + wt * (BT / WT) + t * 16; };

    f32x4_t acc[NF][NT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15, g4 = lane >> 4;
    const int nk = K / (kRowBytes / kEB);

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cb = kt & 1;
        if (kt + 1 < nk) load_global(kt + 1);
        const uint8_t *sb = smem[cb];
#pragma unroll
        for (int kk = 0; kk < EL::kSub; ++kk) {
            if constexpr (kBF16) {
                bf16x8_t a[NF], b[NT];
#pragma unroll
                for (int f = 0; f < NF; ++f)
                    a[f] = *reinterpret_cast<const bf16x8_t *>(
                        sb + (wrow(f) + r16) * kLdsStride + kk * EL::kSubBytes + g4 * 16);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    b[t] = *reinterpret_cast<const bf16x8_t *>(
                        sb + (trow(t) + r16) * kLdsStride + kk * EL::kSubBytes + g4 * 16);
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], b[t],
                                                                            acc[f][t], 0, 0, 0);
            } else {
                float a[NF], b[NT];
#pragma unroll
                for (int f = 0; f < NF; ++f)
                    a[f] = *reinterpret_cast<const float *>(
                        sb + (wrow(f) + r16) * kLdsStride + kk * EL::kSubBytes + g4 * 4);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    b[t] = *reinterpret_cast<const float *>(
                        sb + (trow(t) + r16) * kLdsStride + kk * EL::kSubBytes + g4 * 4);
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[f], b[t], acc[f][t],
                                                                         0, 0, 0);
            }
        }
        if (kt + 1 < nk) store_lds(cb ^ 1);
        __syncthreads();
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

template <bool kBF16, int BW, int BT, int WF, int WT>
hipError_t run_ffn(const moe_dims &dm, const void *x_perm, const void *w13, const void *w2,
                   void *h, float *y, const int32_t *tiles, int64_t mtiles,
                   void *const *ev, hipStream_t s) {
    const int d = dm.d, I = dm.inter;
    const int nft13 = (I + BW / 2 - 1) / (BW / 2);
    const int nft2 = (d + BW - 1) / BW;
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[0]), s) != hipSuccess)
        return hipErrorInvalidValue;
    grouped_gemm_kernel<kBF16, true, BW, BT, WF, WT>
        <<<dim3((unsigned)(mtiles * nft13)), dim3(256), 0, s>>>(
            static_cast<const uint8_t *>(x_perm), static_cast<const uint8_t *>(w13), h, tiles,
            d, I, nft13);
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[1]), s) != hipSuccess)
        return hipErrorInvalidValue;
    grouped_gemm_kernel<kBF16, false, BW, BT, WF, WT>
        <<<dim3((unsigned)(mtiles * nft2)), dim3(256), 0, s>>>(
            static_cast<const uint8_t *>(h), static_cast<const uint8_t *>(w2), y, tiles, I, d,
            nft2);
    if (ev && hipEventRecord(static_cast<hipEvent_t>(ev[2]), s) != hipSuccess)
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool kBF16>
hipError_t dispatch_ffn(const moe_dims &dm, int bt, const void *x_perm, const void *w13,
                        const void *w2, void *h, float *y, const int32_t *tiles,
                        int64_t mtiles, void *const *ev, hipStream_t s) {
    switch (bt) {
    case 16:
        return run_ffn<kBF16, 128, 16, 4, 1>(dm, x_perm, w13, w2, h, y, tiles, mtiles, ev, s);
    case 32:
        return run_ffn<kBF16, 128, 32, 4, 1>(dm, x_perm, w13, w2, h, y, tiles, mtiles, ev, s);
    case 64:
        return run_ffn<kBF16, 128, 64, 2, 2>(dm, x_perm, w13, w2, h, y, tiles, mtiles, ev, s);
    default:
        return run_ffn<kBF16, 256, 128, 2, 2>(dm, x_perm, w13, w2, h, y, tiles, mtiles, ev, s);
    }
}

}  // namespace

int select_tile_m(const moe_dims &dm) {
    if (dm.tile_m) return dm.tile_m;
    const int64_t A = dm.T * dm.k;
    const int64_t avg = A / dm.E;          // mean rows per expert
    if (dm.T <= 16 || avg <= 16) return 16;
    if (dm.T <= 32 || avg <= 32) return 32;
    if (dm.T <= 64 || avg <= 96) return 64;
    return 128;
}

int64_t max_m_tiles(int64_t A, int E, int tile_m) { return (A + tile_m - 1) / tile_m + E; }

hipError_t launch_grouped_ffn(const moe_dims &dm, const void *x_perm, const int32_t *offsets,
                              const void *w13, const void *w2, void *h, float *y,
                              const Workspace &ws, void *const *prof_events, hipStream_t s) {
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
    build_tiles_kernel<<<dim3(1), dim3(256), 0, s>>>(offsets, dm.E, A, bt, cap, ws.tiles);
    if (dm.dtype == MOE_BF16)
        return dispatch_ffn<true>(dm, bt, x_perm, w13, w2, h, y, ws.tiles, cap, prof_events, s);
    return dispatch_ffn<false>(dm, bt, x_perm, w13, w2, h, y, ws.tiles, cap, prof_events, s);
}

}  // namespace moe
