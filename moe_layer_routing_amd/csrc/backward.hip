// backward.hip -- backward of the MoE layer: combine, SwiGLU experts, softmax router.
//
// The derivative of the forward definitions ("0 train-infer mismatch for Open-weight MoE RL
// in Open-source code": "The experts: keeping the route weight inside the accumulator",
// "SwiGLU: rounding after the multiply", "The router: matching expert ids and weights"),
// with every reduction in one fixed order:
//   dy[p]      = (s w[t,j]) dout[t]             (p = inv[t*k+j], s = routed scaling factor)
//   dw[t,j]    = s <dout[t], y[p]>              (per-lane partials, fixed DPP tree)
//   g, u       = the forward's pre-activations, recomputed by the forward's own GEMM
//   dh         = dy w2[e]                       (FP32 MFMA, K = d ascending)
//   dg, du     = dh u silu'(g), dh silu(g)
//   dxp        = [dg du] w13[e]                 (FP32 MFMA, K = 2I ascending)
//   dx[t]      = sum over slots of dxp rows, slot order, + the router's part
//   dw2[e]     = sum over the segment's rows of dy^T h      (rows ascending)
//   dw13[e]    = sum over the segment's rows of [dg du]^T x  (rows ascending)
//   router:    dl = the softmax / top-k / renormalisation Jacobian at the router's own
//              choice applied to dw by slot; dw_router = dl^T x; dx += dl w_router.
// Under routing replay ("Total Router Recall": the layer passes w - sg[w] + w*) the value
// the experts saw is the sampler's w*, and the router's gradient flows through its own
// renormalised weights at its own top-k, slot by slot: the same router step.
//
// The gradient GEMMs read token-major activations and row-major weights directly: the
// FP32 MFMA (v_mfma_f32_16x16x4f32) takes one element per lane (lane l: row / column l%16,
// K index l/16), so a K x N weight tile staged row-major in LDS and a rows x K activation
// tile staged row-major both serve it without a transpose. Operands are FP32 (bf16
// storage widened exactly); every output is one sum over K (or over the segment's rows)
// in increasing order of 4-wide MFMA steps.
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kKc = 16;   // K elements per LDS stage of the FP32 gradient GEMMs

// ------------------------------------------------------------------ combine backward
// One wave per token: lane l takes features 4l, 4l + 256, ... of every slot's y row;
// dy = (s w_j) dout; the partial dot products <dout, y_j> are summed per lane in feature
// order and then over the wave in the fixed DPP tree.
template <bool kBF16, bool kDyBF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const void *__restrict__ dout, const float *__restrict__ y,
    const int32_t *__restrict__ inv, const float *__restrict__ topk_w, int64_t T, int k,
    int d, int64_t A, float scale, void *__restrict__ dyv, float *__restrict__ dw) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    int64_t src[kMaxK];
    float ws[kMaxK], acc[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        int32_t p = (j < k) ? inv[t * k + j] : 0;
        p = (p < 0 || p >= A) ? 0 : p;
        src[j] = (int64_t)p * d;
        ws[j] = (j < k) ? scale * topk_w[t * k + j] : 0.f;
        acc[j] = 0.f;
    }
    for (int c = lane * 4; c < d; c += 256) {
        // issue every slot's y load before the first use, so k rows are in flight at once
        float g[4];
        if constexpr (kBF16) {
            const uint2 raw = *reinterpret_cast<const uint2 *>(
                static_cast<const uint16_t *>(dout) + t * d + c);
            g[0] = bf16_to_f32((uint16_t)(raw.x & 0xffffu));
            g[1] = bf16_to_f32((uint16_t)(raw.x >> 16));
            g[2] = bf16_to_f32((uint16_t)(raw.y & 0xffffu));
            g[3] = bf16_to_f32((uint16_t)(raw.y >> 16));
        } else {
            const float4 raw = *reinterpret_cast<const float4 *>(static_cast<const float *>(dout) + t * d + c);
            g[0] = raw.x;
            g[1] = raw.y;
            g[2] = raw.z;
            g[3] = raw.w;
        }
        float4 yv[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) yv[j] = load_nt(y + src[j] + c);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k) {
                if constexpr (kDyBF16) {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16(ws[j] * g[0]) | ((uint32_t)f32_to_bf16(ws[j] * g[1]) << 16);
                    pk.y = (uint32_t)f32_to_bf16(ws[j] * g[2]) | ((uint32_t)f32_to_bf16(ws[j] * g[3]) << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dyv) + src[j] + c) = pk;
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(dyv) + src[j] + c) =
                        make_float4(ws[j] * g[0], ws[j] * g[1], ws[j] * g[2], ws[j] * g[3]);
                }
                acc[j] = acc[j] + g[0] * yv[j].x;
                acc[j] = acc[j] + g[1] * yv[j].y;
                acc[j] = acc[j] + g[2] * yv[j].z;
                acc[j] = acc[j] + g[3] * yv[j].w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
            const float tot = wave_sum(acc[j]);
            if (lane == 0) dw[t * k + j] = scale * tot;
        }
    }
}

// ----------------------------------------------------------------- SwiGLU backward
template <bool kOutBF16>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float *__restrict__ gu,
                                                         const float *__restrict__ dh,
                                                         int64_t A, int I,
                                                         void *__restrict__ dguv) {
    // four consecutive features per thread (I is a multiple of 4): 16-byte loads, 8- or
    // 16-byte stores; the per-element arithmetic is unchanged
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= A * I) return;
    const int64_t p = i / I;
    const int n = (int)(i - p * I);
    const float4 g4 = *reinterpret_cast<const float4 *>(gu + p * 2 * I + n);
    const float4 u4 = *reinterpret_cast<const float4 *>(gu + p * 2 * I + I + n);
    const float4 d4 = *reinterpret_cast<const float4 *>(dh + i);
    const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, uv[4] = {u4.x, u4.y, u4.z, u4.w};
    const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
    float dg[4], du[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) swiglu_grad(gv[q], uv[q], dv[q], dg[q], du[q]);
    store_dgu4<kOutBF16>(dguv, p * 2 * I + n, I, dg, du);
}

// ------------------------------------------------------------ dx: slot-order sum
// One wave per (token, 512-feature slice); lane l takes features s*512 + 4l and
// s*512 + 256 + 4l. The token's k slot indices are loaded first, then every row load of
// both chunks (and the router part) is issued before the sums consume them.
constexpr int kDxSlice = 512;
__global__ __launch_bounds__(256) void dx_sum_kernel(const float *__restrict__ dxp,
                                                     const int32_t *__restrict__ inv,
                                                     const float *__restrict__ dxr,
                                                     int64_t T, int k, int d, int64_t A,
                                                     float *__restrict__ dx) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nslice = (d + kDxSlice - 1) / kDxSlice;
    const int64_t W = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = W / nslice;
    if (t >= T) return;
    const int c0 = (int)(W % nslice) * kDxSlice + lane * 4;
    int64_t src[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        int32_t p = (j < k) ? inv[t * k + j] : 0;
        p = (p < 0 || p >= A) ? 0 : p;
        src[j] = (int64_t)p * d;
    }
    float4 v[2][kMaxK], r[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = min(c0 + 256 * u, d - 4);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) v[u][j] = load_nt(dxp + src[j] + c);
        if (dxr) r[u] = *reinterpret_cast<const float4 *>(dxr + t * d + c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = c0 + 256 * u;
        if (c >= d) break;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j < k) {
                a0 = a0 + v[u][j].x;
                a1 = a1 + v[u][j].y;
                a2 = a2 + v[u][j].z;
                a3 = a3 + v[u][j].w;
            }
        }
        if (dxr) {
            a0 = a0 + r[u].x;
            a1 = a1 + r[u].y;
            a2 = a2 + r[u].z;
            a3 = a3 + r[u].w;
        }
        *reinterpret_cast<float4 *>(dx + t * d + c) = make_float4(a0, a1, a2, a3);
    }
}

// ------------------------------------------------------------------ router backward
// One 16-lane row per token (lane c holds experts c, c + 16, ...), as the forward router:
// the router's own top-k by (logit desc, id asc), p = exp(l - max) / Z with Z in the
// forward's order, then
//   s = ((p_sel0 + p_sel1) + ...), a = sum_j dw_j (p_selj / s), dp_j = (dw_j - a) / s,
//   c = sum_j dp_j p_selj, dl_e = p_e (dp_e - c)   (dp_e = 0 for an expert not chosen).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float *__restrict__ logits,
                                                         const float *__restrict__ dw,
                                                         int64_t T, int E, int k,
                                                         float *__restrict__ dl) {
    const int lane = threadIdx.x & 63, c = lane & 15;
    const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool tv = t < T;
    const int nv = (E + 15) >> 4;
    float lv[kRowVals];
    uint32_t hi[kRowVals];
    bool valid[kRowVals];
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) {
        valid[i] = i < nv && c + 16 * i < E;
        lv[i] = (tv && valid[i]) ? logits[t * E + c + 16 * i] : 0.f;
        hi[i] = valid[i] ? ordered_bits(lv[i]) : 0u;
    }
    uint32_t taken = 0, mkey0 = 0;
    int sel[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        sel[j] = -1;
        if (j < k) {
            uint32_t best = 0;
#pragma unroll
            for (int i = 0; i < kRowVals; ++i)
                if (i < nv && valid[i] && !((taken >> i) & 1u) && hi[i] > best) best = hi[i];
            const uint32_t m = row_max_u32(best);
            int cand = 0x7fffffff;
#pragma unroll
            for (int i = kRowVals - 1; i >= 0; --i)
                if (i < nv && valid[i] && !((taken >> i) & 1u) && hi[i] == m) cand = c + 16 * i;
            const int e = row_min_i32(cand);
            sel[j] = e;
            if (j == 0) mkey0 = m;
            if ((e & 15) == c) taken |= 1u << (e >> 4);
        }
    }
    const float mx = from_ordered_bits(mkey0);
    float p[kRowVals];
    float zl = 0.f;
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) {
        p[i] = valid[i] ? expf(lv[i] - mx) : 0.f;
        if (i < nv) zl = (i == 0) ? p[0] : zl + p[i];
    }
    const float Z = row_sum(zl);
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) p[i] = valid[i] ? p[i] / Z : 0.f;
    float ps[kMaxK], dwj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        ps[j] = (j < k) ? row_pick(p, sel[j], c, nv) : 0.f;
        dwj[j] = (j < k && tv) ? dw[t * k + j] : 0.f;
    }
    float s = ps[0];
#pragma unroll
    for (int j = 1; j < kMaxK; ++j)
        if (j < k) s = s + ps[j];
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
        if (j < k) a = a + dwj[j] * (ps[j] / s);
    float dp[kMaxK], cc = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        dp[j] = 0.f;
        if (j < k) {
            dp[j] = (dwj[j] - a) / s;
            cc = cc + dp[j] * ps[j];
        }
    }
    if (!tv) return;
#pragma unroll
    for (int i = 0; i < kRowVals; ++i) {
        if (!valid[i]) continue;
        const int e = c + 16 * i;
        float dpe = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k && sel[j] == e) dpe = dp[j];
        dl[t * E + e] = p[i] * (dpe - cc);
    }
}

// ---------------------------------------------------- FP32 gradient GEMMs (MFMA)
// Data gradient: out[p, n] = sum_k act[p, k] wgt[e, k, n] for the rows p of each segment
// (tile list (e, first row, rows)); act FP32 [rows, K], wgt [E, K, N] row-major (bf16 or
// FP32), out FP32 [rows, N]. Block: BN features x BT rows, four waves of (BN/2) x (BT/2).
// MFMA operand A = weight (rows = features n, K), B = activations (K, columns = rows p):
// lane l holds wgt[k0 + l/16][n + l%16] and act[p + l%16][k0 + l/16]; the result lane l
// holds row p + l%16, features n + 4(l/16) + 0..3.
template <bool kWBF16, int BN, int BT>
__global__ __launch_bounds__(256) void dgrad_kernel(const float *__restrict__ act,
                                                    const void *__restrict__ wgt,
                                                    float *__restrict__ out,
                                                    const int32_t *__restrict__ tiles, int K,
                                                    int N, int nft) {
    constexpr int WN = BN / 2, WTk = BT / 2, NF = WN / 16, NT = WTk / 16;
    constexpr int kAS = kKc + 1;                 // padded LDS row (floats), activations
    constexpr int kWS = BN + 4;                  // padded LDS row (floats), weights
    __shared__ float sa[2][BT * kAS];
    __shared__ float sw[2][kKc * kWS];
    const int mt = blockIdx.x / nft, ft = blockIdx.x % nft;
    if (mt >= tiles[0]) return;
    const int e = tiles[1 + 3 * mt], p0 = tiles[2 + 3 * mt], nrows = tiles[3 + 3 * mt];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn = wv & 1, wt = wv >> 1;
    const int n0 = ft * BN;
    const int64_t wbase = (int64_t)e * K * N;

    // staging: activations BT rows x kKc (float4 per thread per 64 rows),
    // weights kKc rows x BN (4 consecutive features per thread per 4*64 features)
    constexpr int AR = BT * kKc / 4 / 256;       // float4 loads per thread (activations)
    constexpr int WR = kKc * BN / 4 / 256;       // 4-element loads per thread (weights)
    static_assert(AR >= 1 && WR >= 1, "tile too small for 256 threads");
    float4 ra[AR], rw[WR];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int q = tid + 256 * i, r = q / (kKc / 4), kc = (q % (kKc / 4)) * 4;
            const int row = min(r, nrows - 1);
            ra[i] = *reinterpret_cast<const float4 *>(act + (int64_t)(p0 + row) * K + k0 + kc);
        }
#pragma unroll
        for (int i = 0; i < WR; ++i) {
            const int q = tid + 256 * i, r = q / (BN / 4), nc = (q % (BN / 4)) * 4;
            const int n = min(n0 + nc, N - 4);
            const int64_t o = wbase + (int64_t)(k0 + r) * N + n;
            if constexpr (kWBF16) {
                const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(wgt) + o);
                rw[i] = make_float4(bf16_to_f32((uint16_t)(v.x & 0xffff)), bf16_to_f32((uint16_t)(v.x >> 16)),
                                    bf16_to_f32((uint16_t)(v.y & 0xffff)), bf16_to_f32((uint16_t)(v.y >> 16)));
            } else {
                rw[i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(wgt) + o);
            }
        }
    };
    auto store = [&](int b) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int q = tid + 256 * i, r = q / (kKc / 4), kc = (q % (kKc / 4)) * 4;
            float *d = sa[b] + r * kAS + kc;
            d[0] = ra[i].x; d[1] = ra[i].y; d[2] = ra[i].z; d[3] = ra[i].w;
        }
#pragma unroll
        for (int i = 0; i < WR; ++i) {
            const int q = tid + 256 * i, r = q / (BN / 4), nc = (q % (BN / 4)) * 4;
            *reinterpret_cast<float4 *>(sw[b] + r * kWS + nc) = rw[i];
        }
    };
    f32x4_t acc[NF][NT];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15, g4 = lane >> 4;
    const int nk = K / kKc;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int b = kt & 1;
        if (kt + 1 < nk) load((kt + 1) * kKc);
#pragma unroll
        for (int kk = 0; kk < kKc; kk += 4) {
            float av[NF], bv[NT];
#pragma unroll
            for (int f = 0; f < NF; ++f) av[f] = sw[b][(kk + g4) * kWS + wn * WN + f * 16 + r16];
#pragma unroll
            for (int t = 0; t < NT; ++t) bv[t] = sa[b][(wt * WTk + t * 16 + r16) * kAS + kk + g4];
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[f], bv[t], acc[f][t], 0, 0, 0);
        }
        if (kt + 1 < nk) store(b ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = wt * WTk + t * 16 + r16;
        if (m >= nrows) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int n = n0 + wn * WN + f * 16 + g4 * 4;
            if (n >= N) continue;
            *reinterpret_cast<float4 *>(out + (int64_t)(p0 + m) * N + n) =
                make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]);
        }
    }
}

// Weight gradient: out[e, n, c] = sum over the segment's rows p ascending of
// a[p, n] b[p, c]; a FP32 [rows, N], b [rows, C] (bf16 or FP32; row of b = bperm[p] / bk
// when bperm is given: the gathered token rows), out FP32 [E, N, C]. Segment e = rows
// [off[e], off[e+1]) (off NULL: segments of seg_rows rows, or with seg_rows 0 one segment
// of nrows rows). Block: BN x BC outputs of one
// expert, four waves of (BN/2) x (BC/2); K = the segment's rows in stages of KC, the tail
// zero-filled. MFMA operand A = a (rows n, K = p), B = b (K = p, columns c): lane l holds
// a[p0 + l/16][n + l%16] and b[p0 + l/16][c + l%16]; the result lane l holds column
// c + l%16 of rows n + 4(l/16) + 0..3.
template <bool kBBF16, int BN, int BC, int KC = kKc>
__global__ __launch_bounds__(256) void wgrad_kernel(const float *__restrict__ a,
                                                    const void *__restrict__ b,
                                                    const int32_t *__restrict__ bperm, int bk,
                                                    int64_t bT, const int32_t *__restrict__ off,
                                                    int64_t nrows, int N, int C, int nbn,
                                                    int nbc, float *__restrict__ out,
                                                    int64_t seg_rows = 0) {
    constexpr int WN = BN / 2, WC = BC / 2, NF = WN / 16, NC = WC / 16;
    constexpr int kAS = BN + 4, kBS = BC + 4;
    __shared__ float sa[2][KC * kAS];
    __shared__ float sb[2][KC * kBS];
    const int per_e = nbn * nbc;
    const int e = blockIdx.x / per_e, rem = blockIdx.x % per_e;
    const int n0 = (rem / nbc) * BN, c0 = (rem % nbc) * BC;
    int64_t r0 = 0, r1 = nrows;
    if (off) {
        r0 = min<int64_t>(max(off[e], 0), nrows);
        r1 = min<int64_t>(max<int64_t>(off[e + 1], r0), nrows);
    } else if (seg_rows > 0) {
        r0 = min<int64_t>((int64_t)e * seg_rows, nrows);
        r1 = min<int64_t>(r0 + seg_rows, nrows);
    }
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn = wv & 1, wc = wv >> 1;
    // float4 copies per thread and stage (threads past KC * BN / 4 copy nothing)
    constexpr int AR = (KC * BN / 4 + 255) / 256, BR = (KC * BC / 4 + 255) / 256;
    constexpr int AQ = KC * BN / 4, BQ = KC * BC / 4;
    static_assert(NF >= 1 && NC >= 1, "tile too small");
    float4 ra[AR], rb[BR];
    auto load = [&](int64_t p0) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int q = tid + 256 * i, r = q / (BN / 4), nc = (q % (BN / 4)) * 4;
            const int64_t p = p0 + r;
            ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (q < AQ && p < r1)
                ra[i] = *reinterpret_cast<const float4 *>(a + p * N + min(n0 + nc, N - 4));
        }
#pragma unroll
        for (int i = 0; i < BR; ++i) {
            const int q = tid + 256 * i, r = q / (BC / 4), cc = (q % (BC / 4)) * 4;
            const int64_t p = p0 + r;
            rb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (q < BQ && p < r1) {
                int64_t row = p;
                if (bperm) row = min<int64_t>((int64_t)max(bperm[p], 0) / bk, bT - 1);
                const int64_t o = row * C + min(c0 + cc, C - 4);
                if constexpr (kBBF16) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(b) + o);
                    rb[i] = make_float4(bf16_to_f32((uint16_t)(v.x & 0xffff)), bf16_to_f32((uint16_t)(v.x >> 16)),
                                        bf16_to_f32((uint16_t)(v.y & 0xffff)), bf16_to_f32((uint16_t)(v.y >> 16)));
                } else {
                    rb[i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(b) + o);
                }
            }
        }
    };
    auto store = [&](int s) {
#pragma unroll
        for (int i = 0; i < AR; ++i) {
            const int q = tid + 256 * i, r = q / (BN / 4), nc = (q % (BN / 4)) * 4;
            if (q < AQ) *reinterpret_cast<float4 *>(sa[s] + r * kAS + nc) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BR; ++i) {
            const int q = tid + 256 * i, r = q / (BC / 4), cc = (q % (BC / 4)) * 4;
            if (q < BQ) *reinterpret_cast<float4 *>(sb[s] + r * kBS + cc) = rb[i];
        }
    };
    f32x4_t acc[NF][NC];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NC; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t nk = (r1 - r0 + KC - 1) / KC;
    if (nk > 0) {
        load(r0);
        store(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int s = (int)(kt & 1);
            if (kt + 1 < nk) load(r0 + (kt + 1) * KC);
#pragma unroll
            for (int kk = 0; kk < KC; kk += 4) {
                float av[NF], bv[NC];
#pragma unroll
                for (int f = 0; f < NF; ++f) av[f] = sa[s][(kk + g4) * kAS + wn * WN + f * 16 + r16];
#pragma unroll
                for (int t = 0; t < NC; ++t) bv[t] = sb[s][(kk + g4) * kBS + wc * WC + t * 16 + r16];
#pragma unroll
                for (int f = 0; f < NF; ++f)
#pragma unroll
                    for (int t = 0; t < NC; ++t)
                        acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[f], bv[t], acc[f][t], 0, 0, 0);
            }
            if (kt + 1 < nk) store(s ^ 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int cc = c0 + wc * WC + t * 16 + r16;
        if (cc >= C) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = n0 + wn * WN + f * 16 + g4 * 4 + i;
                if (n < N) out[((int64_t)e * N + n) * C + cc] = acc[f][t][i];
            }
        }
    }
}

// ------------------------------------------------- bf16 weight gradient (MFMA 16x16x32)
// out[e, n, c] = sum over the segment's rows p ascending of a[p, n] b[p, c], a and b bf16
// (b gathered through bperm / bk when given), FP32 accumulation and output.
// Stages of 32 rows x 512 bytes (256 features) per operand are copied global -> LDS by DMA
// (global_load_lds) into an NS-slot ring, NS - 1 stages in flight: one 1 KB DMA
// instruction per 2 rows, lane l moving 16-byte chunk (l % 32) ^ kmajor_swz(row) of row
// 2i + l/32, so row r's chunk c sits at c ^ kmajor_swz(r).
// The MFMA wants 8 consecutive K values (rows p) per lane; gfx950's transposing LDS read
// (ds_read_b64_tr_b16) delivers them: within each 16-lane group, lane s names 4
// consecutive features of one row, and lane i receives, in slot j, the element that lane
// 4j + i/4 named at position i % 4. With lane s of group g naming row 8g + j0 + s/4
// (j0 = 0, then 4) at features f0 + 4(s % 4) .. +3, lane i gets feature f0 + i at rows
// 8g + j0 + 0..3: two reads give the MFMA operand of feature f0 + i, K = rows 8g .. 8g + 7
// of the stage. Rows past the segment are fetched from its last row and zeroed in the
// fragments of the last stage (their products are 0 * 0). With bperm, the activation
// rows' token indices of stage s + 2 are loaded while stage s is issued (two register
// sets; wave-uniform, so through the scalar unit, whose lgkmcnt does not pace the ring).
// Block: 256 x 256 outputs on 8 waves of 64 x 128; the result lane l holds column
// c + l%16 of rows n + 4(l/16) + 0..3.
template <int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wgrad_dma_kernel(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b,
                      const int32_t *__restrict__ bperm, int bk, int64_t bT,
                      const int32_t *__restrict__ off, int64_t nrows, int N, int C, int nbn,
                      int nbc, float *__restrict__ out) {
    constexpr int BN = 256, BC = 256, KR = 32, WNW = 4, NW = 8;
    constexpr int WN = BN / WNW, WC = BC / (NW / WNW), NF = WN / 16, NC = WC / 16;
    constexpr int kOpBytes = KR * 2 * BN;               // one operand's stage: 16 KB
    constexpr int kStage = 2 * kOpBytes;
    static_assert(BN == BC && 2 * BN == 512, "512-byte rows: 2 rows per DMA instruction");
    // the epilogue reuses the ring for two passes of 128 output rows of kOutStride floats
    constexpr int kOutStride = BC + 4;
    constexpr int kRing = NS * kStage, kOut = 128 * kOutStride * 4;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing > kOut ? kRing : kOut];
    const int per_e = nbn * nbc;
    const int e = blockIdx.x / per_e, rem = blockIdx.x % per_e;
    const int n0 = (rem / nbc) * BN, c0 = (rem % nbc) * BC;
    int64_t r0 = 0, r1 = nrows;
    if (off) {
        r0 = min<int64_t>(max(off[e], 0), nrows);
        r1 = min<int64_t>(max<int64_t>(off[e + 1], r0), nrows);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wn = wv % WNW, wc = wv / WNW;
    const int64_t nk = (r1 - r0 + KR - 1) / KR;
    // DMA roles: instructions i = 0, 1 move a-rows 2 (wv + 8 i) + lane / 32, i = 2, 3 the
    // b-rows 2 (wv + 8 (i - 2)) + lane / 32; the lane's chunk position is lane % 32
    const int pc = lane & 31;
    const int rA0 = 2 * wv + (lane >> 5), rA1 = rA0 + 16;      // rows of this lane's DMAs
    const int colA0 = min(n0 + 8 * (pc ^ kmajor_swz<32>(rA0)), N - 8);
    const int colA1 = min(n0 + 8 * (pc ^ kmajor_swz<32>(rA1)), N - 8);
    const int colB0 = min(c0 + 8 * (pc ^ kmajor_swz<32>(rA0)), C - 8);
    const int colB1 = min(c0 + 8 * (pc ^ kmajor_swz<32>(rA1)), C - 8);
    auto row_of = [&](int64_t s, int r) { return min<int64_t>(r0 + s * KR + r, r1 - 1); };
    auto src_of = [&](int32_t idx) {
        return min<int64_t>((int64_t)max(idx, 0) / bk, bT - 1);
    };
    // token indices (bperm) of the wave's four b-rows 2 wv + {0, 1, 16, 17} of a stage:
    // wave-uniform, so they come through the scalar unit (lgkmcnt, not the vmcnt that
    // paces the DMA ring); the half-wave picks its row's value
    int32_t ix[2][4];
    auto load_idx = [&](int64_t s, int32_t (&dst)[4]) {
        const int64_t sc = min<int64_t>(s, nk - 1);            // past the end: any valid row
        dst[0] = bperm[row_of(sc, 2 * wv)];
        dst[1] = bperm[row_of(sc, 2 * wv + 1)];
        dst[2] = bperm[row_of(sc, 2 * wv + 16)];
        dst[3] = bperm[row_of(sc, 2 * wv + 17)];
    };
    auto issue = [&](int64_t s, const int32_t (&idx)[4]) {
#if defined(__HIP_DEVICE_COMPILE__)
        uint8_t *slot = ring + (int)(s % NS) * kStage;
        const int64_t pa0 = row_of(s, rA0), pa1 = row_of(s, rA1);
        const bool hi = lane >= 32;
        const int64_t pb0 = bperm ? src_of(hi ? idx[1] : idx[0]) : pa0;
        const int64_t pb1 = bperm ? src_of(hi ? idx[3] : idx[2]) : pa1;
        __builtin_amdgcn_global_load_lds(a + pa0 * N + colA0,
            (__attribute__((address_space(3))) void *)(slot + wv * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a + pa1 * N + colA1,
            (__attribute__((address_space(3))) void *)(slot + (wv + 8) * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(b + pb0 * C + colB0,
            (__attribute__((address_space(3))) void *)(slot + kOpBytes + wv * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(b + pb1 * C + colB1,
            (__attribute__((address_space(3))) void *)(slot + kOpBytes + (wv + 8) * 1024), 16, 0, 0);
#endif
    };

    f32x4_t acc[NF][NC];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int t = 0; t < NC; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15, g4 = lane >> 4;
    // transposing reads: this lane names row 8 g4 + r16/4 (+4) at features 4 (r16 % 4) .. +3
    // of a fragment; both rows share kmajor_swz
    const int trow = (8 * g4 + (r16 >> 2)) * (2 * BN);
    const int tsw = kmajor_swz<32>(8 * g4 + (r16 >> 2));
    auto frag_ptr = [&](const uint8_t *base, int feat0) {
        const int byte = 2 * feat0 + 8 * (r16 & 3);
        return base + trow + ((((byte >> 4) ^ tsw) << 4) | (byte & 15));
    };
    auto compute = [&](const uint8_t *slot, int valid) {
        i32x2_t alo[NF], ahi[NF], blo[NC], bhi[NC];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const uint8_t *p = frag_ptr(slot, wn * WN + f * 16);
            alo[f] = tr_read(p);
            ahi[f] = tr_read(p + 4 * (2 * BN));
        }
#pragma unroll
        for (int t = 0; t < NC; ++t) {
            const uint8_t *p = frag_ptr(slot + kOpBytes, wc * WC + t * 16);
            blo[t] = tr_read(p);
            bhi[t] = tr_read(p + 4 * (2 * BN));
        }
        tr_fence();
        bf16x8_t av[NF], bv[NC];
#pragma unroll
        for (int f = 0; f < NF; ++f) av[f] = tr_take(alo[f], ahi[f]);
#pragma unroll
        for (int t = 0; t < NC; ++t) bv[t] = tr_take(blo[t], bhi[t]);
        if (valid < KR) {   // last stage: rows 8 g4 + j (j < 8) at or past `valid` hold 0
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (8 * g4 + j >= valid) {
#pragma unroll
                    for (int f = 0; f < NF; ++f) av[f][j] = (__bf16)0.0f;
#pragma unroll
                    for (int t = 0; t < NC; ++t) bv[t][j] = (__bf16)0.0f;
                }
            }
        }
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int t = 0; t < NC; ++t)
                acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[f], bv[t], acc[f][t], 0, 0, 0);
    };

    if (nk > 0) {
        // prologue: stages 0 .. NS-2 (their index loads waited on in place), then the
        // index sets of stages NS-1 and NS
#pragma unroll
        for (int st = 0; st < NS - 1; ++st) {
            if (st < nk) {
                int32_t idx[4] = {0, 0, 0, 0};
                if (bperm) load_idx(st, idx);
                issue(st, idx);
            }
        }
        if (bperm) {
            load_idx(NS - 1, ix[(NS - 1) & 1]);
            load_idx(NS, ix[NS & 1]);
        }
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        // iteration kt issues stage kt + NS - 1 (index set of its parity) and reloads that
        // set with stage kt + NS + 1's indices
        for (int64_t kt = 0; kt < nk; kt += 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t k2 = kt + h;
                if (k2 >= nk) break;
                constexpr int par = (NS - 1) & 1;     // parity of kt + NS - 1 for even kt
                const bool issuing = k2 + NS - 1 < nk;
                if (issuing) {
                    issue(k2 + NS - 1, ix[par ^ h]);
                    if (bperm) load_idx(k2 + NS + 1, ix[par ^ h]);
                }
                compute(ring + (int)(k2 % NS) * kStage,
                        (int)min<int64_t>(KR, r1 - (r0 + k2 * KR)));
                if (k2 + 1 < nk) {
                    // stage kt + 1's DMA was followed by NS - 2 iterations of 4 DMAs each
                    // (the index loads are scalar: lgkmcnt, which this also drains)
                    if (issuing) wait_vm_lgkm0<(NS - 2) * 4>();
                    else wait_vm_lgkm0<0>();
                    __builtin_amdgcn_s_barrier();
                }
            }
        }
    }
    // epilogue through LDS, in two passes of 128 rows x 256 columns (rows f = 2 pass, 2 pass
    // + 1 of every wave); a row stride of 260 floats puts the four 4-row groups of one
    // scalar LDS store in different banks; each row then leaves as 64 lanes x 16 bytes
    static_assert(NF == 4 && WNW * 32 == 128 && (NW / WNW) * WC == BC, "epilogue tiling");
    float *stage = reinterpret_cast<float *>(ring);
    __syncthreads();   // every wave is past its last fragment read
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int fh = 0; fh < 2; ++fh)
#pragma unroll
            for (int t = 0; t < NC; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    stage[(wn * 32 + fh * 16 + g4 * 4 + i) * kOutStride + wc * WC + t * 16 + r16] =
                        acc[2 * pass + fh][t][i];
        __syncthreads();
        const int cc = c0 + 4 * lane;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int lr = wv + 8 * q;                         // staged row 0 .. 127
            const int n = n0 + (lr >> 5) * WN + 32 * pass + (lr & 31);
            const float4 v = *reinterpret_cast<const float4 *>(stage + lr * kOutStride + 4 * lane);
            if (n < N && cc < C)
                store_nt(out + ((int64_t)e * N + n) * C + cc, v);
        }
        if (pass == 0) __syncthreads();
    }
}

}  // namespace

// ------------------------------------------------------------------------ launchers
constexpr int kDgBN = 128, kDgBT = 64;     // data-gradient tile: features x rows
constexpr int kWgBN = 64, kWgBC = 64;      // weight-gradient tile

hipError_t launch_combine_bwd(const moe_dims &dm, const void *dout, const float *y,
                              const int32_t *inv, const float *topk_w, float scale, void *dy,
                              float *dw, bool dy_bf16, hipStream_t s) {
    if (dm.T == 0) return hipGetLastError();
    const dim3 grid((unsigned)((dm.T + 3) / 4));
    const int64_t A = dm.T * dm.k;
    if (dm.dtype == MOE_BF16 && dy_bf16)
        combine_bwd_kernel<true, true><<<grid, dim3(256), 0, s>>>(dout, y, inv, topk_w, dm.T,
                                                                  dm.k, dm.d, A, scale, dy, dw);
    else if (dm.dtype == MOE_BF16)
        combine_bwd_kernel<true, false><<<grid, dim3(256), 0, s>>>(dout, y, inv, topk_w, dm.T,
                                                                   dm.k, dm.d, A, scale, dy, dw);
    else
        combine_bwd_kernel<false, false><<<grid, dim3(256), 0, s>>>(dout, y, inv, topk_w, dm.T,
                                                                    dm.k, dm.d, A, scale, dy, dw);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const moe_dims &dm, const float *gu, const float *dh, void *dgu,
                             bool out_bf16, hipStream_t s) {
    const int64_t n = dm.T * dm.k * dm.inter / 4;     // four features per thread
    if (n == 0) return hipGetLastError();
    const dim3 grid((unsigned)((n + 255) / 256));
    if (out_bf16)
        swiglu_bwd_kernel<true><<<grid, dim3(256), 0, s>>>(gu, dh, dm.T * dm.k, dm.inter, dgu);
    else
        swiglu_bwd_kernel<false><<<grid, dim3(256), 0, s>>>(gu, dh, dm.T * dm.k, dm.inter, dgu);
    return hipGetLastError();
}

// bf16 weight gradient over segments (see wgrad_dma_kernel); N and C multiples of 8.
hipError_t launch_wgrad_bf16(int nseg, const void *a, const void *b, const int32_t *bperm,
                             int bk, int64_t bT, const int32_t *off, int64_t nrows, int N,
                             int C, float *out, hipStream_t s) {
    if (N % 8 || C % 8 || nseg < 1) return hipErrorInvalidValue;
    constexpr int NS = 4;   // ring slots: 3 stages in flight
    const int nbn = (N + 255) / 256, nbc = (C + 255) / 256;
    wgrad_dma_kernel<NS><<<dim3((unsigned)((int64_t)nseg * nbn * nbc)), dim3(512), 0, s>>>(
        static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(b), bperm, bk, bT, off,
        nrows, N, C, nbn, nbc, out);
    return hipGetLastError();
}


hipError_t launch_dx_sum(const moe_dims &dm, const float *dxp, const int32_t *inv,
                         const float *dxr, float *dx, hipStream_t s) {
    if (dm.T == 0) return hipGetLastError();
    const int64_t waves = dm.T * ((dm.d + kDxSlice - 1) / kDxSlice);
    dx_sum_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s>>>(
        dxp, inv, dxr, dm.T, dm.k, dm.d, dm.T * dm.k, dx);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const moe_dims &dm, const float *logits, const float *dw,
                             float *dl, hipStream_t s) {
    if (dm.T == 0) return hipGetLastError();
    router_bwd_kernel<<<dim3((unsigned)((dm.T + 15) / 16)), dim3(256), 0, s>>>(
        logits, dw, dm.T, dm.E, dm.k, dl);
    return hipGetLastError();
}

// out[p, :] = act[p, :] wgt[e] over the segments of offsets (tiles built into ws.tiles).
hipError_t launch_dgrad(const moe_dims &dm, const float *act, const void *wgt, bool wbf16,
                        int K, int N, const int32_t *offsets, float *out, const Workspace &ws,
                        hipStream_t s) {
    const int64_t A = dm.T * dm.k;
    if (A == 0) return hipGetLastError();
    if (K % kKc || N % 4) return hipErrorInvalidValue;
    const int64_t cap = max_m_tiles(A, dm.E, kDgBT);
    const hipError_t e = launch_build_tiles(offsets, dm.E, A, kDgBT, cap, ws.tiles, s);
    if (e != hipSuccess) return e;
    const int nft = (N + kDgBN - 1) / kDgBN;
    const dim3 grid((unsigned)(cap * nft));
    if (wbf16)
        dgrad_kernel<true, kDgBN, kDgBT><<<grid, dim3(256), 0, s>>>(act, wgt, out, ws.tiles, K, N, nft);
    else
        dgrad_kernel<false, kDgBN, kDgBT><<<grid, dim3(256), 0, s>>>(act, wgt, out, ws.tiles, K, N, nft);
    return hipGetLastError();
}

// out[e] = a^T b over each segment's rows (off NULL: one segment of nrows rows).
hipError_t launch_wgrad(int nseg, const float *a, const void *b, bool bbf16,
                        const int32_t *bperm, int bk, int64_t bT, const int32_t *off,
                        int64_t nrows, int N, int C, float *out, hipStream_t s) {
    if (N % 4 || C % 4 || nseg < 1) return hipErrorInvalidValue;
    const int nbn = (N + kWgBN - 1) / kWgBN, nbc = (C + kWgBC - 1) / kWgBC;
    const dim3 grid((unsigned)((int64_t)nseg * nbn * nbc));
    if (bbf16)
        wgrad_kernel<true, kWgBN, kWgBC><<<grid, dim3(256), 0, s>>>(a, b, bperm, bk, bT, off,
                                                                   nrows, N, C, nbn, nbc, out);
    else
        wgrad_kernel<false, kWgBN, kWgBC><<<grid, dim3(256), 0, s>>>(a, b, bperm, bk, bT, off,
                                                                    nrows, N, C, nbn, nbc, out);
    return hipGetLastError();
}

// dx_r[t, c] = sum over e of dl[t, e] w_router[e, c] on FP32 MFMA (16x16x4): a block of
// 4 waves covers 64 tokens x 64 features, wave w tokens 16w .. 16w+15; A = 16 router-weight
// features x 4 experts, B = 4 experts x 16 tokens, K = the experts ascending, 4 per step.
// Each 64-expert chunk of dl (64 tokens) and of the weights (64 features, widened to FP32)
// is copied to LDS with coalesced loads first; the result goes through LDS so that every
// output row leaves as 16 lanes x 16 bytes.
constexpr int kRdxT = 64, kRdxC = 64, kRdxE = 64, kRdxLd = kRdxE + 1, kRdxOut = kRdxC + 4;
__global__ __launch_bounds__(256) void router_dx_kernel(const float *__restrict__ dl,
                                                        const void *__restrict__ wr, bool bf16,
                                                        int64_t T, int E, int d,
                                                        float *__restrict__ dx) {
    __shared__ float sdl[kRdxT * kRdxLd];      // [token][expert of the chunk]
    __shared__ float sw[kRdxE * kRdxOut];      // [expert of the chunk][feature]
    __shared__ float sout[kRdxT * kRdxOut];    // [token][feature]
    const int ncb = (d + kRdxC - 1) / kRdxC;
    const int64_t t0 = (int64_t)(blockIdx.x / ncb) * kRdxT;
    const int c0 = (int)(blockIdx.x % ncb) * kRdxC;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    f32x4_t acc[kRdxC / 16];
#pragma unroll
    for (int f = 0; f < kRdxC / 16; ++f) acc[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int e0 = 0; e0 < E; e0 += kRdxE) {
        const int ne = min(kRdxE, E - e0);
        __syncthreads();   // the previous chunk's LDS reads are done
        if (E % 4 == 0) {   // 16-byte loads of dl rows
            for (int i = tid; i < kRdxT * kRdxE / 4; i += 256) {
                const int tt = i / (kRdxE / 4), ee = (i % (kRdxE / 4)) * 4;
                const int64_t t = t0 + tt;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (t < T && ee < ne) v = *reinterpret_cast<const float4 *>(dl + t * E + e0 + ee);
                float *q = sdl + tt * kRdxLd + ee;
                q[0] = v.x;
                q[1] = v.y;
                q[2] = v.z;
                q[3] = v.w;
            }
        } else {
            for (int i = tid; i < kRdxT * kRdxE; i += 256) {
                const int tt = i / kRdxE, ee = i % kRdxE;
                const int64_t t = t0 + tt;
                sdl[tt * kRdxLd + ee] = (t < T && ee < ne) ? dl[t * E + e0 + ee] : 0.f;
            }
        }
        // router weights: 8 features (16 or 32 bytes) per load; d is a multiple of 64
        for (int i = tid; i < kRdxE * kRdxC / 8; i += 256) {
            const int ee = i / (kRdxC / 8), cc = (i % (kRdxC / 8)) * 8;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (ee < ne) {
                const int64_t o = (int64_t)(e0 + ee) * d + c0 + cc;
                if (bf16) {
                    const uint4 raw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(wr) + o);
                    const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v[2 * q] = bf16_to_f32((uint16_t)(wv[q] & 0xffffu));
                        v[2 * q + 1] = bf16_to_f32((uint16_t)(wv[q] >> 16));
                    }
                } else {
                    const float4 x0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(wr) + o);
                    const float4 x1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(wr) + o + 4);
                    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
                    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
                }
            }
            *reinterpret_cast<float4 *>(sw + ee * kRdxOut + cc) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(sw + ee * kRdxOut + cc + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
        __syncthreads();
        for (int k0 = 0; k0 < ne; k0 += 4) {
            const float b = sdl[(16 * wave + r) * kRdxLd + k0 + g];
#pragma unroll
            for (int f = 0; f < kRdxC / 16; ++f) {
                const float a = sw[(k0 + g) * kRdxOut + 16 * f + r];
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[f], 0, 0, 0);
            }
        }
    }
    // result lane l: token 16 wave + l%16, features 16 f + 4 (l/16) + 0..3
#pragma unroll
    for (int f = 0; f < kRdxC / 16; ++f)
        *reinterpret_cast<float4 *>(sout + (16 * wave + r) * kRdxOut + 16 * f + 4 * g) =
            make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]);
    __syncthreads();
    for (int i = tid; i < kRdxT * (kRdxC / 4); i += 256) {
        const int tt = i / (kRdxC / 4), cc = (i % (kRdxC / 4)) * 4;
        const int64_t t = t0 + tt;
        if (t < T && c0 + cc < d)
            *reinterpret_cast<float4 *>(dx + t * d + c0 + cc) =
                *reinterpret_cast<const float4 *>(sout + tt * kRdxOut + cc);
    }
}

// dw_router[e, c] = sum over t ascending of dl[t, e] x[t, c] when E is not a multiple of 4
// (the MFMA weight-gradient kernel reads 4 experts at a time).
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float *__restrict__ dl,
                                                           const void *__restrict__ x, bool bf16,
                                                           int64_t T, int E, int d,
                                                           float *__restrict__ dwr) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)E * d) return;
    const int e = (int)(i / d), c = (int)(i - (int64_t)e * d);
    float acc = 0.f;
    for (int64_t t = 0; t < T; ++t) {
        const float xv = bf16 ? bf16_to_f32(static_cast<const uint16_t *>(x)[t * d + c])
                              : static_cast<const float *>(x)[t * d + c];
        acc = acc + dl[t * E + e] * xv;
    }
    dwr[i] = acc;
}

// dwr[i] = part[0][i] + part[1][i] + ... + part[S-1][i], left to right.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float *__restrict__ part, int S,
                                                        int64_t n, float *__restrict__ out) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float4 acc = *reinterpret_cast<const float4 *>(part + i);
    for (int j = 1; j < S; ++j) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (int64_t)j * n + i);
        acc.x = acc.x + v.x;
        acc.y = acc.y + v.y;
        acc.z = acc.z + v.z;
        acc.w = acc.w + v.w;
    }
    *reinterpret_cast<float4 *>(out + i) = acc;
}

hipError_t launch_router_wgrad(const moe_dims &dm, const float *dl, const void *x, float *dwr,
                               float *scratch, int64_t scratch_floats, hipStream_t s) {
    if (dm.E % 4 == 0 && dm.d % 4 == 0) {
        // only E x d outputs, over a T-long sum: 32 x 32 tiles (E d / 1024 blocks) with
        // 64-row stages, and, when the scratch holds them, the rows split into S ascending
        // segments of at least 256 rows whose partials are then added in segment order
        const int64_t n = (int64_t)dm.E * dm.d;
        int S = (int)std::max<int64_t>(1, std::min<int64_t>(kRouterWgradSplit, dm.T / 256));
        if (!scratch || scratch_floats < S * n) S = 1;
        const int64_t seg = (dm.T + S - 1) / S;
        float *dst = S > 1 ? scratch : dwr;
        const int nbn = (dm.E + 31) / 32, nbc = (dm.d + 31) / 32;
        const dim3 grid((unsigned)((int64_t)S * nbn * nbc));
        if (dm.dtype == MOE_BF16)
            wgrad_kernel<true, 32, 32, 64><<<grid, dim3(256), 0, s>>>(
                dl, x, nullptr, 1, dm.T, nullptr, dm.T, dm.E, dm.d, nbn, nbc, dst,
                S > 1 ? seg : 0);
        else
            wgrad_kernel<false, 32, 32, 64><<<grid, dim3(256), 0, s>>>(
                dl, x, nullptr, 1, dm.T, nullptr, dm.T, dm.E, dm.d, nbn, nbc, dst,
                S > 1 ? seg : 0);
        if (S > 1)
            sum_parts_kernel<<<dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s>>>(
                scratch, S, n, dwr);
        return hipGetLastError();
    }
    const int64_t n = (int64_t)dm.E * dm.d;
    router_wgrad_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
        dl, x, dm.dtype == MOE_BF16, dm.T, dm.E, dm.d, dwr);
    return hipGetLastError();
}

hipError_t launch_router_dx(const moe_dims &dm, const float *dl, const void *w_router,
                            float *dx, hipStream_t s) {
    if (dm.T == 0) return hipGetLastError();
    const int64_t blocks = (dm.T + kRdxT - 1) / kRdxT * ((dm.d + kRdxC - 1) / kRdxC);
    router_dx_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        dl, w_router, dm.dtype == MOE_BF16, dm.T, dm.E, dm.d, dx);
    return hipGetLastError();
}

}  // namespace moe
