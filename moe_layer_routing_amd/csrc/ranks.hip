// ranks.hip -- expert-parallel output on one device: rank partial outputs, their FP64
// pairwise tree, and the shared expert sharded over the ranks.
//
// "0 train-infer mismatch for Open-weight MoE RL in Open-source code", "Sharding the
// experts": with R ranks each owning E/R expert slots, rank r accumulates every routing
// slot of a token in FP32 in slot order, a slot owned by another rank contributing an
// exact zero, adds its shard of the shared expert and rounds once to BF16; the R partial
// outputs, in logical rank order, are reduced by adding adjacent pairs in FP64 (an odd last
// contributor is carried to the next level unchanged) until one value remains, which is
// rounded once to BF16. The routed scaling factor ("Choosing GLM's eight experts")
// multiplies the routed sum before the shared shard is added.
//
// The shared expert (the shared-expert passage: the dense fixed-K projections and SwiGLU,
// one shard per rank along the inter dimension) is the grouped GEMM with R segments, each
// holding every token: segment r has rows p = r*T + t gathered from token t (perm[p] =
// t*R + r, read as perm[p] / R), and rank r's weights. Its rows are therefore bitwise the
// rows of any other batch size, like every routed row.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSlice = 512;   // features per wave, as the plain combine

// Round a double to bf16, to nearest with ties to even, in one step: the double is first
// rounded toward zero to FP32 with the lowest bit forced to 1 when inexact ("round to
// odd"); FP32 keeps 16 more significand bits than bf16, so the RNE rounding of that odd
// value to bf16 is the RNE rounding of the double (no double-rounding error).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    float t = __double2float_rz(x);
    if ((double)t != x) t = __uint_as_float(__float_as_uint(t) | 1u);
    return f32_to_bf16(t);
}

// One wave per (token, 512-feature slice); lane l takes features s*512 + 4l and
// s*512 + 256 + 4l, as the plain combine. The R partials of each feature stay in
// registers; the tree's shape is fixed by R alone.
template <bool kBF16, int R>
__global__ __launch_bounds__(256) void combine_ranks_kernel(
    const float *__restrict__ y, const int32_t *__restrict__ inv,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ slot_map, int64_t T, int k, int d, int E, int64_t A,
    float scale, const float *__restrict__ ys, void *__restrict__ partials,
    void *__restrict__ out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nslice = (d + kSlice - 1) / kSlice;
    const int64_t W = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = W / nslice;
    if (t >= T) return;
    const int c0 = (int)(W % nslice) * kSlice + lane * 4;
    const int H = E / R;
    int64_t src[kMaxK];
    float w[kMaxK];
    int owner[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        int32_t p = (j < k) ? inv[t * k + j] : 0;
        p = (p < 0 || p >= A) ? 0 : p;
        src[j] = (int64_t)p * d;
        w[j] = (j < k) ? topk_w[t * k + j] : 0.f;
        owner[j] = -1;
        if (j < k) {
            const int e = topk_idx[t * k + j];
            int v = (e >= 0 && e < E) ? (slot_map ? slot_map[e] : e) : -1;
            owner[j] = (v >= 0 && v < E) ? v / H : -1;
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = c0 + 256 * u;
        if (c >= d) break;
        float4 v[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) v[j] = *reinterpret_cast<const float4 *>(y + src[j] + c);
        float4 prod[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k)
                prod[j] = make_float4(w[j] * v[j].x, w[j] * v[j].y, w[j] * v[j].z, w[j] * v[j].w);
        double lv[4][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    const bool own = owner[j] == r;
                    a0 = a0 + (own ? prod[j].x : 0.f);
                    a1 = a1 + (own ? prod[j].y : 0.f);
                    a2 = a2 + (own ? prod[j].z : 0.f);
                    a3 = a3 + (own ? prod[j].w : 0.f);
                }
            }
            a0 = scale * a0;
            a1 = scale * a1;
            a2 = scale * a2;
            a3 = scale * a3;
            if (ys) {
                const float4 s4 = *reinterpret_cast<const float4 *>(ys + ((int64_t)r * T + t) * d + c);
                a0 = a0 + s4.x;
                a1 = a1 + s4.y;
                a2 = a2 + s4.z;
                a3 = a3 + s4.w;
            }
            if constexpr (kBF16) {
                const uint16_t b0 = f32_to_bf16(a0), b1 = f32_to_bf16(a1), b2 = f32_to_bf16(a2),
                               b3 = f32_to_bf16(a3);
                if (partials) {
                    uint2 pk;
                    pk.x = (uint32_t)b0 | ((uint32_t)b1 << 16);
                    pk.y = (uint32_t)b2 | ((uint32_t)b3 << 16);
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(partials) +
                                               ((int64_t)r * T + t) * d + c) = pk;
                }
                lv[0][r] = bf16_to_f32(b0);
                lv[1][r] = bf16_to_f32(b1);
                lv[2][r] = bf16_to_f32(b2);
                lv[3][r] = bf16_to_f32(b3);
            } else {
                if (partials)
                    *reinterpret_cast<float4 *>(static_cast<float *>(partials) +
                                                ((int64_t)r * T + t) * d + c) =
                        make_float4(a0, a1, a2, a3);
                lv[0][r] = a0;
                lv[1][r] = a1;
                lv[2][r] = a2;
                lv[3][r] = a3;
            }
        }
        // adjacent pairs in FP64, the odd last value carried, level by level
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int n = R; n > 1; n = (n + 1) / 2) {
#pragma unroll
                for (int i = 0; i < n / 2; ++i) lv[q][i] = lv[q][2 * i] + lv[q][2 * i + 1];
                if (n & 1) lv[q][n / 2] = lv[q][n - 1];
            }
        }
        if constexpr (kBF16) {
            uint2 pk;
            pk.x = (uint32_t)f64_to_bf16(lv[0][0]) | ((uint32_t)f64_to_bf16(lv[1][0]) << 16);
            pk.y = (uint32_t)f64_to_bf16(lv[2][0]) | ((uint32_t)f64_to_bf16(lv[3][0]) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + t * d + c) = pk;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(out) + t * d + c) =
                make_float4((float)lv[0][0], (float)lv[1][0], (float)lv[2][0], (float)lv[3][0]);
        }
    }
}

// Rows of the shared expert's grouped GEMM: segment r = rows [r*T, (r+1)*T), row r*T + t
// gathered from token t (flat id t*R + r), offsets r*T.
__global__ __launch_bounds__(256) void shared_rows_kernel(int64_t T, int R,
                                                          int32_t *__restrict__ perm,
                                                          int32_t *__restrict__ offsets) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < T * R) {
        const int64_t r = i / T, t = i - r * T;
        perm[i] = (int32_t)(t * R + r);
    }
    if (i <= R) offsets[i] = (int32_t)(i * T);
}

template <bool kBF16, int R>
void launch_ranks_t(const moe_dims &dm, const float *y, const int32_t *inv, const float *w,
                    const int32_t *idx, const int32_t *map, float scale, const float *ys,
                    void *partials, void *out, hipStream_t s) {
    const int64_t waves = dm.T * ((dm.d + kSlice - 1) / kSlice);
    combine_ranks_kernel<kBF16, R><<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s>>>(
        y, inv, w, idx, map, dm.T, dm.k, dm.d, dm.E, dm.T * dm.k, scale, ys, partials, out);
}

template <bool kBF16>
bool launch_ranks_d(const moe_dims &dm, int R, const float *y, const int32_t *inv,
                    const float *w, const int32_t *idx, const int32_t *map, float scale,
                    const float *ys, void *partials, void *out, hipStream_t s) {
#define MOE_RANKS_CASE(n) \
    case n: launch_ranks_t<kBF16, n>(dm, y, inv, w, idx, map, scale, ys, partials, out, s); return true;
    switch (R) {
        MOE_RANKS_CASE(1) MOE_RANKS_CASE(2) MOE_RANKS_CASE(3) MOE_RANKS_CASE(4)
        MOE_RANKS_CASE(5) MOE_RANKS_CASE(6) MOE_RANKS_CASE(7) MOE_RANKS_CASE(8)
        MOE_RANKS_CASE(9) MOE_RANKS_CASE(10) MOE_RANKS_CASE(11) MOE_RANKS_CASE(12)
        MOE_RANKS_CASE(13) MOE_RANKS_CASE(14) MOE_RANKS_CASE(15) MOE_RANKS_CASE(16)
    }
#undef MOE_RANKS_CASE
    return false;
}

}  // namespace

hipError_t launch_combine_ranks(const moe_dims &dm, int R, const float *y, const int32_t *inv,
                                const float *topk_w, const int32_t *topk_idx,
                                const int32_t *slot_map, float scale, const float *ys,
                                void *partials, void *out, hipStream_t s) {
    if (R < 1 || R > kMaxRanks || dm.E % R) return hipErrorInvalidValue;
    if (dm.T > 0) {
        const bool ok = dm.dtype == MOE_BF16
                            ? launch_ranks_d<true>(dm, R, y, inv, topk_w, topk_idx, slot_map,
                                                   scale, ys, partials, out, s)
                            : launch_ranks_d<false>(dm, R, y, inv, topk_w, topk_idx, slot_map,
                                                    scale, ys, partials, out, s);
        if (!ok) return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

moe_dims shared_dims(const moe_dims &dm, int R, int inter_shared) {
    moe_dims s = dm;
    s.E = R;
    s.k = R;
    s.inter = inter_shared / R;
    return s;
}

size_t shared_workspace_bytes(const moe_dims &dm, int R, int inter_shared) {
    const moe_dims s = shared_dims(dm, R, inter_shared);
    const int64_t A = dm.T * R;
    return carve_workspace(s, nullptr).total + align_up(sizeof(int32_t) * (A + 1), 256) +
           align_up(sizeof(int32_t) * (R + 1), 256);
}

hipError_t launch_shared_ffn(const moe_dims &dm, int R, int inter_shared, const void *x,
                             const void *w13s, const void *w2s, void *h_s, float *y_s,
                             void *workspace, hipStream_t s) {
    if (dm.T == 0) return hipGetLastError();
    const moe_dims sd = shared_dims(dm, R, inter_shared);
    const Workspace ws = carve_workspace(sd, workspace);
    char *base = static_cast<char *>(workspace) + ws.total;
    const int64_t A = dm.T * R;
    int32_t *perm = reinterpret_cast<int32_t *>(base);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + align_up(sizeof(int32_t) * (A + 1), 256));
    const int64_t n = std::max<int64_t>(A, R + 1);
    shared_rows_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(dm.T, R, perm,
                                                                              offsets);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_grouped_ffn(sd, nullptr, offsets, w13s, w2s, h_s, y_s, ws, nullptr, s, x,
                              perm);
}

}  // namespace moe
