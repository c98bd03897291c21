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

// Round a double to bf16, to nearest with ties to even, in one step: the double is first
// rounded toward zero to FP32 with the lowest bit forced to 1 when inexact ("round to
// odd"); FP32 keeps 16 more significand bits than bf16, so the RNE rounding of that odd
// value to bf16 is the RNE rounding of the double (no double-rounding error).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    float t = __double2float_rz(x);
    if ((double)t != x) t = __uint_as_float(__float_as_uint(t) | 1u);
    return f32_to_bf16(t);
}

// Vector loads and stores of V consecutive floats / bf16 values (V = 1, 2, 4).
template <int V>
__device__ __forceinline__ void load_f(const float *p, float (&v)[V]) {
    if constexpr (V == 4) {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else if constexpr (V == 2) {
        const float2 q = *reinterpret_cast<const float2 *>(p);
        v[0] = q.x; v[1] = q.y;
    } else {
        v[0] = *p;
    }
}
template <int V>
__device__ __forceinline__ void store_f(float *p, const float (&v)[V]) {
    if constexpr (V == 4) *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (V == 2) *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    else *p = v[0];
}
template <int V>
__device__ __forceinline__ void store_b(uint16_t *p, const uint16_t (&b)[V]) {
    if constexpr (V == 4) {
        uint2 pk;
        pk.x = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
        pk.y = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
        *reinterpret_cast<uint2 *>(p) = pk;
    } else if constexpr (V == 2) {
        *reinterpret_cast<uint32_t *>(p) = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
    } else {
        *p = b[0];
    }
}

// Features per lane: fewer as R grows, so that the R partials of every feature a lane
// holds, and the FP64 tree over them, stay in registers at a useful occupancy.
template <int R>
constexpr int ranks_vec() { return R <= 8 ? 4 : 2; }

// One wave per (token, slice of 128 V features); lane l takes features slice*128V + V*l
// and slice*128V + 64V + V*l (two chunks). For each chunk: the k weighted expert rows
// (FP32 products), then per rank the slot-order sum with foreign slots as exact zeros,
// the factor, the shared shard and the rounding; then per feature the FP64 tree over the
// R partials, whose shape is fixed by R alone.
template <bool kBF16, int R>
__global__ __launch_bounds__(256) void combine_ranks_kernel(
    const float *__restrict__ y, const int32_t *__restrict__ inv,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ slot_map, int64_t T, int k, int d, int E, int64_t A,
    float scale, const float *__restrict__ ys, void *__restrict__ partials,
    void *__restrict__ out) {
    constexpr int V = ranks_vec<R>();
    constexpr int kSl = 128 * V;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nslice = (d + kSl - 1) / kSl;
    const int64_t W = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = W / nslice;
    if (t >= T) return;
    const int c0 = (int)(W % nslice) * kSl + lane * V;
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
        const int c = c0 + 64 * V * u;
        if (c >= d) break;
        float prod[kMaxK][V];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) load_f<V>(y + src[j] + c, prod[j]);
        float part[R][V];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (ys) load_f<V>(ys + ((int64_t)r * T + t) * d + c, part[r]);
            else
#pragma unroll
                for (int q = 0; q < V; ++q) part[r][q] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k)
#pragma unroll
                for (int q = 0; q < V; ++q) prod[j][q] = w[j] * prod[j][q];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a[V];
#pragma unroll
            for (int q = 0; q < V; ++q) a[q] = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    const bool own = owner[j] == r;
#pragma unroll
                    for (int q = 0; q < V; ++q) a[q] = a[q] + (own ? prod[j][q] : 0.f);
                }
            }
#pragma unroll
            for (int q = 0; q < V; ++q) {
                a[q] = scale * a[q];
                if (ys) a[q] = a[q] + part[r][q];
            }
            if constexpr (kBF16) {
                uint16_t b[V];
#pragma unroll
                for (int q = 0; q < V; ++q) {
                    b[q] = f32_to_bf16(a[q]);
                    part[r][q] = bf16_to_f32(b[q]);
                }
                if (partials)
                    store_b<V>(static_cast<uint16_t *>(partials) + ((int64_t)r * T + t) * d + c, b);
            } else {
#pragma unroll
                for (int q = 0; q < V; ++q) part[r][q] = a[q];
                if (partials)
                    store_f<V>(static_cast<float *>(partials) + ((int64_t)r * T + t) * d + c, a);
            }
        }
        // per feature: adjacent pairs in FP64, the odd last value carried, level by level
        uint16_t ob[V];
        float of[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
            double lv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) lv[r] = part[r][q];
#pragma unroll
            for (int n = R; n > 1; n = (n + 1) / 2) {
#pragma unroll
                for (int i = 0; i < n / 2; ++i) lv[i] = lv[2 * i] + lv[2 * i + 1];
                if (n & 1) lv[n / 2] = lv[n - 1];
            }
            if constexpr (kBF16) ob[q] = f64_to_bf16(lv[0]);
            else of[q] = (float)lv[0];
        }
        if constexpr (kBF16) store_b<V>(static_cast<uint16_t *>(out) + t * d + c, ob);
        else store_f<V>(static_cast<float *>(out) + t * d + c, of);
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
    constexpr int kSl = 128 * ranks_vec<R>();
    const int64_t waves = dm.T * ((dm.d + kSl - 1) / kSl);
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
