// combine.hip -- weighted combine of the k expert outputs of every token.
//
// "0 train-infer mismatch for Open-weight MoE RL in Open-source code", "Sharding the
// experts" and "The experts: keeping the route weight inside the accumulator": each
// token's routing slots are accumulated in FP32 in slot order, the route weight applied
// inside that FP32 accumulator, and the sum rounded once to the output type. Here
// acc = ((0 + w_0*y_0) + w_1*y_1) + ... with every product and sum a separate FP32
// operation (the library is built without floating-point contraction). A routed scaling
// factor ("Choosing GLM's eight experts": the expert kernel applies the factor to the
// FP32-weighted result) multiplies acc once, in FP32, before the rounding; the factor 1
// leaves every bit unchanged.
#include "moe_internal.h"

namespace moe {
namespace {

// One wave per (token, 512-feature slice); lane l handles features s*512 + 4*l and
// s*512 + 256 + 4*l. Slicing only spreads the rows over more waves (every output feature
// is the same slot-order sum whichever wave computes it), so decode-sized batches still
// fill the chip.
constexpr int kSlice = 512;

template <bool kBF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const int32_t *__restrict__ inv,
                                                      const float *__restrict__ topk_w,
                                                      int64_t T, int k, int d, int64_t A,
                                                      float scale, void *__restrict__ out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nslice = (d + kSlice - 1) / kSlice;
    const int64_t W = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = W / nslice;
    if (t >= T) return;
    const int c0 = (int)(W % nslice) * kSlice + lane * 4;
    int64_t src[kMaxK];
    float w[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        int32_t p = (j < k) ? inv[t * k + j] : 0;
        p = (p < 0 || p >= A) ? 0 : p;   // invalid ids were reported by the permute step
        src[j] = (int64_t)p * d;
        w[j] = (j < k) ? topk_w[t * k + j] : 0.f;
    }
    // two 256-feature chunks: 2k 16-byte loads in flight per lane
    {
        float4 v[2][kMaxK];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = min(c0 + 256 * u, d - 4);
#pragma unroll
            for (int j = 0; j < kMaxK; ++j)
                if (j < k) v[u][j] = load_nt(y + src[j] + c);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = c0 + 256 * u;
            if (c >= d) break;
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    a0 = a0 + w[j] * v[u][j].x;
                    a1 = a1 + w[j] * v[u][j].y;
                    a2 = a2 + w[j] * v[u][j].z;
                    a3 = a3 + w[j] * v[u][j].w;
                }
            }
            a0 = scale * a0;
            a1 = scale * a1;
            a2 = scale * a2;
            a3 = scale * a3;
            if constexpr (kBF16) {
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16);
                pk.y = (uint32_t)f32_to_bf16(a2) | ((uint32_t)f32_to_bf16(a3) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + t * d + c) = pk;
            } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(out) + t * d + c) =
                    make_float4(a0, a1, a2, a3);
            }
        }
    }
}

}  // namespace

hipError_t launch_combine(const moe_dims &dm, const float *y, const int32_t *inv,
                          const float *topk_w, void *out, hipStream_t s, float scale) {
    if (dm.T > 0) {
        const int64_t waves = dm.T * ((dm.d + kSlice - 1) / kSlice);
        const dim3 grid((unsigned)((waves + 3) / 4));
        const int64_t A = dm.T * dm.k;
        if (dm.dtype == MOE_BF16)
            combine_kernel<true><<<grid, dim3(256), 0, s>>>(y, inv, topk_w, dm.T, dm.k, dm.d,
                                                            A, scale, out);
        else
            combine_kernel<false><<<grid, dim3(256), 0, s>>>(y, inv, topk_w, dm.T, dm.k, dm.d,
                                                             A, scale, out);
    }
    return hipGetLastError();
}

}  // namespace moe
