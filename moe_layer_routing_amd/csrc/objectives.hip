// objectives.hip -- objective statistics of one routed batch.
//
// "HARTS ...", eq. (20) and "MoE execution and objectives": the multiplicity q_t of a
// compact token weights its router z-loss term, the probability mass and the top-k
// assignment counts of the load-balancing loss, and the counts that update the expert
// routing bias. With S = sum_t q_t semantic positions:
//   z_loss   = (1/S) sum_t q_t lse_t^2,
//   aux_loss = E / (k S^2) sum_e C_e M_e   (= E sum_e (C_e / kS)(M_e / S)),
//   bias[e] += rate * sign(mean_e' C_e' - C_e), the comparison done exactly in integers.
// All of it is a few kilobytes of input, so one block does it: thread i accumulates the
// tokens i, i + 1024, ... in FP64 (z) and int64 (S) in increasing order, then a fixed
// binary tree over the threads; the per-expert products C_e M_e (FP64) and counts go
// through a fixed tree over 256 entries. The order depends only on T and E.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kObjThreads = 1024;

__global__ __launch_bounds__(kObjThreads) void objectives_kernel(
    const float *__restrict__ lse, const int32_t *__restrict__ q, int64_t T,
    const int64_t *__restrict__ wc, const float *__restrict__ mass,
    const int32_t *__restrict__ map, int E, int k, float rate, float *__restrict__ bias,
    double *__restrict__ out, int32_t *__restrict__ d_err) {
    __shared__ double zs[kObjThreads];
    __shared__ long long ss[kObjThreads];
    __shared__ double am[kMaxE];
    __shared__ long long ct[kMaxE];
    const int tid = threadIdx.x;
    double z = 0.0;
    long long S = 0;
#pragma unroll 8
    for (int64_t t = tid; t < T; t += kObjThreads) {
        const long long qt = q ? q[t] : 1;
        S += qt;
        if (lse) {
            const double l = lse[t];
            z = z + (double)qt * (l * l);
        }
    }
    zs[tid] = z;
    ss[tid] = S;
    int err = 0;
    long long c = 0;
    double cm = 0.0;
    if (tid < E && wc) {
        int v = tid;
        if (map) {
            v = map[tid];
            if (v < 0 || v >= E) {
                err |= MOE_DERR_SLOTMAP;
                v = -1;
            }
        }
        c = v >= 0 ? wc[v] : 0;
        if (mass) cm = (double)c * (double)mass[tid];
    }
    if (tid < kMaxE) {
        am[tid] = cm;
        ct[tid] = c;
    }
    __syncthreads();
#pragma unroll
    for (int s = kObjThreads / 2; s >= 1; s >>= 1) {
        if (tid < s) {
            zs[tid] = zs[tid] + zs[tid + s];
            ss[tid] += ss[tid + s];
            if (s < kMaxE) {
                am[tid] = am[tid] + am[tid + s];
                ct[tid] += ct[tid + s];
            }
        }
        __syncthreads();
    }
    const long long Stot = ss[0], Ctot = ct[0];
    if (tid == 0) {
        out[0] = (lse && Stot > 0) ? zs[0] / (double)Stot : 0.0;
        out[1] = (wc && mass && Stot > 0)
                     ? am[0] * (double)E / ((double)k * (double)Stot * (double)Stot)
                     : 0.0;
        out[2] = (double)Stot;
    }
    if (bias && wc && tid < E) {
        const long long ec = (long long)E * c;
        if (ec < Ctot) bias[tid] = bias[tid] + rate;
        else if (ec > Ctot) bias[tid] = bias[tid] + (-rate);
    }
    raise_err(d_err, err);
}

}  // namespace

hipError_t launch_objectives(const moe_dims &dm, const float *lse, const int32_t *q,
                             const int64_t *wcounts, const float *mass,
                             const int32_t *slot_map, float rate, float *bias, double *out,
                             int32_t *d_err, hipStream_t s) {
    static_assert(kObjThreads >= kMaxE && kMaxE == 256, "tree shapes");
    objectives_kernel<<<dim3(1), dim3(kObjThreads), 0, s>>>(lse, q, dm.T, wcounts, mass,
                                                            slot_map, dm.E, dm.k, rate, bias,
                                                            out, d_err);
    return hipGetLastError();
}

}  // namespace moe
