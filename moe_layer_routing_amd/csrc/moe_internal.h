// moe_internal.h -- device helpers and the host-side launchers each kernel file
// exports to the C-ABI layer (moe_api.hip). Internal to the HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxE = 256;         // experts per layer supported by the LDS-resident paths
constexpr int kMaxK = 8;           // experts per token
constexpr int kPermChunk = 2048;   // flat assignments per permute block (fixed, T-free)
constexpr int kTopkTokPerBlock = 16;  // 4 waves x 4 tokens
constexpr int kSmallT = 64;           // largest batch the single-block routing tail takes
constexpr int kMaxRanks = 16;         // ranks of the emulated expert-parallel output
constexpr int kRouterWgradSplit = 8;  // row segments of the router weight gradient

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte store with the nontemporal hint (global_store ... nt): for large outputs that no
// later kernel of the step finds in cache anyway; the CU issues them markedly faster.
__device__ __forceinline__ void store_nt(float *p, float4 v) {
    __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t *>(p));
}
// 16-byte load with the nontemporal hint, for rows read once (the combine's gathered y rows)
__device__ __forceinline__ float4 load_nt(const float *p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Block barrier for hand-overs through LDS only: each wave waits for its own LDS
// operations, then s_barrier. __syncthreads also waits for the wave's outstanding global
// stores (about a microsecond of write latency); a block whose later steps never read back
// what it stored to memory does not need that.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with vmcnt(N), lgkmcnt(0), expcnt untouched (gfx9 immediate encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Row-major (K-major) LDS tiles read with ds_read_b64_tr_b16: the 16 rows one transposing
// read touches (8g + 0..3, g = 0..3) get distinct 32-byte bank groups within each
// half-wave when 16-byte chunk c of row r is stored at c ^ kmajor_swz(r) (XOR 2 * (bits
// 0-1 and 3 of the row), limited to the row's CPR chunks).
template <int CPR>
__device__ __forceinline__ int kmajor_swz(int r) {
    return (2 * ((r & 3) | (((r >> 3) & 1) << 2))) & (CPR - 1);
}

// Transposing LDS reads issued from inline assembly. The compiler, not knowing which LDS
// bytes the ds_read_b64_tr_b16 intrinsic reads, waits for every outstanding global->LDS
// DMA (vmcnt(0)) before it, which would stall a DMA ring on its newest stage; these reads
// carry no such wait. The caller issues a batch of them, then tr_fence() (lgkmcnt(0)) and
// tr_take() on every result before use, which ties the results to the fence.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ i32x2_t tr_read(const uint8_t *p) {
    i32x2_t v;
    const uint32_t a = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const uint8_t *)(p));
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
__device__ __forceinline__ void tr_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ bf16x8_t tr_take(i32x2_t &lo, i32x2_t &hi) {
    asm volatile("" : "+v"(lo), "+v"(hi));
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    const i32x4_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
    return __builtin_bit_cast(bf16x8_t, v);
}

// bfloat16 widening (exact) and narrowing (round to nearest, ties to even; NaN kept quiet).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// SwiGLU derivative of one element, h = silu(g) u: dg = (d u) silu'(g), du = d silu(g),
// with silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + exp(-g)). One definition serves the
// elementwise backward kernel and the fused gate/up recomputation, so both give the same bits.
__device__ __forceinline__ void swiglu_grad(float g, float u, float d, float &dg, float &du) {
    const float e = expf(-g);
    const float sg = 1.0f / (1.0f + e);
    const float silu = g / (1.0f + e);
    const float dsilu = sg * (1.0f + g * (1.0f - sg));
    dg = (d * u) * dsilu;
    du = d * silu;
}

// four consecutive features of d_gu's gate part at o and of its up part at o + I
template <bool kBF16>
__device__ __forceinline__ void store_dgu4(void *dgu, int64_t o, int I, const float (&dg)[4],
                                           const float (&du)[4]) {
    if constexpr (kBF16) {
        uint16_t *q = static_cast<uint16_t *>(dgu) + o;
        uint2 pg, pu;
        pg.x = (uint32_t)f32_to_bf16(dg[0]) | ((uint32_t)f32_to_bf16(dg[1]) << 16);
        pg.y = (uint32_t)f32_to_bf16(dg[2]) | ((uint32_t)f32_to_bf16(dg[3]) << 16);
        pu.x = (uint32_t)f32_to_bf16(du[0]) | ((uint32_t)f32_to_bf16(du[1]) << 16);
        pu.y = (uint32_t)f32_to_bf16(du[2]) | ((uint32_t)f32_to_bf16(du[3]) << 16);
        *reinterpret_cast<uint2 *>(q) = pg;
        *reinterpret_cast<uint2 *>(q + I) = pu;
    } else {
        float *q = static_cast<float *>(dgu) + o;
        *reinterpret_cast<float4 *>(q) = make_float4(dg[0], dg[1], dg[2], dg[3]);
        *reinterpret_cast<float4 *>(q + I) = make_float4(du[0], du[1], du[2], du[3]);
    }
}

// Error word update: one atomic OR, taken only when a check failed.
__device__ __forceinline__ void raise_err(int32_t *d_err, int32_t bits) {
    if (d_err && bits) atomicOr(d_err, bits);
}

// prob_mass[e] from the per-block partials, by one wave: the sum of 256 virtual threads
// (virtual thread i adds the partials of blocks i, i+256, ... in order) followed by a fixed
// binary tree over them (step s: i += i + s for i < s, s = 128 .. 1). Lane l holds
// virtual threads l, l+64, l+128, l+192; the steps 128 and 64 stay inside the lane and the
// rest pair lane l with lane l + s. The order depends only on the number of partials (i.e.
// on T).
__device__ __forceinline__ void mass_reduce_wave(const float *__restrict__ part, int64_t nblk,
                                                 int E, int e, float *__restrict__ mass) {
    const int lane = threadIdx.x & 63;
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float acc = 0.f;
        for (int64_t b = lane + 64 * u; b < nblk; b += 256) acc = acc + part[b * E + e];
        v[u] = acc;
    }
    v[0] = v[0] + v[2];   // s = 128
    v[1] = v[1] + v[3];
    float x = v[0] + v[1];   // s = 64
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = x + __shfl_down(x, s, 64);
    if (lane == 0) mass[e] = x;
}

// Physical slot of routed expert id e under a placement map (identity when map is null):
// -1 for an id outside [0, E) (*bits gets MOE_DERR_IDX_RANGE) or a map entry outside [0, E)
// (*bits gets MOE_DERR_SLOTMAP).
__device__ __forceinline__ int slot_of(const int32_t *map, int e, int E, int &bits) {
    if (e < 0 || e >= E) {
        bits |= MOE_DERR_IDX_RANGE;
        return -1;
    }
    if (!map) return e;
    const int v = map[e];
    if (v < 0 || v >= E) {
        bits |= MOE_DERR_SLOTMAP;
        return -1;
    }
    return v;
}

// Lanes of the wave whose 9-bit key equals this lane's, found with one ballot per key bit.
__device__ __forceinline__ uint64_t wave_match9(uint32_t key) {
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
        const bool b = (key >> bit) & 1u;
        const uint64_t m = __ballot(b);
        peers &= b ? m : ~m;
    }
    return peers;
}

// Inclusive prefix sum over the 64 lanes (integers: exact in any order).
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace carving
// Every entry point uses the same layout so that moe_forward can run all steps in one
// workspace. Offsets are 256-byte aligned.
struct Workspace {
    float *logits;            // [T,E]   router logits when the caller passes none
    float *mass_part;         // [ceil(T/64), E] per-block probability mass
    int32_t *blk_hist;        // [nchunks, E] per-chunk expert histogram -> chunk offsets
    uint64_t *blk_whist;      // [nchunks, E] per-chunk multiplicity-weighted histogram
    int32_t *tiles;           // [1 + 3*max_tiles] grouped-GEMM tile list
    float *logit_part;        // [16, T, E] router-logit chain partials, T * E <= 2048 only
    size_t total;
};

int64_t perm_chunks(int64_t A);
// Most token tiles any routing of A rows over E experts can produce at tile height tile_m.
int64_t max_m_tiles(int64_t A, int E, int tile_m);
Workspace carve_workspace(const moe_dims &d, void *base);

// ---------------------------------------------------------------- router variants
enum { kScoreSoftmax = MOE_SCORE_SOFTMAX, kScoreSigmoid = MOE_SCORE_SIGMOID,
       kScoreSqrtSoftplus = MOE_SCORE_SQRT_SOFTPLUS };

// Router variant inputs as the kernels take them (validated by the API layer).
struct RouteOpts {
    int fn = kScoreSoftmax;
    const float *corr_bias = nullptr;   // [E], scored routers only
    const int32_t *hash_table = nullptr;  // [vocab, k]
    const int32_t *token_ids = nullptr;   // [T]
    int vocab = 0;
    float *lse = nullptr;                 // [T] output
    bool plain() const { return fn == kScoreSoftmax && !hash_table; }
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error. Sizes are already validated.
hipError_t launch_route(const moe_dims &dm, const void *x, const void *w_router,
                        const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                        float *mass_part, float *prob_mass, const int32_t *token_mult,
                        int32_t *d_err, hipStream_t s, const RouteOpts &opts = RouteOpts(),
                        bool defer_mass = false);   // true: prob_mass is left to launch_permute
hipError_t launch_replay(const moe_dims &dm, const int32_t *idx_in, const float *w_in,
                         int32_t *topk_idx, float *topk_w, int32_t *d_err, hipStream_t s);
hipError_t launch_permute(const moe_dims &dm, const int32_t *topk_idx, const void *x,
                          void *x_perm, int32_t *perm, int32_t *inv, int32_t *counts,
                          int32_t *offsets, const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t *seq_counts, const int32_t *token_mult,
                          int64_t *weighted_counts, int32_t *d_err, const Workspace &ws,
                          hipStream_t s, const int32_t *slot_map = nullptr,
                          int tiles_bt = 0,    // > 0: also write ws.tiles for this tile height
                          const float *mass_part = nullptr, int64_t mass_nblk = 0,
                          float *prob_mass = nullptr);   // the mass launch_route deferred
// Raises MOE_DERR_SLOTMAP unless map[0..E-1] is a permutation of 0..E-1 (one block).
hipError_t launch_check_slot_map(const int32_t *map, int E, int32_t *d_err, hipStream_t s);
// x_perm == nullptr: gather token rows of x through perm inside the gate/up GEMM.
hipError_t launch_grouped_ffn(const moe_dims &dm, const void *x_perm, const int32_t *offsets,
                              const void *w13, const void *w2, void *h, float *y,
                              const Workspace &ws, void *const *prof_events, hipStream_t s,
                              const void *x = nullptr, const int32_t *perm = nullptr,
                              bool tiles_ready = false, float *gu_out = nullptr,
                              bool gate_up_only = false);
// Decode-sized bf16 layers (T*k <= 16, 16-row tiles, d/16 >= 256 blocks, inter % 768 == 0):
// the down GEMM and the plain weighted combine in one launch (y is still written); records
// prof_events[2] after it.
bool down_combine_small_ok(const moe_dims &dm);
hipError_t launch_down_combine_small(const moe_dims &dm, const void *h, const void *w2, float *y,
                                     const int32_t *tiles, const int32_t *inv,
                                     const float *topk_w, float scale, void *out,
                                     void *const *prof_events, hipStream_t s);
// Decode steps of one or two tokens, bf16, plain softmax router (T <= 2, T k <= 16,
// E <= 128, 16-row tiles): the gate/up launch (gathered from x, records prof_events[0] and
// [1] around it) forms the logits from the logit-chain partials and routes the tokens in
// every block, with the routing tail's arithmetic; its last block writes every output
// launch_small_tail writes for such a batch without a placement map (pointers as there;
// prob_mass, weighted_counts, lse and q may be null). The tile list it writes serves the
// down GEMM launch after it.
struct DecodeRoute {
    const float *part;   // [kLogitChains][E] chain partials
    const float *bias;   // [E] or null
    const int32_t *q;    // [1] token multiplicity or null
    float *logits, *topk_w, *prob_mass, *lse;
    int32_t *topk_idx, *counts, *offsets, *perm, *inv, *tiles, *d_err;
    int64_t *weighted_counts;
};
bool decode_self_route_ok(const moe_dims &dm);
hipError_t launch_decode_self_route(const moe_dims &dm, const DecodeRoute &r, const void *x,
                                    const void *w13, void *h, float *gu_out,
                                    void *const *prof_events, hipStream_t s);
hipError_t launch_combine(const moe_dims &dm, const float *y, const int32_t *inv,
                          const float *topk_w, void *out, hipStream_t s, float scale = 1.0f);
// Rank partial outputs and their FP64 pairwise tree (1 <= R <= kMaxRanks, R divides E).
hipError_t launch_combine_ranks(const moe_dims &dm, int R, const float *y, const int32_t *inv,
                                const float *topk_w, const int32_t *topk_idx,
                                const int32_t *slot_map, float scale, const float *ys,
                                void *partials, void *out, hipStream_t s);
// The shared expert sharded over R ranks: the grouped problem it runs as, its workspace,
// and the launch (rows gathered from x, so x must be under 4 GiB).
moe_dims shared_dims(const moe_dims &dm, int R, int inter_shared);
size_t shared_workspace_bytes(const moe_dims &dm, int R, int inter_shared);
hipError_t launch_shared_ffn(const moe_dims &dm, int R, int inter_shared, const void *x,
                             const void *w13s, const void *w2s, void *h_s, float *y_s,
                             void *workspace, hipStream_t s);
// Grouped-GEMM helpers shared with the backward: the token-tile list for tile height bt,
// and the plain FP32-output GEMM (the forward's down launch) with N features over K = d;
// kmajor (bf16 only): the weights are stored wgt[e][k][n] instead of wgt[e][n][k].
hipError_t launch_build_tiles(const int32_t *offsets, int E, int64_t A, int bt, int64_t cap,
                              int32_t *tiles, hipStream_t s);
hipError_t launch_gate_up_grad(const moe_dims &dm, const void *act, const int32_t *gperm,
                               const void *w13, const float *dh, void *dgu, bool dgu_bf16,
                               const int32_t *offsets, const Workspace &ws, hipStream_t s);
hipError_t launch_plain_gemm(const moe_dims &dm, const void *act, const int32_t *gperm,
                             const void *wgt, float *out, int N, const int32_t *offsets,
                             const Workspace &ws, hipStream_t s, int K = 0,
                             bool kmajor = false);
// Backward steps (backward.hip).
hipError_t launch_combine_bwd(const moe_dims &dm, const void *dout, const float *y,
                              const int32_t *inv, const float *topk_w, float scale, void *dy,
                              float *dw, bool dy_bf16, hipStream_t s);
hipError_t launch_swiglu_bwd(const moe_dims &dm, const float *gu, const float *dh, void *dgu,
                             bool out_bf16, hipStream_t s);
hipError_t launch_wgrad_bf16(int nseg, const void *a, const void *b, const int32_t *bperm,
                             int bk, int64_t bT, const int32_t *off, int64_t nrows, int N,
                             int C, float *out, hipStream_t s);
hipError_t launch_dx_sum(const moe_dims &dm, const float *dxp, const int32_t *inv,
                         const float *dxr, float *dx, hipStream_t s);
hipError_t launch_router_bwd(const moe_dims &dm, const float *logits, const float *dw,
                             float *dl, hipStream_t s);
hipError_t launch_dgrad(const moe_dims &dm, const float *act, const void *wgt, bool wbf16,
                        int K, int N, const int32_t *offsets, float *out, const Workspace &ws,
                        hipStream_t s);
hipError_t launch_wgrad(int nseg, const float *a, const void *b, bool bbf16,
                        const int32_t *bperm, int bk, int64_t bT, const int32_t *off,
                        int64_t nrows, int N, int C, float *out, hipStream_t s);
// scratch: scratch_floats floats the call may overwrite (NULL: no row split)
hipError_t launch_router_wgrad(const moe_dims &dm, const float *dl, const void *x, float *dwr,
                               float *scratch, int64_t scratch_floats, hipStream_t s);
hipError_t launch_router_dx(const moe_dims &dm, const float *dl, const void *w_router,
                            float *dx, hipStream_t s);
// Objective statistics (one block): out[3] = z_loss, aux_loss, S; optional bias update.
hipError_t launch_objectives(const moe_dims &dm, const float *lse, const int32_t *q,
                             const int64_t *wcounts, const float *mass,
                             const int32_t *slot_map, float rate, float *bias, double *out,
                             int32_t *d_err, hipStream_t s);

int select_tile_m(const moe_dims &dm);

// Router logits only (the first step of launch_route).
hipError_t launch_router_logits(const moe_dims &dm, const void *x, const void *w_router,
                                const float *bias, float *logits, hipStream_t s);
// The router logits' kLogitChains K-chains as separate waves: part[c][t][e] (chain c's
// partial, the same bits as inside launch_router_logits); launch_small_tail adds them.
constexpr int kLogitChains = 16;
constexpr int64_t kChainSumMax = 2048;    // T * E up to which the small-batch path uses them
hipError_t launch_router_logit_chains(const moe_dims &dm, const void *x, const void *w_router,
                                      float *part, hipStream_t s);
// Token-major row gather x -> x_perm through inv (part of launch_permute).
hipError_t launch_gather(const moe_dims &dm, const void *x, const int32_t *inv, void *x_perm,
                         hipStream_t s);
// Routing tail of a small batch (1 <= T <= kSmallT) in one block: top-k from logits (or,
// with idx_in, replay validation), probability mass, counts, offsets, weighted counts,
// perm / inv, and the token-tile list for tile height select_tile_m(dm). Every output is
// bitwise the one the multi-kernel steps produce for the same T. With logit_part (router
// mode), the block first forms logits[t][e] = (part[0] + ... + part[15]) + bias[e] in chain
// order, as launch_router_logits does, and writes them to logits.
hipError_t launch_small_tail(const moe_dims &dm, const float *logits, const int32_t *q,
                             const int32_t *idx_in, const float *w_in, int32_t *topk_idx,
                             float *topk_w, float *prob_mass, int32_t *counts,
                             int32_t *offsets, int32_t *perm, int32_t *inv,
                             int64_t *weighted_counts, int32_t *tiles, int32_t *d_err,
                             hipStream_t s, const int32_t *slot_map = nullptr,
                             const RouteOpts &opts = RouteOpts(),
                             const float *logit_part = nullptr, const float *bias = nullptr);

}  // namespace moe
