// permute.hip -- expert histogram, exclusive offsets, stable scatter into
// expert-contiguous order, row gather, and load statistics.
//
// The counts are the planners' routing-replay demand ("RoutePack ...", Sec. 2.1 eq. (1),
// Sec. 3.3: per-sample and aggregate assignment counts per expert) and the
// multiplicity-weighted assignment counts of "HARTS ..." (eq. (20), "MoE execution and
// objectives"). No assignment is dropped: every (token, slot) lands in exactly one row
// of its expert's segment, in increasing flat order a = t*k + j.
//
// Determinism without order-defined atomics: the flat assignments are cut into fixed
// chunks of kPermChunk; each chunk's histogram is an integer count (any order gives the
// same value); one block scans those counts in chunk order; each chunk then ranks its own
// assignments stably with wave ballots. Positions therefore depend only on the ids.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kSubChunk = kPermChunk / 4;  // per wave

// Also (when given): zeroes seq_counts (nzero entries, over the grid) for the scatter
// kernel's per-sequence histogram, and forms prob_mass from the router's per-block
// partials (wave w of block b reduces expert 4b + w, then every 4 * grid further).
__global__ __launch_bounds__(256) void hist_kernel(const int32_t *__restrict__ idx, int64_t A,
                                                   int k, int E,
                                                   const int32_t *__restrict__ q,
                                                   int32_t *__restrict__ blk_hist,
                                                   uint64_t *__restrict__ blk_whist,
                                                   int32_t *__restrict__ d_err,
                                                   const int32_t *__restrict__ slot,
                                                   int32_t *__restrict__ zero, int64_t nzero,
                                                   const float *__restrict__ mass_part,
                                                   int64_t mass_nblk,
                                                   float *__restrict__ prob_mass) {
    __shared__ int32_t hist[kMaxE];
    __shared__ unsigned long long whist[kMaxE];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nzero;
         i += (int64_t)gridDim.x * 256)
        zero[i] = 0;
    for (int e = threadIdx.x; e < E; e += 256) {
        hist[e] = 0;
        whist[e] = 0;
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kPermChunk;
    int err = 0;
    for (int i = threadIdx.x; i < kPermChunk; i += 256) {
        const int64_t a = base + i;
        if (a >= A) break;
        const int e = slot_of(slot, idx[a], E, err);
        if (e < 0) continue;
        atomicAdd(&hist[e], 1);
        if (blk_whist && q) atomicAdd(&whist[e], (unsigned long long)(uint32_t)q[a / k]);
    }
    raise_err(d_err, err);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        blk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
        if (blk_whist) blk_whist[(int64_t)blockIdx.x * E + e] = whist[e];
    }
    if (prob_mass)   // one wave per expert
        for (int e = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); e < E; e += gridDim.x * 4)
            mass_reduce_wave(mass_part, mass_nblk, E, e, prob_mass);
}

// One block: counts, offsets, and each chunk's starting position per expert; with tiles,
// also the grouped GEMM's token-tile list for tile height bt (ceil(count / bt) tiles per
// expert in expert order, at most cap; tiles[0] = their number), as build_tiles_kernel
// forms it from the offsets.
__global__ __launch_bounds__(256) void scan_kernel(int32_t *__restrict__ blk_hist,
                                                   const uint64_t *__restrict__ blk_whist,
                                                   int64_t nchunks, int E, bool have_q,
                                                   int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ offsets,
                                                   int64_t *__restrict__ weighted_counts,
                                                   int bt, int64_t cap,
                                                   int32_t *__restrict__ tiles) {
    static_assert(kMaxE == 256, "one thread per expert, 256 threads");
    __shared__ int32_t cnt[kMaxE + 1];
    __shared__ int32_t tpre[kMaxE + 1];
    const int e = threadIdx.x;
    int32_t run = 0;
    // chunk counts are read kScanBatch at a time, all loads before the stores of the batch,
    // so the chain costs nchunks / kScanBatch memory round trips instead of nchunks
    constexpr int kScanBatch = 16;
    if (e < E) {
        uint64_t wsum = 0;
        for (int64_t b0 = 0; b0 < nchunks; b0 += kScanBatch) {
            int32_t c[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                c[j] = (b0 + j < nchunks) ? blk_hist[(b0 + j) * E + e] : 0;
            if (have_q && weighted_counts) {
#pragma unroll
                for (int j = 0; j < kScanBatch; ++j)
                    wsum += (b0 + j < nchunks) ? blk_whist[(b0 + j) * E + e] : 0;
            }
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                if (b0 + j < nchunks) {
                    blk_hist[(b0 + j) * E + e] = run;
                    run += c[j];
                }
            }
        }
        counts[e] = run;
        if (weighted_counts) weighted_counts[e] = have_q ? (int64_t)wsum : (int64_t)run;
    }
    // exclusive prefix sums over the experts of the counts and of the tile counts: a
    // Hillis-Steele scan over the 256 threads (E <= 256; experts past E count 0, so entry E
    // of the exclusive sum is the total)
    const int32_t c_e = (e < E) ? run : 0;
    const int32_t nt_e = (e < E) ? (c_e + bt - 1) / bt : 0;
    int32_t xs = c_e, ys = nt_e;
    for (int sh = 1; sh < 256; sh <<= 1) {
        __syncthreads();
        cnt[e] = xs;
        tpre[e] = ys;
        __syncthreads();
        if (e >= sh) {
            xs += cnt[e - sh];
            ys += tpre[e - sh];
        }
    }
    __syncthreads();
    cnt[e] = xs - c_e;
    tpre[e] = ys - nt_e;
    if (e == 255) {
        cnt[256] = xs;
        if (tiles) tiles[0] = (int32_t)min<int64_t>(ys, cap);
    }
    __syncthreads();
    if (e < E) {
        const int32_t off = cnt[e];
        offsets[e] = off;
        for (int64_t b0 = 0; b0 < nchunks; b0 += kScanBatch) {
            int32_t c[kScanBatch];
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                c[j] = (b0 + j < nchunks) ? blk_hist[(b0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                if (b0 + j < nchunks) blk_hist[(b0 + j) * E + e] = c[j] + off;
        }
        if (tiles) {
            const int32_t c = cnt[e + 1] - off, nt = (c + bt - 1) / bt;
            for (int i = 0; i < nt; ++i) {
                const int64_t slot = (int64_t)tpre[e] + i;
                if (slot >= cap) break;
                int32_t *d = tiles + 1 + 3 * slot;
                d[0] = e;
                d[1] = off + i * bt;
                d[2] = min(bt, c - i * bt);
            }
        }
    }
    if (e == 0) offsets[E] = cnt[E];
}

// Stable ranks inside a chunk. Wave w owns the sub-chunk [w*512, (w+1)*512) of the chunk;
// a first pass counts each wave's experts, a second pass walks 64 assignments at a time
// and places each one after the earlier lanes that hold the same expert (found with
// ballots over the bits of the id).
// With seq_counts: also the per-sequence counts of the chunk's assignments (for each
// sequence s overlapping it, an LDS histogram of its assignments cu[s]*k .. cu[s+1]*k in
// the chunk, whose non-zero bins are added to seq_counts[s] with integer atomics: any
// order, the same sums; seq_counts was zeroed by the histogram kernel).
__device__ __forceinline__ void seq_hist_chunk(const int32_t *__restrict__ idx, int64_t a_lo,
                                               int64_t a_hi, int k, int E,
                                               const int32_t *__restrict__ cu, int S,
                                               int32_t *__restrict__ seq_counts,
                                               const int32_t *__restrict__ slot,
                                               int32_t *hist) {
    // first sequence whose assignments end past a_lo (empty sequences are skipped)
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid + 1] * k <= a_lo) lo = mid + 1;
        else hi = mid;
    }
    for (int s = lo; s < S && (int64_t)cu[s] * k < a_hi; ++s) {
        const int64_t a0 = max<int64_t>(a_lo, (int64_t)cu[s] * k);
        const int64_t a1 = min<int64_t>(a_hi, (int64_t)cu[s + 1] * k);
        if (a1 <= a0) continue;
        for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
        __syncthreads();
        for (int64_t a = a0 + threadIdx.x; a < a1; a += 256) {
            int bits = 0;
            const int e = slot_of(slot, idx[a], E, bits);
            if (e >= 0) atomicAdd(&hist[e], 1);
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += 256)
            if (hist[e]) atomicAdd(&seq_counts[(int64_t)s * E + e], hist[e]);
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t *__restrict__ idx,
                                                      int64_t A, int E,
                                                      const int32_t *__restrict__ blk_off,
                                                      int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ inv,
                                                      const int32_t *__restrict__ slot,
                                                      int k, const int32_t *__restrict__ cu,
                                                      int S, int32_t *__restrict__ seq_counts,
                                                      int32_t *__restrict__ d_err) {
    __shared__ int32_t cur[4][kMaxE];
    __shared__ int32_t shist[kMaxE];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 4 * kMaxE; i += 256) (&cur[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kPermChunk + wave * kSubChunk;
    for (int it = 0; it < kSubChunk / kWave; ++it) {
        const int64_t a = base + it * kWave + lane;
        int bits = 0;
        const int e = a < A ? slot_of(slot, idx[a], E, bits) : -1;
        if (e >= 0) atomicAdd(&cur[wave][e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        int32_t run = blk_off[(int64_t)blockIdx.x * E + e];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int32_t c = cur[w][e];
            cur[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int it = 0; it < kSubChunk / kWave; ++it) {
        const int64_t a = base + it * kWave + lane;
        int bits = 0;
        const int e0 = a < A ? slot_of(slot, idx[a], E, bits) : -1;
        const bool valid = e0 >= 0;
        const uint32_t key = valid ? (uint32_t)e0 : 0x1ffu;  // 9 bits; invalid never matches
        const uint64_t peers = wave_match9(key);
        if (valid) {
            const int32_t before = __popcll(peers & lt_mask);
            const int32_t pos = cur[wave][e0] + before;
            perm[pos] = (int32_t)a;
            inv[a] = pos;
        } else if (a < A) {
            inv[a] = -1;
        }
        // the highest lane of each group advances that expert's cursor; the next
        // iteration's reads come after this write in the wave's LDS order
        const bool leader = valid && ((peers >> lane) == 1ull);
        __builtin_amdgcn_wave_barrier();
        if (leader) cur[wave][e0] += __popcll(peers);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (seq_counts) {
        // validate cu_seqlens: 0 = c_0 <= c_1 <= ... <= c_S = T
        const int64_t T = A / k;
        int bad = 0;
        for (int s = threadIdx.x; s < S; s += 256)
            if (cu[s + 1] < cu[s]) bad = 1;
        if (threadIdx.x == 0 && (cu[0] != 0 || (int64_t)cu[S] != T)) bad = 1;
        if (__syncthreads_or(bad)) {
            if (blockIdx.x == 0 && threadIdx.x == 0) raise_err(d_err, MOE_DERR_SEQLENS);
            return;
        }
        const int64_t a_lo = (int64_t)blockIdx.x * kPermChunk;
        seq_hist_chunk(idx, a_lo, min<int64_t>(a_lo + kPermChunk, A), k, E, cu, S, seq_counts,
                       slot, shist);
    }
}

// Token-major gather: each wave reads one token's row once and writes it to its k rows.
template <int kElemBytes>
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t *__restrict__ x, int64_t T,
                                                     int k, int64_t row_bytes,
                                                     const int32_t *__restrict__ inv,
                                                     int64_t A,
                                                     uint8_t *__restrict__ x_perm) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    int32_t dst[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) dst[j] = (j < k) ? inv[t * k + j] : -1;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + t * row_bytes);
    const int64_t nvec = row_bytes >> 4;
    for (int64_t v = lane; v < nvec; v += kWave) {
        const uint4 val = src[v];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            const int32_t p = dst[j];
            if (j < k && p >= 0 && p < A)
                reinterpret_cast<uint4 *>(x_perm + (int64_t)p * row_bytes)[v] = val;
        }
    }
}

__global__ void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256)
        p[i] = v;
}

// MOE_DERR_SLOTMAP unless map is a permutation of 0..E-1 (E <= kMaxE).
__global__ __launch_bounds__(256) void check_slot_map_kernel(const int32_t *__restrict__ map,
                                                             int E, int32_t *__restrict__ d_err) {
    __shared__ int32_t seen[kMaxE];
    for (int v = threadIdx.x; v < E; v += 256) seen[v] = 0;
    __syncthreads();
    int bad = 0;
    for (int e = threadIdx.x; e < E; e += 256) {
        const int v = map[e];
        if (v < 0 || v >= E) bad = 1;
        else atomicAdd(&seen[v], 1);
    }
    __syncthreads();
    for (int v = threadIdx.x; v < E; v += 256)
        if (seen[v] != 1) bad = 1;
    if (bad) raise_err(d_err, MOE_DERR_SLOTMAP);
}

}  // namespace

hipError_t launch_check_slot_map(const int32_t *map, int E, int32_t *d_err, hipStream_t s) {
    check_slot_map_kernel<<<dim3(1), dim3(256), 0, s>>>(map, E, d_err);
    return hipGetLastError();
}

hipError_t launch_gather(const moe_dims &dm, const void *x, const int32_t *inv, void *x_perm,
                         hipStream_t s) {
    if (dm.T > 0) {
        const int64_t row_bytes = (int64_t)dm.d * (dm.dtype == MOE_BF16 ? 2 : 4);
        gather_kernel<16><<<dim3((unsigned)((dm.T + 3) / 4)), dim3(256), 0, s>>>(
            static_cast<const uint8_t *>(x), dm.T, dm.k, row_bytes, inv, dm.T * dm.k,
            static_cast<uint8_t *>(x_perm));
    }
    return hipGetLastError();
}

hipError_t launch_permute(const moe_dims &dm, const int32_t *topk_idx, const void *x,
                          void *x_perm, int32_t *perm, int32_t *inv, int32_t *counts,
                          int32_t *offsets, const int32_t *cu_seqlens, int32_t num_seqs,
                          int32_t *seq_counts, const int32_t *token_mult,
                          int64_t *weighted_counts, int32_t *d_err, const Workspace &ws,
                          hipStream_t s, const int32_t *slot_map, int tiles_bt,
                          const float *mass_part, int64_t mass_nblk, float *prob_mass) {
    const int64_t T = dm.T, A = dm.T * dm.k;
    const int E = dm.E, k = dm.k;
    const int64_t nchunks = perm_chunks(A);
    const bool have_q = token_mult != nullptr;
    if (slot_map) {
        const hipError_t me = launch_check_slot_map(slot_map, E, d_err, s);
        if (me != hipSuccess) return me;
    }
    // per-sequence counts ride on the histogram (zeroing) and scatter (counting) launches
    const bool seqs = seq_counts && num_seqs > 0 && T > 0;
    if (seq_counts && num_seqs > 0 && T == 0) {
        const int64_t n = (int64_t)num_seqs * E;
        fill_i32_kernel<<<dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256),
                          0, s>>>(seq_counts, n, 0);
    }
    if (nchunks > 0)
        hist_kernel<<<dim3((unsigned)nchunks), dim3(256), 0, s>>>(
            topk_idx, A, k, E, token_mult, ws.blk_hist,
            (weighted_counts && have_q) ? ws.blk_whist : nullptr, d_err, slot_map,
            seqs ? seq_counts : nullptr, seqs ? (int64_t)num_seqs * E : 0, mass_part,
            mass_nblk, prob_mass);
    else if (prob_mass)
        return hipErrorInvalidValue;   // a deferred mass needs the histogram launch
    // the forward's tile list comes with the scan (tiles_bt > 0)
    const int bt = tiles_bt > 0 ? tiles_bt : 1;
    scan_kernel<<<dim3(1), dim3(256), 0, s>>>(
        ws.blk_hist, ws.blk_whist, nchunks, E, have_q, counts, offsets, weighted_counts, bt,
        tiles_bt > 0 ? max_m_tiles(A, E, bt) : 0, tiles_bt > 0 ? ws.tiles : nullptr);
    if (nchunks > 0)
        scatter_kernel<<<dim3((unsigned)nchunks), dim3(256), 0, s>>>(
            topk_idx, A, E, ws.blk_hist, perm, inv, slot_map, k, cu_seqlens, num_seqs,
            seqs ? seq_counts : nullptr, d_err);
    if (x_perm) {
        const hipError_t ge = launch_gather(dm, x, inv, x_perm, s);
        if (ge != hipSuccess) return ge;
    }
    return hipGetLastError();
}

}  // namespace moe
