// Token permutation: a stable counting sort of the (token, slot) pairs by
// expert, so that each expert's rows are contiguous for the grouped GEMMs
// of the latent-space experts (Nemotron 3 overview, section 2.2 step 2).
//
// Many pairs (prefill):
//   1. hist:      one block per chunk of kChunk pairs; LDS histogram of the
//                 chunk's expert ids -> hist[chunk][e].
//   2. chunkscan: one wave per expert; exclusive scan of its column over the
//                 chunks -> hist[chunk][e] = pairs of e in earlier chunks,
//                 counts[e] = the column total.
//   3. offsets:   one block; exclusive scan over experts -> offsets, and the
//                 grouped-GEMM tile table.
//   4. scatter:   one wavefront per chunk walks its pairs in order, 64 at a
//                 time, from cursor offsets[e] + hist[chunk][e]; lanes
//                 holding the same expert are found with ballots over the id
//                 bits, so the rank within the wave (and thus the whole
//                 sort) is stable.
// Few pairs (decode): one block does all four steps with its 16 waves as
// the chunks and the histograms in LDS.
// No global atomics: the result is the same on every run.  Pairs whose
// expert id is outside [0, E) are left out of counts, and get inv = -1.
#include "device_common.hpp"
#include "lmoe_internal.hpp"
#include "perm_block.hpp"

namespace lmoe {

constexpr int kChunk = 1024;

int permute_nchunks(int64_t n_pairs) { return (int)((n_pairs + kChunk - 1) / kChunk); }

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int64_t n_pairs,
                                                        int E, int32_t* __restrict__ hist) {
    __shared__ int h[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kChunk;
    const int64_t p1 = min(n_pairs, p0 + kChunk);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, kWave);
        if (lane >= o) v += u;
    }
    return v;
}

// One wave per expert: hist[c][e] <- sum of hist[c'][e] over c' < c.
__global__ __launch_bounds__(1024) void perm_chunkscan_kernel(int32_t* __restrict__ hist, int nchunks, int E,
                                                              int32_t* __restrict__ counts) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 16 + (threadIdx.x >> 6);
    if (e >= E) return;  // whole wave
    int carry = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
        const int c = c0 + lane;
        const int v = (c < nchunks) ? hist[(int64_t)c * E + e] : 0;
        const int incl = wave_inclusive_scan(v);
        if (c < nchunks) hist[(int64_t)c * E + e] = carry + incl - v;
        carry += __shfl(incl, 63, kWave);
    }
    if (lane == 0) counts[e] = carry;
}

// One block: offsets = exclusive scan of counts over experts; tile table.
__global__ __launch_bounds__(1024) void perm_offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                            int32_t* __restrict__ offsets, TileTable tt,
                                                            int build_tiles) {
    const int e = threadIdx.x;
    const int total = (e < E) ? counts[e] : 0;
    int all;
    const int off = block_exclusive_scan_1024(total, &all);
    if (e < E) offsets[e] = off;
    if (e == 0) offsets[E] = all;
    if (build_tiles) {
        int ts, nt;
        write_tiles(e, E, total, off, tt, &ts, &nt);
    }
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                           TileTable tt) {
    const int e = threadIdx.x;
    const int off = (e < E) ? offsets[e] : 0;
    const int cnt = (e < E) ? offsets[e + 1] - off : 0;
    int ts, nt;
    write_tiles(e, E, cnt, off, tt, &ts, &nt);
}

__global__ __launch_bounds__(64) void perm_scatter_kernel(const int32_t* __restrict__ idx, int64_t n_pairs,
                                                          int E, const int32_t* __restrict__ base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
    __shared__ int cur[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += 64) cur[e] = offsets[e] + base[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kChunk;
    scatter_range(idx, p0, min(n_pairs, p0 + kChunk), E, cur, perm, inv);
}

// Few pairs: all of it in one block of 16 waves.
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                          TileTable tt, int build_tiles) {
    __shared__ int h[kSmallWaves][kMaxExperts];
    perm_block(idx, n_pairs, E, counts, offsets, perm, inv, tt, build_tiles, h);
}

hipError_t launch_permute(const int32_t* idx, int64_t n_pairs, int E, int32_t* hist, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, const TileTable* tiles,
                          hipStream_t s) {
    if (E > kMaxExperts) return hipErrorInvalidValue;
    TileTable tt{};
    if (tiles) tt = *tiles;
    if (n_pairs <= kSmallMaxPairs) {
        LMOE_LAUNCH("perm_small", s,
                    perm_small_kernel<<<1, 1024, 0, s>>>(idx, n_pairs, E, counts, offsets, perm, inv, tt,
                                                         tiles ? 1 : 0));
        return hipGetLastError();
    }
    const int nchunks = permute_nchunks(n_pairs);
    LMOE_LAUNCH("perm_hist", s, perm_hist_kernel<<<nchunks, 256, 0, s>>>(idx, n_pairs, E, hist));
    LMOE_LAUNCH("perm_chunkscan", s, perm_chunkscan_kernel<<<(E + 15) / 16, 1024, 0, s>>>(hist, nchunks, E, counts));
    LMOE_LAUNCH("perm_offsets", s,
                perm_offsets_kernel<<<1, 1024, 0, s>>>(counts, E, offsets, tt, tiles ? 1 : 0));
    LMOE_LAUNCH("perm_scatter", s,
                perm_scatter_kernel<<<nchunks, 64, 0, s>>>(idx, n_pairs, E, hist, offsets, perm, inv));
    return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, const TileTable& tt, hipStream_t s) {
    if (E > kMaxExperts) return hipErrorInvalidValue;
    LMOE_LAUNCH("build_tiles", s, build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, tt));
    return hipGetLastError();
}

}  // namespace lmoe
