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

namespace lmoe {

constexpr int kChunk = 1024;
constexpr int kMaxExperts = 1024;

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

// Exclusive scan of one int per thread over a block of 1024 threads.
__device__ int block_exclusive_scan_1024(int v, int* total_out) {
    __shared__ int wsum[16];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int i = 0; i < 16; ++i) {
        const int s = wsum[i];
        if (i < w) base += s;
        total += s;
    }
    __syncthreads();
    *total_out = total;
    return base + incl - v;
}

__device__ void write_tiles(int e, int E, int count, int offset, const TileTable& tt,
                            int* tile_start_out, int* ntiles_out) {
    const int bm = tt.bm;
    const int nt = (e < E) ? (count + bm - 1) / bm : 0;
    int total_tiles;
    const int ts = block_exclusive_scan_1024(nt, &total_tiles);
    if (e < E) {
        int4* tiles = const_cast<int4*>(tt.tiles);
        for (int m = 0; m < nt; ++m)
            tiles[ts + m] = make_int4(e, offset + m * bm, min(bm, count - m * bm), m | (nt << 16));
        const_cast<int*>(tt.expert_tile_start)[e] = ts;
        const_cast<int*>(tt.expert_ntiles)[e] = nt;
    }
    if (threadIdx.x == 0) const_cast<int*>(tt.tile_count)[0] = total_tiles;
    for (int i = threadIdx.x; i < tt.sk_count_len; i += blockDim.x) tt.sk_count[i] = 0;
    *tile_start_out = ts;
    *ntiles_out = nt;
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

// One wave scatters pairs [p0, p1) in order; cur[e] is the next position of
// expert e and belongs to this wave alone.
__device__ __forceinline__ void scatter_range(const int32_t* __restrict__ idx, int64_t p0, int64_t p1, int E,
                                              int* cur, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int lane = threadIdx.x & 63;
    const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t q = p0; q < p1; q += 64) {
        const int64_t p = q + lane;
        const int e = (p < p1) ? idx[p] : -1;
        const bool valid = (e >= 0) && (e < E);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        const int pos = valid ? cur[e] + rank : -1;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            perm[pos] = (int32_t)p;
            // the highest lane of each group of equal ids advances the cursor
            if ((peers >> lane) == 1ull) cur[e] = pos + 1;
        }
        if (p < p1) inv[p] = pos;
        __builtin_amdgcn_wave_barrier();
    }
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

// All of it in one block of 16 waves: wave w owns pairs [w*len, (w+1)*len).
constexpr int kSmallWaves = 16;
constexpr int64_t kSmallMaxPairs = 32768;

__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* __restrict__ idx, int64_t n_pairs, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                          TileTable tt, int build_tiles) {
    __shared__ int h[kSmallWaves][kMaxExperts];
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kSmallWaves * kMaxExperts; i += 1024) (&h[0][0])[i] = 0;
    __syncthreads();
    const int64_t len = (n_pairs + kSmallWaves - 1) / kSmallWaves;
    const int64_t p0 = min(n_pairs, (int64_t)w * len), p1 = min(n_pairs, p0 + len);
    for (int64_t p = p0 + (threadIdx.x & 63); p < p1; p += 64) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicAdd(&h[w][e], 1);
    }
    __syncthreads();
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        for (int v = 0; v < kSmallWaves; ++v) {
            const int c = h[v][e];
            h[v][e] = total;
            total += c;
        }
    }
    int all;
    const int off = block_exclusive_scan_1024(e < E ? total : 0, &all);
    if (e < E) {
        counts[e] = total;
        offsets[e] = off;
        for (int v = 0; v < kSmallWaves; ++v) h[v][e] += off;
    }
    if (e == 0) offsets[E] = all;
    if (build_tiles) {
        int ts, nt;
        write_tiles(e, E, total, off, tt, &ts, &nt);
    }
    __syncthreads();
    scatter_range(idx, p0, p1, E, h[w], perm, inv);
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
