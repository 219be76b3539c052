// The single-block stable counting sort of the token permutation, shared by
// the permutation kernel for few pairs (permute.hip) and the decode-sized
// router reduction that runs it in its last block (gemm_mfma.hip).  Pairs
// (token, slot) are sorted by expert id, stably, so that each expert's rows
// are contiguous for the grouped GEMMs of the latent-space experts
// (Nemotron 3 overview, section 2.2 step 2); the pages do not describe this
// grouping, so the counting sort is this layer's own specification of it.
#pragma once

#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

constexpr int kMaxExperts = 1024;
constexpr int kSmallWaves = 16;
constexpr int64_t kSmallMaxPairs = 32768;

// Exclusive scan of one int per thread over a block of 1024 threads.
static __device__ int block_exclusive_scan_1024(int v, int* total_out) {
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

static __device__ void write_tiles(int e, int E, int count, int offset, const TileTable& tt,
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

// One wave scatters pairs [p0, p1) in order; cur[e] is the next position of
// expert e and belongs to this wave alone.
__device__ __forceinline__ void scatter_range(const int32_t* idx, int64_t p0, int64_t p1, int E,
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

// The whole sort in one block of 1024 threads (16 waves): wave w counts and
// then scatters pairs [w*len, (w+1)*len) with its own LDS histogram row h[w];
// a block scan gives the offsets (and the grouped-GEMM tile table).  idx may
// be in global memory or LDS.
__device__ __forceinline__ void perm_block(const int32_t* idx, int64_t n_pairs, int E,
                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                           const TileTable& tt, int build_tiles, int (&h)[kSmallWaves][kMaxExperts]) {
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

}  // namespace lmoe
