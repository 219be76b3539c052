// Router top-k and gate.
//
// For each token: the k largest of its E fp32 logits, in the order (logit
// desc, expert id asc), and gates = softmax over the k selected logits.
// Ultra routes each token to 22 of 512 experts (Nemotron 3 Ultra release
// news, architecture paragraph); the overview article (section 2.2 step 2)
// places routing in the latent stage.  The softmax-over-selected gate is
// this library's specification.
//
// One wavefront per token; each lane holds S = ceil(E/64) logits.
//
// k <= 64 (radix select): the k-th largest logit X is found bit by bit from
// the top of the order-preserving 32-bit encoding (X is the largest value
// with at least k logits >= X; each bit costs S ballots and popcounts).
// The selection is every logit above X plus the lowest ids among those equal
// to X.  The k selected (logit, id) keys are ranked against each other in
// LDS, and lane j takes the key of rank j.
//
// k > 64 (repeated max): 64-bit keys (logit bits << 32 | ~expert id), so a
// plain max over keys picks the larger logit and, on equal logits, the
// smaller id.  Each lane sorts its keys once (descending), so its head is
// its largest; k rounds then take the wave-wide max of the heads (DPP row
// shifts and row broadcasts) and the winning lane drops its head.  Lane
// j % 64 keeps selection j in register slot j / 64.
#include "device_common.hpp"
#include "lmoe_internal.hpp"
#include "topk_row.hpp"

namespace lmoe {

constexpr int kMaxE = 1024;

// v = max(v, v moved by one DPP pattern); lanes the pattern does not reach
// read 0, the smallest key.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xf, false);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    return v > w ? v : w;
}

// Wave-wide max, returned uniform: row_shr 1, 2, 4, 8 leave each 16-lane
// row's max in its lane 15; row_bcast 15 and 31 carry it to lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
    v = dpp_max_step<0x111>(v);
    v = dpp_max_step<0x112>(v);
    v = dpp_max_step<0x114>(v);
    v = dpp_max_step<0x118>(v);
    v = dpp_max_step<0x142, 0xa>(v);
    v = dpp_max_step<0x143, 0xc>(v);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void cswap_desc(uint64_t& a, uint64_t& b) {
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
}

// Descending sort of S keys (odd-even transposition: S rounds, S <= 16).
template <int S>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[S]) {
    static_for<S>([&](auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        static_for<S / 2>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = 2 * decltype(ic)::value + (r & 1);
            if constexpr (i + 1 < S) cswap_desc(key[i], key[i + 1]);
        });
    });
}

template <int S>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int32_t* __restrict__ idx, float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave exits together
    const float* s = logits + (int64_t)t * E;

    uint64_t key[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int e = lane + i * kWave;
        key[i] = (e < E) ? (((uint64_t)ordered_bits(s[e]) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
    }
    sort_desc<S>(key);

    float sel_v[S];
    int sel_e[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        sel_v[i] = 0.f;
        sel_e[i] = 0;
    }

    for (int j = 0; j < k; ++j) {
        const uint64_t best = wave_max_key(key[0]);
        const int e = (int)(~(uint32_t)best);
        const float v = unordered_value((uint32_t)(best >> 32));
        if (lane == (e & 63)) {  // the owner drops its head
#pragma unroll
            for (int i = 0; i + 1 < S; ++i) key[i] = key[i + 1];
            key[S - 1] = 0;
        }
        const int jl = j & 63, js = j >> 6;  // js is uniform
        static_for<S>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if (i == js && lane == jl) {
                sel_v[i] = v;
                sel_e[i] = e;
            }
        });
    }

    // gate = softmax over the selected logits; selection 0 holds the max.
    const float vmax = __shfl(sel_v[0], 0, kWave);
    float w[S];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int j = lane + i * kWave;
        w[i] = (j < k) ? expf(sel_v[i] - vmax) : 0.f;
        part += w[i];
    }
    const float inv_sum = 1.0f / wave_sum(part);
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int j = lane + i * kWave;
        if (j < k) {
            idx[(int64_t)t * k + j] = sel_e[i];
            gate[(int64_t)t * k + j] = w[i] * inv_sum;
        }
    }
}

template <int S>
__global__ __launch_bounds__(256) void topk_select_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ idx, float* __restrict__ gate) {
    __shared__ uint64_t by_id[4][kWave], by_rank[4][kWave];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;  // whole wave exits together
    topk_select_row<S>(logits + (int64_t)t * E, E, k, t, by_id[wv], by_rank[wv], idx, gate);
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                               hipStream_t s) {
    if (E > kMaxE) return hipErrorInvalidValue;
    dim3 grid((T + 3) / 4);
    if (k <= kWave) {
        if (E <= 64)
            LMOE_LAUNCH("topk_softmax", s, topk_select_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
        else if (E <= 128)
            LMOE_LAUNCH("topk_softmax", s, topk_select_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
        else if (E <= 256)
            LMOE_LAUNCH("topk_softmax", s, topk_select_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
        else if (E <= 512)
            LMOE_LAUNCH("topk_softmax", s, topk_select_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
        else
            LMOE_LAUNCH("topk_softmax", s, topk_select_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
        return hipGetLastError();
    }
    if (E <= 64)
        LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    else if (E <= 128)
        LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    else if (E <= 256)
        LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    else if (E <= 512)
        LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    else
        LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    return hipGetLastError();
}

}  // namespace lmoe
