// Top-k (k <= 64) and softmax gate of one token's logits, by one wavefront:
// shared by the router kernel (route.hip) and the decode-sized reduction
// that finishes the first dense GEMM (gemm_mfma.hip).  The selection order
// is (logit desc, expert id asc); Ultra routes each token to 22 of 512
// experts (Nemotron 3 Ultra release news, architecture paragraph), and the
// softmax over the selected logits is this library's gate.
#pragma once

#include "device_common.hpp"

namespace lmoe {

// Order-preserving 32-bit encoding of a float (larger value, larger code).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
    uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0: equal logits compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_value(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Gates of the k (<= 64) selections held by lanes 0..k-1, in rank order:
// softmax with the rank-0 logit as the shift.  COHERENT_IDX stores the ids
// with device-coherent (agent-scope) stores, for a reader on another XCD
// within the same kernel.
template <bool COHERENT_IDX = false>
__device__ __forceinline__ void write_gates(float v, int e, int lane, int64_t t, int k, int32_t* __restrict__ idx,
                                            float* __restrict__ gate) {
    const float vmax = __shfl(v, 0, kWave);
    const float w = lane < k ? expf(v - vmax) : 0.f;
    const float inv_sum = 1.0f / wave_sum(w);
    if (lane < k) {
        if constexpr (COHERENT_IDX)
            __hip_atomic_store(idx + t * k + lane, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            idx[t * k + lane] = e;
        gate[t * k + lane] = w * inv_sum;
    }
}

// Radix select over the E logits s[0..E) (global memory or LDS), S = E/64
// rounded up logits per lane: the k-th largest logit X is found bit by bit
// from the top of the encoding (X is the largest value with at least k
// logits >= X; each bit costs S ballots and popcounts).  The selection is
// every logit above X plus the lowest ids among those equal to X; the k
// selected (logit, id) keys are ranked against each other in the wave's LDS
// scratch (by_id, by_rank: 64 keys each) and lane j writes the key of rank j.
template <int S, bool COHERENT_IDX = false>
__device__ __forceinline__ void topk_select_row(const float* s, int E, int k, int64_t t, uint64_t* by_id,
                                                uint64_t* by_rank, int32_t* __restrict__ idx,
                                                float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t v[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int e = lane + i * kWave;
        v[i] = (e < E) ? ordered_bits(s[e]) : 0u;  // 0 is below every encoded logit
    }
    auto count_ge = [&](uint32_t y) __attribute__((always_inline)) {
        int c = 0;
#pragma unroll
        for (int i = 0; i < S; ++i) c += __popcll(__ballot(v[i] >= y));
        return c;
    };
    uint32_t X = 0;
    for (int b = 31; b >= 0; --b) {
        const uint32_t y = X | (1u << b);
        if (count_ge(y) >= k) X = y;
    }
    // logits above X are all selected; ties at X go to the lowest ids
    int need = k;
#pragma unroll
    for (int i = 0; i < S; ++i) need -= __popcll(__ballot(v[i] > X));
    int base = 0;  // position of this slot's first selection in id order
#pragma unroll
    for (int i = 0; i < S; ++i) {
        const int e = lane + i * kWave;
        const bool eq = e < E && v[i] == X;
        const uint64_t m_eq = __ballot(eq);
        const bool take = v[i] > X || (eq && __popcll(m_eq & lt_mask) < need);
        need -= min(need, __popcll(m_eq));
        const uint64_t m = __ballot(take);
        if (take) by_id[base + __popcll(m & lt_mask)] = ((uint64_t)v[i] << 32) | (uint32_t)(~(uint32_t)e);
        base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // rank = the number of selected keys above this one (keys are distinct)
    if (lane < k) {
        const uint64_t key = by_id[lane];
        int rank = 0;
        for (int q = 0; q < k; ++q) rank += by_id[q] > key;
        by_rank[rank] = key;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t key = lane < k ? by_rank[lane] : 0ull;
    write_gates<COHERENT_IDX>(unordered_value((uint32_t)(key >> 32)), (int)(~(uint32_t)key), lane, t, k, idx, gate);
}

}  // namespace lmoe
