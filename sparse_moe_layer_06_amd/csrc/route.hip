// Router top-k and gate.
//
// For each token: the k largest of its E fp32 logits, in the order (logit
// desc, expert id asc), and gates = softmax over the k selected logits.
// Ultra routes each token to 22 of 512 experts (Nemotron 3 Ultra release
// news, architecture paragraph); the overview article (section 2.2 step 2)
// places routing in the latent stage.  The softmax-over-selected gate is
// this library's specification.
//
// One wavefront per token.  Each lane holds E/64 logits as 64-bit keys
// (order-preserving logit bits << 32 | ~expert id), so a plain max over keys
// picks the larger logit and, on equal logits, the smaller id.  k rounds of
// a local max plus a 6-step xor-shuffle max; the winner's owner lane clears
// it.  Lane j % 64 keeps selection j in register slot j / 64.
#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

constexpr int kMaxE = 1024;
constexpr int kSlots = kMaxE / kWave;  // 16 logits per lane at most

__device__ __forceinline__ uint32_t ordered_bits(float v) {
    uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0: equal logits compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered_value(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = v > w ? v : w;
    }
    return v;
}

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int32_t* __restrict__ idx,
                                                           float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave exits together
    const float* s = logits + (int64_t)t * E;

    uint64_t key[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int e = lane + i * kWave;
        key[i] = (e < E) ? (((uint64_t)ordered_bits(s[e]) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
    }

    float sel_v[kSlots];
    int sel_e[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        sel_v[i] = 0.f;
        sel_e[i] = 0;
    }

    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kSlots; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
        const float v = unordered_value((uint32_t)(best >> 32));
        const int owner = e & 63, slot = e >> 6;
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if (i == slot && lane == owner) key[i] = 0;
        const int jl = j & 63, js = j >> 6;
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if (i == js && lane == jl) {
                sel_v[i] = v;
                sel_e[i] = e;
            }
    }

    // gate = softmax over the selected logits; selection 0 holds the max.
    const float vmax = __shfl(sel_v[0], 0, kWave);
    float w[kSlots];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int j = lane + i * kWave;
        w[i] = (j < k) ? expf(sel_v[i] - vmax) : 0.f;
        part += w[i];
    }
    const float inv_sum = 1.0f / wave_sum(part);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int j = lane + i * kWave;
        if (j < k) {
            idx[(int64_t)t * k + j] = sel_e[i];
            gate[(int64_t)t * k + j] = w[i] * inv_sum;
        }
    }
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* gate,
                               hipStream_t s) {
    if (E > kMaxE) return hipErrorInvalidValue;
    dim3 grid((T + 3) / 4);
    LMOE_LAUNCH("topk_softmax", s, topk_softmax_kernel<<<grid, 256, 0, s>>>(logits, T, E, k, idx, gate));
    return hipGetLastError();
}

}  // namespace lmoe
