// Combine in the latent space: c_t = sum_{j=0..k-1} g_tj Y[inv[t*k + j]]
// with the router gates g (Nemotron 3 overview, section 2.2 step 3: the
// latent result is what gets projected back up to d).
//
// Each token's k rows are gathered and summed in fixed j order in fp32, so
// there are no atomics and the result is bit-identical run to run.  One
// block per (token, 2048-column slab); each thread owns one 16-byte vector
// of columns.  inv and gate entries are block-uniform loads.
#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ Y,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ gate, int k, int l,
                                                           uint16_t* __restrict__ c) {
    const int t = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (col >= l) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    const int32_t* row = inv + (int64_t)t * k;
    const float* grow = gate + (int64_t)t * k;
    for (int j = 0; j < k; ++j) {
        const int p = row[j];
        if (p < 0) continue;  // pair left out by the permutation (invalid expert id)
        const float gj = grow[j];
        const uint4 v = *reinterpret_cast<const uint4*>(Y + (int64_t)p * l + col);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(gj, __uint_as_float(w[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(gj, __uint_as_float(w[i] & 0xFFFF0000u), acc[2 * i + 1]);
        }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(c + (int64_t)t * l + col) = o;
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ Y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gate, int k, int l,
                                                          float* __restrict__ c) {
    const int t = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (col >= l) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int32_t* row = inv + (int64_t)t * k;
    for (int j = 0; j < k; ++j) {
        const int p = row[j];
        if (p < 0) continue;
        const float gj = gate[(int64_t)t * k + j];
        const float4 v = *reinterpret_cast<const float4*>(Y + (int64_t)p * l + col);
        acc.x = fmaf(gj, v.x, acc.x);
        acc.y = fmaf(gj, v.y, acc.y);
        acc.z = fmaf(gj, v.z, acc.z);
        acc.w = fmaf(gj, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(c + (int64_t)t * l + col) = acc;
}

hipError_t launch_combine(const void* Y, const int32_t* inv, const float* gate, int T, int k, int l,
                          int act_dtype, void* c, hipStream_t s) {
    if (act_dtype == LMOE_BF16) {
        dim3 grid(T, (l / 8 + 255) / 256);
        LMOE_LAUNCH("combine", s,
                    combine_bf16_kernel<<<grid, 256, 0, s>>>((const uint16_t*)Y, inv, gate, k, l, (uint16_t*)c));
    } else {
        dim3 grid(T, (l / 4 + 255) / 256);
        LMOE_LAUNCH("combine", s, combine_f32_kernel<<<grid, 256, 0, s>>>((const float*)Y, inv, gate, k, l, (float*)c));
    }
    return hipGetLastError();
}

}  // namespace lmoe
