// Combine in the latent space: c_t = sum_{j=0..k-1} g_tj Y[inv[t*k + j]]
// with the router gates g (Nemotron 3 overview, section 2.2 step 3: the
// latent result is what gets projected back up to d).
//
// Each token's k rows are gathered and summed in fixed j order in fp32, so
// there are no atomics and the result is bit-identical run to run.  One
// block per (token, 2048-column slab); each thread owns one 16-byte vector
// of columns.  The rows are fetched kGroup at a time, all loads of a group
// in flight together, then accumulated in j order.
#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

constexpr int kGroup = 8;

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
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        int p[kGroup];
        float gj[kGroup];
        u32x4_t v[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            // p < 0: pair left out by the permutation (invalid expert id)
            p[i] = (j0 + i < k) ? row[j0 + i] : -1;
            gj[i] = (j0 + i < k) ? grow[j0 + i] : 0.f;
        }
        // each row of Y is read exactly once: non-temporal loads
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
            v[i] = (p[i] >= 0) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Y + (int64_t)p[i] * l + col))
                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if (p[i] < 0) continue;
            const uint32_t w[4] = {v[i][0], v[i][1], v[i][2], v[i][3]};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = fmaf(gj[i], __uint_as_float(w[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = fmaf(gj[i], __uint_as_float(w[q] & 0xFFFF0000u), acc[2 * q + 1]);
            }
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
    const float* grow = gate + (int64_t)t * k;
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        int p[kGroup];
        float gj[kGroup];
        float4 v[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            p[i] = (j0 + i < k) ? row[j0 + i] : -1;
            gj[i] = (j0 + i < k) ? grow[j0 + i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
            v[i] = (p[i] >= 0) ? *reinterpret_cast<const float4*>(Y + (int64_t)p[i] * l + col)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
            if (p[i] < 0) continue;
            acc.x = fmaf(gj[i], v[i].x, acc.x);
            acc.y = fmaf(gj[i], v[i].y, acc.y);
            acc.z = fmaf(gj[i], v[i].z, acc.z);
            acc.w = fmaf(gj[i], v[i].w, acc.w);
        }
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
