// fp32 GEMMs on the vector ALUs (fp32 FMA, fp32 accumulation), for layers
// stored in fp32.  Same problem descriptors and epilogues as the bf16 MFMA
// kernels; every output is stored in fp32.
//
// 64x64 output tile, K step 16, 256 threads, 4x4 outputs per thread.  The
// K-slices of A and B are stored k-major in LDS so each thread reads 4
// consecutive rows/columns as one float4.
#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

constexpr int kFT = 64;   // tile edge
constexpr int kFK = 16;   // K step

__device__ __forceinline__ void fma_step(const float (*As)[kFT], const float (*Bs)[kFT], float (&acc)[4][4],
                                         int ty, int tx) {
#pragma unroll
    for (int k = 0; k < kFK; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(&As[k][ty * 4]);
        const float4 b = *reinterpret_cast<const float4*>(&Bs[k][tx * 4]);
        const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
}

// Loads a 64 x 16 slice (rows given by per-thread row pointer) and stores it k-major.
__device__ __forceinline__ void fma_load(float (*S)[kFT], const float* row_ptr, int k0, int tid) {
    const float4 v = *reinterpret_cast<const float4*>(row_ptr + k0 + (tid & 3) * 4);
    const int r = tid >> 2, kq = (tid & 3) * 4;
    S[kq + 0][r] = v.x;
    S[kq + 1][r] = v.y;
    S[kq + 2][r] = v.z;
    S[kq + 3][r] = v.w;
}

__device__ __forceinline__ const NGroup& pick_group_f(const DenseGemm& g, int n) {
    if (g.ngroups > 2 && n >= g.g[2].n_begin) return g.g[2];
    if (g.ngroups > 1 && n >= g.g[1].n_begin) return g.g[1];
    return g.g[0];
}

__global__ __launch_bounds__(256) void dense_fma_kernel(DenseGemm g) {
    __shared__ float As[kFK][kFT], Bs[kFK][kFT];
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int m0 = blockIdx.y * kFT, n0 = blockIdx.x * kFT;
    const int lr = tid >> 2;  // row this thread loads
    float acc[4][4] = {};
    for (int s = 0; s < g.nseg; ++s) {
        const float* a_row = (const float*)g.A[s] + (int64_t)min(m0 + lr, g.M - 1) * g.lda[s];
        const int n = min(n0 + lr, g.N - 1);
        const NGroup& G = pick_group_f(g, n);
        const float* b_row = (const float*)G.B[s] + (int64_t)(n - G.n_begin) * g.K[s];
        for (int k0 = 0; k0 < g.K[s]; k0 += kFK) {
            fma_load(As, a_row, k0, tid);
            fma_load(Bs, b_row, k0, tid);
            __syncthreads();
            fma_step(As, Bs, acc, ty, tx);
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= g.N) continue;
            const NGroup& G = pick_group_f(g, n);
            const int nc = n - G.n_begin;
            float v = acc[i][j];
            if (G.epi == EPI_F32_BIAS && G.bias) v += G.bias[nc];
            if (G.epi == EPI_RELU2) {
                v = fmaxf(v, 0.f);
                v *= v;
            }
            float* c = (float*)G.C + (int64_t)m * G.ldc + nc;
            *c = G.epi == EPI_ADD ? *c + v : v;
        }
    }
}

// Grouped: blockIdx.y = M tile (of the device tile table, height 64),
// blockIdx.x = N tile.
__global__ __launch_bounds__(256) void grouped_fma_kernel(GroupedGemm g) {
    __shared__ float As[kFK][kFT], Bs[kFK][kFT];
    if ((int)blockIdx.y >= *g.tt.tile_count) return;
    const int4 tile = g.tt.tiles[blockIdx.y];
    const int e = tile.x, row0 = tile.y, rows = tile.z;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int n0 = blockIdx.x * kFT;
    const int lr = tid >> 2;
    const int p_load = row0 + min(lr, rows - 1);
    const int ar = g.a_row_map ? g.a_row_map[p_load] / g.a_row_div : p_load;
    const float* a_row = (const float*)g.A + (int64_t)ar * g.lda;
    const float* b_row = (const float*)g.B + ((int64_t)e * g.N + min(n0 + lr, g.N - 1)) * g.K;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += kFK) {
        fma_load(As, a_row, k0, tid);
        fma_load(Bs, b_row, k0, tid);
        __syncthreads();
        fma_step(As, Bs, acc, ty, tx);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ml = ty * 4 + i;
        if (ml >= rows) continue;
        const int p = row0 + ml;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= g.N) continue;
            float v = acc[i][j];
            if (g.epi == EPI_RELU2) {
                v = fmaxf(v, 0.f);
                v *= v;
            }
            ((float*)g.C)[(int64_t)p * g.ldc + n] = v;
        }
    }
}

hipError_t launch_dense_gemm_f32(const DenseGemm& g, hipStream_t s) {
    dim3 grid((g.N + kFT - 1) / kFT, (g.M + kFT - 1) / kFT);
    LMOE_LAUNCH("dense_gemm_f32", s, dense_fma_kernel<<<grid, 256, 0, s>>>(g));
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_f32(const GroupedGemm& g, hipStream_t s) {
    dim3 grid((g.N + kFT - 1) / kFT, g.tt.max_tiles);
    LMOE_LAUNCH("grouped_gemm_f32", s, grouped_fma_kernel<<<grid, 256, 0, s>>>(g));
    return hipGetLastError();
}

}  // namespace lmoe
