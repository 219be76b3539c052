// bf16 GEMMs on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation.  Both operands are fan-in (K) contiguous: C = A * B^T.
//
// Used for every contraction of the layer (Nemotron 3 overview, section 2.2
// steps 1-3; the overview's mixed-precision table keeps the latent
// projections in BF16):
//   dense   x [W_down; W_r; W_s1]^T  -> z (bf16), logits (fp32 + bias),
//                                        hs = relu(.)^2 (bf16)
//   dense   [c | hs] [W_up | W_s2]^T -> out (two K segments, one accumulator)
//   grouped per-expert z[perm] W1_e^T -> H = relu(.)^2 ; H W2_e^T -> Y * gate
//
// Block tile BM x BN x 64, 4 waves in a WAVES_M x WAVES_N grid, each wave a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA tiles.  Global -> register
// staging of tile k+1 overlaps the MFMAs of tile k; two LDS buffers, one
// barrier per K step.  LDS rows are 64 bf16 = 8 16-byte chunks, stored with
// chunk' = chunk ^ (row & 7) so the fragment reads of 32 rows at one chunk
// spread over the banks.
//
// Block -> tile mapping is XCD-aware: consecutive block ids go round-robin to
// the 8 XCDs, so block b is the (b/8)-th block of XCD b%8; each XCD is given
// a contiguous range of the tile order, so tiles that share operands run
// together under one L2.
#include "device_common.hpp"
#include "lmoe_internal.hpp"

namespace lmoe {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct MfmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int RPP = NT / 8;  // rows covered by one pass of 16-byte chunk loads
    static constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    static constexpr int LDS_CHUNKS = 2 * (BM + BN) * 8;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of NT/8");
};

__device__ __forceinline__ int swz(int row, int ch) { return (row << 3) | (ch ^ (row & 7)); }

// Output (m, n) of register r of the 32x32 tile for this lane, when the MFMA
// is issued as mfma(B-fragment, A-fragment): m = lane % 32,
// n = 8 * (r / 4) + 4 * (lane / 32) + r % 4.
template <class C>
__device__ __forceinline__ void mma_tile(const u32x4_t* __restrict__ As, const u32x4_t* __restrict__ Bs,
                                         f32x16_t (&acc)[C::TM][C::TN], int wm, int wn, int lane) {
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
        const int ch = ks * 2 + (lane >> 5);
        bf16x8_t af[C::TM], bfr[C::TN];
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) af[tm] = as_bf16x8(As[swz(wm * C::WM + tm * 32 + (lane & 31), ch)]);
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bfr[tn] = as_bf16x8(Bs[swz(wn * C::WN + tn * 32 + (lane & 31), ch)]);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = mfma32x32x16(bfr[tn], af[tm], acc[tm][tn]);
    }
}

// Software pipeline over nk K-tiles.  gload(kt) fetches tile kt into the
// caller's staging registers, lstore(As, Bs) writes them to one LDS buffer.
template <class C, class GLoad, class LStore>
__device__ __forceinline__ void mainloop(int nk, GLoad&& gload, LStore&& lstore, u32x4_t* smem,
                                         f32x16_t (&acc)[C::TM][C::TN], int wm, int wn, int lane) {
    constexpr int BUF = (C::BM + C::BN) * 8;
    gload(0);
    lstore(smem, smem + C::BM * 8);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) gload(kt + 1);
        u32x4_t* cur = smem + (kt & 1) * BUF;
        mma_tile<C>(cur, cur + C::BM * 8, acc, wm, wn, lane);
        if (more) {
            u32x4_t* nxt = smem + ((kt + 1) & 1) * BUF;
            lstore(nxt, nxt + C::BM * 8);
        }
        __syncthreads();
    }
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[C::TM][C::TN]) {
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;
}

// XCD-aware position of block b in a work list of W items (b < grid).
// Returns -1 for a block with no work.
__device__ __forceinline__ int xcd_work_index(int b, int W) {
    const int x = b & 7, s = b >> 3;
    const int per = W >> 3, rem = W & 7;
    const int cnt = per + (x < rem ? 1 : 0);
    if (s >= cnt) return -1;
    return x * per + min(x, rem) + s;
}

// ---------------------------------------------------------------------------
// Dense GEMM
// ---------------------------------------------------------------------------

__device__ __forceinline__ const NGroup& pick_group(const DenseGemm& g, int n) {
    if (g.ngroups > 2 && n >= g.g[2].n_begin) return g.g[2];
    if (g.ngroups > 1 && n >= g.g[1].n_begin) return g.g[1];
    return g.g[0];
}

__device__ __forceinline__ float apply_epi(int epi, float v, float bias_v) {
    if (epi == EPI_RELU2) {
        v = fmaxf(v, 0.f);
        return v * v;
    }
    if (epi == EPI_F32_BIAS) return v + bias_v;
    return v;
}

__device__ __forceinline__ void dense_store1(const DenseGemm& g, int m, int n, float v) {
    const NGroup& G = pick_group(g, n);
    const int nc = n - G.n_begin;
    const int64_t off = (int64_t)m * G.ldc + nc;
    if (G.epi == EPI_F32_BIAS) {
        ((float*)G.C)[off] = v + (G.bias ? G.bias[nc] : 0.f);
    } else {
        ((uint16_t*)G.C)[off] = f32_to_bf16_rne(apply_epi(G.epi, v, 0.f));
    }
}

// 4 consecutive columns n..n+3 of row m.
__device__ __forceinline__ void dense_store4(const DenseGemm& g, int m, int n, const float (&v)[4]) {
    const NGroup& G = pick_group(g, n);
    const int nc = n - G.n_begin;
    if (n + 3 < G.n_end && (nc & 3) == 0 && (G.ldc & 3) == 0) {
        const int64_t off = (int64_t)m * G.ldc + nc;
        if (G.epi == EPI_F32_BIAS) {
            float4 o = make_float4(v[0], v[1], v[2], v[3]);
            if (G.bias) {
                const float4 b = *reinterpret_cast<const float4*>(G.bias + nc);
                o.x += b.x;
                o.y += b.y;
                o.z += b.z;
                o.w += b.w;
            }
            *reinterpret_cast<float4*>((float*)G.C + off) = o;
        } else {
            uint2 o;
            o.x = pack_bf16x2(apply_epi(G.epi, v[0], 0.f), apply_epi(G.epi, v[1], 0.f));
            o.y = pack_bf16x2(apply_epi(G.epi, v[2], 0.f), apply_epi(G.epi, v[3], 0.f));
            *reinterpret_cast<uint2*>((uint16_t*)G.C + off) = o;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (n + i < g.N) dense_store1(g, m, n + i, v[i]);
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void dense_gemm_kernel(DenseGemm g, int tiles_m, int tiles_n,
                                                              int group_m) {
    __shared__ u32x4_t smem[C::LDS_CHUNKS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    const int w = xcd_work_index(blockIdx.x, tiles_m * tiles_n);
    if (w < 0) return;
    const int width = group_m * tiles_n;
    const int first_m = (w / width) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int m0 = (first_m + (w % width) % gsz) * C::BM;
    const int n0 = ((w % width) / gsz) * C::BN;

    const int ch = tid & 7, r0 = tid >> 3;
    const uint16_t* a_ptr[C::A_LD];
    const uint16_t* b_ptr[C::B_LD];
    auto setup_seg = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) {
            const int m = min(m0 + r0 + i * C::RPP, g.M - 1);
            a_ptr[i] = (const uint16_t*)g.A[s] + (int64_t)m * g.lda[s] + ch * 8;
        }
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) {
            const int n = min(n0 + r0 + i * C::RPP, g.N - 1);
            const NGroup& G = pick_group(g, n);
            b_ptr[i] = (const uint16_t*)G.B[s] + (int64_t)(n - G.n_begin) * g.K[s] + ch * 8;
        }
    };

    const int nk0 = g.K[0] / C::BK;
    const int nk = nk0 + (g.nseg > 1 ? g.K[1] / C::BK : 0);
    int cur_seg = 0;
    setup_seg(0);

    u32x4_t ra[C::A_LD], rb[C::B_LD];
    auto gload = [&](int kt) __attribute__((always_inline)) {
        if (kt == nk0 && cur_seg == 0) {
            cur_seg = 1;
            setup_seg(1);
        }
        const int kk = (kt - (cur_seg ? nk0 : 0)) * C::BK;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_ptr[i] + kk);
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(b_ptr[i] + kk);
    };
    auto lstore = [&](u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) As[swz(r0 + i * C::RPP, ch)] = ra[i];
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) Bs[swz(r0 + i * C::RPP, ch)] = rb[i];
    };

    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    mainloop<C>(nk, gload, lstore, smem, acc, wm, wn, lane);

#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
        const int m = m0 + wm * C::WM + tm * 32 + (lane & 31);
        if (m >= g.M) continue;
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * C::WN + tn * 32 + q * 8 + (lane >> 5) * 4;
                if (n >= g.N) continue;
                const float v[4] = {acc[tm][tn][q * 4 + 0], acc[tm][tn][q * 4 + 1], acc[tm][tn][q * 4 + 2],
                                    acc[tm][tn][q * 4 + 3]};
                dense_store4(g, m, n, v);
            }
    }
}

// ---------------------------------------------------------------------------
// Grouped (per-expert) GEMM
// ---------------------------------------------------------------------------

// 8 E2M1 codes (one 32-bit word, element i in bits 4i..4i+3) times an E4M3
// block scale -> 8 bf16.  E2M1: sign bit 3, exponent bits 2-1 (bias 1),
// mantissa bit 0, so the magnitudes are {0, .5, 1, 1.5, 2, 3, 4, 6}; the
// product with an E4M3 value has at most 6 significant bits and is exact in
// bf16 (Nemotron 3 overview, section 3.1.1: E2M1 elements, 16-element
// micro-blocks, E4M3 block scale).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float v = (e == 0) ? (float)m * 0.001953125f  // 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
    return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, float scale) {
    // twice the magnitude of each 3-bit code, 4 bits per entry
    constexpr uint32_t kMag2 = 0xC8643210u;
    const float hs = 0.5f * scale;
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t c = (codes >> (8 * i + 4 * j)) & 15u;
            const float mag = (float)((kMag2 >> ((c & 7u) * 4u)) & 15u) * hs;
            const uint32_t bits = __float_as_uint(mag) ^ ((c & 8u) << 28);
            h[j] = bits >> 16;  // exact: no rounding needed
        }
        out[i] = h[0] | (h[1] << 16);
    }
    u32x4_t r;
    r.x = out[0];
    r.y = out[1];
    r.z = out[2];
    r.w = out[3];
    return r;
}

template <class C, int BFMT>
__global__ __launch_bounds__(C::NT, 1) void grouped_gemm_kernel(GroupedGemm g, int nN) {
    __shared__ u32x4_t smem[C::LDS_CHUNKS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    const int total_tiles = *g.tt.tile_count;
    const int w = xcd_work_index(blockIdx.x, total_tiles * nN);
    if (w < 0) return;
    // Work order: expert-major, then N tile, then M tile, so the M tiles of one
    // (expert, N tile) pair run back to back on the same XCD.
    const int e = g.tt.tiles[w / nN].x;
    const int ts0 = g.tt.expert_tile_start[e], nt = g.tt.expert_ntiles[e];
    const int local = w - ts0 * nN;
    const int n0 = (local / nt) * C::BN;
    const int4 tile = g.tt.tiles[ts0 + local % nt];
    const int row0 = tile.y, rows = tile.z;

    const int ch = tid & 7, r0 = tid >> 3;
    const int N = g.N, K = g.K;
    const uint16_t* a_ptr[C::A_LD];
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const int p = row0 + min(r0 + i * C::RPP, rows - 1);
        const int ar = g.a_row_map ? g.a_row_map[p] / g.a_row_div : p;
        a_ptr[i] = (const uint16_t*)g.A + (int64_t)ar * g.lda + ch * 8;
    }
    const uint16_t* b_ptr[C::B_LD];
    const uint32_t* c_ptr[C::B_LD];
    const uint8_t* s_ptr[C::B_LD];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const int64_t n = (int64_t)e * N + min(n0 + r0 + i * C::RPP, N - 1);
        if constexpr (BFMT == LMOE_NVFP4) {
            c_ptr[i] = (const uint32_t*)(g.B_codes + n * (K / 2)) + ch;
            s_ptr[i] = g.B_scales + n * (K / 16) + (ch >> 1);
        } else {
            b_ptr[i] = (const uint16_t*)g.B + n * K + ch * 8;
        }
    }

    u32x4_t ra[C::A_LD], rb[C::B_LD];
    uint32_t rc[C::B_LD], rs[C::B_LD];
    auto gload = [&](int kt) __attribute__((always_inline)) {
        const int kk = kt * C::BK;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_ptr[i] + kk);
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) {
            if constexpr (BFMT == LMOE_NVFP4) {
                rc[i] = c_ptr[i][kt * 8];  // 32 code bytes per row per K tile
                rs[i] = s_ptr[i][kt * 4];  // 4 scale bytes per row per K tile
            } else {
                rb[i] = *reinterpret_cast<const u32x4_t*>(b_ptr[i] + kk);
            }
        }
    };
    auto lstore = [&](u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) As[swz(r0 + i * C::RPP, ch)] = ra[i];
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) {
            if constexpr (BFMT == LMOE_NVFP4)
                Bs[swz(r0 + i * C::RPP, ch)] = decode_e2m1x8(rc[i], e4m3_to_f32(rs[i]));
            else
                Bs[swz(r0 + i * C::RPP, ch)] = rb[i];
        }
    };

    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    mainloop<C>(K / C::BK, gload, lstore, smem, acc, wm, wn, lane);

    const float scale = (BFMT == LMOE_NVFP4) ? g.B_ts[e] : 1.0f;
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
        const int ml = wm * C::WM + tm * 32 + (lane & 31);
        if (ml >= rows) continue;
        const int p = row0 + ml;
        float rs_ = scale;
        if (g.epi == EPI_GATE) rs_ *= g.gate[g.gate_map[p]];
        uint16_t* crow = (uint16_t*)g.C + (int64_t)p * g.ldc;
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * C::WN + tn * 32 + q * 8 + (lane >> 5) * 4;
                if (n >= N) continue;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = acc[tm][tn][q * 4 + i] * rs_;
                    if (g.epi == EPI_RELU2) {
                        v[i] = fmaxf(v[i], 0.f);
                        v[i] *= v[i];
                    }
                }
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(crow + n) = o;
            }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

template <class C>
static hipError_t run_dense(const DenseGemm& g, hipStream_t s) {
    const int tiles_m = (g.M + C::BM - 1) / C::BM, tiles_n = (g.N + C::BN - 1) / C::BN;
    LMOE_LAUNCH("dense_gemm", s, dense_gemm_kernel<C><<<tiles_m * tiles_n, C::NT, 0, s>>>(g, tiles_m, tiles_n, 8));
    return hipGetLastError();
}

hipError_t launch_dense_gemm_bf16(const DenseGemm& g, hipStream_t s) {
    if (g.M <= 64) return run_dense<MfmaCfg<64, 64, 2, 2>>(g, s);
    return run_dense<MfmaCfg<128, 256, 2, 2>>(g, s);
}

template <class C>
static hipError_t run_grouped(const GroupedGemm& g, hipStream_t s) {
    const int nN = (g.N + C::BN - 1) / C::BN;
    const int grid = g.tt.max_tiles * nN;
    if (g.b_fmt == LMOE_NVFP4)
        LMOE_LAUNCH("grouped_gemm_nvfp4", s, grouped_gemm_kernel<C, LMOE_NVFP4><<<grid, C::NT, 0, s>>>(g, nN));
    else
        LMOE_LAUNCH("grouped_gemm", s, grouped_gemm_kernel<C, LMOE_BF16><<<grid, C::NT, 0, s>>>(g, nN));
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, hipStream_t s) {
    if (g.tt.bm == 128) return run_grouped<MfmaCfg<128, 256, 2, 2>>(g, s);
    if (g.tt.bm == 32) return run_grouped<MfmaCfg<32, 128, 1, 4>>(g, s);
    return hipErrorInvalidValue;
}

}  // namespace lmoe
