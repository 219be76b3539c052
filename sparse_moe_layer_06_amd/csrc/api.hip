// C ABI of the LatentMoE forward: host-side validation, workspace plan and
// the launch sequence.  Every step runs in this library's kernels; nothing
// here allocates device memory or synchronises the host.
//
// Launch sequence of latentmoe_forward (Nemotron 3 overview, section 2.2,
// steps 1-3; shared expert per the paragraph after its table):
//   1. dense MFMA GEMM  x [W_down; W_r; W_s1]^T -> z, logits (+bias), hs
//   2. top-k + softmax gate                     -> idx, gate
//      (with few tokens: in step 1's split-K reduction)
//   3. permutation (hist, scan + tile table, stable scatter; with few tokens
//      in the last token block of step 2's reduction)
//   4. grouped GEMM  H = relu(z[perm] W1_e^T)^2
//   5. grouped GEMM  Y = H W2_e^T
//   6. combine       c_t = sum_j gate_tj Y[inv(t, j)]
//   7. dense GEMM    out = [c | hs] [W_up | W_s2]^T
// With FP8 weights the shared expert's products and the projections run as
// fp8 GEMMs of their own, each after a per-token quantisation of its input.
#include <string.h>

#include <mutex>
#include <new>

#include "lmoe_internal.hpp"

namespace lmoe {

hipError_t launch_dense_gemm_bf16(const DenseGemm& g, void* splitk_ws, size_t splitk_bytes, hipStream_t s);
hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, hipStream_t s);
hipError_t launch_dense_gemm_f32(const DenseGemm& g, hipStream_t s);
hipError_t launch_grouped_gemm_f32(const GroupedGemm& g, hipStream_t s);

hipError_t launch_dense_gemm(const DenseGemm& g, int act_dtype, int /*T_hint*/, void* splitk_ws,
                             size_t splitk_bytes, hipStream_t s) {
    return act_dtype == LMOE_BF16 ? launch_dense_gemm_bf16(g, splitk_ws, splitk_bytes, s)
                                  : launch_dense_gemm_f32(g, s);
}

hipError_t launch_grouped_gemm(const GroupedGemm& g, int act_dtype, hipStream_t s) {
    return act_dtype == LMOE_BF16 ? launch_grouped_gemm_bf16(g, s) : launch_grouped_gemm_f32(g, s);
}

// Rows per expert tile, which also picks the expert GEMM configuration:
// 192-row tiles when experts see many rows, 64-row tiles otherwise.
int grouped_bm(const lmoe_dims& d) {
    if (d.act_dtype == LMOE_F32) return 64;
    const double avg = (double)d.T * (double)d.k / (double)d.E;
    return avg >= 96.0 ? 192 : 64;
}

static int64_t max_tiles(const lmoe_dims& d) {
    const int64_t n = d.T * d.k;
    const int bm = grouped_bm(d);
    return (n + bm - 1) / bm + (d.E < n ? d.E : n);
}

// The shared expert with FP8 weights runs its two products as fp8 GEMMs of
// their own; with weights in the activation dtype it rides in the dense
// GEMMs (W_s1 as extra columns of the first, W_s2 as a second K segment of
// the last).
static bool shared_fp8(const lmoe_dims& d) { return d.f_s > 0 && d.shared_dtype == LMOE_FP8_E4M3; }
static bool shared_dense(const lmoe_dims& d) { return d.f_s > 0 && d.shared_dtype != LMOE_FP8_E4M3; }
// 8-bit down- and up-projections: fp8 GEMMs of their own, like the shared
// expert's, with per-row scales (FP8) or MXFP8 blocks.
static bool proj_fp8(const lmoe_dims& d) { return d.proj_dtype == LMOE_FP8_E4M3; }
static bool proj_mx(const lmoe_dims& d) { return d.proj_dtype == LMOE_MXFP8; }
static bool proj_8bit(const lmoe_dims& d) { return proj_fp8(d) || proj_mx(d); }
// Whether the last dense GEMM only adds the shared expert to an out that
// already holds the routed result (standard MoE, or an 8-bit up-projection).
static bool out_add_only(const lmoe_dims& d) { return d.standard_moe || proj_8bit(d); }

// x [W_down; W_r; W_s1]^T -> z, logits (+ bias), hs (the shared expert's
// hidden layer, only with f_s > 0 in the activation dtype).  With a latent
// router the logits are left to gemm_router; with FP8 projections z is left
// to the fp8 GEMM.  N may be 0 (nothing left for this GEMM).
static DenseGemm gemm_in(const lmoe_dims& d, const void* x, const void* W_down, const void* W_r, const float* bias,
                         const void* W_s1, void* z, float* logits, void* hs) {
    DenseGemm g{};
    const int L = (d.standard_moe || proj_8bit(d)) ? 0 : (int)d.l;  // latent columns here
    const int E = d.router_latent ? 0 : (int)d.E;       // router columns in this GEMM
    const int fs = shared_dense(d) ? (int)d.f_s : 0;
    g.M = (int)d.T;
    g.N = L + E + fs;
    g.nseg = 1;
    g.A[0] = x;
    g.lda[0] = d.d;
    g.K[0] = (int)d.d;
    g.ngroups = 0;
    if (L > 0) g.g[g.ngroups++] = NGroup{0, L, {W_down, nullptr}, EPI_STORE, z, d.l, nullptr};
    if (E > 0) g.g[g.ngroups++] = NGroup{L, L + E, {W_r, nullptr}, EPI_F32_BIAS, logits, d.E, bias};
    if (fs > 0) g.g[g.ngroups++] = NGroup{L + E, g.N, {W_s1, nullptr}, EPI_RELU2, hs, d.f_s, nullptr};
    return g;
}

// Latent router: z W_r^T (+ bias) -> logits, from the stored z.
static DenseGemm gemm_router(const lmoe_dims& d, const void* z, const void* W_r, const float* bias, float* logits) {
    DenseGemm g{};
    g.M = (int)d.T;
    g.N = (int)d.E;
    g.nseg = 1;
    g.A[0] = z;
    g.lda[0] = d.l;
    g.K[0] = (int)d.l;
    g.ngroups = 1;
    g.g[0] = NGroup{0, (int)d.E, {W_r, nullptr}, EPI_F32_BIAS, logits, d.E, bias};
    return g;
}

// [c | hs] [W_up | W_s2]^T -> out.  Standard MoE or FP8 up-projection: out
// (holding the routed result already) += hs W_s2^T.
static DenseGemm gemm_out(const lmoe_dims& d, const void* c, const void* hs, const void* W_up, const void* W_s2,
                          void* out) {
    DenseGemm g{};
    if (out_add_only(d)) {
        g.M = (int)d.T;
        g.N = (int)d.d;
        g.nseg = 1;
        g.A[0] = hs;
        g.lda[0] = d.f_s;
        g.K[0] = (int)d.f_s;
        g.ngroups = 1;
        g.g[0] = NGroup{0, (int)d.d, {W_s2, nullptr}, EPI_ADD, out, d.d, nullptr};
        return g;
    }
    const bool two = shared_dense(d);
    g.M = (int)d.T;
    g.N = (int)d.d;
    g.nseg = two ? 2 : 1;
    g.A[0] = c;
    g.lda[0] = d.l;
    g.K[0] = (int)d.l;
    if (two) {
        g.A[1] = hs;
        g.lda[1] = d.f_s;
        g.K[1] = (int)d.f_s;
    }
    g.ngroups = 1;
    g.g[0] = NGroup{0, (int)d.d, {W_up, two ? W_s2 : nullptr}, EPI_STORE, out, d.d, nullptr};
    return g;
}

struct Layout {
    size_t z, logits, idx, gate, counts, offsets, perm, inv, hist, tiles, tile_count, tile_start, ntiles, H, Y,
        c, hs, splitk, splitk_bytes, sk_part, sk_count, sk_count_len, q_x, s_x, q_h, s_h, q_c, s_c, mq_x, ms_x, mq_c,
        ms_c, arrive, total;
};

// Whether the few-rows expert GEMMs may take the split-K 64 x 128 tiles
// (64-row expert tiles, outputs at least 1024 wide): they then need the
// partial-sum buffer and one counter per work item.
static bool expert_split_k(const lmoe_dims& d) {
    return d.act_dtype == LMOE_BF16 && grouped_bm(d) == kSkBM && (d.f >= 1024 || d.l >= 1024);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static Layout plan(const lmoe_dims& d) {
    const size_t es = d.act_dtype == LMOE_BF16 ? 2 : 4;
    const size_t n = (size_t)d.T * (size_t)d.k;
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    L.z = take(d.standard_moe ? 0 : (size_t)d.T * d.l * es);
    L.logits = take((size_t)d.T * d.E * 4);
    L.idx = take(n * 4);
    L.gate = take(n * 4);
    L.counts = take((size_t)d.E * 4);
    L.offsets = take(((size_t)d.E + 1) * 4);
    L.perm = take(n * 4);
    L.inv = take(n * 4);
    L.hist = take((size_t)permute_nchunks((int64_t)n) * d.E * 4);
    L.tiles = take((size_t)max_tiles(d) * 16);
    L.tile_count = take(4);
    L.tile_start = take((size_t)d.E * 4);
    L.ntiles = take((size_t)d.E * 4);
    L.arrive = take(4);  // arrival counter of the decode router reduction that also permutes
    L.H = take(n * d.f * es);
    L.Y = take(n * d.l * es);
    L.c = take(d.standard_moe ? 0 : (size_t)d.T * d.l * es);
    L.hs = take((size_t)d.T * d.f_s * es);
    // fp32 split-K partials of the dense GEMMs of few-token (decode) calls
    // and of the split last round of many-token ones
    const size_t widest = (size_t)((max(d.l + d.E + d.f_s, d.d) + 3) / 4 * 4);
    if (d.act_dtype == LMOE_BF16 && d.T <= 64) {
        L.splitk_bytes = 16 * (size_t)d.T * widest * 4;
    } else if (d.act_dtype == LMOE_BF16) {
        const DenseGemm gi = gemm_in(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
        const size_t a = gi.N > 0 ? dense_tail_split_bytes(gi) : 0;
        const size_t b = (!out_add_only(d) || shared_dense(d))
                             ? dense_tail_split_bytes(gemm_out(d, nullptr, nullptr, nullptr, nullptr, nullptr))
                             : 0;
        const size_t r = d.router_latent ? dense_tail_split_bytes(gemm_router(d, nullptr, nullptr, nullptr, nullptr))
                                         : 0;
        L.splitk_bytes = a > b ? a : b;
        if (r > L.splitk_bytes) L.splitk_bytes = r;
    }
    L.splitk = take(L.splitk_bytes);
    if (shared_fp8(d) || proj_fp8(d)) {  // E4M3 codes and per-token scales of x
        L.q_x = take((size_t)d.T * d.d);
        L.s_x = take((size_t)d.T * 4);
    }
    if (shared_fp8(d)) {  // ... of hs
        L.q_h = take((size_t)d.T * d.f_s);
        L.s_h = take((size_t)d.T * 4);
    }
    if (proj_fp8(d)) {  // ... of c
        L.q_c = take((size_t)d.T * d.l);
        L.s_c = take((size_t)d.T * 4);
    }
    if (proj_mx(d)) {  // MXFP8 codes and block scales of x and c
        L.mq_x = take((size_t)d.T * d.d);
        L.ms_x = take((size_t)d.T * (d.d / 32));
        L.mq_c = take((size_t)d.T * d.l);
        L.ms_c = take((size_t)d.T * (d.l / 32));
    }
    if (expert_split_k(d)) {
        const int64_t widest_n = d.f > d.l ? d.f : d.l;
        L.sk_count_len = (size_t)(max_tiles(d) * ((widest_n + kSkBN - 1) / kSkBN));
        L.sk_count = take(L.sk_count_len * 4);
        L.sk_part = take(kSkPartialBytes);
    }
    L.total = o;
    return L;
}

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
    if (e == hipSuccess) return LMOE_OK;
    g_last_hip_error = (int)e;
    return LMOE_ERR_HIP;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!p) return LMOE_ERR_NULL;
    for (const void* p : ps)
        if (!aligned16(p)) return LMOE_ERR_ALIGN;
    return LMOE_OK;
}

static int check_optional(const void* p) { return (p && !aligned16(p)) ? LMOE_ERR_ALIGN : LMOE_OK; }

static int check_workspace(const lmoe_dims& d, const void* ws, size_t bytes) {
    if (!ws || bytes < plan(d).total) return LMOE_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return LMOE_ERR_ALIGN;
    return LMOE_OK;
}

static int check_experts(const lmoe_dims& d, const lmoe_experts* x) {
    if (!x) return LMOE_ERR_NULL;
    if (d.expert_dtype == LMOE_NVFP4 || d.expert_dtype == LMOE_NVFP4_2D)
        return check_ptrs({x->W1_codes, x->W1_scales, x->W1_ts, x->W2_codes, x->W2_scales, x->W2_ts});
    return check_ptrs({x->W1, x->W2});
}

// W_down or W_up as passed: a device array, or with FP8 projections a host
// lmoe_fp8_matrix naming the codes and the per-row scales.
static int check_proj(const lmoe_dims& d, const void* W) {
    if (!proj_8bit(d)) return check_ptrs({W});
    if (!W) return LMOE_ERR_NULL;
    if (proj_mx(d)) {
        const lmoe_mxfp8_matrix* m = (const lmoe_mxfp8_matrix*)W;
        return check_ptrs({m->codes, m->scales});
    }
    const lmoe_fp8_matrix* m = (const lmoe_fp8_matrix*)W;
    return check_ptrs({m->codes, m->scales});
}

static int check_shared(const lmoe_dims& d, const lmoe_shared* sh) {
    if ((sh != nullptr) != (d.f_s > 0)) return LMOE_ERR_SHAPE;
    if (sh && shared_fp8(d)) return check_ptrs({sh->W_s1, sh->W_s2, sh->W_s1_scale, sh->W_s2_scale});
    if (sh) return check_ptrs({sh->W_s1, sh->W_s2});
    return LMOE_OK;
}

#define LMOE_TRY(expr)              \
    do {                            \
        const int st_ = (expr);     \
        if (st_ != LMOE_OK) return st_; \
    } while (0)

static TileTable tile_table(const lmoe_dims& d, char* ws, const Layout& L) {
    TileTable tt;
    tt.tile_count = (const int*)(ws + L.tile_count);
    tt.tiles = (const int4*)(ws + L.tiles);
    tt.expert_tile_start = (const int*)(ws + L.tile_start);
    tt.expert_ntiles = (const int*)(ws + L.ntiles);
    tt.max_tiles = (int)max_tiles(d);
    tt.bm = grouped_bm(d);
    tt.sk_count = L.sk_count_len ? (int*)(ws + L.sk_count) : nullptr;
    tt.sk_count_len = (int)L.sk_count_len;
    return tt;
}

// ---- the steps, shared by the fused and the staged entry points --------

// pf (the fused forward's permutation outputs, or null): with few tokens the
// router reduction also permutes the pairs, and *perm_done says so.
static hipError_t run_project_route(const lmoe_dims& d, const void* x, const void* W_down, const void* W_r,
                                    const float* bias, const lmoe_shared* sh, void* z, float* logits,
                                    int32_t* idx, float* gate, void* hs, char* ws, const Layout& L,
                                    hipStream_t s, const PermFused* pf = nullptr, bool* perm_done = nullptr) {
    if (perm_done) *perm_done = false;
    const DenseGemm g = gemm_in(d, x, W_down, W_r, bias, sh ? sh->W_s1 : nullptr, z, logits, hs);
    hipError_t e = hipSuccess;
    // Few tokens with the router in d: the top-k is taken in this GEMM's
    // split-K reduction, from the logits columns (after the latent ones).
    const bool route_fused = !d.router_latent && d.act_dtype == LMOE_BF16 &&
                             dense_topk_fusable(g, L.splitk_bytes, (int)d.E, (int)d.k);
    if (route_fused) {
        const int lc0 = (d.standard_moe || proj_8bit(d)) ? 0 : (int)d.l;
        e = launch_dense_gemm_topk_bf16(g, ws + L.splitk, L.splitk_bytes, lc0, (int)d.E, bias, (int)d.k, idx, gate,
                                        pf, s);
        if (pf && perm_done) *perm_done = e == hipSuccess;
    } else if (g.N > 0) {
        e = launch_dense_gemm(g, d.act_dtype, (int)d.T, ws + L.splitk, L.splitk_bytes, s);
    }
    if (e != hipSuccess) return e;
    uint8_t* qx = (uint8_t*)(ws + L.q_x);
    float* sx = (float*)(ws + L.s_x);
    if (shared_fp8(d) || proj_fp8(d)) {
        e = launch_quantize_rows_fp8((const uint16_t*)x, d.T, (int)d.d, d.d, qx, sx, s);
        if (e != hipSuccess) return e;
    }
    if (proj_fp8(d)) {  // z = s_x * (q_x W_down^T) * s_down
        const lmoe_fp8_matrix* W = (const lmoe_fp8_matrix*)W_down;
        e = launch_fp8_gemm(Fp8Gemm{(int)d.T, (int)d.l, (int)d.d, qx, d.d, sx, W->codes, d.d, W->scales, EPI_STORE,
                                    (uint16_t*)z, d.l},
                            ws + L.splitk, L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (proj_mx(d)) {  // z = MX(x) MX(W_down)^T
        uint8_t* mq = (uint8_t*)(ws + L.mq_x);
        uint8_t* ms = (uint8_t*)(ws + L.ms_x);
        e = launch_quantize_blocks_mxfp8((const uint16_t*)x, d.T, (int)d.d, d.d, mq, ms, s);
        if (e != hipSuccess) return e;
        const lmoe_mxfp8_matrix* W = (const lmoe_mxfp8_matrix*)W_down;
        e = launch_fp8_gemm(Fp8Gemm{(int)d.T, (int)d.l, (int)d.d, mq, d.d, nullptr, W->codes, d.d, nullptr,
                                    EPI_STORE, (uint16_t*)z, d.l, ms, W->scales},
                            ws + L.splitk, L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (d.router_latent) {
        e = launch_dense_gemm(gemm_router(d, z, W_r, bias, logits), d.act_dtype, (int)d.T, ws + L.splitk,
                              L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (shared_fp8(d)) {  // hs = relu(s_x * (q_x W_s1^T) * s_w1)^2
        Fp8Gemm f{};
        f.M = (int)d.T;
        f.N = (int)d.f_s;
        f.K = (int)d.d;
        f.A = qx;
        f.lda = d.d;
        f.a_scale = sx;
        f.B = (const uint8_t*)sh->W_s1;
        f.ldb = d.d;
        f.b_scale = sh->W_s1_scale;
        f.epi = EPI_RELU2;
        f.C = (uint16_t*)hs;
        f.ldc = d.f_s;
        e = launch_fp8_gemm(f, ws + L.splitk, L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (route_fused) return hipSuccess;
    return launch_topk_softmax(logits, (int)d.T, (int)d.E, (int)d.k, idx, gate, s);
}

static hipError_t run_experts(const lmoe_dims& d, const void* z, const int32_t* perm, const lmoe_experts* ex,
                              void* H, void* Y, const TileTable& tt, char* ws, const Layout& L, hipStream_t s) {
    GroupedGemm g1{};
    g1.N = (int)d.f;
    g1.K = (int)d.l;
    g1.tt = tt;
    g1.A = z;
    g1.lda = d.l;
    g1.a_row_map = perm;
    g1.a_row_div = (int)d.k;
    g1.n_rows = (int)(d.T * d.k);
    g1.b_fmt = d.expert_dtype;
    g1.B = ex->W1;
    g1.B_codes = ex->W1_codes;
    g1.B_scales = ex->W1_scales;
    g1.B_ts = ex->W1_ts;
    g1.epi = EPI_RELU2;
    g1.C = H;
    g1.ldc = d.f;
    g1.sk_part = L.sk_count_len ? (float*)(ws + L.sk_part) : nullptr;
    hipError_t e = launch_grouped_gemm(g1, d.act_dtype, s);
    if (e != hipSuccess) return e;

    GroupedGemm g2 = g1;
    g2.N = (int)d.l;
    g2.K = (int)d.f;
    g2.A = H;
    g2.lda = d.f;
    g2.a_row_map = nullptr;
    g2.a_row_div = 1;
    g2.B = ex->W2;
    g2.B_codes = ex->W2_codes;
    g2.B_scales = ex->W2_scales;
    g2.B_ts = ex->W2_ts;
    g2.epi = EPI_STORE;
    g2.C = Y;
    g2.ldc = d.l;
    return launch_grouped_gemm(g2, d.act_dtype, s);
}

// c_opt: the caller's c, or NULL.  A standard MoE combines straight into
// out (then copied to c_opt if given) and adds the shared expert there.
static hipError_t run_combine_up(const lmoe_dims& d, const void* Y, const int32_t* inv, const float* gate,
                                 const void* W_up, const lmoe_shared* sh, const void* hs, void* c_opt, void* out,
                                 char* ws, const Layout& L, hipStream_t s) {
    void* c = d.standard_moe ? out : (c_opt ? c_opt : ws + L.c);
    hipError_t e = launch_combine(Y, inv, gate, (int)d.T, (int)d.k, (int)d.l, d.act_dtype, c, s);
    if (e != hipSuccess) return e;
    if (d.standard_moe && c_opt) {
        const size_t es = d.act_dtype == LMOE_BF16 ? 2 : 4;
        e = hipMemcpyAsync(c_opt, out, (size_t)d.T * d.l * es, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return e;
    }
    if (proj_fp8(d)) {  // out = s_c * (q_c W_up^T) * s_up, from c as stored
        uint8_t* qc = (uint8_t*)(ws + L.q_c);
        float* sc = (float*)(ws + L.s_c);
        e = launch_quantize_rows_fp8((const uint16_t*)c, d.T, (int)d.l, d.l, qc, sc, s);
        if (e != hipSuccess) return e;
        const lmoe_fp8_matrix* W = (const lmoe_fp8_matrix*)W_up;
        e = launch_fp8_gemm(Fp8Gemm{(int)d.T, (int)d.d, (int)d.l, qc, d.l, sc, W->codes, d.l, W->scales, EPI_STORE,
                                    (uint16_t*)out, d.d},
                            ws + L.splitk, L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (proj_mx(d)) {  // out = MX(c) MX(W_up)^T, from c as stored
        uint8_t* mq = (uint8_t*)(ws + L.mq_c);
        uint8_t* ms = (uint8_t*)(ws + L.ms_c);
        e = launch_quantize_blocks_mxfp8((const uint16_t*)c, d.T, (int)d.l, d.l, mq, ms, s);
        if (e != hipSuccess) return e;
        const lmoe_mxfp8_matrix* W = (const lmoe_mxfp8_matrix*)W_up;
        e = launch_fp8_gemm(Fp8Gemm{(int)d.T, (int)d.d, (int)d.l, mq, d.l, nullptr, W->codes, d.l, nullptr,
                                    EPI_STORE, (uint16_t*)out, d.d, ms, W->scales},
                            ws + L.splitk, L.splitk_bytes, s);
        if (e != hipSuccess) return e;
    }
    if (!out_add_only(d) || shared_dense(d)) {
        const DenseGemm g = gemm_out(d, c, hs, W_up, sh ? sh->W_s2 : nullptr, out);
        e = launch_dense_gemm(g, d.act_dtype, (int)d.T, ws + L.splitk, L.splitk_bytes, s);
    }
    if (e != hipSuccess || !shared_fp8(d)) return e;
    // out += s_h * (q_h W_s2^T) * s_w2, added to the bf16 up-projection
    uint8_t* qh = (uint8_t*)(ws + L.q_h);
    float* sh_scale = (float*)(ws + L.s_h);
    e = launch_quantize_rows_fp8((const uint16_t*)hs, d.T, (int)d.f_s, d.f_s, qh, sh_scale, s);
    if (e != hipSuccess) return e;
    Fp8Gemm f{};
    f.M = (int)d.T;
    f.N = (int)d.d;
    f.K = (int)d.f_s;
    f.A = qh;
    f.lda = d.f_s;
    f.a_scale = sh_scale;
    f.B = (const uint8_t*)sh->W_s2;
    f.ldb = d.f_s;
    f.b_scale = sh->W_s2_scale;
    f.epi = EPI_ADD;
    f.C = (uint16_t*)out;
    f.ldc = d.d;
    return launch_fp8_gemm(f, ws + L.splitk, L.splitk_bytes, s);
}

}  // namespace lmoe

using namespace lmoe;

// ---- the allocation-free forward's workspace ------------------------------
// One array per GPU the library runs on, held until the process ends.  In
// host code its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
static __device__ __align__(256) unsigned char scratch[LMOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (hipGetSymbolAddress on its first use
// on that device).
hipError_t static_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" {

int lmoe_validate_dims(const lmoe_dims* d) {
    if (!d) return LMOE_ERR_NULL;
    if (d->T < 1 || d->T > (1 << 24)) return LMOE_ERR_SHAPE;
    if (d->d < 256 || d->d % 256 != 0 || d->d > 65536) return LMOE_ERR_SHAPE;
    if (d->standard_moe != 0 && d->standard_moe != 1) return LMOE_ERR_SHAPE;
    if (d->standard_moe ? (d->l != d->d || d->router_latent != 0) : d->l * 4 != d->d) return LMOE_ERR_SHAPE;
    if (d->E < 1 || d->E > 1024) return LMOE_ERR_SHAPE;
    if (d->k < 1 || d->k > d->E) return LMOE_ERR_SHAPE;
    if (d->router_latent != 0 && d->router_latent != 1) return LMOE_ERR_SHAPE;
    if (d->f < 64 || d->f % 64 != 0 || d->f > 65536) return LMOE_ERR_SHAPE;
    if (d->f_s < 0 || d->f_s % 64 != 0 || d->f_s > 262144) return LMOE_ERR_SHAPE;
    if (d->T * d->k > (int64_t)1 << 30) return LMOE_ERR_SHAPE;
    if (d->act_dtype == LMOE_F32) {
        if (d->expert_dtype != LMOE_F32) return LMOE_ERR_DTYPE;
        if (max_tiles(*d) > 65535) return LMOE_ERR_SHAPE;  // grid.y of the fp32 grouped kernel
    } else if (d->act_dtype == LMOE_BF16) {
        if (d->expert_dtype != LMOE_BF16 && d->expert_dtype != LMOE_BF16_TILED && d->expert_dtype != LMOE_NVFP4 &&
            d->expert_dtype != LMOE_NVFP4_2D)
            return LMOE_ERR_DTYPE;
    } else {
        return LMOE_ERR_DTYPE;
    }
    if (d->shared_dtype != d->act_dtype && !(d->act_dtype == LMOE_BF16 && d->shared_dtype == LMOE_FP8_E4M3))
        return LMOE_ERR_DTYPE;
    if (d->shared_dtype == LMOE_FP8_E4M3 && d->f_s % 128 != 0) return LMOE_ERR_SHAPE;  // fp8 K step
    if (d->proj_dtype != d->act_dtype &&
        !(d->act_dtype == LMOE_BF16 && (d->proj_dtype == LMOE_FP8_E4M3 || d->proj_dtype == LMOE_MXFP8) &&
          d->standard_moe == 0))
        return LMOE_ERR_DTYPE;
    if ((d->proj_dtype == LMOE_FP8_E4M3 || d->proj_dtype == LMOE_MXFP8) && d->l % 128 != 0)
        return LMOE_ERR_SHAPE;  // fp8 K step of W_up
    return LMOE_OK;
}

size_t lmoe_workspace_bytes(const lmoe_dims* d) {
    if (lmoe_validate_dims(d) != LMOE_OK) return 0;
    return plan(*d).total;
}

const char* lmoe_strerror(int st) {
    switch (st) {
        case LMOE_OK: return "ok";
        case LMOE_ERR_NULL: return "a required pointer is NULL";
        case LMOE_ERR_SHAPE: return "a size is out of range";
        case LMOE_ERR_DTYPE: return "unsupported dtype or dtype combination";
        case LMOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LMOE_ERR_WORKSPACE: return "workspace missing or too small";
        case LMOE_ERR_HIP: return "a HIP launch failed";
        default: return "unknown status";
    }
}

int lmoe_last_hip_error(void) { return g_last_hip_error; }

int lmoe_pack_expert_weights(int64_t E, int64_t rows, int64_t cols, const void* W, void* packed, void* stream) {
    if (E < 1 || E > 1024 || rows < 64 || rows % 64 != 0 || cols < 64 || cols % 64 != 0 || rows > 65536 ||
        cols > 65536)
        return LMOE_ERR_SHAPE;
    LMOE_TRY(check_ptrs({W, packed}));
    const uintptr_t a = (uintptr_t)W, b = (uintptr_t)packed, n = (uintptr_t)(E * rows * cols * 2);
    if (a < b + n && b < a + n) return LMOE_ERR_SHAPE;  // overlapping buffers
    return hip_status(launch_pack_experts(W, packed, E, (int)rows, (int)cols, (hipStream_t)stream));
}

int lmoe_quantize_rows_fp8(int64_t rows, int64_t cols, const void* src, uint8_t* codes, float* scales,
                           void* stream) {
    if (rows < 1 || rows > ((int64_t)1 << 31) || cols < 8 || cols % 8 != 0 || cols > (1 << 20))
        return LMOE_ERR_SHAPE;
    LMOE_TRY(check_ptrs({src, codes, scales}));
    return hip_status(launch_quantize_rows_fp8((const uint16_t*)src, rows, (int)cols, cols, codes, scales,
                                               (hipStream_t)stream));
}

int lmoe_quantize_rows_mxfp8(int64_t rows, int64_t cols, const void* src, uint8_t* codes, uint8_t* scales,
                             void* stream) {
    if (rows < 1 || rows > ((int64_t)1 << 31) || cols < 32 || cols % 32 != 0 || cols > (1 << 20))
        return LMOE_ERR_SHAPE;
    LMOE_TRY(check_ptrs({src, codes, scales}));
    return hip_status(launch_quantize_blocks_mxfp8((const uint16_t*)src, rows, (int)cols, cols, codes, scales,
                                                   (hipStream_t)stream));
}

int latentmoe_forward(const lmoe_dims* dims, const void* x, const void* W_down, const void* W_router,
                      const float* router_bias, const lmoe_experts* experts, const void* W_up,
                      const lmoe_shared* shared, int k, void* out, void* workspace, size_t workspace_bytes,
                      const lmoe_debug* dbg, void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    const lmoe_dims& d = *dims;
    if (k != d.k) return LMOE_ERR_SHAPE;
    LMOE_TRY(check_ptrs({x, W_router, out}));
    if (!d.standard_moe) {
        LMOE_TRY(check_proj(d, W_down));
        LMOE_TRY(check_proj(d, W_up));
    }
    LMOE_TRY(check_optional(router_bias));
    LMOE_TRY(check_experts(d, experts));
    LMOE_TRY(check_shared(d, shared));
    lmoe_debug dv{};
    if (dbg) dv = *dbg;
    LMOE_TRY(check_optional(dv.z));
    LMOE_TRY(check_optional(dv.logits));
    LMOE_TRY(check_optional(dv.topk_idx));
    LMOE_TRY(check_optional(dv.topk_gate));
    LMOE_TRY(check_optional(dv.counts));
    LMOE_TRY(check_optional(dv.offsets));
    LMOE_TRY(check_optional(dv.perm));
    LMOE_TRY(check_optional(dv.inv));
    LMOE_TRY(check_optional(dv.c));
    // the workspace is checked last in every entry point
    LMOE_TRY(check_workspace(d, workspace, workspace_bytes));

    char* ws = (char*)workspace;
    const Layout L = plan(d);
    hipStream_t s = (hipStream_t)stream;
    const void* z = d.standard_moe ? x : (dv.z ? dv.z : ws + L.z);
    float* logits = dv.logits ? dv.logits : (float*)(ws + L.logits);
    int32_t* idx = dv.topk_idx ? dv.topk_idx : (int32_t*)(ws + L.idx);
    float* gate = dv.topk_gate ? dv.topk_gate : (float*)(ws + L.gate);
    int32_t* counts = dv.counts ? dv.counts : (int32_t*)(ws + L.counts);
    int32_t* offsets = dv.offsets ? dv.offsets : (int32_t*)(ws + L.offsets);
    int32_t* perm = dv.perm ? dv.perm : (int32_t*)(ws + L.perm);
    int32_t* inv = dv.inv ? dv.inv : (int32_t*)(ws + L.inv);
    void* hs = ws + L.hs;
    const TileTable tt = tile_table(d, ws, L);

    const PermFused pf{counts, offsets, perm, inv, tt, (int*)(ws + L.arrive)};
    bool perm_done = false;
    hipError_t e = run_project_route(d, x, W_down, W_router, router_bias, shared, (void*)z, logits, idx, gate, hs,
                                     ws, L, s, &pf, &perm_done);
    if (e == hipSuccess && !perm_done)
        e = launch_permute(idx, d.T * d.k, (int)d.E, (int32_t*)(ws + L.hist), counts, offsets, perm, inv, &tt, s);
    if (e == hipSuccess) e = run_experts(d, z, perm, experts, ws + L.H, ws + L.Y, tt, ws, L, s);
    if (e == hipSuccess) e = run_combine_up(d, ws + L.Y, inv, gate, W_up, shared, hs, dv.c, out, ws, L, s);
    return hip_status(e);
}

int lmoe_project_route(const lmoe_dims* dims, const void* x, const void* W_down, const void* W_router,
                       const float* router_bias, const lmoe_shared* shared, void* z, float* logits,
                       int32_t* topk_idx, float* topk_gate, void* hs, void* workspace, size_t workspace_bytes,
                       void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    const lmoe_dims& d = *dims;
    LMOE_TRY(check_ptrs({x, W_router, logits, topk_idx, topk_gate}));
    if (!d.standard_moe) {  // a standard MoE has no z of its own
        LMOE_TRY(check_ptrs({z}));
        LMOE_TRY(check_proj(d, W_down));
    }
    LMOE_TRY(check_optional(router_bias));
    LMOE_TRY(check_shared(d, shared));
    if (shared) LMOE_TRY(check_ptrs({hs}));
    LMOE_TRY(check_workspace(d, workspace, workspace_bytes));
    const Layout L = plan(d);
    return hip_status(run_project_route(d, x, W_down, W_router, router_bias, shared, z, logits, topk_idx,
                                        topk_gate, hs, (char*)workspace, L, (hipStream_t)stream));
}

int lmoe_permute(const lmoe_dims* dims, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv, void* workspace, size_t workspace_bytes, void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    const lmoe_dims& d = *dims;
    LMOE_TRY(check_ptrs({topk_idx, counts, offsets, perm, inv}));
    LMOE_TRY(check_workspace(d, workspace, workspace_bytes));
    char* ws = (char*)workspace;
    const Layout L = plan(d);
    return hip_status(launch_permute(topk_idx, d.T * d.k, (int)d.E, (int32_t*)(ws + L.hist), counts, offsets,
                                     perm, inv, nullptr, (hipStream_t)stream));
}

int lmoe_experts_ffn(const lmoe_dims* dims, const void* z, const int32_t* offsets, const int32_t* perm,
                     const lmoe_experts* experts, void* Y, void* workspace, size_t workspace_bytes, void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    const lmoe_dims& d = *dims;
    LMOE_TRY(check_ptrs({z, offsets, perm, Y}));
    LMOE_TRY(check_experts(d, experts));
    LMOE_TRY(check_workspace(d, workspace, workspace_bytes));
    char* ws = (char*)workspace;
    const Layout L = plan(d);
    const TileTable tt = tile_table(d, ws, L);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_build_tiles(offsets, (int)d.E, tt, s);
    if (e == hipSuccess) e = run_experts(d, z, perm, experts, ws + L.H, Y, tt, ws, L, s);
    return hip_status(e);
}

int lmoe_combine_up(const lmoe_dims* dims, const void* Y, const int32_t* inv, const float* topk_gate,
                    const void* W_up, const lmoe_shared* shared, const void* hs, void* c, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    const lmoe_dims& d = *dims;
    LMOE_TRY(check_ptrs({Y, inv, topk_gate, out}));
    if (!d.standard_moe) LMOE_TRY(check_proj(d, W_up));
    LMOE_TRY(check_shared(d, shared));
    if (shared) LMOE_TRY(check_ptrs({hs}));
    LMOE_TRY(check_optional(c));
    LMOE_TRY(check_workspace(d, workspace, workspace_bytes));
    char* ws = (char*)workspace;
    const Layout L = plan(d);
    return hip_status(run_combine_up(d, Y, inv, topk_gate, W_up, shared, hs, c, out, ws, L, (hipStream_t)stream));
}

struct lmoe_ctx {
    int device;
    void* ws;
    size_t bytes;
};

int lmoe_create(lmoe_ctx** ctx, int device) {
    if (!ctx) return LMOE_ERR_NULL;
    *ctx = nullptr;
    int count = 0;
    const hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return hip_status(e);
    if (device < 0 || device >= count) return hip_status(hipErrorInvalidDevice);
    lmoe_ctx* c = new (std::nothrow) lmoe_ctx{device, nullptr, 0};
    if (!c) return hip_status(hipErrorOutOfMemory);
    *ctx = c;
    return LMOE_OK;
}

int lmoe_destroy(lmoe_ctx* ctx) {
    if (!ctx) return LMOE_OK;
    hipError_t e = hipSuccess;
    if (ctx->ws) e = hipFree(ctx->ws);
    delete ctx;
    return hip_status(e);
}

int lmoe_ctx_reserve(lmoe_ctx* ctx, const lmoe_dims* dims) {
    if (!ctx) return LMOE_ERR_NULL;
    LMOE_TRY(lmoe_validate_dims(dims));
    const size_t need = plan(*dims).total;
    if (need <= ctx->bytes) return LMOE_OK;
    // the new buffer first: if it cannot be had, the context keeps the old one
    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    const bool other = e == hipSuccess && prev != ctx->device;
    if (other) e = hipSetDevice(ctx->device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipMalloc(&p, need);
    if (e == hipSuccess) {
        if (ctx->ws) e = hipFree(ctx->ws);
        ctx->ws = p;
        ctx->bytes = need;
    }
    if (other) (void)hipSetDevice(prev);
    return hip_status(e);
}

size_t lmoe_ctx_workspace_bytes(const lmoe_ctx* ctx) { return ctx ? ctx->bytes : 0; }

int lmoe_static_forward(const lmoe_dims* dims, const void* x, const void* W_down, const void* W_router,
                        const float* router_bias, const lmoe_experts* experts, const void* W_up,
                        const lmoe_shared* shared, int k, void* out, const lmoe_debug* dbg, void* stream) {
    LMOE_TRY(lmoe_validate_dims(dims));
    if (plan(*dims).total > (size_t)LMOE_STATIC_SCRATCH_BYTES) return LMOE_ERR_WORKSPACE;
    void* ws = nullptr;
    const hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
    return latentmoe_forward(dims, x, W_down, W_router, router_bias, experts, W_up, shared, k, out, ws,
                             (size_t)LMOE_STATIC_SCRATCH_BYTES, dbg, stream);
}

int lmoe_ctx_forward(lmoe_ctx* ctx, const lmoe_dims* dims, const void* x, const void* W_down, const void* W_router,
                     const float* router_bias, const lmoe_experts* experts, const void* W_up,
                     const lmoe_shared* shared, int k, void* out, const lmoe_debug* dbg, void* stream) {
    if (!ctx) return LMOE_ERR_NULL;
    int cur = -1;
    const hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    if (cur != ctx->device) return hip_status(hipErrorInvalidDevice);
    return latentmoe_forward(dims, x, W_down, W_router, router_bias, experts, W_up, shared, k, out, ctx->ws,
                             ctx->bytes, dbg, stream);
}

}  // extern "C"
