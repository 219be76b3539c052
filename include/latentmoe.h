/*
 * latentmoe.h -- C ABI of the LatentMoE layer forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (Nemotron 3 overview article, section 2.2 "LatentMoE", steps 1-3
 * and the paragraph after its comparison table; Nemotron 3 Super blog,
 * section "Latent MoE"; Nemotron 3 Ultra release news, architecture
 * paragraph):
 *
 *   z_t   = W_down x_t                      hidden d -> latent l = d/4
 *   s_t   = W_r x_t + b                     router logits over E experts (reads x in d),
 *     or  W_r z_t + b                       with dims.router_latent (reads the latent z)
 *   I_t   = top-k of s_t, ordered (logit desc, expert id asc)
 *   g_t   = softmax over the k selected logits
 *   y_tj  = W2_e (max(0, W1_e z_t))^2       routed expert e = I_t[j], ReLU^2 FFN in l
 *   c_t   = sum_j g_tj y_tj                 combine in the latent space
 *   out_t = W_up c_t  [+ W_s2 (max(0, W_s1 x_t))^2]   back to d, optional shared expert in d
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *     never frees, keeps or reallocates it after the call returns, and it
 *     never allocates device memory itself: scratch comes from the caller's
 *     workspace (see lmoe_workspace_bytes).
 *   - Weights are stored out x in, row-major (fan-in contiguous):
 *       W_down [l][d], W_r [E][d] ([E][l] with dims.router_latent),
 *       W1 [E][f][l], W2 [E][l][f], W_up [d][l], W_s1 [f_s][d], W_s2 [d][f_s].
 *       x and out are [T][d] row-major.
 *   - Activation dtype (dims.act_dtype) is the storage type of x, W_down,
 *     W_r, W_up, W_s1, W_s2, out and of the latent intermediates.  Every
 *     product accumulates in fp32.  Router logits and gates are fp32.
 *   - Calls are asynchronous: kernels are enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and the call returns without a
 *     host synchronisation.  Device faults surface at the caller's next
 *     synchronisation.
 *   - Errors are returned as negative codes, and are detected on the host
 *     before anything is enqueued: on error no output is touched.  A launch
 *     failure returns LMOE_ERR_HIP (detail: lmoe_last_hip_error()).
 *   - Pointers must be 16-byte aligned.  NaN/Inf inputs give undefined
 *     outputs.  Calls that share a workspace must not run concurrently.
 */
#ifndef LATENTMOE_H
#define LATENTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define LMOE_OK             0
#define LMOE_ERR_NULL      -1  /* a required pointer is NULL */
#define LMOE_ERR_SHAPE     -2  /* a size is out of range (see lmoe_dims) */
#define LMOE_ERR_DTYPE     -3  /* unknown dtype or unsupported combination */
#define LMOE_ERR_ALIGN     -4  /* a pointer is not 16-byte aligned */
#define LMOE_ERR_WORKSPACE -5  /* workspace missing or smaller than lmoe_workspace_bytes */
#define LMOE_ERR_HIP       -6  /* a HIP launch failed */

/* ---- dtypes ---------------------------------------------------------- */
#define LMOE_F32   0  /* IEEE binary32 */
#define LMOE_BF16  1  /* bfloat16 */
#define LMOE_NVFP4 2  /* routed-expert weights only, see lmoe_experts */
#define LMOE_BF16_TILED 3  /* routed-expert bf16 weights in the tiled layout, see lmoe_pack_expert_weights */
#define LMOE_FP8_E4M3 4    /* shared-expert and projection weights, see lmoe_shared, lmoe_fp8_matrix */
#define LMOE_NVFP4_2D 5    /* routed-expert weights only: NVFP4 with 16 x 16 scale blocks, see lmoe_experts */
#define LMOE_MXFP8 6       /* projection weights only: OCP MXFP8, see lmoe_mxfp8_matrix */

/*
 * Layer sizes.  Constraints (LMOE_ERR_SHAPE otherwise):
 *   T >= 1 tokens; d >= 256 and d % 256 == 0; l == d / 4 (latent width,
 *   overview section 2.2 step 1); 1 <= E <= 1024 experts; 1 <= k <= E;
 *   f >= 64 and f % 64 == 0; f_s == 0 (no shared expert) or f_s % 64 == 0.
 * Dtypes (LMOE_ERR_DTYPE otherwise):
 *   act_dtype LMOE_F32 with expert_dtype LMOE_F32, or
 *   act_dtype LMOE_BF16 with expert_dtype LMOE_BF16, LMOE_BF16_TILED,
 *   LMOE_NVFP4 or LMOE_NVFP4_2D.
 * router_latent (0 or 1, LMOE_ERR_SHAPE otherwise): 0 = the router reads x in
 *   d, W_r [E][d] (the overview's paragraph after the section 2.2 table keeps
 *   the gate in d); 1 = the router reads the latent z as stored (act dtype),
 *   W_r [E][l] (overview section 2.2 step 2 and the Super blog, "Latent
 *   MoE", place routing in the latent space).
 * shared_dtype: the shared expert's weight format, the activation dtype or,
 *   with bf16 activations, LMOE_FP8_E4M3 (the Ultra release news lists FP8
 *   shared experts; see lmoe_shared; f_s must then be a multiple of 128).
 *   LMOE_ERR_DTYPE otherwise; it is checked even when f_s == 0.
 * standard_moe (0 or 1): 1 runs the same kernels as a standard MoE layer,
 *   the comparison point of the overview's section 2.2 table (128 experts,
 *   top-6, experts in the hidden width): no down- or up-projection, l == d
 *   (instead of d/4), routed experts W1 [E][f][d], W2 [E][d][f], z = x and
 *   out = c (+ shared expert); router_latent must be 0.  W_down and W_up are
 *   then ignored and may be NULL.  LMOE_ERR_SHAPE when violated.
 * proj_dtype: the down- and up-projection weight format, the activation
 *   dtype or, with bf16 activations and standard_moe = 0, LMOE_FP8_E4M3
 *   (LMOE_ERR_DTYPE otherwise): then the W_down and W_up arguments each
 *   point to an lmoe_fp8_matrix, l must be a multiple of 128
 *   (LMOE_ERR_SHAPE), and each projection quantises its input per token as
 *   lmoe_quantize_rows_fp8 does (x before W_down; the combined latent c, as
 *   stored in bf16, before W_up) and runs as an fp8 x fp8 MFMA GEMM with
 *   fp32 accumulation; z and out stay bf16.  The router and the expert FFNs
 *   are unchanged.  LMOE_MXFP8 (the Ultra model card's "Model design" names
 *   MXFP8 for the latent projections) works the same way with OCP MXFP8
 *   blocks instead: W_down and W_up point to lmoe_mxfp8_matrix, and x and c
 *   are quantised as lmoe_quantize_rows_mxfp8 does; the scaled fp8 MFMA
 *   applies the block scales.
 */
typedef struct lmoe_dims {
    int64_t T, d, l, E, k, f, f_s;
    int32_t act_dtype;
    int32_t expert_dtype;
    int32_t router_latent;
    int32_t shared_dtype;
    int32_t standard_moe;
    int32_t proj_dtype;
} lmoe_dims;

/*
 * An E4M3 weight matrix [rows][cols] with one scale per output row (weight
 * = E4M3(code) * scale): codes [rows][cols] uint8 and scales [rows] fp32,
 * both device memory, 16-byte aligned.  The struct itself is host memory,
 * read during the call.  Used for W_down [l][d] and W_up [d][l] with
 * dims.proj_dtype = LMOE_FP8_E4M3.
 */
typedef struct lmoe_fp8_matrix {
    const uint8_t* codes;
    const float* scales;
} lmoe_fp8_matrix;

/*
 * An MXFP8 weight matrix [rows][cols] (OCP microscaling: E4M3 elements, one
 * E8M0 scale 2^(s - 127) per 32 consecutive elements of a row): codes
 * [rows][cols] uint8 and scales [rows][cols/32] uint8, both device memory,
 * 16-byte aligned; the struct itself is host memory, read during the call.
 * Used for W_down and W_up with dims.proj_dtype = LMOE_MXFP8.
 */
typedef struct lmoe_mxfp8_matrix {
    const uint8_t* codes;
    const uint8_t* scales;
} lmoe_mxfp8_matrix;

/*
 * Routed-expert weights.  Dense formats (F32/BF16) use W1 [E][f][l] and
 * W2 [E][l][f] in the activation dtype.  NVFP4 (overview section 3.1.1,
 * NVFP4 format: E2M1 elements in 16-element micro-blocks with an E4M3 block
 * scale; the Ultra release news, quantisation paragraph: 4-bit weights run
 * against 16-bit activations) uses, per matrix M in {W1, W2} of shape
 * [E][rows][K]:
 *   M_codes  [E][rows][K/2] uint8: E2M1 codes, element 2i in the low nibble
 *                                  and 2i+1 in the high nibble;
 *   M_scales [E][rows][K/16] uint8: E4M3 (FN) scale of each 16-element block
 *                                   along K;
 *   M_ts     [E] fp32: per-expert tensor scale.
 * The weight is w = E2M1(code) * E4M3(scale) * ts.  LMOE_NVFP4_2D (the Ultra
 * release news: weights quantised in two-dimensional blocks) shares one
 * scale among 16 rows x 16 elements: M_scales [E][rows/16][K/16], the
 * weight in row r and column c taking scale [r/16][c/16]; codes and ts as
 * above.  LMOE_BF16_TILED uses
 * W1 and W2 as written by lmoe_pack_expert_weights from the BF16 stacks (the
 * same values; results are identical to passing the BF16 stacks).  Unused
 * fields are ignored.
 */
typedef struct lmoe_experts {
    const void* W1;
    const void* W2;
    const uint8_t* W1_codes;
    const uint8_t* W1_scales;
    const float* W1_ts;
    const uint8_t* W2_codes;
    const uint8_t* W2_scales;
    const float* W2_ts;
} lmoe_experts;

/* Shared expert in d (overview section 2.2, paragraph after the table):
 * W_s1 [f_s][d], W_s2 [d][f_s] in the activation dtype.  Pass NULL to the
 * entry points (and f_s = 0) for a layer without one.
 * With dims.shared_dtype = LMOE_FP8_E4M3, W_s1 and W_s2 are E4M3 (FN) codes,
 * one byte per weight, with one fp32 scale per output row: W_s1_scale [f_s],
 * W_s2_scale [d] (weight = E4M3(code) * scale).  The shared expert's inputs
 * are then quantised per token as lmoe_quantize_rows_fp8 does (x before the
 * first matrix, the hidden layer hs before the second) and both products run
 * as fp8 x fp8 MFMA GEMMs with fp32 accumulation; hs stays bf16 in between,
 * and the second product is added to the bf16 up-projection output.  The
 * scale fields are ignored for bf16 weights. */
typedef struct lmoe_shared {
    const void* W_s1;
    const void* W_s2;
    const float* W_s1_scale;
    const float* W_s2_scale;
} lmoe_shared;

/*
 * Optional views of the intermediates of latentmoe_forward.  Each non-NULL
 * field is used as the storage of that intermediate (no extra copy); NULL
 * fields live in the workspace.
 *   z [T][l] act dtype; logits [T][E] fp32 (bias included); topk_idx [T][k]
 *   int32; topk_gate [T][k] fp32; counts [E] int32; offsets [E+1] int32;
 *   perm [T*k] int32; inv [T*k] int32; c [T][l] act dtype.
 */
typedef struct lmoe_debug {
    void* z;
    float* logits;
    int32_t* topk_idx;
    float* topk_gate;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    void* c;
} lmoe_debug;

/* ---- sizing, validation, diagnostics (host only, no GPU needed) ------ */

/* Bytes of device workspace the forward and staged entry points need for
 * these sizes; 0 if dims is invalid.  The workspace is caller-owned device
 * memory, 256-byte aligned, reusable across calls with the same or smaller
 * sizes. */
size_t lmoe_workspace_bytes(const lmoe_dims* dims);

/* Checks sizes and dtypes (see lmoe_dims) without touching the GPU. */
int lmoe_validate_dims(const lmoe_dims* dims);

/* Short English text for a status code. */
const char* lmoe_strerror(int status);

/* hipError_t of the last failed launch in this thread (0 if none). */
int lmoe_last_hip_error(void);

/* ---- optional context: a workspace the library owns ------------------ */

/*
 * For callers that would rather not manage the workspace.  A context holds
 * one device buffer, grown by lmoe_ctx_reserve (hipMalloc, outside any
 * forward call) and used by lmoe_ctx_forward, which never allocates.  One
 * context per stream; a context is not thread-safe.
 */
typedef struct lmoe_ctx lmoe_ctx;

/* *ctx = a new context for device `device` (the device must exist;
 * LMOE_ERR_HIP otherwise, LMOE_ERR_NULL for ctx == NULL).  No device memory
 * is allocated yet. */
int lmoe_create(lmoe_ctx** ctx, int device);

/* Frees the context and its workspace (the device must be idle for it);
 * NULL is a no-op. */
int lmoe_destroy(lmoe_ctx* ctx);

/* Grows the context's workspace to lmoe_workspace_bytes(dims) if it is
 * smaller, on the context's device (the old buffer is freed after the new
 * one is allocated; hipFree waits for the device).  Validation errors as
 * for lmoe_validate_dims; LMOE_ERR_HIP if the allocation fails, and the
 * context then keeps its previous workspace. */
int lmoe_ctx_reserve(lmoe_ctx* ctx, const lmoe_dims* dims);

/* Bytes of the context's workspace (0 before the first reserve). */
size_t lmoe_ctx_workspace_bytes(const lmoe_ctx* ctx);

/* latentmoe_forward on the context's workspace.  LMOE_ERR_WORKSPACE if the
 * context was not reserved for dims; LMOE_ERR_HIP if the caller's current
 * device is not the context's (nothing is launched then). */
int lmoe_ctx_forward(lmoe_ctx* ctx, const lmoe_dims* dims, const void* x, const void* W_down,
                     const void* W_router, const float* router_bias,
                     const lmoe_experts* experts, const void* W_up,
                     const lmoe_shared* shared, int k, void* out,
                     const lmoe_debug* dbg, void* stream);

/* ---- per-kernel timing (optional) ------------------------------------ */

/* One timed kernel launch: the kernel's name and its duration between two
 * hipEvents recorded on the launch's stream right before and after it. */
typedef struct lmoe_kernel_time {
    const char* name;
    float ms;
} lmoe_kernel_time;

/* Starts recording: every kernel launched by the entry points from now on is
 * bracketed by a pair of hipEvents on its stream, up to `capacity` launches
 * (later launches are not recorded).  Events are created here, on the host
 * thread's current device.  Not thread-safe: one recorder per process. */
int lmoe_timing_start(int capacity);

/* Waits for the recorded events, writes up to `capacity` records to `out`,
 * sets *count to the number recorded, releases the events and stops
 * recording.  Returns LMOE_ERR_HIP if an event query fails. */
int lmoe_timing_stop(lmoe_kernel_time* out, int capacity, int* count);

/* ---- weight preparation --------------------------------------------- */

/*
 * Repacks one routed-expert bf16 weight stack W [E][rows][cols] (row-major:
 * W1 with rows = f, cols = l; W2 with rows = l, cols = f) into the
 * LMOE_BF16_TILED layout, the order of the expert GEMMs' matrix-core
 * fragments: in 16-byte chunks,
 *   packed[e][rb][kt][s][l] = W[e][32 rb + l % 32][64 kt + 16 s + 8 (l / 32) .. +8]
 * for 32-row blocks rb, 64-wide K steps kt, 16-wide sub-steps s < 4 and
 * lanes l < 64, so that each sub-step of a block is one contiguous kilobyte
 * that a wave loads in one instruction, into registers or into LDS.  A
 * one-time preparation of static weights, not part of the forward.  packed must hold E*rows*cols*2 bytes, may not
 * overlap W, and both must be 16-byte aligned.  rows and cols must be
 * positive multiples of 64 (LMOE_ERR_SHAPE).  Asynchronous on stream.
 */
int lmoe_pack_expert_weights(int64_t E, int64_t rows, int64_t cols, const void* W, void* packed,
                             void* stream);

/*
 * Per-row FP8 quantisation of a bf16 matrix src [rows][cols] (row-major):
 * scales[r] = max_c |src[r][c]| / 448 in fp32 (1 for an all-zero row), and
 * codes[r][c] = E4M3(src[r][c] / scales[r]), the fp32 quotient rounded to the
 * nearest E4M3 (FN) value, ties to even.  This is how the fp8 shared expert
 * quantises its inputs (one scale per token); callers may use it for FP8
 * weights (one scale per output row).  codes [rows][cols] uint8, scales
 * [rows] fp32.  rows >= 1, cols a positive multiple of 8 up to 2^20
 * (LMOE_ERR_SHAPE); pointers 16-byte aligned.  Asynchronous on stream.
 */
int lmoe_quantize_rows_fp8(int64_t rows, int64_t cols, const void* src, uint8_t* codes, float* scales,
                           void* stream);

/*
 * MXFP8 quantisation (OCP microscaling) of a row-major bf16 matrix [rows]
 * [cols], as the MXFP8 projections quantise their inputs: per block of 32
 * consecutive elements of a row, e = floor(log2 max|v|) - 8 (the largest
 * E4M3 exponent), clamped to [-127, 127] and 0 for an all-zero block; the
 * scale byte is e + 127 (E8M0) and each element's code is E4M3 (FN, nearest,
 * ties to even) of v / 2^e saturated to +-448.  codes [rows][cols] uint8,
 * scales [rows][cols/32] uint8.  rows >= 1, cols a positive multiple of 32
 * up to 2^20 (LMOE_ERR_SHAPE); pointers 16-byte aligned.  Asynchronous on
 * stream.
 */
int lmoe_quantize_rows_mxfp8(int64_t rows, int64_t cols, const void* src, uint8_t* codes, uint8_t* scales,
                             void* stream);

/* ---- the layer ------------------------------------------------------- */

/*
 * The whole forward of the LatentMoE layer (Nemotron 3 overview, section 2.2
 * "LatentMoE", steps 1-3: project the hidden vector down to the latent width
 * l = d/4, route it and run the selected experts in the latent space, then
 * project the combined result back up to d; the shared expert stays in d per
 * the paragraph after that section's table; Ultra release news: 512 experts,
 * top-22): out [T][d] = LatentMoE(x).  router_bias [E] fp32 may be
 * NULL (no bias); shared may be NULL (then dims.f_s must be 0); dbg may be
 * NULL.  W_down and W_up are device arrays in the activation dtype, or
 * host pointers to lmoe_fp8_matrix with dims.proj_dtype = LMOE_FP8_E4M3, or
 * to lmoe_mxfp8_matrix with dims.proj_dtype = LMOE_MXFP8.  workspace (device,
 * caller-owned, 256-byte aligned) must hold lmoe_workspace_bytes(dims) bytes.
 * The result equals running lmoe_project_route, lmoe_permute,
 * lmoe_experts_ffn and lmoe_combine_up in that order.  Errors are returned
 * before the first launch (out untouched); the call is asynchronous on
 * stream.
 */
int latentmoe_forward(const lmoe_dims* dims, const void* x, const void* W_down,
                      const void* W_router, const float* router_bias,
                      const lmoe_experts* experts, const void* W_up,
                      const lmoe_shared* shared, int k, void* out,
                      void* workspace, size_t workspace_bytes,
                      const lmoe_debug* dbg, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * forward of latentmoe_forward without a workspace argument.  Its workspace
 * is a library-owned array of LMOE_STATIC_SCRATCH_BYTES (128 MiB) per GPU,
 * allocated when the library's code is loaded on that GPU and held until
 * the process ends; the call allocates and frees nothing.  The array of the
 * current device is used (stream must belong to it).  Returns
 * LMOE_ERR_WORKSPACE before any launch when lmoe_workspace_bytes(dims)
 * exceeds LMOE_STATIC_SCRATCH_BYTES (decode-sized layers fit: 60 MiB at
 * T = 64, d = 8192, E = 512, k = 22); other arguments and errors as for
 * latentmoe_forward.  Every call on one GPU shares that GPU's array and
 * finds it holding the previous call's data (nothing in it needs to start
 * at zero): calls that overlap in time on one GPU (other streams or host
 * threads) race, so serialise them.
 */
#define LMOE_STATIC_SCRATCH_BYTES (128u << 20)
int lmoe_static_forward(const lmoe_dims* dims, const void* x, const void* W_down,
                        const void* W_router, const float* router_bias,
                        const lmoe_experts* experts, const void* W_up,
                        const lmoe_shared* shared, int k, void* out,
                        const lmoe_debug* dbg, void* stream);

/* ---- staged entry points (same conventions) -------------------------- */

/*
 * Steps 1-4 (overview section 2.2 step 1; Ultra release news, 512 experts
 * with top-22): z = x W_down^T [T][l] (act dtype; not written with
 * dims.standard_moe, where z is x itself and may be NULL), logits = x W_r^T
 * + b [T][E] fp32 (z W_r^T + b with dims.router_latent, from the stored z),
 * topk_idx [T][k] int32 in (logit desc, id asc) order,
 * topk_gate [T][k] fp32 = softmax of the selected logits.  If shared is
 * non-NULL also hs = (max(0, x W_s1^T))^2 [T][f_s] (act dtype), the first
 * half of the shared expert (it reads the same x).  hs may be NULL iff
 * shared is NULL.
 */
int lmoe_project_route(const lmoe_dims* dims, const void* x, const void* W_down,
                       const void* W_router, const float* router_bias,
                       const lmoe_shared* shared, void* z, float* logits,
                       int32_t* topk_idx, float* topk_gate, void* hs,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Token permutation.  The pages do not describe how the routed tokens are
 * grouped by expert; this stable counting sort is this layer's own
 * specification of that step: counts[e] = number of (t, j) with topk_idx[t][j] = e;
 * offsets[e] = sum of counts below e, offsets[E] = T*k; perm[p] = the flat
 * pair index t*k + j at sorted position p, stable (pairs ascend within each
 * expert); inv = perm^-1.  Integer results are exact and deterministic.
 */
int lmoe_permute(const lmoe_dims* dims, const int32_t* topk_idx, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routed experts in the latent space (overview section 2.2 step 2), in
 * sorted order: for each sorted position p with pair (t, j) = perm[p] and
 * expert e, Y[p] = W2_e (max(0, W1_e z_t))^2, Y [T*k][l] act dtype (the gate
 * is applied by the combine).  NVFP4 weights are decoded in the kernel.
 */
int lmoe_experts_ffn(const lmoe_dims* dims, const void* z, const int32_t* offsets,
                     const int32_t* perm, const lmoe_experts* experts, void* Y,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Combine and up-projection (overview section 2.2 step 3): c_t = sum over
 * j = 0..k-1, in that order, of topk_gate[t][j] * Y[inv[t*k + j]] in fp32 (no
 * atomics; deterministic), out = c W_up^T [+ hs W_s2^T if shared]; with
 * dims.standard_moe, out = c [+ hs W_s2^T] and W_up may be NULL.
 * c [T][l] may be NULL (then it lives in the workspace).
 */
int lmoe_combine_up(const lmoe_dims* dims, const void* Y, const int32_t* inv,
                    const float* topk_gate, const void* W_up,
                    const lmoe_shared* shared, const void* hs, void* c, void* out,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LATENTMOE_H */
