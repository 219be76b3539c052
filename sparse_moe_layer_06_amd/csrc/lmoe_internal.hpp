// Internal interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "latentmoe.h"

namespace lmoe {

// Epilogue of a GEMM output group.
enum Epi : int {
    EPI_STORE = 0,     // C = acc, stored in the activation dtype
    EPI_F32_BIAS = 1,  // C = acc (+ bias[col]), stored fp32
    EPI_RELU2 = 2,     // C = max(0, acc * scale)^2, activation dtype
    EPI_ADD = 3,       // C = C + acc (times the fp8 scales), in place, activation dtype
};

// One contiguous range of output columns [n_begin, n_end) of a dense GEMM,
// with its own B rows (one pointer per K segment, rows of K[s] elements) and
// its own output tensor (column n - n_begin, leading dimension ldc).
struct NGroup {
    int n_begin, n_end;
    const void* B[2];
    int epi;
    void* C;
    int64_t ldc;
    const float* bias;
};

// C[M][N] = sum over K segments s of A_s[M][K_s] * B_s[N][K_s]^T.
// Segment 1 (if nseg == 2) continues the same accumulation: this fuses
// "c W_up^T + hs W_s2^T" into one GEMM.  All K_s are multiples of 64.
struct DenseGemm {
    int M, N;
    int nseg;
    const void* A[2];
    int64_t lda[2];
    int K[2];
    int ngroups;
    NGroup g[3];
};

// Device tile table of a grouped GEMM: M-tiles of BM sorted rows per expert.
// tiles[i] = {expert, first sorted row, rows, m | nt << 16} for the m-th of
// the expert's nt tiles; expert_tile_start/ntiles give each expert's tile
// range.  Built on the device from the offsets.
struct TileTable {
    const int* tile_count;
    const int4* tiles;
    const int* expert_tile_start;
    const int* expert_ntiles;
    int max_tiles;
    int bm;
    // Arrival counters of the tail-split expert GEMMs, one per work item; the
    // kernels that build the table zero them, and each GEMM leaves them zero.
    int* sk_count;
    int sk_count_len;
};

// Tail splitting of the few-rows expert GEMM: whole work items fill as many
// full rounds of the blocks as they can; each item of the last, partial
// round is split along K over up to kSkMaxParts blocks, and the block that
// finishes last sums the parts in part order.  One partial-sum slot per block.
constexpr int kSkBM = 64, kSkBN = 128;
constexpr int kSkMaxBlocks = 512, kSkMaxParts = 4;
constexpr size_t kSkPartialBytes = (size_t)kSkMaxBlocks * kSkBM * kSkBN * sizeof(float);

// Per-expert GEMM over sorted rows: for every tile (expert e, rows p),
// C[p][n] = epi( scale_e * sum_k A[arow(p)][k] * W_e[n][k] ), with
// arow(p) = a_row_map ? a_row_map[p] / a_row_div : p and scale_e the NVFP4
// tensor scale (1 for dense weights).
struct GroupedGemm {
    int N, K;
    TileTable tt;
    const void* A;
    int64_t lda;
    const int* a_row_map;
    int a_row_div;
    int n_rows;  // sorted rows in total (T * k): bound of a_row_map
    int b_fmt;  // LMOE_F32 / LMOE_BF16 dense stack [E][N][K], LMOE_BF16_TILED, LMOE_NVFP4 or LMOE_NVFP4_2D
    const void* B;
    const uint8_t* B_codes;   // [E][N][K/2]
    const uint8_t* B_scales;  // [E][N][K/16], or [E][N/16][K/16] with 2-D blocks
    const float* B_ts;        // [E]
    int epi;                  // EPI_RELU2 or EPI_STORE
    void* C;
    int64_t ldc;
    float* sk_part;           // kSkPartialBytes of tail-split partial sums, or null (whole items only)
};

// FP8 (E4M3 x E4M3) GEMM with per-row scales, fp32 accumulate:
// C[m][n] = epi(a_scale[m] * b_scale[n] * sum_k A[m][k] * B[n][k]), epi
// EPI_STORE, EPI_RELU2 (both store bf16) or EPI_ADD.  K is a multiple of
// 128; N, lda, ldb and ldc are multiples of 16.  Calls with M <= 64 split K
// over the given fp32 partial-sum workspace when it has room.
struct Fp8Gemm {
    int M, N, K;
    const uint8_t* A;
    int64_t lda;
    const float* a_scale;
    const uint8_t* B;
    int64_t ldb;
    const float* b_scale;
    int epi;
    uint16_t* C;
    int64_t ldc;
    // MXFP8 instead of the per-row scales (both or neither): E8M0 scale bytes
    // of each 32-code block along K, a_mx [M][K/32], b_mx [N][K/32]
    const uint8_t* a_mx;
    const uint8_t* b_mx;
};
// The decode-sized first dense GEMM (bf16, split along K) with the router's
// top-k and gates taken in its reduction, from the logits columns
// [lc0, lc0 + E) (+ bias): dense_topk_fusable says whether a call takes
// that path (at most 64 rows, k <= 64, a split, E <= 1024).
bool dense_topk_fusable(const DenseGemm& g, size_t splitk_bytes, int E, int k);
// The permutation's outputs when the last token block of that reduction
// also sorts the pairs (the fused forward): arrive is a workspace counter
// the GEMM clears before the reduction counts its token blocks in.
struct PermFused {
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* inv;
    TileTable tt;
    int* arrive;
};
hipError_t launch_dense_gemm_topk_bf16(const DenseGemm& g, void* splitk_ws, size_t splitk_bytes, int lc0, int E,
                                       const float* bias, int k, int32_t* idx, float* gate, const PermFused* pf,
                                       hipStream_t s);
hipError_t launch_fp8_gemm(const Fp8Gemm& g, void* splitk_ws, size_t splitk_bytes, hipStream_t s);

// MXFP8 quantisation of a bf16 matrix [rows][cols] (cols % 32 == 0, row
// stride ld): codes [rows][cols], E8M0 scales [rows][cols/32].
hipError_t launch_quantize_blocks_mxfp8(const uint16_t* src, int64_t rows, int cols, int64_t ld, uint8_t* codes,
                                        uint8_t* scales, hipStream_t s);

// Per-row FP8 quantisation of a bf16 matrix [rows][cols] (row stride ld):
// scale = max |v| / 448 (1 for an all-zero row), code = E4M3(v / scale),
// round to nearest even.  cols and ld are multiples of 8.
hipError_t launch_quantize_rows_fp8(const uint16_t* src, int64_t rows, int cols, int64_t ld, uint8_t* codes,
                                    float* scales, hipStream_t s);

// Partial-sum bytes the split last round of a many-token dense GEMM needs on
// this device (0: no split).
size_t dense_tail_split_bytes(const DenseGemm& g);

// ---- optional per-launch event timing (timing.hip) -----------------------

void timer_mark_begin(const char* name, hipStream_t s);
void timer_mark_end(hipStream_t s);

// Enqueues one kernel launch, bracketed by timing events when recording is on.
#define LMOE_LAUNCH(name, stream, ...)            \
    do {                                          \
        ::lmoe::timer_mark_begin(name, stream);   \
        __VA_ARGS__;                              \
        ::lmoe::timer_mark_end(stream);           \
    } while (0)

// ---- launchers (return hipSuccess or the launch error) ------------------

hipError_t launch_dense_gemm(const DenseGemm& g, int act_dtype, int T_hint, void* splitk_ws,
                             size_t splitk_bytes, hipStream_t s);
hipError_t launch_grouped_gemm(const GroupedGemm& g, int act_dtype, hipStream_t s);
// W [E][rows][cols] bf16 -> the LMOE_BF16_TILED image (rows, cols multiples of 64)
hipError_t launch_pack_experts(const void* W, void* P, int64_t E, int rows, int cols, hipStream_t s);

// Grouped-GEMM M-tile height for these sizes (the tile table is built for it).
int grouped_bm(const lmoe_dims& d);

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx,
                               float* gate, hipStream_t s);

// Permutation: hist scratch is [nchunks][E] ints.  If tiles is non-null the
// scan also writes the grouped-GEMM tile table for tile height bm.
int permute_nchunks(int64_t n_pairs);
hipError_t launch_permute(const int32_t* idx, int64_t n_pairs, int E, int32_t* hist,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                          const TileTable* tiles, hipStream_t s);
// Tile table from offsets alone (staged entry point).
hipError_t launch_build_tiles(const int32_t* offsets, int E, const TileTable& tt, hipStream_t s);

hipError_t launch_combine(const void* Y, const int32_t* inv, const float* gate, int T, int k, int l,
                          int act_dtype, void* c, hipStream_t s);

}  // namespace lmoe
