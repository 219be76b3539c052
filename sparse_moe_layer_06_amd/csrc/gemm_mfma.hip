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
// Block tile BM x BN x BK over WAVES_M x WAVES_N waves; each wave owns a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 MFMA tiles.  Operand tiles
// go through a ring of STAGES LDS stages, so STAGES - 1 K tiles are in
// flight while one is multiplied; they reach LDS one of two ways:
//   DMA   global_load_lds_dwordx4: each wave instruction moves 64 16-byte
//         chunks from global memory straight into 1 KB of LDS, no registers,
//         no LDS write instructions; per K step one vmcnt wait for the oldest
//         tile and one barrier.
//   REG   16-byte global loads into registers, then LDS writes (needed when
//         the tile is transformed on the way, as for the NVFP4 weights).
// Tile rows are stored as 16-byte chunks XOR-swizzled by row (swz_bits), so
// the fragment reads (32 consecutive rows at one logical chunk) hit distinct
// bank groups both per 8 and per 16 lanes.
//
// Block -> tile mapping is XCD-aware: consecutive block ids go round-robin to
// the 8 XCDs, so block b is the (b/8)-th block of XCD b%8; each XCD is given
// a contiguous range of the tile order, so tiles that share operands run
// together under one L2.
#include <algorithm>

#include "device_common.hpp"
#include "lmoe_internal.hpp"
#include "perm_block.hpp"
#include "topk_row.hpp"

namespace lmoe {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, bool DMA_, int BK_ = 64, int STAGES_ = 2, int MINB_ = 1,
          bool B_NT_ = false>
struct MfmaCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
    static constexpr int MINB = MINB_;  // blocks per CU the register budget is sized for
    // Weights fetched with the non-temporal hint: for weight streams read once
    // per call (few rows per expert); it costs L2 reuse when tiles share weights.
    static constexpr bool B_NT = B_NT_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = 64 * NW;
    static constexpr bool DMA = DMA_;
    static constexpr int CPR = BK / 8;  // 16-byte chunks per tile row
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int RPP = NT / CPR;  // rows per pass of one chunk per thread
    static constexpr int STAGE_CHUNKS = (BM + BN) * CPR;
    static_assert(BK == 32 || BK == 64, "K step is 32 or 64");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
};

// Physical chunk of logical chunk c in tile row r.  The fragment reads touch
// 32 consecutive rows at one logical chunk; the XOR keeps every 8 and every
// 16 consecutive lanes on distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz_bits(int r) {
    if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
    return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

template <class C>
__device__ __forceinline__ int lds_idx(int row, int c) { return row * C::CPR + (c ^ swz_bits<C::CPR>(row)); }

// Load slots: each thread moves one 16-byte chunk per slot and K step.
//   DMA: wave w owns LDS chunks [w*CPW, (w+1)*CPW) of the tile; slot j is one
//        instruction covering chunks w*CPW + 64 j + lane (lanes past CPW are
//        inactive).  Chunk q is physical chunk q % CPR of row q / CPR.
//   REG: slot j of thread t covers row t/CPR + j*RPP, logical chunk t % CPR.
template <class C, int ROWS>
struct Slots {
    static constexpr int CPW = C::DMA ? ROWS * C::CPR / C::NW : 0;  // chunks per wave
    static constexpr int N = C::DMA ? (CPW + 63) / 64 : ROWS / C::RPP;
    static constexpr int RPI = 64 / C::CPR;  // rows per DMA instruction
    static_assert(!C::DMA || (ROWS * C::CPR) % C::NW == 0, "DMA chunks must split evenly over the waves");
    static_assert(C::DMA || ROWS % C::RPP == 0, "register slots must tile the rows");
    __device__ static __forceinline__ int chunk(int j, int tid) { return (tid >> 6) * CPW + j * 64 + (tid & 63); }
    __device__ static __forceinline__ bool active(int j, int tid) { return !C::DMA || j * 64 + (tid & 63) < CPW; }
    __device__ static __forceinline__ int row(int j, int tid) {
        if constexpr (C::DMA) return min(chunk(j, tid), ROWS * C::CPR - 1) / C::CPR;
        return tid / C::CPR + j * C::RPP;
    }
    __device__ static __forceinline__ int lchunk(int j, int tid) {
        if constexpr (C::DMA) return (chunk(j, tid) % C::CPR) ^ swz_bits<C::CPR>(row(j, tid));
        return tid % C::CPR;
    }
    // LDS destination of DMA slot j for wave `wave` (wave-uniform)
    __device__ static __forceinline__ u32x4_t* dst(u32x4_t* base, int wave, int j) { return base + wave * CPW + j * 64; }
};

// One LDS-DMA instruction: 16 bytes per lane from `src` into LDS starting at
// the wave-uniform `dst` (lane i lands at dst + 16 i).
// AUX is the instruction's cache-policy field; 2 sets the non-temporal bit.
template <int AUX = 0>
__device__ __forceinline__ void dma16(const void* src, u32x4_t* dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, AUX);
}

// Scalar-memory loads of wave-uniform data.  They complete on lgkmcnt, which
// the asm waits for before returning, so using their result never makes the
// compiler drain the vector-memory counter that tracks the DMA tiles still
// in flight (it cannot count those across loop iterations and would wait for
// all of them).  Reads only; the pointer is made uniform explicitly.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ i32x4_t sload4(const void* p) {
    i32x4_t v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
    return v;
}

__device__ __forceinline__ i32x8_t sload8(const void* p) {
    i32x8_t v;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
    return v;
}

__device__ __forceinline__ i32x16_t sload16(const void* p) {
    i32x16_t v;
    asm volatile("s_load_dwordx16 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
    return v;
}

__device__ __forceinline__ float sload_f32(const float* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(uniform_ptr(p)) : "memory");
    return __int_as_float(v);
}

// s_waitcnt with vmcnt(N) only (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with vmcnt(N) and lgkmcnt(0): also this wave's LDS writes done.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Writes and reads of an output tile staged in LDS beside a DMA ring.  The
// compiler cannot tell that the K steps still landing by DMA go to other
// bytes of the same array, and before a plain LDS access it waits for every
// one of them (the steps prefetched for the next item); before these asm
// accesses it does not.  The reads wait for their own data in the same asm
// statement; the caller orders the writes before the reads with
// lgkmcnt(0) and a barrier.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void lds_write_b64(void* p, uint32_t lo, uint32_t hi) {
    const uint64_t v = (uint64_t)lo | ((uint64_t)hi << 32);
    asm volatile("ds_write_b64 %0, %1" : : "v"(lds_offset(p)), "v"(v) : "memory");
}

// N 16-byte reads at p + i * STRIDE bytes (N = 2 or 6)
template <int N, int STRIDE>
__device__ __forceinline__ void lds_read_b128xn(const void* p, u32x4_t (&v)[N]) {
    static_assert((N == 2 || N == 6) && (N - 1) * STRIDE < 65536 && STRIDE % 16 == 0, "ds offset range");
    const uint32_t a = lds_offset(p);
    if constexpr (N == 2) {
        asm volatile(
            "ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1])
            : "v"(a), "i"(STRIDE)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %6\n\tds_read_b128 %1, %6 offset:%7\n\tds_read_b128 %2, %6 offset:%8\n\t"
            "ds_read_b128 %3, %6 offset:%9\n\tds_read_b128 %4, %6 offset:%10\n\t"
            "ds_read_b128 %5, %6 offset:%11\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
            : "v"(a), "i"(STRIDE), "i"(2 * STRIDE), "i"(3 * STRIDE), "i"(4 * STRIDE), "i"(5 * STRIDE)
            : "memory");
    }
}

// Waits until at most `ahead` K tiles of this wave's DMA are still in flight
// (`per_tile` instructions each), then the workgroup barrier.  The empty asm
// statements keep the compiler from moving memory accesses across.
template <int MAXAHEAD, int PER_TILE>
__device__ __forceinline__ void wait_tiles_barrier(int ahead) {
    asm volatile("" ::: "memory");
    if constexpr (MAXAHEAD >= 3) {
        if (ahead >= 3) wait_vmcnt<3 * PER_TILE>();
    }
    if constexpr (MAXAHEAD >= 2) {
        if (ahead == 2) wait_vmcnt<2 * PER_TILE>();
    }
    if constexpr (MAXAHEAD >= 1) {
        if (ahead == 1) wait_vmcnt<PER_TILE>();
    }
    if (ahead <= 0) __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One LDS tile of MFMAs for this wave.  Output (m, n) of register r of each
// 32x32 block for this lane, when the MFMA is issued as mfma(B-fragment,
// A-fragment): m = lane % 32, n = 8 * (r / 4) + 4 * (lane / 32) + r % 4.
//
// The fragments of 16-wide K sub-step ks + 1 are read into the second of two
// register sets while the MFMAs of sub-step ks run, one read issued after
// each MFMA, so each read has most of an MFMA group to land and the MFMA pipe
// is fed while the reads go out.  Each sub-step first waits for the reads
// issued one group earlier (lgkmcnt(0) while only those are in flight: they
// have landed by then); the compiler would otherwise wait for all reads
// right before the MFMAs, including the ones just issued.
// BFRAG: the B tile is in fragment order (packed expert weights): the 32-row
// block rb's fragment of sub-step ks is the 64 chunks at (4 rb + ks) * 64,
// lane l's at + l.
template <class C, bool BFRAG = false>
__device__ __forceinline__ void mma_tile(const u32x4_t* __restrict__ As, const u32x4_t* __restrict__ Bs,
                                         f32x16_t (&acc)[C::TM][C::TN], int wm, int wn, int lane) {
    constexpr int KS = C::BK / 16, NM = C::TM * C::TN, NR = C::TM + C::TN;
    bf16x8_t af[2][C::TM], bfr[2][C::TN];
    auto read = [&](int ks, int b) __attribute__((always_inline)) {
        const int ch = ks * 2 + (lane >> 5);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
            af[b][tm] = as_bf16x8(As[lds_idx<C>(wm * C::WM + tm * 32 + (lane & 31), ch)]);
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn)
            bfr[b][tn] = as_bf16x8(BFRAG ? Bs[((wn * C::WN / 32 + tn) * KS + ks) * 64 + lane]
                                         : Bs[lds_idx<C>(wn * C::WN + tn * 32 + (lane & 31), ch)]);
    };
    read(0, 0);
    static_for<KS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value, b = ks & 1;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ks + 1 < KS) read(ks + 1, b ^ 1);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = mfma32x32x16(bfr[b][tn], af[b][tm], acc[tm][tn]);
        if constexpr (ks + 1 < KS) {  // issue order: MFMA m, then its share of the reads
            static_for<NM>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value, r = (m + 1) * NR / NM - m * NR / NM;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// fp8 variant of mma_tile: the LDS tile holds K step 128 fp8 codes per row
// (the same 8 chunks of 16 B as a K step of 64 bf16), multiplied in two
// sub-steps of K 64; a lane's fragment is two adjacent chunks (32 codes).
template <class C>
__device__ __forceinline__ void mma_tile_fp8(const u32x4_t* __restrict__ As, const u32x4_t* __restrict__ Bs,
                                             f32x16_t (&acc)[C::TM][C::TN], int wm, int wn, int lane) {
    constexpr int KS = 2, NM = C::TM * C::TN, NR = 2 * (C::TM + C::TN);
    i32x8_t af[2][C::TM], bfr[2][C::TN];
    auto frag = [&](const u32x4_t* T, int row, int ch) __attribute__((always_inline)) {
        const u32x4_t lo = T[lds_idx<C>(row, ch)], hi = T[lds_idx<C>(row, ch + 1)];
        return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read = [&](int ks, int b) __attribute__((always_inline)) {
        const int ch = ks * 4 + (lane >> 5) * 2;
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) af[b][tm] = frag(As, wm * C::WM + tm * 32 + (lane & 31), ch);
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bfr[b][tn] = frag(Bs, wn * C::WN + tn * 32 + (lane & 31), ch);
    };
    read(0, 0);
    static_for<KS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value, b = ks & 1;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ks + 1 < KS) read(ks + 1, b ^ 1);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = mfma32x32x64_fp8(bfr[b][tn], af[b][tm], acc[tm][tn]);
        if constexpr (ks + 1 < KS) {
            static_for<NM>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value, r = (m + 1) * NR / NM - m * NR / NM;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// MXFP8 variant of mma_tile_fp8: the stage also holds one 32-bit word of
// E8M0 block scales per A row and per B row (the 4 blocks of 32 codes of
// this K step, block b in byte b) at S: A rows first, then B rows.  Sub-step
// ks multiplies blocks 2 ks and 2 ks + 1, and lane l passes the scale of
// block 2 ks + l / 32 of its row (measured on the device: lanes 0..31's
// scales cover the sub-step's k 0..31, lanes 32..63's k 32..63).  Each lane
// shifts its words right by 8 (l / 32) once, so the byte it needs is byte
// 2 ks for every lane, picked by the MFMA's operand select, and no scale
// register is rewritten between the tile's MFMAs.
template <class C>
__device__ __forceinline__ void mma_tile_mx(const u32x4_t* __restrict__ As, const u32x4_t* __restrict__ Bs,
                                            const u32x4_t* __restrict__ S, f32x16_t (&acc)[C::TM][C::TN], int wm,
                                            int wn, int lane) {
    constexpr int KS = 2, NM = C::TM * C::TN, NR = 2 * (C::TM + C::TN);
    const uint32_t* Su = reinterpret_cast<const uint32_t*>(S);
    const int lane_shift = 8 * (lane >> 5);
    int sa[C::TM], sb[C::TN];
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) sa[tm] = (int)(Su[wm * C::WM + tm * 32 + (lane & 31)] >> lane_shift);
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) sb[tn] = (int)(Su[C::BM + wn * C::WN + tn * 32 + (lane & 31)] >> lane_shift);
    i32x8_t af[2][C::TM], bfr[2][C::TN];
    // The MFMA's true K order: lane l's first four registers are k 16 (l/32)
    // + [0, 16) and its last four k 32 + 16 (l/32) + [0, 16), so scale block
    // 0 (k 0..31, the scale of lanes 0..31) is code chunks 0 and 1 of the
    // sub-step, held in the low halves of both lane halves.
    auto frag = [&](const u32x4_t* T, int row, int ch) __attribute__((always_inline)) {
        const u32x4_t lo = T[lds_idx<C>(row, ch)], hi = T[lds_idx<C>(row, ch + 2)];
        return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read = [&](int ks, int b) __attribute__((always_inline)) {
        const int ch = ks * 4 + (lane >> 5);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) af[b][tm] = frag(As, wm * C::WM + tm * 32 + (lane & 31), ch);
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) bfr[b][tn] = frag(Bs, wn * C::WN + tn * 32 + (lane & 31), ch);
    };
    read(0, 0);
    static_for<KS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int ks = decltype(kc)::value, b = ks & 1;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ks + 1 < KS) read(ks + 1, b ^ 1);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn)
                acc[tm][tn] = mfma32x32x64_mxfp8<2 * ks>(bfr[b][tn], af[b][tm], acc[tm][tn], sb[tn], sa[tm]);
        if constexpr (ks + 1 < KS) {
            static_for<NM>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value, r = (m + 1) * NR / NM - m * NR / NM;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
            });
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// K loop over nk tiles through a ring of C::STAGES LDS stages.
//   fill(kt, As, Bs)  starts moving tile kt into a stage (DMA issue, and/or
//                     global loads into registers);
//   land(As, Bs)      finishes the move (writes staged registers to LDS).
// Tile kt + STAGES - 1 is issued while tile kt is multiplied, so up to
// STAGES - 1 tiles are in flight.  PER_TILE is the number of DMA
// instructions per tile and wave; 0 means "wait for everything" (register
// staged operands already wait in land).  MODE: 0 bf16, 1 fp8, 2 MXFP8,
// whose stages carry EXTRA more chunks (the block scales) after the tiles.
template <class C, int PER_TILE, int MODE = 0, int EXTRA = 0, class Fill, class Land>
__device__ __forceinline__ void kloop(int nk, Fill&& fill, Land&& land, u32x4_t* ring,
                                      f32x16_t (&acc)[C::TM][C::TN], int wm, int wn, int lane) {
    constexpr int S = C::STAGES, STG = C::STAGE_CHUNKS + EXTRA, AOFF = C::BM * C::CPR;
    constexpr int MAXAHEAD = PER_TILE > 0 ? S - 2 : 0;
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
        if (s < nk) {
            fill(s, ring + s * STG, ring + s * STG + AOFF);
            land(ring + s * STG, ring + s * STG + AOFF);
        }
    }
    int cur = 0, nxt = S - 1;  // stage of tile kt, stage for tile kt + S - 1
    for (int kt = 0; kt < nk; ++kt) {
        wait_tiles_barrier<MAXAHEAD, PER_TILE>(min(MAXAHEAD, nk - 1 - kt));
        const bool more = kt + S - 1 < nk;
        u32x4_t* ns = ring + nxt * STG;
        if (more) fill(kt + S - 1, ns, ns + AOFF);
        u32x4_t* cs = ring + cur * STG;
        if constexpr (MODE == 2)
            mma_tile_mx<C>(cs, cs + AOFF, cs + C::STAGE_CHUNKS, acc, wm, wn, lane);
        else if constexpr (MODE == 1)
            mma_tile_fp8<C>(cs, cs + AOFF, acc, wm, wn, lane);
        else
            mma_tile<C>(cs, cs + AOFF, acc, wm, wn, lane);
        if (more) land(ns, ns + AOFF);
        cur = (cur + 1 == S) ? 0 : cur + 1;
        nxt = (nxt + 1 == S) ? 0 : nxt + 1;
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

__device__ __forceinline__ float apply_epi(int epi, float v) {
    if (epi == EPI_RELU2) {
        v = fmaxf(v, 0.f);
        return v * v;
    }
    return v;
}

__device__ __forceinline__ void dense_store1(const DenseGemm& g, int m, int n, float v) {
    const NGroup& G = pick_group(g, n);
    const int nc = n - G.n_begin;
    const int64_t off = (int64_t)m * G.ldc + nc;
    if (G.epi == EPI_F32_BIAS) {
        ((float*)G.C)[off] = v + (G.bias ? G.bias[nc] : 0.f);
    } else if (G.epi == EPI_ADD) {
        uint16_t* c = (uint16_t*)G.C + off;
        *c = f32_to_bf16_rne(bf16_to_f32(*c) + v);
    } else {
        ((uint16_t*)G.C)[off] = f32_to_bf16_rne(apply_epi(G.epi, v));
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
        } else if (G.epi == EPI_ADD) {
            uint2* c = reinterpret_cast<uint2*>((uint16_t*)G.C + off);
            const uint2 old = *c;
            uint2 o;
            o.x = pack_bf16x2(bf16_to_f32((uint16_t)(old.x & 0xFFFFu)) + v[0], bf16_to_f32((uint16_t)(old.x >> 16)) + v[1]);
            o.y = pack_bf16x2(bf16_to_f32((uint16_t)(old.y & 0xFFFFu)) + v[2], bf16_to_f32((uint16_t)(old.y >> 16)) + v[3]);
            *c = o;
        } else {
            uint2 o;
            o.x = pack_bf16x2(apply_epi(G.epi, v[0]), apply_epi(G.epi, v[1]));
            o.y = pack_bf16x2(apply_epi(G.epi, v[2]), apply_epi(G.epi, v[3]));
            *reinterpret_cast<uint2*>((uint16_t*)G.C + off) = o;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (n + i < g.N) dense_store1(g, m, n + i, v[i]);
}

// With splits > 1 (split-K, for few-row GEMMs whose tiles alone cannot fill
// the GPU), block (tile, split) accumulates the K steps
// [split * nk / splits, (split + 1) * nk / splits) and stores its fp32
// partial tile to partial[split][M][ldp]; splitk_reduce_kernel sums the
// splits in order and applies the column-group epilogue.
template <class C>
__global__ __launch_bounds__(C::NT, C::MINB) void dense_gemm_kernel(DenseGemm g, int tiles_m, int tiles_n,
                                                              int group_m, int splits, float* partial,
                                                              int ldp, int* clear) {
    __shared__ u32x4_t ring[C::STAGES * C::STAGE_CHUNKS];
    const int tid = threadIdx.x, lane = tid & 63;
    if (clear && blockIdx.x == 0 && tid == 0) *clear = 0;  // a counter of the kernel that follows
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    const int ws_ = xcd_work_index(blockIdx.x, tiles_m * tiles_n * splits);
    if (ws_ < 0) return;
    const int split = ws_ % splits, w = ws_ / splits;
    const int width = group_m * tiles_n;
    const int first_m = (w / width) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int m0 = (first_m + (w % width) % gsz) * C::BM;
    const int n0 = ((w % width) / gsz) * C::BN;

    using SA = Slots<C, C::BM>;
    using SB = Slots<C, C::BN>;
    const uint16_t* a_ptr[SA::N];
    const uint16_t* b_ptr[SB::N];
    auto setup_seg = [&](int s) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SA::N; ++j) {
            const int m = min(m0 + SA::row(j, tid), g.M - 1);
            a_ptr[j] = (const uint16_t*)g.A[s] + (int64_t)m * g.lda[s] + SA::lchunk(j, tid) * 8;
        }
#pragma unroll
        for (int j = 0; j < SB::N; ++j) {
            const int n = min(n0 + SB::row(j, tid), g.N - 1);
            const NGroup& G = pick_group(g, n);
            b_ptr[j] = (const uint16_t*)G.B[s] + (int64_t)(n - G.n_begin) * g.K[s] + SB::lchunk(j, tid) * 8;
        }
    };

    const int nk0 = g.K[0] / C::BK;
    const int nk = nk0 + (g.nseg > 1 ? g.K[1] / C::BK : 0);
    const int kb = split * nk / splits, ke = (split + 1) * nk / splits;
    int cur_seg = kb >= nk0 ? 1 : 0;
    if (cur_seg)  // constant segment indices keep the argument arrays out of scratch
        setup_seg(1);
    else
        setup_seg(0);

    u32x4_t ra[C::DMA ? 1 : SA::N], rb[C::DMA ? 1 : SB::N];
    auto fill = [&](int kt_local, u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
        const int kt = kb + kt_local;
        if (kt >= nk0 && cur_seg == 0) {
            cur_seg = 1;
            setup_seg(1);
        }
        const int kk = (kt - (cur_seg ? nk0 : 0)) * C::BK;
        if constexpr (C::DMA) {
#pragma unroll
            for (int j = 0; j < SA::N; ++j)
                if (SA::active(j, tid)) dma16(a_ptr[j] + kk, SA::dst(As, wave, j));
#pragma unroll
            for (int j = 0; j < SB::N; ++j)
                if (SB::active(j, tid)) dma16<C::B_NT ? 2 : 0>(b_ptr[j] + kk, SB::dst(Bs, wave, j));
        } else {
#pragma unroll
            for (int j = 0; j < SA::N; ++j) ra[j] = *reinterpret_cast<const u32x4_t*>(a_ptr[j] + kk);
#pragma unroll
            for (int j = 0; j < SB::N; ++j) rb[j] = *reinterpret_cast<const u32x4_t*>(b_ptr[j] + kk);
        }
    };
    auto land = [&](u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
        if constexpr (!C::DMA) {
#pragma unroll
            for (int j = 0; j < SA::N; ++j) As[lds_idx<C>(SA::row(j, tid), SA::lchunk(j, tid))] = ra[j];
#pragma unroll
            for (int j = 0; j < SB::N; ++j) Bs[lds_idx<C>(SB::row(j, tid), SB::lchunk(j, tid))] = rb[j];
        }
    };

    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    kloop<C, C::DMA ? SA::N + SB::N : 0>(ke - kb, fill, land, ring, acc, wm, wn, lane);

    static_for<C::TM>([&](auto tmc) __attribute__((always_inline)) {
        constexpr int tm = decltype(tmc)::value;
        const int m = m0 + wm * C::WM + tm * 32 + (lane & 31);
        if (m < g.M) {
            static_for<C::TN * 4>([&](auto tqc) __attribute__((always_inline)) {
                constexpr int tn = decltype(tqc)::value / 4, q = decltype(tqc)::value % 4;
                const int n = n0 + wn * C::WN + tn * 32 + q * 8 + (lane >> 5) * 4;
                if (n < g.N) {
                    const float v[4] = {acc[tm][tn][q * 4 + 0], acc[tm][tn][q * 4 + 1], acc[tm][tn][q * 4 + 2],
                                        acc[tm][tn][q * 4 + 3]};
                    if (partial) {
                        // ldp is a multiple of 4, so the 4 columns are one aligned float4
                        *reinterpret_cast<float4*>(partial + ((int64_t)split * g.M + m) * ldp + n) =
                            make_float4(v[0], v[1], v[2], v[3]);
                    } else {
                        dense_store4(g, m, n, v);
                    }
                }
            });
        }
    });
}

// Sums the split-K partials in split order (deterministic) and applies the
// epilogue.  One thread per 4 consecutive columns of one row.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(DenseGemm g, int splits, const float* __restrict__ partial,
                                                            int ldp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int q = ldp / 4;
    const int m = (int)(i / q), n = (int)(i % q) * 4;
    if (m >= g.M || n >= g.N) return;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    // eight splits' loads in flight at a time, added in split order
    constexpr int kBatch = 8;
    for (int sp0 = 0; sp0 < splits; sp0 += kBatch) {
        float4 p[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (sp0 + b < splits)
                p[b] = *reinterpret_cast<const float4*>(partial + ((int64_t)(sp0 + b) * g.M + m) * ldp + n);
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (sp0 + b < splits) {
                v[0] += p[b].x;
                v[1] += p[b].y;
                v[2] += p[b].z;
                v[3] += p[b].w;
            }
    }
    if (n + 3 < g.N) {
        dense_store4(g, m, n, v);
    } else {
        for (int c = 0; c < 4 && n + c < g.N; ++c) dense_store1(g, m, n + c, v[c]);
    }
}

// Pairs the fused permutation sorts at most (up to 64 rows of top-64).
constexpr int kMaxFusedPairs = 64 * kWave;

// The decode-sized first GEMM's reduction with the router folded in.  Two
// blocks per token row sum the row's split partials in split order and
// store them through the column groups' epilogues, as splitk_reduce_kernel
// does: block m < M the float4 chunks holding the logits (columns [lc0,
// lc0 + E)), block M + m the other columns, so that the first finishes its
// loads early.  Block m keeps the row's logits (bias added: the values the
// logits epilogue stores) in LDS; its first wave then selects the token's
// top-k and gates from there, as the router kernel does from the stored
// logits.  This saves the router kernel's launch and its re-read.  1024
// threads, so each part of a decode row takes one pass of float4 chunks,
// with up to 16 splits' loads in flight per thread.
//
// PERM (the fused forward): the row's ids are stored device-coherently, and
// each selecting block counts itself in once they have completed; the last
// of the M token blocks reads every id back (device-coherent loads) and runs
// the permutation's single-block counting sort, so that kernel's launch
// goes.  Every block's ids are complete before its arrival is counted, so
// the last one reads all of them.
template <int S, bool PERM>
__global__ __launch_bounds__(1024) void splitk_reduce_topk_kernel(DenseGemm g, int splits,
                                                                 const float* __restrict__ partial, int ldp,
                                                                 int lc0, int E, const float* __restrict__ bias,
                                                                 int k, int32_t* __restrict__ idx,
                                                                 float* __restrict__ gate, PermFused pf) {
    __shared__ float s_l[S * kWave];
    __shared__ uint64_t by_id[kWave], by_rank[kWave];
    const bool sel = (int)blockIdx.x < g.M;  // this block selects the row's top-k
    const int m = sel ? blockIdx.x : blockIdx.x - g.M;
    const int lo = lc0 & ~3, hi = lc0 + E;  // float4 chunks starting in [lo, hi) hold logits
    for (int n = (sel ? lo : 0) + threadIdx.x * 4; n < (sel ? hi : g.N); n += 1024 * 4) {
        if (!sel && n >= lo && n < hi) continue;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        constexpr int kBatch = 16;
        for (int sp0 = 0; sp0 < splits; sp0 += kBatch) {
            float4 p[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (sp0 + b < splits)
                    p[b] = *reinterpret_cast<const float4*>(partial + ((int64_t)(sp0 + b) * g.M + m) * ldp + n);
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (sp0 + b < splits) {
                    v[0] += p[b].x;
                    v[1] += p[b].y;
                    v[2] += p[b].z;
                    v[3] += p[b].w;
                }
        }
        if (n + 3 < g.N) {
            dense_store4(g, m, n, v);
        } else {
            for (int c = 0; c < 4 && n + c < g.N; ++c) dense_store1(g, m, n + c, v[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = n + c - lc0;
            if (e >= 0 && e < E) s_l[e] = v[c] + (bias ? bias[e] : 0.f);
        }
    }
    if (!sel) return;
    __syncthreads();
    if (threadIdx.x < kWave) topk_select_row<S, PERM>(s_l, E, k, m, by_id, by_rank, idx, gate);
    if constexpr (PERM) {
        __shared__ int s_last;
        __shared__ int32_t s_idx[kMaxFusedPairs];
        __shared__ int h[kSmallWaves][kMaxExperts];
        __builtin_amdgcn_s_waitcnt(0);  // this thread's id stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(pf.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g.M - 1;
        __syncthreads();
        if (!s_last) return;
        const int n = g.M * k;
        for (int p = threadIdx.x; p < n; p += 1024)
            s_idx[p] = __hip_atomic_load(idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        perm_block(s_idx, n, E, pf.counts, pf.offsets, pf.perm, pf.inv, pf.tt, 1, h);
        if (threadIdx.x == 0) *pf.arrive = 0;
    }
}

// ---------------------------------------------------------------------------
// Grouped (per-expert) GEMM
// ---------------------------------------------------------------------------

// NVFP4 weight decode (Nemotron 3 overview, section 3.1.1: E2M1 elements,
// 16-element micro-blocks, E4M3 block scale).  An E4M3 scale byte is split
// into a power of two pw and a factor mt: normal 2^(e-7) * (1 + m/8),
// subnormal 2^-6 * (m/8), the sign on mt (0x7F / 0xFF is NaN).
__device__ __forceinline__ void e4m3_parts(uint32_t b, float& pw, float& mt) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    pw = __uint_as_float((e == 0u ? 121u : e + 120u) << 23);
    mt = (e == 0u ? 0.f : 1.f) + (float)m * 0.125f;
    if (e == 15u && m == 7u) mt = __uint_as_float(0x7FC00000u);
    if (b & 0x80u) mt = -mt;
}

// The same split of an E4M3 scale already converted to fp32 (exactly, by the
// hardware's OCP E4M3 conversion): pw keeps its exponent bits, mt takes its
// sign and mantissa with the exponent of 1, so pw * mt is the scale for every
// nonzero finite value (an E4M3 subnormal is a normal fp32).  A zero scale
// gives pw = 1, mt = 0; a NaN one mt = NaN.
__device__ __forceinline__ void e4m3_split_f32(float s, float& pw, float& mt) {
    const uint32_t u = __float_as_uint(s);
    const bool zero = (u & 0x7FFFFFFFu) == 0u;
    pw = zero ? 1.f : __uint_as_float(u & 0x7F800000u);
    mt = zero ? 0.f : __uint_as_float((u & 0x807FFFFFu) | 0x3F800000u);
    if (s != s) mt = s;
}

// 8 E2M1 codes (one 32-bit word, element i in bits 4i..4i+3, so byte j holds
// elements 2j and 2j+1) -> 8 bf16.  The hardware conversion scales by the
// power of two exactly; the product with mt has at most 6 significant bits
// (an E2M1 value has up to 2, an E4M3 factor up to 4: 1.5 x 1.875 =
// 10.1101b), so it is exact in fp32 and its upper half (8 bits) is the exact
// bf16.
__device__ __forceinline__ u32x4_t decode_e2m1x8(uint32_t codes, float pw, float mt) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    u32x4_t r;
    static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        const f32x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, pw, j);
        r[j] = __builtin_amdgcn_perm(__float_as_uint(v.y * mt), __float_as_uint(v.x * mt), 0x07060302u);
    });
    return r;
}

// Persistent grouped GEMM.  A grid of MINB blocks per CU walks a list of
// work items, each one M tile of one expert (tiles[i] = {expert, first
// sorted row, rows}) times one BN-wide N tile.  The list holds an expert's
// items together (its M tiles times the nN N tiles); an XCD's blocks (block
// b runs on XCD b % 8) take the XCD's contiguous range of the list
// round-robin, so each round covers consecutive items, and within an expert
// the M tiles that share a weight tile are neighbours (see load_item).
//
// The K steps of all the block's items form one flattened loop through the
// LDS ring: the first stages of the next item are in flight while the
// current item finishes and writes its epilogue, and the next item's
// descriptor is fetched one item ahead, so short-K items (K = l or f) do not
// pay a pipeline fill each.
//
// A (gathered activation rows) always uses the tile's loader policy; B is a
// dense bf16 expert stack (same policy) or NVFP4 codes decoded into the LDS
// weight tile, the codes staged through LDS-DMA (SPLITB, the prefill tiles)
// or through registers (the other tiles).
// A-row gather modes of the grouped GEMM.
enum Gather : int { GATHER_NONE = 0, GATHER_SCALAR = 1, GATHER_LANE = 2 };

// Work items are (expert tile, N tile) pairs, W = tiles * nN of them.
//   SK = false: whole items; XCD x takes the x-th eighth of the list and its
//               blocks take every nbx-th item of it.
//   SK = true:  if the last round is at most half full (T = W - R G tail
//               items, R = W / G full rounds), R full rounds of whole items
//               (spread over the XCDs as above), then each tail item split
//               along K into P >= 2 parts, one per block; the last part to
//               finish sums them (sk_finish).  A lone tail item would
//               otherwise be streamed by one block while the rest idle.
template <class C, int BFMT, int GATHER, bool SK = false>
__global__ __launch_bounds__(C::NT, C::MINB) void grouped_gemm_kernel(GroupedGemm g, int nN) {
    // NVFP4 prefill tiles with 3 stages (SPLITB): the A ring has 3 stages,
    // the decoded weight tiles a 2-slot ring of their own, and the raw codes
    // and scale words (RAW chunks per step) a 2-slot ring; see the K loop.
    constexpr bool SPLITB = (BFMT == LMOE_NVFP4 || BFMT == LMOE_NVFP4_2D) && !SK && C::STAGES == 3 && C::BM >= 128;
    constexpr int RAW = C::NT + C::NT / 4;  // a 16-byte chunk of codes and a 4-byte scale word per thread
    __shared__ u32x4_t ring[SPLITB ? (C::STAGES * C::BM + 2 * C::BN) * C::CPR + 2 * RAW
                                   : C::STAGES * C::STAGE_CHUNKS];
    __shared__ int sk_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int N = g.N, K = g.K;
    const int nk = K / C::BK;

    const int W = *g.tt.tile_count * nN;
    int w_first, stride, n_items, total;
    // SK: full rounds, parts per tail item, this block's tail item and part
    // K range [sk_kb, sk_ke) (sk_t < 0: no tail part; sk_R < 0: no split)
    int sk_R = -1, sk_P = 1, sk_t = -1, sk_kb = 0, sk_ke = 0;
    if constexpr (SK) {
        const int G = gridDim.x, R = W / G, T = W - R * G;
        if (T > 0) sk_P = max(1, min(min(G / T, kSkMaxParts), nk));
        if (sk_P > 1) {
            const int b = blockIdx.x;
            sk_R = R;
            if (b < T * sk_P) {
                sk_t = R * G + b / sk_P;
                const int p = b % sk_P;
                sk_kb = p * nk / sk_P;
                sk_ke = (p + 1) * nk / sk_P;
            }
            n_items = R + (sk_t >= 0 ? 1 : 0);
            if (n_items == 0) return;
            total = R * nk + (sk_ke - sk_kb);
            // full rounds XCD by XCD as for whole items: XCD b % 8 takes the
            // (b % 8)-th eighth of the first R G items
            const int nbx = G >> 3;
            w_first = (b & 7) * R * nbx + (b >> 3);
            stride = nbx;
        }
    }
    if (sk_R < 0) {  // whole items only
        const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, nbx = gridDim.x >> 3;
        const int per = W >> 3, rem = W & 7;
        const int first = x * per + min(x, rem);
        const int end = first + per + (x < rem ? 1 : 0);
        if (first + slot >= end) return;
        n_items = (end - 1 - first - slot) / nbx + 1;
        total = n_items * nk;
        w_first = first + slot;
        stride = nbx;
    }
    // first K step of item i (only a tail part starts inside its item)
    auto item_kt0 = [&](int i) __attribute__((always_inline)) { return (SK && i == sk_R) ? sk_kb : 0; };
    auto item_w = [&](int i) __attribute__((always_inline)) {
        i = min(i, n_items - 1);
        return __builtin_amdgcn_readfirstlane((SK && i == sk_R) ? sk_t : w_first + i * stride);
    };
    // descriptor {expert, first sorted row, rows, n0} of this block's item i.
    // Without the tail split an expert's items (its nt M tiles times the nN
    // N tiles, consecutive in the list) are taken N-tile-major: the nt
    // items that share a weight tile are neighbours, so they run together
    // on one XCD and the weight tile comes from HBM once.  Taken
    // M-tile-major, an expert whose items straddle two rounds of the XCD's
    // blocks reads its weights twice (measured at prefill: 6.9-7.0 GB read
    // per launch, against 5.6-5.7 GB in this order).
    auto load_item = [&](int i) __attribute__((always_inline)) {
        const int w = item_w(i);
        const int t = w / nN;
        const i32x4_t d = sload4(g.tt.tiles + t);
        if constexpr (SK) {
            return make_int4(d.x, d.y, d.z, (w % nN) * C::BN);
        } else {
            const int nt = d.w >> 16, t0 = t - (d.w & 0xFFFF);
            const int local = w - t0 * nN;
            const i32x4_t e = sload4(g.tt.tiles + t0 + local % nt);
            return make_int4(e.x, e.y, e.z, (local / nt) * C::BN);
        }
    };

    // NVFP4 weights, with block scales per 16 fan-in elements of a row or
    // (LMOE_NVFP4_2D) per 16 x 16 block
    constexpr bool FP4 = BFMT == LMOE_NVFP4 || BFMT == LMOE_NVFP4_2D;
    constexpr bool B_DMA = C::DMA && !FP4;
    static_assert(BFMT != LMOE_BF16_TILED || (C::DMA && C::BK == 64 && C::BN % 64 == 0),
                  "packed weights: LDS-DMA, K step 64, whole 64-row tiles");
    using SA = Slots<C, C::BM>;
    using SB = Slots<C, C::BN>;
    // NVFP4 weights: each weight row's K step is split over LPR lanes, EPL
    // elements (EPL/2 code bytes, EPL/16 scale bytes) per lane, loaded into
    // registers and decoded into the LDS tile.
    constexpr int LPR = C::NT / C::BN, EPL = C::BK / (LPR > 0 ? LPR : 1);
    static_assert(!FP4 || (C::NT % C::BN == 0 && (LPR == 2 || LPR == 4) && C::BK == 64),
                  "NVFP4 tiles: 2 or 4 lanes per weight row, K step 64");
    typedef uint32_t code_words_t __attribute__((ext_vector_type(EPL >= 16 ? EPL / 8 : 2)));

    // ---- fill side: pointers of the item whose K steps are being issued
    const uint16_t* a_ptr[SA::N];
    const uint16_t* b_ptr[FP4 ? 1 : SB::N];
    const uint8_t* c_ptr = nullptr;  // NVFP4: this lane's codes and scales
    const uint8_t* s_ptr = nullptr;
    int4 fdesc = load_item(0);
    int4 fnext = load_item(1);
    int f_item = 0, f_kt = item_kt0(0);
    // A row of sorted row p for slot j.  GATHER_SCALAR (DMA slots): the
    // slot's RPI rows are read with one scalar load of the permutation
    // (clamped inside [0, n_rows)) and each lane picks its row.
    constexpr int RPI = SA::RPI;
    static_assert(GATHER != GATHER_SCALAR || (C::DMA && (RPI == 8 || RPI == 16)), "scalar gather needs DMA slots");
    auto a_row = [&](int j, int row0, int rows) __attribute__((always_inline)) {
        const int p = row0 + min(SA::row(j, tid), rows - 1);
        if constexpr (GATHER == GATHER_NONE) {
            return p;
        } else if constexpr (GATHER == GATHER_SCALAR) {
            const int rb = __builtin_amdgcn_readfirstlane((wave * SA::CPW + j * 64) / C::CPR);
            const int q0 = __builtin_amdgcn_readfirstlane(min(row0 + rb, g.n_rows - RPI));
            const int idx = min(max(p - q0, 0), RPI - 1);
            int v;
            if constexpr (RPI == 8) {
                const i32x8_t r = sload8(g.a_row_map + q0);
                v = r[0];
#pragma unroll
                for (int t = 1; t < 8; ++t) v = (idx == t) ? r[t] : v;
            } else {
                const i32x16_t r = sload16(g.a_row_map + q0);
                v = r[0];
#pragma unroll
                for (int t = 1; t < 16; ++t) v = (idx == t) ? r[t] : v;
            }
            return v / g.a_row_div;
        } else {
            return g.a_row_map[p] / g.a_row_div;
        }
    };
    auto setup = [&](const int4& d) __attribute__((always_inline)) {
        const int e = d.x, row0 = d.y, rows = d.z, n0 = d.w;
#pragma unroll
        for (int j = 0; j < SA::N; ++j) {
            const int ar = a_row(j, row0, rows);
            a_ptr[j] = (const uint16_t*)g.A + (int64_t)ar * g.lda + SA::lchunk(j, tid) * 8;
        }
        if constexpr (FP4) {
            const int64_t n = (int64_t)e * N + min(n0 + tid / LPR, N - 1);
            c_ptr = g.B_codes + n * (K / 2) + (tid % LPR) * (EPL / 2);
            // 2-D blocks: N is a multiple of 16, so weight row n of the stack
            // has scale row n / 16 of [E][N/16][K/16].  A lane loads the
            // row's whole 4-byte scale word of a K step (4-byte aligned: K is
            // a multiple of 64 and the stack 16-byte aligned) and uses its
            // own EPL/16 bytes of it.
            const int64_t srow = BFMT == LMOE_NVFP4_2D ? n >> 4 : n;
            s_ptr = g.B_scales + srow * (K / 16);
        } else if constexpr (BFMT == LMOE_BF16_TILED) {
            // packed weights: the 4 KB fragment-ordered K step of each 32-row
            // block, the K steps of a block consecutive; LDS chunk q of the
            // tile (block q / 256 of the tile, chunk q % 256 of its K step)
            // comes from the same chunk of the packed step
#pragma unroll
            for (int j = 0; j < SB::N; ++j) {
                const int q = min(SB::chunk(j, tid), C::BN * C::CPR - 1);
                const int rb = min(n0 / 32 + q / 256, N / 32 - 1);
                b_ptr[j] = (const uint16_t*)g.B + (((int64_t)e * (N / 32) + rb) * nk * 256 + q % 256) * 8;
            }
        } else {
#pragma unroll
            for (int j = 0; j < SB::N; ++j) {
                const int64_t n = (int64_t)e * N + min(n0 + SB::row(j, tid), N - 1);
                b_ptr[j] = (const uint16_t*)g.B + n * K + SB::lchunk(j, tid) * 8;
            }
        }
    };
    setup(fdesc);

    u32x4_t ra[C::DMA ? 1 : SA::N], rb[B_DMA || FP4 ? 1 : SB::N];
    code_words_t rc;   // NVFP4: EPL codes
    uint32_t rs = 0;   // NVFP4: the weight row's 4 scale bytes of a K step
    // issues the next K step of the fill item into stage (As, Bs); with
    // SPLITB, Bs is the raw slot the NVFP4 codes and scale words go to
    auto fill_next = [&](u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
        if (f_kt == nk) {  // next item: its descriptor was fetched one item ahead
            ++f_item;
            f_kt = item_kt0(f_item);
            fdesc = fnext;
            setup(fdesc);
            fnext = load_item(f_item + 1);
        }
        const int kt = f_kt++;
        const int kk = kt * C::BK;
        if constexpr (FP4) {
            if constexpr (SPLITB) {
                // this thread's 16 code bytes to chunk tid, the row's scale word
                // to word tid of the slot: each wave stages exactly the rows it
                // decodes, so its own vmcnt orders the staging and the decode
                static_assert(EPL == 32, "SPLITB: 16 code bytes per thread");
                dma16(c_ptr + kt * (C::BK / 2), Bs + wave * 64);
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(s_ptr + kt * (C::BK / 16)),
                                                 (__attribute__((address_space(3))) void*)(Bs + C::NT + wave * 16), 4, 0, 0);
            } else {
                // register loads first, so waiting for them does not wait for the DMA
                rc = *reinterpret_cast<const code_words_t*>(c_ptr + kt * (C::BK / 2));
                rs = *reinterpret_cast<const uint32_t*>(s_ptr + kt * (C::BK / 16));
            }
        } else if constexpr (B_DMA) {
            // packed weights: K step kt of a 32-row block is 4 KB past step kt - 1
            const int bk = BFMT == LMOE_BF16_TILED ? kt * 32 * 64 : kk;
#pragma unroll
            for (int j = 0; j < SB::N; ++j)
                if (SB::active(j, tid)) dma16<C::B_NT ? 2 : 0>(b_ptr[j] + bk, SB::dst(Bs, wave, j));
        } else {
#pragma unroll
            for (int j = 0; j < SB::N; ++j) rb[j] = *reinterpret_cast<const u32x4_t*>(b_ptr[j] + kk);
        }
        if constexpr (C::DMA) {
#pragma unroll
            for (int j = 0; j < SA::N; ++j)
                if (SA::active(j, tid)) dma16(a_ptr[j] + kk, SA::dst(As, wave, j));
        } else {
#pragma unroll
            for (int j = 0; j < SA::N; ++j) ra[j] = *reinterpret_cast<const u32x4_t*>(a_ptr[j] + kk);
        }
    };
    // finishes the move of a K step: staged registers to LDS; NVFP4 decoded
    // into the weight tile Bs (with SPLITB from the raw slot Raw)
    auto land = [&](u32x4_t* As, u32x4_t* Bs, const u32x4_t* Raw = nullptr) __attribute__((always_inline)) {
        if constexpr (!C::DMA) {
#pragma unroll
            for (int j = 0; j < SA::N; ++j) As[lds_idx<C>(SA::row(j, tid), SA::lchunk(j, tid))] = ra[j];
        }
        if constexpr (FP4) {
            code_words_t codes = rc;
            uint32_t sw = rs;
            if constexpr (SPLITB) {
                const u32x4_t v = Raw[tid];
                codes = code_words_t{v[0], v[1], v[2], v[3]};
                sw = reinterpret_cast<const uint32_t*>(Raw + C::NT)[tid];
            }
            static_for<EPL / 8>([&](auto wc) __attribute__((always_inline)) {
                constexpr int w = decltype(wc)::value;  // 8 elements; scale block w / 2
                float pw, mt;
                e4m3_parts((sw >> (8 * ((tid % LPR) * (EPL / 16) + w / 2))) & 0xFFu, pw, mt);
                Bs[lds_idx<C>(tid / LPR, (tid % LPR) * (EPL / 8) + w)] = decode_e2m1x8(codes[w], pw, mt);
            });
        } else if constexpr (!B_DMA) {
#pragma unroll
            for (int j = 0; j < SB::N; ++j) Bs[lds_idx<C>(SB::row(j, tid), SB::lchunk(j, tid))] = rb[j];
        }
    };

    // ---- multiply side: the item whose K steps are being multiplied, and its
    // epilogue scale (the NVFP4 tensor scale, 1 for dense weights).
    int4 mdesc = fdesc;
    float mscale = 1.0f;
    auto fetch_scale = [&](const int4& d) __attribute__((always_inline)) {
        if constexpr (FP4) mscale = sload_f32(g.B_ts + d.x);
    };
    fetch_scale(mdesc);
    auto epilogue = [&](const int4& d, f32x16_t (&acc)[C::TM][C::TN]) __attribute__((always_inline)) {
        const int row0 = d.y, rows = d.z, n0 = d.w;
        static_for<C::TM>([&](auto tmc) __attribute__((always_inline)) {
            constexpr int tm = decltype(tmc)::value;
            const int ml = wm * C::WM + tm * 32 + (lane & 31);
            if (ml < rows) {
                uint16_t* crow = (uint16_t*)g.C + (int64_t)(row0 + ml) * g.ldc;
                static_for<C::TN * 4>([&](auto tqc) __attribute__((always_inline)) {
                    constexpr int tn = decltype(tqc)::value / 4, q = decltype(tqc)::value % 4;
                    const int n = n0 + wn * C::WN + tn * 32 + q * 8 + (lane >> 5) * 4;
                    if (n < N) {
                        float v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v[i] = acc[tm][tn][q * 4 + i] * mscale;
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
                });
            }
        });
    };

    // Tail part: the block stores its partial sums (thread-fragment order,
    // coalesced; rows past the item's end are skipped), then counts itself
    // in; the last of the item's P blocks adds the partials in part order
    // (its own from registers) and runs the epilogue.  Every block of an
    // item takes the same additions in the same order, so the result does
    // not depend on which one finishes last.
    // The partials move through device-coherent (agent-scope) stores and
    // loads, which bypass the per-XCD L2 copies; the stores have completed
    // (vmcnt 0) before the block's arrival is counted.  Fences would write
    // back and invalidate whole L2s instead.
    auto sk_finish = [&](const int4& d, f32x16_t (&acc)[C::TM][C::TN]) __attribute__((always_inline)) {
        constexpr int NF4 = C::TM * C::TN * 4;
        const int rows = d.z, b0 = blockIdx.x - blockIdx.x % sk_P, me = blockIdx.x - b0;
        // two 64-bit words (4 floats) per thread and fragment quad j
        auto part_of = [&](int b) {
            return reinterpret_cast<uint64_t*>(g.sk_part) + (int64_t)b * (NF4 * C::NT * 2);
        };
        auto row_ok = [&](int j) { return wm * C::WM + (j / 4 / C::TN) * 32 + (lane & 31) < rows; };
        auto pack2 = [](float a, float b) {
            return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
        };
        uint64_t* mine = part_of(blockIdx.x);
        static_for<NF4>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value, r = (j % 4) * 4;
            const f32x16_t& a = acc[j / 4 / C::TN][(j / 4) % C::TN];
            uint64_t* at = mine + ((int64_t)j * C::NT + tid) * 2;
            if (row_ok(j)) {
                __hip_atomic_store(at, pack2(a[r], a[r + 1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(at + 1, pack2(a[r + 2], a[r + 3]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        });
        __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
        __syncthreads();
        if (tid == 0) {
            const int before =
                __hip_atomic_fetch_add(g.tt.sk_count + sk_t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sk_last = (before == sk_P - 1);
        }
        __syncthreads();
        if (!sk_last) return;
        // parts in order, one part's loads in flight at a time (few registers)
        float sum[NF4][4];
        for (int p = 0; p < sk_P; ++p) {
            uint64_t v[NF4][2];
            if (p != me) {
                const uint64_t* src = part_of(b0 + p);
                static_for<NF4>([&](auto jc) __attribute__((always_inline)) {
                    constexpr int j = decltype(jc)::value;
                    const uint64_t* at = src + ((int64_t)j * C::NT + tid) * 2;
                    if (row_ok(j)) {
                        v[j][0] = __hip_atomic_load(at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        v[j][1] = __hip_atomic_load(at + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                });
            }
            static_for<NF4>([&](auto jc) __attribute__((always_inline)) {
                constexpr int j = decltype(jc)::value, r = (j % 4) * 4;
                if (!row_ok(j)) return;
                const f32x16_t& a = acc[j / 4 / C::TN][(j / 4) % C::TN];
                float f[4];
                if (p == me) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) f[t] = a[r + t];
                } else {
                    f[0] = __uint_as_float((uint32_t)v[j][0]);
                    f[1] = __uint_as_float((uint32_t)(v[j][0] >> 32));
                    f[2] = __uint_as_float((uint32_t)v[j][1]);
                    f[3] = __uint_as_float((uint32_t)(v[j][1] >> 32));
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) sum[j][t] = p == 0 ? f[t] : sum[j][t] + f[t];
            });
        }
        static_for<NF4>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value, r = (j % 4) * 4;
            if (!row_ok(j)) return;
            f32x16_t& a = acc[j / 4 / C::TN][(j / 4) % C::TN];
#pragma unroll
            for (int t = 0; t < 4; ++t) a[r + t] = sum[j][t];
        });
        epilogue(d, acc);
        if (tid == 0) __hip_atomic_store(g.tt.sk_count + sk_t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    constexpr int S = C::STAGES, STG = C::STAGE_CHUNKS, AOFF = C::BM * C::CPR;
    constexpr int PER_TILE = (C::DMA && B_DMA) ? SA::N + SB::N : 0;
    constexpr int MAXAHEAD = PER_TILE > 0 ? S - 2 : 0;
    // whole items through two DMA stages (the 192-row tiles): the late-barrier loop below
    constexpr bool LATE = !SPLITB && !SK && S == 2 && PER_TILE > 0;
    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    if constexpr (SPLITB) {
        // NVFP4, three A stages.  Step q multiplies A stage q % 3 and decoded
        // weight slot q % 2.  Its iteration waits for A stage q, issues step
        // q + 2 (A by DMA; the raw codes and scale words by DMA into raw slot
        // q % 2, the one step q's decode has finished with), multiplies, then
        // waits for step q + 1's staging (issued an iteration earlier) and
        // decodes it into weight slot (q + 1) % 2, last read by step q - 1,
        // which every wave finished before this iteration's barrier.  A
        // thread issues the same PT DMA instructions per step (A, codes,
        // scales), so waiting for vmcnt(PT) leaves exactly the newest step in
        // flight.  Every iteration issues a step, also past the end (the fill
        // side then re-reads the block's last item, at valid addresses, into
        // stages nothing multiplies), so the count never changes.
        constexpr int ACH = C::BM * C::CPR, BCH = C::BN * C::CPR, PT = SA::N + 2;
        u32x4_t* const bring = ring + S * ACH;
        u32x4_t* const raw = bring + 2 * BCH;
        fill_next(ring, raw);
        fill_next(ring + ACH, raw + RAW);
        wait_vmcnt<PT>();
        land(nullptr, bring, raw);
        int m_item = 0, m_kt = 0;
        for (int q = 0; q < total; ++q) {
            asm volatile("" ::: "memory");
            if (q + 1 < total)
                wait_vmcnt_lgkm0<PT>();
            else
                __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            fill_next(ring + ((q + 2) % S) * ACH, raw + (q & 1) * RAW);
            mma_tile<C>(ring + (q % S) * ACH, bring + (q & 1) * BCH, acc, wm, wn, lane);
            if (q + 1 < total) {
                wait_vmcnt<PT>();
                asm volatile("" ::: "memory");
                land(nullptr, bring + ((q + 1) & 1) * BCH, raw + ((q + 1) & 1) * RAW);
            }
            if (++m_kt == nk) {
                epilogue(mdesc, acc);
                zero_acc<C>(acc);
                ++m_item;
                m_kt = 0;
                mdesc = nk >= S - 1 ? fdesc : load_item(m_item);
                fetch_scale(mdesc);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the steps issued past the end have landed
        return;
    }
    if constexpr (LATE) {
        // Two stages, both operands by DMA, the barrier late: step q's last
        // 16-wide sub-step waits for step q + 1's tile (the only DMA in
        // flight), then the barrier, after which every wave holds step q's
        // last fragments in registers, so stage q % 2 takes step q + 2's
        // DMA; step q + 1's first fragments are read under the last
        // sub-step's MFMAs instead of after the next barrier.
        constexpr int KS = C::BK / 16, NM = C::TM * C::TN, NR = C::TM + C::TN;
        bf16x8_t af[2][C::TM], bfr[2][C::TN];
        // A fragment row starts at a multiple of 32, so the swizzle of every
        // row this lane reads is that of lane & 31: one address per operand
        // and sub-step, the 32-row blocks at constant offsets from it
        static_assert(C::CPR == 8 && C::WM % 32 == 0 && C::WN % 32 == 0, "late-barrier loop: K step 64");
        const int l31 = lane & 31, hi = lane >> 5, sw = swz_bits<C::CPR>(l31);
        const int arow = (wm * C::WM + l31) * C::CPR, brow = (wn * C::WN + l31) * C::CPR;
        auto read = [&](const u32x4_t* As, const u32x4_t* Bs, int ks, int b) __attribute__((always_inline)) {
            const int c = (ks * 2 + hi) ^ sw;
            const u32x4_t* pa = As + arow + c;
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm) af[b][tm] = as_bf16x8(pa[tm * 32 * C::CPR]);
            if constexpr (BFMT == LMOE_BF16_TILED) {  // fragment-ordered weight tile
                const u32x4_t* pb = Bs + (wn * C::WN / 32 * KS + ks) * 64 + lane;
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) bfr[b][tn] = as_bf16x8(pb[tn * KS * 64]);
            } else {
                const u32x4_t* pb = Bs + brow + c;
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) bfr[b][tn] = as_bf16x8(pb[tn * 32 * C::CPR]);
            }
        };
        auto mfmas = [&](int b) __attribute__((always_inline)) {
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = mfma32x32x16(bfr[b][tn], af[b][tm], acc[tm][tn]);
        };
        auto interleave = [&]() __attribute__((always_inline)) {  // MFMA m, then its share of the reads
            static_for<NM>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value, r = (m + 1) * NR / NM - m * NR / NM;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
            });
        };
        fill_next(ring, ring + AOFF);
        if (total > 1) {
            fill_next(ring + STG, ring + STG + AOFF);
            wait_vmcnt<PER_TILE>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        read(ring, ring + AOFF, 0, 0);
        int m_item = 0, m_kt = 0;
        for (int q = 0; q < total; ++q) {
            u32x4_t* const cs = ring + (q & 1) * STG;
            const u32x4_t* const ns = ring + ((q + 1) & 1) * STG;
            static_for<KS>([&](auto kc) __attribute__((always_inline)) {
                constexpr int ks = decltype(kc)::value, b = ks & 1;
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this sub-step's fragments
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (ks + 1 < KS) {
                    read(cs, cs + AOFF, ks + 1, b ^ 1);
                    mfmas(b);
                    interleave();
                } else {
                    // also on the block's last step (the reads then fetch a
                    // stage nothing multiplies): no branch around the MFMAs
                    asm volatile("" ::: "memory");
                    wait_vmcnt<0>();  // step q + 1 (and any epilogue stores) complete
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    // stage q % 2 is free: every wave holds step q's last
                    // fragments in registers
                    if (q + 2 < total) fill_next(cs, cs + AOFF);
                    __builtin_amdgcn_sched_barrier(0);
                    read(ns, ns + AOFF, 0, b ^ 1);
                    mfmas(b);
                    interleave();
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if (++m_kt == nk) {
                epilogue(mdesc, acc);
                zero_acc<C>(acc);
                ++m_item;
                m_kt = 0;
                // the fill side is on the next item already unless items
                // are one K step long (it is two steps ahead here)
                mdesc = nk >= 2 ? fdesc : load_item(m_item);
                fetch_scale(mdesc);
            }
        }
        return;
    }
#pragma unroll
    for (int st = 0; st < S - 1; ++st) {
        if (st < total) {
            fill_next(ring + st * STG, ring + st * STG + AOFF);
            land(ring + st * STG, ring + st * STG + AOFF);
        }
    }
    int cur = 0, nxt = S - 1, m_item = 0, m_kt = item_kt0(0), m_kt0 = m_kt;
    for (int q = 0; q < total; ++q) {
        wait_tiles_barrier<MAXAHEAD, PER_TILE>(min(MAXAHEAD, total - 1 - q));
        const bool more = q + S - 1 < total;
        u32x4_t* ns = ring + nxt * STG;
        if (more) fill_next(ns, ns + AOFF);
        u32x4_t* cs = ring + cur * STG;
        mma_tile<C, BFMT == LMOE_BF16_TILED>(cs, cs + AOFF, acc, wm, wn, lane);
        if (more) land(ns, ns + AOFF);
        cur = (cur + 1 == S) ? 0 : cur + 1;
        nxt = (nxt + 1 == S) ? 0 : nxt + 1;
        ++m_kt;
        // a tail part is the block's last item and ends the loop; it is
        // finished after the loop, which keeps the loop free of its stores,
        // atomics and barriers (and of the waits the compiler adds for them)
        if (SK && q == total - 1 && !(m_kt0 == 0 && m_kt == nk)) break;
        if (m_kt == nk) {
            epilogue(mdesc, acc);
            zero_acc<C>(acc);
            // the fill side is on the next item already unless items are
            // shorter than the prefetch distance
            ++m_item;
            m_kt = m_kt0 = item_kt0(m_item);
            mdesc = nk >= S - 1 ? fdesc : load_item(m_item);
            fetch_scale(mdesc);
        }
    }
    if constexpr (SK) {
        if (m_item < n_items && sk_t >= 0) sk_finish(mdesc, acc);
    }
}

// Prefill expert GEMM with the packed weights streamed into registers.
//
// 192 x 256 tiles over 8 waves of 192 x 32: each wave owns one 32-row block
// of weights (output columns) of the tile and every one of its 192
// activation rows.  The packed layout keeps each block's K step as four
// 1 KB sub-step fragments in lane order, so a wave reads its weight
// fragments straight into the registers the MFMAs take with four contiguous
// 1 KB loads per K step: the weights need no LDS and no barrier.  (The same
// fragments read from a row-major stack touch 32 rows per load; measured on
// L2-resident data that streams 3.4 times slower per byte.)  The gathered
// activation rows, which all 8 waves read, go through a ring of NB = D + 1
// LDS stages by DMA (24 KB per K step).  The barrier comes late: the last
// 16-wide sub-step of step q waits for step q + 1's loads and passes the
// barrier, refills stage q with step q + NB's activation rows, reads step
// q + 1's first fragments under its own MFMAs and then loads step q + NB's
// weights into the register set those MFMAs have just used.
//
// Every thread issues the same PT loads per step, also past the block's
// last step (the fill side then re-reads the last item, at valid
// addresses, into stages and registers nothing uses), so waiting for
// vmcnt((D - 1) PT) leaves exactly steps q + 2 .. q + D in flight.
// Epilogue stores issued since count among the outstanding operations too,
// so after an epilogue that wait can only be longer than needed, never
// short.  The output tile leaves through LDS (see the epilogue) in whole
// 512-byte rows.  The work list and the items' order are the persistent
// grouped GEMM's (whole items, N-tile-major within an expert).
template <int BFMT, int GATHER, int D>
__global__ __launch_bounds__(512, 1) void grouped_gemm_breg_kernel(GroupedGemm g, int nN) {
    using C = MfmaCfg<192, 256, 1, 8, true, 64, D + 1>;
    using SA = Slots<C, C::BM>;
    constexpr int NB = D + 1, ACH = C::BM * C::CPR, KS = C::BK / 16;
    constexpr int PT = SA::N + KS;  // vector-memory instructions per step and thread
    static_assert(BFMT == LMOE_BF16_TILED, "packed bf16 weights");
    static_assert(C::TN == 1 && C::WN == 32 && SA::CPW % 64 == 0, "8 waves of 192 x 32");
    static_assert(D >= 1 && D * PT < 64, "vmcnt range");
    // one LDS array for the activation ring and the output staging (with a
    // second array the compiler waits for all DMA in flight before every
    // LDS read, unable to tell the two apart; with one it still waits once
    // per item, before the first staging write)
    constexpr int CPITCH = C::BN * 2 + 16;  // bytes per output row staged in LDS
    __shared__ u32x4_t ring[NB * ACH + C::BM / 2 * CPITCH / 16];
    uint8_t* const cbuf = reinterpret_cast<uint8_t*>(ring + NB * ACH);
    const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, hi = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = g.N, K = g.K, nk = K / C::BK;

    const int W = *g.tt.tile_count * nN;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, nbx = gridDim.x >> 3;
    const int per = W >> 3, rem = W & 7;
    const int first = x * per + min(x, rem);
    const int end = first + per + (x < rem ? 1 : 0);
    if (first + slot >= end) return;
    const int n_items = (end - 1 - first - slot) / nbx + 1;
    const int total = n_items * nk;
    const int w_first = first + slot;
    // descriptor {expert, first sorted row, rows, n0} of this block's item i
    // (clamped to the last), the expert's items taken N-tile-major
    auto load_item = [&](int i) __attribute__((always_inline)) {
        const int w = __builtin_amdgcn_readfirstlane(w_first + min(i, n_items - 1) * nbx);
        const int t = w / nN;
        const i32x4_t d = sload4(g.tt.tiles + t);
        const int nt = d.w >> 16, t0 = t - (d.w & 0xFFFF);
        const int local = w - t0 * nN;
        const i32x4_t e = sload4(g.tt.tiles + t0 + local % nt);
        return make_int4(e.x, e.y, e.z, (local / nt) * C::BN);
    };

    // ---- fill side
    constexpr int RPI = SA::RPI;
    static_assert(GATHER != GATHER_SCALAR || RPI == 8, "scalar gather: 8 rows per DMA instruction");
    auto a_row = [&](int j, int row0, int rows) __attribute__((always_inline)) {
        const int p = row0 + min(SA::row(j, tid), rows - 1);
        if constexpr (GATHER == GATHER_NONE) {
            return p;
        } else if constexpr (GATHER == GATHER_SCALAR) {
            const int rb = __builtin_amdgcn_readfirstlane((wave * SA::CPW + j * 64) / C::CPR);
            const int q0 = __builtin_amdgcn_readfirstlane(min(row0 + rb, g.n_rows - RPI));
            const int idx = min(max(p - q0, 0), RPI - 1);
            const i32x8_t r = sload8(g.a_row_map + q0);
            int v = r[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) v = (idx == t) ? r[t] : v;
            return v / g.a_row_div;
        } else {
            return g.a_row_map[p] / g.a_row_div;
        }
    };
    // this lane's chunk of the wave's weight block: sub-step ks of K step kt
    // at b_ptr + kt * 2048 + ks * 512 (bf16 elements)
    const uint16_t* a_ptr[SA::N];
    const uint16_t* b_ptr;
    auto setup = [&](const int4& d) __attribute__((always_inline)) {
        const int e = d.x, row0 = d.y, rows = d.z, n0 = d.w;
#pragma unroll
        for (int j = 0; j < SA::N; ++j) {
            const int ar = a_row(j, row0, rows);
            a_ptr[j] = (const uint16_t*)g.A + (int64_t)ar * g.lda + SA::lchunk(j, tid) * 8;
        }
        const int rb = min(n0 / 32 + wave, N / 32 - 1);
        b_ptr = (const uint16_t*)g.B + (((int64_t)e * (N / 32) + rb) * nk * 256 + lane) * 8;
    };
    int4 fdesc = load_item(0);
    int4 fnext = load_item(1);
    int f_item = 0, f_kt = 0;
    setup(fdesc);
    u32x4_t breg[NB][KS];
    // issue the next K step of the fill item: fill_a its activation rows by
    // DMA into stage As (moving to the next item first when the current one
    // is done), fill_b its weights into registers br; no other vector-memory
    // operation comes between the two
    int f_kk = 0;
    auto fill_a = [&](u32x4_t* As) __attribute__((always_inline)) {
        if (f_kt == nk) {  // next item: its descriptor was fetched one item ahead
            ++f_item;
            f_kt = 0;
            fdesc = fnext;
            setup(fdesc);
            fnext = load_item(f_item + 1);
        }
        f_kk = f_kt++;
#pragma unroll
        for (int j = 0; j < SA::N; ++j) dma16(a_ptr[j] + f_kk * C::BK, SA::dst(As, wave, j));
    };
    auto fill_b = [&](u32x4_t (&br)[KS]) __attribute__((always_inline)) {
        const uint16_t* bp = b_ptr + f_kk * 2048;
#pragma unroll
        for (int s = 0; s < KS; ++s) br[s] = *reinterpret_cast<const u32x4_t*>(bp + s * 512);
    };

    // ---- multiply side
    f32x16_t acc[C::TM][1];
    zero_acc<C>(acc);
    bf16x8_t af[2][C::TM];
    const int arow = l31 * C::CPR, asw = swz_bits<8>(l31);  // A row tm * 32 + l31 has l31's swizzle
    auto read = [&](const u32x4_t* As, int ks, int b) __attribute__((always_inline)) {
        const u32x4_t* pa = As + arow + ((ks * 2 + hi) ^ asw);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) af[b][tm] = as_bf16x8(pa[tm * 32 * C::CPR]);
    };
    // One K step, the barrier late: sub-step ks reads the fragments of
    // ks + 1 under its MFMAs.  The last sub-step first waits for step q + 1
    // (its own loads, then the barrier for everyone's), refills stage q with
    // step q + NB's activation rows (every wave has read stage q's last
    // fragments by then), reads step q + 1's first fragments under its
    // MFMAs, and then loads step q + NB's weights into the register set
    // those MFMAs have just taken theirs from.
    auto mma = [&](u32x4_t* As, u32x4_t (&br)[KS], const u32x4_t* Asn) __attribute__((always_inline)) {
        static_for<KS>([&](auto kc) __attribute__((always_inline)) {
            constexpr int ks = decltype(kc)::value, b = ks & 1;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this sub-step's fragments
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ks + 1 < KS) {
                read(As, ks + 1, b ^ 1);
            } else {
                asm volatile("" ::: "memory");
                wait_vmcnt<(D - 1) * PT>();    // this thread's loads of step q + 1
                __builtin_amdgcn_s_barrier();  // everyone's
                asm volatile("" ::: "memory");
                fill_a(As);
                __builtin_amdgcn_sched_barrier(0);
                read(Asn, 0, b ^ 1);
            }
            const bf16x8_t bf = as_bf16x8(br[ks]);
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm) acc[tm][0] = mfma32x32x16(bf, af[b][tm], acc[tm][0]);
            static_for<C::TM>([&](auto) __attribute__((always_inline)) {  // MFMA tm, then fragment tm
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            });
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ks + 1 == KS) {
                fill_b(br);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    // Barrier for LDS traffic only: this wave's LDS accesses complete, then
    // the workgroup barrier.  (__syncthreads would also wait for every load
    // in flight, the steps prefetched for the next item.)
    auto lds_barrier = []() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // The output tile goes out through LDS, half of its rows at a time: each
    // wave writes its 32 columns of 96 rows (a lane's 4 consecutive values
    // per 8-byte write), then every thread stores 16-byte pieces of whole
    // 512-byte output rows, so a wave's store covers 2 rows instead of 32.
    // Rows are padded by 16 bytes in LDS.  Two barriers per half: the
    // writes are complete before the reads, the reads before the next
    // half's writes.
    auto epilogue = [&](const int4& d) __attribute__((always_inline)) {
        const int row0 = d.y, rows = d.z, n0 = d.w;
        static_for<2>([&](auto hc) __attribute__((always_inline)) {
            constexpr int half = decltype(hc)::value;
            static_for<C::TM / 2>([&](auto tc) __attribute__((always_inline)) {
                constexpr int t = decltype(tc)::value, tm = half * (C::TM / 2) + t;
                uint32_t* crow = reinterpret_cast<uint32_t*>(cbuf) + (t * 32 + l31) * (CPITCH / 4);
                static_for<4>([&](auto qc) __attribute__((always_inline)) {
                    constexpr int q = decltype(qc)::value;
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = acc[tm][0][q * 4 + i];
                        if (g.epi == EPI_RELU2) {
                            v[i] = fmaxf(v[i], 0.f);
                            v[i] *= v[i];
                        }
                    }
                    lds_write_b64(crow + (wave * C::WN + q * 8 + hi * 4) / 2, pack_bf16x2(v[0], v[1]),
                                  pack_bf16x2(v[2], v[3]));
                });
            });
            lds_barrier();
            constexpr int PIECES = C::BM / 2 * (C::BN / 8);  // 16-byte pieces of the half tile
            constexpr int RPP = C::NT / (C::BN / 8);         // rows per pass
            static_assert(PIECES % C::NT == 0, "whole passes");
            const int r0 = tid / (C::BN / 8), p = tid % (C::BN / 8);
            u32x4_t v[PIECES / C::NT];
            lds_read_b128xn<PIECES / C::NT, RPP * CPITCH>(cbuf + r0 * CPITCH + p * 16, v);
#pragma unroll
            for (int i = 0; i < PIECES / C::NT; ++i) {
                const int ml = half * (C::BM / 2) + r0 + i * RPP;
                if (ml < rows)
                    *reinterpret_cast<u32x4_t*>((uint16_t*)g.C + (int64_t)(row0 + ml) * g.ldc + n0 + p * 8) = v[i];
            }
            lds_barrier();
        });
    };

    // steps 0 .. D in flight, then step 0's first fragments
    static_for<NB>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        fill_a(ring + u * ACH);
        fill_b(breg[u]);
    });
    asm volatile("" ::: "memory");
    wait_vmcnt<D * PT>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read(ring, 0, 0);
    int4 mdesc = fdesc;
    int m_kt = 0;
    for (int q0 = 0; q0 < total; q0 += NB) {  // total is a multiple of NB (nk is)
        static_for<NB>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            mma(ring + u * ACH, breg[u], ring + ((u + 1) % NB) * ACH);
            if (++m_kt == nk) {
                epilogue(mdesc);
                zero_acc<C>(acc);
                m_kt = 0;
                mdesc = fdesc;  // the fill side is NB <= nk steps ahead, in the next item
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);  // the steps issued past the end have landed
}

// Prefill NVFP4 expert GEMM with the weights decoded in registers.
//
// 192 x 256 tiles over 8 waves of 192 x 32: each wave owns one 32-row
// block of weights and decodes it alone (with waves of 96 x 64 two waves
// decoded every block, and the decode's VALU work set the pace; reading
// all 192 activation rows' fragments from LDS costs less).  Each K step
// moves by LDS-DMA into a ring of NB = D + 1 stages: the gathered activation rows
// (24 KB) and the tile's raw weight codes and scale words (thread t stages
// 16 code bytes of weight row t / 2, half t % 2, and that row's 4-byte
// scale word: 10 KB).  A lane then reads from LDS the 32 codes of its own
// weight row that its MFMA fragments of the step hold, with the row's
// scale word, and decodes a sub-step's 8 codes to bf16 in registers right
// before the MFMAs that take them: no decoded weight tile is written to or
// read from LDS.  The K positions inside a step are renumbered (sub-step s
// of lane half h takes k = 32 h + 8 s .. +8, the activation fragments
// read from LDS take the same k), which leaves the product unchanged and
// makes a lane's codes of a step one 16-byte chunk.  Step q's last
// sub-step waits for step q + 1's DMA, passes the barrier, issues step
// q + NB into stage q, and reads step q + 1's codes and first activation
// fragments under its MFMAs; the decode of that first sub-step follows
// (the compiler places it right before the MFMAs that take it).  Every thread issues the same PT DMA instructions per step,
// also past the block's last step (the fill side then re-reads the last
// item at valid addresses into stages nothing uses), so waiting for
// vmcnt((D - 1) PT) leaves exactly steps q + 2 .. q + D in flight
// (epilogue stores issued since can only make that wait longer).  The
// work list and the items' order are the persistent
// grouped GEMM's (whole items, N-tile-major within an expert).
template <int BFMT, int GATHER, int D>
__global__ __launch_bounds__(512, 1) void grouped_gemm_nvfp4_reg_kernel(GroupedGemm g, int nN) {
    using C = MfmaCfg<192, 256, 1, 8, true, 64, D + 1>;
    using SA = Slots<C, C::BM>;
    constexpr int NB = D + 1, ACH = C::BM * C::CPR, KS = C::BK / 16;
    // raw slot: a 16-byte code chunk per thread, then a scale word per thread
    constexpr int RAWC = C::NT + C::NT / 4;
    constexpr int PT = SA::N + 2;  // DMA instructions per step and thread
    static_assert(BFMT == LMOE_NVFP4 || BFMT == LMOE_NVFP4_2D, "NVFP4 weights");
    static_assert(C::WN % 32 == 0 && KS == 4 && SA::CPW % 64 == 0 && C::NT == 2 * C::BN,
                  "waves of whole 32-row weight blocks, two threads per weight row");
    static_assert(D >= 1 && D * PT < 64, "vmcnt range");
    // one LDS array for the ring and the output staging (see the epilogue)
    constexpr int CPITCH = C::BN * 2 + 16;  // bytes per output row staged in LDS
    __shared__ u32x4_t ring[NB * (ACH + RAWC) + 32 * CPITCH / 16];
    uint8_t* const cbuf = reinterpret_cast<uint8_t*>(ring + NB * (ACH + RAWC));
    const int tid = threadIdx.x, lane = tid & 63, l31 = lane & 31, hi = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int N = g.N, K = g.K, nk = K / C::BK;

    const int W = *g.tt.tile_count * nN;
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, nbx = gridDim.x >> 3;
    const int per = W >> 3, rem = W & 7;
    const int first = x * per + min(x, rem);
    const int end = first + per + (x < rem ? 1 : 0);
    if (first + slot >= end) return;
    const int n_items = (end - 1 - first - slot) / nbx + 1;
    const int total = n_items * nk;
    const int w_first = first + slot;
    // descriptor {expert, first sorted row, rows, n0} of this block's item i
    // (clamped to the last), the expert's items taken N-tile-major
    auto load_item = [&](int i) __attribute__((always_inline)) {
        const int w = __builtin_amdgcn_readfirstlane(w_first + min(i, n_items - 1) * nbx);
        const int t = w / nN;
        const i32x4_t d = sload4(g.tt.tiles + t);
        const int nt = d.w >> 16, t0 = t - (d.w & 0xFFFF);
        const int local = w - t0 * nN;
        const i32x4_t e = sload4(g.tt.tiles + t0 + local % nt);
        return make_int4(e.x, e.y, e.z, (local / nt) * C::BN);
    };

    // ---- fill side
    constexpr int RPI = SA::RPI;
    static_assert(GATHER != GATHER_SCALAR || RPI == 8, "scalar gather: 8 rows per DMA instruction");
    auto a_row = [&](int j, int row0, int rows) __attribute__((always_inline)) {
        const int p = row0 + min(SA::row(j, tid), rows - 1);
        if constexpr (GATHER == GATHER_NONE) {
            return p;
        } else if constexpr (GATHER == GATHER_SCALAR) {
            const int rb = __builtin_amdgcn_readfirstlane((wave * SA::CPW + j * 64) / C::CPR);
            const int q0 = __builtin_amdgcn_readfirstlane(min(row0 + rb, g.n_rows - RPI));
            const int idx = min(max(p - q0, 0), RPI - 1);
            const i32x8_t r = sload8(g.a_row_map + q0);
            int v = r[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) v = (idx == t) ? r[t] : v;
            return v / g.a_row_div;
        } else {
            return g.a_row_map[p] / g.a_row_div;
        }
    };
    const uint16_t* a_ptr[SA::N];
    const uint8_t* c_ptr;  // this thread's 16 code bytes of K step 0: weight row tid / 2, half tid % 2
    const uint8_t* s_ptr;  // that row's scale words
    auto setup = [&](const int4& d) __attribute__((always_inline)) {
        const int e = d.x, row0 = d.y, rows = d.z, n0 = d.w;
#pragma unroll
        for (int j = 0; j < SA::N; ++j) {
            const int ar = a_row(j, row0, rows);
            a_ptr[j] = (const uint16_t*)g.A + (int64_t)ar * g.lda + SA::lchunk(j, tid) * 8;
        }
        const int64_t n = (int64_t)e * N + min(n0 + (tid >> 1), N - 1);
        c_ptr = g.B_codes + n * (K / 2) + 16 * (tid & 1);
        // 2-D blocks: N is a multiple of 16, so weight row n of the stack
        // has scale row n / 16 of [E][N/16][K/16]
        s_ptr = g.B_scales + (BFMT == LMOE_NVFP4_2D ? n >> 4 : n) * (K / 16);
    };
    int4 fdesc = load_item(0);
    int4 fnext = load_item(1);
    int f_item = 0, f_kt = 0;
    setup(fdesc);
    // issues the next K step of the fill item by DMA: the activation rows
    // into stage As, the codes and scale words into raw slot Raw
    auto fill = [&](u32x4_t* As, u32x4_t* Raw) __attribute__((always_inline)) {
        if (f_kt == nk) {  // next item: its descriptor was fetched one item ahead
            ++f_item;
            f_kt = 0;
            fdesc = fnext;
            setup(fdesc);
            fnext = load_item(f_item + 1);
        }
        const int kt = f_kt++;
#pragma unroll
        for (int j = 0; j < SA::N; ++j) dma16(a_ptr[j] + kt * C::BK, SA::dst(As, wave, j));
        dma16(c_ptr + kt * (C::BK / 2), Raw + wave * 64);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(s_ptr + kt * (C::BK / 16)),
                                         (__attribute__((address_space(3))) void*)(Raw + C::NT + wave * 16), 4, 0, 0);
    };

    // ---- multiply side
    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    bf16x8_t af[2][C::TM], bfr[2][C::TN];
    const int arow = (wm * C::WM + l31) * C::CPR, asw = swz_bits<8>(l31);  // rows tm * 32 + l31: l31's swizzle
    // sub-step ks of lane half h: logical chunk 4 h + ks, k = 32 h + 8 ks .. +8
    auto read = [&](const u32x4_t* As, int ks, int b) __attribute__((always_inline)) {
        const u32x4_t* pa = As + arow + ((4 * hi + ks) ^ asw);
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) af[b][tm] = as_bf16x8(pa[tm * 32 * C::CPR]);
    };
    // the same k of the lane's weight row: code word ks, scale block 2 h + ks / 2
    // (byte ks / 2 of the scale word shifted right by 16 h)
    auto decode = [&](const u32x4_t (&bc)[C::TN], const uint32_t (&bsh)[C::TN], int ks, int b)
                      __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
            const float sc = (ks >> 1) ? __builtin_amdgcn_cvt_f32_fp8((int)bsh[tn], 1)
                                       : __builtin_amdgcn_cvt_f32_fp8((int)bsh[tn], 0);
            float pw, mt;
            e4m3_split_f32(sc, pw, mt);
            bfr[b][tn] = as_bf16x8(decode_e2m1x8(bc[tn][ks], pw, mt));
        }
    };
    // the lane's weight row of group tn: wn * 64 + tn * 32 + l31, its chunk
    // (and scale word) 2 row + half in the raw slot
    const int rraw = 2 * (wn * C::WN + l31) + hi;
    u32x4_t bc[C::TN];
    uint32_t bs[C::TN];
    auto read_raw = [&](const u32x4_t* Raw) __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
            bc[tn] = Raw[rraw + 64 * tn];
            bs[tn] = reinterpret_cast<const uint32_t*>(Raw + C::NT)[rraw + 64 * tn] >> (16 * hi);
        }
    };
    // One K step, the barrier late: sub-step ks reads and decodes the
    // fragments of ks + 1 under its MFMAs.  The last sub-step first waits
    // for step q + 1 (its own DMA, then the barrier for everyone's), refills
    // stage q with step q + NB (every wave has read stage q's codes and last
    // activation fragments by then), reads step q + 1's codes and first
    // activation fragments under its MFMAs, and then decodes their first
    // sub-step.
    auto mma = [&](u32x4_t* As, u32x4_t* Raw, const u32x4_t* Asn, const u32x4_t* Rawn)
                   __attribute__((always_inline)) {
        static_for<KS>([&](auto kc) __attribute__((always_inline)) {
            constexpr int ks = decltype(kc)::value, b = ks & 1;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this sub-step's activation fragments
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ks + 1 < KS) {
                read(As, ks + 1, b ^ 1);
                decode(bc, bs, ks + 1, b ^ 1);
            } else {
                asm volatile("" ::: "memory");
                wait_vmcnt<(D - 1) * PT>();    // this thread's loads of step q + 1
                __builtin_amdgcn_s_barrier();  // everyone's
                asm volatile("" ::: "memory");
                fill(As, Raw);
                __builtin_amdgcn_sched_barrier(0);
                read_raw(Rawn);
                read(Asn, 0, b ^ 1);
            }
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < C::TN; ++tn)
                    acc[tm][tn] = mfma32x32x16(bfr[b][tn], af[b][tm], acc[tm][tn]);
            if constexpr (ks + 1 < KS) {  // MFMA m, then a fragment read and a share of the decode
                static_for<C::TM * C::TN>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (m < C::TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                });
            } else {  // the codes first, then MFMA m and an activation fragment
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::TN, 0);
                static_for<C::TM * C::TN>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value;
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (m < C::TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ks + 1 == KS) {
                decode(bc, bs, 0, b ^ 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    float mscale = 1.0f;
    // Barrier for LDS traffic only (__syncthreads would also wait for the
    // steps prefetched for the next item).
    auto lds_barrier = []() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // The output tile leaves through LDS 32 rows at a time (the LDS left
    // beside the ring holds 32 padded rows): the waves that own those rows
    // write their values (a lane's 4 consecutive columns per 8-byte write),
    // then every thread stores 16-byte pieces of whole 512-byte rows, so a
    // wave's store covers 2 rows instead of 32.
    auto epilogue = [&](const int4& d) __attribute__((always_inline)) {
        const int row0 = d.y, rows = d.z, n0 = d.w;
        static_for<C::WAVES_M * C::TM>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value, tm = r % C::TM;
            if (wm == r / C::TM) {
                uint32_t* crow = reinterpret_cast<uint32_t*>(cbuf) + l31 * (CPITCH / 4);
                static_for<C::TN * 4>([&](auto tqc) __attribute__((always_inline)) {
                    constexpr int tn = decltype(tqc)::value / 4, q = decltype(tqc)::value % 4;
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = acc[tm][tn][q * 4 + i] * mscale;
                        if (g.epi == EPI_RELU2) {
                            v[i] = fmaxf(v[i], 0.f);
                            v[i] *= v[i];
                        }
                    }
                    lds_write_b64(crow + (wn * C::WN + tn * 32 + q * 8 + hi * 4) / 2, pack_bf16x2(v[0], v[1]),
                                  pack_bf16x2(v[2], v[3]));
                });
            }
            lds_barrier();
            constexpr int PIECES = 32 * (C::BN / 8);  // 16-byte pieces of 32 rows
            constexpr int RPP = C::NT / (C::BN / 8);  // rows per pass
            static_assert(PIECES % C::NT == 0, "whole passes");
            const int r0 = tid / (C::BN / 8), p = tid % (C::BN / 8);
            u32x4_t v[PIECES / C::NT];
            lds_read_b128xn<PIECES / C::NT, RPP * CPITCH>(cbuf + r0 * CPITCH + p * 16, v);
#pragma unroll
            for (int i = 0; i < PIECES / C::NT; ++i) {
                const int ml = r * 32 + r0 + i * RPP;
                if (ml < rows)
                    *reinterpret_cast<u32x4_t*>((uint16_t*)g.C + (int64_t)(row0 + ml) * g.ldc + n0 + p * 8) = v[i];
            }
            lds_barrier();
        });
    };

    // steps 0 .. D in flight, then step 0's codes, first fragments and first decode
    u32x4_t* const raw = ring + NB * ACH;
    static_for<NB>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        fill(ring + u * ACH, raw + u * RAWC);
    });
    asm volatile("" ::: "memory");
    wait_vmcnt<D * PT>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_raw(raw);
    read(ring, 0, 0);
    decode(bc, bs, 0, 0);
    int4 mdesc = fdesc;
    mscale = sload_f32(g.B_ts + mdesc.x);
    int m_kt = 0;
    for (int q0 = 0; q0 < total; q0 += NB) {  // total is a multiple of NB (nk is)
        static_for<NB>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value, un = (u + 1) % NB;
            mma(ring + u * ACH, raw + u * RAWC, ring + un * ACH, raw + un * RAWC);
            if (++m_kt == nk) {
                epilogue(mdesc);
                zero_acc<C>(acc);
                m_kt = 0;
                mdesc = fdesc;  // the fill side is NB <= nk steps ahead, in the next item
                mscale = sload_f32(g.B_ts + mdesc.x);
            }
        });
    }
    __builtin_amdgcn_s_waitcnt(0);  // the steps issued past the end have landed
}

// ---------------------------------------------------------------------------
// FP8 dense GEMM (the shared expert with E4M3 weights and activations)
// ---------------------------------------------------------------------------
//
// The LDS tile, DMA slots, swizzle and K loop are the bf16 GEMM's: a row's
// K step is 128 codes = 128 bytes = 8 chunks of 16 B, as 64 bf16 values
// are.  Each K step runs two 32x32x64 fp8 MFMAs per 32x32 block, twice the
// K of the bf16 step for the same bytes and the same MFMA issue time.
// With splits > 1 (few-row calls) block (tile, split) takes the K steps
// [split * nk / splits, (split + 1) * nk / splits) and stores its scaled
// fp32 partial tile to partial[split][M][ldp]; splitk_reduce_kernel adds the
// splits in order and applies the epilogue.
// MX (MXFP8, OCP microscaling): instead of the per-row fp32 scales applied
// in the epilogue, each 32-code block of A and B rows carries an E8M0 scale
// that the scaled MFMA applies.  Each stage then also moves, by one 4-byte
// DMA instruction per wave, the stage's 32-bit scale word of every A row and
// every B row (blocks 4 kt .. 4 kt + 3 of the row), into MxWords after the
// tiles; lanes past the BM + BN rows repeat row 0 of A into the padding.
template <class C, bool MX>
__global__ __launch_bounds__(C::NT, C::MINB) void fp8_gemm_kernel(Fp8Gemm g, int tiles_m, int tiles_n, int group_m,
                                                                  int splits, float* partial, int ldp) {
    static_assert(C::DMA && C::CPR == 8, "fp8 tiles: LDS-DMA, 128-byte K step");
    constexpr int MX_WORDS = C::NW * 64;  // one 4-byte DMA lane per wave lane
    static_assert(!MX || MX_WORDS >= C::BM + C::BN, "a scale word for every A and B row");
    constexpr int EXTRA = MX ? MX_WORDS / 4 : 0;  // chunks of 16 B
    __shared__ u32x4_t ring[C::STAGES * (C::STAGE_CHUNKS + EXTRA)];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    const int ws_ = xcd_work_index(blockIdx.x, tiles_m * tiles_n * splits);
    if (ws_ < 0) return;
    const int split = ws_ % splits, w = ws_ / splits;
    const int nk = g.K / 128;
    const int kb = split * nk / splits, ke = (split + 1) * nk / splits;
    const int width = group_m * tiles_n;
    const int first_m = (w / width) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int m0 = (first_m + (w % width) % gsz) * C::BM;
    const int n0 = ((w % width) / gsz) * C::BN;

    using SA = Slots<C, C::BM>;
    using SB = Slots<C, C::BN>;
    const uint8_t* a_ptr[SA::N];
    const uint8_t* b_ptr[SB::N];
#pragma unroll
    for (int j = 0; j < SA::N; ++j)
        a_ptr[j] = g.A + (int64_t)min(m0 + SA::row(j, tid), g.M - 1) * g.lda + SA::lchunk(j, tid) * 16;
#pragma unroll
    for (int j = 0; j < SB::N; ++j)
        b_ptr[j] = g.B + (int64_t)min(n0 + SB::row(j, tid), g.N - 1) * g.ldb + SB::lchunk(j, tid) * 16;

    // MX: this lane's scale word source (row q of A, then of B, else A row 0)
    const uint8_t* mx_src = nullptr;
    if constexpr (MX) {
        const int q = wave * 64 + lane;
        const int64_t bpr = g.K / 32;  // scale bytes per row
        if (q < C::BM)
            mx_src = g.a_mx + (int64_t)min(m0 + q, g.M - 1) * bpr;
        else if (q < C::BM + C::BN)
            mx_src = g.b_mx + (int64_t)min(n0 + q - C::BM, g.N - 1) * bpr;
        else
            mx_src = g.a_mx + (int64_t)min(m0, g.M - 1) * bpr;
    }
    auto fill = [&](int kt, u32x4_t* As, u32x4_t* Bs) __attribute__((always_inline)) {
        const int kk = (kb + kt) * 128;
#pragma unroll
        for (int j = 0; j < SA::N; ++j)
            if (SA::active(j, tid)) dma16(a_ptr[j] + kk, SA::dst(As, wave, j));
#pragma unroll
        for (int j = 0; j < SB::N; ++j)
            if (SB::active(j, tid)) dma16<C::B_NT ? 2 : 0>(b_ptr[j] + kk, SB::dst(Bs, wave, j));
        if constexpr (MX) {  // the stage's scale words sit right after its B tile
            u32x4_t* words = As + C::STAGE_CHUNKS + wave * 16;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(mx_src + (kb + kt) * 4),
                                             (__attribute__((address_space(3))) void*)words, 4, 0, 0);
        }
    };
    auto land = [](u32x4_t*, u32x4_t*) {};

    f32x16_t acc[C::TM][C::TN];
    zero_acc<C>(acc);
    kloop<C, SA::N + SB::N + (MX ? 1 : 0), MX ? 2 : 1, EXTRA>(ke - kb, fill, land, ring, acc, wm, wn, lane);

    static_for<C::TM>([&](auto tmc) __attribute__((always_inline)) {
        constexpr int tm = decltype(tmc)::value;
        const int m = m0 + wm * C::WM + tm * 32 + (lane & 31);
        if (m < g.M) {
            const float sa = MX ? 1.0f : g.a_scale[m];
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
            static_for<C::TN * 4>([&](auto tqc) __attribute__((always_inline)) {
                constexpr int tn = decltype(tqc)::value / 4, q = decltype(tqc)::value % 4;
                const int n = n0 + wn * C::WN + tn * 32 + q * 8 + (lane >> 5) * 4;
                if (n < g.N) {  // N % 16 == 0: columns n..n+3 are all inside
                    const float4 sb = MX ? make_float4(1.f, 1.f, 1.f, 1.f)
                                         : *reinterpret_cast<const float4*>(g.b_scale + n);
                    float v[4] = {acc[tm][tn][q * 4 + 0] * sa * sb.x, acc[tm][tn][q * 4 + 1] * sa * sb.y,
                                  acc[tm][tn][q * 4 + 2] * sa * sb.z, acc[tm][tn][q * 4 + 3] * sa * sb.w};
                    if (partial) {  // ldp is a multiple of 4: one aligned float4
                        *reinterpret_cast<float4*>(partial + ((int64_t)split * g.M + m) * ldp + n) =
                            make_float4(v[0], v[1], v[2], v[3]);
                        return;
                    }
                    uint2* dst = reinterpret_cast<uint2*>(crow + n);
                    if (g.epi == EPI_ADD) {
                        const uint2 old = *dst;
                        v[0] += bf16_to_f32((uint16_t)(old.x & 0xFFFFu));
                        v[1] += bf16_to_f32((uint16_t)(old.x >> 16));
                        v[2] += bf16_to_f32((uint16_t)(old.y & 0xFFFFu));
                        v[3] += bf16_to_f32((uint16_t)(old.y >> 16));
                    } else if (g.epi == EPI_RELU2) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) v[i] = fmaxf(v[i], 0.f) * fmaxf(v[i], 0.f);
                    }
                    uint2 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    *dst = o;
                }
            });
        }
    });
}

// E4M3 codes of 8 consecutive values v[0..7] / scale (two packed words).
__device__ __forceinline__ uint2 fp8_codes8(const u32x4_t& v, float scale) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float a = bf16_to_f32((uint16_t)(v[2 * h] & 0xFFFFu)) / scale;
        const float b = bf16_to_f32((uint16_t)(v[2 * h] >> 16)) / scale;
        const float cc = bf16_to_f32((uint16_t)(v[2 * h + 1] & 0xFFFFu)) / scale;
        const float d = bf16_to_f32((uint16_t)(v[2 * h + 1] >> 16)) / scale;
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(cc, d, p, true);
        w[h] = (uint32_t)p;
    }
    return make_uint2(w[0], w[1]);
}

// One wave per row: the row's max |v| (a first pass), then the codes (a
// second pass over the same 16-byte chunks, mostly cache hits).
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                                int cols, int64_t ld, uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // whole wave
    const uint16_t* row = src + r * ld;
    float amax = 0.f;
    for (int c = lane * 8; c < cols; c += 512) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[i] & 0xFFFFu))));
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[i] >> 16))));
        }
    }
    amax = wave_max(amax);
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* out = codes + r * (int64_t)cols;
    for (int c = lane * 8; c < cols; c += 512)
        *reinterpret_cast<uint2*>(out + c) = fp8_codes8(*reinterpret_cast<const u32x4_t*>(row + c), scale);
    if (lane == 0) scales[r] = scale;
}

// Few rows (decode-sized calls): one 256-thread block per row, so a row's
// loads are spread over four waves instead of queued on one.  The same
// scale and codes as quantize_rows_fp8_kernel.
__global__ __launch_bounds__(256) void quantize_row_fp8_block_kernel(const uint16_t* __restrict__ src, int cols,
                                                                     int64_t ld, uint8_t* __restrict__ codes,
                                                                     float* __restrict__ scales) {
    __shared__ float part[4];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* row = src + r * ld;
    float amax = 0.f;
#pragma unroll 4
    for (int c = tid * 8; c < cols; c += 2048) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[i] & 0xFFFFu))));
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[i] >> 16))));
        }
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) part[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* out = codes + r * (int64_t)cols;
#pragma unroll 4
    for (int c = tid * 8; c < cols; c += 2048)
        *reinterpret_cast<uint2*>(out + c) = fp8_codes8(*reinterpret_cast<const u32x4_t*>(row + c), scale);
    if (tid == 0) scales[r] = scale;
}

hipError_t launch_quantize_rows_fp8(const uint16_t* src, int64_t rows, int cols, int64_t ld, uint8_t* codes,
                                    float* scales, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (rows <= 1024) {
        LMOE_LAUNCH("quantize_fp8", s,
                    quantize_row_fp8_block_kernel<<<(unsigned)rows, 256, 0, s>>>(src, cols, ld, codes, scales));
        return hipGetLastError();
    }
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    LMOE_LAUNCH("quantize_fp8", s,
                quantize_rows_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, ld, codes, scales));
    return hipGetLastError();
}

// MXFP8 quantisation (OCP microscaling) of a bf16 matrix [rows][cols]
// (cols a multiple of 32, row stride ld), one thread per block of 32
// consecutive elements: e = floor(log2 max|v|) - 8 (8: the largest E4M3
// exponent), clamped to [-127, 127] (0 for an all-zero block); the scale is
// the E8M0 byte e + 127 and each code is E4M3 (nearest, ties to even) of
// v * 2^-e saturated to +-448.  Scaling by a power of two is exact.
__global__ __launch_bounds__(256) void quantize_blocks_mxfp8_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                                    int cols, int64_t ld,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int bpr = cols / 32;
    if (i >= rows * bpr) return;
    const int64_t r = i / bpr;
    const int b = (int)(i % bpr);
    const uint16_t* p = src + r * ld + b * 32;
    u32x4_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const u32x4_t*>(p + 8 * j);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[j][h] & 0xFFFFu))));
            amax = fmaxf(amax, fabsf(bf16_to_f32((uint16_t)(v[j][h] >> 16))));
        }
    // floor(log2 amax) from the exponent field (a subnormal amax reads -127
    // and is clamped like every block below 2^-119)
    int e = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 8 : 0;
    e = min(max(e, -127), 127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e: e <= 119 for finite bf16
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            auto q = [&](uint32_t bits) { return fminf(fmaxf(bf16_to_f32((uint16_t)bits) * inv, -448.f), 448.f); };
            const uint32_t lo = v[j][2 * h], hi = v[j][2 * h + 1];
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q(lo & 0xFFFFu), q(lo >> 16), 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(q(hi & 0xFFFFu), q(hi >> 16), pk, true);
            w[2 * j + h] = (uint32_t)pk;
        }
    uint8_t* out = codes + r * (int64_t)cols + b * 32;
    *reinterpret_cast<u32x4_t*>(out) = u32x4_t{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4_t*>(out + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
    scales[r * bpr + b] = (uint8_t)(e + 127);
}

hipError_t launch_quantize_blocks_mxfp8(const uint16_t* src, int64_t rows, int cols, int64_t ld, uint8_t* codes,
                                        uint8_t* scales, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (cols % 32 != 0) return hipErrorInvalidValue;
    const int64_t blocks = (rows * (cols / 32) + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    LMOE_LAUNCH("quantize_mxfp8", s,
                quantize_blocks_mxfp8_kernel<<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, ld, codes, scales));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Repacking of bf16 expert weights into the tiled layout
// ---------------------------------------------------------------------------
//
// W [E][rows][cols] row-major -> MFMA-fragment order (16-byte chunks):
// P[e][rb][kt][ks][l] = W[e][32 rb + l % 32][64 kt + 16 ks + 8 (l / 32) ..+8]
// for 32-row blocks rb, 64-wide K steps kt, 16-wide sub-steps ks and lanes
// l < 64: exactly the 8 values lane l of a 32x32x16 MFMA takes for weight
// row l % 32, so each sub-step of a block is 1 KB of contiguous weights,
// one wave-wide 16-byte load (into registers, or by LDS-DMA into a tile
// that keeps the same order), and a block's K steps follow each other.
__global__ __launch_bounds__(256) void pack_experts_kernel(const u32x4_t* __restrict__ W, u32x4_t* __restrict__ P,
                                                           int64_t n_chunks, int rows, int cols) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= n_chunks) return;
    const int kts = cols / 64, rbs = rows / 32;
    const int l = (int)(o % 64), ks = (int)((o / 64) % 4);
    const int64_t step = o / 256;  // (e, rb, kt)
    const int kt = (int)(step % kts);
    const int64_t erb = step / kts;  // e * rbs + rb
    const int64_t row = (erb / rbs) * rows + (erb % rbs) * 32 + l % 32;
    P[o] = W[row * (cols / 8) + kt * 8 + 2 * ks + l / 32];
}

hipError_t launch_pack_experts(const void* W, void* P, int64_t E, int rows, int cols, hipStream_t s) {
    const int64_t n_chunks = E * rows * (int64_t)cols / 8;
    const int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    LMOE_LAUNCH("pack_experts", s,
                pack_experts_kernel<<<(unsigned)blocks, 256, 0, s>>>((const u32x4_t*)W, (u32x4_t*)P, n_chunks,
                                                                      rows, cols));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static int persistent_grid();

// Split-K factor for a dense GEMM whose tiles alone cannot fill the GPU:
// aim for as many tile-splits as blocks fit on the GPU at once (more splits
// only add fp32 partial traffic), keep >= 4 K steps per split, and fit the
// partials in the given workspace.
static int splitk_factor(int tiles, int nk, int M, int ldp, size_t ws_bytes, int blocks_per_cu) {
    const int cus = persistent_grid();
    if (ws_bytes == 0 || tiles >= 2 * cus) return 1;
    int splits = blocks_per_cu * cus / tiles;  // one round of blocks
    const int by_k = nk / 4 > 1 ? nk / 4 : 1;
    if (splits > by_k) splits = by_k;
    const size_t per = (size_t)M * ldp * sizeof(float);
    const size_t by_ws = ws_bytes / per < 64 ? ws_bytes / per : 64;
    if ((size_t)splits > by_ws) splits = (int)by_ws;
    return splits > 1 ? splits : 1;
}

template <class C>
static hipError_t run_dense(const DenseGemm& g, void* ws, size_t ws_bytes, hipStream_t s) {
    const int tiles_m = (g.M + C::BM - 1) / C::BM, tiles_n = (g.N + C::BN - 1) / C::BN;
    const int nk = g.K[0] / C::BK + (g.nseg > 1 ? g.K[1] / C::BK : 0);
    const int ldp = (g.N + 3) / 4 * 4;
    const int splits = splitk_factor(tiles_m * tiles_n, nk, g.M, ldp, ws_bytes, C::MINB);
    float* partial = splits > 1 ? (float*)ws : nullptr;
    LMOE_LAUNCH("dense_gemm", s,
                dense_gemm_kernel<C><<<tiles_m * tiles_n * splits, C::NT, 0, s>>>(g, tiles_m, tiles_n, 8, splits,
                                                                                  partial, ldp, nullptr));
    if (splits > 1) {
        const int64_t threads = (int64_t)g.M * (ldp / 4);
        LMOE_LAUNCH("splitk_reduce", s,
                    splitk_reduce_kernel<<<(int)((threads + 255) / 256), 256, 0, s>>>(g, splits, partial, ldp));
    }
    return hipGetLastError();
}

// Persistent grid: one block per CU (a multiple of 8, one slot per XCD),
// times the blocks per CU the tile configuration is sized for.
static int persistent_grid() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return (cus + 7) / 8 * 8;
}

template <class C, int BFMT, bool SK>
static void launch_grouped_fmt(const GroupedGemm& g, int grid, int nN, hipStream_t s) {
    constexpr int RPI = Slots<C, C::BM>::RPI;
    constexpr bool can_scalar = C::DMA && (RPI == 8 || RPI == 16);
    const char* name = (BFMT == LMOE_NVFP4 || BFMT == LMOE_NVFP4_2D) ? "grouped_gemm_nvfp4" : "grouped_gemm";
    if (!g.a_row_map)
        LMOE_LAUNCH(name, s, grouped_gemm_kernel<C, BFMT, GATHER_NONE, SK><<<grid, C::NT, 0, s>>>(g, nN));
    else if (can_scalar && g.n_rows >= RPI)
        LMOE_LAUNCH(name, s,
                    grouped_gemm_kernel<C, BFMT, can_scalar ? GATHER_SCALAR : GATHER_LANE, SK>
                    <<<grid, C::NT, 0, s>>>(g, nN));
    else
        LMOE_LAUNCH(name, s, grouped_gemm_kernel<C, BFMT, GATHER_LANE, SK><<<grid, C::NT, 0, s>>>(g, nN));
}

template <class C, bool SK>
static void launch_grouped_any(const GroupedGemm& g, int grid, int nN, hipStream_t s) {
    if (g.b_fmt == LMOE_NVFP4)
        launch_grouped_fmt<C, LMOE_NVFP4, SK>(g, grid, nN, s);
    else if (g.b_fmt == LMOE_NVFP4_2D)
        launch_grouped_fmt<C, LMOE_NVFP4_2D, SK>(g, grid, nN, s);
    else if (g.b_fmt == LMOE_BF16_TILED)
        launch_grouped_fmt<C, LMOE_BF16_TILED, SK>(g, grid, nN, s);
    else
        launch_grouped_fmt<C, LMOE_BF16, SK>(g, grid, nN, s);
}

// Steps in flight of the register-decode NVFP4 expert GEMM and of the
// register-weight bf16 one.
constexpr int kFp4RegD = 3;
constexpr int kBregD = 3;

template <int BFMT>
static void launch_grouped_fp4reg(const GroupedGemm& g, int grid, int nN, hipStream_t s) {
    if (!g.a_row_map)
        LMOE_LAUNCH("grouped_gemm_nvfp4", s,
                    grouped_gemm_nvfp4_reg_kernel<BFMT, GATHER_NONE, kFp4RegD><<<grid, 512, 0, s>>>(g, nN));
    else if (g.n_rows >= 8)
        LMOE_LAUNCH("grouped_gemm_nvfp4", s,
                    grouped_gemm_nvfp4_reg_kernel<BFMT, GATHER_SCALAR, kFp4RegD><<<grid, 512, 0, s>>>(g, nN));
    else
        LMOE_LAUNCH("grouped_gemm_nvfp4", s,
                    grouped_gemm_nvfp4_reg_kernel<BFMT, GATHER_LANE, kFp4RegD><<<grid, 512, 0, s>>>(g, nN));
}

// Split-K scheduling for the 64 x 128 few-rows tiles when the caller gave
// the partial-sum buffer and enough counters; whole items otherwise.
template <class C>
static hipError_t run_grouped(const GroupedGemm& g, hipStream_t s) {
    const int nN = (g.N + C::BN - 1) / C::BN;
    const int grid = persistent_grid() * C::MINB;
    if constexpr (C::BM == kSkBM && C::BN == kSkBN) {
        if (g.sk_part && g.tt.sk_count && grid <= kSkMaxBlocks &&
            (int64_t)g.tt.max_tiles * nN <= (int64_t)g.tt.sk_count_len) {
            launch_grouped_any<C, true>(g, grid, nN, s);
            return hipGetLastError();
        }
    }
    launch_grouped_any<C, false>(g, grid, nN, s);
    return hipGetLastError();
}

// Columns [n0, n1) of a dense GEMM as a GEMM of their own: groups clipped
// to the range, their weight rows, outputs and biases offset to match.
static DenseGemm sub_columns(const DenseGemm& g, int n0, int n1) {
    DenseGemm h = g;
    h.N = n1 - n0;
    h.ngroups = 0;
    for (int i = 0; i < g.ngroups; ++i) {
        const NGroup& G = g.g[i];
        const int b = G.n_begin > n0 ? G.n_begin : n0, e = G.n_end < n1 ? G.n_end : n1;
        if (b >= e) continue;
        const int skip = b - G.n_begin;  // columns of G before the range
        NGroup H = G;
        H.n_begin = b - n0;
        H.n_end = e - n0;
        for (int sg = 0; sg < g.nseg; ++sg)
            if (G.B[sg]) H.B[sg] = (const uint16_t*)G.B[sg] + (int64_t)skip * g.K[sg];
        H.C = G.epi == EPI_F32_BIAS ? (void*)((float*)G.C + skip) : (void*)((uint16_t*)G.C + skip);
        if (G.bias) H.bias = G.bias + skip;
        h.g[h.ngroups++] = H;
    }
    return h;
}

// Tail split of a many-row dense GEMM: when the last round of 256 x 256
// tiles over the CUs is at most half full and made of whole N-tile columns,
// those columns run as a split-K GEMM of their own (one round of blocks, the
// partials summed in split order), so the last round costs a fraction of a
// tile instead of a whole one.  A GEMM with at most half a round of tiles is
// split whole.  Returns the first tail column (N: no split) and the
// partial-sum bytes the tail needs.
static int dense_tail_split(const DenseGemm& g, int cus, size_t* bytes) {
    constexpr int T = 256;
    const int tiles_m = (g.M + T - 1) / T, tiles_n = (g.N + T - 1) / T;
    const int tiles = tiles_m * tiles_n, rounds = tiles / cus, tail = tiles - rounds * cus;
    *bytes = 0;
    if (tail == 0 || tail > cus / 2 || tail % tiles_m != 0) return g.N;
    const int n0 = (tiles_n - tail / tiles_m) * T;
    for (int i = 0; i < g.ngroups; ++i) {  // the split must keep 8-column alignment of outputs
        const NGroup& G = g.g[i];
        if (n0 > G.n_begin && n0 < G.n_end && (n0 - G.n_begin) % 8 != 0) return g.N;
    }
    const int nk = g.K[0] / 64 + (g.nseg > 1 ? g.K[1] / 64 : 0);
    const int splits = std::min(std::min(cus / tail, 4), std::max(1, nk / 4));
    if (splits < 2) return g.N;
    const size_t ldp = (size_t)((g.N - n0 + 3) / 4 * 4);
    *bytes = (size_t)splits * g.M * ldp * sizeof(float);
    return n0;
}

size_t dense_tail_split_bytes(const DenseGemm& g) {
    size_t bytes = 0;
    dense_tail_split(g, persistent_grid(), &bytes);
    return bytes;
}

// Dense: 256x256 tiles over 8 waves (2 per SIMD), each wave 64 x 128, the
// fastest shape measured for the 8192-wide projections; 256x192 where that
// fills the GPU better (narrow N, few M tiles).  Decode-sized M uses 64x64
// tiles with split-K.
// Few rows (decode): weight streaming with 64x64 tiles, 4 stages, 2 blocks
// per CU, split-K.
using DecodeDenseCfg = MfmaCfg<64, 64, 2, 2, true, 64, 4, 2, true>;

static int decode_dense_splits(const DenseGemm& g, size_t ws_bytes) {
    using C = DecodeDenseCfg;
    const int tiles = (g.M + C::BM - 1) / C::BM * ((g.N + C::BN - 1) / C::BN);
    const int nk = g.K[0] / C::BK + (g.nseg > 1 ? g.K[1] / C::BK : 0);
    return splitk_factor(tiles, nk, g.M, (g.N + 3) / 4 * 4, ws_bytes, C::MINB);
}

bool dense_topk_fusable(const DenseGemm& g, size_t splitk_bytes, int E, int k) {
    return g.M <= 64 && k <= kWave && E <= 1024 && decode_dense_splits(g, splitk_bytes) > 1;
}

hipError_t launch_dense_gemm_topk_bf16(const DenseGemm& g, void* splitk_ws, size_t splitk_bytes, int lc0, int E,
                                       const float* bias, int k, int32_t* idx, float* gate, const PermFused* pf,
                                       hipStream_t s) {
    using C = DecodeDenseCfg;
    if (!dense_topk_fusable(g, splitk_bytes, E, k) || lc0 < 0 || lc0 + E > g.N) return hipErrorInvalidValue;
    if (pf && (!pf->arrive || g.M * k > kMaxFusedPairs || E > kMaxExperts)) return hipErrorInvalidValue;
    const int tiles_m = (g.M + C::BM - 1) / C::BM, tiles_n = (g.N + C::BN - 1) / C::BN;
    const int ldp = (g.N + 3) / 4 * 4;
    const int splits = decode_dense_splits(g, splitk_bytes);
    float* partial = (float*)splitk_ws;
    const PermFused none{};
    LMOE_LAUNCH("dense_gemm", s,
                dense_gemm_kernel<C><<<tiles_m * tiles_n * splits, C::NT, 0, s>>>(g, tiles_m, tiles_n, 8, splits,
                                                                                  partial, ldp,
                                                                                  pf ? pf->arrive : nullptr));
#define LMOE_REDUCE_TOPK(S_)                                                                                   \
    do {                                                                                                       \
        if (pf)                                                                                                \
            LMOE_LAUNCH("splitk_reduce_topk_perm", s,                                                          \
                        splitk_reduce_topk_kernel<S_, true><<<2 * g.M, 1024, 0, s>>>(g, splits, partial, ldp, lc0, \
                                                                                   E, bias, k, idx, gate, *pf)); \
        else                                                                                                   \
            LMOE_LAUNCH("splitk_reduce_topk", s,                                                               \
                        splitk_reduce_topk_kernel<S_, false><<<2 * g.M, 1024, 0, s>>>(g, splits, partial, ldp,   \
                                                                                    lc0, E, bias, k, idx, gate, \
                                                                                    none));                    \
    } while (0)
    if (E <= 64)
        LMOE_REDUCE_TOPK(1);
    else if (E <= 128)
        LMOE_REDUCE_TOPK(2);
    else if (E <= 256)
        LMOE_REDUCE_TOPK(4);
    else if (E <= 512)
        LMOE_REDUCE_TOPK(8);
    else
        LMOE_REDUCE_TOPK(16);
#undef LMOE_REDUCE_TOPK
    return hipGetLastError();
}

hipError_t launch_dense_gemm_bf16(const DenseGemm& g, void* splitk_ws, size_t splitk_bytes, hipStream_t s) {
    if (g.M <= 64) return run_dense<DecodeDenseCfg>(g, splitk_ws, splitk_bytes, s);
    using C256 = MfmaCfg<256, 256, 4, 2, true, 64, 2>;
    // The cost of a shape is its rounds of tiles over the CUs times the tile
    // width (a split tail round costs about a quarter); 256-wide tiles
    // unless 192-wide ones are clearly cheaper.
    const int cus = persistent_grid(), tiles_m = (g.M + 255) / 256;
    size_t tail_bytes = 0;
    const int n_tail = dense_tail_split(g, cus, &tail_bytes);
    const bool split_tail = n_tail < g.N && tail_bytes <= splitk_bytes;
    const int full_rounds = tiles_m * ((g.N + 255) / 256) / cus;
    const double r256 = split_tail ? full_rounds + 0.25
                                   : (double)((tiles_m * ((g.N + 255) / 256) + cus - 1) / cus);
    const double r192 = (double)((tiles_m * ((g.N + 191) / 192) + cus - 1) / cus) * 0.75;
    if (r192 < 0.85 * r256) return run_dense<MfmaCfg<256, 192, 4, 2, true, 64, 2>>(g, nullptr, 0, s);
    if (!split_tail) return run_dense<C256>(g, nullptr, 0, s);
    if (n_tail > 0) {
        const hipError_t e = run_dense<C256>(sub_columns(g, 0, n_tail), nullptr, 0, s);
        if (e != hipSuccess) return e;
    }
    return run_dense<C256>(sub_columns(g, n_tail, g.N), splitk_ws, splitk_bytes, s);
}
// FP8 shared expert: 256x256 tiles (64x64 for decode-sized M), one tile per
// block; N and K are the shared expert's (multiples of 64 and 128).
template <class C, bool MX>
static hipError_t run_fp8(const Fp8Gemm& g, void* ws, size_t ws_bytes, hipStream_t s) {
    const int tiles_m = (g.M + C::BM - 1) / C::BM, tiles_n = (g.N + C::BN - 1) / C::BN;
    const int ldp = (g.N + 3) / 4 * 4;
    const int splits = splitk_factor(tiles_m * tiles_n, g.K / 128, g.M, ldp, ws_bytes, C::MINB);
    float* partial = splits > 1 ? (float*)ws : nullptr;
    LMOE_LAUNCH("fp8_gemm", s,
                fp8_gemm_kernel<C, MX><<<tiles_m * tiles_n * splits, C::NT, 0, s>>>(g, tiles_m, tiles_n, 8, splits,
                                                                                   partial, ldp));
    if (splits > 1) {  // the reduction's epilogue: one column group writing g.C
        DenseGemm r{};
        r.M = g.M;
        r.N = g.N;
        r.ngroups = 1;
        r.g[0] = NGroup{0, g.N, {nullptr, nullptr}, g.epi, g.C, g.ldc, nullptr};
        const int64_t threads = (int64_t)g.M * (ldp / 4);
        LMOE_LAUNCH("splitk_reduce", s,
                    splitk_reduce_kernel<<<(int)((threads + 255) / 256), 256, 0, s>>>(r, splits, partial, ldp));
    }
    return hipGetLastError();
}

hipError_t launch_fp8_gemm(const Fp8Gemm& g, void* splitk_ws, size_t splitk_bytes, hipStream_t s) {
    if (g.K % 128 != 0 || g.N % 16 != 0) return hipErrorInvalidValue;
    if (g.epi != EPI_STORE && g.epi != EPI_RELU2 && g.epi != EPI_ADD) return hipErrorInvalidValue;
    const bool mx = g.a_mx != nullptr;
    if (mx != (g.b_mx != nullptr)) return hipErrorInvalidValue;
    using Few = MfmaCfg<64, 64, 2, 2, true, 64, 4, 2, true>;
    using Many = MfmaCfg<256, 256, 4, 2, true, 64, 2>;
    if (g.M <= 64)  // weight streaming: split-K over the partial-sum workspace
        return mx ? run_fp8<Few, true>(g, splitk_ws, splitk_bytes, s) : run_fp8<Few, false>(g, splitk_ws, splitk_bytes, s);
    return mx ? run_fp8<Many, true>(g, nullptr, 0, s) : run_fp8<Many, false>(g, nullptr, 0, s);
}

// Grouped: 192-row expert tiles (about 352 rows per expert at prefill pad to
// 384) by 256 columns over 8 waves, each wave 96 x 64.  Few-row experts
// (decode) stream their weights with the non-temporal hint (each call reads
// them once), two blocks per CU: 64x128 tiles, 3 LDS stages, for wide
// outputs (each activation row fetched per K step then feeds 128 weight rows,
// not 64), else 64x64 tiles, 4 stages.  A plain weight stream through LDS-DMA
// with two 4-wave blocks per CU reached 6.8 TB/s; one 8-wave block per CU with
// the same bytes in flight, 5.6.
hipError_t launch_grouped_gemm_bf16(const GroupedGemm& g, hipStream_t s) {
    if (g.tt.bm == 192 && (g.b_fmt == LMOE_NVFP4 || g.b_fmt == LMOE_NVFP4_2D) && g.N % 256 == 0 &&
        (g.K / 64) % (kFp4RegD + 1) == 0 && g.K / 64 > kFp4RegD) {
        // NVFP4 decoded in registers
        const int grid = persistent_grid(), nN = g.N / 256;
        if (g.b_fmt == LMOE_NVFP4)
            launch_grouped_fp4reg<LMOE_NVFP4>(g, grid, nN, s);
        else
            launch_grouped_fp4reg<LMOE_NVFP4_2D>(g, grid, nN, s);
        return hipGetLastError();
    }
    if (g.tt.bm == 192 && (g.b_fmt == LMOE_NVFP4 || g.b_fmt == LMOE_NVFP4_2D)) {
        // NVFP4: three A stages and the decoded weights in a ring of their own
        using C = MfmaCfg<192, 256, 2, 4, true, 64, 3>;
        const int grid = persistent_grid() * C::MINB, nN = (g.N + C::BN - 1) / C::BN;
        if (g.b_fmt == LMOE_NVFP4)
            launch_grouped_fmt<C, LMOE_NVFP4, false>(g, grid, nN, s);
        else
            launch_grouped_fmt<C, LMOE_NVFP4_2D, false>(g, grid, nN, s);
        return hipGetLastError();
    }
    if (g.tt.bm == 192 && g.b_fmt == LMOE_BF16_TILED && g.N % 256 == 0 && (g.K / 64) % (kBregD + 1) == 0 &&
        g.K / 64 > kBregD) {
        // packed weights streamed into registers
        const int grid = persistent_grid(), nN = g.N / 256;
        if (!g.a_row_map)
            LMOE_LAUNCH("grouped_gemm", s,
                        grouped_gemm_breg_kernel<LMOE_BF16_TILED, GATHER_NONE, kBregD><<<grid, 512, 0, s>>>(g, nN));
        else if (g.n_rows >= 8)
            LMOE_LAUNCH("grouped_gemm", s,
                        grouped_gemm_breg_kernel<LMOE_BF16_TILED, GATHER_SCALAR, kBregD><<<grid, 512, 0, s>>>(g, nN));
        else
            LMOE_LAUNCH("grouped_gemm", s,
                        grouped_gemm_breg_kernel<LMOE_BF16_TILED, GATHER_LANE, kBregD><<<grid, 512, 0, s>>>(g, nN));
        return hipGetLastError();
    }
    if (g.tt.bm == 192) return run_grouped<MfmaCfg<192, 256, 2, 4, true, 64, 2>>(g, s);
    if (g.tt.bm == 64 && g.N >= 1024) return run_grouped<MfmaCfg<64, 128, 2, 2, true, 64, 3, 2, true>>(g, s);
    if (g.tt.bm == 64) return run_grouped<MfmaCfg<64, 64, 2, 2, true, 64, 4, 2, true>>(g, s);
    return hipErrorInvalidValue;
}

}  // namespace lmoe
