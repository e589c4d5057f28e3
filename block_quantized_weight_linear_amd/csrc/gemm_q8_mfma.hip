// Prefill (M >= 256 activation rows): Q8_0 weights x float32 activations on the bf16
// matrix cores of gfx950 (v_mfma_f32_32x32x16_bf16), float32 accumulation and output.
//
// With hundreds of rows the linear is a dense contraction (the tensor-core vs GEMV
// kernel-class boundary of the fucina DGX Spark README, Performance): each weight is
// used M times, so the matrix cores, not memory, bound it.  The weights stay Q8_0 in
// HBM ("14. Model families and example applications", section 14.1: no global
// dequantization); each tile dequantizes the blocks it needs.
//
// Tile: 128 activation rows x BN = 4*WN weight rows, four waves, one block per CU.  Each
// wave owns WN weight rows (fused gate_up: WN/2 outputs; in each 32-row fragment rows 0..15
// are gate rows and rows 16..31 the up rows of the same 16 outputs) for all 128 activation
// rows, so a weight is dequantized by exactly one wave: its Q8_0 bytes reach the wave's
// own LDS ring by direct-to-LDS 16-byte copies (a lane's 32-bit offset into the matrix is
// fixed for the whole K loop, the step is a scalar base), and the wave turns them into
// MFMA B operands in registers (bf16(fp32(d) * q), one rounding; d*q needs at most 19
// significant bits).  The activations of a K step (128 x 64 float32) come into registers
// one step ahead and are rounded to bf16 (nearest even) once per block into one of two
// tiles the four waves share (steps alternate), so a step needs one barrier.  Per wave a K
// step is 4 x 4 x WN/32 v_mfma_f32_32x32x16_bf16 on a 128 x WN accumulator tile (on gfx950
// this shape keeps the matrix cores busy from one wave per SIMD; 16x16x32 with as many
// accumulators does not).
//
// Inputs of a Q8_0 block are multiplied in a permuted order: the four groups of 8 inputs
// run as groups 0, 2, 1, 3 (both operands alike, so the products and sums are those of
// the block): then the 16 quants a lane needs are contiguous in the block, and the lane
// reads them as whole 16-byte LDS chunks (conflict-free across the 32 rows of a fragment).
//
// Pipeline: weight bytes go to a ring of three stages per wave, activations to two
// register sets.  A K step is two runs of MFMAs, one per block of the pair; after every
// MFMA of a run come two weights of the other block's dequantization (block 1 of this
// step in the first run, block 0 of the next step in the second), in fixed program order,
// and the loads for two steps ahead go out one at a time between the MFMAs (activations in
// the first run, weight copies in the second) so the vector-memory queue drains while the
// matrix cores work.  The step loop is unrolled by four, the period of a pair's position
// inside its 16-byte chunks.
//
// Dense grids map tiles to blocks so that the 128-row tiles sharing a weight tile land
// on the same XCD (blocks are handed to the 8 XCDs in turn), where they share its L2.
//
// MFMA lane layout (checked on the device): lane l supplies A[l%32][8*(l/32) + i] and
// B[8*(l/32) + i][l%32], i = 0..7, and register j of D holds D[8*(j/4) + 4*(l/32) + j%4][l%32].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "q8_internal.h"

namespace q8k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // activation rows per tile
constexpr int kBK = 64;           // inputs per K step (one Q8_0 block pair per weight row)
constexpr int kXStride = 72;      // bf16 per LDS row of the activation tile (144 bytes)
constexpr int kMfWaves = 4;
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kWRing = 3;         // weight stages per wave
constexpr int kXcds = 8;          // dense grids: tiles sharing weights go to one XCD

// Per-wave weight stage for WN weight rows.  A row's pair for K step s is bytes 68s ..
// 68s+67 of the row; the stage holds the five aligned 16-byte chunks that contain it (80
// bytes from 68s - 4*(s%4): rows are 16-byte aligned and hold a multiple of four pairs, so
// the chunks never pass the row's end), copied as 64 chunks per instruction, padded to
// whole copies.  The pair starts at dword s%4 of its 20-dword stage row.
template <int WN>
struct WStage {
    static constexpr int kChunks = 5;
    static constexpr int kRowDwords = 4 * kChunks;
    static constexpr int kCopies = (WN * kChunks + 63) / 64;
    static constexpr int kDwords = kCopies * 256;
};

constexpr int kXbfElems = kBM * kXStride;                  // one bf16 activation tile
constexpr size_t kXbfBytes = (size_t)kXbfElems * 2;
template <int WN>
constexpr size_t mfma_lds_bytes() {
    return 2 * kXbfBytes + (size_t)kMfWaves * kWRing * WStage<WN>::kDwords * 4;
}

__device__ __forceinline__ float mf_half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float mf_half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ float mf_sbyte(uint32_t v, int b) { return (float)(int)(int8_t)(v >> (8 * b)); }

// One wave-wide direct-to-LDS 16-byte copy with a scalar base: lane l copies the 16 bytes
// at base + off to lds + 16*l.  base and lds are wave-uniform (an SGPR pair and M0); M0 is
// saved and restored, and a write of M0 needs one wait state before the copy reads it.
__device__ __forceinline__ void lds_copy16_sbase(const uint8_t* base, uint32_t off, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds)
        : "memory");
}

template <int N>
__device__ __forceinline__ void mf_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Expert-grouped tiles (the MoE prefill form): tile t of the grid's tile list belongs to
// the expert e with tile_start[e] <= t < tile_start[e + 1]; its activation rows are the
// positions offsets[e] + 128 * (t - tile_start[e]) + r of the expert-sorted pair list.
// gather: row of position pos is x[sorted[pos] / k] (the token's input); else x[pos].
// The output row of position pos is y[pos].
struct GroupArgs {
    const int32_t* offsets;     // [n_exp + 1] pair positions per expert
    const int32_t* tile_start;  // [n_exp + 1] first 128-row tile of each expert
    const int32_t* sorted;      // [pairs] pair index (token * k + slot) at each position
    int n_exp, k;
    size_t expert_bytes;        // bytes of one expert's Q8_0 matrix
    bool gather;
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Four bf16 weights d*q from the quant bytes of dword v (byte b: weight b), each rounded
// to nearest even once; converted as one vector so the pairs pack directly.
__device__ __forceinline__ bf16x4 dq4(uint32_t v, float d) {
    const f32x4v f = {mf_sbyte(v, 0) * d, mf_sbyte(v, 1) * d, mf_sbyte(v, 2) * d, mf_sbyte(v, 3) * d};
    return __builtin_convertvector(f, bf16x4);
}
__device__ __forceinline__ bf16x8 join4(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int WN, bool SILU, bool GROUPED>
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_q8_mfma_kernel(
    const uint8_t* __restrict__ w, int n_out, int P, const float* __restrict__ x, int M, int ldx,
    float* __restrict__ y, int ldy, int m_tiles, int n_tiles, int tiles, GroupArgs g) {
    constexpr int BN = kMfWaves * WN;
    constexpr int NF = WN / 32;  // 32-column fragments per wave
    constexpr int L = WStage<WN>::kCopies;
    static_assert(WN % 32 == 0, "whole 32-column fragments per wave");
    static_assert(L < 64, "copies of a stage must fit the vmcnt counter");
    extern __shared__ __attribute__((aligned(16))) uint8_t mf_smem[];
    __bf16* xs = reinterpret_cast<__bf16*>(mf_smem);                          // [2][kBM][kXStride] bf16
    uint32_t* wr = reinterpret_cast<uint32_t*>(mf_smem + 2 * kXbfBytes);     // [waves][ring][stage]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int mt, nt, mbase = 0;
    if constexpr (GROUPED) {
        const int t = blockIdx.x / n_tiles;
        nt = blockIdx.x - t * n_tiles;
        if (t >= g.tile_start[g.n_exp]) return;  // past the tile list (block-uniform, before any barrier)
        int lo = 0, hi = g.n_exp;                 // largest lo with tile_start[lo] <= t
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.tile_start[mid] <= t) lo = mid;
            else hi = mid;
        }
        mbase = g.offsets[lo] + kBM * (t - g.tile_start[lo]);
        const int rows = g.offsets[lo + 1] - mbase;
        M = rows < kBM ? rows : kBM;
        mt = 0;
        w += (size_t)__builtin_amdgcn_readfirstlane(lo) * g.expert_bytes;
    } else {
        const int per_xcd = (tiles + kXcds - 1) / kXcds;
        const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
        if (t >= tiles) return;  // block-uniform, before any barrier
        mt = t % m_tiles;
        nt = t / m_tiles;
    }
    const uint32_t row_bytes = (uint32_t)P * 68u;

    // Weight row of the wave's column c (0 <= c < WN); past the matrix: the last row.
    auto w_row = [&](int c) __attribute__((always_inline)) {
        if constexpr (SILU) {
            const int f = c >> 5, w32 = c & 31;
            int o = nt * (BN / 2) + wave * (WN / 2) + 16 * f + (w32 & 15);
            o = o < n_out ? o : n_out - 1;
            return (w32 >= 16) ? o + n_out : o;
        } else {
            const int n = nt * BN + wave * WN + c;
            return n < n_out ? n : n_out - 1;
        }
    };
    // Copy j of a stage moves stage chunks 64j .. 64j+63: chunk i is chunk i % 5 of column
    // i / 5 (the padding past WN*5 re-reads the last column's chunks).
    uint32_t woff[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int i = 64 * j + lane;
        int r = i / WStage<WN>::kChunks;
        const int c = i - WStage<WN>::kChunks * r;
        r = r < WN ? r : WN - 1;
        woff[j] = (uint32_t)w_row(r) * row_bytes + 16u * (uint32_t)c;
    }
    const uint32_t wr_lds = (uint32_t)(uintptr_t)wr + (uint32_t)(wave * kWRing * WStage<WN>::kDwords * 4);
    auto copy_w = [&](int s, int slot, int j) __attribute__((always_inline)) {
        const uint8_t* base = w + (size_t)s * 68 - 4 * (s & 3);  // 16-byte aligned within the row
        const uint32_t lds = __builtin_amdgcn_readfirstlane(wr_lds + (uint32_t)(slot * WStage<WN>::kDwords * 4));
        lds_copy16_sbase(base, woff[j], lds + 1024u * j);
    };
    auto issue_w = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < L; ++j) copy_w(s, slot, j);
    };

    // Activations: thread t loads inputs 4xc .. 4xc + 3 of a step (xc = t % 16) of the tile
    // rows t/16 + 16q (q = 0..7) into registers two steps ahead (two register sets); past
    // the call's rows a thread re-reads the last row.  They are rounded to bf16 into the tile buffer of their
    // step (two buffers, steps alternate), where within each 32-input block the groups of
    // 8 inputs are stored in the order 0, 2, 1, 3.
    const int xc = tid & 15;
    const float* xrow[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        int r = mt * kBM + (tid >> 4) + 16 * q;
        r = r < M ? r : M - 1;
        size_t ri = (size_t)r;
        if constexpr (GROUPED) ri = g.gather ? (size_t)(g.sorted[mbase + r] / g.k) : (size_t)(mbase + r);
        xrow[q] = x + ri * (size_t)ldx + 4 * xc;
    }
    float4 xr[2][8];  // X(t) in set t % 2
    auto load_xq = [&](int set, int s, int q) __attribute__((always_inline)) {
        xr[set][q] = *reinterpret_cast<const float4*>(xrow[q] + (size_t)kBK * s);
    };
    auto load_x = [&](int set, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 8; ++q) load_xq(set, s, q);
    };
    const int xgrp = (xc >> 1) & 3;                // the chunk's group of 8 within its block
    const int xpos = 32 * (xc >> 3) + 8 * ((xgrp == 1) ? 2 : (xgrp == 2) ? 1 : xgrp) + 4 * (xc & 1);
    auto store_x = [&](int set, int buf) __attribute__((always_inline)) {
        __bf16* t = xs + buf * kXbfElems + (tid >> 4) * kXStride + xpos;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4v v = {xr[set][q].x, xr[set][q].y, xr[set][q].z, xr[set][q].w};
            *reinterpret_cast<bf16x4*>(t + 16 * q * kXStride) = __builtin_convertvector(v, bf16x4);
        }
    };

    const int h = lane >> 5, c32 = lane & 31;
    f32x16 acc[4][NF];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][f][e] = 0.f;

    // The weight side of block HB of a pair that starts at dword U of its 20-dword stage row:
    // the three 16-byte chunks a lane reads (scale chunk, then the two chunks holding its
    // quants 16h .. 16h + 15), the scale, and four-weight piece (sub, half) of its B operand
    // (quants 16h + 8sub + 4half .. + 3).  HB 0: scale in the low half of dword U, quants at
    // bytes 2 + 16h .. of the pair (dwords U + 4h .. U + 4h + 4, chunks h and h + 1); HB 1:
    // scale in the high half of dword U + 8 (chunk 2), quants at dwords U + 9 + 4h .. U + 12
    // + 4h (chunks 2 + h and 3 + h).
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    auto read_chunks = [&](auto hbc, const uint32_t* stage, int f, u32x4 (&ch)[3]) __attribute__((always_inline)) {
        constexpr int HB = decltype(hbc)::value;
        const u32x4* row = reinterpret_cast<const u32x4*>(stage + (32 * f + c32) * WStage<WN>::kRowDwords);
        ch[0] = row[2 * HB];
        ch[1] = row[2 * HB + h];
        ch[2] = row[2 * HB + h + 1];
    };
    auto scale_of = [&](auto uc, auto hbc, const u32x4 (&ch)[3]) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value, HB = decltype(hbc)::value;
        return HB == 0 ? mf_half_lo(ch[0][U]) : mf_half_hi(ch[0][U]);
    };
    auto piece_word = [&](auto uc, auto hbc, const u32x4 (&ch)[3], int sub, int half)
                          __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value, HB = decltype(hbc)::value;
        const int k = 2 * sub + half;
        auto qw = [&](int j) {  // dword j of the lane's quant run
            const int at = (HB == 0 ? U : U + 1) + j;
            return at < 4 ? ch[1][at] : ch[2][at - 4];
        };
        return HB == 0 ? __builtin_amdgcn_alignbyte(qw(k + 1), qw(k), 2) : qw(k);
    };
    auto piece = [&](auto uc, auto hbc, const u32x4 (&ch)[3], float d, int sub, int half)
                     __attribute__((always_inline)) { return dq4(piece_word(uc, hbc, ch, sub, half), d); };
    // Block HB of the pair in `stage` into B operands bq[sub][f] (quants 16h + 8sub .. + 7).
    auto dequant_block = [&](auto uc, auto hbc, const uint32_t* stage, bf16x8 (&bq)[2][NF])
                             __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            u32x4 ch[3];
            read_chunks(hbc, stage, f, ch);
            const float d = scale_of(uc, hbc, ch);
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
                bq[sub][f] = join4(piece(uc, hbc, ch, d, sub, 0), piece(uc, hbc, ch, d, sub, 1));
        }
    };
    // The MFMAs of block hb of a step (B operands bq, activations of tile buffer buf: LDS
    // positions 32hb .. 32hb + 31 of its rows), with block HB of the pair in `stage`
    // dequantized into bn in between: two weights after every MFMA (a four-weight piece per
    // two MFMAs), in this order (scheduling fences), so the conversions issue while the
    // matrix cores work.  side(j) issues the loads that go out after MFMA j.
    auto mma_dq = [&](auto uc, auto hbc, int buf, int hb, const bf16x8 (&bq)[2][NF], const uint32_t* stage,
                      bf16x8 (&bn)[2][NF], auto&& side) __attribute__((always_inline)) {
        const __bf16* xb = xs + buf * kXbfElems + c32 * kXStride + 32 * hb + 8 * h;
        bf16x8 af[2][4];
        u32x4 ch[NF][3];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(xb + 32 * i * kXStride);
        read_chunks(hbc, stage, 0, ch[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[1][i] = *reinterpret_cast<const bf16x8*>(xb + 32 * i * kXStride + 16);
#pragma unroll
        for (int f = 1; f < NF; ++f) read_chunks(hbc, stage, f, ch[f]);
        float d[NF];
        bf16x4 lo;
        f32x4v wf;
        uint32_t pv;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8 * NF; ++j) {
            const int sub = j / (4 * NF), i = (j / NF) & 3, f = j % NF;
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[sub][i], bq[sub][f], acc[i][f], 0, 0, 0);
            // piece p = j / 2: two of its four weights after each MFMA
            const int p = j >> 1, pf = p >> 2;
            if ((j & 1) == 0) {
                if ((p & 3) == 0) d[pf] = scale_of(uc, hbc, ch[pf]);
                pv = piece_word(uc, hbc, ch[pf], (p >> 1) & 1, p & 1);
                wf[0] = mf_sbyte(pv, 0) * d[pf];
                wf[1] = mf_sbyte(pv, 1) * d[pf];
            } else {
                wf[2] = mf_sbyte(pv, 2) * d[pf];
                wf[3] = mf_sbyte(pv, 3) * d[pf];
                const bf16x4 part = __builtin_convertvector(wf, bf16x4);
                if ((p & 1) == 0) {
                    lo = part;
                } else {
                    bn[(p >> 1) & 1][pf] = join4(lo, part);
                    // keep the finished operand here: otherwise its conversions may sink to
                    // the code that uses it, past the next step's start
                    asm volatile("" : "+v"(bn[(p >> 1) & 1][pf]));
                }
            }
            side(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage_of = [&](int t) __attribute__((always_inline)) {
        return wr + (size_t)(wave * kWRing + t % kWRing) * WStage<WN>::kDwords;
    };

    // Loads for later steps go out one at a time between the MFMAs, so the vector-memory
    // queue drains while the matrix cores work instead of stalling the wave in one burst:
    // the activations of step s+2 during step s's first run (into the register set X(s)
    // used), the weights of step s+2 during its second run.  In issue order X(s+1), W(s+1),
    // X(s+2), so waiting for X(s+1) in the middle of step s leaves X(s+2) in flight and
    // also completes W(s+1), which the second run needs.
    constexpr int kNM = 8 * NF;
    auto spread = [&](int j, int items, auto&& item) __attribute__((always_inline)) {
#pragma unroll
        for (int t = j * items / kNM; t < (j + 1) * items / kNM; ++t) item(t);
    };

    // prologue: X(0) to tile 0; W(1) and X(1) in flight; block 0 of step 0 dequantized
    bf16x8 b0[2][NF], b1[2][NF];
    load_x(0, 0);
    issue_w(0, 0);
    store_x(0, 0);  // X(0) arrived, and W(0), issued after it
    issue_w(1, 1);  // P >= 4
    load_x(1, 1);
    dequant_block(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, stage_of(0), b0);
    auto step = [&](int s, auto uc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;  // s % 4
        // past the end the loads fetch step P - 1 again and the runs dequantize a stale
        // stage; neither is used
        const int sn = s + 2 < P ? s + 2 : P - 1;
        __syncthreads();  // tile s % 2 is complete; every wave is done with tile (s + 1) % 2
        mma_dq(uc, std::integral_constant<int, 1>{}, s & 1, 0, b0, stage_of(s), b1,
               [&](int j) __attribute__((always_inline)) {
                   spread(j, 8, [&](int q) __attribute__((always_inline)) { load_xq(U & 1, sn, q); });
               });
        // X(s+1) arrived, and W(s+1), issued before X(s+2).  Unconditional (past the end:
        // into the tile no wave reads any more) so that no branch lets the compiler sink
        // the loads of X(s+1) from where they are issued to here.
        store_x((U + 1) & 1, (s + 1) & 1);
        mf_wait_vmcnt<8>();  // W(s+1): older than the 8 loads of X(s+2)
        // W(s+2) goes to the stage of W(s-1), free since the previous step's first run
        const int slot = (s + 2) % kWRing;
        mma_dq(std::integral_constant<int, (U + 1) & 3>{}, std::integral_constant<int, 0>{}, s & 1, 1, b1,
               stage_of(s + 1), b0, [&](int j) __attribute__((always_inline)) {
                   spread(j, L, [&](int c) __attribute__((always_inline)) { copy_w(sn, slot, c); });
               });
    };
    for (int s = 0; s < P; s += 4) {  // P is a multiple of 4
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
    }
    mf_wait_vmcnt<0>();  // the last loads and copies (of step P - 1 again) have landed

    // epilogue: register e of fragment (i, f) holds row 32i + 8(e/4) + 4h + e%4, column
    // 32f + c32 of the wave's tile
    if constexpr (GROUPED) y += (size_t)mbase * ldy;
    // the lane's outputs: columns c0 + step * f; a tile inside the call's rows and columns
    // (block-uniform) stores without per-element checks
    auto store_tile = [&](int c0, int step, bool cols_inside) __attribute__((always_inline)) {
        const int m0 = mt * kBM + 4 * h;
        if (mt * kBM + kBM <= M && cols_inside) {
            float* yl = y + (size_t)m0 * ldy + c0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e)
#pragma unroll
                    for (int f = 0; f < NF; ++f)
                        yl[(size_t)(32 * i + 8 * (e >> 2) + (e & 3)) * ldy + step * f] = acc[i][f][e];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + 32 * i + 8 * (e >> 2) + (e & 3);
#pragma unroll
                    for (int f = 0; f < NF; ++f) {
                        const int c = c0 + step * f;
                        if (m < M && c < n_out) y[(size_t)m * ldy + c] = acc[i][f][e];
                    }
                }
        }
    };
    if constexpr (SILU) {
        // Columns 0..15 of a fragment are gate rows, 16..31 the up rows of the same outputs:
        // swapping the 16-lane rows of each half wave brings a gate lane (c32 < 16) its up
        // value; SiLU(gate) * up is formed in place (every lane, the up lanes' results
        // unused), then the gate lanes store.
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float v = acc[i][f][e];
                    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                    acc[i][f][e] = v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)) * __uint_as_float(sw[1]);
                }
        if (c32 < 16) store_tile(nt * (BN / 2) + wave * (WN / 2) + c32, 16, nt * (BN / 2) + BN / 2 <= n_out);
    } else {
        store_tile(nt * BN + wave * WN + c32, 32, nt * BN + BN <= n_out);
    }
}

namespace {

// The widest per-wave tile (96, 64 or 32 weight rows) that wastes at most a tenth of
// its columns on the output edge and, for dense grids, still gives every CU a tile.
// Failing that, the one of those that gives the most tiles (a grid short of the CU
// count leaves CUs idle: 8B down at 512 rows runs 128 tiles of 32-column waves in two
// thirds of the time of 64 tiles of 64-column ones); with none within a tenth, the
// least waste.
int pick_wn(int64_t n_out, bool silu, int64_t row_tiles, int cu_count) {
    const int cand[3] = {96, 64, 32};
    int best = 32, most = 0;
    int64_t most_tiles = 0;
    double best_fill = -1.0;
    for (int wn : cand) {
        const int64_t cols = silu ? 2 * wn : 4 * wn;
        const int64_t nt = (n_out + cols - 1) / cols;
        const double fill = (double)n_out / (double)(nt * cols);
        if (fill >= 0.9 && nt * row_tiles >= cu_count) return wn;
        if (fill >= 0.9 && nt * row_tiles > most_tiles) {
            most_tiles = nt * row_tiles;
            most = wn;
        }
        if (fill > best_fill + 1e-9) {
            best_fill = fill;
            best = wn;
        }
    }
    return most ? most : best;
}

template <int WN, bool SILU, bool GROUPED>
hipError_t launch_wn(unsigned blocks, const uint8_t* w, int n_out, int P, const float* x, int m, int ldx, float* y,
                     int ldy, int m_tiles, int n_tiles, int tiles, const GroupArgs& g, hipStream_t stream) {
    auto kernel = gemm_q8_mfma_kernel<WN, SILU, GROUPED>;
    const size_t lds = mfma_lds_bytes<WN>();
    // once per device and kernel: raise the dynamic LDS limit above the default
    static thread_local uint64_t allowed = 0;  // bit d: done on device d
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 64 || !((allowed >> dev) & 1)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        if (e != hipSuccess) return e;
        if (dev < 64) allowed |= uint64_t(1) << dev;
    }
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(kMfThreads), lds, stream, w, n_out, P, x, m, ldx, y, ldy, m_tiles,
                       n_tiles, tiles, g);
    return hipGetLastError();
}

template <bool SILU, bool GROUPED>
hipError_t launch_any(int wn, unsigned blocks, const uint8_t* w, int n_out, int P, const float* x, int m, int ldx,
                      float* y, int ldy, int m_tiles, int n_tiles, int tiles, const GroupArgs& g,
                      hipStream_t stream) {
    switch (wn) {
        case 96: return launch_wn<96, SILU, GROUPED>(blocks, w, n_out, P, x, m, ldx, y, ldy, m_tiles, n_tiles, tiles, g, stream);
        case 64: return launch_wn<64, SILU, GROUPED>(blocks, w, n_out, P, x, m, ldx, y, ldy, m_tiles, n_tiles, tiles, g, stream);
        default: return launch_wn<32, SILU, GROUPED>(blocks, w, n_out, P, x, m, ldx, y, ldy, m_tiles, n_tiles, tiles, g, stream);
    }
}

}  // namespace

hipError_t launch_gemm_q8_mfma_grouped(const uint8_t* w_stack, size_t expert_bytes, int64_t n_out, int64_t k,
                                       bool silu_pairs, const float* x, int64_t ldx, float* y, int64_t ldy,
                                       const int32_t* offsets, const int32_t* tile_start, const int32_t* sorted,
                                       int n_exp, int top_k, bool gather, int64_t max_tiles, hipStream_t stream) {
    const int P = (int)(k / kBK);
    const int wn = pick_wn(n_out, silu_pairs, 1, 0);
    const int64_t cols = silu_pairs ? 2 * wn : 4 * wn;
    const int n_tiles = (int)((n_out + cols - 1) / cols);
    const int64_t blocks = max_tiles * n_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const GroupArgs g{offsets, tile_start, sorted, n_exp, top_k, expert_bytes, gather};
    return silu_pairs ? launch_any<true, true>(wn, (unsigned)blocks, w_stack, (int)n_out, P, x, 0, (int)ldx, y,
                                               (int)ldy, 1, n_tiles, 0, g, stream)
                      : launch_any<false, true>(wn, (unsigned)blocks, w_stack, (int)n_out, P, x, 0, (int)ldx, y,
                                                (int)ldy, 1, n_tiles, 0, g, stream);
}

hipError_t launch_gemm_q8_mfma(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                               const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / kBK);
    // Weight offsets are 32-bit within the matrix: larger matrices run the float32 path.
    const uint64_t matrix_bytes = (uint64_t)(silu_pairs ? 2 * n_out : n_out) * (uint64_t)P * 68u;
    if (matrix_bytes >= (uint64_t(1) << 32)) return launch_gemv_q8(dev, w, n_out, k, silu_pairs, x, m, ldx, y, ldy, stream);
    const int m_tiles = (int)((m + kBM - 1) / kBM);
    const int wn = pick_wn(n_out, silu_pairs, m_tiles, dev.cu_count);
    const int64_t cols = silu_pairs ? 2 * wn : 4 * wn;
    const int64_t n_tiles = (n_out + cols - 1) / cols;
    const int64_t tiles = n_tiles * m_tiles;
    const int64_t blocks = (tiles + kXcds - 1) / kXcds * kXcds;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const GroupArgs none{};
    return silu_pairs ? launch_any<true, false>(wn, (unsigned)blocks, w, (int)n_out, P, x, (int)m, (int)ldx, y,
                                                (int)ldy, m_tiles, (int)n_tiles, (int)tiles, none, stream)
                      : launch_any<false, false>(wn, (unsigned)blocks, w, (int)n_out, P, x, (int)m, (int)ldx, y,
                                                 (int)ldy, m_tiles, (int)n_tiles, (int)tiles, none, stream);
}

}  // namespace q8k
