// Dense Q8_0 x float32 linears for 1..8 activation rows per launch (gfx950).
//
// The packed-weight linear of "14. Model families and example applications" section
// 14.1 (LinearWeight: quant forms run packed kernels, no global dequantization; q/k/v
// and gate/up fused into one wider matrix each) and the SwiGLU FFN of section 14.2.
// Lockstep batch decode multiplies one pass over the weights by several activation
// rows (section 14.2), so all rows of a launch share every weight load.
//
// Two kernels: gemv_one_row_kernel for one activation row (weights streamed through LDS
// with coalesced direct copies, activations in registers) and gemv_rows_kernel for 2..8
// rows per launch (weights in registers, activations through LDS).  Both run persistent
// grids of the blocks that fit on the device at once, each walking its share of the rows.
// See gemv_core.h for the pair layout and the one-row summation order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "gemv_core.h"
#include "lds_dma.h"
#include "q8_internal.h"

namespace q8k {

// Calls f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{}).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int M>
struct XArr {
    const float4 (&v)[M][16];
    __device__ __forceinline__ float4 get(int m, int, int c) const { return v[m][c]; }
};

// Block-pair formats.  A "pair" is two consecutive blocks (64 weights); rows are 16-byte
// aligned, so pairs start on dword boundaries.  weights<HALF> (the rows kernel) gives the 4
// weights, as exact float32, of inputs 4*cc .. 4*cc+3 of block HALF; mac_row (the one-row
// kernel) adds one pair of R rows against the lane's 64 activations x (float4 c holds inputs
// 4c .. 4c+3 of the pair) and their per-block sums sx.
struct FmtQ8_0 {  // 68 bytes: [d0 | 32 q] [d1 | 32 q]
    static constexpr int kPairBytes = 68, kDwords = 17, kLoads = 5, kMaxR = 4, kSums = 2;
    static __host__ __device__ size_t row_bytes(int P) { return (size_t)P * kPairBytes; }
    // pair j of a row's bytes in LDS (the one-row kernel)
    static __device__ __forceinline__ void lds_load(const uint8_t* item_row, int j, uint32_t (&w)[kDwords]) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(item_row + kPairBytes * j);
#pragma unroll
        for (int q = 0; q < kDwords; ++q) w[q] = src[q];
    }
    static __device__ __forceinline__ void load(const uint8_t* p, uint32_t (&w)[kDwords]) { load_pair(p, w); }
    static __device__ __forceinline__ void load(const uint8_t* row, int pc, uint32_t (&w)[kDwords]) {
        load_pair(row + (size_t)kPairBytes * pc, w);
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4], int = 0) {
        if constexpr (HALF == 0) {  // block 0: scale in dword 0 (low half), quants at bytes 2..33
            const float d = half_lo(w[0]);
            wf[0] = sbyte<2>(w[cc]) * d;
            wf[1] = sbyte<3>(w[cc]) * d;
            wf[2] = sbyte<0>(w[cc + 1]) * d;
            wf[3] = sbyte<1>(w[cc + 1]) * d;
        } else {  // block 1: scale in dword 8 (high half), quants in dwords 9..16
            const float d = half_hi(w[8]);
            const uint32_t v = w[9 + cc];
            wf[0] = sbyte<0>(v) * d;
            wf[1] = sbyte<1>(v) * d;
            wf[2] = sbyte<2>(v) * d;
            wf[3] = sbyte<3>(v) * d;
        }
    }
    // per block: t = sum q*x, then acc = fma(d, t, acc) (gemv_core.h mac_pair)
    template <int R>
    static __device__ __forceinline__ void mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                   const float (&)[2], float (&acc)[R][1], int);
};

// The 4 quants (exact in float32, no scale) of inputs 4*cc .. 4*cc+3 of block HALF of a
// Q8_0 pair held as 17 dwords (the layout FmtQ8_0::weights reads).
template <int HALF>
__device__ __forceinline__ void q8_quants(const uint32_t (&w)[17], int cc, float (&wq)[4]) {
    if constexpr (HALF == 0) {  // quants at bytes 2..33
        wq[0] = sbyte<2>(w[cc]);
        wq[1] = sbyte<3>(w[cc]);
        wq[2] = sbyte<0>(w[cc + 1]);
        wq[3] = sbyte<1>(w[cc + 1]);
    } else {  // quants in dwords 9..16
        wq[0] = sbyte<0>(w[9 + cc]);
        wq[1] = sbyte<1>(w[9 + cc]);
        wq[2] = sbyte<2>(w[9 + cc]);
        wq[3] = sbyte<3>(w[9 + cc]);
    }
}

// GGUF Q4_0: 36 bytes a pair, [d0 | 16 bytes] [d1 | 16 bytes]; weight j < 16 of a block is
// the low nibble of its byte j, weight j + 16 the high nibble; w = d * (nibble - 8), exact
// in float32 (a 4-bit integer times an 11-bit scale).
struct FmtQ4_0 {
    static constexpr int kPairBytes = 36, kDwords = 9, kLoads = 3, kMaxR = 4, kSums = 2;
    static __host__ __device__ size_t row_bytes(int P) { return (size_t)P * kPairBytes; }
    static __device__ __forceinline__ void lds_load(const uint8_t* item_row, int j, uint32_t (&w)[kDwords]) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(item_row + kPairBytes * j);
#pragma unroll
        for (int q = 0; q < kDwords; ++q) w[q] = src[q];
    }
    static __device__ __forceinline__ void load(const uint8_t* row, int pc, uint32_t (&w)[kDwords]) {
        load(row + (size_t)kPairBytes * pc, w);
    }
    static __device__ __forceinline__ void load(const uint8_t* p, uint32_t (&w)[kDwords]) {
        const u32x4_a4 a = *reinterpret_cast<const u32x4_a4*>(p);
        const u32x4_a4 b = *reinterpret_cast<const u32x4_a4*>(p + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        w[8] = *reinterpret_cast<const uint32_t*>(p + 32);
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4], int = 0) {
        const int c4 = cc & 3;  // quant dword of the block: bytes 4*c4 .. 4*c4+3
        float d;
        uint32_t v;
        if constexpr (HALF == 0) {  // scale = low half of dword 0, quant bytes at 2..17
            d = half_lo(w[0]);
            v = __builtin_amdgcn_alignbyte(w[c4 + 1], w[c4], 2);
        } else {  // scale = high half of dword 4, quant bytes in dwords 5..8
            d = half_hi(w[4]);
            v = w[5 + c4];
        }
        const uint32_t nib = (cc < 4 ? v : v >> 4) & 0x0F0F0F0Fu;  // inputs 4cc..: low nibbles, then high
        // q*d - 8d in one fma: the exact value (q - 8)*d has at most 15 significant bits
        const float m8d = -8.0f * d;
        wf[0] = __builtin_fmaf((float)(nib & 0xFFu), d, m8d);
        wf[1] = __builtin_fmaf((float)((nib >> 8) & 0xFFu), d, m8d);
        wf[2] = __builtin_fmaf((float)((nib >> 16) & 0xFFu), d, m8d);
        wf[3] = __builtin_fmaf((float)(nib >> 24), d, m8d);
    }
    // per block: t = sum nibble*x (nibbles 0..15, exact), then acc = fma(d, t - 8*sx, acc):
    // sum (nibble - 8)*d*x with the offset carried by the block's activation sum sx
    template <int R>
    static __device__ __forceinline__ void mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                   const float (&sx)[2], float (&acc)[R][1], int) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float d = half == 0 ? half_lo(w[r][0]) : half_hi(w[r][4]);
                float t = 0.0f;
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    // quant bytes 4*c4 .. 4*c4+3 of the block: weights j = 4*c4 + i (low nibbles)
                    // and 16 + j (high nibbles)
                    const uint32_t v = half == 0 ? __builtin_amdgcn_alignbyte(w[r][c4 + 1], w[r][c4], 2) : w[r][5 + c4];
                    const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
                    const float4 xl = x[0][8 * half + c4], xh = x[0][8 * half + 4 + c4];
                    t = __builtin_fmaf((float)(lo & 0xFFu), xl.x, t);
                    t = __builtin_fmaf((float)((lo >> 8) & 0xFFu), xl.y, t);
                    t = __builtin_fmaf((float)((lo >> 16) & 0xFFu), xl.z, t);
                    t = __builtin_fmaf((float)(lo >> 24), xl.w, t);
                    t = __builtin_fmaf((float)(hi & 0xFFu), xh.x, t);
                    t = __builtin_fmaf((float)((hi >> 8) & 0xFFu), xh.y, t);
                    t = __builtin_fmaf((float)((hi >> 16) & 0xFFu), xh.z, t);
                    t = __builtin_fmaf((float)(hi >> 24), xh.w, t);
                }
                acc[r][0] = __builtin_fmaf(d, t - 8.0f * sx[half], acc[r][0]);
            }
        }
    }
};

// d*sc and dmin*m of sub-block 2c + HALF from a Q4_K / Q5_K header (w0: d | dmin, w1..w3: the
// 12 scale bytes).  Sub-blocks 0..3: the low six bits of bytes j and j + 4; 4..7: a nibble of
// byte j + 4 below the top two bits of byte j - 4 (scale) or j (min).  Lanes of a wave hold
// different pairs, so the choice is a bit select, not a branch.
template <int HALF>
__device__ __forceinline__ void kq_scale_min(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, int c, float& ds,
                                             float& dm) {
    const uint32_t sh = 8u * (uint32_t)(2 * (c & 1) + HALF);
    const uint32_t b1 = (w1 >> sh) & 0xFFu, b2 = (w2 >> sh) & 0xFFu, b3 = (w3 >> sh) & 0xFFu;
    const uint32_t hi = 0u - (uint32_t)(c >> 1);  // all ones for sub-blocks 4..7
    const uint32_t sc = ((b1 & 63u) & ~hi) | (((b3 & 15u) | ((b1 >> 2) & 0x30u)) & hi);
    const uint32_t mn = ((b2 & 63u) & ~hi) | (((b3 >> 4) | ((b2 >> 2) & 0x30u)) & hi);
    ds = half_lo(w0) * (float)sc;
    dm = half_hi(w0) * (float)mn;
}

// acc += d*sc * sum(q*x) - dmin*m * sum(x) over the 32 inputs of one sub-block: t is a chain
// of fmas over the quants (integers 0..31, exact), sx the sub-block's activation sum
__device__ __forceinline__ float kq_chain4(uint32_t v, float4 xv, float t) {
    t = __builtin_fmaf((float)(v & 0xFFu), xv.x, t);
    t = __builtin_fmaf((float)((v >> 8) & 0xFFu), xv.y, t);
    t = __builtin_fmaf((float)((v >> 16) & 0xFFu), xv.z, t);
    return __builtin_fmaf((float)(v >> 24), xv.w, t);
}

// GGUF Q4_K: 144-byte super-blocks of 256 weights (four pairs each): d and dmin
// (binary16), 12 bytes of packed 6-bit sub-block scales and mins, 128 bytes of nibbles.
// Pair c of a super-block (inputs 64c .. 64c+63) is sub-block 2c (the low nibbles of quant
// bytes 32c .. 32c+31) then sub-block 2c+1 (their high nibbles); w = d*sc*q - dmin*m,
// computed as fma(q, d*sc, -dmin*m) (the two products are exact in float32).
struct FmtQ4_K {
    // w[0]: d | dmin, w[1..3]: the scale bytes, w[4..11]: the pair's 32 quant bytes
    static constexpr int kDwords = 12, kLoads = 3, kMaxR = 2, kSums = 2;
    static __host__ __device__ size_t row_bytes(int P) { return (size_t)(P / 4) * 144; }
    // pair j of a row's bytes in LDS (the one-row kernel; rows start on 16-byte boundaries)
    static __device__ __forceinline__ void lds_load(const uint8_t* item_row, int j, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = item_row + 144 * (j >> 2);
        const uint32_t* h = reinterpret_cast<const uint32_t*>(sb);
        const uint32_t* q = reinterpret_cast<const uint32_t*>(sb + 16 + 32 * (j & 3));
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = h[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[4 + i] = q[i];
    }
    // per sub-block: t = sum nibble*x, acc = fma(d*sc, t, acc), acc = fma(-dmin*m, sx, acc)
    template <int R>
    static __device__ __forceinline__ void mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                   const float (&sx)[2], float (&acc)[R][1], int p) {
        const int c = p & 3;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float ds[2], dm[2];
            kq_scale_min<0>(w[r][0], w[r][1], w[r][2], w[r][3], c, ds[0], dm[0]);
            kq_scale_min<1>(w[r][0], w[r][1], w[r][2], w[r][3], c, ds[1], dm[1]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                float t = 0.0f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) t = kq_chain4((w[r][4 + cc] >> (4 * hb)) & 0x0F0F0F0Fu, x[0][8 * hb + cc], t);
                acc[r][0] = __builtin_fmaf(ds[hb], t, acc[r][0]);
                acc[r][0] = __builtin_fmaf(-dm[hb], sx[hb], acc[r][0]);
            }
        }
    }
    static __device__ __forceinline__ void load(const uint8_t* row, int pc, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = row + (size_t)(pc >> 2) * 144;
        const u32x4_a4 h = *reinterpret_cast<const u32x4_a4*>(sb);
        const u32x4_a4 a = *reinterpret_cast<const u32x4_a4*>(sb + 16 + 32 * (pc & 3));
        const u32x4_a4 b = *reinterpret_cast<const u32x4_a4*>(sb + 32 + 32 * (pc & 3));
        w[0] = h.x; w[1] = h.y; w[2] = h.z; w[3] = h.w;
        w[4] = a.x; w[5] = a.y; w[6] = a.z; w[7] = a.w;
        w[8] = b.x; w[9] = b.y; w[10] = b.z; w[11] = b.w;
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4], int pc) {
        // sub-block j = 2c + HALF; its scale-byte position within dwords 1, 2, 3 is j % 4
        const int c = pc & 3;
        const uint32_t sh = 8u * (uint32_t)(2 * (c & 1) + HALF);
        const uint32_t b1 = (w[1] >> sh) & 0xFFu, b2 = (w[2] >> sh) & 0xFFu, b3 = (w[3] >> sh) & 0xFFu;
        // sub-blocks 0..3: the low six bits of bytes j and j + 4; sub-blocks 4..7: a nibble
        // of byte j + 4 below the top two bits of byte j - 4 (scale) or j (min).  Lanes of
        // a wave hold different pairs, so the choice is a bit select, not a branch.
        const uint32_t hi = 0u - (uint32_t)(c >> 1);  // all ones for sub-blocks 4..7
        const uint32_t sc = ((b1 & 63u) & ~hi) | (((b3 & 15u) | ((b1 >> 2) & 0x30u)) & hi);
        const uint32_t mn = ((b2 & 63u) & ~hi) | (((b3 >> 4) | ((b2 >> 2) & 0x30u)) & hi);
        const float ds = half_lo(w[0]) * (float)sc, dm = half_hi(w[0]) * (float)mn;
        const uint32_t v = (w[4 + cc] >> (4 * HALF)) & 0x0F0F0F0Fu;  // inputs 4cc .. 4cc+3 of the half
        wf[0] = __builtin_fmaf((float)(v & 0xFFu), ds, -dm);
        wf[1] = __builtin_fmaf((float)((v >> 8) & 0xFFu), ds, -dm);
        wf[2] = __builtin_fmaf((float)((v >> 16) & 0xFFu), ds, -dm);
        wf[3] = __builtin_fmaf((float)(v >> 24), ds, -dm);
    }
};

// GGUF Q5_K: 176-byte super-blocks of 256 weights (four pairs each): the Q4_K header (d,
// dmin, 12 bytes of 6-bit scales and mins), 32 bytes qh, 128 bytes of nibbles.  Pair c is
// sub-block 2c (low nibbles of quant bytes 32c .. 32c+31) then 2c+1 (high nibbles); the
// quant of input l of sub-block 2c + HALF gains 16 when bit 2c + HALF of qh[l] is set;
// w = fma(q, d*sc, -dmin*m) as for Q4_K.
struct FmtQ5_K {
    // w[0..3]: the header, w[4..11]: qh, w[12..19]: the pair's 32 quant bytes
    static constexpr int kDwords = 20, kLoads = 5, kMaxR = 2, kSums = 2;
    static __host__ __device__ size_t row_bytes(int P) { return (size_t)(P / 4) * 176; }
    static __device__ __forceinline__ void lds_load(const uint8_t* item_row, int j, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = item_row + 176 * (j >> 2);
        const uint32_t* h = reinterpret_cast<const uint32_t*>(sb);  // header and qh: dwords 0..11
        const uint32_t* q = reinterpret_cast<const uint32_t*>(sb + 48 + 32 * (j & 3));
#pragma unroll
        for (int i = 0; i < 12; ++i) w[i] = h[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[12 + i] = q[i];
    }
    template <int R>
    static __device__ __forceinline__ void mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                   const float (&sx)[2], float (&acc)[R][1], int p) {
        const int c = p & 3;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float ds[2], dm[2];
            kq_scale_min<0>(w[r][0], w[r][1], w[r][2], w[r][3], c, ds[0], dm[0]);
            kq_scale_min<1>(w[r][0], w[r][1], w[r][2], w[r][3], c, ds[1], dm[1]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                float t = 0.0f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const uint32_t top = (w[r][4 + cc] >> (uint32_t)(2 * c + hb)) & 0x01010101u;
                    const uint32_t v = ((w[r][12 + cc] >> (4 * hb)) & 0x0F0F0F0Fu) | (top << 4);
                    t = kq_chain4(v, x[0][8 * hb + cc], t);
                }
                acc[r][0] = __builtin_fmaf(ds[hb], t, acc[r][0]);
                acc[r][0] = __builtin_fmaf(-dm[hb], sx[hb], acc[r][0]);
            }
        }
    }
    static __device__ __forceinline__ void load(const uint8_t* row, int pc, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = row + (size_t)(pc >> 2) * 176;
        const uint8_t* src[5] = {sb, sb + 16, sb + 32, sb + 48 + 32 * (pc & 3), sb + 64 + 32 * (pc & 3)};
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(src[i]);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4], int pc) {
        const int c = pc & 3;
        const uint32_t sh = 8u * (uint32_t)(2 * (c & 1) + HALF);
        const uint32_t b1 = (w[1] >> sh) & 0xFFu, b2 = (w[2] >> sh) & 0xFFu, b3 = (w[3] >> sh) & 0xFFu;
        const uint32_t hi = 0u - (uint32_t)(c >> 1);  // sub-blocks 4..7: bit select, not a branch
        const uint32_t sc = ((b1 & 63u) & ~hi) | (((b3 & 15u) | ((b1 >> 2) & 0x30u)) & hi);
        const uint32_t mn = ((b2 & 63u) & ~hi) | (((b3 >> 4) | ((b2 >> 2) & 0x30u)) & hi);
        const float ds = half_lo(w[0]) * (float)sc, dm = half_hi(w[0]) * (float)mn;
        const uint32_t top = (w[4 + cc] >> (uint32_t)(2 * c + HALF)) & 0x01010101u;
        const uint32_t v = ((w[12 + cc] >> (4 * HALF)) & 0x0F0F0F0Fu) | (top << 4);
        wf[0] = __builtin_fmaf((float)(v & 0xFFu), ds, -dm);
        wf[1] = __builtin_fmaf((float)((v >> 8) & 0xFFu), ds, -dm);
        wf[2] = __builtin_fmaf((float)((v >> 16) & 0xFFu), ds, -dm);
        wf[3] = __builtin_fmaf((float)(v >> 24), ds, -dm);
    }
};

// GGUF Q6_K: 210-byte super-blocks of 256 weights (four pairs each): ql[128], qh[64],
// int8 scales[16], d (binary16).  Pair c of a super-block lies in half t = c/2; its block
// HALF holds the weights 128t + 32k + l (l < 32) with k = 2(c%2) + HALF: their low four
// bits are the low (c%2 == 0) or high nibble of ql[64t + 32 HALF + l], their top two bits
// bits 2k, 2k+1 of qh[32t + l], their scale scales[8t + 2k + l/16];
// w = fma(q, d*scale, -32 d*scale), exact in float32 (at most 23 significant bits).
// Super-blocks start on 2-byte boundaries: the loads read whole dwords from the dword
// boundary at or below each field (never past the super-block: d is a 16-bit load) and
// the weights realign them with v_alignbyte by 0 or 2 bytes.
struct FmtQ6_K {
    // w[0..16]: ql of half t, w[17..25]: qh of half t, w[26..27]: the pair's four scale
    // bytes, w[28]: d, w[29]: the realignment (0 or 2 bytes)
    static constexpr int kDwords = 30, kLoads = 11, kMaxR = 2, kSums = 4;
    static __host__ __device__ size_t row_bytes(int P) { return (size_t)(P / 4) * 210; }
    // pair j of a row's bytes in LDS, realigned as in load (rows start on 16-byte boundaries;
    // the one-row kernel takes Q6_K rows of a multiple of 8 super-blocks)
    static __device__ __forceinline__ void lds_load(const uint8_t* item_row, int j, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = item_row + 210 * (j >> 2);
        const uint32_t shift = (uint32_t)(uintptr_t)sb & 3u;  // 0 or 2
        const int t = (j >> 1) & 1;
        const uint32_t* ql = reinterpret_cast<const uint32_t*>(sb + 64 * t - shift);
        const uint32_t* qh = reinterpret_cast<const uint32_t*>(sb + 128 + 32 * t - shift);
        const uint32_t* scl = reinterpret_cast<const uint32_t*>(sb + 192 + 8 * t + 4 * (j & 1) - shift);
#pragma unroll
        for (int i = 0; i < 17; ++i) w[i] = ql[i];
#pragma unroll
        for (int i = 0; i < 9; ++i) w[17 + i] = qh[i];
        w[26] = scl[0];
        w[27] = scl[1];  // used only when realigning (then it ends at byte 209); else it may reach
                         // 2 bytes into the next super-block of the LDS slot, unused
        w[28] = *reinterpret_cast<const uint16_t*>(sb + 208);
        w[29] = shift;
    }
    // per group of 16 weights (scale s): t = sum q*x, then acc = fma(d*s, t - 32*sx, acc)
    template <int R>
    static __device__ __forceinline__ void mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                   const float (&sx)[4], float (&acc)[R][1], int p) {
        const int hi_nib = p & 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t shift = w[r][29];
            const float d = half_lo(w[r][28]);
            const uint32_t scw = __builtin_amdgcn_alignbyte(w[r][27], w[r][26], shift);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int k = 2 * hi_nib + hb;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    float t = 0.0f;
#pragma unroll
                    for (int cc = 4 * g; cc < 4 * g + 4; ++cc) {
                        const uint32_t qlw = __builtin_amdgcn_alignbyte(w[r][8 * hb + cc + 1], w[r][8 * hb + cc], shift);
                        const uint32_t qhw = __builtin_amdgcn_alignbyte(w[r][17 + cc + 1], w[r][17 + cc], shift);
                        const uint32_t q6 =
                            ((qlw >> (4 * hi_nib)) & 0x0F0F0F0Fu) | (((qhw >> (2 * k)) & 0x03030303u) << 4);
                        t = kq_chain4(q6, x[0][8 * hb + cc], t);
                    }
                    const float ds = d * (float)(int)(int8_t)(scw >> (8 * (2 * hb + g)));
                    acc[r][0] = __builtin_fmaf(ds, t - 32.0f * sx[2 * hb + g], acc[r][0]);
                }
            }
        }
    }
    static __device__ __forceinline__ void load(const uint8_t* row, int pc, uint32_t (&w)[kDwords]) {
        const uint8_t* sb = row + (size_t)(pc >> 2) * 210;
        const uint32_t shift = (uint32_t)(uintptr_t)sb & 3u;  // 0 or 2
        const int t = (pc >> 1) & 1;
        const uint8_t* ql = sb + 64 * t - shift;
        const uint8_t* qh = sb + 128 + 32 * t - shift;
        const uint8_t* scl = sb + 192 + 8 * t + 4 * (pc & 1) - shift;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(ql + 16 * i);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
        w[16] = *reinterpret_cast<const uint32_t*>(ql + 64);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(qh + 16 * i);
            w[17 + 4 * i] = v.x; w[18 + 4 * i] = v.y; w[19 + 4 * i] = v.z; w[20 + 4 * i] = v.w;
        }
        w[25] = *reinterpret_cast<const uint32_t*>(qh + 32);
        w[26] = *reinterpret_cast<const uint32_t*>(scl);
        w[27] = *reinterpret_cast<const uint32_t*>(scl + (shift ? 4 : 0));  // only read when realigning
        w[28] = *reinterpret_cast<const uint16_t*>(sb + 208);
        w[29] = shift;
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4], int pc) {
        const uint32_t shift = w[29];
        const int hi_nib = pc & 1;             // c % 2
        const int k = 2 * hi_nib + HALF;
        const uint32_t qlw = __builtin_amdgcn_alignbyte(w[8 * HALF + cc + 1], w[8 * HALF + cc], shift);
        const uint32_t qhw = __builtin_amdgcn_alignbyte(w[17 + cc + 1], w[17 + cc], shift);
        const uint32_t scw = __builtin_amdgcn_alignbyte(w[27], w[26], shift);
        const uint32_t q6 = ((qlw >> (4 * hi_nib)) & 0x0F0F0F0Fu) | (((qhw >> (2 * k)) & 0x03030303u) << 4);
        const float sc = (float)(int)(int8_t)(scw >> (8 * (2 * HALF + (cc >> 2))));
        const float ds = half_lo(w[28]) * sc;
        const float m32 = -32.0f * ds;
        wf[0] = __builtin_fmaf((float)(q6 & 0xFFu), ds, m32);
        wf[1] = __builtin_fmaf((float)((q6 >> 8) & 0xFFu), ds, m32);
        wf[2] = __builtin_fmaf((float)((q6 >> 16) & 0xFFu), ds, m32);
        wf[3] = __builtin_fmaf((float)(q6 >> 24), ds, m32);
    }
};

template <int R>
__device__ __forceinline__ void FmtQ8_0::mac_row(const uint32_t (&w)[R][kDwords], const float4 (&x)[1][16],
                                                 const float (&)[2], float (&acc)[R][1], int) {
    mac_pair<1, R>(w, XArr<1>{x}, 0, acc);
}

// One activation row (the decode class).  A wave works on "items": the pairs j + S*i
// (slot j, round i) of one row group, i.e. one contiguous stretch of at most 4352 weight
// bytes per row (64 pairs; with G > 1 rows per wave, G whole rows).  The wave copies an
// item's bytes (and, fused, the matching up rows' bytes) straight into its own LDS slot
// with five wave-wide loads per row, each lane reading consecutive bytes (1 KB per load
// instruction), so every load is fully coalesced; each lane then reads its 68-byte pair
// from LDS (a 17-dword stride: conflict-free) and multiplies it in registers.  Reading the
// pairs directly (a 68-byte stride across lanes) made every load instruction touch every
// cache line of the row and measured ~20% slower.  A slot is refilled with the item D
// ahead as soon as its bytes are in registers, so D items per wave stay in flight while
// one is multiplied.
//
// Activations: each block copies x into LDS with 1 KB direct copies (the activations of
// 4 pairs each), pair p's 256 bytes at p * kXRow with its 16-byte chunk c rotated to
// position (c + p) mod 16, so that the lanes' reads of their own pair's chunk c fall in 16
// different bank groups (conflict-free; an unrotated layout conflicts 64 ways, a padded one
// needs one 256-byte copy per pair and measured 5-12% slower); each lane then keeps the
// activations of its pairs in registers.  The activation copies are issued before the first
// weight copies, so the wait for them (then a barrier) leaves the weights in flight.
//
// Items of wave w: the row groups w, w + W, w + 2W, ... (W waves in the grid, `ipw`
// items per wave, a multiple of NR), so the grid streams one window of the matrix at a
// time; items past the end repeat the last row group (same bits to the same address).
// Per-output order and arithmetic are those of gemv_core.h (mac_pair, then the xor
// butterfly over the S slots).
constexpr int kXRow = 256;

template <class Fmt, int R, int NR, int D, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void gemv_one_row_kernel(const uint8_t* __restrict__ w, int n_out, int P,
                                                              int log2S, const float* __restrict__ x,
                                                              float* __restrict__ y, int ipw) {
    static_assert((D - 1) * 5 * R < 64 && D * 5 * R < 64, "copies in flight must fit the vmcnt counter");
    extern __shared__ float4 smem4[];
    uint8_t* smem = reinterpret_cast<uint8_t*>(smem4);
    const int S = 1 << log2S;
    const int G = 64 >> log2S;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & (S - 1);
    const int g = lane >> log2S;
    const size_t row_bytes = Fmt::row_bytes(P);
    const int total = ((n_out + G - 1) / G) * NR;  // items: (row group, round)
    const int wid = blockIdx.x * NW + wv;
    const int nw = gridDim.x * NW;
    uint8_t* ring = smem + (size_t)P * kXRow + (size_t)wv * (D * R * kLdsItemBytes);
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ring);
    const uint32_t x_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

    // local item -> (row group, round), clamped to the last row group past the end
    auto item_of = [&](int itl, int& rg, int& i) __attribute__((always_inline)) {
        const int it = (wid + (itl / NR) * nw) * NR + (itl % NR);
        const int itc = it < total ? it : total - NR + (it % NR);
        rg = itc / NR;
        i = itc % NR;
    };
    // copy item itl's bytes (R rows) into LDS slot `slot`: 5 * R vmcnt events
    auto issue = [&](int itl, int slot) __attribute__((always_inline)) {
        int rg, i;
        item_of(itl, rg, i);
        rg = __builtin_amdgcn_readfirstlane(rg);
        i = __builtin_amdgcn_readfirstlane(i);
        const int row0 = rg * G;
        int len;
        if (G > 1) {  // G whole rows (P <= S): the rows that exist
            const int rows = (n_out - row0) < G ? (n_out - row0) : G;
            len = rows * (int)row_bytes;
        } else {  // pairs S*i .. of one row
            const int pairs = (P - S * i) < S ? (P - S * i) : S;
            len = (int)Fmt::row_bytes(pairs);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            lds_copy_4352<NT>(w + (size_t)(row0 + r * n_out) * row_bytes + Fmt::row_bytes(S * i), len,
                          ring_lds + (slot * R + r) * kLdsItemBytes, lane);
    };

    const bool active = wid < total / NR;
    const int n_pro = active ? (ipw < D ? ipw : D) : 0;
    for (int q = wv; q < (P >> 2); q += NW) {  // 1 KB = the activations of 4 pairs per copy
        const int p = 4 * q + (lane >> 4), pos = lane & 15;
        const int c = (pos - p) & 15;  // chunk c of pair p lands in position (c + p) mod 16
        lds_copy16(reinterpret_cast<const uint8_t*>(x) + 256 * p + 16 * c,
                   reinterpret_cast<void*>((uintptr_t)(x_lds + 1024 * q)));
    }
    static_for<D>([&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        if (s < n_pro) issue(s, s);
    });
    // the activation copies are the oldest: wait until at most the weight prologue is
    // outstanding, then every wave's share of x is in LDS after the barrier
    static_for<D + 1>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if (n_pro == k) wait_vmcnt_mem<k * 5 * R>();
    });
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (!active) return;
    float4 xr[NR][1][16];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = j + S * i;
        const int pc = p < P ? p : p - P;  // a slot past the row: any pair (not multiplied)
#pragma unroll
        for (int c = 0; c < 16; ++c)
            xr[i][0][c] = *reinterpret_cast<const float4*>(smem + kXRow * pc + 16 * ((c + pc) & 15));
    }
    // per-block activation sums of the lane's pairs (used by formats with an offset)
    // (per group of 64 / kSums inputs: 2 groups of 32, or 4 of 16 for Q6_K's scale groups)
    constexpr int kS = Fmt::kSums, kGroupF4 = 16 / kS;
    float sx[NR][kS];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int hb = 0; hb < kS; ++hb) {
            float a = 0.0f;
#pragma unroll
            for (int c = 0; c < kGroupF4; ++c) {
                const float4 v = xr[i][0][kGroupF4 * hb + c];
                a += v.x;
                a += v.y;
                a += v.z;
                a += v.w;
            }
            sx[i][hb] = a;
        }
    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.0f;
    // Outputs wait in registers: the result of the wave's t-th row group stays in lanes
    // j == t % S (one per output row of the group) and goes out in one store per S row
    // groups.  A store between the weight copies would also be counted by the vmcnt waits
    // above and make them wait for the newest copies.
    float keep = 0.0f;
    int kept_base = 0;  // local row group of lane j == 0's kept value
    auto flush = [&](int count) __attribute__((always_inline)) {
        if (j < count) {
            int rg, ii;
            item_of((kept_base + j) * NR, rg, ii);
            const int n = rg * G + g;
            y[n < n_out ? n : n_out - 1] = keep;  // a clamped duplicate stores the same bits
        }
    };

    for (int rgl = 0; rgl < ipw / NR; ++rgl) {
        static_for<NR>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const int itl = rgl * NR + i;
            const int slot = itl % D;
            // items itl .. min(itl + D - 1, ipw - 1) are in flight: wait for the oldest
            const int rem = ipw - 1 - itl;
            if (rem >= D - 1) {
                wait_vmcnt_mem<(D - 1) * 5 * R>();
            } else {
                static_for<D - 1>([&](auto kc) __attribute__((always_inline)) {
                    constexpr int k = decltype(kc)::value;
                    if (rem == k) wait_vmcnt_mem<k * 5 * R>();
                });
            }
            int rg, ii;
            item_of(itl, rg, ii);
            const int n = rg * G + g;
            const int nc = n < n_out ? n : n_out - 1;  // a lane past the matrix: the last row
            const int lds_off = G > 1 ? (nc - rg * G) * (int)row_bytes : 0;  // the lane's row in the item
            uint32_t wr[R][Fmt::kDwords];
#pragma unroll
            for (int r = 0; r < R; ++r) Fmt::lds_load(ring + (slot * R + r) * kLdsItemBytes + lds_off, j, wr[r]);
            wait_lgkmcnt_mem<0>();
            if (itl + D < ipw) issue(itl + D, slot);  // refill the slot just read
            if (j + S * i < P) Fmt::template mac_row<R>(wr, xr[i], sx[i], acc, j + S * i);
            if constexpr (i == NR - 1) {
                for (int off = S >> 1; off >= 1; off >>= 1) {
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][0] += __shfl_xor(acc[r][0], off, 64);
                }
                // every lane of the row holds the same bits
                const float v = R == 2 ? silu_mul(acc[0][0], acc[R - 1][0]) : acc[0][0];
                const int t = rgl - kept_base;
                if (j == t) keep = v;
                if (t == S - 1) {
                    flush(S);
                    kept_base = rgl + 1;
                }
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r][0] = 0.0f;
            }
        });
    }
    flush(ipw / NR - kept_base);
}

// Several activation rows (1 <= M <= 8 per launch; the class used for 2..255 rows).  A
// block tile is 8*R rows (fused: R gate/up row pairs) over the whole K, worked on by two
// groups of 2 waves: group h takes the chunks h, h+2, h+4, ... of 16 pairs (1024 inputs)
// each.  16 lanes share a row (lane j owns pair j of a chunk), 4 row slots per wave, R
// rows (or row pairs) per lane, so each activation value read from LDS feeds R (or 2R)
// rows.  Each step copies both groups' activation chunks into slot-major LDS with
// direct-to-LDS loads (no register round trip); the weights of the step after next are
// loaded while a step is multiplied (a ring of two steps in registers).  Q8_0: per block
// t = fma chain of q_k * x_k (the quants exact in float32), then acc = fma(d, t, acc);
// the other formats: weights dequantized exactly in float32, one fma per weight and
// activation row.
//
// Per-output order: over the lane's weights (its pair of each of the group's chunks in
// increasing order, blocks and inputs in increasing order), the xor butterfly over the
// 16 lanes (8, 4, 2, 1), then group 0's sum + group 1's sum.  It depends only on K,
// never on M or R, so every row of a 2..255-row call is bit-identical to the same row in
// any other such call.
constexpr int kRowsThreads = 256;

template <class Fmt, int M, int R, bool SILU>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemv_rows_kernel(
    const uint8_t* __restrict__ w, int n_out, int P, const float* __restrict__ x, int ldx, float* __restrict__ y,
    int ldy) {
    constexpr int RR = SILU ? 2 * R : R;  // weight rows per lane
    // Activations of one half chunk per group (inputs of block 0, or of block 1, of each
    // of the chunk's 16 pairs), slot-major [m][c][j] float4 with c the quant dword 0..7 of
    // the half.  Half 0 lives in xa and half 1 in xb: while one is multiplied the other is
    // being filled.  Two variables rather than one array, so that the copy into one is
    // known not to touch the other.
    __shared__ float4 xa[2][M * 128];
    __shared__ float4 xb[2][M * 128];
    __shared__ float part[8 * RR * M];    // group 1's row sums: [slot][r][m]
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS copy bases)
    const int h = wv >> 1;                // group
    const int lane = tid & 63;
    const int j = lane & 15;
    const int slot = (wv & 1) * 4 + (lane >> 4);  // row slot within the group, 0..7
    const size_t row_bytes = Fmt::row_bytes(P);
    const int nch = (P + 15) >> 4;
    const int steps = (nch + 1) >> 1;
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    // this block's tiles: blockIdx.x, + gridDim.x, ...; its items: (tile, step) in order
    const int my_tiles = (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int items = my_tiles * steps;
    __builtin_assume(steps >= 1);  // P >= 4 (K is a positive multiple of 256)
    __builtin_assume(items >= 1);  // the grid has at most `tiles` blocks

    // first output row of the lane's slot in tile i of this block (past the end: clamped,
    // so the lane duplicates the last row, same bits)
    auto out_row = [&](int i, int r) __attribute__((always_inline)) {
        const int n = ((int)blockIdx.x + i * (int)gridDim.x) * (8 * R) + slot * R + r;
        return n < n_out ? n : n_out - 1;
    };
    // the group's chunk at step st, clamped to a valid chunk (a clamped step is not used)
    auto chunk_of = [&](int st) __attribute__((always_inline)) {
        const int ch = h + 2 * st;
        return ch < nch ? ch : nch - 1;
    };
    auto load_w = [&](int i, int st, uint32_t(&wr)[RR][Fmt::kDwords]) __attribute__((always_inline)) {
        const int p = 16 * chunk_of(st) + j;
        const int pc = p < P ? p : P - 1;  // past the row: a pair of the same row (unused)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = out_row(i, r);
            Fmt::load(w + (size_t)n * row_bytes, pc, wr[r]);
            if constexpr (SILU) Fmt::load(w + (size_t)(n + n_out) * row_bytes, pc, wr[R + r]);
        }
    };
    // Half `half` of the group's activation chunk for step st: 2*M wave-wide copies of 64
    // float4; the group's two waves take every other one.  Copy q covers float4
    // [64q, 64q + 64) of the buffer = (m = q/2, c = 4(q%2) + lane/16, j = lane%16), i.e.
    // inputs 64*pair + 32*half + 4c .. + 3.
    auto stage_x = [&](int st, int half, float4* buf) __attribute__((always_inline)) {
        const int c_lo = lane >> 4;
        int pc = 16 * chunk_of(st) + j;
        pc = pc < P ? pc : P - 1;
#pragma unroll
        for (int qq = 0; qq < M; ++qq) {
            const int q = 2 * qq + (wv & 1);
            const int m = q >> 1;
            const int c = 4 * (q & 1) + c_lo;
            const float* src = x + (size_t)m * ldx + 64 * (size_t)pc + 32 * half + 4 * c;
            lds_copy16(src, buf + 64 * q);
        }
    };
    constexpr int kWLoads = Fmt::kLoads * RR;  // loads per weight step

    float acc[RR][M];
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    // Quant dwords 8*HALF .. 8*HALF + 7 of the lane's pair against the half chunk in xs.
    auto compute = [&](auto half, int st, const uint32_t(&wc)[RR][Fmt::kDwords], const float4* xs)
                       __attribute__((always_inline)) {
        constexpr int HALF = decltype(half)::value;
        const int ch = h + 2 * st;
        if (ch < nch && 16 * ch + j < P) {
            if constexpr (std::is_same<Fmt, FmtQ8_0>::value) {
                // Q8_0: per block t = sum q*x (the quants exact in float32), then
                // acc = fma(d, t, acc); d is the lane's own (its pair's block HALF)
                float t[RR][M];
#pragma unroll
                for (int r = 0; r < RR; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) t[r][m] = 0.0f;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    float wq[RR][4];
#pragma unroll
                    for (int r = 0; r < RR; ++r) q8_quants<HALF>(wc[r], cc, wq[r]);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float4 xv = xs[(m * 8 + cc) * 16 + j];
#pragma unroll
                        for (int r = 0; r < RR; ++r) {
                            t[r][m] = __builtin_fmaf(wq[r][0], xv.x, t[r][m]);
                            t[r][m] = __builtin_fmaf(wq[r][1], xv.y, t[r][m]);
                            t[r][m] = __builtin_fmaf(wq[r][2], xv.z, t[r][m]);
                            t[r][m] = __builtin_fmaf(wq[r][3], xv.w, t[r][m]);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < RR; ++r) {
                    const float d = HALF == 0 ? half_lo(wc[r][0]) : half_hi(wc[r][8]);
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(d, t[r][m], acc[r][m]);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    float wf[RR][4];
#pragma unroll
                    for (int r = 0; r < RR; ++r) Fmt::template weights<HALF>(wc[r], cc, wf[r], 16 * ch + j);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float4 xv = xs[(m * 8 + cc) * 16 + j];
#pragma unroll
                        for (int r = 0; r < RR; ++r) {
                            acc[r][m] = __builtin_fmaf(wf[r][0], xv.x, acc[r][m]);
                            acc[r][m] = __builtin_fmaf(wf[r][1], xv.y, acc[r][m]);
                            acc[r][m] = __builtin_fmaf(wf[r][2], xv.z, acc[r][m]);
                            acc[r][m] = __builtin_fmaf(wf[r][3], xv.w, acc[r][m]);
                        }
                    }
                }
            }
        }
    };
    // Tile i done: butterfly over the 16 lanes, group 1 hands its sums to group 0
    // through LDS (lane j == 0 of each row writes), group 0 adds and stores.
    auto finish_tile = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
        }
        if (h == 1 && j == 0) {
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) part[(slot * RR + r) * M + m] = acc[r][m];
        }
        __syncthreads();
        if (h == 0) {
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] += part[(slot * RR + r) * M + m];
            // every lane of the 16 holds the same bits: all store
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = out_row(i, r);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if constexpr (SILU)
                        y[(size_t)m * ldy + n] = silu_mul(acc[r][m], acc[R + r][m]);
                    else
                        y[(size_t)m * ldy + n] = acc[r][m];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    };

    uint32_t wc[RR][Fmt::kDwords], wn[RR][Fmt::kDwords];
    stage_x(0, 0, xa[h]);
    load_w(0, 0, wc);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay above the wait
    wait_vmcnt<0>();
    __syncthreads();
    // Item (tile i, step st), half 0: copy half 1 into xb and load the next item's
    // weights into wn while multiplying half 0 (xa); wait for the copy only (the weights
    // may stay in flight).  Half 1: copy the next item's half 0 into xa while multiplying
    // half 1 (xb); finish the tile after its last step; wait for everything, wc = wn.  A
    // barrier ends each half.  The part array of finish_tile is not touched by the copies.
    int i = 0, st = 0;
    for (int it = 0; it < items; ++it) {
        const bool more = it + 1 < items;
        const bool last_step = st + 1 == steps;
        const int ni = last_step ? i + 1 : i;
        const int nst = last_step ? 0 : st + 1;
        stage_x(st, 1, xb[h]);
        if (more) load_w(ni, nst, wn);
        __builtin_amdgcn_sched_barrier(0);
        compute(std::integral_constant<int, 0>{}, st, wc, xa[h]);
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
            wait_vmcnt<kWLoads>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        if (more) stage_x(nst, 0, xa[h]);
        __builtin_amdgcn_sched_barrier(0);
        compute(std::integral_constant<int, 1>{}, st, wc, xb[h]);
        if (last_step) finish_tile(i);
        if (more) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<0>();
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int q = 0; q < Fmt::kDwords; ++q) wc[r][q] = wn[r][q];
            __syncthreads();
        }
        i = ni;
        st = nst;
    }
}

// The rows kernel's arithmetic on the matrix cores.  v_mfma_f32_4x4x1_16b_f32 computes,
// in each of its 16 blocks, a 4 x 4 outer product added to a 4 x 4 accumulator with one
// rounding per element (a fused multiply-add, checked against fmaf on the device), and it
// runs at twice the non-packed float32 VALU rate.  Block b stands for lane j = b of the
// float32 rows kernel: its four A values are the weights of four row slots, its four B
// values one input of four activation rows, so that one instruction performs, for 16
// pairs at once, the fma that 16 rows kernel lanes would do for 4 rows x 4 activation
// rows.  The instruction stream follows the rows kernel's order exactly (per chain:
// chunks of the group in increasing order, the pair's inputs in increasing order; then the
// xor butterfly over the 16 blocks and group 0 + group 1), so every output is
// bit-identical to the rows kernel's.  A block whose pair lies past the row multiplies
// zero by zero: its accumulator, which can never hold -0 (it starts at +0 and every
// fma in round-to-nearest keeps +0 + -0 = +0), is unchanged.
//
// Lane layout: lane l is (b = l / 4, t = l % 4): it supplies the weight of row slot t
// and the input of activation row 4q + t; register i of accumulator (g, q) then holds
// row slot i of weight row group g against activation row 4q + t.  Tiles, groups, the
// activation staging (MT rows, rows past m_rows copy the last one and are not stored) and
// the weight ring are those of gemv_rows_kernel.  Up to 16 activation rows per launch.
template <class Fmt, int MT, int R, bool SILU>
__global__ __launch_bounds__(kRowsThreads) __attribute__((amdgpu_waves_per_eu(MT <= 8 ? 2 : 1, 2))) void gemv_rows_mfma_kernel(
    const uint8_t* __restrict__ w, int n_out, int P, const float* __restrict__ x, int ldx, int m_rows,
    float* __restrict__ y, int ldy) {
    static_assert(MT % 4 == 0 && MT <= 16, "activation rows in groups of four, at most 16");
    constexpr int RR = SILU ? 2 * R : R;  // weight row groups per wave (fused: R gate, R up)
    constexpr int QG = MT / 4;            // activation row groups
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    // activation rows at a stride of 132 float4 (128 + 4 of padding): the four row slots
    // t of a read then fall in different LDS banks
    constexpr int kXm = 132;
    __shared__ float4 xa[2][MT * kXm];
    __shared__ float4 xb[2][MT * kXm];
    __shared__ float part[8 * RR * MT];   // group 1's row sums: [slot][g][m]
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = wv >> 1;                // group
    const int lane = tid & 63;
    const int b = lane >> 2;              // pair within the chunk (the rows kernel's lane j)
    const int t = lane & 3;               // row slot within the wave / activation row in a group
    const int slot = (wv & 1) * 4 + t;    // the lane's weight row slot within the group, 0..7
    const size_t row_bytes = Fmt::row_bytes(P);
    const int nch = (P + 15) >> 4;
    const int steps = (nch + 1) >> 1;
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    const int my_tiles = (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int items = my_tiles * steps;
    __builtin_assume(steps >= 1);
    __builtin_assume(items >= 1);

    // weight row of slot s, row r of the tile's slots in tile i (clamped past the end)
    auto out_row = [&](int i, int s, int r) __attribute__((always_inline)) {
        const int n = ((int)blockIdx.x + i * (int)gridDim.x) * (8 * R) + s * R + r;
        return n < n_out ? n : n_out - 1;
    };
    auto chunk_of = [&](int st) __attribute__((always_inline)) {
        const int ch = h + 2 * st;
        return ch < nch ? ch : nch - 1;
    };
    auto load_w = [&](int i, int st, uint32_t(&wr)[RR][Fmt::kDwords]) __attribute__((always_inline)) {
        const int p = 16 * chunk_of(st) + b;
        const int pc = p < P ? p : P - 1;  // past the row: a pair of the same row (multiplied as zero)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = out_row(i, slot, r);
            Fmt::load(w + (size_t)n * row_bytes, pc, wr[r]);
            if constexpr (SILU) Fmt::load(w + (size_t)(n + n_out) * row_bytes, pc, wr[R + r]);
        }
    };
    // as in gemv_rows_kernel: 2*MT wave-wide copies of 64 float4 per half chunk, layout
    // [m][c][j] (rows kXm float4 apart); activation rows past m_rows repeat the last row
    auto stage_x = [&](int st, int half, float4* buf) __attribute__((always_inline)) {
        const int c_lo = lane >> 4;
        int pc = 16 * chunk_of(st) + (lane & 15);
        pc = pc < P ? pc : P - 1;
#pragma unroll
        for (int qq = 0; qq < MT; ++qq) {
            const int q = 2 * qq + (wv & 1);
            int m = q >> 1;
            m = m < m_rows ? m : m_rows - 1;
            const int c = 4 * (q & 1) + c_lo;
            const float* src = x + (size_t)m * ldx + 64 * (size_t)pc + 32 * half + 4 * c;
            lds_copy16(src, buf + (q >> 1) * kXm + 64 * (q & 1));
        }
    };
    constexpr int kWLoads = Fmt::kLoads * RR;

    f32x4 acc[RR][QG];
#pragma unroll
    for (int g = 0; g < RR; ++g)
#pragma unroll
        for (int q = 0; q < QG; ++q) acc[g][q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](auto half, int st, const uint32_t(&wc)[RR][Fmt::kDwords], const float4* xs)
                       __attribute__((always_inline)) {
        constexpr int HALF = decltype(half)::value;
        const int ch = h + 2 * st;
        // a chunk past the row's end (partial: some pairs missing) masks its dead pairs.
        // Per quant dword: the activations of the 4 inputs and the 4 weights of every row
        // group as one batch, then all the MFMAs that use them back to back (the fp32
        // matrix-core instructions and VALU work do not overlap, and alternating them
        // costs cycles); every accumulator still sees its inputs in increasing order.
        auto body = [&](auto partial) __attribute__((always_inline)) {
            constexpr bool PARTIAL = decltype(partial)::value;
            const bool live = 16 * ch + b < P;
            // Q8_0: per block t = sum q*x on the matrix cores (the quants exact in float32),
            // then acc = fma(d, t, acc), as the rows kernel; other formats: the exact weights,
            // one fma per weight.  Either way register e holds weight row slot e, whose
            // block scale lane 4b + e holds (its own row).
            constexpr bool kBlockScale = std::is_same<Fmt, FmtQ8_0>::value;
            f32x4 blk[RR][QG];
            if constexpr (kBlockScale) {
#pragma unroll
                for (int g = 0; g < RR; ++g)
#pragma unroll
                    for (int q = 0; q < QG; ++q) blk[g][q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                float4 xv[QG];
#pragma unroll
                for (int q = 0; q < QG; ++q) {
                    xv[q] = xs[(4 * q + t) * kXm + cc * 16 + b];
                    if constexpr (PARTIAL) {
                        if (!live) xv[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    }
                }
                float wf[RR][4];
#pragma unroll
                for (int g = 0; g < RR; ++g) {
                    if constexpr (kBlockScale)
                        q8_quants<HALF>(wc[g], cc, wf[g]);
                    else
                        Fmt::template weights<HALF>(wc[g], cc, wf[g], 16 * ch + b);
                    if constexpr (PARTIAL) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) wf[g][e] = live ? wf[g][e] : 0.0f;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < RR; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int q = 0; q < QG; ++q) {
                            const float xe = e == 0 ? xv[q].x : e == 1 ? xv[q].y : e == 2 ? xv[q].z : xv[q].w;
                            if constexpr (kBlockScale)
                                blk[g][q] = __builtin_amdgcn_mfma_f32_4x4x1f32(wf[g][e], xe, blk[g][q], 0, 0, 0);
                            else
                                acc[g][q] = __builtin_amdgcn_mfma_f32_4x4x1f32(wf[g][e], xe, acc[g][q], 0, 0, 0);
                        }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (kBlockScale) {
#pragma unroll
                for (int g = 0; g < RR; ++g) {
                    const float dl = HALF == 0 ? half_lo(wc[g][0]) : half_hi(wc[g][8]);
                    float dr[4];
                    static_for<4>([&](auto ec) __attribute__((always_inline)) {  // quad_perm [e, e, e, e]
                        constexpr int e = decltype(ec)::value;
                        dr[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dl), 0x55 * e, 0xF, 0xF, false));
                    });
#pragma unroll
                    for (int q = 0; q < QG; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[g][q][e] = __builtin_fmaf(dr[e], blk[g][q][e], acc[g][q][e]);
                }
            }
        };
        if (ch < nch) {  // wave-uniform
            if (16 * ch + 16 <= P)
                body(std::false_type{});
            else
                body(std::true_type{});
        }
    };
    // Tile i done: butterfly over the 16 blocks (lane offsets 32, 16, 8, 4 for the rows
    // kernel's 8, 4, 2, 1), group 1's sums to group 0 through LDS, group 0 adds and stores
    // (lane (b, t) with b < 4 stores slot b of activation row 4q + t).
    auto finish_tile = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int off = 32; off >= 4; off >>= 1) {
#pragma unroll
            for (int g = 0; g < RR; ++g)
#pragma unroll
                for (int q = 0; q < QG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[g][q][e] += __shfl_xor(acc[g][q][e], off, 64);
        }
        if (h == 1 && b == 0) {
#pragma unroll
            for (int g = 0; g < RR; ++g)
#pragma unroll
                for (int q = 0; q < QG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) part[(((wv & 1) * 4 + e) * RR + g) * MT + 4 * q + t] = acc[g][q][e];
        }
        __syncthreads();
        if (h == 0 && b < 4) {
#pragma unroll
            for (int g = 0; g < RR; ++g)
#pragma unroll
                for (int q = 0; q < QG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[g][q][e] += part[(((wv & 1) * 4 + e) * RR + g) * MT + 4 * q + t];
            const int s = (wv & 1) * 4 + b;  // the slot this lane stores
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = out_row(i, s, r);
#pragma unroll
                for (int q = 0; q < QG; ++q) {
                    const int m = 4 * q + t;
                    float v = acc[r][q][0];
#pragma unroll
                    for (int e = 1; e < 4; ++e) v = b == e ? acc[r][q][e] : v;
                    if constexpr (SILU) {
                        float u = acc[R + r][q][0];
#pragma unroll
                        for (int e = 1; e < 4; ++e) u = b == e ? acc[R + r][q][e] : u;
                        v = silu_mul(v, u);
                    }
                    if (m < m_rows) y[(size_t)m * ldy + n] = v;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < RR; ++g)
#pragma unroll
            for (int q = 0; q < QG; ++q) acc[g][q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    };

    uint32_t wc[RR][Fmt::kDwords], wn[RR][Fmt::kDwords];
    stage_x(0, 0, xa[h]);
    load_w(0, 0, wc);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
    int i = 0, st = 0;
    for (int it = 0; it < items; ++it) {
        const bool more = it + 1 < items;
        const bool last_step = st + 1 == steps;
        const int ni = last_step ? i + 1 : i;
        const int nst = last_step ? 0 : st + 1;
        stage_x(st, 1, xb[h]);
        if (more) load_w(ni, nst, wn);
        __builtin_amdgcn_sched_barrier(0);
        compute(std::integral_constant<int, 0>{}, st, wc, xa[h]);
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
            wait_vmcnt<kWLoads>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        if (more) stage_x(nst, 0, xa[h]);
        __builtin_amdgcn_sched_barrier(0);
        compute(std::integral_constant<int, 1>{}, st, wc, xb[h]);
        if (last_step) finish_tile(i);
        if (more) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<0>();
#pragma unroll
            for (int g = 0; g < RR; ++g)
#pragma unroll
                for (int q = 0; q < Fmt::kDwords; ++q) wc[g][q] = wn[g][q];
            __syncthreads();
        }
        i = ni;
        st = nst;
    }
}

// Several activation rows with K <= 4096, streamed (2..16 rows per launch).  One wave
// per chunk of 16 pairs (up to four waves), each holding its lanes' activations for the
// whole call in registers: lane (b, t) keeps pair 16w + b of activation rows t, 4 + t, ...
// An item is a group of 4 weight rows (fused: 4 gate rows and their 4 up rows); each wave
// copies its chunk of the item's rows (4 x 1088 bytes per weight row group) into its own
// LDS ring with coalesced direct copies, D items ahead, reads its pair, and runs the
// per-block arithmetic of the one-row kernel on the fp32 matrix cores: per Q8_0 block
// t = sum q*x as a chain of v_mfma_f32_4x4x1_16b_f32 (the quants exact in float32, one
// rounding per fma; block b of the instruction for pair b, four weight rows against four
// activation rows, one instruction per input), then acc = fma(d, t, acc) on the VALU
// (block 0, then block 1 of the pair).  Per output: that chain per pair, a fixed
// lane-exchange sum over the 16 pairs of the chunk (lane swaps and row rotations, no
// LDS), then the chunks' sums added in chunk order.  The
// matrix-core fp32 instructions and the VALU dequantization do not overlap on this chip,
// so the per-item exchange and address work is kept to a few instructions; the copies of
// a row group inside the matrix use one scalar base and fixed lane offsets.  The order
// depends only on K, so every row of a call
// with 2..255 rows is bit-identical whatever the other rows are; it is the class of these
// K (the float32 rows kernel serves larger K).  Each wave leaves its chunk sums of every
// item in LDS and runs on without waiting for the others; one barrier at the end, then
// the block adds the chunks and stores (so no store is counted by the copies' vmcnt
// waits).
constexpr int kStreamMaxChunks = 4;

// Sum of v[0..3] over the 16 lane groups of four (lane >> 2), each lane keeping one of the
// four values: across the wave halves (v[0] with v[2], v[1] with v[3]: each half keeps one
// of each pair), across row pairs (keeping one of the two), then within each row of 16
// lanes (rotations by 8 and 4).  Which value a lane ends with follows from the exchanges
// alone; reduce_scatter_tag runs them on the value indices.  Eight VALU instructions, no
// LDS; the order of the additions is fixed.
__device__ __forceinline__ float reduce_scatter_pairs(float v0, float v1, float v2, float v3) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
    const float u0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
    const float u1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
    const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(u0), __float_as_uint(u1), false, false);
    float z = __uint_as_float(s2[0]) + __uint_as_float(s2[1]);
    z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0x128, 0xF, 0xF, false));  // row_ror:8
    z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0x124, 0xF, 0xF, false));  // row_ror:4
    return z;
}
__device__ __forceinline__ float reduce_scatter_tag(const float (&v)[4]) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
    const auto s2 = __builtin_amdgcn_permlane16_swap(s0[0], s1[0], false, false);
    return __uint_as_float(s2[0]);
}

template <int MT, bool SILU, int D>
__global__ __launch_bounds__(64 * kStreamMaxChunks) __attribute__((amdgpu_waves_per_eu(MT <= 8 ? 2 : 1, 2)))
void gemv_rows_stream_kernel(const uint8_t* __restrict__ w, int n_out, int P, const float* __restrict__ x, int ldx,
                             int m_rows, float* __restrict__ y, int ldy) {
    static_assert(MT % 4 == 0 && MT <= 16, "activation rows in groups of four, at most 16");
    constexpr int QG = MT / 4;
    constexpr int RG = SILU ? 2 : 1;  // weight row groups per item
    static_assert(D * 5 * RG < 64, "copies in flight must fit the vmcnt counter");
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    extern __shared__ float4 smem4[];
    uint8_t* smem = reinterpret_cast<uint8_t*>(smem4);
    const int nc = (int)(blockDim.x >> 6);  // waves = chunks of the row
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & 63);
    const int b = lane >> 2, t = lane & 3;
    const int p = 16 * wv + b;
    const bool live = p < P;
    const int pc = live ? p : P - 1;
    const size_t row_bytes = (size_t)P * 68;
    const int seg = ((P - 16 * wv) < 16 ? (P - 16 * wv) : 16) * 68;  // bytes of the wave's chunk per row
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(smem + (size_t)wv * (D * RG * kLdsItemBytes)));
    const uint32_t* ring32 = reinterpret_cast<const uint32_t*>(smem + (size_t)wv * (D * RG * kLdsItemBytes));
    constexpr int kPart = RG * 4 * MT;  // partial sums of a wave per item
    float* part = reinterpret_cast<float*>(smem + (size_t)nc * D * RG * kLdsItemBytes);  // [items][nc][kPart]
    const int row_groups = (n_out + 3) >> 2;
    const int n_items = (row_groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;

    // the lane's activations (rows past m_rows repeat the last one; a pair past the row: zeros)
    float4 xr[QG][16];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        const int m = 4 * q + t < m_rows ? 4 * q + t : m_rows - 1;
        const float4* src = reinterpret_cast<const float4*>(x + (size_t)m * ldx + 64 * (size_t)pc);
#pragma unroll
        for (int c = 0; c < 16; ++c) xr[q][c] = src[c];
    }
    // the compiler's own wait (vmcnt 0, the other counters untouched): its wait insertion
    // then knows the activations have landed and puts no vmcnt wait into the loop, where
    // one would also drain the next item's copies
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (!live) {
#pragma unroll
        for (int q = 0; q < QG; ++q)
#pragma unroll
            for (int c = 0; c < 16; ++c) xr[q][c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }

    // the weight row (0..3) whose pair sum reduce_scatter_pairs leaves in this lane: the
    // same exchanges applied once to the row numbers themselves
    const int row_of_lane = [&] {
        const float tags[4] = {0.0f, 1.0f, 2.0f, 3.0f};
        return (int)reduce_scatter_tag(tags);
    }();
    const bool own = ((lane >> 2) & 3) == 0;  // one lane per (row, activation row) writes

    // item i's rows of the wave's chunk into ring slot `slot`: 5 * RG vmcnt events.  LDS byte
    // o of a row group's 4352 is byte o % 1088 of row o / 1088's chunk.  A short last chunk
    // (a multiple of 4 pairs: seg a multiple of 272 bytes) repeats its own pairs past its
    // end (byte o % 1088 % seg), so a lane past the row reads a whole real pair of its row
    // (finite scale; multiplied by zero activations); rows past the matrix: the last row.
    int crow[5], coff[5];  // the lane's row and byte of each copy (the same for every item)
    uint32_t cbyte[5];     // ... as one offset from the row group's first row
#pragma unroll
    for (int c = 0; c < 5; ++c) {
        const int o = c < 4 ? 1024 * c + 16 * lane : 4096 + 4 * lane;
        crow[c] = o / 1088;
        const int off = o - 1088 * crow[c];
        coff[c] = 1088 * wv + (off < seg ? off : off % seg);
        cbyte[c] = (uint32_t)(crow[c] * row_bytes) + (uint32_t)coff[c];
    }
    auto issue = [&](int i, int slot) __attribute__((always_inline)) {
        const int rg = (int)blockIdx.x + i * (int)gridDim.x;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const uint32_t dst = ring_lds + (uint32_t)((slot * RG + r) * kLdsItemBytes);
            if (4 * rg + 3 < n_out) {  // all four rows in the matrix: one base, lane offsets
                lds_copy_4352_gather_s<true>(w + (size_t)(4 * rg + r * n_out) * row_bytes, cbyte, dst);
            } else {
                const uint8_t* src[5];
#pragma unroll
                for (int c = 0; c < 5; ++c) {
                    int n = 4 * rg + crow[c];
                    n = n < n_out ? n : n_out - 1;
                    src[c] = w + (size_t)(n + r * n_out) * row_bytes + coff[c];
                }
                lds_copy_4352_gather<true>(src, dst);
            }
        }
    };

    const int n_pro = n_items < D ? n_items : D;
    static_for<D>([&](auto sc) __attribute__((always_inline)) {
        constexpr int s0 = decltype(sc)::value;
        if (s0 < n_pro) issue(s0, s0);
    });
    for (int i = 0; i < n_items; ++i) {
        const int slot = i % D;
        // items i+1 .. min(i+D-1, n_items-1) may stay in flight
        const int rem = n_items - 1 - i;
        if (rem >= D - 1) {
            wait_vmcnt_mem<(D - 1) * 5 * RG>();
        } else {
            static_for<D - 1>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                if (rem == k) wait_vmcnt_mem<k * 5 * RG>();
            });
        }
        uint32_t wr[RG][17];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int k = 0; k < 17; ++k) wr[r][k] = ring32[(slot * RG + r) * (kLdsItemBytes / 4) + t * 272 + b * 17 + k];
        wait_lgkmcnt_mem<0>();
        if (i + D < n_items) issue(i + D, slot);  // refill the slot just read

        f32x4 acc[RG][QG];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int q = 0; q < QG; ++q) acc[r][q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        // per block (half of the pair): t = sum q*x over its 32 inputs on the matrix cores
        // (the quants exact in float32), then acc = fma(d, t, acc) on the VALU
        static_for<2>([&](auto hc) __attribute__((always_inline)) {
            constexpr int HALF = decltype(hc)::value;
            // register e holds weight row e, whose scale lane 4b + e holds (its own row)
            float dr[RG][4];
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const float dl = HALF == 0 ? half_lo(wr[r][0]) : half_hi(wr[r][8]);
                static_for<4>([&](auto ec) __attribute__((always_inline)) {  // quad_perm [e, e, e, e]
                    constexpr int e = decltype(ec)::value;
                    dr[r][e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dl), 0x55 * e, 0xF, 0xF, false));
                });
            }
            f32x4 blk[RG][QG];
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int q = 0; q < QG; ++q) blk[r][q] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                // the step's quants as one batch of VALU work, then its MFMAs back to back:
                // switching between the two costs cycles, so the compiler's interleaving
                // (one weight, then the MFMAs that read it) is held off
                float wq[RG][4];
#pragma unroll
                for (int r = 0; r < RG; ++r) q8_quants<HALF>(wr[r], cc, wq[r]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int r = 0; r < RG; ++r)
#pragma unroll
                        for (int q = 0; q < QG; ++q) {
                            const float4 xv = xr[q][8 * HALF + cc];
                            const float xe = e == 0 ? xv.x : e == 1 ? xv.y : e == 2 ? xv.z : xv.w;
                            blk[r][q] = __builtin_amdgcn_mfma_f32_4x4x1f32(wq[r][e], xe, blk[r][q], 0, 0, 0);
                        }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int q = 0; q < QG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[r][q][e] = __builtin_fmaf(dr[r][e], blk[r][q][e], acc[r][q][e]);
        });
        // register e of (r, q) holds weight row e of group r against activation row 4q + t
        // for pair b; sum over the 16 pairs, scattering the four rows over the lanes
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                const float v = reduce_scatter_pairs(acc[r][q][0], acc[r][q][1], acc[r][q][2], acc[r][q][3]);
                if (own) part[(i * nc + wv) * kPart + (r * 4 + row_of_lane) * MT + 4 * q + t] = v;
            }
    }
    __syncthreads();
    // output (item i, weight row j / MT of its group, activation row j % MT)
    for (int o = (int)threadIdx.x; o < n_items * 4 * MT; o += (int)blockDim.x) {
        const int i = o / (4 * MT), j = o - i * (4 * MT);
        const float* pi = part + (size_t)i * nc * kPart + j;
        float s = pi[0];
        for (int c = 1; c < nc; ++c) s += pi[c * kPart];
        if constexpr (SILU) {
            float u = pi[4 * MT];
            for (int c = 1; c < nc; ++c) u += pi[c * kPart + 4 * MT];
            s = silu_mul(s, u);
        }
        const int n = 4 * ((int)blockIdx.x + i * (int)gridDim.x) + j / MT;
        const int m = j % MT;
        if (n < n_out && m < m_rows) y[(size_t)m * ldy + n] = s;
    }
}

namespace {

template <class Fmt, int R, int NR, int D, int NW, bool NT = false>
hipError_t launch_one_row(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x,
                          float* y, hipStream_t stream) {
    auto kernel = gemv_one_row_kernel<Fmt, R, NR, D, NW, NT>;
    const size_t lds = (size_t)P * kXRow + (size_t)NW * D * R * kLdsItemBytes;
    // Once per device: allow the largest dynamic LDS this instance uses (rows of up to
    // 64*NR pairs), above the default limit.  Resident blocks per CU depend on the LDS
    // size: kept for the last few sizes seen (a model alternates a handful of shapes).
    constexpr size_t kLdsMax = (size_t)64 * NR * kXRow + (size_t)NW * D * R * kLdsItemBytes;
    struct Occ { int dev, lds, per_cu; };
    static thread_local int attr_dev = -1;
    static thread_local Occ occ[4] = {{-1, -1, 1}, {-1, -1, 1}, {-1, -1, 1}, {-1, -1, 1}};
    static thread_local int occ_next = 0;
    if (attr_dev != dev.device) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
        if (e != hipSuccess) return e;
        attr_dev = dev.device;
    }
    int per_cu = 0;
    for (const Occ& o : occ)
        if (o.dev == dev.device && o.lds == (int)lds) per_cu = o.per_cu;
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * NW, lds) != hipSuccess || per_cu < 1)
            per_cu = 1;
        occ[occ_next] = {dev.device, (int)lds, per_cu};
        occ_next = (occ_next + 1) & 3;
    }
    // The wide form (8 waves, one slot) runs one block per CU even where more would fit:
    // each wave then streams several row groups instead of one, and the kernel spends
    // less of its time in the ramp and tail of a single round (8B QKV 6144x4096 at one
    // row: 7.66 -> 7.04 us; the fused gate_up and the three-round down unchanged).
    if (D == 1 && NW == 8) per_cu = 1;
    const int G = 64 >> log2S;
    const int total = ((n_out + G - 1) / G) * NR;
    // items per wave: enough to cover the work with the waves that fit at once, a
    // multiple of the rounds per row group
    const int resident = dev.cu_count * per_cu * NW;
    int ipw = (total + resident - 1) / resident;
    ipw = ((ipw + NR - 1) / NR) * NR;
    const int waves = (total + ipw - 1) / ipw;
    const int blocks = (waves + NW - 1) / NW;
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(64 * NW), lds, stream, w, n_out, P, log2S, x, y, ipw);
    return hipGetLastError();
}

// One activation row with K <= 16384 (at most 4 rounds of 64 pairs per row; activations
// in registers).  With at least two items per wave for 8-wave blocks (the 8B shapes):
// 8 waves and one slot each (the slot is refilled as soon as it is read, so one item is in
// flight per wave while another is multiplied), weight copies with the non-temporal hint
// (2-6% faster there).  Smaller matrices (or 4 rounds, where the activations need more
// registers): 4-wave blocks, spread over more CUs, two slots each, plain copies (the hint
// measured slower on the Qwen3-0.6B shapes).  Measured on the Qwen3 shapes.
template <class Fmt, int R>
bool try_one_row(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, float* y,
                 hipStream_t stream, hipError_t* err) {
    const int S = 1 << log2S;
    const int NR = (P + S - 1) / S;
    const int64_t items = (int64_t)((n_out + (64 >> log2S) - 1) / (64 >> log2S)) * NR;
    const bool wide = items >= (int64_t)16 * dev.cu_count;
    switch (NR) {
        case 1:
            *err = wide ? launch_one_row<Fmt, R, 1, 1, 8, true>(dev, w, n_out, P, log2S, x, y, stream)
                        : launch_one_row<Fmt, R, 1, 2, 4>(dev, w, n_out, P, log2S, x, y, stream);
            return true;
        case 2:
            *err = wide ? launch_one_row<Fmt, R, 2, 1, 8, true>(dev, w, n_out, P, log2S, x, y, stream)
                        : launch_one_row<Fmt, R, 2, 2, 4>(dev, w, n_out, P, log2S, x, y, stream);
            return true;
        case 3:
            *err = wide && R == 1 ? launch_one_row<Fmt, R, 3, 1, 8, true>(dev, w, n_out, P, log2S, x, y, stream)
                                  : launch_one_row<Fmt, R, 3, 2, 4>(dev, w, n_out, P, log2S, x, y, stream);
            return true;
        case 4: *err = launch_one_row<Fmt, R, 4, 2, 4>(dev, w, n_out, P, log2S, x, y, stream); return true;
        default: return false;
    }
}

// Blocks of gemv_rows_kernel<Fmt, M, R, SILU> resident per CU (queried once per kernel).
template <class Fmt, int M, int R, bool SILU>
int rows_per_cu() {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_rows_kernel<Fmt, M, R, SILU>, kRowsThreads, 0) !=
                hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    return per_cu;
}

template <class Fmt, int M, int R, bool SILU>
hipError_t launch_rows_r(const DeviceInfo& dev, int n_out, int P, const uint8_t* w, const float* x, int ldx, float* y,
                         int ldy, hipStream_t stream) {
    // persistent grid: one block per resident slot (at most one per tile); each walks
    // its tiles at a stride of the grid
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    const int64_t slots = (int64_t)dev.cu_count * rows_per_cu<Fmt, M, R, SILU>();
    const int blocks = (int)(tiles < slots ? tiles : slots);
    hipLaunchKernelGGL((gemv_rows_kernel<Fmt, M, R, SILU>), dim3(blocks), dim3(kRowsThreads), 0, stream, w, n_out, P, x,
                       ldx, y, ldy);
    return hipGetLastError();
}

// Fraction of a persistent grid's block-steps that do work: tiles spread over `slots`
// blocks, the busiest taking ceil(tiles / slots).
inline double round_fill(int64_t tiles, int64_t slots) {
    const int64_t per = (tiles + slots - 1) / slots;
    const int64_t used = tiles < slots ? tiles : slots;
    return (double)tiles / (double)(per * (used > 0 ? slots : 1));
}

template <class Fmt, int M, bool SILU>
hipError_t launch_rows(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx, float* y,
                       int ldy, hipStream_t stream) {
    // R rows (row pairs) per lane: more rows per lane share each activation read from LDS,
    // fewer spread the tiles more evenly.  Take the largest R within 5% of the best fill;
    // R = 2 already from half the best fill for the fused gate_up (each activation read
    // then feeds four rows) and for Q8_0 with 8 rows, where the activation reads bound the
    // kernel as much as the fmas: measured on the Qwen3-8B and Gemma 4 12B shapes (fused
    // gate_up 24576x4096, M = 8: 52.2 -> 47.3 us; down 4096x12288, M = 8: 32.9 -> 30.6 us;
    // plain rows with fewer activation rows, and Q4_0 down, stay faster with R = 1).
    // A format's kMaxR bounds the weight rows a lane holds (fused: 2R), so that its
    // register ring fits two waves per SIMD.
    constexpr int kRows = SILU ? 2 : 1;
    constexpr bool kTwo = 2 * kRows <= Fmt::kMaxR, kFour = !SILU && 4 <= Fmt::kMaxR;
    const int64_t cus = dev.cu_count;
    const double f1 = round_fill((n_out + 7) / 8, cus * rows_per_cu<Fmt, M, 1, SILU>());
    double f2 = 0.0, f4 = 0.0;
    if constexpr (kTwo) f2 = round_fill((n_out + 15) / 16, cus * rows_per_cu<Fmt, M, 2, SILU>());
    if constexpr (kFour) f4 = round_fill((n_out + 31) / 32, cus * rows_per_cu<Fmt, M, 4, SILU>());
    const double best = f1 > f2 ? (f1 > f4 ? f1 : f4) : (f2 > f4 ? f2 : f4);
    if constexpr (kFour) {
        if (f4 >= 0.95 * best) return launch_rows_r<Fmt, M, 4, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
    }
    if constexpr (kTwo) {
        constexpr bool kPreferTwo = SILU || (std::is_same<Fmt, FmtQ8_0>::value && M >= 8);
        if (f2 >= (kPreferTwo ? 0.5 : 0.95) * best)
            return launch_rows_r<Fmt, M, 2, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
    }
    return launch_rows_r<Fmt, M, 1, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
}

// Blocks of gemv_rows_mfma_kernel<Fmt, MT, R, SILU> resident per CU (queried once per kernel).
template <class Fmt, int MT, int R, bool SILU>
int rows_mfma_per_cu() {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_rows_mfma_kernel<Fmt, MT, R, SILU>, kRowsThreads,
                                                         0) != hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    return per_cu;
}

template <class Fmt, int MT, int R, bool SILU>
hipError_t launch_rows_mfma_r(const DeviceInfo& dev, int n_out, int P, const uint8_t* w, const float* x, int ldx,
                              int m_rows, float* y, int ldy, hipStream_t stream) {
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    const int64_t slots = (int64_t)dev.cu_count * rows_mfma_per_cu<Fmt, MT, R, SILU>();
    const int blocks = (int)(tiles < slots ? tiles : slots);
    hipLaunchKernelGGL((gemv_rows_mfma_kernel<Fmt, MT, R, SILU>), dim3(blocks), dim3(kRowsThreads), 0, stream, w,
                       n_out, P, x, ldx, m_rows, y, ldy);
    return hipGetLastError();
}

// Rows per lane: one gate/up pair for the fused form, up to two plain rows (the largest
// within 5% of the best fill), so that the kernel keeps two waves per SIMD without spills.
template <class Fmt, int MT, bool SILU>
hipError_t launch_rows_mfma(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx,
                            int m_rows, float* y, int ldy, hipStream_t stream) {
    if constexpr (!SILU) {
        const int64_t cus = dev.cu_count;
        const double f1 = round_fill((n_out + 7) / 8, cus * rows_mfma_per_cu<Fmt, MT, 1, SILU>());
        const double f2 = round_fill((n_out + 15) / 16, cus * rows_mfma_per_cu<Fmt, MT, 2, SILU>());
        if (f2 >= 0.95 * f1)
            return launch_rows_mfma_r<Fmt, MT, 2, SILU>(dev, n_out, P, w, x, ldx, m_rows, y, ldy, stream);
    }
    return launch_rows_mfma_r<Fmt, MT, 1, SILU>(dev, n_out, P, w, x, ldx, m_rows, y, ldy, stream);
}

// 9..16 activation rows on the matrix-core form, padded to 12 or 16.
template <class Fmt, bool SILU>
hipError_t launch_rows_mfma_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx,
                              int m, float* y, int ldy, hipStream_t stream) {
    if (m <= 12) return launch_rows_mfma<Fmt, 12, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
    return launch_rows_mfma<Fmt, 16, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
}

// Streaming rows form (K <= 4096): dynamic LDS = the rings and the chunk sums of every
// item of the block.
constexpr int kStreamSlots = 2;
inline size_t stream_lds_bytes(int n_out, int P, int mt, bool silu, int64_t grid) {
    const int nc = (P + 15) >> 4, rg = silu ? 2 : 1;
    const int64_t row_groups = (n_out + 3) >> 2;
    const int64_t items = (row_groups + grid - 1) / grid;
    return (size_t)nc * kStreamSlots * rg * kLdsItemBytes + (size_t)(items * nc * rg * 4 * mt) * 4;
}
constexpr size_t kStreamLdsMax = 160 * 1024;

// The form applies to one call when K <= 4096 and, for 16 activation rows on a grid of one
// block per CU, its LDS fits (the chunk sums of every item of a block wait there).
inline bool stream_fits(const DeviceInfo& dev, int64_t n_out, int P, bool silu) {
    if (P > 16 * kStreamMaxChunks || n_out > (int64_t)1 << 28) return false;
    return stream_lds_bytes((int)n_out, P, 16, silu, dev.cu_count) <= kStreamLdsMax;
}

template <int MT, bool SILU>
hipError_t launch_rows_stream_mt(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx,
                                 int m_rows, float* y, int ldy, hipStream_t stream) {
    auto kernel = gemv_rows_stream_kernel<MT, SILU, kStreamSlots>;
    const int threads = 64 * ((P + 15) >> 4);
    const int64_t row_groups = (n_out + 3) >> 2;
    static thread_local int attr_dev = -1;
    if (attr_dev != dev.device) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax);
        if (e != hipSuccess) return e;
        attr_dev = dev.device;
    }
    // One block per CU: measured faster than two wherever two fit (8B fused gate_up at 8 rows
    // 36.8 -> 33.0 us, QKV at 8 rows 16.6 -> 13.7 us): each CU loads the call's activations
    // once, and each block has twice the items over which to spread its start.
    const int grid = (int)(row_groups < dev.cu_count ? row_groups : dev.cu_count);
    const size_t lds = stream_lds_bytes(n_out, P, MT, SILU, grid);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, stream, w, n_out, P, x, ldx, m_rows, y, ldy);
    return hipGetLastError();
}

template <bool SILU>
hipError_t launch_rows_stream(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx,
                              int m, float* y, int ldy, hipStream_t stream) {
    if (m <= 4) return launch_rows_stream_mt<4, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
    if (m <= 8) return launch_rows_stream_mt<8, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
    if (m <= 12) return launch_rows_stream_mt<12, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
    return launch_rows_stream_mt<16, SILU>(dev, w, n_out, P, x, ldx, m, y, ldy, stream);
}

template <int M, int R>
hipError_t launch_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                    float* y, int ldy, hipStream_t stream) {
    return launch_rows<FmtQ8_0, M, R == 2>(dev, w, n_out, P, x, ldx, y, ldy, stream);
}

template <int R>
hipError_t launch_r(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                    int m, float* y, int ldy, hipStream_t stream) {
    switch (m) {
#define Q8_CASE(MM) \
    case MM: return launch_m<MM, R>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
        Q8_CASE(1) Q8_CASE(2) Q8_CASE(3) Q8_CASE(4) Q8_CASE(5) Q8_CASE(6) Q8_CASE(7) Q8_CASE(8)
#undef Q8_CASE
        default: return hipErrorInvalidValue;
    }
}

template <bool SILU>
hipError_t launch_q4_0_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx, int m,
                         float* y, int ldy, hipStream_t stream) {
    switch (m) {
#define Q4_CASE(MM) \
    case MM: return launch_rows<FmtQ4_0, MM, SILU>(dev, w, n_out, P, x, ldx, y, ldy, stream);
        Q4_CASE(1) Q4_CASE(2) Q4_CASE(3) Q4_CASE(4) Q4_CASE(5) Q4_CASE(6) Q4_CASE(7) Q4_CASE(8)
#undef Q4_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_q4_0(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    // One row, K <= 4096 (one round of pairs) and at least 16 row groups per CU: the
    // LDS-streaming one-row kernel (Gemma 4 12B gate_up 30720x3840: 23.3 -> 19.1 us).  With
    // more rounds (the 3840x15360 down: 13.6 -> 17.1 us) and on small matrices the rows
    // kernel stays faster for Q4_0, whose 36-byte pairs carry half the bytes per item.
    if (m == 1 && P <= 64) {
        const int log2S = slots_log2(P);
        const int64_t groups = (n_out + (64 >> log2S) - 1) / (64 >> log2S);
        if (groups >= (int64_t)16 * dev.cu_count)
            return silu_pairs ? launch_one_row<FmtQ4_0, 2, 1, 1, 8, true>(dev, w, (int)n_out, P, log2S, x, y, stream)
                              : launch_one_row<FmtQ4_0, 1, 1, 1, 8, true>(dev, w, (int)n_out, P, log2S, x, y, stream);
    }
    for (int64_t m0 = 0; m0 < m; m0 += 8) {
        const int mm = (int)((m - m0) < 8 ? (m - m0) : 8);
        const float* xc = x + m0 * ldx;
        float* yc = y + m0 * ldy;
        hipError_t e = silu_pairs ? launch_q4_0_m<true>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream)
                                  : launch_q4_0_m<false>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class Fmt, bool SILU>
hipError_t launch_kq_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const float* x, int ldx, int m,
                       float* y, int ldy, hipStream_t stream) {
    switch (m) {
#define KQ_CASE(MM) \
    case MM: return launch_rows<Fmt, MM, SILU>(dev, w, n_out, P, x, ldx, y, ldy, stream);
        KQ_CASE(1) KQ_CASE(2) KQ_CASE(3) KQ_CASE(4) KQ_CASE(5) KQ_CASE(6) KQ_CASE(7) KQ_CASE(8)
#undef KQ_CASE
        default: return hipErrorInvalidValue;
    }
}

// One activation row of a k-quant matrix runs the one-row kernel for rows of at most three
// rounds of 64 pairs (K <= 12288; fused gate_up: two, K <= 8192, as three spill registers),
// Q6_K for at most two rounds of rows of a multiple of 8 super-blocks (16-byte aligned rows
// for the direct copies).  Its items carry half the bytes of Q8_0's for more VALU work per
// weight (nibble extraction, scale decode), so it is bound by the arithmetic, not by HBM:
// measured on the Qwen3-8B shapes, 8B gate_up 24576x4096 at M = 1: Q4_K 21.1 -> 19.4 us, Q6_K
// 31.5 -> 23.6 us against the rows kernel; down 4096x12288: Q4_K 12.4 -> 11.9 us, Q6_K 15.7 ->
// 17.0 us (so three-round Q6_K rows stay on the rows kernel).
template <class Fmt>
bool kq_one_row(int64_t k, bool silu_pairs) {
    if constexpr (std::is_same<Fmt, FmtQ6_K>::value) return k <= 8192 && k % 2048 == 0;
    return k <= (silu_pairs ? 8192 : 12288);  // three rounds of the fused form spill
}

// GGUF k-quant weights (Q4_K, Q5_K, Q6_K): one row as above, every other row count on the
// float32 rows kernel in 8-row launches.
template <class Fmt>
hipError_t launch_gemv_kq(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                          const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    if (m == 1 && kq_one_row<Fmt>(k, silu_pairs)) {
        hipError_t e = hipSuccess;
        const bool done = silu_pairs
                              ? try_one_row<Fmt, 2>(dev, w, (int)n_out, P, slots_log2(P), x, y, stream, &e)
                              : try_one_row<Fmt, 1>(dev, w, (int)n_out, P, slots_log2(P), x, y, stream, &e);
        if (done) return e;
    }
    for (int64_t m0 = 0; m0 < m; m0 += 8) {
        const int mm = (int)((m - m0) < 8 ? (m - m0) : 8);
        const float* xc = x + m0 * ldx;
        float* yc = y + m0 * ldy;
        hipError_t e = silu_pairs ? launch_kq_m<Fmt, true>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream)
                                  : launch_kq_m<Fmt, false>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_q4_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    return launch_gemv_kq<FmtQ4_K>(dev, w, n_out, k, silu_pairs, x, m, ldx, y, ldy, stream);
}

hipError_t launch_gemv_q6_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    return launch_gemv_kq<FmtQ6_K>(dev, w, n_out, k, silu_pairs, x, m, ldx, y, ldy, stream);
}

hipError_t launch_gemv_q5_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    return launch_gemv_kq<FmtQ5_K>(dev, w, n_out, k, silu_pairs, x, m, ldx, y, ldy, stream);
}

hipError_t launch_gemv_q8(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                          const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    const int log2S = slots_log2(P);
    if (m == 1) {  // one row: the LDS-streaming kernel when K fits it
        hipError_t e;
        if (silu_pairs ? try_one_row<FmtQ8_0, 2>(dev, w, (int)n_out, P, log2S, x, y, stream, &e)
                       : try_one_row<FmtQ8_0, 1>(dev, w, (int)n_out, P, log2S, x, y, stream, &e))
            return e;
    }
    if (m == 1)  // one row with K beyond the one-row kernel: the float32 rows kernel
        return silu_pairs ? launch_r<2>(dev, w, (int)n_out, P, log2S, x, (int)ldx, 1, y, (int)ldy, stream)
                          : launch_r<1>(dev, w, (int)n_out, P, log2S, x, (int)ldx, 1, y, (int)ldy, stream);
    // Several rows with K <= 4096: the streaming form, in launches of up to 16 rows.
    if (stream_fits(dev, n_out, P, silu_pairs)) {
        for (int64_t m0 = 0; m0 < m; m0 += 16) {
            const int mm = (int)((m - m0) < 16 ? (m - m0) : 16);
            hipError_t e = silu_pairs ? launch_rows_stream<true>(dev, w, (int)n_out, P, x + m0 * ldx, (int)ldx, mm,
                                                                 y + m0 * ldy, (int)ldy, stream)
                                      : launch_rows_stream<false>(dev, w, (int)n_out, P, x + m0 * ldx, (int)ldx, mm,
                                                                  y + m0 * ldy, (int)ldy, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // Several rows, in launches of up to 16: 9..16 rows on the matrix-core form (one pass
    // over the weights), up to 8 on the float32 rows kernel, which is faster there; both
    // give the same bits.  Measured on the Qwen3-8B linears at 16 rows (one matrix-core
    // launch against two 8-row launches): QKV 33.3 / 36 us, down 45.9 / 61 us, fused gate_up
    // 90.9 / 89.6 us; at 8 rows the float32 kernel wins (fused gate_up 44.8 / 52.6 us).
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mm = (int)((m - m0) < 16 ? (m - m0) : 16);
        const float* xc = x + m0 * ldx;
        float* yc = y + m0 * ldy;
        hipError_t e;
        if (mm > 8)
            e = silu_pairs
                    ? launch_rows_mfma_m<FmtQ8_0, true>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream)
                    : launch_rows_mfma_m<FmtQ8_0, false>(dev, w, (int)n_out, P, xc, (int)ldx, mm, yc, (int)ldy, stream);
        else
            e = silu_pairs ? launch_r<2>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream)
                           : launch_r<1>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q8k
