// Device building blocks of the Q8_0 x float32 GEMV (gfx950, wave64), shared by the
// dense linears and the grouped MoE expert kernels so that both give the same
// per-row arithmetic.
//
// Work decomposition
//   A "pair" is two consecutive Q8_0 blocks: 64 weights in 68 bytes = 17 dwords.
//   Rows are 16-byte aligned (K % 256 == 0), so every pair starts on a dword
//   boundary and the second block's quants are dword aligned.
//   A row of K weights has P = K/64 pairs.  S lanes share one row ("slots",
//   S = 64 for P >= 64, else the next power of two >= P, at least 4); slot j owns
//   pairs j, j+S, j+2S, ...  A wave covers G = 64/S rows at a time.  Each lane keeps
//   one float32 partial per (row, activation row); the S partials of a row are summed
//   by a fixed xor-butterfly.  A row's result therefore depends only on K, never on
//   how many activation rows share the pass.
//
// Per-output summation order (identical for every number of activation rows):
//   for each of the lane's pairs in increasing order, for each of its two blocks:
//       t = q_0*x_0;  t = fma(q_i, x_i, t) for i = 1..31;   acc = fma(d, t, acc)
//   then the butterfly over the S slots (xor S/2, ..., 1).
//
// Memory: the MoE expert passes (wave_rows in moe.hip) have each lane load its 68-byte
// pair with four 16-byte loads and one dword (load_pair), prefetching the next pair into
// registers while the current one is multiplied.  The dense one-row kernel (gemv_q8.hip)
// instead copies whole row stretches into LDS with coalesced direct copies and reads each
// lane's pair from there; both run mac_pair on the same pairs in the same order.  The int8 ->
// float32 conversion (one v_cvt with a byte select) is done once per weight and shared
// by all activation rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace q8k {

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ float half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
template <int B>
__device__ __forceinline__ float sbyte(uint32_t v) {
    return (float)(int)(int8_t)(v >> (8 * B));
}

// Plain (cached) loads on purpose: a pair shares its first and last cache lines with
// the neighbouring lanes' pairs, and the non-temporal form measured at half the
// bandwidth on gfx950 for this pattern (the shared lines are fetched twice).
__device__ __forceinline__ void load_pair(const uint8_t* p, uint32_t (&w)[17]) {
    const u32x4_a4* v = reinterpret_cast<const u32x4_a4*>(p);
    const u32x4_a4 a = v[0];
    const u32x4_a4 b = v[1];
    const u32x4_a4 c = v[2];
    const u32x4_a4 d = v[3];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    w[8] = c.x; w[9] = c.y; w[10] = c.z; w[11] = c.w;
    w[12] = d.x; w[13] = d.y; w[14] = d.z; w[15] = d.w;
    w[16] = *reinterpret_cast<const uint32_t*>(p + 64);
}

// acc[r][m] += one pair (two blocks) of row r against activation rows 0..M-1.
template <int M, int R, class X>
__device__ __forceinline__ void mac_pair(const uint32_t (&w)[R][17], const X& xs, int p, float (&acc)[R][M]) {
    float t[R][M];
    // block 0: scale = low half of dword 0, quants = bytes 2..33 of the pair
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float q[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            q[r][0] = sbyte<2>(w[r][c]);
            q[r][1] = sbyte<3>(w[r][c]);
            q[r][2] = sbyte<0>(w[r][c + 1]);
            q[r][3] = sbyte<1>(w[r][c + 1]);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 xv = xs.get(m, p, c);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s = (c == 0) ? q[r][0] * xv.x : __builtin_fmaf(q[r][0], xv.x, t[r][m]);
                s = __builtin_fmaf(q[r][1], xv.y, s);
                s = __builtin_fmaf(q[r][2], xv.z, s);
                t[r][m] = __builtin_fmaf(q[r][3], xv.w, s);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float d0 = half_lo(w[r][0]);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(d0, t[r][m], acc[r][m]);
    }
    // block 1: scale = high half of dword 8, quants = dwords 9..16
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float q[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t v = w[r][9 + c];
            q[r][0] = sbyte<0>(v);
            q[r][1] = sbyte<1>(v);
            q[r][2] = sbyte<2>(v);
            q[r][3] = sbyte<3>(v);
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float4 xv = xs.get(m, p, 8 + c);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float s = (c == 0) ? q[r][0] * xv.x : __builtin_fmaf(q[r][0], xv.x, t[r][m]);
                s = __builtin_fmaf(q[r][1], xv.y, s);
                s = __builtin_fmaf(q[r][2], xv.z, s);
                t[r][m] = __builtin_fmaf(q[r][3], xv.w, s);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float d1 = half_hi(w[r][8]);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = __builtin_fmaf(d1, t[r][m], acc[r][m]);
    }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Lanes per row for P pairs: log2 of S.
__host__ __device__ inline int slots_log2(int P) {
    int l = 2;
    while ((1 << l) < P && l < 6) ++l;
    return l;
}

}  // namespace q8k
