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
// Memory: wave_rows below (the MoE expert passes) has each lane load its 68-byte pair
// with four 16-byte loads and one dword, prefetching the next pair into registers while
// the current one is multiplied.  The dense one-row kernel (gemv_q8.hip) instead copies
// whole row stretches into LDS with coalesced direct copies and reads each lane's pair
// from there; both run mac_pair on the same pairs in the same order.  The int8 ->
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

// Activation access: the 4 values of activation row m at k = 64*p + 4*c .. +3.
// LDS copy in slot-major order: float4 index ((m*16 + c) * P + p), so the lanes of a
// wave (consecutive p) read consecutive 16-byte vectors.
struct XLds {
    const float4* base;
    int P;
    __device__ __forceinline__ float4 get(int m, int p, int c) const { return base[(m * 16 + c) * P + p]; }
};
// Straight from global memory (rows of length >= K at stride ldx).
struct XGlobal {
    const float* x;
    int ldx;
    __device__ __forceinline__ float4 get(int m, int p, int c) const {
        return *reinterpret_cast<const float4*>(x + (size_t)m * ldx + 64 * p + 4 * c);
    }
};

// Stage activation rows into the slot-major LDS layout.  row_ptr(m) gives the global
// address of row m (nullptr -> a row of zeros).  All threads of the block take part;
// the caller synchronizes afterwards.
template <class RowPtr>
__device__ __forceinline__ void stage_x_lds(float4* lds, int m_rows, int P, RowPtr row_ptr, int tid, int nthreads) {
    const int k4 = P * 16;
    for (int i = tid; i < m_rows * k4; i += nthreads) {
        const int m = i / k4;
        const int kk = i - m * k4;
        const int p = kk >> 4;
        const int c = kk & 15;
        const float* src = row_ptr(m);
        lds[(m * 16 + c) * P + p] = src ? *reinterpret_cast<const float4*>(src + 4 * kk) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
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

// One wave walks row groups first, first+stride, ... < end (G = 64/S rows each) of a
// Q8_0 matrix.  For R = 2 the lane also multiplies row n + r_off (gate/up pairs).
// out(n, acc) is called on the lane with slot 0 of each valid row n < n_out.
// NRC: the rounds per row when known at compile time (1: a row fits the S lanes once),
// 0 = computed from P (the per-item index arithmetic then divides by it).
template <int M, int R, int NRC, class X, class Out>
__device__ __forceinline__ void wave_rows(const uint8_t* __restrict__ w, int n_out, int r_off, int P, int log2S,
                                          const X& xs, int first, int stride, int end, Out&& out) {
    if (first >= end) return;
    const int S = 1 << log2S;
    const int G = 64 >> log2S;
    const int lane = threadIdx.x & 63;
    const int j = lane & (S - 1);
    const int g = lane >> log2S;
    const size_t row_bytes = (size_t)P * 68;
    const int n_rounds = NRC ? NRC : (P + S - 1) / S;
    const int n_items = ((end - 1 - first) / stride + 1) * n_rounds;

    auto item = [&](int it, int& n, int& p) {
        const int rg = first + (it / n_rounds) * stride;
        n = rg * G + g;
        p = j + S * (it % n_rounds);
    };
    // Loads are unconditional so the compiler keeps the next item's loads in flight
    // (a load inside a branch makes it wait for all of them): a row past the matrix
    // loads the last row, a pair past the row loads a pair of the same row; neither is
    // multiplied or stored under its own index.
    auto load_item = [&](int it, uint32_t(&wr)[R][17]) __attribute__((always_inline)) {
        int n, p;
        item(it, n, p);
        const int nc = n < n_out ? n : n_out - 1;
        const int pc = p < P ? p : p % P;
#pragma unroll
        for (int r = 0; r < R; ++r) load_pair(w + (size_t)(nc + r * r_off) * row_bytes + 68 * (size_t)pc, wr[r]);
    };

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    auto finish_item = [&](int it, const uint32_t(&wr)[R][17]) __attribute__((always_inline)) {
        int n, p;
        item(it, n, p);
        const int nc = n < n_out ? n : n_out - 1;
        if (p < P) mac_pair<M, R>(wr, xs, p, acc);
        if (it % n_rounds == n_rounds - 1) {
            for (int off = S >> 1; off >= 1; off >>= 1) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
            }
            // after the butterfly every lane of the row holds the same bits: all store
            // (a lane past the matrix multiplies the last row and stores what its owner
            // stores)
            out(nc, acc);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
        }
    };

    // Two register buffers, alternating: load item it+1 while multiplying item it.
    uint32_t wa[R][17], wb[R][17];
    load_item(0, wa);
    int it = 0;
    for (; it + 1 < n_items; it += 2) {
        load_item(it + 1, wb);
        finish_item(it, wa);
        load_item(it + 2 < n_items ? it + 2 : it + 1, wa);  // past the end: a reload, unused
        finish_item(it + 1, wb);
    }
    if (it < n_items) finish_item(it, wa);
}

}  // namespace q8k
