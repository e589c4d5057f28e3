// Prefill (M >= 256 activation rows): Q8_0 weights x float32 activations on the bf16
// matrix cores of gfx950 (v_mfma_f32_16x16x32_bf16), float32 accumulation and output.
//
// With hundreds of rows the linear is a dense contraction (the tensor-core vs GEMV
// kernel-class boundary of the fucina DGX Spark README, Performance): each weight is
// used M times, so the matrix cores, not memory, bound it.  The weights stay Q8_0 in
// HBM ("14. Model families and example applications", section 14.1: no global
// dequantization); every block is dequantized once per tile into LDS.
//
// Tile: 128 activation rows x BN weight rows (BN = 256 with 8 waves, or 128 / 64 with 4;
// fused gate_up: BN/2 gate + BN/2 up rows, interleaved in groups of 16 so a lane holds gate
// and up of the same output), K in steps of 64 (one Q8_0 block pair per weight row).  Per
// step the threads dequantize the tile's Q8_0 blocks (d * q rounded to bf16, exactly: d*q
// needs at most 19 significant bits, then one rounding) and convert 128 x 64 activations to
// bf16 (round to nearest even), both into LDS rows padded to 144 bytes; each wave then runs
// a 64 x BN/(waves/2) sub-tile as 16 x 16 MFMA tiles, two K=32 steps.  Every weight tile
// re-reads (from L2) and re-converts the float32 activations, so wider tiles cut that
// traffic per flop: 256-wide tiles measured 1.16x (M = 512) to 1.45x (M = 2048) faster than
// 128-wide ones on the Qwen3-8B gate_up.

// Latency: the Q8_0 bytes come from HBM, so each thread keeps a ring of the next
// kRing steps' blocks in registers (9 dwords a step); activations are re-read by every
// weight tile and mostly hit L2, so one step of look-ahead covers them.  LDS is double
// buffered: one barrier per step.
//
// MFMA lane layout (checked on the device): lane l supplies A[l%16][8*(l/16) + i] and
// B[8*(l/16) + i][l%16], i = 0..7, and receives D[4*(l/16) + i][l%16], i = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "q8_internal.h"

namespace q8k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4m __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kBM = 128;           // activation rows per tile
constexpr int kBK = 64;            // inputs per K step (one Q8_0 block pair per weight row)
constexpr int kLdsRow = kBK + 8;   // bf16 per LDS row (144 bytes: 16-byte steps between rows)
constexpr int kRing = 4;           // K steps of Q8_0 bytes in flight per thread (K/64 is a multiple of 4)

// Calls f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>) in order.
template <typename F, int... I>
__device__ __forceinline__ void mf_static_for(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

__device__ __forceinline__ float mf_half_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float mf_half_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Weight row of tile column c for output tile nt (BN columns; fused: BN/2 outputs with
// gate and up columns interleaved in groups of 16).
template <int BN, bool SILU>
__device__ __forceinline__ int tile_row(int nt, int c, int n_out) {
    if constexpr (SILU) {
        int f = nt * (BN / 2) + 16 * (c >> 5) + (c & 15);
        f = f < n_out ? f : n_out - 1;
        return ((c >> 4) & 1) ? f + n_out : f;
    } else {
        const int n = nt * BN + c;
        return n < n_out ? n : n_out - 1;
    }
}

struct Q8Pair {  // 9 dwords of one Q8_0 block as it sits in its pair (see the loader)
    uint32_t dw[9];
};

// Expert-grouped tiles (the MoE prefill form): tile t of the grid's tile list belongs to
// the expert e with tile_start[e] <= t < tile_start[e + 1]; its activation rows are the
// positions offsets[e] + 128 * (t - tile_start[e]) + r of the expert-sorted pair list.
// gather: row of position pos is x[sorted[pos] / k] (the token's input); else x[pos].
// The output row of position pos is y[pos].
struct GroupArgs {
    const int32_t* offsets;     // [n_exp + 1] pair positions per expert
    const int32_t* tile_start;  // [n_exp + 1] first 128-row tile of each expert
    const int32_t* sorted;      // [pairs] pair index (token * k + slot) at each position
    int n_exp, k, n_tiles;      // n_tiles: output tiles per expert (grid = tiles x n_tiles)
    size_t expert_bytes;        // bytes of one expert's Q8_0 matrix
    bool gather;
};

template <int BN, bool SILU, bool GROUPED, int NT = 256>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_q8_mfma_kernel(const uint8_t* __restrict__ w, int n_out, int P,
                                                           const float* __restrict__ x, int M, int ldx,
                                                           float* __restrict__ y, int ldy, int m_tiles,
                                                           GroupArgs g) {
    constexpr int WN = NT / 128;       // waves along n (two along m)
    constexpr int TJ = BN / (16 * WN); // 16x16 tiles per wave along n
    constexpr int SPLIT = NT / (2 * BN);  // threads per Q8_0 block (1: whole block, 2: 16 quants each)
    static_assert(SPLIT == 1 || SPLIT == 2, "2*BN blocks per step over NT threads");
    constexpr int XPT = kBM * kBK / NT;   // activations per thread per step (32 or 16)
    constexpr int XPR = kBK / XPT;        // threads per activation row
    __shared__ __attribute__((aligned(16))) __bf16 xs[2][kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) __bf16 ws[2][BN * kLdsRow];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;  // wn < WN
    int mt = blockIdx.x % m_tiles;  // m tiles of one n tile run side by side (shared weights)
    int nt = blockIdx.x / m_tiles;
    int mbase = 0;  // grouped: first position of the tile (its rows are positions mbase + r)
    if constexpr (GROUPED) {
        const int t = blockIdx.x / g.n_tiles;
        nt = blockIdx.x - t * g.n_tiles;
        if (t >= g.tile_start[g.n_exp]) return;  // past the tile list (block-uniform, no barrier yet)
        int lo = 0, hi = g.n_exp;  // tile_start[lo] <= t < tile_start[hi]: the expert is the largest such lo
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.tile_start[mid] <= t) lo = mid;
            else hi = mid;
        }
        mbase = g.offsets[lo] + kBM * (t - g.tile_start[lo]);
        const int rows = g.offsets[lo + 1] - mbase;
        M = rows < kBM ? rows : kBM;
        mt = 0;
        w += (size_t)lo * g.expert_bytes;
    }
    const size_t row_bytes = (size_t)P * 68;

    // weight role: block wb of the pair of tile column wc (part hh of it when SPLIT = 2).
    // In a pair (68 bytes) block 0 is bytes [0, 34) and block 1 bytes [34, 68); the 9
    // dwords loaded from byte 32*wb hold block 0 at byte 0 (scale) and 2..33 (quants), or
    // block 1 at bytes 2..3 (scale) and 4..35 (quants).
    const int wc = (tid / (2 * SPLIT)), wb = (tid / SPLIT) & 1, hh = tid & (SPLIT - 1);
    const uint8_t* wrow = w + (size_t)tile_row<BN, SILU>(nt, wc, n_out) * row_bytes + 32 * wb;
    // activation role: XPT inputs (part xh of the step) of tile row xr
    const int xr = tid / XPR, xh = tid % XPR;
    int xm = mt * kBM + xr;
    xm = xm < M ? xm : M - 1;
    size_t xoff = (size_t)xm;
    if constexpr (GROUPED) xoff = g.gather ? (size_t)(g.sorted[mbase + xm] / g.k) : (size_t)(mbase + xm);
    const float* xrow = x + xoff * ldx + XPT * xh;

    f32x4 acc[4][TJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Q8Pair ring[kRing];
    float4 rx[XPT / 4];
    auto load_w = [&](Q8Pair& r, int s) __attribute__((always_inline)) {
        const uint8_t* src = wrow + (size_t)68 * s;
        const u32x4_a4m a = *reinterpret_cast<const u32x4_a4m*>(src);
        const u32x4_a4m b = *reinterpret_cast<const u32x4_a4m*>(src + 16);
        r.dw[0] = a.x; r.dw[1] = a.y; r.dw[2] = a.z; r.dw[3] = a.w;
        r.dw[4] = b.x; r.dw[5] = b.y; r.dw[6] = b.z; r.dw[7] = b.w;
        r.dw[8] = *reinterpret_cast<const uint32_t*>(src + 32);
    };
    auto load_x = [&](int s) __attribute__((always_inline)) {
        const float4* src = reinterpret_cast<const float4*>(xrow + kBK * s);
#pragma unroll
        for (int i = 0; i < XPT / 4; ++i) rx[i] = src[i];
    };
    auto store_w = [&](const Q8Pair& r, int buf) __attribute__((always_inline)) {
        const float d = wb == 0 ? mf_half_lo(r.dw[0]) : mf_half_hi(r.dw[0]);
        constexpr int NQ = 32 / SPLIT;  // quants this thread converts
        bf16x8 v[NQ / 8];
#pragma unroll
        for (int g = 0; g < NQ / 4; ++g) {
            // quant dword g + hh*NQ/4 of the block (selects, not a dynamic register index)
            uint32_t lo = r.dw[g], hi = r.dw[g + 1];
            if constexpr (SPLIT == 2) {
                lo = hh ? r.dw[g + 4] : lo;
                hi = hh ? r.dw[g + 5] : hi;
            }
            const uint32_t q4 = wb == 0 ? __builtin_amdgcn_alignbit(hi, lo, 16) : hi;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                v[g >> 1][4 * (g & 1) + b] = (__bf16)((float)(int)(int8_t)(q4 >> (8 * b)) * d);
        }
        bf16x8* dst = reinterpret_cast<bf16x8*>(&ws[buf][wc * kLdsRow + 32 * wb + NQ * hh]);
#pragma unroll
        for (int i = 0; i < NQ / 8; ++i) dst[i] = v[i];
    };
    auto store_x = [&](int buf) __attribute__((always_inline)) {
        bf16x8 v[XPT / 8];
#pragma unroll
        for (int i = 0; i < XPT / 4; ++i) {
            v[i >> 1][4 * (i & 1) + 0] = (__bf16)rx[i].x;
            v[i >> 1][4 * (i & 1) + 1] = (__bf16)rx[i].y;
            v[i >> 1][4 * (i & 1) + 2] = (__bf16)rx[i].z;
            v[i >> 1][4 * (i & 1) + 3] = (__bf16)rx[i].w;
        }
        bf16x8* dst = reinterpret_cast<bf16x8*>(&xs[buf][xr * kLdsRow + XPT * xh]);
#pragma unroll
        for (int i = 0; i < XPT / 8; ++i) dst[i] = v[i];
    };
    auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            bf16x8 af[4], bfr[TJ];
            const int ko = kk + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&xs[buf][(64 * wm + 16 * i + (lane & 15)) * kLdsRow + ko]);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(&ws[buf][((BN / WN) * wn + 16 * j + (lane & 15)) * kLdsRow + ko]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    // prologue: K steps 0..kRing-1 of Q8_0 bytes, step 0 of the activations (P >= kRing)
    // Issue order matters: the wait counter retires loads in order, so the activations a
    // step needs next are issued before the weight loads it needs kRing steps later.
    load_w(ring[0], 0);
    load_x(0);
    __builtin_amdgcn_sched_barrier(0);
    mf_static_for([&](auto j) __attribute__((always_inline)) {
        if constexpr (j.value > 0) load_w(ring[j.value], j.value);
    }, std::make_integer_sequence<int, kRing>{});
    for (int s0 = 0; s0 < P; s0 += kRing) {
        mf_static_for([&](auto j) __attribute__((always_inline)) {
            const int s = s0 + j.value;
            const int buf = j.value & 1;  // kRing is even, so buf == s & 1
            store_x(buf);
            store_w(ring[j.value], buf);
            load_x(s + 1 < P ? s + 1 : s);
            __builtin_amdgcn_sched_barrier(0);
            load_w(ring[j.value], s + kRing < P ? s + kRing : s);
            __syncthreads();
            mma(buf);
            // keep the next step's conversions (which wait for its loads) below this step's MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }, std::make_integer_sequence<int, kRing>{});
    }

    // ---- epilogue: lane holds D[m = 4*(lane/16) + e][n = lane%16] of each 16 x 16 tile
    if constexpr (GROUPED) y += (size_t)mbase * ldy;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = mt * kBM + 64 * wm + 16 * i + 4 * (lane >> 4) + e;
            if (m >= M) continue;
            if constexpr (SILU) {
#pragma unroll
                for (int jp = 0; jp < TJ / 2; ++jp) {
                    // wave columns (BN/WN)*wn + 16*j: even j gate, odd j up of the same outputs
                    const int f = nt * (BN / 2) + (BN / (2 * WN)) * wn + 16 * jp + (lane & 15);
                    if (f < n_out) {
                        const float g = acc[i][2 * jp][e];
                        const float u = acc[i][2 * jp + 1][e];
                        y[(size_t)m * ldy + f] = g / (1.0f + __expf(-g)) * u;
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const int n = nt * BN + (BN / WN) * wn + 16 * j + (lane & 15);
                    if (n < n_out) y[(size_t)m * ldy + n] = acc[i][j][e];
                }
            }
        }
    }
}

template <int BN, int NT = 256>
hipError_t launch_tiles(const uint8_t* w, int64_t n_out, int P, bool silu, const float* x, int64_t m, int64_t ldx,
                        float* y, int64_t ldy, hipStream_t stream) {
    const GroupArgs none{};
    const int m_tiles = (int)((m + kBM - 1) / kBM);
    const int64_t cols = silu ? BN / 2 : BN;  // outputs per tile
    const int64_t blocks = (n_out + cols - 1) / cols * m_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (silu)
        hipLaunchKernelGGL((gemm_q8_mfma_kernel<BN, true, false, NT>), dim3((unsigned)blocks), dim3(NT), 0, stream, w,
                           (int)n_out, P, x, (int)m, (int)ldx, y, (int)ldy, m_tiles, none);
    else
        hipLaunchKernelGGL((gemm_q8_mfma_kernel<BN, false, false, NT>), dim3((unsigned)blocks), dim3(NT), 0, stream, w,
                           (int)n_out, P, x, (int)m, (int)ldx, y, (int)ldy, m_tiles, none);
    return hipGetLastError();
}

hipError_t launch_gemm_q8_mfma_grouped(const uint8_t* w_stack, size_t expert_bytes, int64_t n_out, int64_t k,
                                       bool silu_pairs, const float* x, int64_t ldx, float* y, int64_t ldy,
                                       const int32_t* offsets, const int32_t* tile_start, const int32_t* sorted,
                                       int n_exp, int top_k, bool gather, int64_t max_tiles, hipStream_t stream) {
    const int P = (int)(k / kBK);
    const int64_t cols = silu_pairs ? 128 : 256;  // outputs per 128 x 256 tile
    const int n_tiles = (int)((n_out + cols - 1) / cols);
    const int64_t blocks = max_tiles * n_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const GroupArgs g{offsets, tile_start, sorted, n_exp, top_k, n_tiles, expert_bytes, gather};
    if (silu_pairs)
        hipLaunchKernelGGL((gemm_q8_mfma_kernel<256, true, true, 512>), dim3((unsigned)blocks), dim3(512), 0, stream,
                           w_stack, (int)n_out, P, x, 0, (int)ldx, y, (int)ldy, 1, g);
    else
        hipLaunchKernelGGL((gemm_q8_mfma_kernel<256, false, true, 512>), dim3((unsigned)blocks), dim3(512), 0, stream,
                           w_stack, (int)n_out, P, x, 0, (int)ldx, y, (int)ldy, 1, g);
    return hipGetLastError();
}

hipError_t launch_gemm_q8_mfma(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                               const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / kBK);
    // The widest tiles that still give at least one tile per CU: 128 x 256 (8 waves),
    // 128 x 128, else 128 x 64 (small N stays spread over the chip at the cost of reading
    // the activations more often).
    const int64_t cols128 = silu_pairs ? 64 : 128;
    const int64_t tiles128 = ((n_out + cols128 - 1) / cols128) * ((m + kBM - 1) / kBM);
    const int64_t tiles256 = (tiles128 + 1) / 2;
    if (tiles256 >= dev.cu_count) return launch_tiles<256, 512>(w, n_out, P, silu_pairs, x, m, ldx, y, ldy, stream);
    if (tiles128 >= dev.cu_count) return launch_tiles<128>(w, n_out, P, silu_pairs, x, m, ldx, y, ldy, stream);
    return launch_tiles<64>(w, n_out, P, silu_pairs, x, m, ldx, y, ldy, stream);
}

}  // namespace q8k
