// Integer Q8_0 x q8 linears: activations quantized to int8 codes per block of 32
// inputs, block dot products in 32-bit integers (gfx950 v_dot4 on packed bytes).
//
// The DGX Spark README (Features; Architecture) names quantized GEMV kernels that read
// Q8_0 directly through int8 dot products, and the qwen3 runner README names an
// integer q8 x q8 dot path over quantized blocks.  The activation code used here (no
// page defines one): per block of 32 inputs, amax = max |x|, dx = amax / 127 and
// q = round-half-even(x * (127 / amax)), every quotient and product rounded to
// float32; a block with amax below 2^-120 is coded as zero with dx = 0 (127 / amax
// would leave the float32 range).
//
// Output: y[m][n] = sum over blocks b of (d_w[n][b] * dx[m][b]) * isum, where
// isum = sum_i q_w[n][b][i] * q_x[m][b][i] is exact (|isum| <= 32 * 128 * 128 < 2^24,
// so it also converts to float32 exactly).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemv_core.h"
#include "lds_dma.h"
#include "q8_internal.h"

namespace q8k {

// ------------------------------------------------------------------ quantize
//
// One block of 32 inputs per 8 lanes (a float4 each); the block maximum by an xor
// butterfly over the 8 lanes; four codes packed into one dword store per lane.
constexpr int kQuantThreads = 256;

__global__ __launch_bounds__(kQuantThreads) void quantize_act_kernel(const float* __restrict__ x, int ldx, int nb,
                                                                     int64_t total, int8_t* __restrict__ xq,
                                                                     float* __restrict__ xd) {
    const int64_t g = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    const int64_t b = g >> 3;  // block index over the whole [m][nb]; its 8 lanes agree on b
    if (b >= total) return;
    const int sub = threadIdx.x & 7;
    const int64_t row = b / nb;
    const int blk = (int)(b - row * nb);
    const float4 v = *reinterpret_cast<const float4*>(x + row * ldx + 32 * blk + 4 * sub);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1, 8));
    a = fmaxf(a, __shfl_xor(a, 2, 8));
    a = fmaxf(a, __shfl_xor(a, 4, 8));
    const bool nz = a >= 0x1p-120f;
    const float inv = nz ? __fdiv_rn(127.0f, a) : 0.0f;
    const float d = nz ? __fdiv_rn(a, 127.0f) : 0.0f;
    auto code = [&](float t) __attribute__((always_inline)) {
        const float r = fminf(fmaxf(rintf(t * inv), -127.0f), 127.0f);
        return (uint32_t)((int)r & 0xFF);
    };
    const uint32_t packed = code(v.x) | (code(v.y) << 8) | (code(v.z) << 16) | (code(v.w) << 24);
    *reinterpret_cast<uint32_t*>(xq + row * (int64_t)nb * 32 + 32 * blk + 4 * sub) = packed;
    if (sub == 0) xd[row * nb + blk] = d;
}

hipError_t launch_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, int8_t* xq, float* xd,
                               hipStream_t stream) {
    const int nb = (int)(k / 32);
    const int64_t total = m * nb;
    const int64_t blocks = (total * 8 + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(quantize_act_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, x, (int)ldx, nb,
                       total, xq, xd);
    return hipGetLastError();
}

// ------------------------------------------------------------------ linear
//
// Up to M (1, 2, 4, 8 or 16) activation rows per launch; m_rows <= M of them are real
// and rows past m_rows repeat row m_rows - 1 (same bits, stored to the same place).
// The block tile and the split of the work are those of the float32 rows kernel: a
// tile is 8*R rows (fused: R gate/up row pairs) over the whole K, two groups of two
// waves take alternate chunks of 16 pairs (1024 inputs), 16 lanes share a row (lane j
// owns pair j of a chunk), 4 row slots per wave, R rows per lane.  A chunk of one
// activation row is 1024 code bytes and 32 scales; each step copies the next step's
// chunk of every row into LDS with direct-to-LDS loads while the current one is
// multiplied, and the weights of the next step are loaded into registers meanwhile.
//
// Per-output order: for each of the lane's pairs in increasing order, block 0 then
// block 1: acc = fma(d_w * dx, float(isum), acc); then the xor butterfly over the 16
// lanes (8, 4, 2, 1) and group 0's sum + group 1's sum.  It depends only on K: every
// row of a call is bit-identical to the same row in any other call.
constexpr int kActThreads = 256;

template <int M, int R, bool SILU>
__global__ __launch_bounds__(kActThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemv_q8act_kernel(
    const uint8_t* __restrict__ w, int n_out, int P, const int8_t* __restrict__ xq, const float* __restrict__ xd,
    int m_rows, float* __restrict__ y, int ldy) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16, "M");
    constexpr int RR = SILU ? 2 * R : R;  // weight rows per lane
    constexpr int CPW = (M + 1) / 2;      // code-row copies per wave and step
    // [buffer][group]: codes of row m at 16-byte unit m*64 + 16*c4 + j (bytes 16*c4 ..
    // 16*c4 + 15 of pair j); scales copied 8 rows per wave: row m's 32 at float
    // ((m & 1) * 8 + (m >> 1)) * 32.
    __shared__ int4 xc[2][2][M * 64];
    __shared__ float4 xs[2][2][128];
    __shared__ float part[8 * RR * M];  // group 1's row sums: [slot][r][m]
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS copy bases)
    const int h = wv >> 1;                                    // group
    const int par = wv & 1;                                   // wave within the group
    const int lane = tid & 63;
    const int j = lane & 15;
    const int slot = par * 4 + (lane >> 4);  // row slot within the group, 0..7
    const size_t row_bytes = (size_t)P * 68;
    const int ldq = 64 * P;  // code bytes per activation row (= K)
    const int ldd = 2 * P;   // scales per activation row (= K / 32)
    const int nch = (P + 15) >> 4;
    const int steps = (nch + 1) >> 1;
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    const int my_tiles = (tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int items = my_tiles * steps;
    __builtin_assume(steps >= 1);  // P >= 4 (K is a positive multiple of 256)
    __builtin_assume(items >= 1);  // the grid has at most `tiles` blocks
    __builtin_assume(m_rows >= 1);

    auto out_row = [&](int i, int r) __attribute__((always_inline)) {
        const int n = ((int)blockIdx.x + i * (int)gridDim.x) * (8 * R) + slot * R + r;
        return n < n_out ? n : n_out - 1;
    };
    auto chunk_of = [&](int st) __attribute__((always_inline)) {
        const int ch = h + 2 * st;
        return ch < nch ? ch : nch - 1;
    };
    auto act_row = [&](int m) __attribute__((always_inline)) { return m < m_rows ? m : m_rows - 1; };
    auto load_w = [&](int i, int st, uint32_t(&wr)[RR][17]) __attribute__((always_inline)) {
        const int p = 16 * chunk_of(st) + j;
        const int pc = p < P ? p : P - 1;  // past the row: a pair of the same row (unused)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = out_row(i, r);
            load_pair(w + (size_t)n * row_bytes + 68 * (size_t)pc, wr[r]);
            if constexpr (SILU) load_pair(w + (size_t)(n + n_out) * row_bytes + 68 * (size_t)pc, wr[R + r]);
        }
    };
    // The chunk of step st for every activation row: CPW code copies (1024 bytes of one
    // row each; lane l takes unit (c4 = l / 16, j = l % 16)) and one scale copy (8 rows,
    // lane l takes 4 scales of row 2*(l/8) + par).
    auto stage = [&](int st, int buf) __attribute__((always_inline)) {
        const int ch = chunk_of(st);
        int pc = 16 * ch + j;
        pc = pc < P ? pc : P - 1;
#pragma unroll
        for (int qq = 0; qq < CPW; ++qq) {
            const int mr = 2 * qq + par < M ? 2 * qq + par : M - 1;
            const int8_t* src = xq + (size_t)act_row(mr) * ldq + 64 * (size_t)pc + 16 * (lane >> 4);
            lds_copy16(src, &xc[buf][h][mr * 64]);
        }
        const int ms = 2 * (lane >> 3) + par;
        const int mc = ms < M ? ms : M - 1;
        int sidx = 32 * ch + 4 * (lane & 7);
        sidx = sidx < ldd ? sidx : ldd - 4;  // past the row: scales of the same row (unused)
        lds_copy16(xd + (size_t)act_row(mc) * ldd + sidx, &xs[buf][h][par * 64]);
    };

    float acc[RR][M];
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    auto compute = [&](int st, const uint32_t(&wc)[RR][17], int buf) __attribute__((always_inline)) {
        const int ch = h + 2 * st;
        if (ch < nch && 16 * ch + j < P) {
            uint32_t q0[RR][8];  // block 0's quants realigned to dwords (bytes 2..33 of the pair)
            float d0[RR], d1[RR];
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                d0[r] = half_lo(wc[r][0]);
                d1[r] = half_hi(wc[r][8]);
#pragma unroll
                for (int c = 0; c < 8; ++c) q0[r][c] = __builtin_amdgcn_alignbyte(wc[r][c + 1], wc[r][c], 2);
            }
            const int4* cb = xc[buf][h];
            const float* sb = reinterpret_cast<const float*>(xs[buf][h]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int4 a0 = cb[m * 64 + j];
                const int4 a1 = cb[m * 64 + 16 + j];
                const int4 b0 = cb[m * 64 + 32 + j];
                const int4 b1 = cb[m * 64 + 48 + j];
                const float2 s = *reinterpret_cast<const float2*>(sb + ((m & 1) * 8 + (m >> 1)) * 32 + 2 * j);
#pragma unroll
                for (int r = 0; r < RR; ++r) {
                    int i0 = __builtin_amdgcn_sdot4((int)q0[r][0], a0.x, 0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][1], a0.y, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][2], a0.z, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][3], a0.w, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][4], a1.x, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][5], a1.y, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][6], a1.z, i0, false);
                    i0 = __builtin_amdgcn_sdot4((int)q0[r][7], a1.w, i0, false);
                    int i1 = __builtin_amdgcn_sdot4((int)wc[r][9], b0.x, 0, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][10], b0.y, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][11], b0.z, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][12], b0.w, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][13], b1.x, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][14], b1.y, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][15], b1.z, i1, false);
                    i1 = __builtin_amdgcn_sdot4((int)wc[r][16], b1.w, i1, false);
                    acc[r][m] = __builtin_fmaf(d0[r] * s.x, (float)i0, acc[r][m]);
                    acc[r][m] = __builtin_fmaf(d1[r] * s.y, (float)i1, acc[r][m]);
                }
            }
        }
    };
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
            // every lane of the 16 holds the same bits: all store (rows past m_rows
            // store their copy of row m_rows - 1)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = out_row(i, r);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float* dst = y + (size_t)act_row(m) * ldy + n;
                    if constexpr (SILU)
                        *dst = silu_mul(acc[r][m], acc[R + r][m]);
                    else
                        *dst = acc[r][m];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    };

    uint32_t wc[RR][17], wn[RR][17];
    stage(0, 0);
    load_w(0, 0, wc);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay above the wait
    wait_vmcnt<0>();
    __syncthreads();
    // Item (tile i, step st): copy the next item's chunk into the other buffer and load
    // its weights into wn while multiplying this one; finish the tile after its last
    // step; wait for everything, wc = wn, barrier.  The part array of finish_tile is not
    // touched by the copies.
    int i = 0, st = 0;
    for (int it = 0; it < items; ++it) {
        const bool more = it + 1 < items;
        const bool last_step = st + 1 == steps;
        const int ni = last_step ? i + 1 : i;
        const int nst = last_step ? 0 : st + 1;
        const int cur = it & 1;
        if (more) {
            stage(nst, cur ^ 1);
            load_w(ni, nst, wn);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(st, wc, cur);
        if (last_step) finish_tile(i);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();
        if (more) {
#pragma unroll
            for (int r = 0; r < RR; ++r)
#pragma unroll
                for (int q = 0; q < 17; ++q) wc[r][q] = wn[r][q];
        }
        __syncthreads();
        i = ni;
        st = nst;
    }
}

namespace {

template <int M, int R, bool SILU>
int q8act_per_cu() {
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_q8act_kernel<M, R, SILU>, kActThreads, 0) !=
                hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    return per_cu;
}

template <int M, int R, bool SILU>
hipError_t launch_q8act_r(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const int8_t* xq,
                          const float* xd, int m_rows, float* y, int ldy, hipStream_t stream) {
    // persistent grid: one block per resident slot (at most one per tile)
    const int tiles = (n_out + 8 * R - 1) / (8 * R);
    const int64_t slots = (int64_t)dev.cu_count * q8act_per_cu<M, R, SILU>();
    const int blocks = (int)(tiles < slots ? tiles : slots);
    hipLaunchKernelGGL((gemv_q8act_kernel<M, R, SILU>), dim3(blocks), dim3(kActThreads), 0, stream, w, n_out, P, xq,
                       xd, m_rows, y, ldy);
    return hipGetLastError();
}

// Fraction of a persistent grid's block-steps that do work.
inline double fill(int64_t tiles, int64_t slots) {
    const int64_t per = (tiles + slots - 1) / slots;
    const int64_t used = tiles < slots ? tiles : slots;
    return (double)tiles / (double)(per * (used > 0 ? slots : 1));
}

// R rows (row pairs) per lane: the largest R within 5% of the best fill.  Four weight
// rows per lane (R = 4, or fused R = 2) up to 8 activation rows; two at 16.
template <int M, bool SILU>
hipError_t launch_q8act_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const int8_t* xq,
                          const float* xd, int m_rows, float* y, int ldy, hipStream_t stream) {
    constexpr bool kWide = M <= 8;
    const int64_t cus = dev.cu_count;
    const double f1 = fill((n_out + 7) / 8, cus * q8act_per_cu<M, 1, SILU>());
    double f2 = 0.0, f4 = 0.0;
    if constexpr (!SILU || kWide) f2 = fill((n_out + 15) / 16, cus * q8act_per_cu<M, (!SILU || kWide) ? 2 : 1, SILU>());
    if constexpr (!SILU && kWide) f4 = fill((n_out + 31) / 32, cus * q8act_per_cu<M, kWide ? 4 : 1, SILU>());
    const double best = f1 > f2 ? (f1 > f4 ? f1 : f4) : (f2 > f4 ? f2 : f4);
    if constexpr (!SILU && kWide) {
        if (f4 >= 0.95 * best) return launch_q8act_r<M, 4, SILU>(dev, w, n_out, P, xq, xd, m_rows, y, ldy, stream);
    }
    if constexpr (!SILU || kWide) {
        if (f2 >= 0.95 * best) return launch_q8act_r<M, 2, SILU>(dev, w, n_out, P, xq, xd, m_rows, y, ldy, stream);
    }
    return launch_q8act_r<M, 1, SILU>(dev, w, n_out, P, xq, xd, m_rows, y, ldy, stream);
}

template <bool SILU>
hipError_t launch_q8act_rows(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, const int8_t* xq,
                             const float* xd, int mm, float* y, int ldy, hipStream_t stream) {
    if (mm <= 1) return launch_q8act_m<1, SILU>(dev, w, n_out, P, xq, xd, mm, y, ldy, stream);
    if (mm <= 2) return launch_q8act_m<2, SILU>(dev, w, n_out, P, xq, xd, mm, y, ldy, stream);
    if (mm <= 4) return launch_q8act_m<4, SILU>(dev, w, n_out, P, xq, xd, mm, y, ldy, stream);
    if (mm <= 8) return launch_q8act_m<8, SILU>(dev, w, n_out, P, xq, xd, mm, y, ldy, stream);
    return launch_q8act_m<16, SILU>(dev, w, n_out, P, xq, xd, mm, y, ldy, stream);
}

}  // namespace

hipError_t launch_gemv_q8act(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                             const int8_t* xq, const float* xd, int64_t m, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mm = (int)((m - m0) < 16 ? (m - m0) : 16);
        const int8_t* xqc = xq + m0 * k;
        const float* xdc = xd + m0 * (k / 32);
        float* yc = y + m0 * ldy;
        hipError_t e = silu_pairs ? launch_q8act_rows<true>(dev, w, (int)n_out, P, xqc, xdc, mm, yc, (int)ldy, stream)
                                  : launch_q8act_rows<false>(dev, w, (int)n_out, P, xqc, xdc, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q8k
