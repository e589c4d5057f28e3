// Dense Q8_0 x float32 linears for 1..16 activation rows per launch (gfx950).
//
// The packed-weight linear of "14. Model families and example applications" section
// 14.1 (LinearWeight: quant forms run packed kernels, no global dequantization; q/k/v
// and gate/up fused into one wider matrix each) and the SwiGLU FFN of section 14.2.
// Lockstep batch decode multiplies one pass over the weights by several activation
// rows (section 14.2), so all rows of a launch share every weight load.
//
// Grid: persistent workgroups of 4 waves, as many as fit on the device at once (at
// most one row group per wave); each wave walks row groups at a stride of the total
// wave count.  Activation rows are staged in LDS once per workgroup when they fit in
// 64 KB, else read from global memory (L2-resident).  See gemv_core.h for the lane
// layout and the summation order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "gemv_core.h"
#include "lds_dma.h"
#include "q8_internal.h"

namespace q8k {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

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

template <int M, int R, int NR, int D, int WPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, WPE))) void gemv_xreg_kernel(const uint8_t* __restrict__ w, int n_out, int P, int log2S,
                                                             const float* __restrict__ x, int ldx,
                                                             float* __restrict__ y, int ldy, int ipw) {
    static_assert(D % NR == 0, "the ring depth must be a multiple of the rounds per row");
    extern __shared__ float4 x_lds[];
    const int S = 1 << log2S;
    const int G = 64 >> log2S;
    const int lane = threadIdx.x & 63;
    const int j = lane & (S - 1);
    const int g = lane >> log2S;
    const size_t row_bytes = (size_t)P * 68;

    const int total = ((n_out + G - 1) / G) * NR;  // items: (row group, round)
    const int wid = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int nw = gridDim.x * kWaves;

    // Wave w takes the row groups w, w + W, w + 2W, ... (W waves in the grid; `ipw` items
    // per wave, a multiple of D and of NR), so at any time the grid streams one window of
    // the matrix.  Every load and
    // store below is unconditional so the compiler counts the outstanding memory
    // operations exactly and keeps the ring's loads in flight while an item is
    // multiplied (a load inside a branch makes it wait for all of them):
    //  - a lane whose pair index is past the row (p >= P, only when S does not divide
    //    P) loads pair p - P of the same row instead and skips the multiply;
    //  - a lane whose row is past the matrix, and any item past the last one (only in
    //    the grid's last wave), work on the last row group again and store the same
    //    bits its owner stores.
    // After the xor butterfly every lane of a row holds the same bits, so all of them
    // store it.

    // local item it -> row (clamped) of this lane; its round is it % NR
    auto item_row = [&](int itl) __attribute__((always_inline)) {
        const int it = (wid + (itl / NR) * nw) * NR + (itl % NR);
        const int itc = it < total ? it : total - NR + (it % NR);
        const int n = (itc / NR) * G + g;
        return n < n_out ? n : n_out - 1;
    };
    auto load_item = [&](int it, int i, uint32_t(&wr)[R][17]) __attribute__((always_inline)) {
        const int n = item_row(it);
        const int p = j + S * i;
        const int pc = p < P ? p : p - P;
#pragma unroll
        for (int r = 0; r < R; ++r) load_pair(w + (size_t)(n + r * n_out) * row_bytes + 68 * (size_t)pc, wr[r]);
    };

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    // The ring's first weight loads are issued before the activations are staged, so the
    // weights' HBM latency runs under the staging instead of after it (with one round per
    // row; with more, the extra live registers cost the ring its overlap).
    uint32_t ring[D][R][17];
    auto ring_prologue = [&]() __attribute__((always_inline)) {
        static_for<D - 1>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            load_item(s, s % NR, ring[s]);
        });
    };
    if constexpr (NR == 1) ring_prologue();
    // Activations: one coalesced pass from global into the slot-major LDS layout per
    // block, then each lane copies the values of its own pair slots into registers.
    stage_x_lds(x_lds, M, P, [&](int m) { return x + (size_t)m * ldx; }, threadIdx.x, kThreads);
    __syncthreads();
    if (wid >= total / NR) return;
    float4 xr[NR][M][16];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = j + S * i;
        const int pc = p < P ? p : p - P;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < 16; ++c) xr[i][m][c] = x_lds[(m * 16 + c) * P + pc];
    }
    if constexpr (NR > 1) ring_prologue();

    // One ring step: prefetch item it+D-1 (when LOAD), multiply item it, and finish the
    // row after its last round.
    auto step = [&](int it0, auto sc, auto load_tag) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        constexpr int i = s % NR;
        const int it = it0 + s;
        if constexpr (decltype(load_tag)::value) load_item(it + D - 1, (s + D - 1) % NR, ring[(s + D - 1) % D]);
        if (j + S * i < P) mac_pair<M, R>(ring[s], XArr<M>{xr[i]}, j + S * i, acc);
        if constexpr (i == NR - 1) {
            for (int off = S >> 1; off >= 1; off >>= 1) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
            }
            const int n = item_row(it);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if constexpr (R == 2)
                    y[(size_t)m * ldy + n] = silu_mul(acc[0][m], acc[1][m]);
                else
                    y[(size_t)m * ldy + n] = acc[0][m];
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
        }
    };
    // Steady state: every step prefetches.  The last ring of the wave is straight-line
    // code that only prefetches the wave's final item, so no load sits in a branch.
    const int last = ipw - D;
    for (int it0 = 0; it0 < last; it0 += D)
        static_for<D>([&](auto sc) __attribute__((always_inline)) { step(it0, sc, std::true_type{}); });
    static_for<D>([&](auto sc) __attribute__((always_inline)) {
        step(last, sc, std::integral_constant<bool, decltype(sc)::value == 0>{});
    });
}

// Block-pair formats of the rows kernel.  A "pair" is two consecutive blocks (64
// weights); rows are 16-byte aligned, so pairs start on dword boundaries.  weights<HALF>
// gives the 4 weights, as exact float32, of inputs 4*cc .. 4*cc+3 of block HALF.
struct FmtQ8_0 {  // 68 bytes: [d0 | 32 q] [d1 | 32 q]
    static constexpr int kPairBytes = 68, kDwords = 17, kLoads = 5;
    static __device__ __forceinline__ void load(const uint8_t* p, uint32_t (&w)[kDwords]) { load_pair(p, w); }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4]) {
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
};

// GGUF Q4_0: 36 bytes a pair, [d0 | 16 bytes] [d1 | 16 bytes]; weight j < 16 of a block is
// the low nibble of its byte j, weight j + 16 the high nibble; w = d * (nibble - 8), exact
// in float32 (a 4-bit integer times an 11-bit scale).
struct FmtQ4_0 {
    static constexpr int kPairBytes = 36, kDwords = 9, kLoads = 3;
    static __device__ __forceinline__ void load(const uint8_t* p, uint32_t (&w)[kDwords]) {
        const u32x4_a4 a = *reinterpret_cast<const u32x4_a4*>(p);
        const u32x4_a4 b = *reinterpret_cast<const u32x4_a4*>(p + 16);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        w[8] = *reinterpret_cast<const uint32_t*>(p + 32);
    }
    template <int HALF>
    static __device__ __forceinline__ void weights(const uint32_t (&w)[kDwords], int cc, float (&wf)[4]) {
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
};

// Several activation rows (1 <= M <= 8 per launch; the class used for 2..255 rows).  A
// block tile is 8*R rows (fused: R gate/up row pairs) over the whole K, worked on by two
// groups of 2 waves: group h takes the chunks h, h+2, h+4, ... of 16 pairs (1024 inputs)
// each.  16 lanes share a row (lane j owns pair j of a chunk), 4 row slots per wave, R
// rows (or row pairs) per lane, so each activation value read from LDS feeds R (or 2R)
// rows.  Each step copies both groups' activation chunks into slot-major LDS with
// direct-to-LDS loads (no register round trip); the weights of the step after next are
// loaded while a step is multiplied (a ring of two steps in registers).  Weights are
// dequantized exactly (fp32(d) * q needs at most 19 significant bits), one fma per
// weight and activation row.
//
// Per-output order: acc = fma(w_k, x_k, acc) over the lane's weights (its pair of each
// of the group's chunks in increasing order, inputs in increasing order), the xor
// butterfly over the 16 lanes (8, 4, 2, 1), then group 0's sum + group 1's sum.  It
// depends only on K, never on M or R, so every row of a 2..255-row call is bit-identical
// to the same row in any other such call.
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
    const size_t row_bytes = (size_t)P * Fmt::kPairBytes;
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
            Fmt::load(w + (size_t)n * row_bytes + Fmt::kPairBytes * (size_t)pc, wr[r]);
            if constexpr (SILU) Fmt::load(w + (size_t)(n + n_out) * row_bytes + Fmt::kPairBytes * (size_t)pc, wr[R + r]);
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
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                float wf[RR][4];
#pragma unroll
                for (int r = 0; r < RR; ++r) Fmt::template weights<HALF>(wc[r], cc, wf[r]);
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

namespace {

// Blocks resident per CU for a kernel, queried once per kernel and LDS size.
template <class K>
int resident_blocks(K kernel, size_t lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return per_cu;
}

inline int grid_for(const DeviceInfo& dev, int per_cu, int row_groups) {
    const int want = (row_groups + kWaves - 1) / kWaves;
    int blocks = dev.cu_count * per_cu;
    if (blocks > want) blocks = want;
    return blocks < 1 ? 1 : blocks;
}

template <int M, int R, int NR, int D, int WPE>
hipError_t launch_xreg(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                       float* y, int ldy, hipStream_t stream) {
    const size_t lds = (size_t)M * P * 256;
    static thread_local int cached_lds = -1, per_cu = 1;
    if (cached_lds != (int)lds) {
        per_cu = resident_blocks(gemv_xreg_kernel<M, R, NR, D, WPE>, lds);
        cached_lds = (int)lds;
    }
    const int G = 64 >> log2S;
    const int total = ((n_out + G - 1) / G) * NR;
    // items per wave: enough to cover the work with the waves that fit at once, rounded
    // up to a multiple of the ring depth (at least one ring)
    const int resident = dev.cu_count * per_cu * kWaves;
    int ipw = (total + resident - 1) / resident;
    ipw = ((ipw + D - 1) / D) * D;
    const int waves = (total + ipw - 1) / ipw;
    const int blocks = (waves + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((gemv_xreg_kernel<M, R, NR, D, WPE>), dim3(blocks), dim3(kThreads), lds, stream, w, n_out, P,
                       log2S, x, ldx, y, ldy, ipw);
    return hipGetLastError();
}

// Register-resident activations for one row and at most 4 pair rounds per lane
// (K <= 16384); the ring depth is a multiple of the rounds.
template <int M, int R>
bool try_xreg_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
              float* y, int ldy, hipStream_t stream, hipError_t* err) {
    const int S = 1 << log2S;
    const int NR = (P + S - 1) / S;
    // (ring depth, waves per SIMD) per shape: the ring and the activations stay in registers
    switch (NR) {
        case 1: {
            // A matrix with few row groups would leave most SIMDs idle if every wave had to
            // fill a whole ring: shallower rings give one wave per SIMD first.
            const int items = (n_out + (64 >> log2S) - 1) / (64 >> log2S);
            const int simds = dev.cu_count * kWaves;
            if (items <= simds) *err = launch_xreg<M, R, 1, 1, 4>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
            else if (items <= 2 * simds) *err = launch_xreg<M, R, 1, 2, 3>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
            else *err = launch_xreg<M, R, 1, (R == 1 ? 4 : 3), (R == 1 ? 3 : 2)>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
            return true;
        }
        case 2: *err = launch_xreg<M, R, 2, (R == 1 ? 4 : 2), 2>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        case 3: *err = launch_xreg<M, R, 3, 3, 1>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        case 4: *err = launch_xreg<M, R, 4, 4, 1>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
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
    // R rows (row pairs) per lane: more rows per lane share each activation read, fewer
    // spread the tiles more evenly.  Take the largest R within 5% of the best fill.
    const int64_t cus = dev.cu_count;
    const double f1 = round_fill((n_out + 7) / 8, cus * rows_per_cu<Fmt, M, 1, SILU>());
    const double f2 = round_fill((n_out + 15) / 16, cus * rows_per_cu<Fmt, M, 2, SILU>());
    double f4 = 0.0;
    if constexpr (!SILU) f4 = round_fill((n_out + 31) / 32, cus * rows_per_cu<Fmt, M, 4, SILU>());
    const double best = f1 > f2 ? (f1 > f4 ? f1 : f4) : (f2 > f4 ? f2 : f4);
    if constexpr (!SILU) {
        if (f4 >= 0.95 * best) return launch_rows_r<Fmt, M, 4, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
    }
    if (f2 >= 0.95 * best) return launch_rows_r<Fmt, M, 2, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
    return launch_rows_r<Fmt, M, 1, SILU>(dev, n_out, P, w, x, ldx, y, ldy, stream);
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

hipError_t launch_gemv_q8(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                          const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    const int log2S = slots_log2(P);
    if (m == 1) {  // one row: the register-ring kernel when K fits it
        hipError_t e;
        if (silu_pairs ? try_xreg_m<1, 2>(dev, w, (int)n_out, P, log2S, x, (int)ldx, y, (int)ldy, stream, &e)
                       : try_xreg_m<1, 1>(dev, w, (int)n_out, P, log2S, x, (int)ldx, y, (int)ldy, stream, &e))
            return e;
    }
    // several rows (or one row with K beyond the register kernel): 8-row launches
    for (int64_t m0 = 0; m0 < m; m0 += 8) {
        const int mm = (int)((m - m0) < 8 ? (m - m0) : 8);
        const float* xc = x + m0 * ldx;
        float* yc = y + m0 * ldy;
        hipError_t e = silu_pairs ? launch_r<2>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream)
                                  : launch_r<1>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q8k
