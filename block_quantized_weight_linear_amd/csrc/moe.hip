// Grouped Q8_0 SwiGLU expert mixture (gfx950).
//
// "14. Model families and example applications" section 14.2: the MoE FFN is the
// router-weighted SwiGLU mixture (moeSwiGluFfnSeq), and with several tokens the work is
// grouped per expert so that one pass over an expert's weights serves all the tokens
// routed to it.  Section 14.4 ("MoE expert kernels"): a counting-sort route plan orders
// the (token, slot) pairs by expert, and each token's sum keeps a fixed order.
//
// Four launches on one stream, no host synchronization:
//   1. plan      one workgroup of 4 or 16 waves: counting sort of the m*k (token, slot)
//                pairs by expert, stable in pair order; offsets[e], sorted pair list,
//                and the inverse map pair -> position.
//   2. gate_up   grid (expert, row tile): an expert with no pairs exits at once;
//                otherwise its tokens' activation rows are staged in LDS (up to 4 at a
//                time) and one pass over the tile's rows serves all of them (same
//                per-row arithmetic as the dense one-row call).  The 2f gate and up rows
//                run as separate rows: hidden[position][0..2f) = gate sums, up sums.
//   3. down      grid (expert, row tile): the activation row of a position is
//                SiLU(gate) * up, formed from its hidden row while staging (hidden rows
//                of an expert's positions are contiguous); out[position][h].
//   4. combine   grid (token, 256 columns): y[t] = sum_j w[t][j] * out[pos(t, j)] in
//                slot order j = 0..k-1 (float32 fma chain, no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "gemv_core.h"
#include "q8_internal.h"
#include "q8_validate.h"

namespace q8k {

constexpr int kMoeThreads = 256;
constexpr int kMoeWaves = kMoeThreads / 64;
// Row groups each wave takes in one (expert, tile) unit: longer units amortize the
// per-unit staging and pipeline start; measured on the A3B layer, 8 suits the gate_up
// pass (2f rows of K = h) and 4 the down pass (h rows of K = f).
template <bool GATE_UP>
constexpr int moe_groups_per_wave() { return GATE_UP ? 8 : 4; }
constexpr int kMoeMaxRows = 4;        // activation rows staged per pass
// Route-plan block: 16 waves for many routed pairs; 4 for up to kPlanSmallPairs (decode,
// where the bigger block measured 9.8 against about 4 us on the A3B layer at 16 tokens).
constexpr int kPlanSmallPairs = 4096;

// ---------------------------------------------------------------- 1. route plan

// NW waves; wave w owns the contiguous pair segment [w*seg, (w+1)*seg) (seg a
// multiple of 64), so a stable order needs no block barrier inside the scatter:
//   a. each wave counts its segment's pairs per expert into its own LDS histogram row;
//   b. thread e sums expert e's row entries (the count) and turns them into exclusive
//      prefixes over the waves;
//   c. scans over the experts give offsets, the active-expert list and the first
//      matrix-core tile of each expert; every wave's running position for expert e
//      becomes offsets[e] + the count of e in the segments before it;
//   d. each wave walks its segment 64 pairs at a time (ids loaded 16 steps ahead in one
//      batch, as in a.): a pair's place is its wave's
//      running position for its expert plus the number of earlier lanes of the step
//      with the same expert (found with eight ballots, one per bit of the id, ids < 256);
//      the highest such lane advances the running position.
constexpr int kPlanBatch = 16;  // pair ids a lane loads at once

template <int kPlanWaves>
__global__ __launch_bounds__(64 * kPlanWaves) void moe_plan_kernel(const int32_t* __restrict__ idx, int n_pairs,
                                                                int n_exp, int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted,
                                                                int32_t* __restrict__ inv,
                                                                int32_t* __restrict__ active,
                                                                int32_t* __restrict__ tile_start) {
    __shared__ int run[kPlanWaves][q8v::kMaxExperts];  // per-wave counts, then running positions
    __shared__ int base_of[q8v::kMaxExperts];
    __shared__ int wave_total[kPlanWaves], wave_active[kPlanWaves], wave_tiles[kPlanWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    for (int x = tid; x < kPlanWaves * q8v::kMaxExperts; x += (64 * kPlanWaves)) (&run[0][0])[x] = 0;
    __syncthreads();
    const int seg = (n_pairs + 64 * kPlanWaves - 1) / (64 * kPlanWaves) * 64;
    const int s0 = wv * seg;
    const int s1 = s0 + seg < n_pairs ? s0 + seg : n_pairs;
    // the segment's expert ids, kPlanBatch per lane at a time (all loads issued together):
    // id j of batch bb is pair bb + 64 j + lane; -1 past the segment or out of range
    auto load_batch = [&](int bb, int (&ids)[kPlanBatch]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPlanBatch; ++j) {
            const int i = bb + 64 * j + lane;
            const int e = i < s1 ? idx[i] : -1;
            ids[j] = (e >= 0 && e < n_exp) ? e : -1;
        }
    };
    // a. per-wave histogram (LDS atomics on the wave's own row)
    for (int bb = s0; bb < s1; bb += 64 * kPlanBatch) {
        int ids[kPlanBatch];
        load_batch(bb, ids);
#pragma unroll
        for (int j = 0; j < kPlanBatch; ++j)
            if (ids[j] >= 0) atomicAdd(&run[wv][ids[j]], 1);
    }
    __syncthreads();
    // b. thread e: count of expert e, per-wave exclusive prefixes
    int c = 0;
    if (tid < n_exp) {
        for (int w = 0; w < kPlanWaves; ++w) {
            const int v = run[w][tid];
            run[w][tid] = c;
            c += v;
        }
    }
    // c. exclusive scans over the experts (thread e holds expert e; n_exp <= 256 <= threads):
    // a shuffle scan per wave, then the totals of the waves before it
    auto wave_incl = [&](int v) {
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off, 64);
            if (lane >= off) v += u;
        }
        return v;
    };
    const int incl = wave_incl(c);
    const int has = c > 0 ? 1 : 0;
    const int aincl = wave_incl(has);
    const int nt = (c + 127) / 128;  // 128-row matrix-core tiles of the expert
    const int tincl = wave_incl(nt);
    if (lane == 63) {
        wave_total[wv] = incl;
        wave_active[wv] = aincl;
        wave_tiles[wv] = tincl;
    }
    __syncthreads();
    int base = 0, abase = 0, tbase = 0;
    for (int w = 0; w < wv; ++w) {
        base += wave_total[w];
        abase += wave_active[w];
        tbase += wave_tiles[w];
    }
    const int excl = base + incl - c;
    if (tid < n_exp) {
        base_of[tid] = excl;
        offsets[tid] = excl;
        tile_start[tid] = tbase + tincl - nt;
    }
    if (tid == n_exp - 1) {
        offsets[n_exp] = excl + c;
        tile_start[n_exp] = tbase + tincl;
    }
    // the experts with pairs, in expert order, and their number at active[n_exp]
    if (has) active[abase + aincl - 1] = tid;
    if (tid == (64 * kPlanWaves) - 1) active[n_exp] = abase + aincl;
    __syncthreads();
    for (int x = tid; x < kPlanWaves * n_exp; x += (64 * kPlanWaves)) {
        const int w = x / n_exp, e = x - w * n_exp;
        run[w][e] += base_of[e];
    }
    __syncthreads();
    // d. stable scatter of the wave's segment
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int bb = s0; bb < s1; bb += 64 * kPlanBatch) {
        int ids[kPlanBatch];
        load_batch(bb, ids);
#pragma unroll
        for (int j = 0; j < kPlanBatch; ++j) {
            const int i = bb + 64 * j + lane;
            const int e = ids[j];
            uint64_t same = __ballot(e >= 0);
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) {
                const uint64_t set = __ballot(e >= 0 && ((e >> bit) & 1));
                same &= ((e >> bit) & 1) ? set : ~set;
            }
            const int pos = e >= 0 ? run[wv][e] + __popcll(same & below) : -1;
            if (i < s1) {
                inv[i] = pos;
                if (pos >= 0) sorted[pos] = i;
            }
            if (e >= 0 && (same >> lane) == 1ull) run[wv][e] = pos + 1;  // the group's highest lane
        }
    }
}

// ------------------------------------------------------- 2./3. expert GEMV passes

// Activation access: the 4 values of activation row m at k = 64*p + 4*c .. +3.
// LDS copy in slot-major order: float4 index ((m*16 + c) * P + p), so the lanes of a
// wave (consecutive p) read consecutive 16-byte vectors.
struct XLds {
    const float4* base;
    int P;
    __device__ __forceinline__ float4 get(int m, int p, int c) const { return base[(m * 16 + c) * P + p]; }
};
// One wave walks row groups first, first+stride, ... < end (G = 64/S rows each) of a
// Q8_0 matrix (the lane layout and order of gemv_core.h).  For R = 2 the lane also multiplies row n + r_off (gate/up pairs).
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


// One pass of the experts' rows, one row per lane group (the lane layout and per-row
// order of the one-row dense kernel: S lanes per row, lane j takes the pairs j, j + S,
// ..., block chains in mac_pair, then the xor butterfly).
// GATE_UP: the rows are the 2f gate and up rows of the expert, the activation rows the
//          tokens' x rows (x[sorted[pos] / k]); out[pos][n] for n < 2f.
// else (down): the activation row of position pos is SiLU(gate) * up of that position's
//          gate_up output (row pos of `x`, gate in [0, ldx/2), up in [ldx/2, ldx)),
//          formed while staging; out[pos][n] for n < h.
// Computing the gate and up rows as separate rows keeps one weight row per lane (the
// fused two-row form needs twice the registers); SiLU(gate) * up is formed from the
// same two row sums, with the same function, as in the dense fused call.
// ONE_ROUND: every row fits the S lanes of its group once (P <= S), so the per-item
// indexing needs no division.
template <bool GATE_UP, bool ONE_ROUND>
__global__ __launch_bounds__(kMoeThreads) void moe_expert_kernel(const uint8_t* __restrict__ w_stack,
                                                                 size_t expert_bytes, int n_out, int P, int log2S,
                                                                 const float* __restrict__ x, int ldx,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ sorted,
                                                                 const int32_t* __restrict__ active, int n_exp,
                                                                 int k, float* __restrict__ out, int ldo,
                                                                 int rows_per_pass, int tiles) {
    extern __shared__ float4 x_lds[];
    const int G = 64 >> log2S;
    const int row_groups = (n_out + G - 1) / G;
    const int tile_groups = kMoeWaves * moe_groups_per_wave<GATE_UP>();
    const int wave = threadIdx.x >> 6;
    const XLds xs{x_lds, P};
    const int k4 = P * 16;  // float4 per activation row
    // units (active expert, row tile), expert-major, over a grid of resident blocks
    const int units = active[n_exp] * tiles;
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int e = active[u / tiles];
        const int tile = u - (u / tiles) * tiles;
        const int pos0 = offsets[e];
        const int cnt = offsets[e + 1] - pos0;
        const uint8_t* w = w_stack + (size_t)e * expert_bytes;
        const int g_begin = tile * tile_groups;
        const int g_end = min(row_groups, g_begin + tile_groups);
        for (int c0 = 0; c0 < cnt; c0 += rows_per_pass) {
            const int cc = min(rows_per_pass, cnt - c0);
            const int mt = cc <= 1 ? 1 : cc <= 2 ? 2 : 4;
            // activation rows of this pass: the row addresses first (one load each, the
            // same for every thread), then the row loads, then LDS (slot-major)
            const float* rowp[kMoeMaxRows];
#pragma unroll
            for (int m = 0; m < kMoeMaxRows; ++m) {
                const int pos = pos0 + c0 + (m < cc ? m : 0);
                if constexpr (GATE_UP)
                    rowp[m] = x + (size_t)(sorted[pos] / k) * ldx;
                else
                    rowp[m] = x + (size_t)pos * ldx;
            }
#pragma unroll
            for (int m = 0; m < kMoeMaxRows; ++m) {
                if (m < mt) {
                    for (int i = threadIdx.x; i < k4; i += kMoeThreads) {
                        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                        if (m < cc) {
                            if constexpr (GATE_UP) {
                                v = *reinterpret_cast<const float4*>(rowp[m] + 4 * i);
                            } else {
                                const float4 gt = *reinterpret_cast<const float4*>(rowp[m] + 4 * i);
                                const float4 up = *reinterpret_cast<const float4*>(rowp[m] + (ldx >> 1) + 4 * i);
                                v = make_float4(silu_mul(gt.x, up.x), silu_mul(gt.y, up.y), silu_mul(gt.z, up.z),
                                                silu_mul(gt.w, up.w));
                            }
                        }
                        x_lds[(m * 16 + (i & 15)) * P + (i >> 4)] = v;
                    }
                }
            }
            __syncthreads();
            float* o = out + (size_t)(pos0 + c0) * ldo;
            auto run = [&](auto mtag) {
                constexpr int MT = decltype(mtag)::value;
                wave_rows<MT, 1, ONE_ROUND ? 1 : 0>(w, n_out, n_out, P, log2S, xs, g_begin + wave, kMoeWaves, g_end,
                                 [&](int n, const float(&acc)[1][MT]) {
#pragma unroll
                                     for (int m = 0; m < MT; ++m)
                                         if (m < cc) o[(size_t)m * ldo + n] = acc[0][m];
                                 });
            };
            if (mt == 1)
                run(std::integral_constant<int, 1>{});
            else if (mt == 2)
                run(std::integral_constant<int, 2>{});
            else
                run(std::integral_constant<int, 4>{});
            __syncthreads();  // the next pass or unit overwrites the staged rows
        }
    }
}

// ------------------------------------------------------------------ 4. combine

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ o, int h,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ wts, int k,
                                                          float* __restrict__ y, int ldy) {
    // block (token t, 256 columns): each thread one column, the k slot loads issued
    // together, then the fma chain in slot order
    const int t = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= h) return;
    float acc = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        float v[8], wj[8];
        bool use[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = j0 + jj < k ? j0 + jj : k - 1;
            const int pos = inv[(size_t)t * k + j];
            use[jj] = j0 + jj < k && pos >= 0;  // a skipped expert id contributes nothing
            wj[jj] = wts[(size_t)t * k + j];
            v[jj] = o[(size_t)(pos >= 0 ? pos : 0) * h + c];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            if (use[jj]) acc = __builtin_fmaf(wj[jj], v[jj], acc);
    }
    y[(size_t)t * ldy + c] = acc;
}

// ------------------------------------------------------------------- launcher

// Activation rows staged per pass: the largest power of two <= 4 whose rows fit in
// 64 KB of LDS (a row of K floats takes P*256 bytes).
static int staged_rows(int P) {
    int rows = kMoeMaxRows;
    while (rows > 1 && (size_t)rows * P * 256 > 65536) rows >>= 1;
    return rows;
}

// Blocks of moe_expert_kernel resident per CU for an LDS size (queried once per size).
template <bool GATE_UP, bool ONE_ROUND>
static int moe_blocks_per_cu(size_t lds) {
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int per_cu = 1;
    if (cached_lds != lds) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, moe_expert_kernel<GATE_UP, ONE_ROUND>, kMoeThreads, lds) !=
                hipSuccess ||
            n < 1)
            n = 1;
        per_cu = n;
        cached_lds = lds;
    }
    return per_cu;
}

template <bool GATE_UP, bool ONE_ROUND>
static hipError_t launch_expert_pass(const DeviceInfo& dev, const uint8_t* w, size_t expert_bytes, int rows_out,
                                     int P, int log2S, const float* x, int ldx, const int32_t* offsets,
                                     const int32_t* sorted, const int32_t* active, int n_exp, int k, float* out,
                                     int ldo, int rows, int tiles, size_t lds, hipStream_t stream) {
    const int64_t max_units = n_exp * (int64_t)tiles;
    const int64_t slots = (int64_t)dev.cu_count * moe_blocks_per_cu<GATE_UP, ONE_ROUND>(lds);
    const unsigned grid = (unsigned)(max_units < slots ? max_units : slots);
    hipLaunchKernelGGL((moe_expert_kernel<GATE_UP, ONE_ROUND>), dim3(grid), dim3(kMoeThreads), lds, stream, w,
                       expert_bytes, rows_out, P, log2S, x, ldx, offsets, sorted, active, n_exp, k, out, ldo, rows,
                       tiles);
    return hipGetLastError();
}

hipError_t launch_moe_grouped(const DeviceInfo& dev, const uint8_t* wgu, const uint8_t* wdn, int64_t n_exp, int64_t f,
                              int64_t h, const float* x, int64_t m, int64_t ldx, const int32_t* idx, const float* wts,
                              int k, float* y, int64_t ldy, void* workspace, hipStream_t stream) {
    const q8v::MoeWorkspace L = q8v::moe_workspace_layout(m, k, n_exp, f, h);
    char* ws = static_cast<char*>(workspace);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets_off);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted_off);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv_off);
    int32_t* active = reinterpret_cast<int32_t*>(ws + L.active_off);
    float* hidden = reinterpret_cast<float*>(ws + L.hidden_off);
    float* outp = reinterpret_cast<float*>(ws + L.out_off);
    const int n_pairs = (int)(m * k);

    int32_t* tile_start = reinterpret_cast<int32_t*>(ws + L.tiles_off);
    if (n_pairs <= kPlanSmallPairs)
        hipLaunchKernelGGL(moe_plan_kernel<4>, dim3(1), dim3(256), 0, stream, idx, n_pairs, (int)n_exp, offsets,
                           sorted, inv, active, tile_start);
    else
        hipLaunchKernelGGL(moe_plan_kernel<16>, dim3(1), dim3(1024), 0, stream, idx, n_pairs, (int)n_exp, offsets,
                           sorted, inv, active, tile_start);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (q8v::moe_uses_matrix_cores(n_pairs, n_exp)) {
        // Prefill: expert-grouped bf16 matrix-core tiles.  gate_up (K = h) writes
        // SiLU(gate) * up straight into hidden [pairs][f]; down (K = f) reads it and writes
        // the per-pair outputs; the grid covers the largest possible tile list.
        const int64_t max_tiles = (n_pairs + 127) / 128 + n_exp;
        e = launch_gemm_q8_mfma_grouped(wgu, (size_t)(2 * f) * (size_t)(h / 32) * 34, f, h, true, x, ldx, hidden, f,
                                        offsets, tile_start, sorted, (int)n_exp, k, true, max_tiles, stream);
        if (e != hipSuccess) return e;
        e = launch_gemm_q8_mfma_grouped(wdn, (size_t)h * (size_t)(f / 32) * 34, h, f, false, hidden, f, outp, h,
                                        offsets, tile_start, sorted, (int)n_exp, k, false, max_tiles, stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)m, (unsigned)((h + 255) / 256)), dim3(256), 0, stream,
                           outp, (int)h, inv, wts, k, y, (int)ldy);
        return hipGetLastError();
    }

    // gate_up: K = h, the 2f gate and up rows of each expert as separate rows; down: K = f,
    // rows h per expert, activation row of a position = SiLU(gate) * up of its gate_up
    // output (hidden rows are contiguous per expert).  Persistent grids of resident
    // blocks walk the (active expert, row tile) units.
    for (int pass = 0; pass < 2; ++pass) {
        const bool gate_up = pass == 0;
        const int K = (int)(gate_up ? h : f);
        const int rows_out = (int)(gate_up ? 2 * f : h);
        const int P = K / 64;
        const int log2S = slots_log2(P);
        const int G = 64 >> log2S;
        const int groups = (rows_out + G - 1) / G;
        const int tile_groups = kMoeWaves * (gate_up ? moe_groups_per_wave<true>() : moe_groups_per_wave<false>());
        const int tiles = (groups + tile_groups - 1) / tile_groups;
        const int rows = staged_rows(P);
        const size_t lds = (size_t)rows * P * 256;
        const size_t expert_bytes = (size_t)rows_out * (size_t)(K / 32) * 34;
        const bool one = P <= (1 << log2S);
        if (gate_up)
            e = one ? launch_expert_pass<true, true>(dev, wgu, expert_bytes, rows_out, P, log2S, x, (int)ldx, offsets,
                                                     sorted, active, (int)n_exp, k, hidden, (int)(2 * f), rows, tiles,
                                                     lds, stream)
                    : launch_expert_pass<true, false>(dev, wgu, expert_bytes, rows_out, P, log2S, x, (int)ldx, offsets,
                                                      sorted, active, (int)n_exp, k, hidden, (int)(2 * f), rows, tiles,
                                                      lds, stream);
        else
            e = one ? launch_expert_pass<false, true>(dev, wdn, expert_bytes, rows_out, P, log2S, hidden, (int)(2 * f),
                                                      offsets, sorted, active, (int)n_exp, k, outp, (int)h, rows, tiles,
                                                      lds, stream)
                    : launch_expert_pass<false, false>(dev, wdn, expert_bytes, rows_out, P, log2S, hidden,
                                                       (int)(2 * f), offsets, sorted, active, (int)n_exp, k, outp,
                                                       (int)h, rows, tiles, lds, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)m, (unsigned)((h + 255) / 256)), dim3(256), 0, stream, outp,
                       (int)h, inv, wts, k, y, (int)ldy);
    return hipGetLastError();
}

}  // namespace q8k
