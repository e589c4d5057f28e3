// Grouped Q8_0 SwiGLU expert mixture (gfx950).
//
// "14. Model families and example applications" section 14.2: the MoE FFN runs the
// router-weighted SwiGLU mixture (moeSwiGluFfnSeq); with several tokens it groups them
// by expert so each expert's weights are read once per batch.  Section 14.4 ("MoE
// expert kernels"): a counting-sort route plan scatters (token, slot) pairs
// expert-major, and each token's sum runs in a fixed order.
//
// Four launches on one stream, no host synchronization:
//   1. plan      one workgroup: counting sort of the m*k (token, slot) pairs by
//                expert, stable in pair order; offsets[e], sorted pair list, and the
//                inverse map pair -> position.
//   2. gate_up   grid (expert, row tile): an expert with no pairs exits at once;
//                otherwise its tokens' activation rows are staged in LDS (up to 8 at a
//                time) and one pass over the tile's gate/up rows serves all of them
//                (same per-row arithmetic as the dense fused gate_up call).  Output:
//                hidden[position][f] = SiLU(gate) * up.
//   3. down      grid (expert, row tile): hidden rows of the expert's positions are
//                contiguous; out[position][h] = W_down[e] . hidden[position].
//   4. combine   one workgroup per token: y[t] = sum_j w[t][j] * out[pos(t, j)] in slot
//                order j = 0..k-1 (float32 fma chain, no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv_core.h"
#include "q8_internal.h"
#include "q8_validate.h"

namespace q8k {

constexpr int kMoeThreads = 256;
constexpr int kMoeWaves = kMoeThreads / 64;
constexpr int kMoeGroupsPerWave = 4;  // row groups each wave takes in one tile
constexpr int kMoeMaxRows = 8;        // activation rows staged per pass
constexpr int kPlanThreads = 256;

// ---------------------------------------------------------------- 1. route plan

__global__ __launch_bounds__(kPlanThreads) void moe_plan_kernel(const int32_t* __restrict__ idx, int n_pairs,
                                                                int n_exp, int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted,
                                                                int32_t* __restrict__ inv) {
    __shared__ int counts[q8v::kMaxExperts + 1];
    __shared__ int running[q8v::kMaxExperts + 1];
    __shared__ int chunk_e[kPlanThreads];
    const int tid = threadIdx.x;
    for (int e = tid; e <= n_exp; e += kPlanThreads) counts[e] = 0;
    __syncthreads();
    for (int i = tid; i < n_pairs; i += kPlanThreads) {
        const int e = idx[i];
        if (e >= 0 && e < n_exp) atomicAdd(&counts[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int e = 0; e < n_exp; ++e) {
            running[e] = acc;
            offsets[e] = acc;
            acc += counts[e];
        }
        offsets[n_exp] = acc;
    }
    __syncthreads();
    // Stable scatter, one chunk of kPlanThreads pairs at a time: a pair's place is the
    // running count of its expert plus the number of earlier pairs of the chunk with
    // the same expert.
    for (int base = 0; base < n_pairs; base += kPlanThreads) {
        const int i = base + tid;
        int e = -1;
        if (i < n_pairs) {
            e = idx[i];
            if (e < 0 || e >= n_exp) e = -1;
        }
        chunk_e[tid] = e;
        __syncthreads();
        int rank = 0;
        bool last = true;
        if (e >= 0) {
            for (int t = 0; t < tid; ++t) rank += (chunk_e[t] == e);
            for (int t = tid + 1; t < kPlanThreads; ++t) last = last && (chunk_e[t] != e);
        }
        const int pos = (e >= 0) ? running[e] + rank : -1;
        if (i < n_pairs) {
            inv[i] = pos;
            if (pos >= 0) sorted[pos] = i;
        }
        __syncthreads();
        if (e >= 0 && last) running[e] = pos + 1;
        __syncthreads();
    }
}

// ------------------------------------------------------- 2./3. expert GEMV passes

// R = 2: gate_up (rows n and n + n_out, SiLU(gate)*up into `out`);  R = 1: down.
// GATHER: activation row i of the expert is x[sorted[pos] / k] (token rows); else it
// is row `pos` of x (the hidden rows, contiguous per expert).
template <int R, bool GATHER>
__global__ __launch_bounds__(kMoeThreads) void moe_expert_kernel(const uint8_t* __restrict__ w_stack,
                                                                 size_t expert_bytes, int n_out, int P, int log2S,
                                                                 const float* __restrict__ x, int ldx,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ sorted, int k,
                                                                 float* __restrict__ out, int ldo, int rows_per_pass) {
    extern __shared__ float4 x_lds[];
    const int e = blockIdx.x;
    const int pos0 = offsets[e];
    const int cnt = offsets[e + 1] - pos0;
    if (cnt == 0) return;
    const uint8_t* w = w_stack + (size_t)e * expert_bytes;
    const int G = 64 >> log2S;
    const int row_groups = (n_out + G - 1) / G;
    const int tile_groups = kMoeWaves * kMoeGroupsPerWave;
    const int g_begin = blockIdx.y * tile_groups;
    const int g_end = min(row_groups, g_begin + tile_groups);
    const int wave = threadIdx.x >> 6;
    const XLds xs{x_lds, P};

    for (int c0 = 0; c0 < cnt; c0 += rows_per_pass) {
        const int cc = min(rows_per_pass, cnt - c0);
        const int mt = cc <= 1 ? 1 : cc <= 2 ? 2 : cc <= 4 ? 4 : 8;
        stage_x_lds(x_lds, mt, P,
                    [&](int m) -> const float* {
                        if (m >= cc) return nullptr;
                        const int pos = pos0 + c0 + m;
                        if constexpr (GATHER)
                            return x + (size_t)(sorted[pos] / k) * ldx;
                        else
                            return x + (size_t)pos * ldx;
                    },
                    threadIdx.x, kMoeThreads);
        __syncthreads();
        float* o = out + (size_t)(pos0 + c0) * ldo;
        auto run = [&](auto mtag) {
            constexpr int MT = decltype(mtag)::value;
            wave_rows<MT, R>(w, n_out, n_out, P, log2S, xs, g_begin + wave, kMoeWaves, g_end,
                             [&](int n, const float(&acc)[R][MT]) {
#pragma unroll
                                 for (int m = 0; m < MT; ++m) {
                                     if (m < cc) {
                                         if constexpr (R == 2)
                                             o[(size_t)m * ldo + n] = silu_mul(acc[0][m], acc[1][m]);
                                         else
                                             o[(size_t)m * ldo + n] = acc[0][m];
                                     }
                                 }
                             });
        };
        if (mt == 1)
            run(std::integral_constant<int, 1>{});
        else if (mt == 2)
            run(std::integral_constant<int, 2>{});
        else if (mt == 4)
            run(std::integral_constant<int, 4>{});
        else
            run(std::integral_constant<int, 8>{});
        __syncthreads();
    }
}

// ------------------------------------------------------------------ 4. combine

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ o, int h,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ wts, int k,
                                                          float* __restrict__ y, int ldy) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x; c < h; c += blockDim.x) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int pos = inv[(size_t)t * k + j];
            if (pos >= 0) acc = __builtin_fmaf(wts[(size_t)t * k + j], o[(size_t)pos * h + c], acc);
        }
        y[(size_t)t * ldy + c] = acc;
    }
}

// ------------------------------------------------------------------- launcher

// Activation rows staged per pass: the largest power of two <= 8 whose rows fit in
// 64 KB of LDS (a row of K floats takes P*256 bytes).  Passes use 1, 2, 4 or 8 rows,
// never more than this.
static int staged_rows(int P) {
    int rows = kMoeMaxRows;
    while (rows > 1 && (size_t)rows * P * 256 > 65536) rows >>= 1;
    return rows;
}

hipError_t launch_moe_grouped(const DeviceInfo&, const uint8_t* wgu, const uint8_t* wdn, int64_t n_exp, int64_t f,
                              int64_t h, const float* x, int64_t m, int64_t ldx, const int32_t* idx, const float* wts,
                              int k, float* y, int64_t ldy, void* workspace, hipStream_t stream) {
    const q8v::MoeWorkspace L = q8v::moe_workspace_layout(m, k, n_exp, f, h);
    char* ws = static_cast<char*>(workspace);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets_off);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted_off);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv_off);
    float* hidden = reinterpret_cast<float*>(ws + L.hidden_off);
    float* outp = reinterpret_cast<float*>(ws + L.out_off);
    const int n_pairs = (int)(m * k);

    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, idx, n_pairs, (int)n_exp, offsets,
                       sorted, inv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // gate_up: K = h, rows 2f per expert
    {
        const int P = (int)(h / 64);
        const int log2S = slots_log2(P);
        const int G = 64 >> log2S;
        const int groups = ((int)f + G - 1) / G;
        const int tiles = (groups + kMoeWaves * kMoeGroupsPerWave - 1) / (kMoeWaves * kMoeGroupsPerWave);
        const int rows = staged_rows(P);
        const size_t lds = (size_t)rows * P * 256;
        const size_t expert_bytes = (size_t)(2 * f) * (size_t)(h / 32) * 34;
        hipLaunchKernelGGL((moe_expert_kernel<2, true>), dim3((unsigned)n_exp, (unsigned)tiles), dim3(kMoeThreads),
                           lds, stream, wgu, expert_bytes, (int)f, P, log2S, x, (int)ldx, offsets, sorted, k, hidden,
                           (int)f, rows);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // down: K = f, rows h per expert, activation rows = hidden (contiguous per expert)
    {
        const int P = (int)(f / 64);
        const int log2S = slots_log2(P);
        const int G = 64 >> log2S;
        const int groups = ((int)h + G - 1) / G;
        const int tiles = (groups + kMoeWaves * kMoeGroupsPerWave - 1) / (kMoeWaves * kMoeGroupsPerWave);
        const int rows = staged_rows(P);
        const size_t lds = (size_t)rows * P * 256;
        const size_t expert_bytes = (size_t)h * (size_t)(f / 32) * 34;
        hipLaunchKernelGGL((moe_expert_kernel<1, false>), dim3((unsigned)n_exp, (unsigned)tiles), dim3(kMoeThreads),
                           lds, stream, wdn, expert_bytes, (int)h, P, log2S, hidden, (int)f, offsets, sorted, k, outp,
                           (int)h, rows);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)m), dim3(256), 0, stream, outp, (int)h, inv, wts, k, y,
                       (int)ldy);
    return hipGetLastError();
}

}  // namespace q8k
