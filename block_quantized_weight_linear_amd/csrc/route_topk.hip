// Softmax top-k MoE router on the device (gfx950).
//
// "14. Model families and example applications" section 14.2: the MoE FFN routes with
// routerTopK (normalize_selected = norm_topk_prob); the engine does that on the host,
// here it stays on the device so the mixture can follow without a host round trip.
//
// One workgroup (16 waves) per token.  Logits: each wave takes experts e = wave,
// wave+16, ..., four at a time so that many loads are in flight; a lane multiplies
// float4 slices k = 4*lane + 256*i (i ascending) and the wave sums its 64 partials with
// a fixed xor-butterfly (float32 throughout).  Softmax and selection run on wave 0: the
// row maximum is subtracted before exp, and the k experts are picked one by one as the
// largest remaining logit, ties to the lower expert index (selecting on the logits
// avoids ties that rounding exp() could create; softmax is monotonic, so the order is
// that of the probabilities).  The chosen probabilities are divided by their sum, taken
// in selection order, when normalize is set.
//
// Adaptive expert top-p (the Config knob moe_expert_top_p of section 14.2; 1.0 = full
// top-k): with c_j the running sum of the chosen probabilities through slot j (float32,
// selection order) and S the sum over all k, slot 0 is kept and slot j >= 1 while
// c_{j-1} < top_p * S; top_p >= 1 keeps all k.  Kept weights are divided by the kept sum
// when normalize is set; a dropped slot gets expert -1 and weight 0.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "lds_dma.h"
#include "q8_internal.h"

namespace q8k {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteBatch = 4;  // experts a wave multiplies together
constexpr int kMaxExperts = 256;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// Cross-lane steps on the DPP network (no LDS round trip): within each row of 16 lanes,
// xor 1 and xor 2 (quad permutes), then the half-row and row mirrors; the four rows are
// then combined from lanes 0, 16, 32, 48 with readlane, in row order.
constexpr int kDppXor1 = 0xB1;        // quad_perm(1, 0, 3, 2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    const int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Every lane gets the wave's best (value, index) under better().
__device__ __forceinline__ void wave_best(float& v, int& i) {
    auto step = [&](auto c) __attribute__((always_inline)) {
        constexpr int C = decltype(c)::value;
        const float ov = dpp_f<C>(v);
        const int oi = dpp_i<C>(i);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    };
    step(std::integral_constant<int, kDppXor1>{});
    step(std::integral_constant<int, kDppXor2>{});
    step(std::integral_constant<int, kDppHalfMirror>{});
    step(std::integral_constant<int, kDppMirror>{});
    float bv = lane_f(v, 0);
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = lane_f(v, 16 * r);
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (better(rv, ri, bv, bi)) {
            bv = rv;
            bi = ri;
        }
    }
    v = bv;
    i = bi;
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Fixed order: the DPP tree within each row, then ((row0 + row1) + row2) + row3.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}

// Softmax, top-k selection and the top-p cut for one token on one wave; logit_of(e)
// returns expert e's float32 logit (e < n_exp).  Lane l owns experts l, l+64, l+128, l+192.
template <class LogitOf>
__device__ __forceinline__ void select_topk(LogitOf&& logit_of, int lane, int tok, int n_exp, int k, int normalize,
                                            float top_p, int32_t* __restrict__ out_idx,
                                            float* __restrict__ out_w) {
    float l[4];
    int taken = 0;  // bit c: expert lane + 64c already selected
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        l[c] = e < n_exp ? logit_of(e) : -INFINITY;
        if (e >= n_exp) taken |= 1 << c;
    }
    const float mx = wave_max(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
    float ex[4];
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        ex[c] = (lane + 64 * c < n_exp) ? expf(l[c] - mx) : 0.0f;
        part += ex[c];
    }
    const float inv_sum = 1.0f / wave_sum(part);

    // k rounds; each picks the wave's best untaken expert (every lane learns it) and the
    // owner lane's probability by readlane.  Lane (j % 64) keeps round j's result in its
    // register slot j / 64; the chosen probabilities are summed in selection order,
    // identically on all lanes.
    int keep_i[4] = {0, 0, 0, 0};
    float keep_p[4] = {0.f, 0.f, 0.f, 0.f};
    float keep_cb[4] = {0.f, 0.f, 0.f, 0.f};  // running sum before the slot
    float keep_ca[4] = {0.f, 0.f, 0.f, 0.f};  // running sum through the slot
    float psum = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = lane + 64 * c;
            if (!(taken & (1 << c)) && better(l[c], e, bv, bi)) {
                bv = l[c];
                bi = e;
            }
        }
        wave_best(bv, bi);
        const int wl = bi & 63, wc = bi >> 6;
        const float mine = wc == 0 ? ex[0] : wc == 1 ? ex[1] : wc == 2 ? ex[2] : ex[3];
        const float bp = lane_f(mine, wl);
        if (lane == wl) taken |= 1 << wc;
        const float p = bp * inv_sum;
        const float before = psum;
        psum += p;
        if ((j & 63) == lane) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if ((j >> 6) == c) {
                    keep_i[c] = bi;
                    keep_p[c] = p;
                    keep_cb[c] = before;
                    keep_ca[c] = psum;
                }
            }
        }
    }
    // top-p cut: every lane holds the same running sums for its slots, so the kept sum is
    // the largest running sum through a kept slot (the sums only grow)
    const bool all = !(top_p < 1.0f);
    const float thr = top_p * psum;
    bool kept[4];
    float ksum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = lane + 64 * c;
        kept[c] = j < k && (all || j == 0 || keep_cb[c] < thr);
        if (kept[c]) ksum = fmaxf(ksum, keep_ca[c]);
    }
    ksum = wave_max(ksum);
    if (all) ksum = psum;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = lane + 64 * c;
        if (j < k) {
            out_idx[(size_t)tok * k + j] = kept[c] ? keep_i[c] : -1;
            out_w[(size_t)tok * k + j] = kept[c] ? (normalize ? keep_p[c] / ksum : keep_p[c]) : 0.0f;
        }
    }
}

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float* __restrict__ x, int h, int ldx,
                                                                   const float* __restrict__ wr, int n_exp, int k,
                                                                   int normalize, float top_p,
                                                                   int32_t* __restrict__ out_idx,
                                                                   float* __restrict__ out_w) {
    __shared__ float logits[kMaxExperts];
    const int tok = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const float* xr = x + (size_t)tok * ldx;

    for (int e0 = wave; e0 < n_exp; e0 += kRouteWaves * kRouteBatch) {
        // experts e0, e0 + 16, e0 + 32, e0 + 48 (past n_exp: expert e0 again, not stored)
        const float* we[kRouteBatch];
#pragma unroll
        for (int b = 0; b < kRouteBatch; ++b) {
            const int e = e0 + kRouteWaves * b;
            we[b] = wr + (size_t)(e < n_exp ? e : e0) * h;
        }
        float acc[kRouteBatch] = {0.0f, 0.0f, 0.0f, 0.0f};
        // chunks of 1024 inputs (h is a multiple of 256; a partial chunk clamps its
        // loads and skips the multiply): every load of a chunk is issued before its fmas
        for (int k0 = 0; k0 < h; k0 += 1024) {
            float4 a[4], v[kRouteBatch][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = k0 + 4 * lane + 256 * i;
                const int kc = kk < h ? kk : 4 * lane;
                a[i] = *reinterpret_cast<const float4*>(xr + kc);
#pragma unroll
                for (int b = 0; b < kRouteBatch; ++b) v[b][i] = *reinterpret_cast<const float4*>(we[b] + kc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (k0 + 256 * i < h) {
#pragma unroll
                    for (int b = 0; b < kRouteBatch; ++b) {
                        acc[b] = __builtin_fmaf(a[i].x, v[b][i].x, acc[b]);
                        acc[b] = __builtin_fmaf(a[i].y, v[b][i].y, acc[b]);
                        acc[b] = __builtin_fmaf(a[i].z, v[b][i].z, acc[b]);
                        acc[b] = __builtin_fmaf(a[i].w, v[b][i].w, acc[b]);
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kRouteBatch; ++b) {
            for (int off = 32; off >= 1; off >>= 1) acc[b] += __shfl_xor(acc[b], off, 64);
            const int e = e0 + kRouteWaves * b;
            if (lane == 0 && e < n_exp) logits[e] = acc[b];
        }
    }
    __syncthreads();
    if (wave != 0) return;
    select_topk([&](int e) { return logits[e]; }, lane, tok, n_exp, k, normalize, top_p, out_idx, out_w);
}

// Two-pass router for many experts or tokens: the logits of a token are spread over
// many CUs (one CU reading the whole router matrix per token is bound by its own L1
// rate), then one wave per token selects.  Pass 1: block (token group t, expert group
// g) stages the x rows of kLogitTokens tokens in LDS; wave w multiplies expert
// 4g + w against them with the same lane slices and butterfly as route_topk_kernel, so
// the logits, and everything selected from them, are bit-identical to the one-kernel
// router's.
constexpr int kLogitThreads = 256;
constexpr int kLogitTokens = 4;
constexpr int kLogitChunk = 2048;  // inputs staged per pass (h is split into such chunks)

__global__ __launch_bounds__(kLogitThreads) void route_logits_kernel(const float* __restrict__ x, int m, int h,
                                                                     int ldx, const float* __restrict__ wr,
                                                                     int n_exp, float* __restrict__ logits) {
    __shared__ float4 xs[kLogitTokens][kLogitChunk / 4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = blockIdx.y * 4 + wave;
    const int t0 = blockIdx.x * kLogitTokens;
    const int ec = e < n_exp ? e : n_exp - 1;  // a wave past the experts repeats the last one, not stored
    const float* we = wr + (size_t)ec * h;
    float acc[kLogitTokens] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < h; c0 += kLogitChunk) {
        const int len = h - c0 < kLogitChunk ? h - c0 : kLogitChunk;  // a multiple of 256
        __syncthreads();
        for (int i = threadIdx.x; i < kLogitTokens * (len / 4); i += kLogitThreads) {
            const int t = i / (len / 4);
            const int q = i - t * (len / 4);
            const int tc = t0 + t < m ? t0 + t : m - 1;
            xs[t][q] = *reinterpret_cast<const float4*>(x + (size_t)tc * ldx + c0 + 4 * q);
        }
        __syncthreads();
        for (int i = 0; i < len / 256; ++i) {
            const float4 v = *reinterpret_cast<const float4*>(we + c0 + 4 * lane + 256 * i);
#pragma unroll
            for (int t = 0; t < kLogitTokens; ++t) {
                const float4 a = xs[t][lane + 64 * i];
                acc[t] = __builtin_fmaf(a.x, v.x, acc[t]);
                acc[t] = __builtin_fmaf(a.y, v.y, acc[t]);
                acc[t] = __builtin_fmaf(a.z, v.z, acc[t]);
                acc[t] = __builtin_fmaf(a.w, v.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kLogitTokens; ++t) {
        for (int off = 32; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off, 64);
        if (lane == 0 && e < n_exp && t0 + t < m) logits[(size_t)(t0 + t) * n_exp + e] = acc[t];
    }
}

// Pass 1 for many tokens: block (token group, expert group) multiplies kTileTokens
// tokens by 32 experts (8 per wave), so each router row read from L2 serves 16 tokens and
// each staged activation value 8 experts (the 4-token form re-reads the router matrix
// once per 4 tokens).  Every logit keeps the lane slices and fma order of
// route_topk_kernel; its 64 lane partials are then summed by a transpose-reduce that
// pairs lanes exactly as the xor butterfly does (lane l with l ^ 32, then ^ 16, ..., ^ 1)
// while halving the values each lane carries at every step: a lane keeps the half whose
// index bit matches its own lane bit and trades the other half with its partner, so the
// 128 logits of a wave need 126 shuffles instead of 768 and come out as values 2l and
// 2l + 1 on lane l, bit-identical to the butterfly's sums.
constexpr int kTileTokens = 16;
// measured on the Qwen3-30B-A3B router (128 x 2048): the 4-token form takes 9.9 us at 192
// tokens and grows linearly; the tiles take 18.6 us at 256 tokens and 19.0 at 512
constexpr int kTiledLogitsMinTokens = 384;
constexpr int kTileExperts = 8;  // per wave
constexpr int kTileChunk = 1024;

__global__ __launch_bounds__(256) void route_logits_tiled_kernel(const float* __restrict__ x, int m, int h, int ldx,
                                                                 const float* __restrict__ wr, int n_exp,
                                                                 float* __restrict__ logits) {
    constexpr int T = kTileTokens, E = kTileExperts, NV = T * E;  // NV = 128 = 2 * 64
    __shared__ float4 xs[T][kTileChunk / 4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * T;
    const int e0 = (blockIdx.y * 4 + wave) * E;
    const float* we[E];
#pragma unroll
    for (int b = 0; b < E; ++b) {
        const int e = e0 + b;
        we[b] = wr + (size_t)(e < n_exp ? e : n_exp - 1) * h;  // past n_exp: not stored
    }
    float acc[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[j] = 0.0f;
    for (int c0 = 0; c0 < h; c0 += kTileChunk) {
        const int len = h - c0 < kTileChunk ? h - c0 : kTileChunk;  // a multiple of 256
        const int steps = len / 256;
        __syncthreads();  // every wave is done with the previous chunk
        // the chunk's activations: T * steps wave-wide direct-to-LDS copies of 1 KB
        // (copy q = token t, 256 inputs c), taken by the four waves in turn
        for (int q = wave; q < T * steps; q += 4) {
            const int t = q / steps, c = q - t * steps;
            const int tc = t0 + t < m ? t0 + t : m - 1;  // past m: the last token, not stored
            lds_copy16(x + (size_t)tc * ldx + c0 + 256 * c + 4 * lane, &xs[t][64 * c]);
        }
        float4 v[E];
#pragma unroll
        for (int b = 0; b < E; ++b) v[b] = *reinterpret_cast<const float4*>(we[b] + c0 + 4 * lane);
        wait_vmcnt_mem<0>();
        __syncthreads();
        for (int i = 0; i < steps; ++i) {
            // the router slices of the next step load while this one is multiplied
            float4 vn[E];
            const int ni = i + 1 < steps ? i + 1 : i;
#pragma unroll
            for (int b = 0; b < E; ++b) vn[b] = *reinterpret_cast<const float4*>(we[b] + c0 + 4 * lane + 256 * ni);
            float4 a = xs[0][lane + 64 * i];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float4 an = xs[t + 1 < T ? t + 1 : t][lane + 64 * i];  // read ahead
#pragma unroll
                for (int b = 0; b < E; ++b) {
                    float& r = acc[t * E + b];
                    r = __builtin_fmaf(a.x, v[b].x, r);
                    r = __builtin_fmaf(a.y, v[b].y, r);
                    r = __builtin_fmaf(a.z, v[b].z, r);
                    r = __builtin_fmaf(a.w, v[b].w, r);
                }
                a = an;
            }
#pragma unroll
            for (int b = 0; b < E; ++b) v[b] = vn[b];
        }
    }
    // transpose-reduce: at the step with offset `off` a lane holds n values; it keeps the
    // upper half if its lane bit `off` is set, else the lower half, and adds the
    // partner's copy of the half it keeps
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        const int off = 32 >> st;
        const int n = NV >> st;
        const bool up = (lane & off) != 0;
#pragma unroll
        for (int r = 0; r < n / 2; ++r) {
            const float keep = up ? acc[n / 2 + r] : acc[r];
            const float send = up ? acc[r] : acc[n / 2 + r];
            acc[r] = keep + __shfl_xor(send, off, 64);
        }
    }
    // lane l holds values j = 2l and 2l + 1, j = t * E + b
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j = 2 * lane + r;
        const int t = t0 + j / E;
        const int e = e0 + j % E;
        if (t < m && e < n_exp) logits[(size_t)t * n_exp + e] = acc[r];
    }
}

// Pass 2: one wave per token.
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ logits, int m, int n_exp, int k,
                                                           int normalize, float top_p,
                                                           int32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_w) {
    const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= m) return;
    const float* lg = logits + (size_t)tok * n_exp;
    select_topk([&](int e) { return lg[e]; }, threadIdx.x & 63, tok, n_exp, k, normalize, top_p, out_idx, out_w);
}

hipError_t launch_route_topk(const DeviceInfo&, const float* x, int64_t m, int64_t h, int64_t ldx,
                             const float* w_router, int64_t n_exp, int k, bool normalize, float top_p, int32_t* idx,
                             float* wts, float* logits, hipStream_t stream) {
    if (logits) {
        if (m >= kTiledLogitsMinTokens) {
            const dim3 grid((unsigned)((m + kTileTokens - 1) / kTileTokens),
                            (unsigned)((n_exp + 4 * kTileExperts - 1) / (4 * kTileExperts)));
            hipLaunchKernelGGL(route_logits_tiled_kernel, grid, dim3(256), 0, stream, x, (int)m, (int)h, (int)ldx,
                               w_router, (int)n_exp, logits);
        } else {
            const dim3 grid((unsigned)((m + kLogitTokens - 1) / kLogitTokens), (unsigned)((n_exp + 3) / 4));
            hipLaunchKernelGGL(route_logits_kernel, grid, dim3(kLogitThreads), 0, stream, x, (int)m, (int)h, (int)ldx,
                               w_router, (int)n_exp, logits);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(route_select_kernel, dim3((unsigned)((m + 3) / 4)), dim3(256), 0, stream, logits, (int)m,
                           (int)n_exp, k, normalize ? 1 : 0, top_p, idx, wts);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)m), dim3(kRouteThreads), 0, stream, x, (int)h, (int)ldx,
                       w_router, (int)n_exp, k, normalize ? 1 : 0, top_p, idx, wts);
    return hipGetLastError();
}

}  // namespace q8k
