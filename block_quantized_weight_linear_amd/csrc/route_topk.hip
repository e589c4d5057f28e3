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

#include "q8_internal.h"

namespace q8k {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteBatch = 4;  // experts a wave multiplies together
constexpr int kMaxExperts = 256;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
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

    // Each lane owns experts lane, lane+64, lane+128, lane+192.
    float l[4];
    int taken = 0;  // bit c: expert lane + 64c already selected
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        l[c] = e < n_exp ? logits[e] : -INFINITY;
        if (e >= n_exp) taken |= 1 << c;
    }
    float mx = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float ex[4];
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        ex[c] = (lane + 64 * c < n_exp) ? expf(l[c] - mx) : 0.0f;
        sum += ex[c];
    }
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const float inv_sum = 1.0f / sum;

    // k rounds; after each butterfly every lane holds the winner.  Lane (j % 64) keeps
    // round j's result in its register slot j / 64; the sum of the chosen
    // probabilities is accumulated in selection order, identically on all lanes.
    int keep_i[4] = {0, 0, 0, 0};
    float keep_p[4] = {0.f, 0.f, 0.f, 0.f};
    float keep_cb[4] = {0.f, 0.f, 0.f, 0.f};  // running sum before the slot
    float keep_ca[4] = {0.f, 0.f, 0.f, 0.f};  // running sum through the slot
    float psum = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        float bp = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = lane + 64 * c;
            if (!(taken & (1 << c)) && (bi == 0x7fffffff || better(l[c], e, bv, bi))) {
                bv = l[c];
                bi = e;
                bp = ex[c];
            }
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            const float op = __shfl_xor(bp, off, 64);
            if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
                bp = op;
            }
        }
        if ((bi & 63) == lane) taken |= 1 << (bi >> 6);
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
    for (int off = 32; off >= 1; off >>= 1) ksum = fmaxf(ksum, __shfl_xor(ksum, off, 64));
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

hipError_t launch_route_topk(const DeviceInfo&, const float* x, int64_t m, int64_t h, int64_t ldx,
                             const float* w_router, int64_t n_exp, int k, bool normalize, float top_p, int32_t* idx,
                             float* wts, hipStream_t stream) {
    hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)m), dim3(kRouteThreads), 0, stream, x, (int)h, (int)ldx,
                       w_router, (int)n_exp, k, normalize ? 1 : 0, top_p, idx, wts);
    return hipGetLastError();
}

}  // namespace q8k
