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
#include "q8_internal.h"

namespace q8k {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxXLdsBytes = 64 * 1024;

template <int M, int R, bool XL>
__global__ __launch_bounds__(kThreads) void gemv_q8_kernel(const uint8_t* __restrict__ w, int n_out, int P, int log2S,
                                                           const float* __restrict__ x, int ldx,
                                                           float* __restrict__ y, int ldy) {
    extern __shared__ float4 x_lds[];
    typename std::conditional<XL, XLds, XGlobal>::type xs;
    if constexpr (XL) {
        stage_x_lds(x_lds, M, P, [&](int m) { return x + (size_t)m * ldx; }, threadIdx.x, kThreads);
        __syncthreads();
        xs.base = x_lds;
        xs.P = P;
    } else {
        xs.x = x;
        xs.ldx = ldx;
    }
    const int G = 64 >> log2S;
    const int row_groups = (n_out + G - 1) / G;
    const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6);
    wave_rows<M, R>(w, n_out, n_out, P, log2S, xs, gw, gridDim.x * kWaves, row_groups,
                    [&](int n, const float(&acc)[R][M]) {
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            if constexpr (R == 2)
                                y[(size_t)m * ldy + n] = silu_mul(acc[0][m], acc[1][m]);
                            else
                                y[(size_t)m * ldy + n] = acc[0][m];
                        }
                    });
}

// Activation rows held in registers (M <= 2).  Each lane keeps the 64*M activation
// values of every pair slot it owns (NR rounds) for the whole kernel, so the hot loop
// reads no LDS.  Weights stream through a ring of D register buffers: the loads of
// item it+D-1 are in flight while item it is multiplied.  Same per-output summation
// order as wave_rows (slot chain over rounds, then the butterfly).
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

template <int M, int R, int NR, int D>
__global__ __launch_bounds__(kThreads) void gemv_xreg_kernel(const uint8_t* __restrict__ w, int n_out, int P, int log2S,
                                                             const float* __restrict__ x, int ldx,
                                                             float* __restrict__ y, int ldy) {
    static_assert(D % NR == 0, "the ring depth must be a multiple of the rounds per row");
    const int S = 1 << log2S;
    const int G = 64 >> log2S;
    const int lane = threadIdx.x & 63;
    const int j = lane & (S - 1);
    const int g = lane >> log2S;
    const size_t row_bytes = (size_t)P * 68;

    const int row_groups = (n_out + G - 1) / G;
    const int stride = gridDim.x * kWaves;
    const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (gw >= row_groups) return;

    float4 xr[NR][M][16];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int p = j + S * i;
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int c = 0; c < 16; ++c)
                xr[i][m][c] = p < P ? *reinterpret_cast<const float4*>(x + (size_t)m * ldx + 64 * p + 4 * c)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int n_items = ((row_groups - 1 - gw) / stride + 1) * NR;
    auto item_n = [&](int it) { return (gw + (it / NR) * stride) * G + g; };
    auto load_item = [&](int it, uint32_t(&wr)[R][17]) {
        const int n = item_n(it);
        const int p = j + S * (it % NR);
        if (n < n_out && p < P) {
#pragma unroll
            for (int r = 0; r < R; ++r) load_pair(w + (size_t)(n + r * n_out) * row_bytes + 68 * (size_t)p, wr[r]);
        }
    };

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    uint32_t ring[D][R][17];
#pragma unroll
    for (int s = 0; s < D - 1; ++s)
        if (s < n_items) load_item(s, ring[s]);

    for (int it0 = 0; it0 < n_items; it0 += D) {
        static_for<D>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int i = s % NR;
            const int it = it0 + s;
            if (it < n_items) {
                if (it + D - 1 < n_items) load_item(it + D - 1, ring[(s + D - 1) % D]);
                const int n = item_n(it);
                const int p = j + S * i;
                if (n < n_out && p < P) mac_pair<M, R>(ring[s], XArr<M>{xr[i]}, p, acc);
                if constexpr (i == NR - 1) {
                    for (int off = S >> 1; off >= 1; off >>= 1) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int m = 0; m < M; ++m) acc[r][m] += __shfl_xor(acc[r][m], off, 64);
                    }
                    if (j == 0 && n < n_out) {
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            if constexpr (R == 2)
                                y[(size_t)m * ldy + n] = silu_mul(acc[0][m], acc[1][m]);
                            else
                                y[(size_t)m * ldy + n] = acc[0][m];
                        }
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
                }
            }
        });
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

template <int M, int R, bool XL>
hipError_t launch_one(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                      float* y, int ldy, hipStream_t stream) {
    const size_t lds = XL ? (size_t)M * P * 256 : 0;
    const int G = 64 >> log2S;
    static thread_local int cached_lds_P = -1, cached_per_cu = 1;
    if (cached_lds_P != (int)lds) {
        cached_per_cu = resident_blocks(gemv_q8_kernel<M, R, XL>, lds);
        cached_lds_P = (int)lds;
    }
    const int blocks = grid_for(dev, cached_per_cu, (n_out + G - 1) / G);
    hipLaunchKernelGGL((gemv_q8_kernel<M, R, XL>), dim3(blocks), dim3(kThreads), lds, stream, w, n_out, P, log2S, x,
                       ldx, y, ldy);
    return hipGetLastError();
}

template <int M, int R, int NR, int D>
hipError_t launch_xreg(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                       float* y, int ldy, hipStream_t stream) {
    static const int per_cu = resident_blocks(gemv_xreg_kernel<M, R, NR, D>, 0);
    const int G = 64 >> log2S;
    const int blocks = grid_for(dev, per_cu, (n_out + G - 1) / G);
    hipLaunchKernelGGL((gemv_xreg_kernel<M, R, NR, D>), dim3(blocks), dim3(kThreads), 0, stream, w, n_out, P, log2S,
                       x, ldx, y, ldy);
    return hipGetLastError();
}

// Register-resident activations for one row and at most 4 pair rounds per lane
// (K <= 16384); the ring depth is a multiple of the rounds.
template <int M, int R>
bool try_xreg_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
              float* y, int ldy, hipStream_t stream, hipError_t* err) {
    const int S = 1 << log2S;
    const int NR = (P + S - 1) / S;
    switch (NR) {
        case 1: *err = launch_xreg<M, R, 1, (R == 1 ? 4 : 3)>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        case 2: *err = launch_xreg<M, R, 2, (R == 1 ? 4 : 2)>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        case 3: *err = launch_xreg<M, R, 3, 3>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        case 4: *err = launch_xreg<M, R, 4, 4>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream); return true;
        default: return false;
    }
}

template <int M, int R>
hipError_t launch_m(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                    float* y, int ldy, hipStream_t stream) {
    if constexpr (M == 1) {
        hipError_t e;
        if (try_xreg_m<1, R>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream, &e)) return e;
    }
    if constexpr (M == 2) {
        // 128 registers of activations per round: one round only (K <= 64 * lanes per row)
        if ((P + (1 << log2S) - 1) >> log2S == 1)
            return launch_xreg<2, R, 1, (R == 1 ? 4 : 3)>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
    }
    if ((size_t)M * P * 256 <= (size_t)kMaxXLdsBytes)
        return launch_one<M, R, true>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
    return launch_one<M, R, false>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
}

template <int R>
hipError_t launch_r(const DeviceInfo& dev, const uint8_t* w, int n_out, int P, int log2S, const float* x, int ldx,
                    int m, float* y, int ldy, hipStream_t stream) {
    switch (m) {
#define Q8_CASE(MM) \
    case MM: return launch_m<MM, R>(dev, w, n_out, P, log2S, x, ldx, y, ldy, stream);
        Q8_CASE(1) Q8_CASE(2) Q8_CASE(3) Q8_CASE(4) Q8_CASE(5) Q8_CASE(6) Q8_CASE(7) Q8_CASE(8)
        Q8_CASE(9) Q8_CASE(10) Q8_CASE(11) Q8_CASE(12) Q8_CASE(13) Q8_CASE(14) Q8_CASE(15) Q8_CASE(16)
#undef Q8_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv_q8(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                          const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream) {
    const int P = (int)(k / 64);
    const int log2S = slots_log2(P);
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mm = (int)((m - m0) < 16 ? (m - m0) : 16);
        const float* xc = x + m0 * ldx;
        float* yc = y + m0 * ldy;
        hipError_t e = silu_pairs ? launch_r<2>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream)
                                  : launch_r<1>(dev, w, (int)n_out, P, log2S, xc, (int)ldx, mm, yc, (int)ldy, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q8k
