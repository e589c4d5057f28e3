// Internal launcher interface between the C ABI (q8_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q8k {

// Per-device facts the launchers size their grids with.
struct DeviceInfo {
    int device = -1;
    int cu_count = 0;
    size_t lds_per_block = 0;
};

// Returns the cached info of the current device (queried once per device).
hipError_t current_device_info(DeviceInfo* out);

// y[m][n] = x[m] . W[n]^T for m < 256 rows (float32 path, 8-row launches).  When silu_pairs is true,
// W has 2*n_out rows and the output is SiLU(gate) * up with gate row j, up row n_out+j.
hipError_t launch_gemv_q8(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                          const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

// GGUF Q4_0 weights (18-byte blocks), every m in 8-row launches of the float32 rows kernel.
hipError_t launch_gemv_q4_0(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

// GGUF Q4_K / Q5_K / Q6_K weights (144 / 176 / 210-byte super-blocks of 256), every m in 8-row
// launches of the float32 rows kernel.
hipError_t launch_gemv_q4_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);
hipError_t launch_gemv_q5_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);
hipError_t launch_gemv_q6_k(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                            const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

// Same contract for m >= 256 rows on the bf16 matrix cores (weights dequantized to bf16
// per tile, activations rounded to bf16, float32 accumulation and output).
hipError_t launch_gemm_q8_mfma(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                               const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

// Int8 activation codes and scales of float32 rows: xq [m][k], xd [m][k/32] (contiguous).
hipError_t launch_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, int8_t* xq, float* xd,
                               hipStream_t stream);

// y[m][n] from int8 activation codes xq [m][k] and scales xd [m][k/32] (contiguous rows),
// 16-row launches; silu_pairs as for launch_gemv_q8.
hipError_t launch_gemv_q8act(const DeviceInfo& dev, const uint8_t* w, int64_t n_out, int64_t k, bool silu_pairs,
                             const int8_t* xq, const float* xd, int64_t m, float* y, int64_t ldy, hipStream_t stream);

// Expert-grouped form of the matrix-core tiles (MoE prefill): tiles from the route plan's
// offsets / tile_start / sorted lists; gather: activation row of a position is
// x[sorted[pos] / top_k], else x[pos]; output row of a position is y[pos].
hipError_t launch_gemm_q8_mfma_grouped(const uint8_t* w_stack, size_t expert_bytes, int64_t n_out, int64_t k,
                                       bool silu_pairs, const float* x, int64_t ldx, float* y, int64_t ldy,
                                       const int32_t* offsets, const int32_t* tile_start, const int32_t* sorted,
                                       int n_exp, int top_k, bool gather, int64_t max_tiles, hipStream_t stream);

// Softmax top-k router with adaptive expert top-p (top_p >= 1: plain top-k).  logits ==
// nullptr: one kernel, one block per token; else a [m][n_exp] float32 workspace for the
// two-pass form (logits over many CUs, then selection), bit-identical results.
hipError_t launch_route_topk(const DeviceInfo& dev, const float* x, int64_t m, int64_t h, int64_t ldx,
                             const float* w_router, int64_t n_exp, int k, bool normalize, float top_p, int32_t* idx,
                             float* wts, float* logits, hipStream_t stream);

// Grouped MoE SwiGLU mixture; workspace laid out by q8v::moe_workspace_layout.
hipError_t launch_moe_grouped(const DeviceInfo& dev, const uint8_t* wgu, const uint8_t* wdn, int64_t n_exp, int64_t f,
                              int64_t h, const float* x, int64_t m, int64_t ldx, const int32_t* idx, const float* wts,
                              int k, float* y, int64_t ldy, void* workspace, hipStream_t stream);

// Measurement aids (include/q8_probe.h): a plain streaming read of `bytes` (a multiple
// of 4096) in launch shape `shape`, one xor word per lane into sink; an empty launch.
int probe_shape_count();
int64_t probe_sink_words(int shape, int cu_count);
hipError_t launch_probe_read(const DeviceInfo& dev, const void* src, int64_t bytes, int shape, uint32_t* sink,
                             hipStream_t stream);
hipError_t launch_probe_empty(int64_t blocks, hipStream_t stream);

}  // namespace q8k
