// C ABI entry points (include/q8_linear.h): validate on the host, then enqueue.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/q8_probe.h"
#include "q8_internal.h"
#include "q8_validate.h"

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

q8_status device_fail(const char* where, hipError_t e) {
    set_err("%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
    return Q8_ERR_DEVICE;
}

constexpr int kMaxDevices = 64;
constexpr int64_t kPrefillRows = 256;  // from this many activation rows on: bf16 matrix-core path
std::mutex g_dev_mu;
q8k::DeviceInfo g_dev[kMaxDevices];

}  // namespace

// Fixed device scratch of q8_moe_grouped_linear_noalloc (Q8_MOE_NOALLOC_SCRATCH_BYTES).
// Each device holds its own copy for the life of the process.  Host code never passes
// the name itself to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[Q8_MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on first use there).
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

namespace q8k {

hipError_t current_device_info(DeviceInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (d.device != dev) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        int lds = 0;
        e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return e;
        d.cu_count = cus;
        d.lds_per_block = (size_t)lds;
        d.device = dev;
    }
    *out = d;
    return hipSuccess;
}

}  // namespace q8k

extern "C" {

int32_t q8_abi_version(void) { return Q8_ABI_VERSION; }

const char* q8_status_string(q8_status s) {
    switch (s) {
        case Q8_OK: return "ok";
        case Q8_ERR_NULL: return "null pointer";
        case Q8_ERR_SHAPE: return "invalid shape";
        case Q8_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case Q8_ERR_WORKSPACE: return "workspace missing or too small";
        case Q8_ERR_DEVICE: return "HIP runtime error";
    }
    return "unknown status";
}

const char* q8_last_error(void) { return g_err; }

static q8_status linear_common(const char* name, const void* w, int64_t n_out, int64_t k, bool silu, const float* x,
                               int64_t m, int64_t ldx, float* y, int64_t ldy, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_linear(w, n_out, k, x, m, ldx, y, ldy, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("%s: %s", name, msg);
        return s;
    }
    if (m == 0 || n_out == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail(name, e);
    const uint8_t* wq = static_cast<const uint8_t*>(w);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    e = m >= kPrefillRows ? q8k::launch_gemm_q8_mfma(dev, wq, n_out, k, silu, x, m, ldx, y, ldy, st)
                          : q8k::launch_gemv_q8(dev, wq, n_out, k, silu, x, m, ldx, y, ldy, st);
    if (e != hipSuccess) return device_fail(name, e);
    return Q8_OK;
}

q8_status q8_linear(const void* w_q8, int64_t n, int64_t k, const float* x, int64_t m, int64_t ldx, float* y,
                    int64_t ldy, void* stream) {
    return linear_common("q8_linear", w_q8, n, k, false, x, m, ldx, y, ldy, stream);
}

q8_status q8_linear_fused_gate_up_silu(const void* w_gate_up_q8, int64_t f, int64_t k, const float* x, int64_t m,
                                       int64_t ldx, float* h, int64_t ldh, void* stream) {
    return linear_common("q8_linear_fused_gate_up_silu", w_gate_up_q8, f, k, true, x, m, ldx, h, ldh, stream);
}

static q8_status q4_0_common(const char* name, const void* w, int64_t n_out, int64_t k, bool silu, const float* x,
                             int64_t m, int64_t ldx, float* y, int64_t ldy, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_linear(w, n_out, k, x, m, ldx, y, ldy, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("%s: %s", name, msg);
        return s;
    }
    if (m == 0 || n_out == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail(name, e);
    e = q8k::launch_gemv_q4_0(dev, static_cast<const uint8_t*>(w), n_out, k, silu, x, m, ldx, y, ldy,
                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(name, e);
    return Q8_OK;
}

q8_status q4_0_linear(const void* w_q4_0, int64_t n, int64_t k, const float* x, int64_t m, int64_t ldx, float* y,
                      int64_t ldy, void* stream) {
    return q4_0_common("q4_0_linear", w_q4_0, n, k, false, x, m, ldx, y, ldy, stream);
}

q8_status q4_0_linear_fused_gate_up_silu(const void* w_gate_up_q4_0, int64_t f, int64_t k, const float* x, int64_t m,
                                         int64_t ldx, float* h, int64_t ldh, void* stream) {
    return q4_0_common("q4_0_linear_fused_gate_up_silu", w_gate_up_q4_0, f, k, true, x, m, ldx, h, ldh, stream);
}

using kq_launcher = hipError_t (*)(const q8k::DeviceInfo&, const uint8_t*, int64_t, int64_t, bool, const float*, int64_t,
                                   int64_t, float*, int64_t, hipStream_t);

static q8_status kq_common(const char* name, kq_launcher launch, const void* w, int64_t n_out, int64_t k, bool silu,
                           const float* x, int64_t m, int64_t ldx, float* y, int64_t ldy, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_linear(w, n_out, k, x, m, ldx, y, ldy, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("%s: %s", name, msg);
        return s;
    }
    if (m == 0 || n_out == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail(name, e);
    e = launch(dev, static_cast<const uint8_t*>(w), n_out, k, silu, x, m, ldx, y, ldy, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(name, e);
    return Q8_OK;
}

q8_status q4_k_linear(const void* w_q4_k, int64_t n, int64_t k, const float* x, int64_t m, int64_t ldx, float* y,
                      int64_t ldy, void* stream) {
    return kq_common("q4_k_linear", q8k::launch_gemv_q4_k, w_q4_k, n, k, false, x, m, ldx, y, ldy, stream);
}

q8_status q4_k_linear_fused_gate_up_silu(const void* w_gate_up_q4_k, int64_t f, int64_t k, const float* x, int64_t m,
                                         int64_t ldx, float* h, int64_t ldh, void* stream) {
    return kq_common("q4_k_linear_fused_gate_up_silu", q8k::launch_gemv_q4_k, w_gate_up_q4_k, f, k, true, x, m, ldx, h,
                     ldh, stream);
}

q8_status q5_k_linear(const void* w_q5_k, int64_t n, int64_t k, const float* x, int64_t m, int64_t ldx, float* y,
                      int64_t ldy, void* stream) {
    return kq_common("q5_k_linear", q8k::launch_gemv_q5_k, w_q5_k, n, k, false, x, m, ldx, y, ldy, stream);
}

q8_status q5_k_linear_fused_gate_up_silu(const void* w_gate_up_q5_k, int64_t f, int64_t k, const float* x, int64_t m,
                                         int64_t ldx, float* h, int64_t ldh, void* stream) {
    return kq_common("q5_k_linear_fused_gate_up_silu", q8k::launch_gemv_q5_k, w_gate_up_q5_k, f, k, true, x, m, ldx, h,
                     ldh, stream);
}

q8_status q6_k_linear(const void* w_q6_k, int64_t n, int64_t k, const float* x, int64_t m, int64_t ldx, float* y,
                      int64_t ldy, void* stream) {
    return kq_common("q6_k_linear", q8k::launch_gemv_q6_k, w_q6_k, n, k, false, x, m, ldx, y, ldy, stream);
}

q8_status q6_k_linear_fused_gate_up_silu(const void* w_gate_up_q6_k, int64_t f, int64_t k, const float* x, int64_t m,
                                         int64_t ldx, float* h, int64_t ldh, void* stream) {
    return kq_common("q6_k_linear_fused_gate_up_silu", q8k::launch_gemv_q6_k, w_gate_up_q6_k, f, k, true, x, m, ldx, h,
                     ldh, stream);
}

q8_status q8_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, int8_t* xq, float* xd, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_quantize_act(x, m, k, ldx, xq, xd, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("q8_quantize_act: %s", msg);
        return s;
    }
    if (m == 0) return Q8_OK;
    hipError_t e = q8k::launch_quantize_act(x, m, k, ldx, xq, xd, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("q8_quantize_act", e);
    return Q8_OK;
}

static q8_status linear_q8act_common(const char* name, const void* w, int64_t n_out, int64_t k, bool silu,
                                     const int8_t* xq, const float* xd, int64_t m, float* y, int64_t ldy,
                                     void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_linear_q8act(w, n_out, k, xq, xd, m, y, ldy, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("%s: %s", name, msg);
        return s;
    }
    if (m == 0 || n_out == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail(name, e);
    e = q8k::launch_gemv_q8act(dev, static_cast<const uint8_t*>(w), n_out, k, silu, xq, xd, m, y, ldy,
                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(name, e);
    return Q8_OK;
}

q8_status q8_linear_q8act(const void* w_q8, int64_t n, int64_t k, const int8_t* xq, const float* xd, int64_t m,
                          float* y, int64_t ldy, void* stream) {
    return linear_q8act_common("q8_linear_q8act", w_q8, n, k, false, xq, xd, m, y, ldy, stream);
}

q8_status q8_linear_fused_gate_up_silu_q8act(const void* w_gate_up_q8, int64_t f, int64_t k, const int8_t* xq,
                                             const float* xd, int64_t m, float* h, int64_t ldh, void* stream) {
    return linear_q8act_common("q8_linear_fused_gate_up_silu_q8act", w_gate_up_q8, f, k, true, xq, xd, m, h, ldh,
                               stream);
}

static q8_status route_common(const char* name, const float* x, int64_t m, int64_t h, int64_t ldx,
                              const float* w_router, int64_t n_exp, int32_t k, int32_t normalize, float top_p,
                              int32_t* topk_idx, float* topk_w, bool with_ws, void* workspace,
                              size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_route(x, m, h, ldx, w_router, n_exp, k, topk_idx, topk_w, msg, sizeof msg);
    if (s == Q8_OK && !(top_p > 0.0f && top_p <= 1.0f)) {
        snprintf(msg, sizeof msg, "top_p must be in (0, 1]");
        s = Q8_ERR_SHAPE;
    }
    if (s == Q8_OK && with_ws && m > 0) s = q8v::check_route_workspace(m, n_exp, workspace, workspace_bytes, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("%s: %s", name, msg);
        return s;
    }
    if (m == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail(name, e);
    e = q8k::launch_route_topk(dev, x, m, h, ldx, w_router, n_exp, k, normalize != 0, top_p, topk_idx, topk_w,
                               with_ws ? static_cast<float*>(workspace) : nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail(name, e);
    return Q8_OK;
}

q8_status moe_route_topk(const float* x, int64_t m, int64_t h, int64_t ldx, const float* w_router, int64_t n_exp,
                         int32_t k, int32_t normalize, int32_t* topk_idx, float* topk_w, void* stream) {
    return route_common("moe_route_topk", x, m, h, ldx, w_router, n_exp, k, normalize, 1.0f, topk_idx, topk_w,
                        false, nullptr, 0, stream);
}

q8_status moe_route_topk_top_p(const float* x, int64_t m, int64_t h, int64_t ldx, const float* w_router,
                               int64_t n_exp, int32_t k, int32_t normalize, float top_p, int32_t* topk_idx,
                               float* topk_w, void* stream) {
    return route_common("moe_route_topk_top_p", x, m, h, ldx, w_router, n_exp, k, normalize, top_p, topk_idx,
                        topk_w, false, nullptr, 0, stream);
}

size_t moe_route_workspace_bytes(int64_t m, int64_t n_exp) {
    if (m < 0 || m > q8v::kMaxDim || n_exp < 1 || n_exp > q8v::kMaxExperts) return 0;
    return q8v::route_workspace_bytes(m, n_exp);
}

q8_status moe_route_topk_ws(const float* x, int64_t m, int64_t h, int64_t ldx, const float* w_router, int64_t n_exp,
                            int32_t k, int32_t normalize, float top_p, int32_t* topk_idx, float* topk_w,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return route_common("moe_route_topk_ws", x, m, h, ldx, w_router, n_exp, k, normalize, top_p, topk_idx, topk_w,
                        true, workspace, workspace_bytes, stream);
}

size_t q8_moe_workspace_bytes(int64_t m, int32_t k, int64_t n_exp, int64_t f, int64_t h) {
    char msg[8];
    if (q8v::check_dim("m", m, msg, sizeof msg) != Q8_OK || q8v::check_k("f", f, msg, sizeof msg) != Q8_OK ||
        q8v::check_k("h", h, msg, sizeof msg) != Q8_OK || h > q8v::kMoeMaxDim || f > q8v::kMoeMaxDim || n_exp < 1 || n_exp > q8v::kMaxExperts || k < 1 ||
        k > n_exp || m * int64_t(k) > (int64_t(1) << 24))
        return 0;
    return q8v::moe_workspace_layout(m, k, n_exp, f, h).total;
}

q8_status q8_moe_grouped_linear(const void* w_gate_up_exps, const void* w_down_exps, int64_t n_exp, int64_t f,
                                int64_t h, const float* x, int64_t m, int64_t ldx, const int32_t* topk_idx,
                                const float* topk_w, int32_t k, float* y, int64_t ldy, void* workspace,
                                size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_moe(w_gate_up_exps, w_down_exps, n_exp, f, h, x, m, ldx, topk_idx, topk_w, k, y, ldy,
                                 workspace, workspace_bytes, msg, sizeof msg);
    if (s != Q8_OK) {
        set_err("q8_moe_grouped_linear: %s", msg);
        return s;
    }
    if (m == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail("q8_moe_grouped_linear", e);
    e = q8k::launch_moe_grouped(dev, static_cast<const uint8_t*>(w_gate_up_exps),
                                static_cast<const uint8_t*>(w_down_exps), n_exp, f, h, x, m, ldx, topk_idx, topk_w, k,
                                y, ldy, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("q8_moe_grouped_linear", e);
    return Q8_OK;
}

q8_status q8_moe_grouped_linear_noalloc(const void* w_gate_up_exps, const void* w_down_exps, int64_t n_exp,
                                         int64_t f, int64_t h, const float* x, int64_t m, int64_t ldx,
                                         const int32_t* topk_idx, const float* topk_w, int32_t k, float* y,
                                         int64_t ldy, void* stream) {
    g_err[0] = 0;
    char msg[256];
    q8_status s = q8v::check_moe_args(w_gate_up_exps, w_down_exps, n_exp, f, h, x, m, ldx, topk_idx, topk_w, k, y,
                                      ldy, msg, sizeof msg);
    if (s == Q8_OK && m > 0) {
        const size_t need = q8v::moe_workspace_layout(m, k, n_exp, f, h).total;
        if (need > (size_t)Q8_MOE_NOALLOC_SCRATCH_BYTES) {
            snprintf(msg, sizeof msg, "these sizes need %lld bytes of scratch; the fixed scratch holds %lld",
                     (long long)need, (long long)Q8_MOE_NOALLOC_SCRATCH_BYTES);
            s = Q8_ERR_WORKSPACE;
        }
    }
    if (s != Q8_OK) {
        set_err("q8_moe_grouped_linear_noalloc: %s", msg);
        return s;
    }
    if (m == 0) return Q8_OK;
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail("q8_moe_grouped_linear_noalloc", e);
    void* ws = nullptr;
    e = scratch_address(&ws);
    if (e != hipSuccess) return device_fail("q8_moe_grouped_linear_noalloc: scratch address", e);
    e = q8k::launch_moe_grouped(dev, static_cast<const uint8_t*>(w_gate_up_exps),
                                static_cast<const uint8_t*>(w_down_exps), n_exp, f, h, x, m, ldx, topk_idx, topk_w, k,
                                y, ldy, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("q8_moe_grouped_linear_noalloc", e);
    return Q8_OK;
}

int32_t q8_probe_shape_count(void) { return q8k::probe_shape_count(); }

int64_t q8_probe_sink_words(int32_t shape) {
    if (shape < 0 || shape >= q8k::probe_shape_count()) return -1;
    q8k::DeviceInfo dev;
    if (q8k::current_device_info(&dev) != hipSuccess) return -1;
    return q8k::probe_sink_words(shape, dev.cu_count);
}

q8_status q8_probe_stream_read(const void* src, int64_t bytes, int32_t shape, uint32_t* sink, int64_t sink_words,
                               void* stream) {
    g_err[0] = 0;
    if (!src || !sink) {
        set_err("q8_probe_stream_read: src and sink must not be NULL");
        return Q8_ERR_NULL;
    }
    if (bytes <= 0 || bytes % 4096 != 0 || shape < 0 || shape >= q8k::probe_shape_count()) {
        set_err("q8_probe_stream_read: bytes must be a positive multiple of 4096 (got %lld) and shape in [0, %d) "
                "(got %d)",
                (long long)bytes, q8k::probe_shape_count(), (int)shape);
        return Q8_ERR_SHAPE;
    }
    if ((uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0) {
        set_err("q8_probe_stream_read: src must be 16-byte and sink 4-byte aligned");
        return Q8_ERR_ALIGN;
    }
    q8k::DeviceInfo dev;
    hipError_t e = q8k::current_device_info(&dev);
    if (e != hipSuccess) return device_fail("q8_probe_stream_read", e);
    const int64_t need = q8k::probe_sink_words(shape, dev.cu_count);
    if (sink_words < need) {
        set_err("q8_probe_stream_read: shape %d needs %lld sink words, got %lld", (int)shape, (long long)need,
                (long long)sink_words);
        return Q8_ERR_WORKSPACE;
    }
    e = q8k::launch_probe_read(dev, src, bytes, shape, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("q8_probe_stream_read", e);
    return Q8_OK;
}

q8_status q8_probe_empty(int64_t blocks, void* stream) {
    g_err[0] = 0;
    if (blocks < 1 || blocks > INT32_MAX) {
        set_err("q8_probe_empty: blocks must be in [1, 2^31 - 1] (got %lld)", (long long)blocks);
        return Q8_ERR_SHAPE;
    }
    hipError_t e = q8k::launch_probe_empty(blocks, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_fail("q8_probe_empty", e);
    return Q8_OK;
}

}  // extern "C"
