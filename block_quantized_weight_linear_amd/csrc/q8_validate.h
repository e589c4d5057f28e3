// Host-side argument checks for the C ABI in include/q8_linear.h.
//
// Pure C++ (no HIP): every check runs before anything is enqueued, and the same
// header builds with g++ for CPU-only tests.  Each function returns Q8_OK or the
// error code, and writes a description into `msg` (capacity `cap`).
#pragma once

#include <stdint.h>
#include <stdio.h>

#include "../../include/q8_linear.h"

namespace q8v {

constexpr int64_t kQK = 32;           // quants per Q8_0 block
constexpr int64_t kBlockBytes = 34;   // binary16 scale + 32 int8
constexpr int64_t kKAlign = 256;      // K multiple: 8 blocks = 272 bytes = 17 x 16 bytes
constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxExperts = 256;
constexpr int64_t kMoeMaxDim = 16384;  // one staged activation row fits in 64 KB of LDS

inline int64_t row_bytes(int64_t k) { return (k / kQK) * kBlockBytes; }

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline q8_status fail(char* msg, size_t cap, q8_status s, const char* fmt, long long a = 0, long long b = 0) {
    if (msg && cap) snprintf(msg, cap, fmt, a, b);
    return s;
}

// K (or H, F) of a Q8_0 operand.
inline q8_status check_k(const char* what, int64_t k, char* msg, size_t cap) {
    if (k <= 0 || k > kMaxDim || k % kKAlign != 0) {
        if (msg && cap) snprintf(msg, cap, "%s=%lld must be a positive multiple of 256 (at most 2^30)", what, (long long)k);
        return Q8_ERR_SHAPE;
    }
    return Q8_OK;
}

inline q8_status check_dim(const char* what, int64_t v, char* msg, size_t cap) {
    if (v < 0 || v > kMaxDim) {
        if (msg && cap) snprintf(msg, cap, "%s=%lld out of range [0, 2^30]", what, (long long)v);
        return Q8_ERR_SHAPE;
    }
    return Q8_OK;
}

// Shared by q8_linear (n_out = n) and the fused gate_up call (n_out = f, weight rows 2f).
inline q8_status check_linear(const void* w, int64_t n_out, int64_t k, const float* x, int64_t m, int64_t ldx,
                              const float* y, int64_t ldy, char* msg, size_t cap) {
    q8_status s;
    if ((s = check_dim("n", n_out, msg, cap)) != Q8_OK) return s;
    if ((s = check_dim("m", m, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("k", k, msg, cap)) != Q8_OK) return s;
    if (ldx < k) return fail(msg, cap, Q8_ERR_SHAPE, "ldx=%lld < k=%lld", ldx, k);
    if (ldy < n_out) return fail(msg, cap, Q8_ERR_SHAPE, "ldy=%lld < n=%lld", ldy, n_out);
    if (ldx > kMaxDim || ldy > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "leading dimension above 2^30");
    if (m == 0 || n_out == 0) return Q8_OK;  // nothing to do; pointers may be anything
    if (!w || !x || !y) return fail(msg, cap, Q8_ERR_NULL, "null pointer (w, x or y)");
    if (!aligned(w, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "weight pointer not 16-byte aligned");
    if (!aligned(x, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "x pointer not 16-byte aligned");
    if (ldx % 4 != 0) return fail(msg, cap, Q8_ERR_ALIGN, "ldx=%lld not a multiple of 4", ldx);
    if (!aligned(y, 4)) return fail(msg, cap, Q8_ERR_ALIGN, "output pointer not 4-byte aligned");
    return Q8_OK;
}

// The integer q8 x q8 linears: codes xq [m][k] and scales xd [m][k/32], contiguous.
inline q8_status check_linear_q8act(const void* w, int64_t n_out, int64_t k, const void* xq, const void* xd,
                                    int64_t m, const float* y, int64_t ldy, char* msg, size_t cap) {
    q8_status s;
    if ((s = check_dim("n", n_out, msg, cap)) != Q8_OK) return s;
    if ((s = check_dim("m", m, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("k", k, msg, cap)) != Q8_OK) return s;
    if (ldy < n_out) return fail(msg, cap, Q8_ERR_SHAPE, "ldy=%lld < n=%lld", ldy, n_out);
    if (ldy > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "leading dimension above 2^30");
    if (m * k > (int64_t(1) << 40)) return fail(msg, cap, Q8_ERR_SHAPE, "m*k=%lld above 2^40", m * k);
    if (m == 0 || n_out == 0) return Q8_OK;
    if (!w || !xq || !xd || !y) return fail(msg, cap, Q8_ERR_NULL, "null pointer (w, xq, xd or y)");
    if (!aligned(w, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "weight pointer not 16-byte aligned");
    if (!aligned(xq, 16) || !aligned(xd, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "xq or xd not 16-byte aligned");
    if (!aligned(y, 4)) return fail(msg, cap, Q8_ERR_ALIGN, "output pointer not 4-byte aligned");
    return Q8_OK;
}

inline q8_status check_quantize_act(const float* x, int64_t m, int64_t k, int64_t ldx, const void* xq,
                                    const void* xd, char* msg, size_t cap) {
    q8_status s;
    if ((s = check_dim("m", m, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("k", k, msg, cap)) != Q8_OK) return s;
    if (ldx < k || ldx > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "ldx=%lld < k=%lld", ldx, k);
    if (m * k > (int64_t(1) << 40)) return fail(msg, cap, Q8_ERR_SHAPE, "m*k=%lld above 2^40", m * k);
    if (m == 0) return Q8_OK;
    if (!x || !xq || !xd) return fail(msg, cap, Q8_ERR_NULL, "null pointer (x, xq or xd)");
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 16))
        return fail(msg, cap, Q8_ERR_ALIGN, "x, xq or xd not 16-byte aligned");
    if (ldx % 4 != 0) return fail(msg, cap, Q8_ERR_ALIGN, "ldx=%lld not a multiple of 4", ldx);
    return Q8_OK;
}

inline q8_status check_route(const float* x, int64_t m, int64_t h, int64_t ldx, const float* w_router, int64_t n_exp,
                             int32_t k, const int32_t* idx, const float* wts, char* msg, size_t cap) {
    q8_status s;
    if ((s = check_dim("m", m, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("h", h, msg, cap)) != Q8_OK) return s;
    if (n_exp < 1 || n_exp > kMaxExperts) return fail(msg, cap, Q8_ERR_SHAPE, "n_exp=%lld out of range [1, 256]", n_exp);
    if (k < 1 || k > n_exp) return fail(msg, cap, Q8_ERR_SHAPE, "k=%lld out of range [1, n_exp=%lld]", k, n_exp);
    if (ldx < h || ldx > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "ldx=%lld < h=%lld", ldx, h);
    if (m == 0) return Q8_OK;
    if (!x || !w_router || !idx || !wts) return fail(msg, cap, Q8_ERR_NULL, "null pointer (x, w_router, topk_idx or topk_w)");
    if (!aligned(x, 16) || !aligned(w_router, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "x or w_router not 16-byte aligned");
    if (ldx % 4 != 0) return fail(msg, cap, Q8_ERR_ALIGN, "ldx=%lld not a multiple of 4", ldx);
    if (!aligned(idx, 4) || !aligned(wts, 4)) return fail(msg, cap, Q8_ERR_ALIGN, "topk outputs not 4-byte aligned");
    return Q8_OK;
}

// Workspace of the two-pass router: the float32 logits [m][n_exp].
inline size_t route_workspace_bytes(int64_t m, int64_t n_exp) {
    const size_t b = sizeof(float) * size_t(m) * size_t(n_exp);
    return b ? (b + 255) / 256 * 256 : 256;
}

inline q8_status check_route_workspace(int64_t m, int64_t n_exp, const void* ws, size_t ws_bytes, char* msg,
                                       size_t cap) {
    if (!ws) return fail(msg, cap, Q8_ERR_WORKSPACE, "workspace is NULL");
    const size_t need = route_workspace_bytes(m, n_exp);
    if (ws_bytes < need) return fail(msg, cap, Q8_ERR_WORKSPACE, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    if (!aligned(ws, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "workspace not 16-byte aligned");
    return Q8_OK;
}

// The grouped MoE call runs on the bf16 matrix cores (expert-grouped 128-row tiles) when
// the routed pairs average at least this many per expert, else on the float32 GEMV
// passes (decode).  Measured on the Qwen3-30B-A3B layer (128 experts): at 4 pairs per
// expert the GEMV passes are faster (about 300 us against 330), at 8 the tiles (333
// against 518 us: the GEMV passes stream an expert's weights once per 4 tokens).
constexpr int64_t kMoeMatrixCorePairsPerExpert = 8;
inline bool moe_uses_matrix_cores(int64_t n_pairs, int64_t n_exp) {
    return n_pairs >= kMoeMatrixCorePairsPerExpert * n_exp;
}

// Workspace of the grouped MoE call: a route plan plus the hidden activations.
struct MoeWorkspace {
    size_t offsets_off, sorted_off, inv_off, active_off, tiles_off, hidden_off, out_off, total;
};

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline MoeWorkspace moe_workspace_layout(int64_t m, int32_t k, int64_t n_exp, int64_t f, int64_t h) {
    MoeWorkspace w{};
    const size_t pairs = size_t(m) * size_t(k);
    size_t off = 0;
    w.offsets_off = off; off = round_up(off + sizeof(int32_t) * size_t(n_exp + 1), 256);
    w.sorted_off = off;  off = round_up(off + sizeof(int32_t) * pairs, 256);
    w.inv_off = off;     off = round_up(off + sizeof(int32_t) * pairs, 256);
    w.active_off = off;  off = round_up(off + sizeof(int32_t) * size_t(n_exp + 1), 256);
    w.tiles_off = off;   off = round_up(off + sizeof(int32_t) * size_t(n_exp + 1), 256);
    w.hidden_off = off;  off = round_up(off + sizeof(float) * pairs * 2 * size_t(f), 256);  // gate and up rows
    w.out_off = off;     off = round_up(off + sizeof(float) * pairs * size_t(h), 256);
    w.total = off;
    return w;
}

// Arguments of the grouped MoE call other than its workspace.
inline q8_status check_moe_args(const void* wgu, const void* wdn, int64_t n_exp, int64_t f, int64_t h, const float* x,
                                int64_t m, int64_t ldx, const int32_t* idx, const float* wts, int32_t k,
                                const float* y, int64_t ldy, char* msg, size_t cap) {
    q8_status s;
    if ((s = check_dim("m", m, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("h", h, msg, cap)) != Q8_OK) return s;
    if ((s = check_k("f", f, msg, cap)) != Q8_OK) return s;
    if (h > kMoeMaxDim || f > kMoeMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "h=%lld and f=%lld must be at most 16384", h, f);
    if (n_exp < 1 || n_exp > kMaxExperts) return fail(msg, cap, Q8_ERR_SHAPE, "n_exp=%lld out of range [1, 256]", n_exp);
    if (k < 1 || k > n_exp) return fail(msg, cap, Q8_ERR_SHAPE, "k=%lld out of range [1, n_exp=%lld]", k, n_exp);
    if (ldx < h || ldx > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "ldx=%lld < h=%lld", ldx, h);
    if (ldy < h || ldy > kMaxDim) return fail(msg, cap, Q8_ERR_SHAPE, "ldy=%lld < h=%lld", ldy, h);
    if (m * int64_t(k) > (int64_t(1) << 24)) return fail(msg, cap, Q8_ERR_SHAPE, "m*k=%lld above 2^24", m * int64_t(k));
    if (m == 0) return Q8_OK;
    if (!wgu || !wdn || !x || !idx || !wts || !y) return fail(msg, cap, Q8_ERR_NULL, "null pointer among the tensor arguments");
    if (!aligned(wgu, 16) || !aligned(wdn, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "expert stacks not 16-byte aligned");
    if (!aligned(x, 16)) return fail(msg, cap, Q8_ERR_ALIGN, "x not 16-byte aligned");
    if (ldx % 4 != 0) return fail(msg, cap, Q8_ERR_ALIGN, "ldx=%lld not a multiple of 4", ldx);
    if (!aligned(idx, 4) || !aligned(wts, 4) || !aligned(y, 4)) return fail(msg, cap, Q8_ERR_ALIGN, "topk or y not 4-byte aligned");
    return Q8_OK;
}

inline q8_status check_moe(const void* wgu, const void* wdn, int64_t n_exp, int64_t f, int64_t h, const float* x,
                           int64_t m, int64_t ldx, const int32_t* idx, const float* wts, int32_t k, const float* y,
                           int64_t ldy, const void* ws, size_t ws_bytes, char* msg, size_t cap) {
    q8_status s = check_moe_args(wgu, wdn, n_exp, f, h, x, m, ldx, idx, wts, k, y, ldy, msg, cap);
    if (s != Q8_OK || m == 0) return s;
    if (!ws) return fail(msg, cap, Q8_ERR_WORKSPACE, "workspace is NULL");
    const size_t need = moe_workspace_layout(m, k, n_exp, f, h).total;
    if (ws_bytes < need) return fail(msg, cap, Q8_ERR_WORKSPACE, "workspace %lld bytes < required %lld", (long long)ws_bytes, (long long)need);
    if (!aligned(ws, 256)) return fail(msg, cap, Q8_ERR_ALIGN, "workspace not 256-byte aligned");
    return Q8_OK;
}

}  // namespace q8v
