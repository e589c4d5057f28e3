// Host-only check of the C ABI's argument validation (q8_validate.h) under AddressSanitizer
// and UndefinedBehaviorSanitizer: every check function is driven through its accepted
// boundary values and each of its error paths, with message buffers of exact size, of
// capacity 1, and absent.  Built with g++ (no HIP); exits non-zero on the first mismatch,
// and the sanitizers abort on any out-of-bounds access, overflow or other UB.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "q8_validate.h"

using namespace q8v;

static int failures = 0;
#define EXPECT(expr, want)                                                                        \
    do {                                                                                          \
        const q8_status got_ = (expr);                                                            \
        if (got_ != (want)) {                                                                     \
            fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #expr, (int)got_, \
                    (int)(want));                                                                 \
            ++failures;                                                                           \
        }                                                                                         \
    } while (0)

// 256-byte aligned dummy buffers (never dereferenced by the checks)
alignas(256) static unsigned char pool[4096];
static void* P(size_t off) { return pool + off; }
static float* F(size_t off) { return reinterpret_cast<float*>(pool + off); }
static int32_t* I(size_t off) { return reinterpret_cast<int32_t*>(pool + off); }

// One message buffer per call, heap-allocated at exactly `cap` bytes so that any write past
// it is caught; cap 0 passes no buffer at all.
struct Msg {
    char* p = nullptr;
    size_t cap = 0;
    explicit Msg(size_t c) : cap(c) { p = c ? static_cast<char*>(malloc(c)) : nullptr; }
    ~Msg() { free(p); }
};

static void linear_cases(size_t cap) {
    const int64_t K = 256, N = 64;
    Msg m(cap);
    EXPECT(check_linear(P(0), N, K, F(0), 1, K, F(0), N, m.p, m.cap), Q8_OK);
    EXPECT(check_linear(P(0), N, int64_t(1) << 30, F(0), 1, int64_t(1) << 30, F(0), N, m.p, m.cap), Q8_OK);
    EXPECT(check_linear(P(0), int64_t(1) << 30, K, F(0), int64_t(1) << 30, K, F(0), int64_t(1) << 30, m.p, m.cap), Q8_OK);
    EXPECT(check_linear(P(0), N, 0, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, -256, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, 32, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, (int64_t(1) << 30) + 256, F(0), 1, int64_t(1) << 31, F(0), N, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, INT64_MAX / 256 * 256, F(0), 1, INT64_MAX, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), -1, K, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), INT64_MIN, K, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, K, F(0), -1, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, K, F(0), INT64_MAX, K, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, K, F(0), 2, K - 4, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, K, F(0), 2, K, F(0), N - 1, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear(P(0), N, K, F(0), 2, INT64_MAX, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    // nothing to do: pointers are not looked at
    EXPECT(check_linear(nullptr, N, K, nullptr, 0, K, nullptr, N, m.p, m.cap), Q8_OK);
    EXPECT(check_linear(nullptr, 0, K, nullptr, 5, K, nullptr, 0, m.p, m.cap), Q8_OK);
    EXPECT(check_linear(nullptr, N, K, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_NULL);
    EXPECT(check_linear(P(0), N, K, nullptr, 1, K, F(0), N, m.p, m.cap), Q8_ERR_NULL);
    EXPECT(check_linear(P(0), N, K, F(0), 1, K, nullptr, N, m.p, m.cap), Q8_ERR_NULL);
    EXPECT(check_linear(P(4), N, K, F(0), 1, K, F(0), N, m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_linear(P(0), N, K, F(8), 1, K, F(0), N, m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_linear(P(0), N, K, F(0), 2, K + 2, F(0), N, m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_linear(P(0), N, K, F(0), 1, K, reinterpret_cast<const float*>(pool + 2), N, m.p, m.cap),
           Q8_ERR_ALIGN);
    EXPECT(check_linear(P(0), N, K, F(0), 1, K, F(4), N + 7, m.p, m.cap), Q8_OK);
}

static void q8act_cases(size_t cap) {
    const int64_t K = 512, N = 32;
    Msg m(cap);
    EXPECT(check_linear_q8act(P(0), N, K, P(0), P(256), 3, F(0), N, m.p, m.cap), Q8_OK);
    EXPECT(check_linear_q8act(P(0), N, K, P(0), P(256), int64_t(1) << 30, F(0), N, m.p, m.cap), Q8_OK);  // 2^39
    EXPECT(check_linear_q8act(P(0), N, 4096, P(0), P(256), int64_t(1) << 30, F(0), N, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_linear_q8act(P(0), N, int64_t(1) << 30, P(0), P(256), int64_t(1) << 30, F(0), N, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_linear_q8act(P(0), N, K, nullptr, P(256), 3, F(0), N, m.p, m.cap), Q8_ERR_NULL);
    EXPECT(check_linear_q8act(P(0), N, K, P(0), P(260), 3, F(0), N, m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_linear_q8act(P(0), N, K, P(0), P(256), 3, F(0), N - 1, m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_quantize_act(F(0), 4, K, K, P(0), P(256), m.p, m.cap), Q8_OK);
    EXPECT(check_quantize_act(F(0), 4, K, K - 4, P(0), P(256), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_quantize_act(F(0), 4, K, K + 2, P(0), P(256), m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_quantize_act(F(0), int64_t(1) << 30, int64_t(1) << 30, int64_t(1) << 30, P(0), P(256), m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_quantize_act(nullptr, 0, K, K, nullptr, nullptr, m.p, m.cap), Q8_OK);
    EXPECT(check_quantize_act(F(0), 1, K, K, P(0), nullptr, m.p, m.cap), Q8_ERR_NULL);
}

static void route_cases(size_t cap) {
    Msg m(cap);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 128, 8, I(0), F(0), m.p, m.cap), Q8_OK);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 256, 256, I(0), F(0), m.p, m.cap), Q8_OK);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 257, 8, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 0, 1, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 8, 9, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 8, 0, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 8, INT32_MIN, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2044, F(0), 8, 2, I(0), F(0), m.p, m.cap), Q8_ERR_SHAPE);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(4), 8, 2, I(0), F(0), m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_route(F(0), 16, 2048, 2048, F(0), 8, 2, reinterpret_cast<int32_t*>(pool + 1), F(0), m.p, m.cap),
           Q8_ERR_ALIGN);
    EXPECT(check_route(F(0), 16, 2048, 2048, nullptr, 8, 2, I(0), F(0), m.p, m.cap), Q8_ERR_NULL);
    EXPECT(check_route_workspace(16, 128, P(0), route_workspace_bytes(16, 128), m.p, m.cap), Q8_OK);
    EXPECT(check_route_workspace(16, 128, P(0), route_workspace_bytes(16, 128) - 1, m.p, m.cap), Q8_ERR_WORKSPACE);
    EXPECT(check_route_workspace(16, 128, P(8), route_workspace_bytes(16, 128), m.p, m.cap), Q8_ERR_ALIGN);
    EXPECT(check_route_workspace(16, 128, nullptr, 1 << 20, m.p, m.cap), Q8_ERR_WORKSPACE);
    if (route_workspace_bytes(0, 128) != 256 || route_workspace_bytes(1, 1) != 256 ||
        route_workspace_bytes(65, 1) != 512) {
        fprintf(stderr, "route_workspace_bytes rounding\n");
        ++failures;
    }
}

static void moe_cases(size_t cap) {
    Msg m(cap);
    const int64_t E = 128, FF = 768, H = 2048, M = 16;
    const int32_t K = 8;
    const size_t need = moe_workspace_layout(M, K, E, FF, H).total;
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, P(0), need, m.p, m.cap), Q8_OK);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, P(0), need - 1, m.p, m.cap),
           Q8_ERR_WORKSPACE);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, P(16), need, m.p, m.cap),
           Q8_ERR_ALIGN);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, nullptr, need, m.p, m.cap),
           Q8_ERR_WORKSPACE);
    EXPECT(check_moe(P(0), P(256), E, FF, 16640, F(0), M, 16640, I(0), F(0), K, F(0), 16640, P(0), need, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), int64_t(1) << 22, H, I(0), F(0), K, F(0), H, P(0), need, m.p,
                     m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), 129, F(0), H, P(0), need, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H - 4, I(0), F(0), K, F(0), H, P(0), need, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H - 1, P(0), need, m.p, m.cap),
           Q8_ERR_SHAPE);
    EXPECT(check_moe(P(0), P(8), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, P(0), need, m.p, m.cap),
           Q8_ERR_ALIGN);
    EXPECT(check_moe(P(0), P(256), E, FF, H, F(0), M, H, I(0), nullptr, K, F(0), H, P(0), need, m.p, m.cap),
           Q8_ERR_NULL);
    EXPECT(check_moe(nullptr, nullptr, E, FF, H, nullptr, 0, H, nullptr, nullptr, K, nullptr, H, nullptr, 0, m.p,
                     m.cap),
           Q8_OK);
    EXPECT(check_moe_args(P(0), P(256), E, FF, H, F(0), M, H, I(0), F(0), K, F(0), H, m.p, m.cap), Q8_OK);
    // the largest accepted call: 2^24 routed pairs, h = f = 16384; the layout's sizes stay
    // far inside size_t and every region starts on a 256-byte boundary, in order
    const MoeWorkspace L = moe_workspace_layout(int64_t(1) << 21, 8, 256, 16384, 16384);
    const size_t offs[] = {L.offsets_off, L.sorted_off, L.inv_off, L.active_off, L.tiles_off, L.hidden_off,
                           L.out_off, L.total};
    for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
        if (offs[i] % 256 || (i && offs[i] <= offs[i - 1])) {
            fprintf(stderr, "moe_workspace_layout region %zu at %zu\n", i, offs[i]);
            ++failures;
        }
    }
    const size_t pairs = size_t(1) << 24;
    if (L.out_off - L.hidden_off < pairs * 2 * 16384 * sizeof(float) ||
        L.total - L.out_off < pairs * 16384 * sizeof(float)) {
        fprintf(stderr, "moe_workspace_layout regions too small\n");
        ++failures;
    }
}

static void message_text() {
    // the text names the argument and fits the buffer, NUL-terminated, however small
    for (size_t cap : {size_t(1), size_t(2), size_t(8), size_t(256)}) {
        Msg m(cap);
        memset(m.p, 'x', cap);
        EXPECT(check_linear(P(0), 64, 100, F(0), 1, 256, F(0), 64, m.p, m.cap), Q8_ERR_SHAPE);
        if (strnlen(m.p, cap) >= cap) {
            fprintf(stderr, "message not terminated within %zu bytes\n", cap);
            ++failures;
        }
        if (cap == 256 && !strstr(m.p, "k=100")) {
            fprintf(stderr, "message lacks the value: %s\n", m.p);
            ++failures;
        }
    }
}

int main() {
    for (size_t cap : {size_t(0), size_t(1), size_t(256)}) {
        linear_cases(cap);
        q8act_cases(cap);
        route_cases(cap);
        moe_cases(cap);
    }
    message_text();
    if (failures) {
        fprintf(stderr, "%d validation mismatches\n", failures);
        return 1;
    }
    printf("validation checks: all cases as expected\n");
    return 0;
}
