// Measurement aids for benchmarks (include/q8_probe.h): the time a plain streaming read
// of a byte count takes in one launch on this GPU, and the cost of a launch that does
// no work.  They bound what any kernel reading those bytes once can reach, and are not
// part of the linears' arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_internal.h"

namespace q8k {

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

// Launch shapes tried for the read: waves per block, 4 KB chunks a wave keeps in flight,
// blocks per CU, non-temporal or cached loads.  Which one is fastest depends on the byte
// count; callers time them all.
struct ProbeShape {
    int waves, unroll, blocks_per_cu;
    bool nt;
};
constexpr ProbeShape kProbeShapes[] = {{8, 2, 1, true},  {8, 4, 1, true},   {8, 2, 2, true},  {16, 2, 1, true},
                                       {4, 4, 2, true},  {8, 4, 2, true},   {8, 2, 1, false}, {8, 2, 2, false},
                                       {16, 2, 1, false}, {8, 4, 1, false}, {8, 8, 1, true},  {16, 4, 1, false}};
constexpr int kProbeShapeCount = sizeof(kProbeShapes) / sizeof(kProbeShapes[0]);

int probe_shape_count() { return kProbeShapeCount; }

int64_t probe_sink_words(int shape, int cu_count) {
    const ProbeShape& p = kProbeShapes[shape];
    return (int64_t)cu_count * p.blocks_per_cu * p.waves * 64;
}

// Wave w of the grid reads the 4 KB chunks w, w + nw, ... (U of them in flight, each as
// four coalesced 16-byte loads per lane) and stores the xor of the words
// it read to sink[w * 64 + lane], so that no load can be dropped: the xor of the whole
// sink is the xor of every 32-bit word of the buffer.
template <int NW, int U, bool NT>
__global__ __launch_bounds__(64 * NW) void probe_read_kernel(const probe_u32x4* __restrict__ src, int64_t chunks,
                                                             uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * NW + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * NW;
    uint32_t acc = 0;
    for (int64_t c0 = wid; c0 < chunks; c0 += U * nw) {
        probe_u32x4 v[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + u * nw;
            const int64_t cc = c < chunks ? c : c0;  // past the end: read chunk c0 again
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const probe_u32x4* a = src + cc * 256 + 64 * q + lane;
                v[u][q] = NT ? __builtin_nontemporal_load(a) : *a;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t t = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) t ^= v[u][q].x ^ v[u][q].y ^ v[u][q].z ^ v[u][q].w;
            if (c0 + u * nw < chunks) acc ^= t;  // a re-read chunk is not counted twice
        }
    }
    sink[wid * 64 + lane] = acc;
}

__global__ __launch_bounds__(256) void probe_empty_kernel() {}

template <int NW, int U, bool NT>
void launch_read(dim3 grid, hipStream_t stream, const probe_u32x4* s, int64_t chunks, uint32_t* sink) {
    hipLaunchKernelGGL((probe_read_kernel<NW, U, NT>), grid, dim3(64 * NW), 0, stream, s, chunks, sink);
}

hipError_t launch_probe_read(const DeviceInfo& dev, const void* src, int64_t bytes, int shape, uint32_t* sink,
                             hipStream_t stream) {
    const ProbeShape& p = kProbeShapes[shape];
    const dim3 grid((unsigned)(dev.cu_count * p.blocks_per_cu));
    const probe_u32x4* s = static_cast<const probe_u32x4*>(src);
    const int64_t chunks = bytes / 4096;
    switch (shape) {
        case 0: launch_read<8, 2, true>(grid, stream, s, chunks, sink); break;
        case 1: launch_read<8, 4, true>(grid, stream, s, chunks, sink); break;
        case 2: launch_read<8, 2, true>(grid, stream, s, chunks, sink); break;
        case 3: launch_read<16, 2, true>(grid, stream, s, chunks, sink); break;
        case 4: launch_read<4, 4, true>(grid, stream, s, chunks, sink); break;
        case 5: launch_read<8, 4, true>(grid, stream, s, chunks, sink); break;
        case 6: launch_read<8, 2, false>(grid, stream, s, chunks, sink); break;
        case 7: launch_read<8, 2, false>(grid, stream, s, chunks, sink); break;
        case 8: launch_read<16, 2, false>(grid, stream, s, chunks, sink); break;
        case 9: launch_read<8, 4, false>(grid, stream, s, chunks, sink); break;
        case 10: launch_read<8, 8, true>(grid, stream, s, chunks, sink); break;
        default: launch_read<16, 4, false>(grid, stream, s, chunks, sink); break;
    }
    return hipGetLastError();
}

hipError_t launch_probe_empty(int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL(probe_empty_kernel, dim3((unsigned)blocks), dim3(256), 0, stream);
    return hipGetLastError();
}

}  // namespace q8k
