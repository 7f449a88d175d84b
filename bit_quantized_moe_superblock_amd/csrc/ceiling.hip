// Measurement kernel: the read ceiling of a set of byte ranges.
//
// Reads every byte of n_ranges ranges of range_bytes bytes each (ranges at
// base + offsets[i]), 16 KB per workgroup with four 16-byte loads per thread
// in flight, and keeps only an xor checksum.  It computes nothing of the
// method: the rates it reaches are what this GPU gives for reading the same
// bytes (the experts a layer touches, or one contiguous buffer) with the
// plainest coalesced access, the figure each hot-path kernel is set against
// next to HBM peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4kceil.h"

namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = 16384;   // bytes per workgroup

__global__ __launch_bounds__(kThreads) void k_read_ranges(const uint8_t *__restrict__ base,
                                                          const int64_t *__restrict__ offsets,
                                                          int64_t per_range, int64_t range_bytes,
                                                          int64_t n_wg, uint32_t *sink) {
    const int64_t w = blockIdx.x;
    if (w >= n_wg)
        return;
    const int64_t r = w / per_range, c = w - r * per_range;
    const uint8_t *p = base + offsets[r] + c * kChunk;
    const int64_t left = range_bytes - c * kChunk;   // > 0
    uint32_t acc = 0;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int64_t off = (int64_t)(i * kThreads + threadIdx.x) * 16;
        v[i] = *(const uint4 *)(p + (off < left ? off : 0));   // clamped: never past the range
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
        acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0x9E3779B9u && threadIdx.x == 0)   // keeps the loads; practically never true
        sink[0] = (uint32_t)w;
}

}  // namespace

extern "C" int q4k_ceiling_read(const void *base, const int64_t *offsets, int64_t n_ranges,
                                int64_t range_bytes, uint32_t *sink, void *stream) {
    if (n_ranges < 1 || range_bytes < 16 || range_bytes % 16)
        return 1;
    if (!base || !offsets || !sink || (reinterpret_cast<uintptr_t>(base) & 15) ||
        (reinterpret_cast<uintptr_t>(offsets) & 7) || (reinterpret_cast<uintptr_t>(sink) & 3))
        return 2;
    const int64_t per = (range_bytes + kChunk - 1) / kChunk;
    const int64_t n_wg = per * n_ranges;
    if (n_wg > 0x7FFFFFFF)
        return 1;
    hipLaunchKernelGGL(k_read_ranges, dim3((unsigned)n_wg), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), (const uint8_t *)base, offsets,
                       per, range_bytes, n_wg, sink);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
