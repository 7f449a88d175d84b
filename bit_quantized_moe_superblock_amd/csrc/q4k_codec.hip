// Q4_K superblock encode and decode on the device.
//
// Decode is the superblock definition w_i = d*scale_j*q_i - dmin*min_j
// (ferrum-kernels q4_k_moe_id_gemv_batched.rs: 256 weights per 144-byte
// block; the field layout is GGML's Q4_K, which the pages use through candle).
// d*scale is exact in fp32 (11 x 6 bits), times q still exact (21 bits), and
// dmin*min is exact, so one fused multiply-add yields the correctly rounded
// value, which is why decode is bit-exact against any correct evaluation.
//
// Encode is a plain min/max affine encoder (the pages quantize with candle and
// do not print its routine).  Every decision is a single IEEE fp32 operation
// taken in a fixed order, so the bytes do not depend on the evaluation unit.
#include "common.hpp"
#include "launch.hpp"

namespace q4k {

__global__ __launch_bounds__(256) void k_q4k_dequant(const uint8_t *__restrict__ blocks,
                                                     float *__restrict__ out, int64_t n_blocks) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t b = gid >> 4;
    if (b >= n_blocks)
        return;
    const int part = (int)(gid & 15);
    const int c = part >> 2;          // 32-byte nibble chunk
    const int l0 = (part & 3) * 8;    // first byte of this thread inside the chunk
    const uint8_t *blk = blocks + b * kBlockBytes;
    const uint4 h = *(const uint4 *)blk;
    const uint2 q = *(const uint2 *)(blk + 16 + 32 * c + l0);
    const UnitScale s = unit_scale(h, c);
    float lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t byte = ((i < 4 ? q.x : q.y) >> (8 * (i & 3))) & 0xFFu;
        lo[i] = __builtin_fmaf(s.kA, (float)(byte & 15u), -s.mA);
        hi[i] = __builtin_fmaf(s.kB, (float)(byte >> 4), -s.mB);
    }
    float4 *o = (float4 *)(out + b * kBlockWeights + 64 * c + l0);
    o[0] = make_float4(lo[0], lo[1], lo[2], lo[3]);
    o[1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
    o[8] = make_float4(hi[0], hi[1], hi[2], hi[3]);   // +32 floats: the high nibbles
    o[9] = make_float4(hi[4], hi[5], hi[6], hi[7]);
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    const _Float16 h = (_Float16)x;   // round to nearest even, subnormals kept
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ int clampi(int v, int lo, int hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// One thread per superblock.  Steps, per sub-block j of 32 weights:
// lo = min(0, min w), hi = max w, a_j = (hi-lo)/15, b_j = -lo; then
// d = fp16(max a / 63), dmin = fp16(max b / 63), scale_j = rne(a_j/d),
// min_j = rne(b_j/dmin), q = rne((w + dmin*min_j)/(d*scale_j)), clamped.
__global__ __launch_bounds__(256) void k_q4k_quant(const float *__restrict__ w,
                                                   uint8_t *__restrict__ out, int64_t n_blocks) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks)
        return;
    const float *x = w + b * kBlockWeights;
    float a[8], bb[8];
    float amax = 0.0f, bmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float lo = 0.0f, hi = x[32 * j];
        for (int i = 0; i < 32; i++) {
            const float v = x[32 * j + i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        a[j] = (hi - lo) / 15.0f;
        bb[j] = 0.0f - lo;
        if (a[j] > amax) amax = a[j];
        if (bb[j] > bmax) bmax = bb[j];
    }
    const uint32_t dh = f32_to_f16_bits(amax / 63.0f);
    const uint32_t mh = f32_to_f16_bits(bmax / 63.0f);
    const float df = f16_bits_to_f32(dh), mf = f16_bits_to_f32(mh);
    int sc[8], mn[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        sc[j] = df > 0.0f ? clampi((int)__builtin_rintf(a[j] / df), 0, 63) : 0;
        mn[j] = mf > 0.0f ? clampi((int)__builtin_rintf(bb[j] / mf), 0, 63) : 0;
    }
    uint8_t hdr[16];
    hdr[0] = dh & 255u;
    hdr[1] = dh >> 8;
    hdr[2] = mh & 255u;
    hdr[3] = mh >> 8;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        hdr[4 + j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        hdr[8 + j] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        hdr[12 + j] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
    uint8_t *o = out + b * kBlockBytes;
    uint4 hv;
    __builtin_memcpy(&hv, hdr, 16);
    *(uint4 *)o = hv;
    for (int cch = 0; cch < 4; cch++) {
        const float sA = df * (float)sc[2 * cch], oA = mf * (float)mn[2 * cch];
        const float sB = df * (float)sc[2 * cch + 1], oB = mf * (float)mn[2 * cch + 1];
        uint8_t qs[32];
        for (int l = 0; l < 32; l++) {
            const float vA = x[64 * cch + l] + oA;
            const float vB = x[64 * cch + 32 + l] + oB;
            const int qA = sA > 0.0f ? clampi((int)__builtin_rintf(vA / sA), 0, 15) : 0;
            const int qB = sB > 0.0f ? clampi((int)__builtin_rintf(vB / sB), 0, 15) : 0;
            qs[l] = (uint8_t)(qA | (qB << 4));
        }
        uint4 v0, v1;
        __builtin_memcpy(&v0, qs, 16);
        __builtin_memcpy(&v1, qs + 16, 16);
        *(uint4 *)(o + 16 + 32 * cch) = v0;
        *(uint4 *)(o + 32 + 32 * cch) = v1;
    }
}

// GGUF row order <-> tile layout (common.hpp), one thread per (matrix, row,
// superblock) block: nine 16-byte pieces moved as they are.  Rows of the last
// row group past n are written as zero blocks (pack) or skipped (unpack).
__global__ __launch_bounds__(256) void k_q4k_pack_tiles(const uint8_t *__restrict__ src,
                                                        uint8_t *__restrict__ dst, int64_t n,
                                                        int nb, int64_t per_mat,
                                                        int64_t n_blocks) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks)   // n_blocks = n_mats * tile_rows(n) * nb
        return;
    const int64_t mi = b / per_mat, rb = b - mi * per_mat;   // per_mat = tile_rows(n) * nb
    const int64_t r = rb / nb;
    const int s = (int)(rb - r * nb);
    uint8_t *t = dst + mi * per_mat * kBlockBytes + tile_offset(r / kTileRows, s, nb);
    const int r8 = (int)(r % kTileRows);
    uint4 p[9];
    if (r < n) {
        const uint4 *g = (const uint4 *)(src + (mi * n * nb + r * nb + s) * kBlockBytes);
#pragma unroll
        for (int i = 0; i < 9; i++)
            p[i] = g[i];
    } else {
#pragma unroll
        for (int i = 0; i < 9; i++)
            p[i] = make_uint4(0, 0, 0, 0);
    }
    *(uint4 *)(t + 16 * r8) = p[0];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        *(uint4 *)(t + kTileHalf0 + 16 * (8 * c + r8)) = p[1 + 2 * c];
        *(uint4 *)(t + kTileHalf1 + 16 * (8 * c + r8)) = p[2 + 2 * c];
    }
}

__global__ __launch_bounds__(256) void k_q4k_unpack_tiles(const uint8_t *__restrict__ src,
                                                          uint8_t *__restrict__ dst, int64_t n,
                                                          int nb, int64_t tiled_mat,
                                                          int64_t n_blocks) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks)   // n_blocks = n_mats * n * nb
        return;
    const int64_t per = n * nb;
    const int64_t mi = b / per, rb = b - mi * per;
    const int64_t r = rb / nb;
    const int s = (int)(rb - r * nb);
    const uint8_t *t = src + mi * tiled_mat + tile_offset(r / kTileRows, s, nb);
    const int r8 = (int)(r % kTileRows);
    uint4 *g = (uint4 *)(dst + b * kBlockBytes);
    g[0] = *(const uint4 *)(t + 16 * r8);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        g[1 + 2 * c] = *(const uint4 *)(t + kTileHalf0 + 16 * (8 * c + r8));
        g[2 + 2 * c] = *(const uint4 *)(t + kTileHalf1 + 16 * (8 * c + r8));
    }
}

hipError_t launch_q4k_pack_tiles(const void *src, void *dst, int64_t n_mats, int64_t n,
                                 int64_t k, bool unpack, hipStream_t st) {
    const int nb = (int)(k >> 8);
    const int64_t per_tiled = tile_rows(n) * nb;
    const int64_t blocks = n_mats * (unpack ? n * nb : per_tiled);
    const dim3 grid((unsigned)((blocks + 255) / 256));
    if (unpack)
        hipLaunchKernelGGL(k_q4k_unpack_tiles, grid, dim3(256), 0, st, (const uint8_t *)src,
                           (uint8_t *)dst, n, nb, per_tiled * kBlockBytes, blocks);
    else
        hipLaunchKernelGGL(k_q4k_pack_tiles, grid, dim3(256), 0, st, (const uint8_t *)src,
                           (uint8_t *)dst, n, nb, per_tiled, blocks);
    return hipGetLastError();
}

hipError_t launch_q4k_dequant(const void *blocks, float *out, int64_t n_blocks, hipStream_t st) {
    if (n_blocks == 0)
        return hipSuccess;
    const int64_t threads = n_blocks * 16;
    hipLaunchKernelGGL(k_q4k_dequant, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                       (const uint8_t *)blocks, out, n_blocks);
    return hipGetLastError();
}

hipError_t launch_q4k_quant(const float *w, void *blocks, int64_t n_blocks, hipStream_t st) {
    if (n_blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_q4k_quant, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, st, w,
                       (uint8_t *)blocks, n_blocks);
    return hipGetLastError();
}

}  // namespace q4k
