// Device-side helpers for the Q4_K and Q4TiledP kernels (gfx950, wave64).
//
// Q4_K superblock (ferrum-kernels q4_k_moe_id_gemv_batched.rs: 256 weights in
// 144 bytes; GGML's layout by way of candle): bytes 0-1 d, 2-3 dmin (fp16),
// 4-15 eight 6-bit scales and mins, 16-143 nibbles where byte 32c+l holds
// weight 64c+l (low nibble) and 64c+32+l (high nibble).
//
// Work unit of one lane: one 32-byte nibble chunk c of one superblock, i.e. 64
// weights = sub-block 2c (the low nibbles) and sub-block 2c+1 (the high ones).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr int kBlockWeights = 256;
constexpr int kBlockBytes = 144;
constexpr int kThreads = 256;   // threads of every GEMV workgroup (4 waves)
constexpr int kMaxTopK = 16;    // largest top_k
constexpr int kTpMaxSegs = 3;   // Q4TiledP tensors in one merged matvec launch
constexpr int kBucketChunk = 8; // pairs per bucketed work item

// ------------------------------------------------------------ tile layout --
// The GEMV kernels read Q4_K matrices in a tile-interleaved order of the same
// 144-byte superblocks (q4k_pack_tiles writes it from GGUF row order).  Rows
// go in groups of kTileRows = 8; tile (G, s) holds superblock s of rows
// 8G .. 8G + 7 in kTileBytes = 1152 bytes at (G * nb + s) * 1152:
//   [0, 128)     the 8 rows' 16-byte headers (d, dmin, packed scales), row r8
//                at 16 r8;
//   [128, 640)   first halves of the 32-byte nibble chunks: bytes 32c .. 32c+15
//                of row r8's 128 nibble bytes at 128 + 16 (8c + r8);
//   [640, 1152)  second halves: bytes 32c+16 .. 32c+31 at 640 + 16 (8c + r8).
// A lane that owns chunk c of row r8 (the unit of the GEMV kernels) thus
// reads its two 16-byte halves from places where the 32 lanes of a tile read
// 512 contiguous bytes per load instruction, whatever the row length.  Rows
// past n up to the next multiple of 8 are zero blocks.
constexpr int kTileRows = 8;
constexpr int kTileBytes = kTileRows * kBlockBytes;   // 1152
constexpr int kTileHalf0 = 128;
constexpr int kTileHalf1 = 640;

__host__ __device__ constexpr int64_t tile_rows(int64_t n) {
    return (n + kTileRows - 1) / kTileRows * kTileRows;
}
// Bytes of an n x k matrix in the tile layout (equal to the GGUF bytes when
// n is a multiple of 8).
__host__ __device__ constexpr int64_t tiles_matrix_bytes(int64_t n, int64_t k) {
    return tile_rows(n) * (k >> 8) * kBlockBytes;
}
// Byte offset of tile (row group G, superblock s) in a matrix of nb
// superblocks per row.
__host__ __device__ constexpr int64_t tile_offset(int64_t G, int s, int nb) {
    return (G * nb + s) * (int64_t)kTileBytes;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Half lanes of a packed register widened to float.  Feeding them straight into
// fmaf lets the compiler emit v_fma_mix_f32, which converts and multiplies in
// one instruction.
__device__ __forceinline__ float lo_half(uint32_t v) {
    return (float)__builtin_bit_cast(half2v, v).x;
}
__device__ __forceinline__ float hi_half(uint32_t v) {
    return (float)__builtin_bit_cast(half2v, v).y;
}

// Index of float i of an activation row in LDS: every 64 floats (one lane's
// unit) are followed by 4 pad floats, so lanes of a row start 68 floats apart
// and their 16-byte LDS reads fall in different banks.
__device__ __forceinline__ int xpad(int i) { return i + ((i >> 6) << 2); }
__host__ __device__ constexpr int xpad_len(int k) { return k + (k >> 4); }

// Scale and min of the lane's two sub-blocks (2c and 2c+1) from the 12 packed
// bytes (header words y, z, w):
//   j < 4 : scale = s[j] & 63, min = s[j+4] & 63
//   j >= 4: scale = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
//           min   = (s[j+4] >> 4) | (s[j]   >> 6) << 4
struct UnitScale {
    float kA, kB;   // d*scale of sub-blocks A and B
    float mA, mB;   // dmin*min of sub-blocks A and B
};

// Branch-free: with c' = c & 1 the chunk reads the byte pairs P = s[2c'..],
// Q = s[4+2c'..], R = s[8+2c'..] (one shift each); the low chunks take
// P & 63, Q & 63 per byte, the high ones (R & 15 | (P >> 6) << 4) and
// (R >> 4 | (Q >> 6) << 4); both are formed and one is selected per lane, and
// the bytes convert to float directly.
__device__ __forceinline__ UnitScale unit_scale(uint4 h, int c) {
    const uint32_t sh = (c & 1) << 4;
    const uint32_t P = h.y >> sh, Q = h.z >> sh, R = h.w >> sh;
    const uint32_t sc_lo = P & 0x3F3Fu, m_lo = Q & 0x3F3Fu;
    const uint32_t sc_hi = (R & 0x0F0Fu) | ((P >> 2) & 0x3030u);
    const uint32_t m_hi = ((R >> 4) & 0x0F0Fu) | ((Q >> 2) & 0x3030u);
    const bool hi = c >= 2;
    const uint32_t sc = hi ? sc_hi : sc_lo, mn = hi ? m_hi : m_lo;
    const float d = lo_half(h.x), dmin = hi_half(h.x);
    UnitScale s;
    s.kA = d * (float)(sc & 0xFFu);   // v_cvt_f32_ubyte0
    s.kB = d * (float)((sc >> 8) & 0xFFu);
    s.mA = dmin * (float)(mn & 0xFFu);
    s.mB = dmin * (float)((mn >> 8) & 0xFFu);
    return s;
}

// Nibble dot products of one unit against the lane's 64 activations in LDS.
// The masked nibbles are used in place as fp16 subnormals: (v & 0x000F000F)
// holds q*2^-24 in each half and (v & 0x00F000F0) holds q*2^-20, so one
// v_fma_mix_f32 per weight converts and accumulates with the product exact.
// accA = 2^-24 * sum q_i x_i over sub-block A, accB = 2^-20 * sum over B.
// Elements are accumulated in ascending order, one fp32 rounding per step.
struct UnitAcc {
    float a, b;
};

__device__ __forceinline__ void nib_fma(uint32_t v, float4 xa, float4 xb, UnitAcc &acc) {
    const uint32_t s = v >> 8;
    const uint32_t r0 = v & 0x000F000Fu, r2 = s & 0x000F000Fu;   // low nibbles: A
    const uint32_t r1 = v & 0x00F000F0u, r3 = s & 0x00F000F0u;   // high nibbles: B
    acc.a = __builtin_fmaf(lo_half(r0), xa.x, acc.a);
    acc.a = __builtin_fmaf(lo_half(r2), xa.y, acc.a);
    acc.a = __builtin_fmaf(hi_half(r0), xa.z, acc.a);
    acc.a = __builtin_fmaf(hi_half(r2), xa.w, acc.a);
    acc.b = __builtin_fmaf(lo_half(r1), xb.x, acc.b);
    acc.b = __builtin_fmaf(lo_half(r3), xb.y, acc.b);
    acc.b = __builtin_fmaf(hi_half(r1), xb.z, acc.b);
    acc.b = __builtin_fmaf(hi_half(r3), xb.w, acc.b);
}

// Unit value: sum over the 64 weights of (d*sc*q - dmin*m) * x, evaluated as
// d*sc_A*(sum q x)_A + d*sc_B*(sum q x)_B - (dmin*m_A*Sx_A + dmin*m_B*Sx_B).
__device__ __forceinline__ float unit_value(const UnitScale &s, const UnitAcc &acc, float sxA,
                                            float sxB) {
    const float dotA = acc.a * 16777216.0f;   // 2^24, exact
    const float dotB = acc.b * 1048576.0f;    // 2^20, exact
    const float pos = __builtin_fmaf(s.kA, dotA, s.kB * dotB);
    const float neg = __builtin_fmaf(s.mA, sxA, s.mB * sxB);
    return pos - neg;
}

// Cross-lane moves for the row reductions.  DPP quad_perm / row mirrors
// exchange within 16-lane rows in one v_add_f32_dpp each; rows are then
// combined through v_readlane (scalar broadcast), not through LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over groups of W consecutive lanes of a wave (W a power of two <= 64).
// Within 16 lanes: xor-1, xor-2, half-row mirror, row mirror, each step adding
// the partner's value, so every lane of a 16-lane row holds the row sum.
// Wider groups add the 16-lane row sums in row order.  The result is exact
// for the group's first lane (and for every lane when W <= 16).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_move<0x141>(v);   // row_half_mirror
    if constexpr (W >= 16) v += dpp_move<0x140>(v);  // row_mirror
    if constexpr (W == 32) {
        const float r0 = lane_value(v, 0), r1 = lane_value(v, 16);
        const float r2 = lane_value(v, 32), r3 = lane_value(v, 48);
        v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    } else if constexpr (W == 64) {
        const float r0 = lane_value(v, 0), r1 = lane_value(v, 16);
        const float r2 = lane_value(v, 32), r3 = lane_value(v, 48);
        v = (r0 + r1) + (r2 + r3);
    }
    return v;
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations have
// completed, then all waves meet.  __syncthreads() also waits for every
// global load still in flight (its release fence covers global memory), which
// would stall a kernel that has issued loads for later work.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

}  // namespace q4k
