// Device core shared by the Q4_K GEMV kernels (q4k_gemv.hip, q4k_mfma.hip):
// kernel arguments, activation staging, the per-unit Q4_K arithmetic, row
// tiles and row reductions, plus a few host-side launch helpers.
//
// Layout conventions (ferrum-kernels q4_k_moe_id_gemv_batched.rs, module doc:
// expert stacks [E, n, k/256] of 144-byte Q4_K blocks, pair p = token*top_k +
// slot, activation row src1 + token*outer + slot*inner):
//   - 256 threads per workgroup; LPR consecutive lanes cover one weight row,
//     lane u owning unit u = (superblock u/4, 32-byte nibble chunk u%4), i.e.
//     64 weights: sub-block 2c in the low nibbles and 2c+1 in the high ones;
//   - activation rows are staged in LDS (padded so a row's lanes hit different
//     banks) with their 32-element sums, each taken in ascending order from 0
//     by one thread, so every vector-unit mode rounds alike and gives
//     identical bits.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace q4k {

enum { EPI_STORE = 0, EPI_SWIGLU = 1 };

struct GemvArgs {
    const uint8_t *w0, *w1;   // routed stacks (w1: the up stack of the fused kernel)
    const uint8_t *s0, *s1;   // shared one-expert stacks (null when m_sh == 0)
    const float *src1;        // routed activations
    const float *src1_sh;     // shared activations: token t at src1_sh + t*outer_sh
    const int32_t *ids;
    const int32_t *bucket;    // bucket workspace (bucketed mode)
    float *dst;               // [n_pairs, n]
    float *dst_sh;            // [m_sh, n]
    int64_t outer, inner, outer_sh;
    int n, k, top_k, num_experts, n_pairs, m_sh;
    int pc;                   // pairs per LDS chunk (bucketed mode)
    int vec;                  // activation rows 16-byte aligned (float4 staging)
};

// Reads every argument field into scalar registers at kernel entry.  Left to
// itself the compiler loads the argument block field by field where each is
// first used, and every load of a new 64-byte line of the block is a separate
// round trip that the wave waits for; naming all fields here issues the loads
// together and waits once.  Input operands only: the values are unchanged.
__device__ __forceinline__ void fetch_args(const GemvArgs &a) {
    asm volatile("" ::"s"(a.w0), "s"(a.w1), "s"(a.s0), "s"(a.s1), "s"(a.src1), "s"(a.src1_sh),
                 "s"(a.ids), "s"(a.bucket));
    asm volatile("" ::"s"(a.dst), "s"(a.dst_sh), "s"(a.outer), "s"(a.inner), "s"(a.outer_sh),
                 "s"(a.n), "s"(a.k), "s"(a.top_k), "s"(a.num_experts), "s"(a.n_pairs),
                 "s"(a.m_sh), "s"(a.pc), "s"(a.vec));
}

// Where pair q (q >= n_pairs: shared pair of token q - n_pairs) reads and writes.
struct PairRef {
    const uint8_t *w0, *w1;   // expert base of the stacks
    const float *x;
    float *out;
    bool valid;
};

__device__ __forceinline__ PairRef pair_ref(const GemvArgs &a, int q) {
    PairRef r;
    const int64_t nb01 = (int64_t)(a.k >> 8) * kBlockBytes;
    if (q < a.n_pairs) {
        const int e = a.ids[q];
        const int t = q / a.top_k, s = q - t * a.top_k;
        r.valid = (unsigned)e < (unsigned)a.num_experts;
        const int64_t off = r.valid ? (int64_t)e * a.n * nb01 : 0;
        r.w0 = a.w0 + off;
        r.w1 = a.w1 ? a.w1 + off : nullptr;
        r.x = a.src1 + t * a.outer + s * a.inner;
        r.out = a.dst + (int64_t)q * a.n;
    } else {
        const int t = q - a.n_pairs;
        r.valid = true;
        r.w0 = a.s0;
        r.w1 = a.s1;
        r.x = a.src1_sh + t * a.outer_sh;
        r.out = a.dst_sh + (int64_t)t * a.n;
    }
    return r;
}

// Activation row of pair q (no id lookup needed).
__device__ __forceinline__ const float *pair_x(const GemvArgs &a, int q) {
    if (q < a.n_pairs) {
        const int t = q / a.top_k, s = q - t * a.top_k;
        return a.src1 + t * a.outer + s * a.inner;
    }
    return a.src1_sh + (q - a.n_pairs) * a.outer_sh;
}

// Same, when the caller knows (uniformly across the workgroup) whether the
// pair is a shared-expert pair.  A lane-varying choice between the two
// argument fields compiles into a per-lane load from the argument segment,
// whose wait would also wait for every weight load in flight.
__device__ __forceinline__ const float *pair_x_known(const GemvArgs &a, bool shared, int q) {
    if (shared)
        return a.src1_sh + (q - a.n_pairs) * a.outer_sh;
    const int t = q / a.top_k, s = q - t * a.top_k;
    return a.src1 + t * a.outer + s * a.inner;
}

// ------------------------------------------------------------ staging ----
// LDS image of one activation row: xpad_len(k) floats (64 + 4 pad per unit),
// then k/32 sub-block sums.  Each sub-block of 32 floats is loaded and summed
// (ascending, one thread) by one thread, which fixes the rounding of the sums.
__host__ __device__ constexpr int row_lds_floats(int k) { return xpad_len(k) + (k >> 5); }

// One staging batch: thread tid owns flattened sub-block base + tid of the
// rows being staged (row-major over (row, sub-block)).
struct StageBatch {
    float4 v[8];
    int f;
};

// VEC: rows and strides are 16-byte aligned (float4 loads); otherwise 4-byte
// loads.  A compile-time choice: with the choice made at run time the compiler
// merges both sides into the 4-byte loads.
template <bool VEC, typename XOf>
__device__ __forceinline__ void stage_issue(XOf x_of, int base, int total, int k,
                                            StageBatch &b) {
    const int nsub = k >> 5;
    b.f = base + (int)threadIdx.x;
    if (total <= 0)
        return;
    // Threads past the end re-load the last sub-block (clamped, never
    // committed) so the loads need no lane-divergent branch.
    const int f = b.f < total ? b.f : total - 1;
    const int row = f / nsub, j = f - row * nsub;
    const float *src = x_of(row) + 32 * j;
    if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < 8; q++)
            b.v[q] = *(const float4 *)(src + 4 * q);
    } else {
#pragma unroll
        for (int q = 0; q < 8; q++)
            b.v[q] = make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
    }
}

__device__ __forceinline__ void stage_commit(const StageBatch &b, int total, int k, float *lds) {
    if (b.f < total) {
        const int nsub = k >> 5;
        const int row = b.f / nsub, j = b.f - row * nsub;
        float *dstrow = lds + row * row_lds_floats(k);
        float4 *d = (float4 *)(dstrow + xpad(32 * j));
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            d[q] = b.v[q];
            s += b.v[q].x;
            s += b.v[q].y;
            s += b.v[q].z;
            s += b.v[q].w;
        }
        dstrow[xpad_len(k) + j] = s;
    }
}

// Stage rows [0, cl) starting at flattened sub-block `from` (batches of 256).
// No barrier.
template <bool VEC, typename XOf>
__device__ __forceinline__ void stage_rows(XOf x_of, int cl, int k, float *lds, int from = 0) {
    const int total = cl * (k >> 5);
    for (int base = from; base < total; base += kThreads) {
        StageBatch b;
        stage_issue<VEC>(x_of, base, total, k, b);
        stage_commit(b, total, k, lds);
    }
}

// ------------------------------------------------------- unit arithmetic ----

// Masked nibbles of one 32-byte chunk: for each of its 8 dwords, the four
// fp16-subnormal pairs (low nibbles of bytes 0,2 and 1,3; high nibbles of the
// same).
struct Masks {
    uint32_t m[8][4];
};

__device__ __forceinline__ void make_masks(const uint4 &qa, const uint4 &qb, Masks &k) {
    const uint32_t w[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int d = 0; d < 8; d++) {
        const uint32_t v = w[d], s = v >> 8;
        k.m[d][0] = v & 0x000F000Fu;
        k.m[d][1] = s & 0x000F000Fu;
        k.m[d][2] = v & 0x00F000F0u;
        k.m[d][3] = s & 0x00F000F0u;
    }
}

// Accumulate one 8-weight step d of a unit (see nib_fma in common.hpp for the
// element order) from precomputed masks.
__device__ __forceinline__ void masked_fma(const uint32_t (&r)[4], float4 xa, float4 xb,
                                           UnitAcc &acc) {
    acc.a = __builtin_fmaf(lo_half(r[0]), xa.x, acc.a);
    acc.a = __builtin_fmaf(lo_half(r[1]), xa.y, acc.a);
    acc.a = __builtin_fmaf(hi_half(r[0]), xa.z, acc.a);
    acc.a = __builtin_fmaf(hi_half(r[1]), xa.w, acc.a);
    acc.b = __builtin_fmaf(lo_half(r[2]), xb.x, acc.b);
    acc.b = __builtin_fmaf(lo_half(r[3]), xb.y, acc.b);
    acc.b = __builtin_fmaf(hi_half(r[2]), xb.z, acc.b);
    acc.b = __builtin_fmaf(hi_half(r[3]), xb.w, acc.b);
}

// Reduce a per-lane unit value over the LPR lanes of its row.  For rows wider
// than a wave the wave sums go through `red` (2 barriers); `slot_lane0` is true
// on the lane that receives the row total.
template <int LPR>
__device__ __forceinline__ float row_reduce(float v, float *red, int nt_index) {
    constexpr int WL = LPR < 64 ? LPR : 64;
    constexpr int WPR = LPR / WL;
    v = group_sum<WL>(v);
    if constexpr (WPR > 1) {
        const int tid = threadIdx.x;
        const int wave = tid >> 6;
        if ((tid & 63) == 0)
            red[nt_index * 4 + wave] = v;
        __syncthreads();
        if ((tid % LPR) == 0) {
            float s = red[nt_index * 4 + wave];
            for (int w = 1; w < WPR; w++)
                s += red[nt_index * 4 + wave + w];
            v = s;
        }
        __syncthreads();
    }
    return v;
}

template <int EPI, int NT>
__device__ __forceinline__ float epilogue(const float (&part)[NT]) {
    if constexpr (EPI == EPI_SWIGLU)
        return silu_mul(part[0], part[NT - 1]);
    else
        return part[0];
}

// Row tile of one lane: ITERS row groups, NT tensors.
template <int NT, int ITERS>
struct Tile {
    uint4 hdr[NT][ITERS];
    uint4 qa[NT][ITERS];
    uint4 qb[NT][ITERS];
};

// Hide a tile's registers from loop-invariant code motion.  Without this the
// compiler hoists the masked and fp32-converted weights out of a per-pair loop
// into (accumulation) registers, which costs a register read plus an fma per
// weight and pair instead of one v_fma_mix_f32 that decodes as it multiplies.
template <int NT, int ITERS>
__device__ __forceinline__ void opaque(Tile<NT, ITERS> &t) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int it = 0; it < ITERS; it++) {
            asm volatile("" : "+v"(t.qa[nt][it].x), "+v"(t.qa[nt][it].y), "+v"(t.qa[nt][it].z),
                         "+v"(t.qa[nt][it].w));
            asm volatile("" : "+v"(t.qb[nt][it].x), "+v"(t.qb[nt][it].y), "+v"(t.qb[nt][it].z),
                         "+v"(t.qb[nt][it].w));
        }
}

template <int LPR, int NT, int ITERS>
__device__ __forceinline__ void load_rows(const uint8_t *w0, const uint8_t *w1, int n, int k,
                                          int row0, bool valid, Tile<NT, ITERS> &t) {
    constexpr int RPI = kThreads / LPR;
    const int tid = threadIdx.x;
    const int nb = k >> 8;
    // Lanes past the row's units and row groups past n load a clamped, valid
    // address instead of branching: their results never reach a reduction or
    // a store, and a lane-divergent load makes the compiler wait for it at the
    // join (register copies out of the loaded registers).
    const int u0 = tid % LPR;
    const int u = u0 < 4 * nb ? u0 : 0;
    const int rsub = tid / LPR;
    const int64_t nb01 = (int64_t)nb * kBlockBytes;
    const int64_t uoff = (int64_t)(u >> 2) * kBlockBytes;
    const int c = u & 3;
    if (!valid) {   // uniform: nothing to load
#pragma unroll
        for (int it = 0; it < ITERS; it++)
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                t.hdr[nt][it] = make_uint4(0, 0, 0, 0);
                t.qa[nt][it] = make_uint4(0, 0, 0, 0);
                t.qb[nt][it] = make_uint4(0, 0, 0, 0);
            }
        return;
    }
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const int r0 = row0 + it * RPI + rsub;
        const int r = r0 < n ? r0 : n - 1;
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const uint8_t *rp = (nt == 0 ? w0 : w1) + uoff + (int64_t)r * nb01;
            t.hdr[nt][it] = *(const uint4 *)rp;
            t.qa[nt][it] = *(const uint4 *)(rp + 16 + 32 * c);
            t.qb[nt][it] = *(const uint4 *)(rp + 32 + 32 * c);
        }
    }
}

// Gate and up units (tile tensors 0 and 1) of row group `it` against the
// staged row at xrow, reading the activations once for both.  Same per-unit
// arithmetic and order as unit_from_tile.
template <int ITERS>
__device__ __forceinline__ void unit_pair_from_tile(const Tile<2, ITERS> &t, int it,
                                                    const float *xrow, int u, int c, int k,
                                                    float &v0, float &v1) {
    const float *xl = xrow + 68 * u;   // xpad(64u)
    const float4 *xa = (const float4 *)xl;
    const float4 *xb = (const float4 *)(xl + 32);
    UnitAcc acc0{0.0f, 0.0f}, acc1{0.0f, 0.0f};
    const uint32_t w0[8] = {t.qa[0][it].x, t.qa[0][it].y, t.qa[0][it].z, t.qa[0][it].w,
                            t.qb[0][it].x, t.qb[0][it].y, t.qb[0][it].z, t.qb[0][it].w};
    const uint32_t w1[8] = {t.qa[1][it].x, t.qa[1][it].y, t.qa[1][it].z, t.qa[1][it].w,
                            t.qb[1][it].x, t.qb[1][it].y, t.qb[1][it].z, t.qb[1][it].w};
#pragma unroll
    for (int d = 0; d < 8; d++) {
        const float4 va = xa[d], vb = xb[d];
        {
            const uint32_t v = w0[d], s = v >> 8;
            const uint32_t r[4] = {v & 0x000F000Fu, s & 0x000F000Fu, v & 0x00F000F0u,
                                   s & 0x00F000F0u};
            masked_fma(r, va, vb, acc0);
        }
        {
            const uint32_t v = w1[d], s = v >> 8;
            const uint32_t r[4] = {v & 0x000F000Fu, s & 0x000F000Fu, v & 0x00F000F0u,
                                   s & 0x00F000F0u};
            masked_fma(r, va, vb, acc1);
        }
    }
    const float *sx = xrow + xpad_len(k);
    const float sxa = sx[2 * u], sxb = sx[2 * u + 1];
    v0 = unit_value(unit_scale(t.hdr[0][it], c), acc0, sxa, sxb);
    v1 = unit_value(unit_scale(t.hdr[1][it], c), acc1, sxa, sxb);
}

// Unit value of tensor (nt, it) of the tile against the staged row at xrow.
template <int NT, int ITERS>
__device__ __forceinline__ float unit_from_tile(const Tile<NT, ITERS> &t, int nt, int it,
                                                const float *xrow, int u, int c, int k) {
    const float *xl = xrow + 68 * u;   // xpad(64u)
    const float4 *xa = (const float4 *)xl;
    const float4 *xb = (const float4 *)(xl + 32);
    UnitAcc acc{0.0f, 0.0f};
    const uint32_t w[8] = {t.qa[nt][it].x, t.qa[nt][it].y, t.qa[nt][it].z, t.qa[nt][it].w,
                           t.qb[nt][it].x, t.qb[nt][it].y, t.qb[nt][it].z, t.qb[nt][it].w};
#pragma unroll
    for (int d = 0; d < 8; d++) {
        const uint32_t v = w[d], s = v >> 8;
        const uint32_t r[4] = {v & 0x000F000Fu, s & 0x000F000Fu, v & 0x00F000F0u,
                               s & 0x00F000F0u};
        masked_fma(r, xa[d], xb[d], acc);
    }
    const float *sx = xrow + xpad_len(k);
    return unit_value(unit_scale(t.hdr[nt][it], c), acc, sx[2 * u], sx[2 * u + 1]);
}

// Bucket workspace views (layout documented with moe_bucket in q4kmoe.h).
struct BucketView {
    const int32_t *counts, *offsets, *pairs, *active, *n_active, *n_chunks, *chunks;
    __device__ BucketView(const int32_t *ws, int E, int P) {
        counts = ws;
        offsets = counts + (E + 1);
        pairs = offsets + (E + 2);
        active = pairs + P;
        n_active = active + (E + 1);
        n_chunks = n_active + 1;
        chunks = n_chunks + 1;
    }
};

// ------------------------------------------------------------ host side ---

// Bucketed mode on the matrix cores (q4k_mfma.hip).
hipError_t launch_q4k_gemv_mfma(const GemvArgs &a, bool fused_swiglu, hipStream_t st);

static inline int lanes_per_row(int k) {
    const int units = 4 * (k >> 8);
    int l = 4;
    while (l < units)
        l <<= 1;
    return l;
}

// Compute units of the current device (256 on MI355X), cached per device.
static inline int cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static inline size_t set_lds(const void *kern, size_t bytes) {
    if (bytes > 65536)
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return bytes;
}


}  // namespace q4k
