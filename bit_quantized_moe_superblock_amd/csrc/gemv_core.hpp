// Device core shared by the Q4_K GEMV kernels (q4k_gemv.hip, q4k_mfma.hip):
// kernel arguments, pair addressing, activation staging, the per-unit Q4_K
// arithmetic on the tile layout, and the row sums of a wave.
//
// Conventions (ferrum-kernels q4_k_moe_id_gemv_batched.rs, module doc: expert
// stacks [E, n, k/256] of 144-byte Q4_K superblocks, pair p = token*top_k +
// slot, activation row src1 + token*outer + slot*inner):
//   - the stacks are in the tile layout of common.hpp: expert e's matrix starts
//     at e * tiles_matrix_bytes(n, k);
//   - a unit is (row, superblock s, 32-byte nibble chunk c): 64 weights, sub-
//     block 2c in the low nibbles and 2c+1 in the high ones;
//   - activation rows are staged in LDS (padded so the lanes of a tile hit
//     different banks) with their 32-element sums, each taken in ascending
//     order from 0 by one thread.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace q4k {

// Epilogues of the vector-unit kernels: store the row value, store
// silu(gate) * up of the two matrices, or (a single matrix) store the values of
// two row groups of it.
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_ROWPAIR = 2 };

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
    int64_t mat;              // bytes of one expert matrix (tile layout)
    int n, k, top_k, num_experts, n_pairs, m_sh;
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
                 "s"(a.mat), "s"(a.n), "s"(a.k), "s"(a.top_k), "s"(a.num_experts),
                 "s"(a.n_pairs), "s"(a.m_sh), "s"(a.vec));
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
    if (q < a.n_pairs) {
        const int e = a.ids[q];
        const int t = q / a.top_k, s = q - t * a.top_k;
        r.valid = (unsigned)e < (unsigned)a.num_experts;
        const int64_t off = r.valid ? (int64_t)e * a.mat : 0;
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

// pair_ref from an id the caller has already loaded (e_raw: ids[q] for a
// routed pair) and the pair's activation row x.
__device__ __forceinline__ PairRef pair_ref_id(const GemvArgs &a, int q, int e_raw,
                                               const float *x) {
    PairRef r;
    r.x = x;
    if (q < a.n_pairs) {
        r.valid = (unsigned)e_raw < (unsigned)a.num_experts;
        const int64_t off = r.valid ? (int64_t)e_raw * a.mat : 0;
        r.w0 = a.w0 + off;
        r.w1 = a.w1 ? a.w1 + off : nullptr;
        r.out = a.dst + (int64_t)q * a.n;
    } else {
        r.valid = true;
        r.w0 = a.s0;
        r.w1 = a.s1;
        r.out = a.dst_sh + (int64_t)(q - a.n_pairs) * a.n;
    }
    return r;
}

// Activation row of pair q, when the caller knows (uniformly across the
// workgroup) whether the pair is a shared-expert pair.  A lane-varying choice
// between the two argument fields compiles into a per-lane load from the
// argument segment, whose wait would also wait for every weight load in flight.
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
    // Threads past the end re-load the last sub-block (clamped, never
    // committed) so the loads need no branch: a load under a branch makes
    // the wait-count pass lose the issue order at the join, and a later
    // wait for an earlier load then drains these too.  total >= 1.
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

// Stage rows [0, cl) starting at flattened sub-block `from`, in batches of
// NTHR (the workgroup's threads).  No barrier.
template <bool VEC, int NTHR, typename XOf>
__device__ __forceinline__ void stage_rows(XOf x_of, int cl, int k, float *lds, int from = 0) {
    const int total = cl * (k >> 5);
    for (int base = from; base < total; base += NTHR) {
        StageBatch b;
        stage_issue<VEC>(x_of, base, total, k, b);
        stage_commit(b, total, k, lds);
    }
}

// ------------------------------------------------------- unit arithmetic ----

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

template <int EPI, int NT>
__device__ __forceinline__ float epilogue(const float (&part)[NT]) {
    if constexpr (EPI == EPI_SWIGLU)
        return silu_mul(part[0], part[NT - 1]);
    else
        return part[0];
}

// ------------------------------------------------------------- tile steps ----
// A vector-unit step is one superblock s of 16 weight rows.  Lane l owns chunk
// c = (l >> 3) & 3 of row r8 = l & 7 of its half j = l >> 5 of the step; the
// halves are two row groups of one matrix (pair mode) or one row group of two
// matrices (token mode, two pairs).  Per load instruction the 32 lanes of a
// half read 512 contiguous bytes of one tile.
//
// The superblocks of a row fall into kClasses step classes, s = cls + 4t, so
// that four waves can share a row.  Every vector-unit kernel forms a row
// value in one order: per lane, the class's unit values in ascending t from
// 0; chunk_sum over the four chunk lanes; then the four class sums as
// ((p0 + p1) + p2) + p3 (a class without superblocks is +0).  Pair,
// bucketed and token modes therefore agree bit for bit, however they spread
// the classes over waves.
constexpr int kClasses = 4;

// Superblocks of class cls in a row of nb.
__host__ __device__ constexpr int class_steps(int nb, int cls) {
    return nb > cls ? (nb - cls + kClasses - 1) / kClasses : 0;
}

template <int NT>
struct Step {
    uint4 hdr[NT], qa[NT], qb[NT];
};

// Issue the lane's unit of superblock s, row group G, for NT matrices.
template <int NT>
__device__ __forceinline__ void load_step(const uint8_t *const (&mat)[NT], int64_t G, int s,
                                          int nb, Step<NT> &st) {
    const int l32 = threadIdx.x & 31, r8 = threadIdx.x & 7;
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const uint8_t *t = mat[nt] + tile_offset(G, s, nb);
        st.hdr[nt] = *(const uint4 *)(t + 16 * r8);
        st.qa[nt] = *(const uint4 *)(t + kTileHalf0 + 16 * l32);
        st.qb[nt] = *(const uint4 *)(t + kTileHalf1 + 16 * l32);
    }
}

// Unit values of a step for the NT matrices, added to acc[nt]: xu holds the
// unit's 64 activations, sums its two 32-element sums.  The activations are
// read once for all NT matrices.
template <int NT>
__device__ __forceinline__ void step_units(const Step<NT> &st, const float *xu, const float *sums,
                                           float (&acc)[NT]) {
    const int c = (threadIdx.x >> 3) & 3;
    const float4 *xa = (const float4 *)xu;
    const float4 *xb = (const float4 *)(xu + 32);
    UnitAcc ua[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
        ua[nt].a = ua[nt].b = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; d++) {
        const float4 va = xa[d], vb = xb[d];
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const uint4 &q = d < 4 ? st.qa[nt] : st.qb[nt];
            const uint32_t v = (d & 3) == 0 ? q.x : (d & 3) == 1 ? q.y : (d & 3) == 2 ? q.z : q.w;
            const uint32_t sh = v >> 8;
            const uint32_t r[4] = {v & 0x000F000Fu, sh & 0x000F000Fu, v & 0x00F000F0u,
                                   sh & 0x00F000F0u};
            masked_fma(r, va, vb, ua[nt]);
        }
    }
    const float sxa = sums[0], sxb = sums[1];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
        acc[nt] += unit_value(unit_scale(st.hdr[nt], c), ua[nt], sxa, sxb);
}

// Row total of a lane's class sum over the four chunk lanes (l ^ 8, then
// l ^ 16).  Lanes 0..7 and 32..39 hold the totals of the two halves' rows.
__device__ __forceinline__ float chunk_sum(float v) {
    v += dpp_move<0x128>(v);   // row_ror:8 within 16 lanes: the partner l ^ 8
    v += __shfl_xor(v, 16);
    return v;
}

// The row value from its four class sums (see kClasses).
__device__ __forceinline__ float class_total(float p0, float p1, float p2, float p3) {
    return ((p0 + p1) + p2) + p3;
}

// Per-wave activation staging of pair mode: a wave stages the superblocks of
// its class, one step (superblock) per kStepFloats LDS floats: the four units
// of 64 floats, each padded by 4 floats, then the 8 sub-block sums.  Lane
// 8u + j stages sub-block j of the wave's u-th superblock (in batches of 8
// superblocks), summing its 32 floats in ascending order from 0 as
// stage_commit does, so both stagings give the same sums.
constexpr int kStepFloats = 4 * 68 + 8;

struct WaveStage {
    float4 v[8];
};

// Lanes past the class's superblocks (or of a class without any) load a
// clamped superblock of the row and commit nothing, so the loads need no
// branch.
template <bool VEC>
__device__ __forceinline__ void wave_stage_issue(const float *x, int cls, int T, int t0, int nb,
                                                 WaveStage &b) {
    const int l = threadIdx.x & 63;
    const int t = t0 + (l >> 3);
    const int tc = t < T ? t : (T > 0 ? T - 1 : 0);
    const int sb = cls + kClasses * tc;
    const float *src = x + 256 * (sb < nb ? sb : nb - 1) + 32 * (l & 7);
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

__device__ __forceinline__ void wave_stage_commit(const WaveStage &b, int T, int t0, float *xw) {
    const int l = threadIdx.x & 63;
    const int t = t0 + (l >> 3), j = l & 7;
    if (t < T) {
        float *step = xw + t * kStepFloats;
        float4 *d = (float4 *)(step + 68 * (j >> 1) + 32 * (j & 1));
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            d[q] = b.v[q];
            s += b.v[q].x;
            s += b.v[q].y;
            s += b.v[q].z;
            s += b.v[q].w;
        }
        step[4 * 68 + j] = s;
    }
}

// This wave's LDS writes are complete and no LDS access moves across: the
// wave reads what its own lanes staged (no other wave is involved).
__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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
