// Indirect-dispatch Q4_K GEMV kernels for gfx950.
//
// What is computed (ferrum-kernels q4_k_moe_id_gemv_batched.rs, module doc and
// dispatch_gemv_q4k_moe_id_batched_on_encoder): for every (token, slot) pair
// p = token*top_k + slot, expert e = ids[p] and the activation row
// x = src1 + token*outer + slot*inner,
//     dst[p, r] = sum_c W_e[r, c] * x[c]   for r < n,
// with W_e stored as [n, k/256] Q4_K superblocks.  The fused variant reads a
// gate and an up stack with the same x and writes silu(gate)*up (the batched
// gate+up+SiLU dispatcher of the same page; moeflux expert_forward.rs SwiGLU).
// An optional shared expert (moeflux: the shared_out term of the combine) runs
// in the same launch as extra pairs, one per token, on its own one-expert stack.
//
// Device layout common to all kernels:
//   - 256 threads per workgroup; LPR consecutive lanes cover one weight row,
//     lane u owning unit u = (superblock u/4, 32-byte nibble chunk u%4), i.e.
//     64 weights: sub-block 2c in the low nibbles and 2c+1 in the high ones.
//     A row is read with coalesced 16-byte loads (header + two nibble halves);
//   - activation rows are staged in LDS (padded so a row's lanes hit different
//     banks) together with their 32-element sums, which carry the dmin*min term;
//   - a row's partial sums are reduced across its lanes (xor butterfly, then
//     through LDS when a row spans more than one wave).
// Kernels:
//   k_rows    pair mode: grid (row tiles, pairs [+ shared pairs]); a workgroup
//             loads ITERS row groups of one pair up front, then computes.
//   k_bucket  bucketed mode: grid (row groups, bucket slots [+ shared bucket]);
//             a workgroup holds one row group of one expert with its nibbles
//             already masked, and runs every pair of the expert's bucket
//             against it, PC pairs per LDS chunk, so each expert's weights are
//             read from HBM once per call (moeflux encode_moe_batched_permute_fuse).
//   k_down_combine  token mode for few tokens: a workgroup computes a row tile
//             of the down projection for all top_k (+ shared) pairs of one
//             token and applies the weighted residual combine in slot order
//             (moeflux moe_combine_residual).
// Every kernel runs the same per-unit arithmetic in the same order, so pair,
// bucketed and token modes give identical bits.
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

template <typename XOf>
__device__ __forceinline__ void stage_issue(XOf x_of, int base, int total, int k, bool vec,
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
    if (vec) {   // uniform
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
template <typename XOf>
__device__ __forceinline__ void stage_rows(XOf x_of, int cl, int k, bool vec, float *lds,
                                           int from = 0) {
    const int total = cl * (k >> 5);
    for (int base = from; base < total; base += kThreads) {
        StageBatch b;
        stage_issue(x_of, base, total, k, vec, b);
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

// ------------------------------------------------------------ pair mode ----

template <int LPR, int NT, int ITERS, int EPI>
__global__ __launch_bounds__(kThreads) void k_rows(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR;
    float *red = lds + row_lds_floats(a.k);
    const int q = blockIdx.y;
    const int row0 = blockIdx.x * (ITERS * RPI);
    const PairRef pr = pair_ref(a, q);
    const int tid = threadIdx.x;
    if (!pr.valid) {   // id outside [0, E): zero row
        for (int i = tid; i < ITERS * RPI; i += kThreads)
            if (row0 + i < a.n)
                pr.out[row0 + i] = 0.0f;
        return;
    }
    Tile<NT, ITERS> t;
    // Activation loads first, then the weights, then the LDS writes: the
    // weight loads are in flight while the activations are committed.
    const int total = a.k >> 5;
    StageBatch sb;
    stage_issue([&](int) { return pr.x; }, 0, total, a.k, a.vec, sb);
    load_rows<LPR, NT, ITERS>(pr.w0, pr.w1, a.n, a.k, row0, true, t);
    stage_commit(sb, total, a.k, lds);
    stage_rows([&](int) { return pr.x; }, 1, a.k, a.vec, lds, kThreads);
    __syncthreads();
    const int u = tid % LPR, rsub = tid / LPR, c = u & 3;
    const bool active = u < 4 * (a.k >> 8);
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        float part[NT];
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            float v = active ? unit_from_tile<NT, ITERS>(t, nt, it, lds, u, c, a.k) : 0.0f;
            part[nt] = row_reduce<LPR>(v, red, nt);
        }
        const int r = row0 + it * RPI + rsub;
        if (u == 0 && r < a.n)
            pr.out[r] = epilogue<EPI, NT>(part);
    }
}

// -------------------------------------------------------- bucketed mode ----

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

// Work item = one chunk (at most kBucketChunk pairs of one bucket, listed by
// the bucketing kernel) x one tile of ITERS*RPI rows.  The chunk's activation
// rows are staged in LDS (pc at a time); each lane keeps its ITERS x NT weight
// units in registers and reads every activation float once per pair for all of
// them.  Chunks past the routed ones carry the shared expert (all tokens).
template <int LPR, int NT, int ITERS, int EPI>
__global__ __launch_bounds__(kThreads) void k_bucket(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR;
    const BucketView bv(a.bucket, a.num_experts, a.n_pairs);
    const int y = blockIdx.y;
    const int nch = *bv.n_chunks;
    const int tid = threadIdx.x;
    const int row0 = blockIdx.x * (ITERS * RPI);
    int start, cnt;
    const uint8_t *w0, *w1;
    bool shared = false, zero = false;
    if (y < nch) {
        const int bkt = bv.chunks[2 * y];
        const int packed = bv.chunks[2 * y + 1];
        start = packed & 0xFFFFFF;
        cnt = packed >> 24;
        zero = bkt == a.num_experts;
        const int64_t off = zero ? 0 : (int64_t)bkt * a.n * (int64_t)(a.k >> 8) * kBlockBytes;
        w0 = a.w0 + off;
        w1 = a.w1 ? a.w1 + off : nullptr;
    } else if (a.m_sh > 0 && (y - nch) * kBucketChunk < a.m_sh) {
        shared = true;
        start = (y - nch) * kBucketChunk;
        cnt = a.m_sh - start < kBucketChunk ? a.m_sh - start : kBucketChunk;
        w0 = a.s0;
        w1 = a.s1;
    } else {
        return;
    }
    auto pair_of = [&](int i) { return shared ? a.n_pairs + start + i : bv.pairs[start + i]; };
    if (zero) {   // ids outside [0, E): zero rows
        for (int i = 0; i < cnt; i++) {
            float *out = a.dst + (int64_t)bv.pairs[start + i] * a.n;
            for (int r = tid; r < ITERS * RPI; r += kThreads)
                if (row0 + r < a.n)
                    out[row0 + r] = 0.0f;
        }
        return;
    }
    const int rl = row_lds_floats(a.k);
    float *red = lds + a.pc * rl;
    const int first = cnt < a.pc ? cnt : a.pc;
    auto xq = [&](int i) { return pair_x_known(a, shared, pair_of(i)); };
    const int total = first * (a.k >> 5);
    StageBatch sb;
    stage_issue(xq, 0, total, a.k, a.vec, sb);
    Tile<NT, ITERS> t;
    load_rows<LPR, NT, ITERS>(w0, w1, a.n, a.k, row0, true, t);
    stage_commit(sb, total, a.k, lds);
    stage_rows(xq, first, a.k, a.vec, lds, kThreads);
    const int u = tid % LPR, rsub = tid / LPR, c = u & 3;
    const bool active = u < 4 * (a.k >> 8);
    UnitScale sc[ITERS][NT];
#pragma unroll
    for (int it = 0; it < ITERS; it++)
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            sc[it][nt] = unit_scale(t.hdr[nt][it], c);
    for (int c0 = 0; c0 < cnt; c0 += a.pc) {
        const int cl = cnt - c0 < a.pc ? cnt - c0 : a.pc;
        if (c0 > 0) {
            __syncthreads();   // the previous pass is consumed
            stage_rows([&](int i) { return pair_x_known(a, shared, pair_of(c0 + i)); }, cl, a.k,
                       a.vec, lds);
        }
        __syncthreads();
        for (int i = 0; i < cl; i++) {
            const float *xrow = lds + i * rl;
            opaque(t);
            UnitAcc acc[ITERS][NT];
#pragma unroll
            for (int it = 0; it < ITERS; it++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    acc[it][nt].a = acc[it][nt].b = 0.0f;
            if (active) {
                const float4 *xa = (const float4 *)(xrow + 68 * u);
                const float4 *xb = xa + 8;
#pragma unroll
                for (int d = 0; d < 8; d++) {
                    const float4 va = xa[d], vb = xb[d];
#pragma unroll
                    for (int it = 0; it < ITERS; it++)
#pragma unroll
                        for (int nt = 0; nt < NT; nt++) {
                            const uint4 &q = d < 4 ? t.qa[nt][it] : t.qb[nt][it];
                            const uint32_t v = (d & 3) == 0 ? q.x : (d & 3) == 1 ? q.y
                                             : (d & 3) == 2 ? q.z : q.w;
                            const uint32_t sh = v >> 8;
                            const uint32_t r[4] = {v & 0x000F000Fu, sh & 0x000F000Fu,
                                                   v & 0x00F000F0u, sh & 0x00F000F0u};
                            masked_fma(r, va, vb, acc[it][nt]);
                        }
                }
            }
            const float *sx = xrow + xpad_len(a.k);
            const float sxA = active ? sx[2 * u] : 0.0f, sxB = active ? sx[2 * u + 1] : 0.0f;
            const int q = pair_of(c0 + i);
            float *out = q < a.n_pairs ? a.dst + (int64_t)q * a.n
                                       : a.dst_sh + (int64_t)(q - a.n_pairs) * a.n;
#pragma unroll
            for (int it = 0; it < ITERS; it++) {
                float part[NT];
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    const float v = active ? unit_value(sc[it][nt], acc[it][nt], sxA, sxB) : 0.0f;
                    part[nt] = row_reduce<LPR>(v, red, nt);
                }
                const int r = row0 + it * RPI + rsub;
                if (u == 0 && r < a.n)
                    out[r] = epilogue<EPI, NT>(part);
            }
        }
    }
}

// ------------------------------------------------ persistent bucketed ----
// A fixed grid of workgroups (CUs x resident workgroups) walks the work items
// (chunk, row tile) round-robin.  The chunk and pair lists are read into LDS
// once; each item's weights and activation loads are issued while the
// previous item computes, so HBM and L2 latency overlap with the arithmetic.
// One staging batch (256 sub-blocks of 32 floats) holds pc = 8192/k pairs;
// items with more pairs than that stage the rest synchronously.

constexpr int kPersistMaxPairs = 1024;

template <int NT, int ITERS>
struct Item {
    Tile<NT, ITERS> t;
    StageBatch xb;
    int chunk, tile;   // chunk < 0: no item
};

template <int LPR, int NT, int ITERS, int EPI>
__global__ __launch_bounds__(kThreads) void k_bucket_persist(GemvArgs a, int n_tiles) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR;
    const int tid = threadIdx.x;
    const int P = a.n_pairs, E = a.num_experts;
    int *meta = (int *)lds;                      // chunks[2P] | pairs[P]
    float *xs = lds + 3 * P;
    const int rl = row_lds_floats(a.k);
    float *red = xs + a.pc * rl;
    // chunk list and pair list into LDS in one round of loads
    const int32_t *ws = a.bucket;
    const int32_t *pairs_g = ws + (E + 1) + (E + 2);
    const int32_t *nch_g = pairs_g + P + (E + 1) + 1;
    const int32_t *chunks_g = nch_g + 1;
    for (int i = tid; i < 2 * P; i += kThreads)
        meta[i] = chunks_g[i];
    for (int i = tid; i < P; i += kThreads)
        meta[2 * P + i] = pairs_g[i];
    const int nch = *nch_g;
    __syncthreads();
    const int n_chunks = nch + (a.m_sh + kBucketChunk - 1) / kBucketChunk;
    const int n_items = n_chunks * n_tiles;
    const int u = tid % LPR, rsub = tid / LPR, c = u & 3;
    const bool active = u < 4 * (a.k >> 8);
    const int64_t mat = (int64_t)a.n * (int64_t)(a.k >> 8) * kBlockBytes;

    // (chunk) -> bucket, first pair position, pair count, weights
    auto chunk_info = [&](int ch, int &bkt, int &first, int &cnt, bool &shared) {
        if (ch < nch) {
            bkt = meta[2 * ch];
            const int pk = meta[2 * ch + 1];
            first = pk & 0xFFFFFF;
            cnt = pk >> 24;
            shared = false;
        } else {
            bkt = -1;
            first = (ch - nch) * kBucketChunk;
            cnt = a.m_sh - first < kBucketChunk ? a.m_sh - first : kBucketChunk;
            shared = true;
        }
    };
    auto pair_at = [&](bool shared, int first, int i) {
        return shared ? P + first + i : meta[2 * P + first + i];
    };
    auto issue = [&](int item, Item<NT, ITERS> &it) {
        if (item >= n_items) {
            it.chunk = -1;
            return;
        }
        it.chunk = item / n_tiles;
        it.tile = item - it.chunk * n_tiles;
        int bkt, first, cnt;
        bool shared;
        chunk_info(it.chunk, bkt, first, cnt, shared);
        const bool zero = !shared && bkt == E;
        const uint8_t *w0 = shared ? a.s0 : a.w0 + (zero ? 0 : (int64_t)bkt * mat);
        const uint8_t *w1 = shared ? a.s1 : (a.w1 ? a.w1 + (zero ? 0 : (int64_t)bkt * mat) : nullptr);
        load_rows<LPR, NT, ITERS>(w0, w1, a.n, a.k, it.tile * ITERS * RPI, !zero, it.t);
        const int cl = cnt < a.pc ? cnt : a.pc;
        stage_issue([&](int i) { return pair_x_known(a, shared, pair_at(shared, first, i)); }, 0,
                    zero ? 0 : cl * (a.k >> 5), a.k, a.vec, it.xb);
    };

    // Two item buffers in ping-pong: the next item loads into the buffer the
    // current one does not use (copying it over would wait for its loads).
    auto step = [&](int item, Item<NT, ITERS> &cur, Item<NT, ITERS> &nxt) {
        int bkt, first, cnt;
        bool shared;
        chunk_info(cur.chunk, bkt, first, cnt, shared);
        const bool zero = !shared && bkt == E;
        const int row0 = cur.tile * ITERS * RPI;
        const int cl0 = cnt < a.pc ? cnt : a.pc;
        __syncthreads();   // LDS of the previous item is consumed
        stage_commit(cur.xb, zero ? 0 : cl0 * (a.k >> 5), a.k, xs);
        issue(item + gridDim.x, nxt);   // next item's loads fly during this item
        if (zero) {
            for (int i = 0; i < cnt; i++) {
                float *out = a.dst + (int64_t)pair_at(false, first, i) * a.n;
                for (int r = tid; r < ITERS * RPI; r += kThreads)
                    if (row0 + r < a.n)
                        out[row0 + r] = 0.0f;
            }
        } else {
            UnitScale sc[ITERS][NT];
#pragma unroll
            for (int it = 0; it < ITERS; it++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    sc[it][nt] = unit_scale(cur.t.hdr[nt][it], c);
            for (int c0 = 0; c0 < cnt; c0 += a.pc) {
                const int cl = cnt - c0 < a.pc ? cnt - c0 : a.pc;
                if (c0 > 0) {
                    __syncthreads();
                    stage_rows([&](int i) {
                        return pair_x_known(a, shared, pair_at(shared, first, c0 + i));
                    }, cl, a.k, a.vec, xs);
                }
                __syncthreads();
                for (int i = 0; i < cl; i++) {
                    const float *xrow = xs + i * rl;
                    opaque(cur.t);
                    UnitAcc acc[ITERS][NT];
#pragma unroll
                    for (int it = 0; it < ITERS; it++)
#pragma unroll
                        for (int nt = 0; nt < NT; nt++)
                            acc[it][nt].a = acc[it][nt].b = 0.0f;
                    if (active) {
                        const float4 *xa = (const float4 *)(xrow + 68 * u);
                        const float4 *xb = xa + 8;
#pragma unroll
                        for (int d = 0; d < 8; d++) {
                            const float4 va = xa[d], vb = xb[d];
#pragma unroll
                            for (int it = 0; it < ITERS; it++)
#pragma unroll
                                for (int nt = 0; nt < NT; nt++) {
                                    const uint4 &q = d < 4 ? cur.t.qa[nt][it] : cur.t.qb[nt][it];
                                    const uint32_t v = (d & 3) == 0 ? q.x : (d & 3) == 1 ? q.y
                                                     : (d & 3) == 2 ? q.z : q.w;
                                    const uint32_t sh = v >> 8;
                                    const uint32_t r[4] = {v & 0x000F000Fu, sh & 0x000F000Fu,
                                                           v & 0x00F000F0u, sh & 0x00F000F0u};
                                    masked_fma(r, va, vb, acc[it][nt]);
                                }
                        }
                    }
                    const float *sx = xrow + xpad_len(a.k);
                    const float sxA = active ? sx[2 * u] : 0.0f;
                    const float sxB = active ? sx[2 * u + 1] : 0.0f;
                    const int q = pair_at(shared, first, c0 + i);
                    float *out = q < P ? a.dst + (int64_t)q * a.n
                                       : a.dst_sh + (int64_t)(q - P) * a.n;
#pragma unroll
                    for (int it = 0; it < ITERS; it++) {
                        float part[NT];
#pragma unroll
                        for (int nt = 0; nt < NT; nt++) {
                            const float v =
                                active ? unit_value(sc[it][nt], acc[it][nt], sxA, sxB) : 0.0f;
                            part[nt] = row_reduce<LPR>(v, red, nt);
                        }
                        const int r = row0 + it * RPI + rsub;
                        if (u == 0 && r < a.n)
                            out[r] = epilogue<EPI, NT>(part);
                    }
                }
            }
        }
            };
    Item<NT, ITERS> A, B;
    issue(blockIdx.x, A);
    for (int item = blockIdx.x; item < n_items; item += 2 * gridDim.x) {
        step(item, A, B);
        if (item + gridDim.x < n_items)
            step(item + gridDim.x, B, A);
    }
}

// ---------------------------------------------------- down + combine mode ----
// Workgroup = (token t, TRT rows).  Slots enumerate (row, pair) with the pair
// fastest: pairs 0..top_k-1 are the token's routed pairs, pair top_k the shared
// expert.  out[t,r] = h_mid[t,r] + sum_s w[t,s]*y_s[r] + g_t*y_sh[r] with the
// same fma order as the combine kernel.

struct CombineArgs {
    const float *h_mid, *route_w, *shared_logit;
    float *out;
    float *expert_out;   // optional [n_pairs, n] copy of the routed rows
    int shared_mode;
};

template <int LPR, int ITERS>
__global__ __launch_bounds__(kThreads) void k_down_combine(GemvArgs a, CombineArgs cb, int trt) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR;
    const int tok = blockIdx.y;
    const int K = a.top_k;
    const int np = K + (a.m_sh > 0 ? 1 : 0);   // pairs of this token
    const int rl = row_lds_floats(a.k);
    float *ybuf = lds + np * rl;                // [trt][np]
    float *red = ybuf + trt * np;
    const int tid = threadIdx.x;
    const int row0 = blockIdx.x * trt;
    // 1. the token's experts: uniform (scalar) loads, issued first
    int ex[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; s++)
        ex[s] = s < K ? a.ids[tok * K + s] : 0;
    // 2. slot it*RPI + rsub -> (row row0 + slot/np, pair slot%np); weight loads
    const int u = tid % LPR, rsub = tid / LPR, c = u & 3;
    const int nb = a.k >> 8;
    const bool active = u < 4 * nb;
    const int64_t nb01 = (int64_t)nb * kBlockBytes;
    Tile<1, ITERS> t;
    int sp[ITERS], sr[ITERS];
    bool sok[ITERS];
    const int ul = active ? u : 0;   // clamped unit (see load_rows)
    const int cl = ul & 3;
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const int slot = it * RPI + rsub;
        sr[it] = slot / np;
        sp[it] = slot - sr[it] * np;
        bool ok = sr[it] < trt && row0 + sr[it] < a.n;
        const uint8_t *base;
        if (sp[it] < K) {
            int e = ex[0];
#pragma unroll
            for (int s = 1; s < kMaxTopK; s++)
                e = sp[it] == s ? ex[s] : e;
            const bool ev = (unsigned)e < (unsigned)a.num_experts;
            ok = ok && ev;
            base = a.w0 + (ev ? (int64_t)e * a.n * nb01 : 0);
        } else {
            base = a.s0;
        }
        sok[it] = ok;
        const int r0 = row0 + sr[it];
        const int r = r0 < a.n ? r0 : a.n - 1;
        const uint8_t *rp = base + (int64_t)(ul >> 2) * kBlockBytes + (int64_t)r * nb01;
        t.hdr[0][it] = *(const uint4 *)rp;
        t.qa[0][it] = *(const uint4 *)(rp + 16 + 32 * cl);
        t.qb[0][it] = *(const uint4 *)(rp + 32 + 32 * cl);
    }
    // 3. combine inputs of this thread's output row, prefetched
    const int ri = tid;
    const int64_t o = (int64_t)tok * a.n + row0 + ri;
    const bool rowok = ri < trt && row0 + ri < a.n;
    const float hm = rowok ? cb.h_mid[o] : 0.0f;
    // 4. activation rows of the token's pairs (routed rows, then the shared
    //    row); both bases are uniform, lanes pick between the two values
    const float *xr = a.src1 + tok * a.outer;
    const float *xsh = a.m_sh > 0 ? a.src1_sh + tok * a.outer_sh : xr;
    const int64_t inner = a.inner;
    stage_rows([&](int s) { return s < K ? xr + s * inner : xsh; }, np, a.k, a.vec, lds);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const float *xrow = lds + sp[it] * rl;
        float v = (active && sok[it]) ? unit_from_tile<1, ITERS>(t, 0, it, xrow, u, c, a.k) : 0.0f;
        v = row_reduce<LPR>(v, red, 0);
        if (u == 0 && sr[it] < trt)
            ybuf[sr[it] * np + sp[it]] = v;
    }
    __syncthreads();
    if (rowok) {
        const int r = row0 + ri;
        float acc = hm;
        for (int s = 0; s < K; s++) {
            const float yv = ybuf[ri * np + s];
            acc = __builtin_fmaf(cb.route_w[tok * K + s], yv, acc);
            if (cb.expert_out)
                cb.expert_out[(int64_t)(tok * K + s) * a.n + r] = yv;
        }
        if (a.m_sh > 0) {
            const float ysh = ybuf[ri * np + K];
            if (cb.shared_mode == 1) {
                const float g = 1.0f / (1.0f + expf(-cb.shared_logit[tok]));
                acc = __builtin_fmaf(g, ysh, acc);
            } else if (cb.shared_mode == 2) {
                acc += ysh;
            }
            if (a.dst_sh)
                a.dst_sh[o] = ysh;
        }
        cb.out[o] = acc;
    }
}

// ------------------------------------------------------------------ host ---

static int lanes_per_row(int k) {
    const int units = 4 * (k >> 8);
    int l = 4;
    while (l < units)
        l <<= 1;
    return l;
}

static int env_int(const char *name, int dflt) {
    const char *s = getenv(name);
    return s ? atoi(s) : dflt;
}

// Row groups per workgroup in pair mode: as tall as possible while the grid
// still gives every CU a workgroup (256 CUs on MI355X).
static int pick_iters(int64_t pairs, int n, int rpi) {
    static const int forced = env_int("Q4KMOE_ITERS", 0);
    if (forced == 1 || forced == 2 || forced == 3 || forced == 4 || forced == 6 || forced == 8)
        return forced;
    const int cand[] = {8, 6, 4, 3, 2};
    for (int it : cand) {
        const int64_t tiles = (n + it * rpi - 1) / (it * rpi);
        if (tiles * pairs >= 256)
            return it;
    }
    return 1;
}

// Compute units of the current device (256 on MI355X), cached per device.
static int cu_count() {
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

static size_t set_lds(const void *kern, size_t bytes) {
    if (bytes > 65536)
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return bytes;
}

template <int LPR, int NT, int EPI, int IT>
static hipError_t go_rows(const GemvArgs &a, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    auto kern = k_rows<LPR, NT, IT, EPI>;
    const size_t lds = set_lds((const void *)kern, (row_lds_floats(a.k) + 8) * sizeof(float));
    dim3 grid((a.n + IT * RPI - 1) / (IT * RPI), a.n_pairs + a.m_sh);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

template <int LPR, int NT, int EPI>
static hipError_t launch_lpr(GemvArgs a, bool bucketed, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    if (bucketed && a.k <= 8192 && a.n_pairs <= kPersistMaxPairs &&
        env_int("Q4KMOE_PERSIST", 1) != 0) {
        constexpr int IT = NT == 2 ? 2 : 4;
        const int rl = row_lds_floats(a.k);
        a.pc = 8192 / a.k < kBucketChunk ? 8192 / a.k : kBucketChunk;
        auto kern = k_bucket_persist<LPR, NT, IT, EPI>;
        const size_t lds = set_lds((const void *)kern,
                                   ((size_t)3 * a.n_pairs + (size_t)a.pc * rl + 8) * sizeof(float));
        const int n_tiles = (a.n + IT * RPI - 1) / (IT * RPI);
        // every workgroup of a persistent grid must be resident at once
        int fit = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, (const void *)kern, kThreads,
                                                         lds) != hipSuccess || fit < 1)
            fit = 1;
        static const int per_cu = env_int("Q4KMOE_PERSIST_WG", 2);
        const int wg = per_cu < fit ? per_cu : fit;
        hipLaunchKernelGGL(kern, dim3(cu_count() * (wg < 1 ? 1 : wg)), dim3(kThreads), lds, st,
                           a, n_tiles);
        return hipGetLastError();
    }
    if (bucketed) {
        constexpr int IT = NT == 2 ? 2 : 4;
        const int rl = row_lds_floats(a.k);
        static const int budget = env_int("Q4KMOE_CHUNK_LDS", 40 * 1024);
        int pc = (int)((budget / 4 - 8) / rl);
        pc = pc < 1 ? 1 : (pc > kBucketChunk ? kBucketChunk : pc);
        a.pc = pc;
        auto kern = k_bucket<LPR, NT, IT, EPI>;
        const size_t lds = set_lds((const void *)kern, ((size_t)pc * rl + 8) * sizeof(float));
        const int shared_chunks = (a.m_sh + kBucketChunk - 1) / kBucketChunk;
        dim3 grid((a.n + IT * RPI - 1) / (IT * RPI), a.n_pairs + shared_chunks);
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
        return hipGetLastError();
    }
    int it = pick_iters(a.n_pairs + a.m_sh, a.n, RPI);
    if (NT == 2 && it > 4)
        it = 4;
    switch (it) {
    case 8: return go_rows<LPR, NT, EPI, (NT == 2 ? 4 : 8)>(a, st);
    case 6: return go_rows<LPR, NT, EPI, (NT == 2 ? 4 : 6)>(a, st);
    case 4: return go_rows<LPR, NT, EPI, 4>(a, st);
    case 3: return go_rows<LPR, NT, EPI, 3>(a, st);
    case 2: return go_rows<LPR, NT, EPI, 2>(a, st);
    default: return go_rows<LPR, NT, EPI, 1>(a, st);
    }
}

template <int NT, int EPI>
static hipError_t launch_any(const GemvArgs &a, bool bucketed, hipStream_t st) {
    switch (lanes_per_row(a.k)) {
    case 4: return launch_lpr<4, NT, EPI>(a, bucketed, st);
    case 8: return launch_lpr<8, NT, EPI>(a, bucketed, st);
    case 16: return launch_lpr<16, NT, EPI>(a, bucketed, st);
    case 32: return launch_lpr<32, NT, EPI>(a, bucketed, st);
    case 64: return launch_lpr<64, NT, EPI>(a, bucketed, st);
    case 128: return launch_lpr<128, NT, EPI>(a, bucketed, st);
    case 256: return launch_lpr<256, NT, EPI>(a, bucketed, st);
    default: return hipErrorInvalidValue;
    }
}

static bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static GemvArgs make_args(const GemvLaunch &L) {
    GemvArgs a{};
    a.w0 = (const uint8_t *)L.w0;
    a.w1 = (const uint8_t *)L.w1;
    a.s0 = (const uint8_t *)L.s0;
    a.s1 = (const uint8_t *)L.s1;
    a.src1 = L.src1;
    a.src1_sh = L.src1_sh;
    a.ids = L.ids;
    a.bucket = L.bucket_ws;
    a.dst = L.dst;
    a.dst_sh = L.dst_sh;
    a.outer = L.outer;
    a.inner = L.inner;
    a.outer_sh = L.outer_sh;
    a.n = (int)L.n;
    a.k = (int)L.k;
    a.top_k = (int)L.top_k;
    a.num_experts = (int)L.num_experts;
    a.n_pairs = (int)L.n_pairs;
    a.m_sh = (int)L.m_sh;
    a.vec = al16(L.src1) && L.outer % 4 == 0 && L.inner % 4 == 0 &&
            (L.m_sh == 0 || (al16(L.src1_sh) && L.outer_sh % 4 == 0));
    return a;
}

hipError_t launch_q4k_gemv(const GemvLaunch &L, hipStream_t st) {
    const GemvArgs a = make_args(L);
    const bool bucketed = L.bucket_ws != nullptr;
    if (L.fused_swiglu)
        return launch_any<2, EPI_SWIGLU>(a, bucketed, st);
    return launch_any<1, EPI_STORE>(a, bucketed, st);
}

template <int LPR, int IT>
static hipError_t go_dc(const GemvArgs &a, const CombineArgs &cb, int trt, hipStream_t st) {
    auto kern = k_down_combine<LPR, IT>;
    const int np = a.top_k + (a.m_sh > 0 ? 1 : 0);
    const size_t lds = set_lds((const void *)kern,
                               ((size_t)np * row_lds_floats(a.k) + trt * np + 8) * sizeof(float));
    if (trt > kThreads)
        return hipErrorInvalidValue;
    dim3 grid((a.n + trt - 1) / trt, (int)(a.n_pairs / a.top_k));
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a, cb, trt);
    return hipGetLastError();
}

template <int LPR>
static hipError_t dc_lpr(const GemvArgs &a, const CombineArgs &cb, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    const int np = a.top_k + (a.m_sh > 0 ? 1 : 0);
    const int m = a.n_pairs / a.top_k;
    // rows per workgroup: the tallest tile that still gives two workgroups
    // per CU (256 CUs) and at most 8 row groups per lane
    static const int forced = env_int("Q4KMOE_DC_ROWS", 0);
    int trt = 1;
    for (int cand = 64; cand >= 1; cand >>= 1) {
        const int its = (cand * np + RPI - 1) / RPI;
        if (its <= 8 && (int64_t)((a.n + cand - 1) / cand) * m >= 512) {
            trt = cand;
            break;
        }
    }
    if (forced > 0 && forced <= 64 && (forced * np + RPI - 1) / RPI <= 8)
        trt = forced;
    const int its = (trt * np + RPI - 1) / RPI;
    if (its <= 1) return go_dc<LPR, 1>(a, cb, trt, st);
    if (its <= 2) return go_dc<LPR, 2>(a, cb, trt, st);
    if (its <= 4) return go_dc<LPR, 4>(a, cb, trt, st);
    if (its <= 6) return go_dc<LPR, 6>(a, cb, trt, st);
    return go_dc<LPR, 8>(a, cb, trt, st);
}

hipError_t launch_q4k_down_combine(const GemvLaunch &L, const float *h_mid, const float *route_w,
                                   const float *shared_logit, float *out, float *expert_out,
                                   int shared_mode, hipStream_t st) {
    const GemvArgs a = make_args(L);
    CombineArgs cb{h_mid, route_w, shared_logit, out, expert_out, shared_mode};
    switch (lanes_per_row(a.k)) {
    case 4: return dc_lpr<4>(a, cb, st);
    case 8: return dc_lpr<8>(a, cb, st);
    case 16: return dc_lpr<16>(a, cb, st);
    case 32: return dc_lpr<32>(a, cb, st);
    case 64: return dc_lpr<64>(a, cb, st);
    case 128: return dc_lpr<128>(a, cb, st);
    case 256: return dc_lpr<256>(a, cb, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace q4k
