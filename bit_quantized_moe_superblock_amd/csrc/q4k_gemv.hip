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
// Device layout common to all kernels (helpers in gemv_core.hpp):
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
//   k_bucket  bucketed mode on the vector units: grid (row groups, chunk
//             slots [+ shared chunks]); a workgroup holds one row group of one
//             expert in registers and runs every pair of its chunk against it,
//             PC pairs per LDS batch, so each expert's weights are read from
//             HBM once per chunk (moeflux encode_moe_batched_permute_fuse).
//             The matrix-core kernels (q4k_mfma.hip) are the default bucketed
//             schedule; this one is selected explicitly.
//   k_down_combine  token mode for few tokens: a workgroup computes a row tile
//             of the down projection for all top_k (+ shared) pairs of one
//             token and applies the weighted residual combine in slot order
//             (moeflux moe_combine_residual).
// Every kernel here runs the same per-unit arithmetic in the same order, so
// pair, vector-unit bucketed and token modes give identical bits.  Activation
// rows need only be 4-byte aligned: staging uses float4 loads when rows and
// strides are 16-byte aligned, 4-byte loads otherwise, with the same sums.
#include <stdint.h>

#include "gemv_core.hpp"

namespace q4k {

// ------------------------------------------------------------ pair mode ----

// The pair's activation row is staged once per workgroup in LDS (a thread
// per 32-float sub-block, loads issued ahead of the weights, committed with
// its sub-block sum) and every lane reads its unit's 64 activations from
// there.
template <int LPR, int NT, int ITERS, int EPI, bool VEC>
__global__ __launch_bounds__(kThreads) void k_rows(GemvArgs a) {
    extern __shared__ float lds[];
    fetch_args(a);
    constexpr int RPI = kThreads / LPR;
    float *red = lds;        // cross-wave row sums (rows wider than a wave)
    float *xs = lds + 16;    // staged activation row
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
    const int u = tid % LPR, rsub = tid / LPR;
    const bool active = u < 4 * (a.k >> 8);
    const int ul = active ? u : 0, cl = ul & 3;   // clamped unit (see load_rows)
    const int nsub = a.k >> 5;
    auto x_of = [&](int) { return pr.x; };
    StageBatch xb;
    stage_issue<VEC>(x_of, 0, nsub, a.k, xb);
    __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the weights
    Tile<NT, ITERS> t;
    load_rows<LPR, NT, ITERS>(pr.w0, pr.w1, a.n, a.k, row0, true, t);
    stage_commit(xb, nsub, a.k, xs);
    stage_rows<VEC>(x_of, 1, a.k, xs, kThreads);   // k > 8192
    lds_barrier();
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        // Computed on every lane (inactive lanes hold a clamped, valid unit)
        // and then selected: under a branch the compiler sinks part of the
        // weight loads into it, and their wait drains the queue.
        float part[NT];
        if constexpr (NT == 2) {
            float v0, v1;
            unit_pair_from_tile<ITERS>(t, it, xs, ul, cl, a.k, v0, v1);
            part[0] = row_reduce<LPR>(active ? v0 : 0.0f, red, 0);
            part[1] = row_reduce<LPR>(active ? v1 : 0.0f, red, 1);
        } else {
            const float uv = unit_from_tile<NT, ITERS>(t, 0, it, xs, ul, cl, a.k);
            part[0] = row_reduce<LPR>(active ? uv : 0.0f, red, 0);
        }
        const int r = row0 + it * RPI + rsub;
        if (u == 0 && r < a.n)
            pr.out[r] = epilogue<EPI, NT>(part);
    }
}

// -------------------------------------------------------- bucketed mode ----


// Work item = one chunk (at most kBucketChunk pairs of one bucket, listed by
// the bucketing kernel) x one tile of ITERS*RPI rows.  The chunk's activation
// rows are staged in LDS (pc at a time); each lane keeps its ITERS x NT weight
// units in registers and reads every activation float once per pair for all of
// them.  Chunks past the routed ones carry the shared expert (all tokens).
template <int LPR, int NT, int ITERS, int EPI, bool VEC>
__global__ __launch_bounds__(kThreads) void k_bucket(GemvArgs a) {
    extern __shared__ float lds[];
    fetch_args(a);
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
    stage_issue<VEC>(xq, 0, total, a.k, sb);
    Tile<NT, ITERS> t;
    load_rows<LPR, NT, ITERS>(w0, w1, a.n, a.k, row0, true, t);
    stage_commit(sb, total, a.k, lds);
    stage_rows<VEC>(xq, first, a.k, lds, kThreads);
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
            stage_rows<VEC>([&](int i) { return pair_x_known(a, shared, pair_of(c0 + i)); }, cl,
                            a.k, lds);
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

template <int LPR, int ITERS, bool VEC>
__global__ __launch_bounds__(kThreads) void k_down_combine(GemvArgs a, CombineArgs cb, int trt) {
    extern __shared__ float lds[];
    fetch_args(a);
    asm volatile("" ::"s"(cb.h_mid), "s"(cb.route_w), "s"(cb.shared_logit), "s"(cb.out),
                 "s"(cb.expert_out), "s"(cb.shared_mode), "s"(trt));
    constexpr int RPI = kThreads / LPR;
    const int tok = blockIdx.y;
    const int K = a.top_k;
    const int np = K + (a.m_sh > 0 ? 1 : 0);   // pairs of this token
    const int rl = row_lds_floats(a.k);
    float *ybuf = lds + np * rl;                // [trt][np]
    float *red = ybuf + trt * np;
    const int tid = threadIdx.x;
    const int row0 = blockIdx.x * trt;
    // 1. the token's experts into LDS (-1 for ids outside [0, E)): one load
    //    per thread, unconditional with a clamped index (a load under a
    //    divergent branch makes later waits drain the whole queue), the only
    //    load in flight when it is waited for.  A per-lane select over the
    //    ids held in registers would become an indexed array in scratch.
    __shared__ int ex_lds[kMaxTopK];
    __shared__ float rw_lds[kMaxTopK];
    const int e_own = a.ids[tok * K + (tid < K ? tid : K - 1)];
    // The combine's routing weights and shared-expert gate logit are loaded
    // here, with the ids, so that the combine at the end waits on no memory.
    const float rw_own = cb.route_w[tok * K + (tid < K ? tid : K - 1)];
    const bool gated = a.m_sh > 0 && cb.shared_mode == 1;   // uniform
    const float logit = gated ? cb.shared_logit[tok] : 0.0f;
    // The first staging batch of the token's activation rows (routed rows,
    // then the shared row; both bases are uniform, lanes pick between the two
    // values) is issued next, ahead of the weights, with a clamped index and
    // no branch: waiting for the ids above leaves it in flight, and
    // committing it below waits for it alone.
    const float *xr = a.src1 + tok * a.outer;
    const float *xsh = a.m_sh > 0 ? a.src1_sh + tok * a.outer_sh : xr;
    const int64_t inner = a.inner;
    auto x_of = [&](int s) { return s < K ? xr + s * inner : xsh; };
    const int nsub = a.k >> 5;
    const int total = np * nsub;
    StageBatch xb;
    stage_issue<VEC>(x_of, 0, total, a.k, xb);
    if (tid < K) {
        ex_lds[tid] = (unsigned)e_own < (unsigned)a.num_experts ? e_own : -1;
        rw_lds[tid] = rw_own;
    }
    lds_barrier();
    // 2. slot it*RPI + rsub -> (row row0 + slot/np, pair slot%np); weight
    //    loads, branch-free (clamped addresses; the shared pair selects its
    //    own stack)
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
        const bool routed = sp[it] < K;
        const int e = ex_lds[routed ? sp[it] : 0];
        sok[it] = sr[it] < trt && row0 + sr[it] < a.n && (!routed || e >= 0);
        const int64_t eoff = routed && e >= 0 ? (int64_t)e * a.n * nb01 : 0;
        const uint8_t *base = (routed ? a.w0 : a.s0) + eoff;
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
    // 4. activation rows of the token's pairs into LDS (first batch, then any
    //    further ones)
    stage_commit(xb, total, a.k, lds);
    stage_rows<VEC>(x_of, np, a.k, lds, kThreads);
    lds_barrier();
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const float *xrow = lds + sp[it] * rl;
        // computed on every lane, then selected (see k_rows)
        const float uv = unit_from_tile<1, ITERS>(t, 0, it, xrow, ul, cl, a.k);
        const float v = row_reduce<LPR>((active && sok[it]) ? uv : 0.0f, red, 0);
        if (u == 0 && sr[it] < trt)
            ybuf[sr[it] * np + sp[it]] = v;
    }
    __syncthreads();
    if (rowok) {
        const int r = row0 + ri;
        float acc = hm;
        for (int s = 0; s < K; s++) {
            const float yv = ybuf[ri * np + s];
            acc = __builtin_fmaf(rw_lds[s], yv, acc);
            if (cb.expert_out)
                cb.expert_out[(int64_t)(tok * K + s) * a.n + r] = yv;
        }
        if (a.m_sh > 0) {
            const float ysh = ybuf[ri * np + K];
            if (cb.shared_mode == 1) {
                const float g = 1.0f / (1.0f + expf(-logit));
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

// Row groups per workgroup in pair mode: as tall as possible while the grid
// still gives every CU a workgroup (256 CUs on MI355X).
static int pick_iters(int64_t pairs, int n, int rpi, int max_it) {
    // Smallest (waves of workgroups over the CUs) x (row groups per
    // workgroup): a grid just past a multiple of the CU count leaves some CUs
    // with twice the work of the rest.  Ties go to a grid that gives every CU
    // a workgroup (one workgroup alone on a CU leaves one wave per SIMD, with
    // nothing to hide its latency), then to the taller tile.
    const int64_t cus = cu_count();
    const int cand[] = {1, 2, 3, 4, 6, 8};
    int best = 1;
    int64_t best_cost = INT64_MAX;
    bool best_fills = false;
    for (int it : cand) {
        if (it > max_it)
            break;
        const int64_t tiles = (n + it * rpi - 1) / (it * rpi);
        const int64_t cost = (tiles * pairs + cus - 1) / cus * it;
        const bool fills = tiles * pairs >= cus;
        if (cost < best_cost || (cost == best_cost && (fills || !best_fills))) {
            best = it;
            best_cost = cost;
            best_fills = fills;
        }
    }
    return best;
}

// Row groups per workgroup with the activation row staged in LDS: the
// shortest tile whose staged row (4k bytes, read from the cache) is at most
// half of its weight bytes and whose grid still gives every CU a workgroup
// (more, smaller workgroups hide each other's latency); otherwise the rule
// above.
static int pick_iters_staged(int64_t pairs, int n, int rpi, int max_it, int k, int nt) {
    const int64_t cus = cu_count();
    const int64_t rowb = (int64_t)(k >> 8) * kBlockBytes;
    const int cand[] = {1, 2, 3, 4, 6, 8};
    for (int it : cand) {
        if (it > max_it)
            break;
        const int64_t tiles = (n + it * rpi - 1) / (it * rpi);
        if (8 * (int64_t)k <= (int64_t)it * rpi * nt * rowb && tiles * pairs >= cus)
            return it;
    }
    return pick_iters(pairs, n, rpi, max_it);
}

template <int LPR, int NT, int EPI, int IT>
static hipError_t go_rows(const GemvArgs &a, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    dim3 grid((a.n + IT * RPI - 1) / (IT * RPI), a.n_pairs + a.m_sh);
    auto go = [&](auto kern) {
        const size_t lds =
            set_lds((const void *)kern, (16 + (size_t)row_lds_floats(a.k)) * sizeof(float));
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
        return hipGetLastError();
    };
    return a.vec ? go(k_rows<LPR, NT, IT, EPI, true>) : go(k_rows<LPR, NT, IT, EPI, false>);
}

// LDS budget of the vector-unit bucketed kernel's staged activation rows.
constexpr int kBucketLdsBytes = 40 * 1024;

template <int LPR, int NT, int EPI>
static hipError_t launch_lpr(GemvArgs a, bool bucketed, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    if (bucketed) {
        constexpr int IT = NT == 2 ? 2 : 4;
        const int rl = row_lds_floats(a.k);
        int pc = (int)((kBucketLdsBytes / 4 - 8) / rl);
        pc = pc < 1 ? 1 : (pc > kBucketChunk ? kBucketChunk : pc);
        a.pc = pc;
        const int shared_chunks = (a.m_sh + kBucketChunk - 1) / kBucketChunk;
        dim3 grid((a.n + IT * RPI - 1) / (IT * RPI), a.n_pairs + shared_chunks);
        auto go = [&](auto kern) {
            const size_t lds = set_lds((const void *)kern, ((size_t)pc * rl + 8) * sizeof(float));
            hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
            return hipGetLastError();
        };
        return a.vec ? go(k_bucket<LPR, NT, IT, EPI, true>) : go(k_bucket<LPR, NT, IT, EPI, false>);
    }
    const int max_it = NT == 2 ? 4 : 8;
    switch (pick_iters_staged(a.n_pairs + a.m_sh, a.n, RPI, max_it, a.k, NT)) {
    case 8: return go_rows<LPR, NT, EPI, (NT == 2 ? 4 : 8)>(a, st);
    case 6: return go_rows<LPR, NT, EPI, (NT == 2 ? 4 : 6)>(a, st);
    case 4: return go_rows<LPR, NT, EPI, 4>(a, st);
    case 3: return go_rows<LPR, NT, EPI, 3>(a, st);
    case 2: return go_rows<LPR, NT, EPI, 2>(a, st);
    default: return go_rows<LPR, NT, EPI, 1>(a, st);
    }
}

// k in [256, Q4K_MAX_IN] and a multiple of 256 (validated by the caller), so
// lanes_per_row(k) is one of the cases.
template <int NT, int EPI>
static hipError_t launch_any(const GemvArgs &a, bool bucketed, hipStream_t st) {
    switch (lanes_per_row(a.k)) {
    case 4: return launch_lpr<4, NT, EPI>(a, bucketed, st);
    case 8: return launch_lpr<8, NT, EPI>(a, bucketed, st);
    case 16: return launch_lpr<16, NT, EPI>(a, bucketed, st);
    case 32: return launch_lpr<32, NT, EPI>(a, bucketed, st);
    case 64: return launch_lpr<64, NT, EPI>(a, bucketed, st);
    case 128: return launch_lpr<128, NT, EPI>(a, bucketed, st);
    default: return launch_lpr<256, NT, EPI>(a, bucketed, st);
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

bool q4k_self_bucket_ok(const GemvLaunch &L) {
    return L.n_pairs <= kSelfBucketMaxPairs && L.num_experts + 1 <= kSelfBucketMaxBuckets;
}

hipError_t launch_q4k_gemv(const GemvLaunch &L, hipStream_t st) {
    const GemvArgs a = make_args(L);
    if (L.self_bucket)   // chunks built in-kernel: the matrix-core kernel only
        return launch_q4k_gemv_mfma(a, L.fused_swiglu, st);
    const bool bucketed = L.bucket_ws != nullptr;
    if (bucketed && !L.vector_units)
        return launch_q4k_gemv_mfma(a, L.fused_swiglu, st);
    if (L.fused_swiglu)
        return launch_any<2, EPI_SWIGLU>(a, bucketed, st);
    return launch_any<1, EPI_STORE>(a, bucketed, st);
}

// LDS of k_down_combine: np staged rows, the slot results of at most 64 rows
// and a few words; the CDNA4 limit is 160 KB per workgroup.
static size_t dc_lds_bytes(int64_t k, int np, int trt) {
    return ((size_t)np * row_lds_floats((int)k) + (size_t)trt * np + 8) * sizeof(float);
}

bool q4k_down_combine_ok(int64_t k, int64_t top_k, bool shared) {
    return dc_lds_bytes(k, (int)top_k + (shared ? 1 : 0), 64) <= 160 * 1024;
}

template <int LPR, int IT>
static hipError_t go_dc(const GemvArgs &a, const CombineArgs &cb, int trt, hipStream_t st) {
    const int np = a.top_k + (a.m_sh > 0 ? 1 : 0);
    dim3 grid((a.n + trt - 1) / trt, (int)(a.n_pairs / a.top_k));
    auto go = [&](auto kern) {
        const size_t lds = set_lds((const void *)kern, dc_lds_bytes(a.k, np, trt));
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a, cb, trt);
        return hipGetLastError();
    };
    return a.vec ? go(k_down_combine<LPR, IT, true>) : go(k_down_combine<LPR, IT, false>);
}

template <int LPR>
static hipError_t dc_lpr(const GemvArgs &a, const CombineArgs &cb, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    const int np = a.top_k + (a.m_sh > 0 ? 1 : 0);
    const int m = a.n_pairs / a.top_k;
    // rows per workgroup: the tallest tile that still gives every CU a
    // workgroup, with at most 8 row groups per lane (every workgroup stages
    // all of the token's activation rows, so taller tiles stage less in all);
    // at most 64 rows, so the combine's thread per row fits the workgroup
    const int64_t cus = cu_count();
    int trt = 1;
    for (int cand = 64; cand >= 1; cand >>= 1) {
        const int its = (cand * np + RPI - 1) / RPI;
        if (its <= 8 && (int64_t)((a.n + cand - 1) / cand) * m >= cus) {
            trt = cand;
            break;
        }
    }
    const int its = (trt * np + RPI - 1) / RPI;
    switch (its) {
    case 1: return go_dc<LPR, 1>(a, cb, trt, st);
    case 2: return go_dc<LPR, 2>(a, cb, trt, st);
    case 3: return go_dc<LPR, 3>(a, cb, trt, st);
    case 4: return go_dc<LPR, 4>(a, cb, trt, st);
    case 5: return go_dc<LPR, 5>(a, cb, trt, st);
    case 6: return go_dc<LPR, 6>(a, cb, trt, st);
    default: return go_dc<LPR, 8>(a, cb, trt, st);
    }
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
    default: return dc_lpr<256>(a, cb, st);
    }
}

}  // namespace q4k
