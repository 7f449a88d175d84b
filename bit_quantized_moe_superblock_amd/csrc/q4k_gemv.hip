// Indirect-dispatch Q4_K GEMV kernels on the vector units (gfx950).
//
// What is computed (ferrum-kernels q4_k_moe_id_gemv_batched.rs, module doc and
// dispatch_gemv_q4k_moe_id_batched_on_encoder): for every (token, slot) pair
// p = token*top_k + slot, expert e = ids[p] and the activation row
// x = src1 + token*outer + slot*inner,
//     dst[p, r] = sum_c W_e[r, c] * x[c]   for r < n,
// with W_e stored as Q4_K superblocks (tile layout, common.hpp).  The fused
// variant reads a gate and an up stack with the same x and writes
// silu(gate)*up (the batched gate+up+SiLU dispatcher of the same page; moeflux
// expert_forward.rs SwiGLU).  An optional shared expert (moeflux: the
// shared_out term of the combine) runs in the same launch as extra pairs, one
// per token, on its own one-expert stack.
//
// Kernels:
//   k_rows    pair mode: a workgroup of four waves covers 16 rows (two row
//             groups, one per half-wave) of one pair; wave w takes the rows'
//             superblocks of class w (gemv_core.hpp), D of them in flight,
//             after staging their activations in its own LDS region.  Given
//             a bucket workspace, the y-th workgroup row takes the y-th pair
//             in bucket order, so the pairs of an expert run next to each
//             other and read its weights through the caches (vector-unit
//             bucketing; moeflux encode_moe_batched_permute_fuse).
//   k_down_combine  token mode for few tokens: a workgroup of W waves
//             computes one row group of the down projection for all top_k
//             (+ shared) pairs of one token -- a wave's halves take two pairs,
//             and the waves take the (pair pair, class) tasks in turn -- and
//             applies the weighted residual combine in slot order (moeflux
//             moe_combine_residual).
// Both form every row value in the one order of gemv_core.hpp, so pair,
// bucketed and token modes give identical bits.  Activation rows need only be
// 4-byte aligned: staging uses float4 loads when rows and strides are 16-byte
// aligned, 4-byte loads otherwise, with the same sums.
#include <stdint.h>

#include "gemv_core.hpp"

namespace q4k {

// ------------------------------------------------------------ pair mode ----

template <int NT, int EPI, bool VEC, int D>
__global__ __launch_bounds__(64 * kClasses) void k_rows(GemvArgs a) {
    extern __shared__ float lds[];   // per wave: its class's staged superblocks
    __shared__ float part[kClasses][NT][2 * kTileRows];
    fetch_args(a);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    int q = blockIdx.y;
    if (a.bucket != nullptr && q < a.n_pairs) {   // bucketed: pairs in bucket order
        const BucketView bv(a.bucket, a.num_experts, a.n_pairs);
        q = bv.pairs[q];
    }
    const int nb = a.k >> 8;
    const int T = class_steps(nb, wave);   // superblocks wave + 4t, t < T
    // The pair's id is requested first and its activations next (they do not
    // depend on the id), so waiting for the id leaves them in flight.
    const bool routed = q < a.n_pairs;
    int e_raw = a.ids[routed ? q : 0];
    __builtin_amdgcn_sched_barrier(0);
    const float *x;
    if (routed) {
        const int t = q / a.top_k, s = q - t * a.top_k;
        x = a.src1 + t * a.outer + s * a.inner;
    } else {
        x = a.src1_sh + (q - a.n_pairs) * a.outer_sh;
    }
    WaveStage xb;
    wave_stage_issue<VEC>(x, wave, T, 0, nb, xb);
    __builtin_amdgcn_sched_barrier(0);
    // first use of the id, after the activation loads: its wait leaves them
    // in flight (left to itself the compiler moves the id into a scalar
    // register, and so waits for it, right after its load)
    asm volatile("" : "+v"(e_raw));
    const PairRef pr = pair_ref_id(a, q, e_raw, x);
    // a workgroup covers RPW pairs of row groups: its half-waves' row groups,
    // and with EPI_ROWPAIR the two row groups after them as the second matrix
    constexpr int RPW = EPI == EPI_ROWPAIR ? 2 : 1;
    const int64_t row0 = (int64_t)blockIdx.x * (2 * kTileRows * RPW);
    if (!pr.valid) {   // id outside [0, E): zero rows
        if (tid < 2 * kTileRows * RPW && row0 + tid < a.n)
            pr.out[row0 + tid] = 0.0f;
        return;
    }
    const int n8 = (a.n + kTileRows - 1) / kTileRows;
    const int64_t Graw = 2 * RPW * (int64_t)blockIdx.x + (lane >> 5);
    const int64_t G = Graw < n8 ? Graw : n8 - 1;   // this lane's row group (clamped;
                                                   // stores are guarded)
    float *xw = lds + wave * class_steps(nb, 0) * kStepFloats;
    const uint8_t *mat[NT];
    mat[0] = pr.w0;
    if constexpr (EPI == EPI_ROWPAIR) {   // the same matrix, two row groups on (clamped)
        const int64_t G2 = Graw + 2 < n8 ? Graw + 2 : n8 - 1;
        mat[NT - 1] = pr.w0 + (G2 - G) * (int64_t)nb * kTileBytes;
    } else if constexpr (NT == 2) {
        mat[1] = pr.w1;
    }
    auto sb_of = [&](int t) { return wave + kClasses * (t < T ? t : T - 1); };   // clamped
    float acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
        acc[nt] = 0.0f;
    if (T > 0) {   // uniform per wave
        Step<NT> buf[D];
#pragma unroll
        for (int d = 0; d < D; d++)
            load_step<NT>(mat, G, sb_of(d), nb, buf[d]);
        wave_stage_commit(xb, T, 0, xw);
        for (int t0 = 8; t0 < T; t0 += 8) {   // more than 8 superblocks per class
            wave_stage_issue<VEC>(pr.x, wave, T, t0, nb, xb);
            wave_stage_commit(xb, T, t0, xw);
        }
        wave_lds_fence();
        const int c = (lane >> 3) & 3;
        // D superblocks per round; the refill loads the ones D ahead (clamped
        // to the last, so that no load sits under a branch)
        for (int t0 = 0; t0 < T; t0 += D) {
#pragma unroll
            for (int d = 0; d < D; d++) {
                if (t0 + d < T) {
                    const float *xs = xw + (t0 + d) * kStepFloats;
                    step_units<NT>(buf[d], xs + 68 * c, xs + 4 * 68 + 2 * c, acc);
                }
                if (t0 + D < T)
                    load_step<NT>(mat, G, sb_of(t0 + D + d), nb, buf[d]);
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const float v = chunk_sum(acc[nt]);
        if ((lane & 24) == 0)   // lanes 0..7 and 32..39
            part[wave][nt][((lane >> 5) << 3) | (lane & 7)] = v;
    }
    __syncthreads();
    const int64_t row = row0 + tid;
    if (tid < 2 * kTileRows && row < a.n) {
        float tot[NT];
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            tot[nt] = class_total(part[0][nt][tid], part[1][nt][tid], part[2][nt][tid],
                                  part[3][nt][tid]);
        if constexpr (EPI == EPI_ROWPAIR) {
            pr.out[row] = tot[0];
            if (row + 2 * kTileRows < a.n)
                pr.out[row + 2 * kTileRows] = tot[NT - 1];
        } else {
            pr.out[row] = epilogue<EPI, NT>(tot);
        }
    }
}

// ---------------------------------------------------- down + combine mode ----
// Workgroup = (RP row groups from G = RP*blockIdx.x, token t), W waves.  The
// token's np pairs (0..top_k-1 routed, top_k the shared expert) go in pair
// pairs (2pp, 2pp + 1; an odd last one repeats its pair and stores nothing for
// it); pair pairs times the row's C = min(4, nb) classes make the tasks, and
// wave w takes tasks w, w + W, ... (task = pp*C + c), each the class's
// superblocks of the two pairs in the RP row groups (RP register tiles per
// step: the staged activations serve 8*RP rows), and leaves the class sums of
// the 8*RP rows in LDS.  Then thread r forms each pair's row value
// (class_total) and applies
// out[t,r] = h_mid[t,r] + sum_s w[t,s]*y_s[r] + g_t*y_sh[r]
// with the same fma order as the combine kernel.

struct CombineArgs {
    const float *h_mid, *route_w, *shared_logit;
    float *out;
    float *expert_out;   // optional [n_pairs, n] copy of the routed rows
    int shared_mode;
};

template <bool VEC, int D, int W, int RP>
__global__ __launch_bounds__(64 * W) void k_down_combine(GemvArgs a, CombineArgs cb) {
    extern __shared__ float lds[];
    fetch_args(a);
    asm volatile("" ::"s"(cb.h_mid), "s"(cb.route_w), "s"(cb.shared_logit), "s"(cb.out),
                 "s"(cb.expert_out), "s"(cb.shared_mode));
    constexpr int NTHR = 64 * W;
    const int tok = blockIdx.y;
    const int K = a.top_k;
    const int np = K + (a.m_sh > 0 ? 1 : 0);   // pairs of this token
    const int rl = row_lds_floats(a.k);
    constexpr int R = RP * kTileRows;           // rows of the workgroup
    float *part = lds + np * rl;                // [np][kClasses][R]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int64_t G = (int64_t)RP * blockIdx.x;
    // the second row group's tiles (clamped to the last group: reloads it and
    // stores nothing for it)
    const int n8 = (a.n + kTileRows - 1) / kTileRows;
    const int64_t dG = RP > 1 && G + 1 < n8 ? 1 : 0;
    // 1. the token's ids, then the combine's routing weights, gate logit and
    //    h_mid, loaded here so that the combine at the end waits on no memory
    //    (one load per thread, unconditional with a clamped index)
    __shared__ float rw_lds[kMaxTopK];
    __shared__ int ex_lds[kMaxTopK];
    const int own = tok * K + (tid < K ? tid : K - 1);
    const int e_own = a.ids[own];   // first: waiting for it leaves the rest in flight
    const float rw_own = cb.route_w[own];
    const bool gated = a.m_sh > 0 && cb.shared_mode == 1;   // uniform
    const float logit = gated ? cb.shared_logit[tok] : 0.0f;
    const int64_t orow = G * kTileRows + (tid < R ? tid : 0);
    const bool rowok = tid < R && orow < a.n;
    const int64_t o = (int64_t)tok * a.n + (orow < a.n ? orow : a.n - 1);
    const float hm = cb.h_mid[o];
    // The first staging batch of the token's activation rows (routed rows,
    // then the shared row; both bases are uniform, lanes pick between the two
    // values), issued ahead of the weights with a clamped index and no branch.
    const float *xr = a.src1 + tok * a.outer;
    const float *xsh = a.m_sh > 0 ? a.src1_sh + tok * a.outer_sh : xr;
    const int64_t inner = a.inner;
    auto x_of = [&](int s) { return s < K ? xr + s * inner : xsh; };
    const int nsub = a.k >> 5;
    const int total = np * nsub;
    StageBatch xb;
    stage_issue<VEC>(x_of, 0, total, a.k, xb);
    __builtin_amdgcn_sched_barrier(0);
    // the token's experts into LDS (-1 for ids outside [0, E))
    if (tid < K) {
        ex_lds[tid] = (unsigned)e_own < (unsigned)a.num_experts ? e_own : -1;
        rw_lds[tid] = rw_own;
    }
    lds_barrier();
    // 2. this wave's tasks j = 0 .. ntask-1 (task wave + W j): pair pair pp,
    //    class c, T(c) superblocks each; S superblocks in all, walked D at a
    //    time with the loads D ahead (clamped to the last: no load under a
    //    branch).  The experts come from scalar loads of the ids.
    const int nb = a.k >> 8;
    const int C = nb < kClasses ? nb : kClasses;
    const int npp = (np + 1) >> 1;
    const int ntask_all = npp * C;
    const int ntask = ntask_all > wave ? (ntask_all - wave + W - 1) / W : 0;   // uniform
    auto task_pp = [&](int j) { return (wave + W * j) / C; };
    auto task_c = [&](int j) { return (wave + W * j) % C; };
    int S = 0;
    for (int j = 0; j < ntask; j++)
        S += class_steps(nb, task_c(j));
    const int jh = lane >> 5;   // this lane's pair of the pair pair
    auto pair_of = [&](int pp) {
        const int p = 2 * pp + jh;
        return p < np ? p : np - 1;
    };
    auto mat_of = [&](int pp) -> const uint8_t * {
        const int p = pair_of(pp);
        if (p >= K)
            return a.s0;
        const int e = ex_lds[p];
        return a.w0 + (int64_t)(e >= 0 ? e : 0) * a.mat;
    };
    int lj = 0, lt = 0, ls = 0;   // load cursor: task lj, its superblock lt
    auto load_next = [&](Step<RP> &b) {
        const uint8_t *m0 = mat_of(task_pp(lj));
        const uint8_t *m[RP];
#pragma unroll
        for (int r = 0; r < RP; r++)
            m[r] = m0 + r * dG * nb * kTileBytes;
        load_step<RP>(m, G, task_c(lj) + kClasses * lt, nb, b);
        if (ls + 1 < S) {   // advance, or stay on the last (clamped reload)
            ls++;
            if (++lt == class_steps(nb, task_c(lj))) {
                lt = 0;
                lj++;
            }
        }
    };
    Step<RP> buf[D];
    if (S > 0) {
#pragma unroll
        for (int d = 0; d < D; d++)
            load_next(buf[d]);
    }
    // 3. activation rows of the token's pairs into LDS (first batch, then any
    //    further ones)
    stage_commit(xb, total, a.k, lds);
    stage_rows<VEC, NTHR>(x_of, np, a.k, lds, NTHR);
    lds_barrier();
    // 4. the superblocks; at the end of a task its class sums go to part
    const int c = (lane >> 3) & 3;
    float acc[RP];
#pragma unroll
    for (int r = 0; r < RP; r++)
        acc[r] = 0.0f;
    int cj = 0, ct = 0;
    for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            if (s0 + d < S) {   // uniform
                const int pp = task_pp(cj), cl = task_c(cj);
                const int p = pair_of(pp);
                const int u = 4 * (cl + kClasses * ct) + c;
                const float *xrow = lds + p * rl;
                step_units<RP>(buf[d], xrow + 68 * u, xrow + xpad_len(a.k) + 2 * u, acc);
                if (++ct == class_steps(nb, cl)) {
#pragma unroll
                    for (int r = 0; r < RP; r++) {
                        const float v = chunk_sum(acc[r]);
                        if ((lane & 24) == 0 && 2 * pp + jh < np)
                            part[(p * kClasses + cl) * R + r * kTileRows + (lane & 7)] = v;
                        acc[r] = 0.0f;
                    }
                    ct = 0;
                    cj++;
                }
            }
            if (s0 + D < S)
                load_next(buf[d]);
        }
    }
    __syncthreads();
    // 5. the combine, one thread per row, slots in order
    if (rowok) {
        auto y_of = [&](int p) {
            const float *pp = part + p * kClasses * R + tid;
            return class_total(pp[0], C > 1 ? pp[R] : 0.0f, C > 2 ? pp[2 * R] : 0.0f,
                               C > 3 ? pp[3 * R] : 0.0f);
        };
        float accr = hm;
        for (int s = 0; s < K; s++) {
            const float yv = ex_lds[s] < 0 ? 0.0f : y_of(s);   // invalid id: no contribution
            accr = __builtin_fmaf(rw_lds[s], yv, accr);
            if (cb.expert_out)
                cb.expert_out[(int64_t)(tok * K + s) * a.n + orow] = yv;
        }
        if (a.m_sh > 0) {
            const float ysh = y_of(K);
            if (cb.shared_mode == 1) {
                const float g = 1.0f / (1.0f + expf(-logit));
                accr = __builtin_fmaf(g, ysh, accr);
            } else if (cb.shared_mode == 2) {
                accr += ysh;
            }
            if (a.dst_sh)
                a.dst_sh[o] = ysh;
        }
        cb.out[o] = accr;
    }
}

// ------------------------------------------------------------------ host ---

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
    a.mat = tiles_matrix_bytes(L.n, L.k);
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

// LDS of k_rows: four waves' staged superblocks.
static size_t rows_lds_bytes(int64_t k) {
    return (size_t)kClasses * class_steps((int)(k >> 8), 0) * kStepFloats * sizeof(float);
}

template <int NT, int EPI, int D>
static hipError_t go_rows(const GemvArgs &a, hipStream_t st) {
    const int n8 = (a.n + kTileRows - 1) / kTileRows;
    constexpr int RPW = EPI == EPI_ROWPAIR ? 2 : 1;   // row-group pairs per workgroup
    dim3 grid((n8 + 2 * RPW - 1) / (2 * RPW), a.n_pairs + a.m_sh);
    auto go = [&](auto kern) {
        const size_t lds = set_lds((const void *)kern, rows_lds_bytes(a.k));
        hipLaunchKernelGGL(kern, grid, dim3(64 * kClasses), lds, st, a);
        return hipGetLastError();
    };
    return a.vec ? go(k_rows<NT, EPI, true, D>) : go(k_rows<NT, EPI, false, D>);
}

// Superblocks in flight per wave: all of a class's when it has one or two,
// two otherwise.
template <int NT, int EPI>
static hipError_t launch_rows(const GemvArgs &a, hipStream_t st) {
    return class_steps(a.k >> 8, 0) <= 1 ? go_rows<NT, EPI, 1>(a, st)
                                         : go_rows<NT, EPI, 2>(a, st);
}

bool q4k_self_bucket_ok(const GemvLaunch &L) {
    return L.n_pairs <= kSelfBucketMaxPairs && L.num_experts + 1 <= kSelfBucketMaxBuckets;
}

hipError_t launch_q4k_gemv(const GemvLaunch &L, hipStream_t st) {
    GemvArgs a = make_args(L);
    if (L.self_bucket)   // chunks built in-kernel: the matrix-core kernel only
        return launch_q4k_gemv_mfma(a, L.fused_swiglu, st);
    const bool bucketed = L.bucket_ws != nullptr;
    if (bucketed && !L.vector_units)
        return launch_q4k_gemv_mfma(a, L.fused_swiglu, st);
    if (L.fused_swiglu)
        return launch_rows<2, EPI_SWIGLU>(a, st);
    // a single matrix: two pairs of row groups per workgroup, so that each
    // staged activation row serves 32 rows (config 4's down at m = 1: 62.9 ->
    // 60.5 us per layer)
    return launch_rows<2, EPI_ROWPAIR>(a, st);
}

// LDS of k_down_combine: np staged rows and the class sums of 8*rp rows.
static size_t dc_lds_bytes(int64_t k, int np, int rp) {
    return ((size_t)np * row_lds_floats((int)k) + (size_t)np * kClasses * kTileRows * rp) *
           sizeof(float);
}

// The token's rows must leave room for several workgroups per CU: with one
// (e.g. top_k 8 at k = 2048: 80 KB) the launch runs in latency-bound rounds
// of one workgroup per CU, slower than pair mode plus the combine.
bool q4k_down_combine_ok(int64_t k, int64_t top_k, bool shared) {
    return dc_lds_bytes(k, (int)top_k + (shared ? 1 : 0), 2) <= 48 * 1024;
}

template <int D, int W, int RP>
static hipError_t go_dc(const GemvArgs &a, const CombineArgs &cb, hipStream_t st) {
    const int np = a.top_k + (a.m_sh > 0 ? 1 : 0);
    const int n8 = (a.n + kTileRows - 1) / kTileRows;
    dim3 grid((n8 + RP - 1) / RP, (int)(a.n_pairs / a.top_k));
    auto go = [&](auto kern) {
        const size_t lds = set_lds((const void *)kern, dc_lds_bytes(a.k, np, RP));
        hipLaunchKernelGGL(kern, grid, dim3(64 * W), lds, st, a, cb);
        return hipGetLastError();
    };
    return a.vec ? go(k_down_combine<true, D, W, RP>) : go(k_down_combine<false, D, W, RP>);
}

// Steps in flight: a wave's whole share up to 4.
template <int W, int RP>
static hipError_t dc_depth(const GemvArgs &a, const CombineArgs &cb, int most, hipStream_t st) {
    switch (most < 4 ? most : 4) {
    case 4: return go_dc<4, W, RP>(a, cb, st);
    case 3: return go_dc<3, W, RP>(a, cb, st);
    case 2: return go_dc<2, W, RP>(a, cb, st);
    default: return go_dc<1, W, RP>(a, cb, st);
    }
}

// Waves: 8 when the grid is short of two waves per SIMD with 4 (a single
// token: one row group per CU) and there are more than 8 tasks, else 4.
hipError_t launch_q4k_down_combine(const GemvLaunch &L, const float *h_mid, const float *route_w,
                                   const float *shared_logit, float *out, float *expert_out,
                                   int shared_mode, hipStream_t st) {
    const GemvArgs a = make_args(L);
    CombineArgs cb{h_mid, route_w, shared_logit, out, expert_out, shared_mode};
    const int nb = a.k >> 8;
    const int C = nb < kClasses ? nb : kClasses;
    const int tasks = (a.top_k + (a.m_sh > 0 ? 1 : 0) + 1) / 2 * C;
    const int64_t tokens = a.n_pairs / a.top_k;
    const int RP = tokens >= 2 ? 2 : 1;
    const int64_t wgs = ((a.n + kTileRows - 1) / kTileRows + RP - 1) / RP * tokens;
    const int W = tasks > 8 && wgs * 4 < 8 * (int64_t)cu_count() ? 8 : 4;
    // superblocks of the busiest wave: its tasks times the longest class
    const int most = (tasks + W - 1) / W * class_steps(nb, 0);
    if (RP == 2)
        return W == 4 ? dc_depth<4, 2>(a, cb, most, st) : dc_depth<8, 2>(a, cb, most, st);
    return W == 4 ? dc_depth<4, 1>(a, cb, most, st) : dc_depth<8, 1>(a, cb, most, st);
}

}  // namespace q4k
