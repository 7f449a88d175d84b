// One whole single-token MoE layer in one launch (gfx950).
//
// What is computed (moeflux expert_forward.rs, gpu_expert_forward and
// encode_moe_combine_residual_n_tokens; ferrum-kernels
// q4_k_moe_id_gemv_batched.rs for the id-GEMV walk), for the token's top_k
// routed experts e_s = ids[s] and an optional shared expert:
//     act_s   = silu(W_gate[e_s] x) * (W_up[e_s] x)            (I values)
//     y_s     = W_down[e_s] act_s                                (H values)
//     out     = h_mid + sum_s w_s y_s + gamma y_shared           (slot order)
// with gamma = sigmoid(logit) or 1.  Ids outside [0, E) contribute zero rows.
//
// Why one launch: at one token the layer reads ~24 MB of expert weights in two
// dependent products.  As two kernels, each pays its own start-up (argument
// and id loads, then weight address generation) and drains a grid whose last
// workgroups decide its end.  Here a grid of one resident workgroup per CU
// runs both products with a device-wide barrier between them, and the down
// weights each workgroup will need are already in flight (into registers,
// then LDS) while the gate/up phase computes.
//
// Phase A (gate/up + SiLU): the P' = top_k (+1 shared) pairs x I rows form one
// list; lane-group L of the grid takes rows L, L + NL, L + 2 NL, ... (NL lane
// groups in all), so every CU gets the same share.  The token's activation
// row is staged once per workgroup in LDS, read once per row for gate and up.  Row i+2's loads are issued while row i computes.
// Phase B (down + combine): workgroup w owns output rows [w*RB, w*RB + RB) of
// all P' down matrices (slots pair-fastest), reads their weights from LDS and
// the P' activation rows from LDS (staged after the barrier), and applies the
// combine in slot order.  The per-unit arithmetic and the reductions are those
// of the pair and token kernels, so the result is bitwise the unfused one.
#include "gemv_core.hpp"
#include "q4kmoe.h"

namespace q4k {

struct LayerArgs {
    const uint8_t *wg, *wu, *wd;   // routed stacks: gate/up [E, I, H/256], down [E, H, I/256]
    const uint8_t *sg, *su, *sd;   // shared one-expert stacks (has_shared)
    const float *x;                // h_post [H]
    const float *h_mid;            // [H]
    const int32_t *ids;            // [K]
    const float *route_w;          // [K]
    const float *logit;            // [1] (shared_mode 1)
    float *out;                    // [H]
    float *act;                    // [P', I] scratch
    uint32_t *sync;                // barrier words (layout at grid_barrier)
    int H, I, E, K, P;             // P = K + has_shared
    int shared_mode, has_shared;
    int rb;                        // output rows per workgroup in phase B
    int vec;                       // x and h_mid 16-byte aligned
};

__device__ __forceinline__ void fetch_layer_args(const LayerArgs &a) {
    asm volatile("" ::"s"(a.wg), "s"(a.wu), "s"(a.wd), "s"(a.sg), "s"(a.su), "s"(a.sd), "s"(a.x),
                 "s"(a.h_mid));
    asm volatile("" ::"s"(a.ids), "s"(a.route_w), "s"(a.logit), "s"(a.out), "s"(a.act),
                 "s"(a.sync), "s"(a.H), "s"(a.I), "s"(a.E), "s"(a.K), "s"(a.P),
                 "s"(a.shared_mode), "s"(a.has_shared), "s"(a.rb), "s"(a.vec));
}

// Bound on barrier polls (each a device-scope load plus ~64 cycles of sleep,
// about a second in all): a missing workgroup is reported through the
// timeout word instead of hanging the device.
constexpr uint32_t kSpinLimit = 1u << 20;

// Device-wide barrier of the G workgroups of this launch.
//
// The data it orders (the act rows) is written with device-coherent stores
// and read back with device-coherent loads, so the barrier needs no cache
// write-back or invalidation (a release or acquire at device scope writes
// back or drops the whole L2 of the XCD, microseconds when every workgroup
// does it).  Arrival: every wave has waited for its stores, then thread 0
// sets the workgroup's flag (word w < kBarMaxGrid of the header) to g0 + 1.
// Workgroup 0 collects all G flags with one wave of loads per round and then
// raises the go word; every other workgroup polls only the go word, so a
// poll round costs G + 64 loads device-wide, not G * G.  Flags and the go
// word count the barriers passed, so they are all equal between launches and
// nothing needs resetting; g0 is read from the own flag at entry.
constexpr int kBarMaxGrid = 512;
constexpr int kBarGo = 544;
constexpr int kBarErr = 576;
static_assert(kBarGo >= kBarMaxGrid && kBarErr >= kBarGo + 32 &&
                  (kBarErr + 1) * 4 <= MOE_LAYER_SYNC_BYTES,
              "sync header layout");
static_assert(kBarErr == MOE_LAYER_SYNC_TIMEOUT_WORD, "timeout word as documented");

__device__ __forceinline__ uint32_t coherent_load(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void grid_barrier(uint32_t *sync, uint32_t g0, int G) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores are done
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid == 0)
        coherent_store(sync + blockIdx.x, g0 + 1u);
    uint32_t spins = 0;
    bool timed_out = false;
    if (blockIdx.x == 0 && tid < 64) {
        for (;;) {
            bool done = true;
            for (int j = tid; j < G; j += 64)
                done &= coherent_load(sync + j) != g0;
            if (__builtin_amdgcn_ballot_w64(!done) == 0)
                break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins == kSpinLimit) {
                timed_out = true;
                break;
            }
        }
        if (tid == 0)
            coherent_store(sync + kBarGo, g0 + 1u);
    } else if (blockIdx.x != 0 && tid == 0) {
        while (coherent_load(sync + kBarGo) == g0) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins == kSpinLimit) {
                timed_out = true;
                break;
            }
        }
    }
    if (timed_out)
        coherent_store(sync + kBarErr, 1u);
    __syncthreads();
}

// 16-byte phase-B weight chunks per lane (8 x 256 x 16 = 32 KB per
// workgroup: 8 output rows of 9 down matrices at inter 768); the kernel holds
// them in eight named registers.
constexpr int kLayerDma = 8;

template <int LPRA, int ITA, int LPRB, int ITB>
__global__ __launch_bounds__(kThreads) void k_layer_m1(LayerArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    fetch_layer_args(a);
    constexpr int RPIA = kThreads / LPRA;
    constexpr int RPIB = kThreads / LPRB;
    const int tid = threadIdx.x;
    const int G = gridDim.x;
    const int K = a.K, P = a.P;
    const int nbH = a.H >> 8, nbI = a.I >> 8;
    const int64_t rowA = (int64_t)nbH * kBlockBytes;   // gate/up row bytes
    const int64_t rowB = (int64_t)nbI * kBlockBytes;   // down row bytes
    const int64_t matA = (int64_t)a.I * rowA, matB = (int64_t)a.H * rowB;

    // LDS: [x row image | act images (P rows) | down weights | y | reduce]
    const int rlA = row_lds_floats(a.H), rlB = row_lds_floats(a.I);
    float *xs = lds;
    float *acts = xs + rlA;
    uint8_t *wlds = (uint8_t *)(acts + P * rlB);
    const int rdots = a.rb * P;                           // phase-B row dots
    const int chunks_per_row = (int)(rowB >> 4);          // 16-byte chunks
    const int n_chunks = rdots * chunks_per_row;
    float *ybuf = (float *)(wlds + (size_t)kLayerDma * kThreads * 16);
    float *red = ybuf + rdots;

    // Loads below are unconditional with clamped addresses: a load under a
    // lane-divergent branch makes the wait-count pass lose track of issue
    // order at the join and wait for everything in flight.
    const uint32_t g0 =
        __hip_atomic_load(&a.sync[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // The token's experts go to LDS once (-1 for ids outside [0, E)); lanes
    // then look up their slot there.  The id loads are issued first and the
    // activation loads right after, so waiting for the ids waits for nothing
    // else (waits on the vector memory counter drain in issue order).  A
    // per-lane select over the K ids in registers would be turned back into
    // an indexed array, which lives in scratch memory.
    __shared__ int ex_lds[kMaxTopK];
    const int e_own = a.ids[tid < K ? tid : K - 1];
    const int totalA = a.H >> 5;
    StageBatch xb;
    stage_issue([&](int) { return a.x; }, 0, totalA, a.H, a.vec, xb);
    if (tid < K)
        ex_lds[tid] = (unsigned)e_own < (unsigned)a.E ? e_own : -1;
    lds_barrier();
    auto expert_of = [&](int s) { return ex_lds[s]; };

    // Combine coefficients of phase B, fetched now (uniform loads).
    float rw[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; s++)
        rw[s] = s < K ? a.route_w[s] : 0.0f;
    const float gamma = a.shared_mode == 1 ? 1.0f / (1.0f + expf(-a.logit[0])) : 1.0f;

    // ---- phase A set-up: every row tile of this lane issued
    const int u = tid % LPRA, rsub = tid / LPRA, c = u & 3;
    const bool activeA = u < 4 * nbH;
    const int ul = activeA ? u : 0;
    const int NL = G * RPIA;                 // lane groups of the grid
    const int L = blockIdx.x * RPIA + rsub;  // this lane's group
    const int rowsA = P * a.I;

    // Row g of the list -> gate/up row addresses (clamped when past the end
    // or for an invalid expert; such rows are never stored).
    auto row_ptr = [&](int g, const uint8_t *&pg, const uint8_t *&pu, bool &ok) {
        const int gg = g < rowsA ? g : rowsA - 1;
        const int s = gg / a.I, r = gg - s * a.I;
        const int64_t off = (int64_t)r * rowA + (int64_t)(ul >> 2) * kBlockBytes;
        const int e = s < K ? expert_of(s) : 0;
        const bool ev = s >= K || e >= 0;
        const int64_t eo = s < K && ev ? (int64_t)e * matA : 0;
        pg = (s < K ? a.wg + eo : a.sg) + off;
        pu = (s < K ? a.wu + eo : a.su) + off;
        ok = ev && g < rowsA;
    };
    Tile<2, ITA> t;
    bool okA[ITA];
#pragma unroll
    for (int it = 0; it < ITA; it++) {
        const uint8_t *pg, *pu;
        bool ok;
        row_ptr(L + it * NL, pg, pu, ok);
        okA[it] = ok;
        t.hdr[0][it] = *(const uint4 *)pg;
        t.qa[0][it] = *(const uint4 *)(pg + 16 + 32 * c);
        t.qb[0][it] = *(const uint4 *)(pg + 32 + 32 * c);
        t.hdr[1][it] = *(const uint4 *)pu;
        t.qa[1][it] = *(const uint4 *)(pu + 16 + 32 * c);
        t.qb[1][it] = *(const uint4 *)(pu + 32 + 32 * c);
    }

    const int row0B = blockIdx.x * a.rb;
    // combine inputs of this thread's output row (phase B), prefetched
    const int rB = row0B + tid;
    const bool rowok = tid < a.rb && rB < a.H;
    const float hm = a.h_mid[rowok ? rB : 0];

    stage_commit(xb, totalA, a.H, xs);
    lds_barrier();

    // ---- phase A compute, first half of the rows
    auto compute_row = [&](int it) {
        float v0 = 0.0f, v1 = 0.0f;
        if (activeA)
            unit_pair_from_tile<ITA>(t, it, xs, ul, c, a.H, v0, v1);
        float part[2];
        part[0] = row_reduce<LPRA>(v0, red, 0);
        part[1] = row_reduce<LPRA>(v1, red, 1);
        const int g = L + it * NL;
        if (u == 0 && g < rowsA) {
            const float v = okA[it] ? epilogue<EPI_SWIGLU, 2>(part) : 0.0f;
            __hip_atomic_store(a.act + g, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    constexpr int HALF = (ITA + 1) / 2;
#pragma unroll
    for (int it = 0; it < HALF; it++)
        compute_row(it);

    // This workgroup's phase-B weights, issued once half of the gate/up rows
    // are consumed (their registers are free again) and written to LDS just
    // before the barrier: chunk q (16 bytes) of row dot d = q / chunks_per_row,
    // row dot d = (local row d / P, pair d % P).  (A direct global-to-LDS copy
    // would make the compiler wait for it before every later use of a gate/up
    // row.)
    uint4 w0, w1, w2, w3, w4, w5, w6, w7;
    auto wchunk = [&](int j) {
        const int q0 = j * kThreads + tid;
        const int q = q0 < n_chunks ? q0 : n_chunks - 1;
        const int d = q / chunks_per_row, ch = q - d * chunks_per_row;
        const int lr = d / P, s = d - lr * P;
        const int r0 = row0B + lr;
        const int r = r0 < a.H ? r0 : a.H - 1;
        const int e = s < K ? expert_of(s) : 0;
        const uint8_t *base = s < K ? a.wd + (e >= 0 ? (int64_t)e * matB : 0) : a.sd;
        return *(const uint4 *)(base + (int64_t)r * rowB + 16 * ch);
    };
    w0 = wchunk(0);
    w1 = wchunk(1);
    w2 = wchunk(2);
    w3 = wchunk(3);
    w4 = wchunk(4);
    w5 = wchunk(5);
    w6 = wchunk(6);
    w7 = wchunk(7);

    // ---- phase A compute, second half
#pragma unroll
    for (int it = HALF; it < ITA; it++)
        compute_row(it);

    auto wput = [&](int j, uint4 v) { *(uint4 *)(wlds + (size_t)(j * kThreads + tid) * 16) = v; };
    wput(0, w0);
    wput(1, w1);
    wput(2, w2);
    wput(3, w3);
    wput(4, w4);
    wput(5, w5);
    wput(6, w6);
    wput(7, w7);

    grid_barrier(a.sync, g0, G);

    // ---- phase B: activation rows into LDS (device-coherent loads: other
    // workgroups wrote them), then down from LDS weights
    {
        const int nsub = a.I >> 5, total = P * nsub;
        for (int f = tid; f < total; f += kThreads) {
            const int row = f / nsub, j = f - row * nsub;
            const uint64_t *src = (const uint64_t *)(a.act + (int64_t)row * a.I + 32 * j);
            float v[32];
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const uint64_t b = __hip_atomic_load(src + q, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                v[2 * q] = __builtin_bit_cast(float, (uint32_t)b);
                v[2 * q + 1] = __builtin_bit_cast(float, (uint32_t)(b >> 32));
            }
            StageBatch sb;
#pragma unroll
            for (int q = 0; q < 8; q++)
                sb.v[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            sb.f = f;
            stage_commit(sb, total, a.I, acts);
        }
    }
    lds_barrier();
    const int ub = tid % LPRB, rsb = tid / LPRB, cb = ub & 3;
    const bool activeB = ub < 4 * nbI;
    const int ulb = activeB ? ub : 0;
#pragma unroll
    for (int it = 0; it < ITB; it++) {
        const int d0 = it * RPIB + rsb;
        const int d = d0 < rdots ? d0 : rdots - 1;
        const int lr = d / P, s = d - lr * P;
        const uint8_t *wr = wlds + (size_t)d * rowB + (size_t)(ulb >> 2) * kBlockBytes;
        Tile<1, 1> tb;
        tb.hdr[0][0] = *(const uint4 *)wr;
        tb.qa[0][0] = *(const uint4 *)(wr + 16 + 32 * cb);
        tb.qb[0][0] = *(const uint4 *)(wr + 32 + 32 * cb);
        const bool ev = s >= K || expert_of(s) >= 0;
        const float *xrow = acts + s * rlB;
        float v = (activeB && ev) ? unit_from_tile<1, 1>(tb, 0, 0, xrow, ulb, cb, a.I) : 0.0f;
        v = row_reduce<LPRB>(v, red, 0);
        if (ub == 0 && d0 < rdots)
            ybuf[d0] = v;
    }
    lds_barrier();
    if (rowok) {
        float acc = hm;
#pragma unroll
        for (int s = 0; s < kMaxTopK; s++)
            if (s < K)
                acc = __builtin_fmaf(rw[s], ybuf[tid * P + s], acc);
        if (a.has_shared) {
            const float ysh = ybuf[tid * P + K];
            if (a.shared_mode == 1)
                acc = __builtin_fmaf(gamma, ysh, acc);
            else if (a.shared_mode == 2)
                acc += ysh;
        }
        a.out[rB] = acc;
    }
}

// ------------------------------------------------------------------ host ---

// LDS bytes of the layer kernel for a grid of G workgroups.
static size_t layer_lds_bytes(const LayerArgs &a) {
    const int P = a.P;
    const size_t rowB = (size_t)(a.I >> 8) * kBlockBytes;
    const size_t dma = (size_t)kLayerDma * kThreads * 16;
    return (size_t)(row_lds_floats(a.H) + P * row_lds_floats(a.I)) * 4 + dma +
           (size_t)a.rb * P * 4 + 8 * 4;
}

template <int LPRA, int ITA, int LPRB, int ITB>
static hipError_t go_layer(const LayerArgs &a, int G, hipStream_t st) {
    auto kern = k_layer_m1<LPRA, ITA, LPRB, ITB>;
    const size_t lds = set_lds((const void *)kern, layer_lds_bytes(a));
    int fit = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, (const void *)kern, kThreads, lds) !=
            hipSuccess ||
        fit < 1)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kern, dim3(G), dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

// Phase-B passes: row dots (rb * P) over RPIB = 256 / LPRB slots.
template <int LPRA, int ITA, int LPRB>
static hipError_t layer_itb(const LayerArgs &a, int G, hipStream_t st) {
    constexpr int RPIB = kThreads / LPRB;
    const int passes = (a.rb * a.P + RPIB - 1) / RPIB;
    if (passes <= 2) return go_layer<LPRA, ITA, LPRB, 2>(a, G, st);
    if (passes <= 4) return go_layer<LPRA, ITA, LPRB, 4>(a, G, st);
    if (passes <= 6) return go_layer<LPRA, ITA, LPRB, 6>(a, G, st);
    if (passes <= 8) return go_layer<LPRA, ITA, LPRB, 8>(a, G, st);
    return hipErrorInvalidValue;
}

template <int LPRA, int ITA>
static hipError_t layer_lprb(const LayerArgs &a, int G, hipStream_t st) {
    switch (lanes_per_row(a.I)) {
    case 4: return layer_itb<LPRA, ITA, 4>(a, G, st);
    case 8: return layer_itb<LPRA, ITA, 8>(a, G, st);
    case 16: return layer_itb<LPRA, ITA, 16>(a, G, st);
    case 32: return layer_itb<LPRA, ITA, 32>(a, G, st);
    default: return hipErrorInvalidValue;
    }
}

template <int LPRA>
static hipError_t layer_ita(const LayerArgs &a, int G, hipStream_t st) {
    constexpr int RPIA = kThreads / LPRA;
    const int64_t rows = (int64_t)a.P * a.I;
    const int64_t its = (rows + (int64_t)G * RPIA - 1) / ((int64_t)G * RPIA);
    if (its <= 2) return layer_lprb<LPRA, 2>(a, G, st);
    if (its <= 4) return layer_lprb<LPRA, 4>(a, G, st);
    if (its <= 6) return layer_lprb<LPRA, 6>(a, G, st);
    return hipErrorInvalidValue;
}

bool layer_m1_supported(int64_t hidden, int64_t inter, int64_t top_k, int has_shared) {
    // Shapes this kernel's tiling covers (others take the two-kernel path):
    // gate/up rows 16..64 lanes wide, down rows 4..32 lanes wide, and phase A
    // and B work within its unrolled iteration counts on the device's CUs.
    const int lA = lanes_per_row((int)hidden), lB = lanes_per_row((int)inter);
    if (lA < 16 || lA > 64 || lB > 32)
        return false;
    const int G = cu_count();
    if (G > kBarMaxGrid)
        return false;
    const int P = (int)top_k + (has_shared ? 1 : 0);
    const int64_t rowsA = (int64_t)P * inter;
    if ((rowsA + (int64_t)G * (kThreads / lA) - 1) / ((int64_t)G * (kThreads / lA)) > 6)
        return false;
    const int rb = (int)((hidden + G - 1) / G);
    if (rb > kThreads || (rb * P + kThreads / lB - 1) / (kThreads / lB) > 8)
        return false;
    if ((int64_t)rb * P * (inter / 256) * (kBlockBytes / 16) > (int64_t)kLayerDma * kThreads)
        return false;   // phase-B weights exceed the fixed LDS copy
    LayerArgs probe{};
    probe.H = (int)hidden;
    probe.I = (int)inter;
    probe.P = P;
    probe.rb = rb;
    return layer_lds_bytes(probe) <= 150 * 1024;
}

hipError_t launch_layer_m1(const LayerLaunch &L, hipStream_t st) {
    LayerArgs a{};
    a.wg = (const uint8_t *)L.w_gate;
    a.wu = (const uint8_t *)L.w_up;
    a.wd = (const uint8_t *)L.w_down;
    a.sg = (const uint8_t *)L.sh_gate;
    a.su = (const uint8_t *)L.sh_up;
    a.sd = (const uint8_t *)L.sh_down;
    a.x = L.h_post;
    a.h_mid = L.h_mid;
    a.ids = L.ids;
    a.route_w = L.route_w;
    a.logit = L.shared_logit;
    a.out = L.out;
    a.act = L.act;
    a.sync = L.sync;
    a.H = (int)L.hidden;
    a.I = (int)L.inter;
    a.E = (int)L.num_experts;
    a.K = (int)L.top_k;
    a.has_shared = L.sh_gate != nullptr;
    a.P = a.K + a.has_shared;
    a.shared_mode = a.has_shared ? L.shared_mode : 0;
    const int G = cu_count();
    a.rb = (a.H + G - 1) / G;
    a.vec = (reinterpret_cast<uintptr_t>(L.h_post) & 15u) == 0 &&
            (reinterpret_cast<uintptr_t>(L.act) & 15u) == 0 && (a.I & 3) == 0;
    switch (lanes_per_row(a.H)) {
    case 16: return layer_ita<16>(a, G, st);
    case 32: return layer_ita<32>(a, G, st);
    case 64: return layer_ita<64>(a, G, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace q4k
