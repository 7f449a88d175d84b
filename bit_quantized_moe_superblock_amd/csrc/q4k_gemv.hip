// Indirect-dispatch Q4_K GEMV kernels for gfx950.
//
// What is computed (ferrum-kernels q4_k_moe_id_gemv_batched.rs, module doc and
// dispatch_gemv_q4k_moe_id_batched_on_encoder): for every (token, slot) pair
// p = token*top_k + slot, expert e = ids[p] and the activation row
// x = src1 + token*outer + slot*inner,
//     dst[p, r] = sum_c W_e[r, c] * x[c]   for r < n,
// with W_e stored as [n, k/256] Q4_K superblocks.  The fused variant reads a
// gate and an up stack with the same x and writes silu(gate)*up (moeflux
// expert_forward.rs, the gate/up/SwiGLU steps of encode_moe_gather_id_fuse).
//
// Layout on the device:
//   - a workgroup is 256 threads; LPR consecutive lanes cover one weight row,
//     lane u handling unit u = (superblock u/4, 32-byte chunk u%4), so one row
//     is read with coalesced 16-byte loads (header + two nibble halves);
//   - the activation row is staged once per workgroup into LDS (padded so a
//     row's lanes hit different banks) with per-32 sums for the min term;
//   - ITERS row groups are loaded before any arithmetic, to keep enough bytes
//     in flight per CU for HBM latency;
//   - partial sums are reduced across the row's lanes (xor butterfly, then LDS
//     across waves when a row spans more than one wave).
// Pair mode: grid (row tiles, pairs).  Bucketed mode: grid (row tiles, bucket
// slots); a workgroup keeps its tile of one expert's weights in registers and
// runs every pair of that expert's bucket against it, so the weights are read
// from HBM once per call (moeflux encode_moe_batched_permute_fuse).
// Both modes run the same unit arithmetic in the same order, so their outputs
// are identical bit for bit.
#include "common.hpp"
#include "launch.hpp"

namespace q4k {

enum { EPI_STORE = 0, EPI_SWIGLU = 1 };

struct GemvArgs {
    const uint8_t *w0;   // stacked experts (gate for the fused kernel)
    const uint8_t *w1;   // up stack (fused kernel only)
    const float *src1;
    const int32_t *ids;       // pair mode
    const int32_t *bucket;    // bucketed mode: workspace from the bucketing kernel
    float *dst;
    int n, k, top_k, num_experts, n_pairs;
    int64_t outer, inner;
};

// Stage the k activations of one pair into LDS (padded) and the 32-element
// sums used by the dmin*min term.  Ends with a barrier.
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int k, float *xs, float *sx) {
    const int tid = threadIdx.x;
    for (int i = tid; i < k; i += kThreads)
        xs[xpad(i)] = x[i];
    __syncthreads();
    for (int j = tid; j < (k >> 5); j += kThreads) {
        const float *p = xs + xpad(j << 5);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; i++)
            s += p[i];
        sx[j] = s;
    }
    __syncthreads();
}

template <int LPR, int NT, int ITERS>
struct Tile {
    uint4 hdr[NT][ITERS];
    uint4 qa[NT][ITERS];
    uint4 qb[NT][ITERS];
};

// Hide the tile registers from loop-invariant code motion: without this the
// compiler hoists every derived mask and scale out of the per-pair loop of the
// bucketed kernel and runs out of registers.
template <int LPR, int NT, int ITERS>
__device__ __forceinline__ void opaque(Tile<LPR, NT, ITERS> &t) {
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int it = 0; it < ITERS; it++) {
            asm volatile("" : "+v"(t.hdr[nt][it].x), "+v"(t.hdr[nt][it].y), "+v"(t.hdr[nt][it].z),
                         "+v"(t.hdr[nt][it].w));
            asm volatile("" : "+v"(t.qa[nt][it].x), "+v"(t.qa[nt][it].y), "+v"(t.qa[nt][it].z),
                         "+v"(t.qa[nt][it].w));
            asm volatile("" : "+v"(t.qb[nt][it].x), "+v"(t.qb[nt][it].y), "+v"(t.qb[nt][it].z),
                         "+v"(t.qb[nt][it].w));
        }
}

// Issue the loads of ITERS rows of expert e for this lane.
template <int LPR, int NT, int ITERS>
__device__ __forceinline__ void load_tile(const GemvArgs &a, int e, int row0, Tile<LPR, NT, ITERS> &t) {
    constexpr int RPI = kThreads / LPR > 0 ? kThreads / LPR : 1;
    const int tid = threadIdx.x;
    const int u = tid % LPR;
    const int rsub = tid / LPR;
    const int nb = a.k >> 8;
    const bool active = u < 4 * nb;
    const int64_t nb01 = (int64_t)nb * kBlockBytes;
    const int64_t off = (int64_t)e * a.n * nb01 + (int64_t)(u >> 2) * kBlockBytes;
    const int c = u & 3;
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const int r = row0 + it * RPI + rsub;
        const bool ok = active && r < a.n;
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const uint8_t *w = nt == 0 ? a.w0 : a.w1;
            if (ok) {
                const uint8_t *rp = w + off + (int64_t)r * nb01;
                t.hdr[nt][it] = *(const uint4 *)rp;
                t.qa[nt][it] = *(const uint4 *)(rp + 16 + 32 * c);
                t.qb[nt][it] = *(const uint4 *)(rp + 32 + 32 * c);
            } else {
                t.hdr[nt][it] = make_uint4(0, 0, 0, 0);
                t.qa[nt][it] = make_uint4(0, 0, 0, 0);
                t.qb[nt][it] = make_uint4(0, 0, 0, 0);
            }
        }
    }
}

// Compute the ITERS rows of the tile against the staged activations of pair p
// and write them.  red: LDS scratch for rows wider than one wave.
template <int LPR, int NT, int ITERS, int EPI>
__device__ __forceinline__ void compute_tile(const GemvArgs &a, int p, int row0,
                                             const Tile<LPR, NT, ITERS> &t, const float *xs,
                                             const float *sx, float *red) {
    constexpr int RPI = kThreads / LPR > 0 ? kThreads / LPR : 1;
    constexpr int WL = LPR < 64 ? LPR : 64;   // lanes of a row inside one wave
    constexpr int WPR = LPR / WL;              // waves per row
    const int tid = threadIdx.x;
    const int u = tid % LPR;
    const int rsub = tid / LPR;
    const int nb = a.k >> 8;
    const bool active = u < 4 * nb;
    const int c = u & 3;
    const float *xl = xs + 68 * u;   // xpad(64u)
    const float sxA = active ? sx[2 * u] : 0.0f;
    const float sxB = active ? sx[2 * u + 1] : 0.0f;
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        float part[NT];
        UnitAcc acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            acc[nt].a = acc[nt].b = 0.0f;
        if (active) {
            const float4 *xa = (const float4 *)xl;
            const float4 *xb = (const float4 *)(xl + 32);
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const float4 va = xa[q], vb = xb[q];
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    const uint4 &src = q < 4 ? t.qa[nt][it] : t.qb[nt][it];
                    const uint32_t v = (q & 3) == 0 ? src.x : (q & 3) == 1 ? src.y
                                     : (q & 3) == 2 ? src.z : src.w;
                    nib_fma(v, va, vb, acc[nt]);
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const UnitScale s = unit_scale(t.hdr[nt][it], c);
            part[nt] = active ? unit_value(s, acc[nt], sxA, sxB) : 0.0f;
            part[nt] = group_sum<WL>(part[nt]);
        }
        const int r = row0 + it * RPI + rsub;
        if constexpr (WPR > 1) {
            const int wave = tid >> 6;
            if ((tid & 63) == 0) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    red[nt * 4 + wave] = part[nt];
            }
            __syncthreads();
            if (u == 0) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    float s = red[nt * 4 + wave];
                    for (int w = 1; w < WPR; w++)
                        s += red[nt * 4 + wave + w];
                    part[nt] = s;
                }
            }
            __syncthreads();
        }
        if (u == 0 && r < a.n) {
            float v;
            if constexpr (EPI == EPI_SWIGLU)
                v = silu_mul(part[0], part[NT - 1]);
            else
                v = part[0];
            a.dst[(int64_t)p * a.n + r] = v;
        }
    }
}

template <int LPR, int NT, int ITERS, int EPI>
__global__ __launch_bounds__(kThreads) void k_pairs(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR > 0 ? kThreads / LPR : 1;
    float *xs = lds;
    float *sx = xs + xpad_len(a.k);
    float *red = sx + (a.k >> 5);
    const int p = blockIdx.y;
    const int row0 = blockIdx.x * (ITERS * RPI);
    const int e = a.ids[p];
    if ((unsigned)e >= (unsigned)a.num_experts) {
        for (int i = threadIdx.x; i < ITERS * RPI; i += kThreads)
            if (row0 + i < a.n)
                a.dst[(int64_t)p * a.n + row0 + i] = 0.0f;
        return;
    }
    Tile<LPR, NT, ITERS> t;
    load_tile<LPR, NT, ITERS>(a, e, row0, t);
    const int tok = p / a.top_k, slot = p % a.top_k;
    stage_x(a.src1 + tok * a.outer + slot * a.inner, a.k, xs, sx);
    compute_tile<LPR, NT, ITERS, EPI>(a, p, row0, t, xs, sx, red);
}

// Bucket workspace views (layout documented with moe_bucket in q4kmoe.h).
struct BucketView {
    const int32_t *counts, *offsets, *pairs, *active, *n_active;
    __device__ BucketView(const int32_t *ws, int E, int P) {
        counts = ws;
        offsets = counts + (E + 1);
        pairs = offsets + (E + 2);
        active = pairs + P;
        n_active = active + (E + 1);
    }
};

template <int LPR, int NT, int ITERS, int EPI>
__global__ __launch_bounds__(kThreads) void k_bucketed(GemvArgs a) {
    extern __shared__ float lds[];
    constexpr int RPI = kThreads / LPR > 0 ? kThreads / LPR : 1;
    float *xs = lds;
    float *sx = xs + xpad_len(a.k);
    float *red = sx + (a.k >> 5);
    const BucketView bv(a.bucket, a.num_experts, a.n_pairs);
    const int slot = blockIdx.y;
    if (slot >= *bv.n_active)
        return;
    const int bkt = bv.active[slot];
    const int beg = bv.offsets[bkt], end = bv.offsets[bkt + 1];
    const int row0 = blockIdx.x * (ITERS * RPI);
    if (bkt == a.num_experts) {   // ids outside [0, E): zero rows
        for (int q = beg; q < end; q++) {
            const int p = bv.pairs[q];
            for (int i = threadIdx.x; i < ITERS * RPI; i += kThreads)
                if (row0 + i < a.n)
                    a.dst[(int64_t)p * a.n + row0 + i] = 0.0f;
        }
        return;
    }
    Tile<LPR, NT, ITERS> t;
    load_tile<LPR, NT, ITERS>(a, bkt, row0, t);
    for (int q = beg; q < end; q++) {
        const int p = bv.pairs[q];
        const int tok = p / a.top_k, slot_ = p % a.top_k;
        stage_x(a.src1 + tok * a.outer + slot_ * a.inner, a.k, xs, sx);
        opaque<LPR, NT, ITERS>(t);
        compute_tile<LPR, NT, ITERS, EPI>(a, p, row0, t, xs, sx, red);
        __syncthreads();   // xs is rewritten for the next pair
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

static int pick_iters(int64_t n_pairs_or_slots, int n, int rpi) {
    static int forced = -1;
    if (forced < 0) {
        const char *s = getenv("Q4KMOE_ITERS");
        forced = s ? atoi(s) : 0;
    }
    if (forced == 1 || forced == 2 || forced == 4)
        return forced;
    // Aim for at least two workgroups per CU (256 CUs) before making tiles taller.
    for (int it = 4; it > 1; it >>= 1) {
        const int64_t tiles = (n + it * rpi - 1) / (it * rpi);
        if (tiles * n_pairs_or_slots >= 512)
            return it;
    }
    return 1;
}

template <int LPR, int NT, int EPI>
static hipError_t launch_lpr(const GemvArgs &a, bool bucketed, int grid_y, hipStream_t st) {
    constexpr int RPI = kThreads / LPR > 0 ? kThreads / LPR : 1;
    const int iters = pick_iters(grid_y, a.n, RPI);
    const size_t lds = (size_t)(xpad_len(a.k) + (a.k >> 5) + 8) * sizeof(float);
    auto go = [&](auto kern, int it) {
        if (lds > 65536)
            hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        dim3 grid((a.n + it * RPI - 1) / (it * RPI), grid_y);
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
        return hipGetLastError();
    };
    if (bucketed) {
        if (iters == 4) return go(k_bucketed<LPR, NT, 4, EPI>, 4);
        if (iters == 2) return go(k_bucketed<LPR, NT, 2, EPI>, 2);
        return go(k_bucketed<LPR, NT, 1, EPI>, 1);
    }
    if (iters == 4) return go(k_pairs<LPR, NT, 4, EPI>, 4);
    if (iters == 2) return go(k_pairs<LPR, NT, 2, EPI>, 2);
    return go(k_pairs<LPR, NT, 1, EPI>, 1);
}

template <int NT, int EPI>
static hipError_t launch_any(const GemvArgs &a, bool bucketed, int grid_y, hipStream_t st) {
    switch (lanes_per_row(a.k)) {
    case 4: return launch_lpr<4, NT, EPI>(a, bucketed, grid_y, st);
    case 8: return launch_lpr<8, NT, EPI>(a, bucketed, grid_y, st);
    case 16: return launch_lpr<16, NT, EPI>(a, bucketed, grid_y, st);
    case 32: return launch_lpr<32, NT, EPI>(a, bucketed, grid_y, st);
    case 64: return launch_lpr<64, NT, EPI>(a, bucketed, grid_y, st);
    case 128: return launch_lpr<128, NT, EPI>(a, bucketed, grid_y, st);
    case 256: return launch_lpr<256, NT, EPI>(a, bucketed, grid_y, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_q4k_gemv(const GemvLaunch &L, hipStream_t st) {
    GemvArgs a;
    a.w0 = (const uint8_t *)L.w0;
    a.w1 = (const uint8_t *)L.w1;
    a.src1 = L.src1;
    a.ids = L.ids;
    a.bucket = L.bucket_ws;
    a.dst = L.dst;
    a.n = (int)L.n;
    a.k = (int)L.k;
    a.top_k = (int)L.top_k;
    a.num_experts = (int)L.num_experts;
    a.n_pairs = (int)L.n_pairs;
    a.outer = L.outer;
    a.inner = L.inner;
    const bool bucketed = L.bucket_ws != nullptr;
    int grid_y = (int)L.n_pairs;
    if (bucketed) {
        const int64_t buckets = L.num_experts + 1;
        grid_y = (int)(L.n_pairs < buckets ? L.n_pairs : buckets);
    }
    if (L.fused_swiglu)
        return launch_any<2, EPI_SWIGLU>(a, bucketed, grid_y, st);
    return launch_any<1, EPI_STORE>(a, bucketed, grid_y, st);
}

}  // namespace q4k
