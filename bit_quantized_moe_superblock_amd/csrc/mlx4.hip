// MLX affine 4-bit and 2-bit expert codecs on gfx950: dequantizers, encoders
// and the id-GEMV over expert blocks.
//
// Format (moeflux expert_forward.rs, "4-bit only" and the gather dispatch's
// strides: K/2 bytes of packed weights per row, K/64 bf16 scales and as many
// bf16 biases per row; the bit layout is MLX's): groups of 64 weights along a
// row, w = scale * q + bias, row byte j holding weight 2j in its low nibble
// and 2j+1 in its high nibble.  An expert's packed weights, scales and biases
// sit at byte offsets inside its block; expert e's block starts at
// e * expert_stride (the gather dispatch's nb02).
//
// id-GEMV: one workgroup per (row tile, pair), as the Q4_K pair mode; the
// fused variant reads the gate and up matrices of the block in the same lanes
// and stores silu(gate) * up.  A lane owns one group of one row: two 16-byte
// loads of its 32 packed bytes, its scale and bias.  The activation row is staged once per workgroup in LDS
// (64 floats per lane, padded by 4 so lanes' reads fall in different banks)
// with its 32-float sums.  The nibbles become fp16 subnormals by masking
// (low nibbles q 2^-24, high nibbles q 2^-20) and feed v_fma_mix_f32, so the
// group's sum q.x costs one instruction per weight; then
//     row value = sum over groups of scale * (q.x) + bias * (sum of x),
// reduced across the row's lanes with DPP.
//
// The 2-bit variant (moeflux's g_use_2bit layout; MLX's 2-bit format): the
// same groups, scales and biases with four 2-bit codes per byte, lowest
// first, so a group is 16 packed bytes and one 16-byte load; its fields are
// masked out at four shifts, all as fp16 subnormals q 2^-24.
#include <type_traits>

#include "gemv_core.hpp"

namespace q4k {

constexpr int kMlxGroup = 64;

struct Mlx4Args {
    const uint8_t *base;                       // expert 0's block
    int64_t stride;
    int64_t packed_off, scales_off, biases_off;        // first matrix (gate when fused)
    int64_t packed_off1, scales_off1, biases_off1;     // up matrix of the fused launch
    const float *src1;
    const int32_t *ids;
    float *dst;                                // [n_pairs, n]
    int64_t outer, inner;
    int n, k, top_k, num_experts;
    int vec;                                   // activation rows 16-byte aligned
};

__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// sum over the 64 weights of one group of q * x, from its 32 packed bytes and
// the group's 64 staged activations
__device__ __forceinline__ float group_qx(const uint4 qa, const uint4 qb, const float *xr) {
    const uint32_t w[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; d++) {
        // dword d = bytes 4d..4d+3 = weights 8d..8d+7
        const float4 xa = *(const float4 *)(xr + 8 * d);
        const float4 xb = *(const float4 *)(xr + 8 * d + 4);
        const uint32_t v = w[d], s = v >> 8;
        const uint32_t m0 = v & 0x000F000Fu;   // weights 8d, 8d+4
        const uint32_t m1 = s & 0x000F000Fu;   // weights 8d+2, 8d+6
        const uint32_t m2 = v & 0x00F000F0u;   // weights 8d+1, 8d+5 (x16)
        const uint32_t m3 = s & 0x00F000F0u;   // weights 8d+3, 8d+7 (x16)
        lo = __builtin_fmaf(lo_half(m0), xa.x, lo);
        lo = __builtin_fmaf(hi_half(m0), xb.x, lo);
        lo = __builtin_fmaf(lo_half(m1), xa.z, lo);
        lo = __builtin_fmaf(hi_half(m1), xb.z, lo);
        hi = __builtin_fmaf(lo_half(m2), xa.y, hi);
        hi = __builtin_fmaf(hi_half(m2), xb.y, hi);
        hi = __builtin_fmaf(lo_half(m3), xa.w, hi);
        hi = __builtin_fmaf(hi_half(m3), xb.w, hi);
    }
    return lo * 16777216.0f + hi * 1048576.0f;
}

// NT = 1: dst[p, r] = row r of the pair's matrix times x.  NT = 2: the gate
// and up matrices of the same expert block against the same x, the lane
// loading both groups, and dst[p, r] = silu(gate) * up.
// sum over the 64 weights of a 2-bit group of q * x, from its 16 packed bytes
__device__ __forceinline__ float group_qx2(const uint4 qa, const float *xr) {
    const uint32_t w[4] = {qa.x, qa.y, qa.z, qa.w};
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; d++) {
        // dword d = bytes 4d..4d+3 = weights 16d..16d+15
        const float4 xa = *(const float4 *)(xr + 16 * d);        // byte 0's weights
        const float4 xb = *(const float4 *)(xr + 16 * d + 4);    // byte 1's
        const float4 xc = *(const float4 *)(xr + 16 * d + 8);    // byte 2's
        const float4 xd = *(const float4 *)(xr + 16 * d + 12);   // byte 3's
        const float ea[4] = {xa.x, xa.y, xa.z, xa.w}, eb[4] = {xb.x, xb.y, xb.z, xb.w};
        const float ec[4] = {xc.x, xc.y, xc.z, xc.w}, ed[4] = {xd.x, xd.y, xd.z, xd.w};
        const uint32_t v = w[d];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t me = (v >> (2 * i)) & 0x00030003u;       // bytes 0 and 2, code i
            const uint32_t mo = (v >> (8 + 2 * i)) & 0x00030003u;   // bytes 1 and 3, code i
            acc = __builtin_fmaf(lo_half(me), ea[i], acc);
            acc = __builtin_fmaf(hi_half(me), ec[i], acc);
            acc = __builtin_fmaf(lo_half(mo), eb[i], acc);
            acc = __builtin_fmaf(hi_half(mo), ed[i], acc);
        }
    }
    return acc * 16777216.0f;
}

// Reduce a per-lane value over the LPR lanes of its row.  For rows wider
// than a wave the wave sums go through `red` (2 barriers); the first lane of
// the row receives the row total.
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

template <int LPR, int NT, int BITS, bool VEC>
__global__ __launch_bounds__(kThreads) void k_mlx4_rows(Mlx4Args a) {
    extern __shared__ float lds[];
    asm volatile("" ::"s"(a.base), "s"(a.stride), "s"(a.packed_off), "s"(a.scales_off),
                 "s"(a.biases_off), "s"(a.src1), "s"(a.ids), "s"(a.dst));
    asm volatile("" ::"s"(a.outer), "s"(a.inner), "s"(a.n), "s"(a.k), "s"(a.top_k),
                 "s"(a.num_experts), "s"(a.vec), "s"(a.packed_off1), "s"(a.scales_off1),
                 "s"(a.biases_off1));
    constexpr int RPI = kThreads / LPR;
    const int tid = threadIdx.x;
    const int q = blockIdx.y;   // pair
    const int t = q / a.top_k, s = q - t * a.top_k;
    const float *x = a.src1 + t * a.outer + s * a.inner;
    auto x_of = [&](int) { return x; };
    const int total = a.k >> 5;   // 32-float sub-blocks of the row
    float *red = lds + row_lds_floats(a.k);
    // 1. the first staging batch ahead of the weights (waiting for it leaves
    //    the weights in flight)
    StageBatch xb;
    stage_issue<VEC>(x_of, 0, total, a.k, xb);
    // 2. the lane's group: clamped addresses, no branch
    const int e = a.ids[q];
    const bool valid = (unsigned)e < (unsigned)a.num_experts;
    const uint8_t *blk = a.base + (valid ? (int64_t)e * a.stride : 0);
    const int gpr = a.k / kMlxGroup;
    const int u = tid % LPR, rsub = tid / LPR;
    const bool active = u < gpr;
    const int gl = active ? u : 0;
    const int r0 = blockIdx.x * RPI + rsub;
    const int r = r0 < a.n ? r0 : a.n - 1;
    constexpr int GB = kMlxGroup * BITS / 8;   // packed bytes of a group
    const int64_t prel = (int64_t)r * (a.k * BITS / 8) + GB * gl;
    const int64_t gi = ((int64_t)r * gpr + gl) * 2;
    uint4 qa[NT], qb[NT];
    uint32_t sh[NT], bh[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const uint8_t *prow = blk + (nt ? a.packed_off1 : a.packed_off) + prel;
        qa[nt] = *(const uint4 *)prow;
        qb[nt] = BITS == 4 ? *(const uint4 *)(prow + 16) : make_uint4(0, 0, 0, 0);
        sh[nt] = *(const uint16_t *)(blk + (nt ? a.scales_off1 : a.scales_off) + gi);
        bh[nt] = *(const uint16_t *)(blk + (nt ? a.biases_off1 : a.biases_off) + gi);
    }
    // 3. the staged row (and any further batches)
    stage_commit(xb, total, a.k, lds);
    stage_rows<VEC, kThreads>(x_of, 1, a.k, lds, kThreads);
    lds_barrier();
    // 4. the group's share, then the row sums
    const float *sx = lds + xpad_len(a.k);
    const float gsum = sx[2 * gl] + sx[2 * gl + 1];
    float part[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const float qx = BITS == 4 ? group_qx(qa[nt], qb[nt], lds + xpad(kMlxGroup * gl))
                                   : group_qx2(qa[nt], lds + xpad(kMlxGroup * gl));
        const float v = __builtin_fmaf(bf16_val(sh[nt]), qx, bf16_val(bh[nt]) * gsum);
        part[nt] = row_reduce<LPR>(active ? v : 0.0f, red, nt);
    }
    if (u == 0 && r0 < a.n)
        a.dst[(int64_t)q * a.n + r0] = valid ? (NT == 2 ? silu_mul(part[0], part[1]) : part[0])
                                             : 0.0f;
}

// One thread per group: w = scale * q + bias in float (scale * q is exact,
// the sum rounds once).
template <int BITS>
__global__ __launch_bounds__(256) void k_mlx4_dequant(const uint8_t *__restrict__ packed,
                                                      const uint16_t *__restrict__ scales,
                                                      const uint16_t *__restrict__ biases,
                                                      float *__restrict__ out, int64_t groups) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= groups)
        return;
    constexpr int GB = kMlxGroup * BITS / 8;   // packed bytes of a group
    constexpr int PW = 32 / BITS;              // codes per 32-bit word
    const uint4 qa = *(const uint4 *)(packed + GB * g);
    const uint4 qb = BITS == 4 ? *(const uint4 *)(packed + GB * g + 16) : make_uint4(0, 0, 0, 0);
    const float sc = bf16_val(scales[g]), bi = bf16_val(biases[g]);
    const uint32_t w[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float4 *o = (float4 *)(out + kMlxGroup * g);
#pragma unroll
    for (int d = 0; d < kMlxGroup / PW; d++) {
#pragma unroll
        for (int j4 = 0; j4 < PW; j4 += 4) {
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float p = sc * (float)((w[d] >> (BITS * (j4 + j))) & ((1u << BITS) - 1u));
                v[j] = p + bi;
            }
            o[(PW * d + j4) / 4] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// Encoder, one thread per group, every decision a single IEEE float
// operation in the same order as the CPU reference encoder: lo, hi = min and
// max; scale = bf16((hi - lo) / 15), bias = bf16(lo);
// q = clamp(rne((w - bias) / scale), 0, 15), 0 where the scale is 0.
template <int BITS>
__global__ __launch_bounds__(256) void k_mlx4_quant(const float *__restrict__ w,
                                                    uint8_t *__restrict__ packed,
                                                    uint16_t *__restrict__ scales,
                                                    uint16_t *__restrict__ biases,
                                                    int64_t groups) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= groups)
        return;
    const float *x = w + kMlxGroup * g;
    float lo = x[0], hi = x[0];
    for (int j = 1; j < kMlxGroup; j++) {
        const float v = x[j];
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
    }
    const float d = hi - lo;
    constexpr int QMAX = (1 << BITS) - 1;
    const uint16_t sh = f32_to_bf16(d / (float)QMAX);
    const uint16_t bh = f32_to_bf16(lo);
    const float sc = bf16_val(sh), bi = bf16_val(bh);
    scales[g] = sh;
    biases[g] = bh;
    constexpr int PW = 32 / BITS;   // codes per 32-bit word
    uint32_t word[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int dw = 0; dw < kMlxGroup / PW; dw++) {
        uint32_t acc = 0;
        for (int j = 0; j < PW; j++) {
            const float tq = (x[PW * dw + j] - bi) / sc;
            int qi = (int)__builtin_rintf(tq);
            qi = qi < 0 ? 0 : (qi > QMAX ? QMAX : qi);
            if (sc == 0.0f)
                qi = 0;
            acc |= (uint32_t)qi << (BITS * j);
        }
        word[dw] = acc;
    }
    uint4 *o = (uint4 *)(packed + kMlxGroup * BITS / 8 * g);
    o[0] = make_uint4(word[0], word[1], word[2], word[3]);
    if (BITS == 4)
        o[1] = make_uint4(word[4], word[5], word[6], word[7]);
}

// ------------------------------------------------------------------ host ---

template <int LPR, int NT, int BITS>
static hipError_t go_mlx4(const Mlx4Args &a, int64_t n_pairs, hipStream_t st) {
    constexpr int RPI = kThreads / LPR;
    dim3 grid((a.n + RPI - 1) / RPI, (unsigned)n_pairs);
    auto go = [&](auto kern) {
        const size_t lds =
            set_lds((const void *)kern, ((size_t)row_lds_floats(a.k) + 8) * sizeof(float));
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a);
        return hipGetLastError();
    };
    return a.vec ? go(k_mlx4_rows<LPR, NT, BITS, true>) : go(k_mlx4_rows<LPR, NT, BITS, false>);
}

static bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipError_t launch_mlx4_gemv(const Mlx4Launch &L, hipStream_t st) {
    Mlx4Args a{};
    a.base = (const uint8_t *)L.base;
    a.stride = L.expert_stride;
    a.packed_off = L.packed_off;
    a.scales_off = L.scales_off;
    a.biases_off = L.biases_off;
    a.packed_off1 = L.packed_off1;
    a.scales_off1 = L.scales_off1;
    a.biases_off1 = L.biases_off1;
    a.src1 = L.src1;
    a.ids = L.ids;
    a.dst = L.dst;
    a.outer = L.outer;
    a.inner = L.inner;
    a.n = (int)L.n;
    a.k = (int)L.k;
    a.top_k = (int)L.top_k;
    a.num_experts = (int)L.num_experts;
    a.vec = al16(L.src1) && L.outer % 4 == 0 && L.inner % 4 == 0;
    const int64_t P = L.m * L.top_k;
    int lpr = 4;
    while (lpr < a.k / kMlxGroup)
        lpr <<= 1;
    auto pick = [&](auto nt, auto bits) -> hipError_t {
        constexpr int N = decltype(nt)::value, B = decltype(bits)::value;
        switch (lpr) {
        case 4: return go_mlx4<4, N, B>(a, P, st);
        case 8: return go_mlx4<8, N, B>(a, P, st);
        case 16: return go_mlx4<16, N, B>(a, P, st);
        case 32: return go_mlx4<32, N, B>(a, P, st);
        case 64: return go_mlx4<64, N, B>(a, P, st);
        case 128: return go_mlx4<128, N, B>(a, P, st);
        case 256: return go_mlx4<256, N, B>(a, P, st);
        default: return hipErrorInvalidValue;
        }
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    if (L.bits == 2)
        return L.fused_swiglu ? pick(I2{}, I2{}) : pick(I1{}, I2{});
    return L.fused_swiglu ? pick(I2{}, I4{}) : pick(I1{}, I4{});
}

hipError_t launch_mlx4_dequant(const void *packed, const void *scales, const void *biases,
                               float *out, int64_t groups, int bits, hipStream_t st) {
    if (groups == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((groups + 255) / 256));
    if (bits == 2)
        hipLaunchKernelGGL(k_mlx4_dequant<2>, grid, dim3(256), 0, st, (const uint8_t *)packed,
                           (const uint16_t *)scales, (const uint16_t *)biases, out, groups);
    else
        hipLaunchKernelGGL(k_mlx4_dequant<4>, grid, dim3(256), 0, st, (const uint8_t *)packed,
                           (const uint16_t *)scales, (const uint16_t *)biases, out, groups);
    return hipGetLastError();
}

hipError_t launch_mlx4_quant(const float *w, void *packed, void *scales, void *biases,
                             int64_t groups, int bits, hipStream_t st) {
    if (groups == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((groups + 255) / 256));
    if (bits == 2)
        hipLaunchKernelGGL(k_mlx4_quant<2>, grid, dim3(256), 0, st, w, (uint8_t *)packed,
                           (uint16_t *)scales, (uint16_t *)biases, groups);
    else
        hipLaunchKernelGGL(k_mlx4_quant<4>, grid, dim3(256), 0, st, w, (uint8_t *)packed,
                           (uint16_t *)scales, (uint16_t *)biases, groups);
    return hipGetLastError();
}

}  // namespace q4k
