// Q4TiledP dense matvec and encoder (cortiq-engine mv_lab.rs, kernel `cur`).
//
// Tensor layout, rows x cols, gpr = cols/32:
//   [0, rows*gpr*16)      group (r,g) at (r*gpr+g)*16: byte i holds element 2i
//                         (low nibble) and 2i+1 (high nibble), value nibble-8;
//   params_off = rows*gpr*16: per row fp16 base then fp16 step;
//   codes_off = params_off + rows*4: per row ceil(5*gpr/8) bytes of 5-bit
//                         codes, group g at bit 5g, least significant bit first;
//   scale(r,g) = 2^(base + code*step).
// y[r] = sum_g scale(r,g) * (sum_j nib*x[32g+j] - 8*sum_j x[32g+j]).
//
// LPR lanes (a power of two >= gpr, at most 64) cover a row, one 16-byte
// group per lane, or NG = ceil(gpr / 64) when a row has more than 64 groups:
// a row never spans two waves, so its sum is one wave-wide DPP reduction; x is
// staged in LDS with per-group sums.  The group scale uses the hardware exp2 (about one
// ulp), as the page's kernel does.
#include <type_traits>

#include "gemv_core.hpp"

namespace q4k {

// Group g's 32 activations start at 36*g floats in LDS (4 pad floats per
// group keeps the 16-byte reads of neighbouring lanes in different banks).
//
// A workgroup of TPB threads takes ITERS x RPI rows (RPI = TPB / LPR).  The
// loads are issued in this order and waited for one by one: x (a thread per
// 32-float group, float4), then every row's (base, step) word, code bytes and
// 16-byte groups (branch-free, clamped indices).  x is committed to LDS with its group sums (ascending, one thread
// per group) while the weights are in flight; LDS-only barriers leave them in
// flight.  Lane u of a row takes groups u, u + LPR, ... (NG of them).
// Up to three tensors of the same width read the same x in one launch (the
// merged q|k|v and gate|up dispatch); their outputs follow one another in y.
// Workgroup tiles never straddle two tensors.
struct TpSegs {
    const uint8_t *t[kTpMaxSegs];
    int rows[kTpMaxSegs];
    int tile_end[kTpMaxSegs];   // cumulative workgroup count
    int yoff[kTpMaxSegs];       // first output row
    int nseg;
};

// A weight group, read once per launch: marked non-temporal so that the
// streamed weights do not push the staged activations, which every workgroup
// on the CU reads, out of the CU's cache.
__device__ __forceinline__ uint4 load_stream(const uint8_t *p) {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v w = __builtin_nontemporal_load((const u4v *)p);
    return make_uint4(w.x, w.y, w.z, w.w);
}

template <int LPR, int NG, int ITERS, bool XV, int TPB>
__global__ __launch_bounds__(TPB) void k_q4tp_matvec(TpSegs sg, const float *__restrict__ x,
                                                     float *__restrict__ yall, int cols) {
    extern __shared__ float lds[];
    // this workgroup's tensor (uniform scalar compares)
    int seg = 0;
#pragma unroll
    for (int i = 1; i < kTpMaxSegs; i++)
        if (i < sg.nseg && (int)blockIdx.x >= sg.tile_end[i - 1])
            seg = i;
    const uint8_t *__restrict__ t = sg.t[seg];
    const int rows = sg.rows[seg];
    float *__restrict__ y = yall + sg.yoff[seg];
    const int tile = (int)blockIdx.x - (seg ? sg.tile_end[seg - 1] : 0);
    static_assert(LPR <= 64, "a row within one wave");
    constexpr int RPI = TPB / LPR;
    constexpr int XU = (LPR * NG + TPB - 1) / TPB;   // staging tasks per thread
    const int gpr = cols >> 5;
    float *xs = lds;            // padded activations
    float *sx = xs + 36 * gpr;  // group sums
    const int tid = threadIdx.x;

    // 1. activations, ahead of everything else
    float4 xv[XU][8];
#pragma unroll
    for (int k = 0; k < XU; k++) {
        const int f = tid + TPB * k;
        const int fc = f < gpr ? f : gpr - 1;
        const float *src = x + 32 * fc;
#pragma unroll
        for (int q = 0; q < 8; q++)
            xv[k][q] = XV ? *(const float4 *)(src + 4 * q)
                          : make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the rows' parameters, codes and groups
    const int64_t params_off = (int64_t)rows * gpr * 16;
    const int64_t codes_off = params_off + (int64_t)rows * 4;
    const int stride = (5 * gpr + 7) >> 3;
    const int u = tid % LPR;
    const int rsub = tid / LPR;
    const int row0 = tile * (ITERS * RPI);
    uint32_t pb[ITERS], c0[ITERS][NG], c1[ITERS][NG];
    uint4 qv[ITERS][NG];
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const int r0 = row0 + it * RPI + rsub;
        const int r = r0 < rows ? r0 : rows - 1;
        pb[it] = *(const uint32_t *)(t + params_off + (int64_t)r * 4);
        const uint8_t *cp = t + codes_off + (int64_t)r * stride;
#pragma unroll
        for (int j = 0; j < NG; j++) {
            const int g0 = u + j * LPR;
            const int g = g0 < gpr ? g0 : gpr - 1;
            const int cb = (5 * g) >> 3;
            c0[it][j] = cp[cb];
            c1[it][j] = cp[cb + 1 < stride ? cb + 1 : cb];
            qv[it][j] = load_stream(t + ((int64_t)r * gpr + g) * 16);
        }
    }

    // 3. activations into LDS, with their group sums
#pragma unroll
    for (int k = 0; k < XU; k++) {
        const int f = tid + TPB * k;
        if (f < gpr) {
            float4 *d = (float4 *)(xs + 36 * f);
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                d[q] = xv[k][q];
                sum += xv[k][q].x;
                sum += xv[k][q].y;
                sum += xv[k][q].z;
                sum += xv[k][q].w;
            }
            sx[f] = sum;
        }
    }
    lds_barrier();

    // 4. rows
#pragma unroll
    for (int it = 0; it < ITERS; it++) {
        const float base = lo_half(pb[it]), step = hi_half(pb[it]);
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NG; j++) {
            const int g0 = u + j * LPR;
            const bool gok = g0 < gpr;
            const int g = gok ? g0 : gpr - 1;
            const uint32_t code = ((c0[it][j] | (c1[it][j] << 8)) >> ((5 * g) & 7)) & 31u;
            const float scale = exp2f(__builtin_fmaf((float)code, step, base));
            const float4 *xp = (const float4 *)(xs + 36 * g);
            // element 8d+e of dword d: even e in the low nibbles, odd in the high
            float lo = 0.0f, hi = 0.0f;
            const uint32_t w4[4] = {qv[it][j].x, qv[it][j].y, qv[it][j].z, qv[it][j].w};
#pragma unroll
            for (int d = 0; d < 4; d++) {
                const uint32_t v = w4[d], sh = v >> 8;
                const float4 x0 = xp[2 * d], x1 = xp[2 * d + 1];
                const uint32_t r0 = v & 0x000F000Fu, r2 = sh & 0x000F000Fu;
                const uint32_t r1 = v & 0x00F000F0u, r3 = sh & 0x00F000F0u;
                lo = __builtin_fmaf(lo_half(r0), x0.x, lo);   // element 0
                hi = __builtin_fmaf(lo_half(r1), x0.y, hi);   // element 1
                lo = __builtin_fmaf(lo_half(r2), x0.z, lo);   // element 2
                hi = __builtin_fmaf(lo_half(r3), x0.w, hi);   // element 3
                lo = __builtin_fmaf(hi_half(r0), x1.x, lo);   // element 4
                hi = __builtin_fmaf(hi_half(r1), x1.y, hi);   // element 5
                lo = __builtin_fmaf(hi_half(r2), x1.z, lo);   // element 6
                hi = __builtin_fmaf(hi_half(r3), x1.w, hi);   // element 7
            }
            // lo = 2^-24 * sum over even elements, hi = 2^-20 * sum over odd ones
            const float dot = __builtin_fmaf(lo, 16777216.0f, hi * 1048576.0f);
            const float part = scale * __builtin_fmaf(-8.0f, sx[g], dot);
            acc += gok ? part : 0.0f;
        }
        acc = group_sum<LPR>(acc);
        const int r = row0 + it * RPI + rsub;
        if (u == 0 && r < rows)
            y[r] = acc;
    }
}

// Lanes per row: the smallest power of two, at least 4, that covers the
// row's groups, at most 64.
static int tp_lanes(int gpr) {
    int l = 4;
    while (l < gpr && l < 64)
        l <<= 1;
    return l;
}

// Row groups per workgroup (tpb / LPR rows each): the fewest whose weight
// bytes are at least twice the staged activations (4 cols bytes, read from the
// cache by every workgroup), at most kMaxIt (fewer as a lane holds more
// groups of a row), while the grid still gives every CU a workgroup.
static int tp_iters(int tpb, int lpr, int max_it, int64_t row_bytes, int cols, int64_t total_rows,
                    int64_t cus) {
    const int rpi = tpb / lpr;
    int it = 1;
    while (it < max_it && (int64_t)it * rpi * row_bytes < 8 * (int64_t)cols &&
           (total_rows + 2 * it * rpi - 1) / (2 * it * rpi) >= cus)
        it <<= 1;
    return it;
}

// Workgroup size: every workgroup stages the whole activation row in LDS, so
// bigger workgroups (more rows per staged row) cut the activation traffic
// from the cache, which at 256 threads was about 0.7x the weight bytes of a
// decode walk.  512 threads in general; 1024 when rows are at most 4096
// columns and the grid then holds at most one workgroup per CU (a small
// tensor, where more waves per CU hide more latency).
template <int LPR, int NG>
static hipError_t tp_launch(const void *const *ts, const int64_t *rows, int nseg, const float *x,
                            float *y, int cols, hipStream_t st) {
    const int gpr = cols >> 5;
    const int64_t row_bytes = (int64_t)gpr * 16 + 4 + ((5 * gpr + 7) >> 3);
    const int64_t cus = cu_count();
    int64_t total_rows = 0;
    for (int i = 0; i < nseg; i++)
        total_rows += rows[i];
    constexpr int kMaxIt = NG == 1 ? 8 : (NG == 2 ? 4 : (NG <= 4 ? 2 : 1));
    int tpb = 512;
    if (NG == 1 && gpr <= 128) {
        const int it1k = tp_iters(1024, LPR, kMaxIt, row_bytes, cols, total_rows, cus);
        const int64_t rows1k = (int64_t)it1k * (1024 / LPR);
        if ((total_rows + rows1k - 1) / rows1k <= cus)
            tpb = 1024;
    }
    const int RPI = tpb / LPR;
    const int it = tp_iters(tpb, LPR, kMaxIt, row_bytes, cols, total_rows, cus);
    const size_t lds = (size_t)(36 * gpr + gpr) * sizeof(float);
    auto go = [&](auto kern, int iters) {
        TpSegs sg{};
        int tiles = 0, yoff = 0;
        for (int i = 0; i < nseg; i++) {
            sg.t[i] = (const uint8_t *)ts[i];
            sg.rows[i] = (int)rows[i];
            tiles += (int)((rows[i] + iters * RPI - 1) / (iters * RPI));
            sg.tile_end[i] = tiles;
            sg.yoff[i] = yoff;
            yoff += (int)rows[i];
        }
        sg.nseg = nseg;
        set_lds((const void *)kern, lds);
        hipLaunchKernelGGL(kern, dim3(tiles), dim3(tpb), lds, st, sg, x, y, cols);
        return hipGetLastError();
    };
    // float4 activation loads need a 16-byte aligned x
    const bool xv = ((uintptr_t)x & 15) == 0;
    // tp_iters returns a power of two no larger than kMaxIt: only those
    // instantiations exist
    auto pick = [&](auto tpbc) -> hipError_t {
        constexpr int T = decltype(tpbc)::value;
        auto run = [&](auto itc) {
            constexpr int I = decltype(itc)::value;
            return xv ? go(k_q4tp_matvec<LPR, NG, I, true, T>, I)
                      : go(k_q4tp_matvec<LPR, NG, I, false, T>, I);
        };
        if constexpr (kMaxIt >= 8)
            if (it >= 8)
                return run(std::integral_constant<int, 8>{});
        if constexpr (kMaxIt >= 4)
            if (it >= 4)
                return run(std::integral_constant<int, 4>{});
        if constexpr (kMaxIt >= 2)
            if (it >= 2)
                return run(std::integral_constant<int, 2>{});
        return run(std::integral_constant<int, 1>{});
    };
    if constexpr (NG == 1)
        if (tpb == 1024)
            return pick(std::integral_constant<int, 1024>{});
    return pick(std::integral_constant<int, 512>{});
}

hipError_t launch_q4tp_matvec_multi(const void *const *ts, const int64_t *rows, int nseg,
                                    const float *x, float *y, int64_t cols, hipStream_t st) {
    const int gpr = (int)(cols >> 5);
    const int c = (int)cols;
    switch (tp_lanes(gpr)) {
    case 4: return tp_launch<4, 1>(ts, rows, nseg, x, y, c, st);
    case 8: return tp_launch<8, 1>(ts, rows, nseg, x, y, c, st);
    case 16: return tp_launch<16, 1>(ts, rows, nseg, x, y, c, st);
    case 32: return tp_launch<32, 1>(ts, rows, nseg, x, y, c, st);
    default:
        switch ((gpr + 63) / 64) {   // groups per lane
        case 1: return tp_launch<64, 1>(ts, rows, nseg, x, y, c, st);
        case 2: return tp_launch<64, 2>(ts, rows, nseg, x, y, c, st);
        case 3: return tp_launch<64, 3>(ts, rows, nseg, x, y, c, st);
        case 4: return tp_launch<64, 4>(ts, rows, nseg, x, y, c, st);
        case 5: return tp_launch<64, 5>(ts, rows, nseg, x, y, c, st);
        case 6: return tp_launch<64, 6>(ts, rows, nseg, x, y, c, st);
        case 7: return tp_launch<64, 7>(ts, rows, nseg, x, y, c, st);
        default: return tp_launch<64, 8>(ts, rows, nseg, x, y, c, st);
        }
    }
}

hipError_t launch_q4tp_matvec(const void *t, const float *x, float *y, int64_t rows,
                              int64_t cols, hipStream_t st) {
    return launch_q4tp_matvec_multi(&t, &rows, 1, x, y, cols, st);
}

// ------------------------------------------------------------- encoder ----
// One workgroup (256 threads) per row; thread g-loop over groups.  Steps:
// t_g = max|w|/7; lt_g = float(log2(double t_g)) for t_g > 0;
// base = fp16(min lt), step = fp16(max(0, max lt - base)/31);
// code_g = clamp(rne((lt_g - base)/step), 0, 31);
// scale = float(exp2(double(base + code*step)));
// nibble = clamp(rne(w/scale), -8, 7) + 8.  log2/exp2 in double, rest fp32.
__global__ __launch_bounds__(256) void k_q4tp_quant(const float *__restrict__ w,
                                                    uint8_t *__restrict__ t, int rows, int cols) {
    __shared__ float lmin_s[256], lmax_s[256];
    __shared__ int any_s[256];
    __shared__ uint32_t codes_w[(5 * 512 + 31) / 32 + 1];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int gpr = cols >> 5;
    const float *x = w + (int64_t)r * cols;
    const int64_t params_off = (int64_t)rows * gpr * 16;
    const int64_t codes_off = params_off + (int64_t)rows * 4;
    const int stride = (5 * gpr + 7) >> 3;
    float lmin = 0.0f, lmax = 0.0f;
    int any = 0;
    for (int g = tid; g < gpr; g += 256) {
        float amax = 0.0f;
        for (int e = 0; e < 32; e++) {
            const float a = fabsf(x[32 * g + e]);
            if (a > amax) amax = a;
        }
        const float tg = amax / 7.0f;
        if (tg > 0.0f) {
            const float lt = (float)log2((double)tg);
            if (!any || lt < lmin) lmin = lt;
            if (!any || lt > lmax) lmax = lt;
            any = 1;
        }
    }
    lmin_s[tid] = lmin;
    lmax_s[tid] = lmax;
    any_s[tid] = any;
    for (int i = tid; i < (int)(sizeof(codes_w) / 4); i += 256)
        codes_w[i] = 0u;
    __syncthreads();
    if (tid == 0) {
        int a = 0;
        float mn = 0.0f, mx = 0.0f;
        for (int i = 0; i < 256; i++) {
            if (!any_s[i]) continue;
            if (!a || lmin_s[i] < mn) mn = lmin_s[i];
            if (!a || lmax_s[i] > mx) mx = lmax_s[i];
            a = 1;
        }
        uint32_t base = 0, step = 0;
        if (a) {
            const _Float16 bh = (_Float16)mn;
            base = __builtin_bit_cast(uint16_t, bh);
            float span = mx - (float)bh;
            if (span < 0.0f) span = 0.0f;
            step = __builtin_bit_cast(uint16_t, (_Float16)(span / 31.0f));
        }
        *(uint32_t *)(t + params_off + (int64_t)r * 4) = base | (step << 16);
        lmin_s[0] = __builtin_bit_cast(float, base | (step << 16));
    }
    __syncthreads();
    const uint32_t pb = __builtin_bit_cast(uint32_t, lmin_s[0]);
    const float bf = lo_half(pb), sf = hi_half(pb);
    for (int g = tid; g < gpr; g += 256) {
        float amax = 0.0f;
        for (int e = 0; e < 32; e++) {
            const float a = fabsf(x[32 * g + e]);
            if (a > amax) amax = a;
        }
        const float tg = amax / 7.0f;
        const bool has = tg > 0.0f;
        int code = 0;
        if (has && sf > 0.0f) {
            const float lt = (float)log2((double)tg);
            code = (int)__builtin_rintf((lt - bf) / sf);
            code = code < 0 ? 0 : (code > 31 ? 31 : code);
        }
        const float L = (float)exp2((double)(bf + (float)code * sf));
        uint8_t grp[16];
        for (int i = 0; i < 16; i++) {
            int nib[2];
            for (int h = 0; h < 2; h++) {
                int q = 0;
                if (has && L > 0.0f) {
                    q = (int)__builtin_rintf(x[32 * g + 2 * i + h] / L);
                    q = q < -8 ? -8 : (q > 7 ? 7 : q);
                }
                nib[h] = q + 8;
            }
            grp[i] = (uint8_t)(nib[0] | (nib[1] << 4));
        }
        uint4 v;
        __builtin_memcpy(&v, grp, 16);
        *(uint4 *)(t + ((int64_t)r * gpr + g) * 16) = v;
        const int bit = 5 * g;
        atomicOr(&codes_w[bit >> 5], (uint32_t)code << (bit & 31));
        if ((bit & 31) > 27)
            atomicOr(&codes_w[(bit >> 5) + 1], (uint32_t)code >> (32 - (bit & 31)));
    }
    __syncthreads();
    uint8_t *cp = t + codes_off + (int64_t)r * stride;
    for (int i = tid; i < stride; i += 256)
        cp[i] = (uint8_t)(codes_w[i >> 2] >> (8 * (i & 3)));
}

hipError_t launch_q4tp_quant(const float *w, void *t, int64_t rows, int64_t cols,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_q4tp_quant, dim3((unsigned)rows), dim3(256), 0, st, w, (uint8_t *)t,
                       (int)rows, (int)cols);
    return hipGetLastError();
}

}  // namespace q4k
