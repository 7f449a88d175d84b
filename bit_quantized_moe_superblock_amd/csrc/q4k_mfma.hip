// Bucketed Q4_K id-GEMV on the matrix cores (gfx950 v_mfma_f32_16x16x32_f16).
//
// What is computed is the bucketed mode of the id-GEMV (ferrum-kernels
// q4_k_moe_id_gemv_batched.rs, module doc; moeflux expert_forward.rs,
// encode_moe_gather_id_fuse): for every expert bucket, every row r of the
// expert's matrix against every pair p of the bucket,
//     dst[p, r] = sum_c W_e[r, c] x_p[c],
// with the gate/up variant storing silu(gate) * up.  When tokens share an
// expert this is a real (rows x pairs) contraction, so it runs on MFMA:
//
//   D[pair][row] = sum_k X[pair][k] * W[row][k]     one sub-block (k = 32)
//
// per v_mfma_f32_16x16x32_f16, with A = 16 pairs x 32 activations and
// B = 32 weights x 16 rows.  Operand lane layouts (checked on the device):
// lane l holds A[l % 16][8 (l / 16) + i], B[8 (l / 16) + i][l % 16] for
// i < 8, and D[4 (l / 16) + j][l % 16] for j < 4.
//
//   - B comes straight from the nibbles: with v the dword of bytes b0..b3,
//     (v & 0x000F000F) is the fp16 pair (q(b0), q(b2)) * 2^-24 and
//     ((v >> 8) & 0x000F000F) is (q(b1), q(b3)) * 2^-24 as subnormals
//     (0x00F000F0 gives the high nibbles, * 2^-20); the matrix core takes
//     fp16 subnormals exactly, so the weights enter with no conversion.  The
//     k order inside each group of 8 is therefore (0,2,1,3,4,6,5,7).
//   - A is the activation split exactly into two fp16 parts,
//     x = hi + lo, hi = fp16(x), lo = fp16(x - hi), staged once per
//     workgroup in LDS in the same k order; D = A_hi B + A_lo B.
//   - Each lane's D column is one weight row: the lane decodes that row's
//     header itself (d, dmin, six-bit scales and mins) and applies, per
//     sub-block j, y += d sc_j 2^24 D - dmin m_j sum_j(x) (2^20 for the high
//     nibbles), the factored form of the superblock formula.
//
// Rounding differs from the vector-unit kernels (the matrix core's own sum
// order, x carried as hi + lo), so this mode matches them within the fp32
// tolerance, not bit for bit.
#include "gemv_core.hpp"

namespace q4k {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kMP = kBucketChunk;   // pairs per workgroup (A rows 8..15 repeat 0..7)
constexpr int kMRows = 64;          // weight rows per workgroup (4 waves x 16)
constexpr int kSubB = 2 * 4 * kMP * 16;   // LDS bytes per staged sub-block: parts x groups x pairs x 16 B
static_assert(kMP == 8, "A-row mapping assumes 8 pairs per workgroup");

// LDS bytes of one slab of SB superblocks: the split activations, then the
// sub-block sums [sub-block][pair].
__host__ __device__ constexpr size_t mfma_lds_bytes(int sb) {
    return (size_t)sb * 8 * kSubB + (size_t)sb * 8 * kMP * 4;
}

struct MfmaTile {
    uint4 hdr;
    uint2 q[4];   // 8 bytes of each 32-byte chunk: bytes 8g..8g+7
};

// Stage pairs [0, cnt) of one slab (sub-blocks j0 .. j0 + 8 SB) into LDS.
// Task (pair, sub-block) loads 32 activations, sums them in ascending order
// from 0, splits each into fp16 hi + lo, and writes the four k groups.
template <int SB, typename XOf>
__device__ __forceinline__ void mfma_stage(XOf x_of, int cnt, int j0, int nsub_total, bool vec,
                                           uint8_t *lds) {
    float *sxs = (float *)(lds + (size_t)SB * 8 * kSubB);
    const int nsub = SB * 8;
    for (int task = threadIdx.x; task < cnt * nsub; task += kThreads) {
        const int p = task / nsub, jl = task - p * nsub;
        const int j = j0 + jl;
        float v[32];
        if (j < nsub_total) {   // uniform per task row; past the end: zeros
            const float *src = x_of(p) + 32 * j;
            if (vec) {
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    const float4 f = *(const float4 *)(src + 4 * q);
                    v[4 * q] = f.x;
                    v[4 * q + 1] = f.y;
                    v[4 * q + 2] = f.z;
                    v[4 * q + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 32; q++)
                    v[q] = src[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 32; q++)
                v[q] = 0.0f;
        }
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; q++)
            s += v[q];
        sxs[jl * kMP + p] = s;
        uint8_t *dst = lds + (size_t)jl * kSubB;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
            h8v hi, lo;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float x = v[8 * g + ord[i]];
                const _Float16 h = (_Float16)x;
                hi[i] = h;
                lo[i] = (_Float16)(x - (float)h);
            }
            *(h8v *)(dst + (size_t)(0 * 4 + g) * (kMP * 16) + p * 16) = hi;
            *(h8v *)(dst + (size_t)(1 * 4 + g) * (kMP * 16) + p * 16) = lo;
        }
    }
}

__device__ __forceinline__ void mfma_load(const uint8_t *row, int sb, int g, MfmaTile &t) {
    const uint8_t *b = row + (size_t)sb * kBlockBytes;
    t.hdr = *(const uint4 *)b;
#pragma unroll
    for (int c = 0; c < 4; c++)
        t.q[c] = *(const uint2 *)(b + 16 + 32 * c + 8 * g);
}

// Per-sub-block factors of the lane's row: k[j] = d sc_j 2^24 (2^20 for the
// odd, high-nibble sub-blocks), m[j] = dmin m_j.
__device__ __forceinline__ void mfma_scales(const uint4 &h, float (&k)[8], float (&m)[8]) {
    const float d = lo_half(h.x), dmin = hi_half(h.x);
    const uint32_t s[3] = {h.y, h.z, h.w};
#pragma unroll
    for (int j = 0; j < 8; j++) {
        uint32_t sc, mn;
        if (j < 4) {
            sc = (s[0] >> (8 * j)) & 63u;
            mn = (s[1] >> (8 * j)) & 63u;
        } else {
            const int i = j - 4;
            sc = ((s[2] >> (8 * i)) & 15u) | (((s[0] >> (8 * i)) >> 6) << 4 & 0x30u);
            mn = ((s[2] >> (8 * i + 4)) & 15u) | (((s[1] >> (8 * i)) >> 6) << 4 & 0x30u);
        }
        k[j] = d * (float)sc * ((j & 1) ? 1048576.0f : 16777216.0f);
        m[j] = dmin * (float)mn;
    }
}

template <int NT>
__device__ __forceinline__ void mfma_superblock(const MfmaTile (&t)[NT], const uint8_t *lds,
                                                const float *sxs, int jl0, float (&y)[NT][4]) {
    const int lane = threadIdx.x & 63;
    const int gp = lane >> 4;   // D rows (pairs) 4 gp .. 4 gp + 3
    float ks[NT][8], ms[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
        mfma_scales(t[nt].hdr, ks[nt], ms[nt]);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        uint4 blo[NT], bhi[NT];
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const uint32_t w0 = t[nt].q[c].x, w1 = t[nt].q[c].y;
            const uint32_t s0 = w0 >> 8, s1 = w1 >> 8;
            blo[nt] = make_uint4(w0 & 0x000F000Fu, s0 & 0x000F000Fu, w1 & 0x000F000Fu,
                                 s1 & 0x000F000Fu);
            bhi[nt] = make_uint4(w0 & 0x00F000F0u, s0 & 0x00F000F0u, w1 & 0x00F000F0u,
                                 s1 & 0x00F000F0u);
        }
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int jl = jl0 + 2 * c + half;   // sub-block within the slab
            const int j = 2 * c + half;          // sub-block within the superblock
            // A row l % 16 is pair (l % 16) % 8: rows 8..15 repeat 0..7 and
            // their D rows are not used
            const uint8_t *xs = lds + (size_t)jl * kSubB + (lane >> 4) * (kMP * 16) +
                                (lane & 7) * 16;
            const h8v ahi = *(const h8v *)xs;
            const h8v alo = *(const h8v *)(xs + 4 * kMP * 16);
            const float4 sx = *(const float4 *)(sxs + jl * kMP + 4 * (gp & 1));
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const h8v b = __builtin_bit_cast(h8v, half ? bhi[nt] : blo[nt]);
                f4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b, acc, 0, 0, 0);
                const float kk = ks[nt][j], mm = ms[nt][j];
                y[nt][0] = __builtin_fmaf(-mm, sx.x, __builtin_fmaf(kk, acc[0], y[nt][0]));
                y[nt][1] = __builtin_fmaf(-mm, sx.y, __builtin_fmaf(kk, acc[1], y[nt][1]));
                y[nt][2] = __builtin_fmaf(-mm, sx.z, __builtin_fmaf(kk, acc[2], y[nt][2]));
                y[nt][3] = __builtin_fmaf(-mm, sx.w, __builtin_fmaf(kk, acc[3], y[nt][3]));
            }
        }
    }
}

// Grid (row tiles of 64, chunk slots + shared chunks).  Slot y < n_slots is
// chunk y of the bucketing kernel's list (at most 8 pairs of one bucket);
// slot n_slots + s is the shared expert's tokens 8 s .. 8 s + 7.
template <int NT, int EPI, int SB>
__global__ __launch_bounds__(kThreads) void k_bucket_mfma(GemvArgs a, int n_slots) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_b[];
    fetch_args(a);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rl = lane & 15, g = lane >> 4;
    const int E = a.num_experts, P = a.n_pairs;
    const int y = blockIdx.y;
    const int32_t *ws = a.bucket;
    const BucketView bv(ws, E, P);
    const int32_t *pairs = bv.pairs;
    int cnt, first, bkt;
    bool shared;
    if (y < n_slots) {
        if (y >= *bv.n_chunks)
            return;
        bkt = bv.chunks[2 * y];
        const int packed = bv.chunks[2 * y + 1];
        first = packed & 0xFFFFFF;
        cnt = packed >> 24;
        shared = false;
    } else {
        const int s = y - n_slots;
        first = s * kMP;
        cnt = a.m_sh - first < kMP ? a.m_sh - first : kMP;
        bkt = 0;
        shared = true;
    }
    const int row0 = blockIdx.x * kMRows;
    auto pair_q = [&](int i) { return shared ? P + first + i : pairs[first + i]; };
    if (!shared && bkt == E) {   // ids outside [0, E): zero rows
        for (int i = 0; i < cnt; i++) {
            float *out = a.dst + (int64_t)pair_q(i) * a.n;
            for (int r = tid; r < kMRows; r += kThreads)
                if (row0 + r < a.n)
                    out[row0 + r] = 0.0f;
        }
        return;
    }
    const int nb = a.k >> 8;                                  // superblocks per row
    const int64_t rowb = (int64_t)nb * kBlockBytes;
    const int64_t mat = (int64_t)a.n * rowb;
    const int r0 = row0 + wave * 16 + rl;                     // this lane's weight row
    const int r = r0 < a.n ? r0 : a.n - 1;
    const uint8_t *wrow[NT];
    wrow[0] = (shared ? a.s0 : a.w0 + (int64_t)bkt * mat) + (int64_t)r * rowb;
    if (NT == 2)
        wrow[NT - 1] = (shared ? a.s1 : a.w1 + (int64_t)bkt * mat) + (int64_t)r * rowb;
    const float *sxs = (const float *)(lds_b + (size_t)SB * 8 * kSubB);
    const int nsub_total = a.k >> 5;

    {   // one chunk: at most kMP pairs
        const int g0 = 0, gc = cnt;
        auto x_of = [&](int i) { return pair_x_known(a, shared, pair_q(g0 + i)); };
        float yv[NT][4];
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                yv[nt][i] = 0.0f;
        for (int sb0 = 0; sb0 < nb; sb0 += SB) {
            __syncthreads();   // the previous slab's LDS is consumed
            // weights of the slab's first superblocks in flight while staging
            // (three superblocks in flight; indices are constants once the
            // loop is unrolled, so the tiles stay in registers)
            MfmaTile tt[3][NT];
            auto issue = [&](int i) {
                const int sb = sb0 + i < nb ? sb0 + i : nb - 1;   // clamped
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    mfma_load(wrow[nt], sb, g, tt[i % 3][nt]);
            };
#pragma unroll
            for (int i = 0; i < (SB < 3 ? SB : 3); i++)
                issue(i);
            mfma_stage<SB>(x_of, gc, sb0 * 8, nsub_total, a.vec, lds_b);
            lds_barrier();
#pragma unroll
            for (int i = 0; i < SB; i++) {
                if (sb0 + i < nb)   // uniform
                    mfma_superblock<NT>(tt[i % 3], lds_b, sxs, i * 8, yv);
                if (i + 3 < SB)
                    issue(i + 3);
            }
        }
        // D rows 4g .. 4g+3 are pairs g0 + 4g + j (rows 8..15 repeat 0..7);
        // this lane's column is row r0
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int i = 4 * g + j;
            if (g < 2 && i < gc && r0 < a.n) {
                const int q = pair_q(g0 + i);
                float *out = q < P ? a.dst + (int64_t)q * a.n : a.dst_sh + (int64_t)(q - P) * a.n;
                float part[NT];
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    part[nt] = yv[nt][j];
                out[r0] = epilogue<EPI, NT>(part);
            }
        }
    }
}

// ------------------------------------------------------------------ host ---

template <int NT, int EPI, int SB>
static hipError_t go_mfma(const GemvArgs &a, hipStream_t st) {
    auto kern = k_bucket_mfma<NT, EPI, SB>;
    const size_t lds = set_lds((const void *)kern, mfma_lds_bytes(SB));
    // chunks of the list: at most one partial chunk per non-empty bucket
    const int64_t nb_max = a.n_pairs < (int64_t)a.num_experts + 1 ? a.n_pairs : a.num_experts + 1;
    const int n_slots = (int)(nb_max + a.n_pairs / kMP);
    const int sh_groups = (a.m_sh + kMP - 1) / kMP;
    dim3 grid((a.n + kMRows - 1) / kMRows, n_slots + sh_groups);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, st, a, n_slots);
    return hipGetLastError();
}

template <int NT, int EPI>
static hipError_t mfma_sb(const GemvArgs &a, hipStream_t st) {
    switch (a.k >> 8 < 8 ? a.k >> 8 : 8) {
    case 1: return go_mfma<NT, EPI, 1>(a, st);
    case 2: return go_mfma<NT, EPI, 2>(a, st);
    case 3: return go_mfma<NT, EPI, 3>(a, st);
    case 4: return go_mfma<NT, EPI, 4>(a, st);
    case 5: return go_mfma<NT, EPI, 5>(a, st);
    case 6: return go_mfma<NT, EPI, 6>(a, st);
    case 7: return go_mfma<NT, EPI, 7>(a, st);
    default: return go_mfma<NT, EPI, 8>(a, st);
    }
}

hipError_t launch_q4k_gemv_mfma(const GemvArgs &a, bool fused_swiglu, hipStream_t st) {
    if (fused_swiglu)
        return mfma_sb<2, EPI_SWIGLU>(a, st);
    return mfma_sb<1, EPI_STORE>(a, st);
}

}  // namespace q4k
