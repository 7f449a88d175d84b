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
//   - B comes straight from the nibbles: lane group g (lanes 16g .. 16g+15,
//     one weight row per lane) holds the row's 32-byte nibble chunk g (the
//     tile layout puts its two 16-byte halves where the lanes of a tile read
//     contiguous bytes), i.e. positions 0..31 of sub-block 2g (low nibbles)
//     and 2g + 1 (high nibbles).  With v a dword of bytes b0..b3,
//     (v & 0x000F000F) holds (q(b0), q(b2)) and ((v >> 8) & 0x000F000F)
//     (q(b1), q(b3)) as 16-bit integers (shifts by 4 and 12 give the high
//     nibbles).  One packed 16-bit multiply by the sub-block's six-bit scale
//     makes them q sc <= 945, which read as fp16 are the subnormals
//     q sc 2^-24; the matrix core takes fp16 subnormals exactly.  MFMA
//     t = 4u + 2hh + e of a superblock takes from every lane group the 8
//     positions 16u + 8e .. 16u + 8e + 7 of its sub-block 2g + hh, in the k
//     order (0,2,1,3,4,6,5,7); the activations are staged in the same order.
//   - A is the activation split into two fp16 parts, staged once per
//     workgroup in LDS in the same k order: A rows 0..7 are the 8 pairs' hi
//     parts, rows 8..15 their lo parts, so one MFMA per sub-block covers both
//     and the halves are added once at the end.  Before the split, each
//     pair's 256 activations of a superblock are scaled by an exact power of
//     two 2^e chosen from their largest magnitude (to [2^9, 2^10)), so
//     x 2^e = hi + lo with hi = fp16(x 2^e), lo = fp16(x 2^e - hi) keeps about
//     22 significant bits and the 32-element sums stay below 2^15, whatever
//     the scale of the inputs; the superblock's D is multiplied by 2^-e
//     (exact) before it is added in.
//   - Each lane's D column is one weight row: the lane decodes that row's
//     header itself (d, dmin, six-bit scales and mins), and the superblock's
//     eight MFMAs accumulate into one D with y += d 2^24 D; the min term
//     -dmin sum_j m_j sum_j(x), the other half of the factored superblock
//     formula, is one more MFMA per superblock over the split sub-block sums
//     and the mins.
//
// Rounding differs from the vector-unit kernels (the matrix core's own sum
// order, x carried as hi + lo), so this schedule matches them within the fp32
// tolerance, not bit for bit; repeated calls of this schedule give identical
// bits.
#include "gemv_core.hpp"

namespace q4k {

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kMP = kBucketChunk;   // pairs per workgroup (A rows: 8 hi parts, 8 lo parts)
constexpr int kMRows = 64;          // weight rows per row group (4 waves x 16)
// EPI_ROWPAIR here: a single-matrix launch whose two register tiles are two
// row groups of the same matrix (rows r and r + kMRows), so that an item
// covers 2 kMRows rows against one staged activation slab.
__host__ __device__ constexpr int item_rows(int epi) { return epi == EPI_ROWPAIR ? 2 * kMRows : kMRows; }
constexpr int kDepth = 2;   // superblocks of weights in flight per wave
constexpr int kSubB = 2 * 4 * kMP * 16;   // LDS bytes per staged sub-block: parts x groups x pairs x 16 B
static_assert(kMP == 8, "A-row mapping assumes 8 pairs per workgroup");

// LDS bytes of one slab of SB superblocks: the split activations, then per
// superblock the split sub-block sums (16 rows x 8 sub-blocks of fp16), then
// per superblock the 8 pairs' undo factors 2^-e (fp32).
__host__ __device__ constexpr size_t mfma_lds_bytes(int sb) {
    return (size_t)sb * 8 * kSubB + (size_t)sb * 256 + (size_t)sb * 32;
}
__host__ __device__ constexpr size_t mfma_lds_scale_off(int sb) {
    return (size_t)sb * 8 * kSubB + (size_t)sb * 256;
}

// One superblock of a lane's row: the header and nibble chunk g (its two
// 16-byte halves u[0], u[1]) for lane group g.
struct MfmaTile {
    uint4 hdr;
    uint4 u[2];
};

// A thread's share of one slab's activations: tasks (pair, sub-block)
// tid, tid + 256, ..., 32 activations each.  The loads are issued before the
// weights so that staging waits on them alone.
template <int SB>
struct XRegs {
    static constexpr int U = (kMP * SB * 8 + kThreads - 1) / kThreads;   // tasks per thread
    float4 v[U][8];
};

// VEC: the rows and strides are 16-byte aligned (float4 loads); otherwise
// four 4-byte loads per float4.
template <int SB, bool VEC>
__device__ __forceinline__ void mfma_x_issue(const float *const (&xrow)[XRegs<SB>::U], int cnt,
                                             int j0, int nsub_total, XRegs<SB> &xr) {
    constexpr int nsub = SB * 8;
#pragma unroll
    for (int u = 0; u < XRegs<SB>::U; u++) {
        const int task = threadIdx.x + u * kThreads;
        const int jl = task % nsub;
        const bool ok = task < cnt * nsub && j0 + jl < nsub_total;
        const float *src = xrow[u] + 32 * (ok ? j0 + jl : 0);   // clamped
        if constexpr (VEC) {
#pragma unroll
            for (int q = 0; q < 8; q++)
                xr.v[u][q] = *(const float4 *)(src + 4 * q);
        } else {
#pragma unroll
            for (int q = 0; q < 8; q++)
                xr.v[u][q] = make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2],
                                         src[4 * q + 3]);
        }
    }
}

// Task (pair p, sub-block jl) scales its 32 activations by the pair's
// power of two for the superblock, sums them in ascending order from 0,
// splits each scaled activation and the sum into fp16 hi + lo, and writes the
// four k groups of both parts and the two sums.  Sub-blocks past the end of
// the row are zeros.  The 8 tasks of one (pair, superblock) are 8
// consecutive lanes of a wave (task = 8 (p SB + s) + j), which find their
// largest magnitude with three DPP steps; the first of them stores the undo
// factor 2^-e.  Every lane takes part in those steps (tasks past the chunk
// contribute zeros and write nothing).
template <int SB>
__device__ __forceinline__ void mfma_x_commit(const XRegs<SB> &xr, int cnt, int j0,
                                              int nsub_total, uint8_t *lds) {
    constexpr int nsub = SB * 8;
    uint8_t *sxa = lds + (size_t)SB * 8 * kSubB;
    float *sfac = (float *)(lds + mfma_lds_scale_off(SB));
#pragma unroll
    for (int u = 0; u < XRegs<SB>::U; u++) {
        const int task = threadIdx.x + u * kThreads;
        const bool ok = task < cnt * nsub;
        const int p = task / nsub, jl = task - p * nsub;
        const bool live = ok && j0 + jl < nsub_total;
        float v[32];
#pragma unroll
        for (int q = 0; q < 8; q++) {
            v[4 * q] = live ? xr.v[u][q].x : 0.0f;
            v[4 * q + 1] = live ? xr.v[u][q].y : 0.0f;
            v[4 * q + 2] = live ? xr.v[u][q].z : 0.0f;
            v[4 * q + 3] = live ? xr.v[u][q].w : 0.0f;
        }
        float mx = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; q++)
            mx = fmaxf(mx, fabsf(v[q]));
        mx = fmaxf(mx, dpp_move<0xB1>(mx));    // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_move<0x4E>(mx));    // quad_perm [2,3,0,1]
        mx = fmaxf(mx, dpp_move<0x141>(mx));   // row_half_mirror: the other quad
        // mx in [2^(E-1), 2^E) -> scaled into [2^9, 2^10); the undo factor
        // 2^-e stays a normal fp32 number
        int e = mx > 0.0f ? 10 - __builtin_amdgcn_frexp_expf(mx) : 0;
        e = e < -126 ? -126 : (e > 126 ? 126 : e);
        if (!ok)
            continue;
#pragma unroll
        for (int q = 0; q < 32; q++)
            v[q] = __builtin_ldexpf(v[q], e);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; q++)
            s += v[q];
        if ((jl & 7) == 0)
            sfac[(jl >> 3) * kMP + p] = __builtin_ldexpf(1.0f, -e);
        const _Float16 sh = (_Float16)s;
        _Float16 *sx = (_Float16 *)(sxa + (size_t)(jl >> 3) * 256) + (jl & 7);
        sx[p * 8] = sh;
        sx[(8 + p) * 8] = (_Float16)(s - (float)sh);
        // sub-block j = 2g + hh of superblock jl / 8 is held by lane group g;
        // its positions 8 q8 .. 8 q8 + 7 (half u = q8 / 2, dword pair
        // e = q8 % 2) feed MFMA t = 4u + 2hh + e
        const int j = jl & 7, g = j >> 1, hh = j & 1;
        uint8_t *dst = lds + (size_t)(jl >> 3) * 8 * kSubB;
#pragma unroll
        for (int q8 = 0; q8 < 4; q8++) {
            const int ord[8] = {0, 2, 1, 3, 4, 6, 5, 7};
            h8v hi, lo;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float x = v[8 * q8 + ord[i]];
                const _Float16 h = (_Float16)x;
                hi[i] = h;
                lo[i] = (_Float16)(x - (float)h);
            }
            const int t = 4 * (q8 >> 1) + 2 * hh + (q8 & 1);
            uint8_t *blk = dst + (size_t)t * kSubB;
            *(h8v *)(blk + (size_t)(0 * 4 + g) * (kMP * 16) + p * 16) = hi;
            *(h8v *)(blk + (size_t)(1 * 4 + g) * (kMP * 16) + p * 16) = lo;
        }
    }
}

// Superblock sb of the lane's row: row r8 of row group G of the matrix at
// mat (tile layout, nb superblocks per row).  The 8 lanes of a tile and
// chunk read 128 contiguous bytes, the 32 lanes of a tile 512.
__device__ __forceinline__ void mfma_load(const uint8_t *mat, int64_t G, int r8, int sb, int nb,
                                          int g, MfmaTile &t) {
    const uint8_t *b = mat + tile_offset(G, sb, nb);
    t.hdr = *(const uint4 *)(b + 16 * r8);
    t.u[0] = *(const uint4 *)(b + kTileHalf0 + 16 * (8 * g + r8));
    t.u[1] = *(const uint4 *)(b + kTileHalf1 + 16 * (8 * g + r8));
}

// One superblock of the lane's row against the staged pairs.  A rows 0..7
// are the pairs' hi parts and rows 8..15 their lo parts; D rows 8..15 (lanes
// 32..63) accumulate the lo half, which the caller adds to the hi half once
// at the end.
//
// Lane group g holds nibble chunk g of its row: sub-blocks 2g (hh = 0, low
// nibbles) and 2g + 1 (hh = 1, high nibbles), positions 16u .. 16u + 15 in
// half u.  Each of its B values is the nibble times the sub-block's six-bit
// scale, an integer q sc <= 945 taken as the fp16 subnormal q sc 2^-24
// (exact), so the eight MFMAs of the superblock accumulate into one D and
//
//   y += d 2^24 D - dmin 2^24 D_min
//
// where D_min is one more MFMA: its A holds the split sub-block sums in
// k = 0..7 (lanes 0..15; zero elsewhere) and its B the six-bit mins as fp16
// subnormals m_j 2^-24.
//
// Both D's are in the superblock's scaled domain: each is multiplied by its
// pair's 2^-e (sfac, exact) before it is added in.
template <int NT>
__device__ __forceinline__ void mfma_superblock(const MfmaTile (&t)[NT], const uint8_t *lds,
                                                const uint8_t *sxa, const float *sfac, int s,
                                                float (&y)[NT][4]) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63;
    // undo factors of this lane's D rows 4 (lane / 16) + j: pairs 4 ((lane / 16) % 2) + j
    const float4 f = *(const float4 *)(sfac + s * kMP + 4 * ((lane >> 4) & 1));
    const float fj[4] = {f.x, f.y, f.z, f.w};
    const int aoff = (((lane >> 3) & 1) * 4 + (lane >> 4)) * (kMP * 16) + (lane & 7) * 16;
    const h8v a_sx = *(const h8v *)(sxa + (size_t)s * 256 + (lane & 15) * 16);
    const h8v zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const h8v amin = lane < 16 ? a_sx : zero8;
    // scale of sub-block 2g + hh: byte 2 (g % 2) + hh of the packed scales of
    // sub-blocks 0..3 (g < 2) or 4..7, into both 16-bit halves
    const int g = lane >> 4;
    const uint32_t gb = (uint32_t)(g & 1) * 2u;
    const uint32_t sel0 = 0x0c000c00u | gb | (gb << 16);
    const uint32_t sel1 = sel0 + 0x00010001u;
    const f4v zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f4v acc[NT];
    uint32_t scp[NT][2];   // [hh]
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const uint4 h = t[nt].hdr;
        const uint32_t sc03 = h.y & 0x3F3F3F3Fu;
        const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
        const uint32_t mn03 = h.z & 0x3F3F3F3Fu;
        const uint32_t mn47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
        const uint32_t scw = g < 2 ? sc03 : sc47;
        scp[nt][0] = __builtin_amdgcn_perm(0u, scw, sel0);
        scp[nt][1] = __builtin_amdgcn_perm(0u, scw, sel1);
        const uint4 bm = make_uint4(__builtin_amdgcn_perm(0u, mn03, 0x0c010c00u),
                                    __builtin_amdgcn_perm(0u, mn03, 0x0c030c02u),
                                    __builtin_amdgcn_perm(0u, mn47, 0x0c010c00u),
                                    __builtin_amdgcn_perm(0u, mn47, 0x0c030c02u));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(amin, __builtin_bit_cast(h8v, bm),
                                                         zero4, 0, 0, 0);
    }
    // the min term first; the accumulators then restart for D
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const float dm24 = -hi_half(t[nt].hdr.x) * 16777216.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
            y[nt][i] = __builtin_fmaf(dm24, acc[nt][i] * fj[i], y[nt][i]);
        acc[nt] = zero4;
    }
    auto scaled = [](uint32_t v, uint32_t sc) {
        return __builtin_bit_cast(uint32_t,
                                  __builtin_bit_cast(u16x2, v) * __builtin_bit_cast(u16x2, sc));
    };
#pragma unroll
    for (int u = 0; u < 2; u++) {
#pragma unroll
        for (int e = 0; e < 2; e++) {
            uint4 blo[NT], bhi[NT];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const uint32_t w0 = e ? t[nt].u[u].z : t[nt].u[u].x;
                const uint32_t w1 = e ? t[nt].u[u].w : t[nt].u[u].y;
                const uint32_t s0 = scp[nt][0], s1 = scp[nt][1];
                blo[nt] = make_uint4(scaled(w0 & 0x000F000Fu, s0), scaled((w0 >> 8) & 0x000F000Fu, s0),
                                     scaled(w1 & 0x000F000Fu, s0), scaled((w1 >> 8) & 0x000F000Fu, s0));
                bhi[nt] = make_uint4(scaled((w0 >> 4) & 0x000F000Fu, s1),
                                     scaled((w0 >> 12) & 0x000F000Fu, s1),
                                     scaled((w1 >> 4) & 0x000F000Fu, s1),
                                     scaled((w1 >> 12) & 0x000F000Fu, s1));
            }
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                const int tk = 4 * u + 2 * hh + e;   // MFMA within the superblock
                const h8v ax = *(const h8v *)(lds + (size_t)(s * 8 + tk) * kSubB + aoff);
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        ax, __builtin_bit_cast(h8v, hh ? bhi[nt] : blo[nt]), acc[nt], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const float d24 = lo_half(t[nt].hdr.x) * 16777216.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
            y[nt][i] = __builtin_fmaf(d24, acc[nt][i] * fj[i], y[nt][i]);
    }
}

// ------------------------------------------------------------ one item ---
// Item = (chunk of at most kMP pairs of one bucket, row tile of item_rows(EPI)
// rows: 64, or 128 as a row pair).  pairs[i]
// is the i-th pair of a routed chunk (ascending pair order); a shared chunk
// is the shared expert's tokens first .. first + cnt - 1.  The first slab
// starts with a barrier, so consecutive items of one workgroup may reuse the
// LDS.
template <int NT, int EPI, int SB, bool VEC>
__device__ __forceinline__ void mfma_item(const GemvArgs &a, bool shared, int bkt, int cnt,
                                          const int32_t *pairs, int first, int row0,
                                          uint8_t *lds_b) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rl = lane & 15, g = lane >> 4;
    const int E = a.num_experts, P = a.n_pairs;
    auto pair_q = [&](int i) { return shared ? P + first + i : pairs[i]; };
    if (!shared && bkt == E) {   // ids outside [0, E): zero rows
        for (int i = 0; i < cnt; i++) {
            float *out = a.dst + (int64_t)pair_q(i) * a.n;
            for (int r = tid; r < item_rows(EPI); r += kThreads)
                if (row0 + r < a.n)
                    out[row0 + r] = 0.0f;
        }
        return;
    }
    const int nb = a.k >> 8;                                  // superblocks per row
    const int r0 = row0 + wave * 16 + rl;                     // this lane's weight row
    // its row group (clamped to the last one; rows past n up to a multiple of
    // 8 are zero blocks in the tile layout) and row within the group
    const int64_t n8 = (a.n + kTileRows - 1) / kTileRows;
    const int r8 = r0 & (kTileRows - 1);
    auto group = [&](int rr) {
        const int64_t G = rr / kTileRows;
        return G < n8 ? G : n8 - 1;
    };
    const uint8_t *wmat[NT];
    int64_t wg[NT];
    wmat[0] = shared ? a.s0 : a.w0 + (int64_t)bkt * a.mat;
    wg[0] = group(r0);
    if constexpr (EPI == EPI_ROWPAIR) {   // the second row group of the same matrix
        wmat[NT - 1] = wmat[0];
        wg[NT - 1] = group(r0 + kMRows);
    } else if (NT == 2) {
        wmat[NT - 1] = shared ? a.s1 : a.w1 + (int64_t)bkt * a.mat;
        wg[NT - 1] = wg[0];
    }
    const uint8_t *sxa = lds_b + (size_t)SB * 8 * kSubB;
    const float *sfac = (const float *)(lds_b + mfma_lds_scale_off(SB));
    const int nsub_total = a.k >> 5;
    const int gc = cnt;
    auto x_of = [&](int i) { return pair_x_known(a, shared, pair_q(i)); };
    // activation rows of this thread's staging tasks (pair = task / (8 SB),
    // clamped to the chunk), looked up once
    const float *xrow[XRegs<SB>::U];
#pragma unroll
    for (int u = 0; u < XRegs<SB>::U; u++) {
        const int p = (tid + u * kThreads) / (SB * 8);
        xrow[u] = x_of(p < gc ? p : gc - 1);
    }
    float yv[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            yv[nt][i] = 0.0f;
    for (int sb0 = 0; sb0 < nb; sb0 += SB) {
        lds_barrier();   // the previous slab's (or item's) LDS is consumed
        // weights of the slab's first superblocks in flight while staging
        // (kDepth superblocks in flight; indices are constants once the
        // loop is unrolled, so the tiles stay in registers)
        MfmaTile tt[kDepth][NT];
        auto issue = [&](int i) {
            const int sb = sb0 + i < nb ? sb0 + i : nb - 1;   // clamped
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
                mfma_load(wmat[nt], wg[nt], r8, sb, nb, g, tt[i % kDepth][nt]);
        };
        XRegs<SB> xr;
        mfma_x_issue<SB, VEC>(xrow, gc, sb0 * 8, nsub_total, xr);
        // the activations ahead of the weights: staging waits on them alone
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < (SB < kDepth ? SB : kDepth); i++)
            issue(i);
        mfma_x_commit<SB>(xr, gc, sb0 * 8, nsub_total, lds_b);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < SB; i++) {
            if (sb0 + i < nb)   // uniform
                mfma_superblock<NT>(tt[i % kDepth], lds_b, sxa, sfac, i, yv);
            if (i + kDepth < SB)
                issue(i + kDepth);
        }
    }
    // hi half (D rows 0..7, lanes 0..31) plus lo half (rows 8..15, lanes
    // 32..63)
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            yv[nt][j] += __shfl_xor(yv[nt][j], 32);
    // D rows 4g .. 4g+3 (g < 2) are pairs 4g + j of the chunk; this lane's
    // column is row r0
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int i = 4 * g + j;
        if (g < 2 && i < gc && r0 < a.n) {
            const int q = pair_q(i);
            float *out = q < P ? a.dst + (int64_t)q * a.n : a.dst_sh + (int64_t)(q - P) * a.n;
            if constexpr (EPI == EPI_ROWPAIR) {
                out[r0] = yv[0][j];
                if (r0 + kMRows < a.n)
                    out[r0 + kMRows] = yv[NT - 1][j];
            } else {
                float part[NT];
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
                    part[nt] = yv[nt][j];
                out[r0] = epilogue<EPI, NT>(part);
            }
        }
    }
}

// ------------------------------------------------------- self-bucketing ---
// The bucketing of the ids (moeflux expert_forward.rs, encode_moe_gather_id_fuse
// step 1) done inside the launch, so that a layer needs no separate bucketing
// launch.  Buckets are the experts plus one (bucket E takes ids outside
// [0, E)); a bucket of c pairs has ceil(c / kMP) chunks; chunks are numbered
// in bucket order, and chunk i of a bucket holds its pairs of ranks
// kMP i .. kMP i + kMP - 1 in ascending pair order.  That is the chunk list
// the bucketing kernel writes, in the same order, so an item computes exactly
// what it computes from that list.
//
// One wave of each workgroup does it, with no barrier until it is done: its
// LDS operations execute in program order, so the counters it zeroes, adds
// to and reads need no synchronisation among themselves.
constexpr int kSelfMaxPairs = 1024;
constexpr int kSelfMaxBuckets = 1024;
constexpr int kSelfIdRegs = kSelfMaxPairs / 64;   // ids per lane of the bucketing wave
static_assert(kSelfMaxPairs == kSelfBucketMaxPairs && kSelfMaxBuckets == kSelfBucketMaxBuckets,
              "self-bucketing limits");
static_assert(kSelfMaxBuckets * 4 <= mfma_lds_bytes(1), "self-bucketing scratch");

struct SelfBuckets {
    int chunk_start[kSelfMaxBuckets + 1];   // first chunk of each bucket; [B] = routed chunks
    int pair_bucket[kSelfMaxPairs];         // bucket of each pair
    int pairs[2][kMP];                      // the current item's pairs (two buffers)
    int info[2][2];                         // the current item's bucket and pair count
};

// Inclusive sum over the lanes of a wave, in lane order: a shift-and-add
// ladder inside each row of 16 lanes, then the totals of the rows before.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = threadIdx.x & 63;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Bucketing wave: the buckets of all pairs (kept in LDS), their counts (in
// the scratch `counts`, B words), and the chunk starts.  Returns the number
// of routed chunks (every lane).
__device__ __forceinline__ int self_bucket(const GemvArgs &a, SelfBuckets &sb, int *counts) {
    const int lane = threadIdx.x & 63;
    const int E = a.num_experts, P = a.n_pairs, B = E + 1;
    // all the ids first, unconditional with a clamped index (no branch for
    // the wait to join at), so their loads are in flight together
    int raw[kSelfIdRegs];
#pragma unroll
    for (int j = 0; j < kSelfIdRegs; j++) {
        const int q = 64 * j + lane;
        raw[j] = a.ids[q < P ? q : P - 1];
    }
    for (int b = lane; b < B; b += 64)
        counts[b] = 0;
#pragma unroll
    for (int j = 0; j < kSelfIdRegs; j++) {
        if (64 * j >= P)   // uniform
            break;
        const int q = 64 * j + lane;
        const int bk = q < P ? ((unsigned)raw[j] < (unsigned)E ? raw[j] : E) : -1;
        sb.pair_bucket[q] = bk;
        if (bk >= 0)
            atomicAdd(&counts[bk], 1);
    }
    // chunk starts: exclusive sum of ceil(count / kMP) in bucket order
    int run = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {   // uniform
        const int b = b0 + lane;
        const int ch = b < B ? (counts[b] + kMP - 1) / kMP : 0;
        const int inc = wave_inclusive_sum(ch);
        if (b < B)
            sb.chunk_start[b] = run + inc - ch;
        run += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0)
        sb.chunk_start[B] = run;
    return run;
}

// Bucketing wave: bucket, pair count and pairs of routed chunk y into
// buffer buf.
__device__ __forceinline__ void self_pick(const GemvArgs &a, SelfBuckets &sb, int y, int buf) {
    const int lane = threadIdx.x & 63;
    const int P = a.n_pairs, B = a.num_experts + 1;
    int b = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {   // uniform
        const int bb = b0 + lane;
        const bool hit = bb < B && sb.chunk_start[bb] <= y && y < sb.chunk_start[bb + 1];
        const uint64_t m = __ballot(hit);
        if (m) {
            b = b0 + __builtin_ctzll(m);
            break;
        }
    }
    const int r0 = kMP * (y - sb.chunk_start[b]);
    int rank = 0;
    for (int q0 = 0; q0 < P; q0 += 64) {   // uniform
        const int q = q0 + lane;
        const bool in = q < P && sb.pair_bucket[q] == b;
        const uint64_t m = __ballot(in);
        const int r = rank + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (in && r >= r0 && r < r0 + kMP)
            sb.pairs[buf][r - r0] = q;
        rank += __popcll(m);
    }
    if (lane == 0) {
        sb.info[buf][0] = b;
        sb.info[buf][1] = rank - r0 < kMP ? rank - r0 : kMP;
    }
}

// Persistent grid over the items (chunk, row tile), chunk-major, the shared
// expert's chunks of 8 tokens after the routed ones.  The host cannot know the
// length of the chunk list, so a grid with one workgroup per possible item
// would mostly be workgroups that find their slot past its end; instead the
// grid holds as many workgroups as are resident at once and workgroup w takes
// items w, w + G, ...  With a bucket workspace the chunk list and pair lists
// come from it (the bucketing kernel's output); without one the workgroup
// builds them (self-bucketing, above).
template <int NT, int EPI, int SB, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SB <= 4 ? 3 : 2)))
void k_bucket_mfma(GemvArgs a, int tiles) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_b[];
    __shared__ SelfBuckets sbk;
    __shared__ int n_chunks_lds;
    fetch_args(a);
    const int tid = threadIdx.x, wave = tid >> 6;
    const int E = a.num_experts, P = a.n_pairs;
    const bool self = a.bucket == nullptr;
    const BucketView bv(self ? sbk.chunk_start : a.bucket, E, P);   // workspace mode only
    int n_chunks;
    if (self) {
        if (wave == 0) {
            const int nc = self_bucket(a, sbk, (int *)lds_b);
            if ((int)blockIdx.x / tiles < nc)
                self_pick(a, sbk, (int)blockIdx.x / tiles, 0);
            if ((tid & 63) == 0)
                n_chunks_lds = nc;
        }
        lds_barrier();
        n_chunks = n_chunks_lds;
    } else {
        n_chunks = *bv.n_chunks;
    }
    const int n_items = (n_chunks + (a.m_sh + kMP - 1) / kMP) * tiles;
    int kit = 0;
    for (int it = blockIdx.x; it < n_items; it += gridDim.x, kit++) {
        const int y = it / tiles, x = it - y * tiles;
        const bool shared = y >= n_chunks;
        const int buf = kit & 1;
        if (self && kit > 0) {
            // the other buffer holds the previous item's pairs, still read
            // by waves that have not finished it
            if (wave == 0 && !shared)
                self_pick(a, sbk, y, buf);
            lds_barrier();
        }
        int bkt = 0, cnt, first = 0;
        const int32_t *pl = sbk.pairs[buf];
        if (shared) {
            first = (y - n_chunks) * kMP;
            cnt = a.m_sh - first < kMP ? a.m_sh - first : kMP;
        } else if (!self) {
            bkt = bv.chunks[2 * y];
            const int packed = bv.chunks[2 * y + 1];
            cnt = packed >> 24;
            pl = bv.pairs + (packed & 0xFFFFFF);
        } else {
            bkt = sbk.info[buf][0];
            cnt = sbk.info[buf][1];
        }
        mfma_item<NT, EPI, SB, VEC>(a, shared, bkt, cnt, pl, first, x * item_rows(EPI), lds_b);
    }
}

// ------------------------------------------------------------------ host ---

template <int NT, int EPI, int SB, bool VEC>
static hipError_t go_mfma(const GemvArgs &a, hipStream_t st) {
    // chunks of the list: at most one partial chunk per non-empty bucket
    const int64_t nb_max = a.n_pairs < (int64_t)a.num_experts + 1 ? a.n_pairs : a.num_experts + 1;
    const int n_slots = (int)(nb_max + a.n_pairs / kMP);
    const int sh_groups = (a.m_sh + kMP - 1) / kMP;
    const int tiles = (a.n + item_rows(EPI) - 1) / item_rows(EPI);
    auto kern = k_bucket_mfma<NT, EPI, SB, VEC>;
    const size_t lds = set_lds((const void *)kern, mfma_lds_bytes(SB));
    // resident workgroups per CU: a property of the kernel and its fixed LDS
    // size, asked once per instantiation
    static const int fit = [&] {
        int f = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&f, (const void *)kern, kThreads, lds) !=
                hipSuccess ||
            f < 1)
            f = 1;
        return f;
    }();
    // as many workgroups as are resident at once, never more than the items
    // the longest possible list gives
    const int64_t items = (int64_t)(n_slots + sh_groups) * tiles;
    const int64_t cap = (int64_t)fit * cu_count();
    hipLaunchKernelGGL(kern, dim3((unsigned)(items < cap ? items : cap)), dim3(kThreads), lds, st,
                       a, tiles);
    return hipGetLastError();
}

// Superblocks per staged activation slab: 4 (three workgroups per CU fit
// beside a 33 KB slab; with two superblocks of weights in flight this beat
// whole-row slabs of 8 at two per CU), fewer when the row is shorter.
template <int NT, int EPI, bool VEC>
static hipError_t mfma_sb(const GemvArgs &a, hipStream_t st) {
    switch (a.k >> 8) {
    case 1: return go_mfma<NT, EPI, 1, VEC>(a, st);
    case 2: return go_mfma<NT, EPI, 2, VEC>(a, st);
    case 3: return go_mfma<NT, EPI, 3, VEC>(a, st);
    default: return go_mfma<NT, EPI, 4, VEC>(a, st);
    }
}

// Gate/up: the gate and up tiles of 64 rows; a single matrix: two 64-row
// groups of it (row pair).
hipError_t launch_q4k_gemv_mfma(const GemvArgs &a, bool fused_swiglu, hipStream_t st) {
    if (fused_swiglu)
        return a.vec ? mfma_sb<2, EPI_SWIGLU, true>(a, st) : mfma_sb<2, EPI_SWIGLU, false>(a, st);
    return a.vec ? mfma_sb<2, EPI_ROWPAIR, true>(a, st) : mfma_sb<2, EPI_ROWPAIR, false>(a, st);
}

}  // namespace q4k
