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
// Epilogue of a single-matrix launch whose two register tiles are two row
// groups of the same matrix (rows r and r + kMRows), so that an item covers
// 2 kMRows rows against one staged activation slab.
constexpr int kEpiRowPair = 2;
static_assert(kEpiRowPair != EPI_STORE && kEpiRowPair != EPI_SWIGLU, "epilogue ids");
__host__ __device__ constexpr int item_rows(int epi) { return epi == kEpiRowPair ? 2 * kMRows : kMRows; }
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
    if constexpr (EPI == kEpiRowPair) {   // the second row group of the same matrix
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
            if constexpr (EPI == kEpiRowPair) {
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
// step 1) done by every workgroup in LDS, so that a layer needs no separate
// bucketing launch: histogram of the ids over E + 1 buckets (bucket E takes
// ids outside [0, E)), chunks of at most kMP pairs per bucket in bucket order,
// the pairs of a bucket in ascending pair order.  This is the chunk list the
// bucketing kernel writes, in the same order, so an item computes exactly what
// it computes from that list.
constexpr int kSelfMaxPairs = 4 * kThreads;    // pairs 4 tid .. 4 tid + 3 per thread
constexpr int kSelfMaxBuckets = 4 * kThreads;  // buckets 4 tid .. 4 tid + 3 per thread
// chunks: at most one partial chunk per non-empty bucket plus P / kMP full ones
constexpr int kSelfMaxChunks = kSelfMaxBuckets + kSelfMaxPairs / kMP;
static_assert(kSelfMaxPairs == kSelfBucketMaxPairs && kSelfMaxBuckets == kSelfBucketMaxBuckets,
              "self-bucketing limits");
static_assert(kSelfMaxBuckets * 4 <= mfma_lds_bytes(1), "self-bucketing scratch");

// Exclusive sum over the workgroup of v (in thread order); wsum is 4 words of
// LDS that no thread reads until this returns.
__device__ __forceinline__ int block_exclusive_sum(int v, int *wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(inc, off, 64);
        if (lane >= off)
            inc += t;
    }
    if (lane == 63)
        wsum[wave] = inc;
    lds_barrier();
    int base = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; w++)
        base += w < wave ? wsum[w] : 0;
    return base + inc - v;
}

// Chunk list entry: bucket (11 bits), chunk index within the bucket (13 bits),
// pair count (<= kMP).
__device__ __forceinline__ int chunk_pack(int b, int i, int c) { return b | (i << 11) | (c << 24); }

// Persistent grid over the items (chunk, row tile), chunk-major, the shared
// expert's chunks of 8 tokens after the routed ones.  The host cannot know the
// length of the chunk list, so a grid with one workgroup per possible item
// would mostly be workgroups that find their slot past its end; instead the
// grid holds as many workgroups as are resident at once and workgroup w takes
// items w, w + G, ...  With a bucket workspace the chunk list and pair lists
// come from it (the bucketing kernel's output); without one the workgroup
// builds them (self-bucketing).
template <int NT, int EPI, int SB, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SB <= 4 ? 3 : 2)))
void k_bucket_mfma(GemvArgs a, int tiles) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_b[];
    __shared__ int chunk_list[kSelfMaxChunks];
    __shared__ int chunk_pairs[kMP];
    __shared__ int wsum[8];
    __shared__ int n_chunks_lds;
    fetch_args(a);
    const int tid = threadIdx.x;
    const int E = a.num_experts, P = a.n_pairs;
    const bool self = a.bucket == nullptr;
    const BucketView bv(self ? chunk_list : a.bucket, E, P);   // workspace mode only
    // 1. self-bucketing: the bucket of each of this thread's pairs
    //    4 tid .. 4 tid + 3 (-1 past P), from clamped unconditional loads
    int b[4] = {-1, -1, -1, -1};
    int n_chunks;
    if (self) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int p = 4 * tid + j;
            const int e = a.ids[p < P ? p : P - 1];
            b[j] = p < P ? ((unsigned)e < (unsigned)E ? e : E) : -1;
        }
        // 2. histogram (scratch in the staging LDS, free until the first item)
        int *counts = (int *)lds_b;
#pragma unroll
        for (int j = 0; j < 4; j++)
            counts[4 * tid + j] = 0;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 4; j++)
            if (b[j] >= 0)
                atomicAdd(&counts[b[j]], 1);
        lds_barrier();
        // 3. chunk list: buckets 4 tid .. 4 tid + 3, ceil(count / kMP) chunks each
        int c[4], hs = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int bb = 4 * tid + j;
            c[j] = bb <= E ? counts[bb] : 0;
            hs += (c[j] + kMP - 1) / kMP;
        }
        int run = block_exclusive_sum(hs, wsum);
#pragma unroll
        for (int j = 0; j < 4; j++)
            for (int i = 0; i * kMP < c[j]; i++) {
                const int n = c[j] - i * kMP < kMP ? c[j] - i * kMP : kMP;
                chunk_list[run++] = chunk_pack(4 * tid + j, i, n);
            }
        if (tid == kThreads - 1)
            n_chunks_lds = run;
        lds_barrier();
        n_chunks = n_chunks_lds;
    } else {
        n_chunks = *bv.n_chunks;
    }
    const int n_items = (n_chunks + (a.m_sh + kMP - 1) / kMP) * tiles;
    // 4. the items of this workgroup
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
        const int y = it / tiles, x = it - y * tiles;
        const bool shared = y >= n_chunks;
        int bkt = 0, cnt, first = 0;
        const int32_t *pl = chunk_pairs;
        if (shared) {
            first = (y - n_chunks) * kMP;
            cnt = a.m_sh - first < kMP ? a.m_sh - first : kMP;
        } else if (!self) {
            bkt = bv.chunks[2 * y];
            const int packed = bv.chunks[2 * y + 1];
            cnt = packed >> 24;
            pl = bv.pairs + (packed & 0xFFFFFF);
        } else {
            const int e = chunk_list[y];
            bkt = e & 0x7FF;
            cnt = e >> 24;
            const int i0 = ((e >> 11) & 0x1FFF) * kMP;
            // ranks of the bucket's pairs (ascending pair order); the
            // previous item has read chunk_pairs before the scan's barrier
            int f = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                f += b[j] == bkt ? 1 : 0;
            int rank = block_exclusive_sum(f, wsum + 4);
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (b[j] == bkt) {
                    if (rank >= i0 && rank < i0 + kMP)
                        chunk_pairs[rank - i0] = 4 * tid + j;
                    rank++;
                }
            lds_barrier();
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
    return a.vec ? mfma_sb<2, kEpiRowPair, true>(a, st) : mfma_sb<2, kEpiRowPair, false>(a, st);
}

}  // namespace q4k
