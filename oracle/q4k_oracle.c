/*
 * q4k_oracle.c -- plain CPU oracle for the Q4_K MoE expert path, the
 * Q4TiledP dense matvec, the MLX affine 4-bit and 2-bit expert codecs and the
 * chained RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers allowed.  The GPU library
 * never links, loads or calls this file, and this file includes nothing from
 * the GPU library: the two share no code, no headers and no tables.
 *
 * Style: scalar loops in the order the operation is defined.  Every floating
 * point sum is accumulated in double in ascending index order and rounded to
 * float once when it is stored.  Where a float decides an integer (the
 * quantizers), the decision is taken in float with plain IEEE operations (no
 * fused multiply-add, no fast-math), so that a GPU encoder following the same
 * steps reaches the same bytes.
 *
 * Sources (the three pages):
 *   [FK] ferrum-kernels 0.7.7, src/backend/metal/q4_k_moe_id_gemv_batched.rs
 *   [MF] moeflux 0.1.0-pre.3, src/riir/moe/expert_forward.rs
 *   [CE] cortiq-engine 0.7.7, examples/mv_lab.rs
 *
 * Parity status of each function is stated at the function.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_QK 256          /* weights per Q4_K superblock ([FK] test: QK_K)  */
#define ORC_BLOCK_BYTES 144 /* bytes per Q4_K superblock ([FK] test: BLOCK_BYTES) */
#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

#define ORC_SHARED_NONE 0
#define ORC_SHARED_SIGMOID 1
#define ORC_SHARED_UNSCALED 2

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, written from the format definition.          */
/* Pinned in the tests against numpy's float16 over all 65536 patterns.     */
/* ------------------------------------------------------------------------ */

double orc_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24  */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* 1.f * 2^(e-15)        */
    return sign ? -v : v;
}

float orc_f16_to_f32(uint16_t h) { return (float)orc_f16_value(h); }

/* Round-to-nearest-even, subnormals kept, overflow to +-inf. */
uint16_t orc_f32_to_f16(float xf)
{
    uint16_t sign = signbit(xf) ? 0x8000u : 0u;
    if (isnan(xf))
        return (uint16_t)(sign | 0x7e00u);
    if (isinf(xf))
        return (uint16_t)(sign | 0x7c00u);
    double a = fabs((double)xf);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);              /* a in [2^(e2-1), 2^e2)                     */
    int E = e2 - 1;             /* unbiased binade exponent                  */
    if (E < -14)
        E = -14;                /* the subnormal range shares the 2^-24 step */
    double quantum = ldexp(1.0, E - 10);
    double r = nearbyint(a / quantum) * quantum; /* exact divide, RNE        */
    if (r >= 65536.0)
        return (uint16_t)(sign | 0x7c00u);
    if (r < ldexp(1.0, -14))
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    frexp(r, &e2);
    E = e2 - 1;
    unsigned mant = (unsigned)(r / ldexp(1.0, E - 10)) - 1024u;
    return (uint16_t)(sign | (unsigned)((E + 15) << 10) | mant);
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 255); p[1] = (uint8_t)(v >> 8); }

/* ------------------------------------------------------------------------ */
/* Q4_K superblock (256 weights, 144 bytes; [FK] test asserts the length).   */
/* Reading of the bit layout (the pages do not print it; they name GGML's   */
/* Q4_K via candle): bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 twelve bytes */
/* holding eight 6-bit scales and eight 6-bit mins, 16-143 the nibbles.     */
/* ------------------------------------------------------------------------ */

/* Sub-block j's 6-bit scale and min out of the 12 packed bytes s[0..11]:
 * j < 4 : scale = low 6 bits of s[j],  min = low 6 bits of s[j+4];
 * j >= 4: scale = low nibble of s[j+4] with the top two bits of s[j-4] above it,
 *         min   = high nibble of s[j+4] with the top two bits of s[j] above it. */
void orc_q4k_get_scale_min(int j, const uint8_t *s, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Inverse of orc_q4k_get_scale_min for eight (scale, min) pairs in 0..63. */
void orc_q4k_set_scale_min(uint8_t *s, const int *sc, const int *m)
{
    for (int j = 0; j < 4; j++) {
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
}

/* Nibble of weight i (0..255) of a superblock.  The 128 nibble bytes form four
 * 32-byte chunks; chunk c covers weights 64c..64c+63: byte 32c+l holds weight
 * 64c+l in its low nibble and weight 64c+32+l in its high nibble. */
int orc_q4k_nibble(const uint8_t *blk, int i)
{
    const uint8_t *qs = blk + 16;
    int c = i / 64, r = i % 64;
    return r < 32 ? (qs[32 * c + r] & 15) : (qs[32 * c + r - 32] >> 4);
}

/* Dequantize: w_i = d*sc_j*q_i - dmin*m_j with j = i/32.  Each product and the
 * difference are exact in double; the one rounding is the store to float.
 * Pinned: hand-built blocks, brute-force scale packing, the fp32 exactness
 * argument checked against a float-only evaluation. */
void orc_q4k_dequantize(const uint8_t *blocks, int64_t n_blocks, float *out)
{
    for (int64_t b = 0; b < n_blocks; b++) {
        const uint8_t *blk = blocks + b * ORC_BLOCK_BYTES;
        double d = orc_f16_value(rd_u16(blk));
        double dmin = orc_f16_value(rd_u16(blk + 2));
        for (int i = 0; i < ORC_QK; i++) {
            int sc, m;
            orc_q4k_get_scale_min(i / 32, blk + 4, &sc, &m);
            double w = d * sc * orc_q4k_nibble(blk, i) - dmin * m;
            out[b * ORC_QK + i] = (float)w;
        }
    }
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* Q4_K quantizer.  The pages quantize with candle's GGML routine and do not
 * print it; this is a plain min/max affine encoder (reading, not GGML's
 * search):
 *   per 32-weight sub-block j: lo = min(0, min w), hi = max w,
 *       a_j = (hi - lo)/15, b_j = -lo;
 *   d = fp16(max_j a_j / 63), dmin = fp16(max_j b_j / 63);
 *   sc_j = clamp(rne(a_j / d), 0, 63), m_j = clamp(rne(b_j / dmin), 0, 63)
 *       (0 when the divisor is 0);
 *   q_i = clamp(rne((w_i + dmin*m_j) / (d*sc_j)), 0, 15)  (0 when d*sc_j == 0).
 * Every step is one IEEE float operation (products d*sc and dmin*m are exact).
 * Parity of the bytes is pinned by decode-error bounds and exact re-encoding of
 * on-grid blocks. */
int orc_q4k_quantize(const float *w, int64_t n_rows, int64_t k, uint8_t *out)
{
    if (k <= 0 || k % ORC_QK != 0 || n_rows < 0)
        return ORC_EINVAL;
    int64_t nb = n_rows * (k / ORC_QK);
    for (int64_t b = 0; b < nb; b++) {
        const float *x = w + b * ORC_QK;
        uint8_t *blk = out + b * ORC_BLOCK_BYTES;
        float a[8], bb[8];
        for (int j = 0; j < 8; j++) {
            float lo = 0.0f, hi = x[32 * j];
            for (int i = 0; i < 32; i++) {
                float v = x[32 * j + i];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            a[j] = (hi - lo) / 15.0f;
            bb[j] = 0.0f - lo;
        }
        float amax = 0.0f, bmax = 0.0f;
        for (int j = 0; j < 8; j++) {
            if (a[j] > amax) amax = a[j];
            if (bb[j] > bmax) bmax = bb[j];
        }
        uint16_t dh = orc_f32_to_f16(amax / 63.0f);
        uint16_t mh = orc_f32_to_f16(bmax / 63.0f);
        float df = orc_f16_to_f32(dh), mf = orc_f16_to_f32(mh);
        int sc[8], mn[8];
        for (int j = 0; j < 8; j++) {
            sc[j] = df > 0.0f ? clampi((int)rintf(a[j] / df), 0, 63) : 0;
            mn[j] = mf > 0.0f ? clampi((int)rintf(bb[j] / mf), 0, 63) : 0;
        }
        wr_u16(blk, dh);
        wr_u16(blk + 2, mh);
        orc_q4k_set_scale_min(blk + 4, sc, mn);
        int q[ORC_QK];
        for (int i = 0; i < ORC_QK; i++) {
            int j = i / 32;
            float s = df * (float)sc[j];
            float o = mf * (float)mn[j];
            float num = x[i] + o;
            q[i] = s > 0.0f ? clampi((int)rintf(num / s), 0, 15) : 0;
        }
        uint8_t *qs = blk + 16;
        for (int c = 0; c < 4; c++)
            for (int l = 0; l < 32; l++)
                qs[32 * c + l] = (uint8_t)(q[64 * c + l] | (q[64 * c + 32 + l] << 4));
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Indirect-dispatch (id) GEMV over a stacked expert tensor.                 */
/* [FK] dispatch_gemv_q4k_moe_id_batched_on_encoder: weights are             */
/* [num_experts, n, k/256] superblocks, nb01 = (k/256)*144 bytes per row,   */
/* nb02 = n*nb01 per expert; ids is flat [m*top_k] with                     */
/* pair = token*top_k + slot; out is [m*top_k, n]; the activation row of a  */
/* pair starts at src1 + token*outer + slot*inner (floats; module doc).     */
/* Reading for ids outside [0, num_experts): the pair's row is zero.        */
/* Definition: dequantize the row, dot it with the activation row in double.*/
/* ------------------------------------------------------------------------ */

static double q4k_row_dot(const uint8_t *row, int64_t k, const float *x, float *tmp)
{
    orc_q4k_dequantize(row, k / ORC_QK, tmp);
    double acc = 0.0;
    for (int64_t c = 0; c < k; c++)
        acc += (double)tmp[c] * (double)x[c];
    return acc;
}

int orc_q4k_moe_id_gemv(const uint8_t *w, int64_t num_experts, int64_t n, int64_t k,
                        const float *src1, const int32_t *ids, int64_t m, int64_t top_k,
                        int64_t outer, int64_t inner, float *dst)
{
    if (k <= 0 || k % ORC_QK || n <= 0 || m < 0 || top_k <= 0 || num_experts <= 0)
        return ORC_EINVAL;
    float *tmp = (float *)malloc((size_t)k * sizeof(float));
    if (!tmp)
        return ORC_ENOMEM;
    int64_t nb01 = (k / ORC_QK) * ORC_BLOCK_BYTES;
    int64_t nb02 = n * nb01;
    for (int64_t p = 0; p < m * top_k; p++) {
        int64_t t = p / top_k, s = p % top_k;
        int64_t e = ids[p];
        const float *x = src1 + t * outer + s * inner;
        for (int64_t r = 0; r < n; r++) {
            if (e < 0 || e >= num_experts)
                dst[p * n + r] = 0.0f;
            else
                dst[p * n + r] = (float)q4k_row_dot(w + e * nb02 + r * nb01, k, x, tmp);
        }
    }
    free(tmp);
    return ORC_OK;
}

/* One output element (pair p, row r) of the id-GEMV, for sampled checks at
 * sizes where the full product is too slow on the CPU. Same definition. */
float orc_q4k_moe_id_gemv_one(const uint8_t *w, int64_t num_experts, int64_t n, int64_t k,
                              const float *src1, const int32_t *ids, int64_t top_k,
                              int64_t outer, int64_t inner, int64_t p, int64_t r)
{
    int64_t e = ids[p];
    if (e < 0 || e >= num_experts)
        return 0.0f;
    float *tmp = (float *)malloc((size_t)k * sizeof(float));
    if (!tmp)
        return NAN;
    int64_t nb01 = (k / ORC_QK) * ORC_BLOCK_BYTES;
    const float *x = src1 + (p / top_k) * outer + (p % top_k) * inner;
    float v = (float)q4k_row_dot(w + e * n * nb01 + r * nb01, k, x, tmp);
    free(tmp);
    return v;
}

/* ------------------------------------------------------------------------ */
/* Expert FFN: gate/up id-GEMV -> SwiGLU -> down id-GEMV.                    */
/* [MF] module doc (the four-dispatch single-expert sequence) and           */
/* encode_moe_gather_id_fuse (gate/up read one row per token, down reads    */
/* one row per (token, slot): outer = top_k*inter, inner = inter).          */
/* Intermediate buffers are float, as the pages store them.                  */
/* SiLU is the textbook z/(1+e^-z); the pages name it without a formula.    */
/* ------------------------------------------------------------------------ */

double orc_silu(double z) { return z / (1.0 + exp(-z)); }
double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

int orc_moe_expert_ffn(const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                       int64_t num_experts, int64_t hidden, int64_t inter,
                       const float *h_post, const int32_t *ids, int64_t m, int64_t top_k,
                       float *gate_out, float *up_out, float *act, float *expert_out)
{
    int64_t P = m * top_k;
    int rc = orc_q4k_moe_id_gemv(w_gate, num_experts, inter, hidden, h_post, ids, m, top_k,
                                 hidden, 0, gate_out);
    if (rc)
        return rc;
    rc = orc_q4k_moe_id_gemv(w_up, num_experts, inter, hidden, h_post, ids, m, top_k,
                             hidden, 0, up_out);
    if (rc)
        return rc;
    for (int64_t i = 0; i < P * inter; i++)
        act[i] = (float)(orc_silu((double)gate_out[i]) * (double)up_out[i]);
    return orc_q4k_moe_id_gemv(w_down, num_experts, hidden, inter, act, ids, m, top_k,
                               top_k * inter, inter, expert_out);
}

/* ------------------------------------------------------------------------ */
/* Weighted combine with residual and shared expert.                         */
/* [MF] module doc and encode_moe_combine_residual_n_tokens:                */
/*   out[t,i] = h_mid[t,i] + sum_s w[t,s]*expert_out[t,s,i] + g_t*shared[t,i]*/
/* with g_t = sigmoid(logit_t) (sigmoid gate), 1 (unscaled: combine_kernel_ */
/* name / the variant comment), or no shared term.  Slots in order.        */
/* ------------------------------------------------------------------------ */

int orc_moe_combine_residual(const float *h_mid, const float *expert_out, const float *route_w,
                             const float *shared_out, const float *shared_gate_logit, float *out,
                             int64_t hidden, int64_t m, int64_t top_k, int shared_mode)
{
    if (shared_mode < ORC_SHARED_NONE || shared_mode > ORC_SHARED_UNSCALED)
        return ORC_EINVAL;
    for (int64_t t = 0; t < m; t++) {
        double g = 0.0;
        if (shared_mode == ORC_SHARED_SIGMOID)
            g = orc_sigmoid((double)shared_gate_logit[t]);
        else if (shared_mode == ORC_SHARED_UNSCALED)
            g = 1.0;
        for (int64_t i = 0; i < hidden; i++) {
            double acc = (double)h_mid[t * hidden + i];
            for (int64_t s = 0; s < top_k; s++)
                acc += (double)route_w[t * top_k + s] *
                       (double)expert_out[(t * top_k + s) * hidden + i];
            if (shared_mode != ORC_SHARED_NONE)
                acc += g * (double)shared_out[t * hidden + i];
            out[t * hidden + i] = (float)acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert bucketing ([MF] encode_moe_batched_permute_fuse: group (token,    */
/* slot) pairs by expert id and process each group once; ExpertBuckets is   */
/* CSR by expert; encode_moe_gather_id_fuse's map0 builds the per-expert    */
/* counts and pair lists on the device).                                    */
/* Output: counts[E+1] (bucket E collects ids outside [0,E)),               */
/* offsets[E+2] (exclusive prefix sum), pairs[P] grouped by bucket, pair    */
/* indices ascending inside a bucket (reading: stable order).               */
/* Integer work; pinned by brute force in the tests.                        */
/* ------------------------------------------------------------------------ */

int orc_moe_bucket(const int32_t *ids, int64_t n_pairs, int64_t num_experts,
                   int32_t *counts, int32_t *offsets, int32_t *pairs)
{
    if (n_pairs < 0 || num_experts <= 0)
        return ORC_EINVAL;
    for (int64_t b = 0; b <= num_experts; b++)
        counts[b] = 0;
    for (int64_t p = 0; p < n_pairs; p++) {
        int64_t e = ids[p];
        counts[(e < 0 || e >= num_experts) ? num_experts : e]++;
    }
    offsets[0] = 0;
    for (int64_t b = 0; b <= num_experts; b++)
        offsets[b + 1] = offsets[b] + counts[b];
    int64_t pos = 0;
    for (int64_t b = 0; b <= num_experts; b++)
        for (int64_t p = 0; p < n_pairs; p++) {
            int64_t e = ids[p];
            int64_t bp = (e < 0 || e >= num_experts) ? num_experts : e;
            if (bp == b)
                pairs[pos++] = (int32_t)p;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Q4TiledP dense tensor ([CE] production kernel `cur` and its helpers).    */
/* rows x cols, gpr = cols/32 groups per row:                               */
/*   bytes [0, rows*gpr*16): group (r,g) at (r*gpr+g)*16; byte i of a group */
/*       holds element 2i in its low nibble and 2i+1 in its high nibble     */
/*       (q4_dot8_fast), value = nibble - 8;                                 */
/*   params_off = rows*gpr*16: per row two fp16, base then step;            */
/*   codes_off = params_off + rows*4: per row ceil(5*gpr/8) bytes, the code */
/*       of group g in bits 5g..5g+4, least significant bit first;          */
/*   scale of a group = 2^(base + code*step).                               */
/* The exponent base + code*step is formed in float as the kernel does      */
/* (the product is exact); 2^e is evaluated in double and rounded to float  */
/* once (reading: the exact power, where the page's exp2 is approximate).   */
/* ------------------------------------------------------------------------ */

int64_t orc_q4tp_bytes(int64_t rows, int64_t cols)
{
    int64_t gpr = cols / 32;
    return rows * gpr * 16 + rows * 4 + rows * ((5 * gpr + 7) / 8);
}

int orc_q4tp_code(const uint8_t *t, int64_t rows, int64_t cols, int64_t r, int64_t g)
{
    int64_t gpr = cols / 32;
    int64_t codes_off = rows * gpr * 16 + rows * 4;
    int64_t stride = (5 * gpr + 7) / 8;
    int code = 0;
    for (int b = 0; b < 5; b++) {
        int64_t bit = 5 * g + b;
        int v = (t[codes_off + r * stride + bit / 8] >> (bit % 8)) & 1;
        code |= v << b;
    }
    return code;
}

float orc_q4tp_rung(uint16_t base, uint16_t step, int code)
{
    float e = orc_f16_to_f32(base) + (float)code * orc_f16_to_f32(step);
    return (float)exp2((double)e);
}

static void q4tp_row_params(const uint8_t *t, int64_t rows, int64_t cols, int64_t r,
                            uint16_t *base, uint16_t *step)
{
    int64_t gpr = cols / 32;
    const uint8_t *p = t + rows * gpr * 16 + r * 4;
    *base = rd_u16(p);
    *step = rd_u16(p + 2);
}

int orc_q4tp_nibble(const uint8_t *t, int64_t cols, int64_t r, int64_t c)
{
    int64_t gpr = cols / 32;
    int64_t g = c / 32, e = c % 32;
    uint8_t byte = t[(r * gpr + g) * 16 + e / 2];
    return (e % 2) ? (byte >> 4) : (byte & 15);
}

void orc_q4tp_dequantize(const uint8_t *t, int64_t rows, int64_t cols, float *out)
{
    int64_t gpr = cols / 32;
    for (int64_t r = 0; r < rows; r++) {
        uint16_t base, step;
        q4tp_row_params(t, rows, cols, r, &base, &step);
        for (int64_t g = 0; g < gpr; g++) {
            double L = orc_q4tp_rung(base, step, orc_q4tp_code(t, rows, cols, r, g));
            for (int64_t e = 0; e < 32; e++)
                out[r * cols + 32 * g + e] =
                    (float)(L * (orc_q4tp_nibble(t, cols, r, 32 * g + e) - 8));
        }
    }
}

/* y[r] = sum_g scale(r,g) * sum_j (nib - 8) * x[32g+j], in double. */
static double q4tp_row_dot(const uint8_t *t, int64_t rows, int64_t cols, int64_t r, const float *x)
{
    int64_t gpr = cols / 32;
    uint16_t base, step;
    q4tp_row_params(t, rows, cols, r, &base, &step);
    double acc = 0.0;
    for (int64_t g = 0; g < gpr; g++) {
        double gs = 0.0;
        for (int64_t e = 0; e < 32; e++)
            gs += (double)(orc_q4tp_nibble(t, cols, r, 32 * g + e) - 8) * (double)x[32 * g + e];
        acc += (double)orc_q4tp_rung(base, step, orc_q4tp_code(t, rows, cols, r, g)) * gs;
    }
    return acc;
}

int orc_q4tp_matvec(const uint8_t *t, int64_t rows, int64_t cols, const float *x, float *y)
{
    if (rows <= 0 || cols <= 0 || cols % 32)
        return ORC_EINVAL;
    for (int64_t r = 0; r < rows; r++)
        y[r] = (float)q4tp_row_dot(t, rows, cols, r, x);
    return ORC_OK;
}

float orc_q4tp_matvec_one(const uint8_t *t, int64_t rows, int64_t cols, const float *x, int64_t r)
{
    return (float)q4tp_row_dot(t, rows, cols, r, x);
}

/* Q4TiledP encoder.  The page reads model files and prints no encoder; this is
 * a plain reading:
 *   per group: t_g = max|w| / 7 (float); lt_g = float(log2(t_g)) for t_g > 0;
 *   per row: base = fp16(min_g lt_g), step = fp16(max(0, max_g lt_g - base)/31)
 *       (both 0 when every group is zero);
 *   code_g = clamp(rne((lt_g - base)/step), 0, 31) (0 if step == 0 or t_g == 0);
 *   q = clamp(rne(w / scale(code_g)), -8, 7), stored as q + 8 (8 for zero groups).
 * log2 and 2^x are evaluated in double and rounded to float; everything else is
 * single float operations. */
int orc_q4tp_quantize(const float *w, int64_t rows, int64_t cols, uint8_t *out)
{
    if (rows <= 0 || cols <= 0 || cols % 32)
        return ORC_EINVAL;
    int64_t gpr = cols / 32;
    int64_t params_off = rows * gpr * 16;
    int64_t codes_off = params_off + rows * 4;
    int64_t stride = (5 * gpr + 7) / 8;
    float *lt = (float *)malloc((size_t)gpr * sizeof(float));
    int *has = (int *)malloc((size_t)gpr * sizeof(int));
    if (!lt || !has) {
        free(lt);
        free(has);
        return ORC_ENOMEM;
    }
    memset(out + codes_off, 0, (size_t)(rows * stride));
    for (int64_t r = 0; r < rows; r++) {
        const float *x = w + r * cols;
        int any = 0;
        float lmin = 0.0f, lmax = 0.0f;
        for (int64_t g = 0; g < gpr; g++) {
            float amax = 0.0f;
            for (int e = 0; e < 32; e++) {
                float a = fabsf(x[32 * g + e]);
                if (a > amax) amax = a;
            }
            float tg = amax / 7.0f;
            has[g] = tg > 0.0f;
            lt[g] = has[g] ? (float)log2((double)tg) : 0.0f;
            if (has[g]) {
                if (!any || lt[g] < lmin) lmin = lt[g];
                if (!any || lt[g] > lmax) lmax = lt[g];
                any = 1;
            }
        }
        uint16_t base = 0, step = 0;
        if (any) {
            base = orc_f32_to_f16(lmin);
            float span = lmax - orc_f16_to_f32(base);
            if (span < 0.0f) span = 0.0f;
            step = orc_f32_to_f16(span / 31.0f);
        }
        float bf = orc_f16_to_f32(base), sf = orc_f16_to_f32(step);
        wr_u16(out + params_off + r * 4, base);
        wr_u16(out + params_off + r * 4 + 2, step);
        for (int64_t g = 0; g < gpr; g++) {
            int code = 0;
            if (has[g] && sf > 0.0f)
                code = clampi((int)rintf((lt[g] - bf) / sf), 0, 31);
            float L = orc_q4tp_rung(base, step, code);
            uint8_t *grp = out + (r * gpr + g) * 16;
            for (int i = 0; i < 16; i++) {
                int nib[2];
                for (int h = 0; h < 2; h++) {
                    int q = 0;
                    if (has[g] && L > 0.0f)
                        q = clampi((int)rintf(x[32 * g + 2 * i + h] / L), -8, 7);
                    nib[h] = q + 8;
                }
                grp[i] = (uint8_t)(nib[0] | (nib[1] << 4));
            }
            for (int b = 0; b < 5; b++) {
                int64_t bit = 5 * g + b;
                if ((code >> b) & 1)
                    out[codes_off + r * stride + bit / 8] |= (uint8_t)(1u << (bit % 8));
            }
        }
    }
    free(lt);
    free(has);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MLX affine 4-bit expert codec ([MF] module doc "4-bit only";             */
/* gpu_expert_forward and encode_matvec: GROUP_SIZE passed to the matvec;   */
/* encode_moe_gather_id_fuse: per-row strides nb01_w = K/2 bytes of packed  */
/* weights and nb01_s = (K/64)*2 bytes of bf16 scales, the same for the     */
/* bf16 biases, sub-tensors at packed/scales/biases offsets inside an       */
/* expert block of expert_stride bytes).                                    */
/*                                                                          */
/* Readings (the pages give the strides, not the bit-level format): the     */
/* public MLX affine layout, group of 64 weights along a row, weight        */
/* w = scale*q + bias with q the 4-bit code; row r's packed byte j holds    */
/* weight 2j in its low nibble and 2j+1 in its high nibble (MLX packs eight */
/* codes per little-endian 32-bit word, lowest code in the lowest bits).    */
/* ------------------------------------------------------------------------ */

#define ORC_MLX_GROUP 64

/* bfloat16 <-> binary32 from the format definition: bf16 is the top half of */
/* a binary32, so widening is exact; narrowing rounds to nearest, ties to   */
/* even, NaN stays a (quiet) NaN.  Pinned against torch's bfloat16.         */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);               /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;                                        /* RNE       */
    return (uint16_t)(u >> 16);
}

int orc_mlx4_nibble(const uint8_t *row, int64_t c)
{
    uint8_t b = row[c / 2];
    return (c & 1) ? (b >> 4) : (b & 15);
}

/* Dequantize one [n, k] matrix.  w = scale*q + bias evaluated in float:    */
/* scale has 8 significant bits and q 4, so scale*q is exact and the one    */
/* rounding is that of the sum (the correctly rounded value of the exact    */
/* scale*q + bias, whatever the evaluation order).  Parity: bit-exact.      */
void orc_mlx4_dequantize(const uint8_t *packed, const uint16_t *scales, const uint16_t *biases,
                         int64_t n, int64_t k, float *out)
{
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            float s = orc_bf16_to_f32(scales[r * gpr + c / ORC_MLX_GROUP]);
            float b = orc_bf16_to_f32(biases[r * gpr + c / ORC_MLX_GROUP]);
            float p = s * (float)orc_mlx4_nibble(packed + r * (k / 2), c);
            out[r * k + c] = p + b;
        }
}

/* Encoder (the pages print none; reading, a plain min/max affine code per  */
/* group, decided in float with IEEE operations): lo = min w, hi = max w,   */
/* scale = bf16((hi - lo)/15), bias = bf16(lo),                             */
/* q = clamp(rne((w - bias)/scale), 0, 15), q = 0 where scale is 0.         */
/* Its reconstruction quality against MLX's own quantizer is parity        */
/* unpinned (MLX is not here); its bytes are compared with the GPU's.       */
int orc_mlx4_quantize(const float *w, int64_t n, int64_t k, uint8_t *packed, uint16_t *scales,
                      uint16_t *biases)
{
    if (n <= 0 || k <= 0 || k % ORC_MLX_GROUP)
        return ORC_EINVAL;
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t r = 0; r < n; r++)
        for (int64_t g = 0; g < gpr; g++) {
            const float *x = w + r * k + g * ORC_MLX_GROUP;
            float lo = x[0], hi = x[0];
            for (int j = 1; j < ORC_MLX_GROUP; j++) {
                lo = x[j] < lo ? x[j] : lo;
                hi = x[j] > hi ? x[j] : hi;
            }
            float d = hi - lo;
            uint16_t sh = orc_f32_to_bf16(d / 15.0f);
            uint16_t bh = orc_f32_to_bf16(lo);
            float s = orc_bf16_to_f32(sh), b = orc_bf16_to_f32(bh);
            scales[r * gpr + g] = sh;
            biases[r * gpr + g] = bh;
            uint8_t *row = packed + r * (k / 2) + g * (ORC_MLX_GROUP / 2);
            for (int j = 0; j < ORC_MLX_GROUP; j += 2) {
                int q[2];
                for (int h = 0; h < 2; h++) {
                    float t = (x[j + h] - b) / s;
                    q[h] = s == 0.0f ? 0 : clampi((int)rintf(t), 0, 15);
                }
                row[j / 2] = (uint8_t)(q[0] | (q[1] << 4));
            }
        }
    return ORC_OK;
}

/* id-GEMV over MLX 4-bit experts ([MF] encode_moe_gather_id_fuse: src0 =  */
/* expert base, expert e's block at e*expert_stride, its packed weights,    */
/* scales and biases at the given offsets inside the block; [FK] module     */
/* doc for the pair walk: pair p = token*top_k + slot, activation row at    */
/* src1 + token*outer + slot*inner).  Ids outside [0, num_experts): zero    */
/* rows.  Definition: dequantize the row, dot in double, ascending column.  */
int orc_mlx4_moe_id_gemv(const uint8_t *base, int64_t expert_stride, int64_t packed_off,
                         int64_t scales_off, int64_t biases_off, int64_t num_experts, int64_t n,
                         int64_t k, const float *src1, const int32_t *ids, int64_t m,
                         int64_t top_k, int64_t outer, int64_t inner, float *dst)
{
    if (k <= 0 || k % ORC_MLX_GROUP || n <= 0 || m < 0 || top_k <= 0 || num_experts <= 0)
        return ORC_EINVAL;
    float *tmp = (float *)malloc((size_t)k * sizeof(float));
    if (!tmp)
        return ORC_ENOMEM;
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t p = 0; p < m * top_k; p++) {
        int64_t t = p / top_k, s = p % top_k;
        int64_t e = ids[p];
        const float *x = src1 + t * outer + s * inner;
        for (int64_t r = 0; r < n; r++) {
            if (e < 0 || e >= num_experts) {
                dst[p * n + r] = 0.0f;
                continue;
            }
            const uint8_t *blk = base + e * expert_stride;
            orc_mlx4_dequantize(blk + packed_off + r * (k / 2),
                                (const uint16_t *)(blk + scales_off) + r * gpr,
                                (const uint16_t *)(blk + biases_off) + r * gpr, 1, k, tmp);
            double acc = 0.0;
            for (int64_t c = 0; c < k; c++)
                acc += (double)tmp[c] * (double)x[c];
            dst[p * n + r] = (float)acc;
        }
    }
    free(tmp);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MLX affine 2-bit expert codec ([MF] module doc: g_use_2bit selects the    */
/* 2-bit matvec and expert-block layout).  Reading: MLX's 2-bit affine       */
/* format, the 4-bit one with 2-bit codes: groups of 64 along a row, bf16   */
/* scale and bias per group, w = scale*q + bias with q in 0..3, row byte j  */
/* holding weights 4j..4j+3 at bits 0-1, 2-3, 4-5, 6-7 (16 codes per        */
/* little-endian 32-bit word, lowest code in the lowest bits).  Packed rows */
/* take k/4 bytes.                                                           */
/* ------------------------------------------------------------------------ */

int orc_mlx2_code(const uint8_t *row, int64_t c)
{
    return (row[c / 4] >> (2 * (c & 3))) & 3;
}

/* Dequantize: scale*q is exact (8 + 2 significant bits), the sum rounds    */
/* once.  Parity: bit-exact.                                                 */
void orc_mlx2_dequantize(const uint8_t *packed, const uint16_t *scales, const uint16_t *biases,
                         int64_t n, int64_t k, float *out)
{
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            float s = orc_bf16_to_f32(scales[r * gpr + c / ORC_MLX_GROUP]);
            float b = orc_bf16_to_f32(biases[r * gpr + c / ORC_MLX_GROUP]);
            float p = s * (float)orc_mlx2_code(packed + r * (k / 4), c);
            out[r * k + c] = p + b;
        }
}

/* Encoder (reading, as the 4-bit one with 3 steps): lo = min w, hi = max w, */
/* scale = bf16((hi - lo)/3), bias = bf16(lo),                              */
/* q = clamp(rne((w - bias)/scale), 0, 3), 0 where the scale is 0.  Parity   */
/* on bytes; quality against MLX's quantizer unpinned.                       */
int orc_mlx2_quantize(const float *w, int64_t n, int64_t k, uint8_t *packed, uint16_t *scales,
                      uint16_t *biases)
{
    if (n <= 0 || k <= 0 || k % ORC_MLX_GROUP)
        return ORC_EINVAL;
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t r = 0; r < n; r++)
        for (int64_t g = 0; g < gpr; g++) {
            const float *x = w + r * k + g * ORC_MLX_GROUP;
            float lo = x[0], hi = x[0];
            for (int j = 1; j < ORC_MLX_GROUP; j++) {
                lo = x[j] < lo ? x[j] : lo;
                hi = x[j] > hi ? x[j] : hi;
            }
            float d = hi - lo;
            uint16_t sh = orc_f32_to_bf16(d / 3.0f);
            uint16_t bh = orc_f32_to_bf16(lo);
            float s = orc_bf16_to_f32(sh), b = orc_bf16_to_f32(bh);
            scales[r * gpr + g] = sh;
            biases[r * gpr + g] = bh;
            uint8_t *row = packed + r * (k / 4) + g * (ORC_MLX_GROUP / 4);
            for (int j = 0; j < ORC_MLX_GROUP; j += 4) {
                int byte = 0;
                for (int h = 0; h < 4; h++) {
                    float t = (x[j + h] - b) / s;
                    int q = s == 0.0f ? 0 : clampi((int)rintf(t), 0, 3);
                    byte |= q << (2 * h);
                }
                row[j / 4] = (uint8_t)byte;
            }
        }
    return ORC_OK;
}

/* id-GEMV over MLX 2-bit experts: as orc_mlx4_moe_id_gemv with the 2-bit   */
/* rows (k/4 packed bytes).                                                   */
int orc_mlx2_moe_id_gemv(const uint8_t *base, int64_t expert_stride, int64_t packed_off,
                         int64_t scales_off, int64_t biases_off, int64_t num_experts, int64_t n,
                         int64_t k, const float *src1, const int32_t *ids, int64_t m,
                         int64_t top_k, int64_t outer, int64_t inner, float *dst)
{
    if (k <= 0 || k % ORC_MLX_GROUP || n <= 0 || m < 0 || top_k <= 0 || num_experts <= 0)
        return ORC_EINVAL;
    float *tmp = (float *)malloc((size_t)k * sizeof(float));
    if (!tmp)
        return ORC_ENOMEM;
    int64_t gpr = k / ORC_MLX_GROUP;
    for (int64_t p = 0; p < m * top_k; p++) {
        int64_t t = p / top_k, s = p % top_k;
        int64_t e = ids[p];
        const float *x = src1 + t * outer + s * inner;
        for (int64_t r = 0; r < n; r++) {
            if (e < 0 || e >= num_experts) {
                dst[p * n + r] = 0.0f;
                continue;
            }
            const uint8_t *blk = base + e * expert_stride;
            orc_mlx2_dequantize(blk + packed_off + r * (k / 4),
                                (const uint16_t *)(blk + scales_off) + r * gpr,
                                (const uint16_t *)(blk + biases_off) + r * gpr, 1, k, tmp);
            double acc = 0.0;
            for (int64_t c = 0; c < k; c++)
                acc += (double)tmp[c] * (double)x[c];
            dst[p * n + r] = (float)acc;
        }
    }
    free(tmp);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Chained RMSNorm of the combine output ([MF] ChainToNormed and the chain  */
/* appendix after the combine: rms_norm_sum_sq, then rms_norm_apply_bf16    */
/* with the next layer's input-norm weight, bf16, and eps):                 */
/*   normed[t,i] = x[t,i] / sqrt(sum_j x[t,j]^2 / H + eps) * w[i].           */
/* The pages name the two kernels and their inputs, not the formula; this   */
/* is the textbook RMSNorm.  Sum of squares and the scaling in double,      */
/* stored as float.                                                          */
/* ------------------------------------------------------------------------ */
int orc_rmsnorm_bf16(const float *x, const uint16_t *w, float eps, int64_t m, int64_t hidden,
                     float *out)
{
    if (m < 0 || hidden <= 0)
        return ORC_EINVAL;
    for (int64_t t = 0; t < m; t++) {
        const float *row = x + t * hidden;
        double ss = 0.0;
        for (int64_t i = 0; i < hidden; i++)
            ss += (double)row[i] * (double)row[i];
        double inv = 1.0 / sqrt(ss / (double)hidden + (double)eps);
        for (int64_t i = 0; i < hidden; i++)
            out[t * hidden + i] = (float)((double)row[i] * inv * (double)orc_bf16_to_f32(w[i]));
    }
    return ORC_OK;
}
