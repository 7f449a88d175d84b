/*
 * q4kmoe.h -- C ABI of the Q4_K MoE expert library for AMD MI355X (gfx950).
 *
 * Sources (the three pages this library implements):
 *   [FK] ferrum-kernels 0.7.7, src/backend/metal/q4_k_moe_id_gemv_batched.rs
 *   [MF] moeflux 0.1.0-pre.3, src/riir/moe/expert_forward.rs
 *   [CE] cortiq-engine 0.7.7, examples/mv_lab.rs
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes.  Scratch memory is a caller
 *     buffer (`ws`, `ws_bytes`) where a call needs one.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns; results are visible to
 *     later work on the same stream.
 *   - Arguments are validated on the host before any HIP call; a bad argument
 *     returns a nonzero status and enqueues nothing.  A failed launch returns
 *     Q4K_ERR_LAUNCH.  q4k_status_string() names every status.
 *   - Strides are in elements (floats), as in [FK]'s module doc.
 *   - Activations and outputs are fp32, row-major.
 *   - Calls are stateless and may be issued from several host threads.
 */
#ifndef Q4KMOE_H
#define Q4KMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    Q4K_OK = 0,
    Q4K_ERR_SHAPE = 1,     /* a size is out of range or not a required multiple */
    Q4K_ERR_NULL = 2,      /* a required pointer is NULL                        */
    Q4K_ERR_STRIDE = 3,    /* an activation stride is negative                  */
    Q4K_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
    Q4K_ERR_LAUNCH = 5,    /* the HIP runtime rejected a launch                 */
    Q4K_ERR_ARG = 6,       /* an enum argument has an unknown value             */
    Q4K_ERR_SCRATCH = 7    /* the no-allocation layer's scratch is too small    */
};

/* Bucketing flag of the id-GEMV, FFN and layer entry points ([MF]
 * encode_moe_batched_permute_fuse: group (token, slot) pairs by expert so each
 * expert's weights are read once).  A flag is one mode, optionally OR-ed with
 * schedule bits.
 *
 * Modes:
 *   OFF      pair mode (token mode in the layer): every pair reads its
 *            expert's rows itself, on the vector units.
 *   ON       bucketed: one work item per chunk of at most Q4K_BUCKET_CHUNK
 *            pairs of one expert, which reads the expert's rows once for all
 *            of them.
 *   AUTO     ON when m >= Q4K_AUTO_BUCKET_MIN_TOKENS, else OFF.  At fewer
 *            tokens most experts serve a single pair, so there is no dense
 *            contraction to gain from.
 *   PREBUILT ON, on a workspace that moe_bucket (or an earlier call) already
 *            filled for the same ids, so gate/up and down pay for one
 *            bucketing pass (the layer entry points treat it as ON).
 * Schedule bits:
 *   Q4K_SCHED_VECTOR        bucketed work runs on the vector units (the same
 *                           per-weight arithmetic and order as pair mode)
 *                           instead of the matrix cores.
 *   Q4K_SCHED_BUCKET_LAUNCH layer entry points: bucket with a separate
 *                           launch into the workspace rather than inside the
 *                           matrix-core launches (both give the same chunk
 *                           lists, so the same bits).  Ignored elsewhere.
 * An unknown mode or bit returns Q4K_ERR_ARG.
 *
 * Numerics: the output depends only on the arguments, never on the process
 * environment.  Pair mode, token mode and vector-unit bucketing share one
 * per-weight arithmetic and summation order, so they agree bit for bit, and
 * a batch equals the same pairs run one token at a time bit for bit.  The
 * matrix-core schedule (ON and PREBUILT without Q4K_SCHED_VECTOR) sums in the
 * matrix core's order with each activation carried as two fp16 parts after
 * an exact power-of-two scaling per (pair, superblock); it agrees with the
 * vector-unit schedules within the fp32 band
 * (max_abs_diff <= 1e-3 * max|out|, cosine >= 0.9999) at any finite
 * activation scale, and repeated calls of it give identical bits. */
enum { Q4K_BUCKET_AUTO = 0, Q4K_BUCKET_OFF = 1, Q4K_BUCKET_ON = 2, Q4K_BUCKET_PREBUILT = 3 };
#define Q4K_BUCKET_MODE_MASK 0xFF
#define Q4K_SCHED_VECTOR 0x100
#define Q4K_SCHED_BUCKET_LAUNCH 0x200
#define Q4K_AUTO_BUCKET_MIN_TOKENS 5

/* Shared-expert term of the combine ([MF] combine_kernel_name and the
 * variant comment: sigmoid-gated for Qwen3 MoE, added unscaled for
 * DeepSeek-V3-style models, or absent). */
enum { MOE_SHARED_NONE = 0, MOE_SHARED_SIGMOID = 1, MOE_SHARED_UNSCALED = 2 };

#define Q4K_BLOCK_WEIGHTS 256 /* [FK] test: QK_K                          */
#define Q4K_BLOCK_BYTES 144   /* [FK] test: BLOCK_BYTES                    */
#define Q4K_MAX_TOP_K 16      /* [MF] MAX_K                                */
#define Q4K_MAX_IN 16384      /* largest in-features (k) of one GEMV       */
#define Q4K_MAX_EXPERTS 1023  /* bucketing keeps E+1 buckets in one block  */
#define Q4K_MAX_PAIRS 8192    /* m*top_k handled by one bucketing launch   */
#define Q4TP_MAX_COLS 16384   /* largest Q4TiledP row                       */
#define Q4TP_MAX_TENSORS 3    /* [CE] merged kernel: tensors per dispatch  */
#define Q4K_BUCKET_CHUNK 8    /* pairs per bucketed work item               */

const char *q4k_status_string(int status);
/* 4: weight stacks in the tile layout (q4k_pack_tiles); bucket_flag takes
 * schedule bits (Q4K_SCHED_*); AUTO buckets from
 * Q4K_AUTO_BUCKET_MIN_TOKENS tokens; the layer workspace has no
 * synchronisation header (moe_layer_workspace_init is gone); activation rows
 * of every entry point need only 4-byte alignment.  3 added the MLX 4-bit and
 * 2-bit entry points and the chained RMSNorm. */
int q4k_abi_version(void);

/* Bytes of an n x k Q4_K matrix: n*(k/256)*144 ([FK]
 * dispatch_gemv_q4k_moe_id_batched_on_encoder, nb01 and nb02).  -1 when k is
 * not a positive multiple of 256 or n < 0. */
int64_t q4k_matrix_bytes(int64_t n, int64_t k);

/* Q4_K superblock layout (reading of [FK]: 256 weights in 144 bytes, GGML's
 * Q4_K by way of candle):
 *   bytes 0-1 d (fp16), 2-3 dmin (fp16), 4-15 eight 6-bit scales and eight
 *   6-bit mins packed in 12 bytes, 16-143 nibbles: byte 32c+l holds weight
 *   64c+l (low nibble) and 64c+32+l (high nibble);
 *   w_i = d*scale_j*q_i - dmin*min_j with j = i/32.
 *
 * q4k_dequantize: `blocks` (n_blocks*144 bytes) -> `out` (n_blocks*256 fp32).
 * The fp32 result is exact (every product fits in 24 bits), so it is
 * bit-identical to any correct evaluation.  n_blocks >= 0. */
int q4k_dequantize(const void *blocks, float *out, int64_t n_blocks, void *stream);

/* q4k_quantize: `w` fp32 [n_rows, k] -> `blocks` [n_rows, k/256] superblocks,
 * k % 256 == 0.  The pages quantize with candle and print no encoder; this is
 * a plain min/max affine encoder whose steps are single IEEE float operations
 * (per sub-block lo = min(0, min w), hi = max w, a = (hi-lo)/15, b = -lo;
 * d = fp16(max a / 63), dmin = fp16(max b / 63); scale = rne(a/d),
 * min = rne(b/dmin), q = rne((w + dmin*min)/(d*scale)), all clamped). */
int q4k_quantize(const float *w, void *blocks, int64_t n_rows, int64_t k, void *stream);

/* ---------------------------------------------------------------------- */
/* Tile layout of the expert stacks.  Every GEMV, FFN and layer entry point  */
/* reads its Q4_K weight stacks in this order, which q4k_pack_tiles writes   */
/* once, at load time, from GGUF row order (the superblocks above, row after */
/* row).  It holds the same 144-byte superblocks, regrouped so that the      */
/* lanes of a GPU wave read contiguous bytes per load instruction:           */
/*   rows go in groups of 8 (the last group padded with zero blocks); for    */
/*   row group G and superblock s (nb = k/256 per row), tile (G, s) of 1152  */
/*   bytes sits at (G*nb + s)*1152 and holds                                 */
/*     bytes    0..127   the 8 rows' 16-byte headers (d, dmin, scales), row  */
/*                       r at 16*r;                                          */
/*     bytes  128..639   for chunk c = 0..3 and row r: nibble bytes          */
/*                       32c .. 32c+15 of the row at 128 + 16*(8c + r);      */
/*     bytes  640..1151  nibble bytes 32c+16 .. 32c+31 at 640 + 16*(8c + r). */
/* An n x k matrix takes q4k_tiles_bytes(n, k) = ceil(n/8)*8*(k/256)*144    */
/* bytes, the GGUF size when n is a multiple of 8; expert e of a stack       */
/* starts at e*q4k_tiles_bytes(n, k).                                         */
/* ---------------------------------------------------------------------- */
int64_t q4k_tiles_bytes(int64_t n, int64_t k);   /* -1 on a bad shape */

/* n_mats matrices of n x k: GGUF row order (n_mats * n*(k/256)*144 bytes at
 * `blocks`) -> tile layout (n_mats * q4k_tiles_bytes(n, k) bytes at `tiles`);
 * a pure permutation of the bytes (zero blocks fill a last partial row
 * group).  q4k_unpack_tiles is its inverse.  n >= 1, k a positive multiple
 * of 256, n_mats >= 0; both pointers 16-byte aligned and distinct.  Errors:
 * Q4K_ERR_SHAPE, Q4K_ERR_NULL. */
int q4k_pack_tiles(const void *blocks, void *tiles, int64_t n_mats, int64_t n, int64_t k,
                   void *stream);
int q4k_unpack_tiles(const void *tiles, void *blocks, int64_t n_mats, int64_t n, int64_t k,
                     void *stream);

/* Scratch bytes that the bucketed modes need for `n_pairs` (token, slot)
 * pairs over `num_experts` experts. */
int64_t moe_bucket_workspace_bytes(int64_t n_pairs, int64_t num_experts);

/* Expert bucketing ([MF] encode_moe_gather_id_fuse step 1, map0; and
 * ExpertBuckets, CSR by expert).  Writes into `ws` (int32 words):
 *   counts[E+1] | offsets[E+2] | pairs[P] | active[E+1] | n_active[1] |
 *   n_chunks[1] | chunks[2*P]
 * where bucket E collects ids outside [0, E), offsets is the exclusive prefix
 * sum of counts, pairs lists pair indices grouped by bucket in ascending order
 * inside a bucket, active lists the non-empty buckets ascending, and chunks
 * lists the work items of at most Q4K_BUCKET_CHUNK pairs each, buckets
 * ascending (n_chunks of them), as (bucket, first | count << 24) where first
 * indexes pairs and count is the item's number of pairs.
 * The layout above is what the bucketed GEMV reads; callers need not read it. */
int moe_bucket(const int32_t *ids, int64_t n_pairs, int64_t num_experts, void *ws,
               int64_t ws_bytes, void *stream);

/* Batched indirect-dispatch Q4_K GEMV ([FK]
 * dispatch_gemv_q4k_moe_id_batched_on_encoder and module doc).
 *   w_stacked : [num_experts] n x k Q4_K matrices in the tile layout
 *               (q4k_pack_tiles), 16-byte aligned; expert e starts at byte
 *               e*q4k_tiles_bytes(n, k).  The caller pre-offsets the pointer
 *               if the stack starts inside a larger buffer ([FK]
 *               weights_byte_offset).
 *   src1      : activations, 4-byte aligned (any float offset and stride;
 *               16-byte aligned rows load faster); pair p = token*top_k + slot
 *               reads the k floats at
 *               src1 + token*src1_outer_stride + slot*src1_inner_stride.
 *               gate/up: outer = k, inner = 0; down: outer = top_k*k, inner = k.
 *   ids       : [m*top_k] int32 expert ids.  An id outside [0, num_experts)
 *               gives a zero output row (the pages leave it undefined).
 *   dst       : [m*top_k, n] fp32.
 *   Requires k % 256 == 0, 256 <= k <= Q4K_MAX_IN, n >= 1, m >= 1,
 *   1 <= top_k <= Q4K_MAX_TOP_K, 1 <= num_experts <= Q4K_MAX_EXPERTS,
 *   m*top_k <= 65535 (Q4K_MAX_PAIRS when bucketed), strides >= 0.  ([FK]
 *   asserts k%256 and n%4; n%4 is not needed here.)
 *   bucket_flag: mode and schedule bits (see Q4K_BUCKET_*); a bucketed call
 *   needs ws_bytes >= moe_bucket_workspace_bytes(m*top_k, num_experts),
 *   otherwise ws may be NULL.  Bits: see the numerics note at Q4K_BUCKET_*. */
int q4k_moe_id_gemv(const void *w_stacked, const float *src1, const int32_t *ids, float *dst,
                    int64_t n, int64_t k, int64_t m, int64_t top_k,
                    int64_t src1_outer_stride, int64_t src1_inner_stride,
                    int64_t num_experts, int bucket_flag, void *ws, int64_t ws_bytes,
                    void *stream);

/* Fused gate + up id-GEMV with SiLU ([FK] test module:
 * dispatch_gemv_q4k_moe_id_gate_up_silu_batched_on_encoder, which writes
 * [m*top_k, n] rows of silu(gate.x) * (up.x); [MF] swiglu_fused).
 *   w_gate, w_up : two stacks of the same shape ([num_experts] n x k
 *                  matrices, tile layout)
 *   out          : [m*top_k, n] fp32, out[p,r] = silu(g)*u with
 *                  g = W_gate[ids[p]][r].x, u = W_up[ids[p]][r].x, x the
 *                  pair's activation row (strides as in q4k_moe_id_gemv).
 *   sh_gate, sh_up, sh_out : optional shared expert ([MF] ExpertPayload
 *                  shared_out) run in the same launch: one-expert stacks of
 *                  the same shape and sh_out [m, n] = silu(G.x_t)*(U.x_t)
 *                  with x_t = src1 + t*src1_outer_stride.  All NULL: none.
 *   Same requirements and bucketing as q4k_moe_id_gemv (bucketed, the shared
 *   expert is one more bucket holding every token). */
int q4k_moe_gate_up_silu(const void *w_gate, const void *w_up, const float *src1,
                         const int32_t *ids, float *out, int64_t n, int64_t k, int64_t m,
                         int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                         int64_t num_experts, const void *sh_gate, const void *sh_up,
                         float *sh_out, int bucket_flag, void *ws, int64_t ws_bytes,
                         void *stream);

/* Expert FFN for all (token, slot) pairs ([MF] module doc: gate and up
 * matvecs, SwiGLU, down matvec; encode_moe_gather_id_fuse for the strides).
 *   w_gate, w_up : [num_experts] inter x hidden matrices, tile layout
 *   w_down       : [num_experts] hidden x inter matrices, tile layout
 *   h_post       : [m, hidden] fp32 (one row per token, shared by its slots)
 *   ids          : [m*top_k] int32
 *   act          : [m*top_k, inter] fp32 out: silu(gate.x) * (up.x)
 *   expert_out   : [m*top_k, hidden] fp32 out: down applied to act
 *   hidden and inter: multiples of 256, at most Q4K_MAX_IN.
 *   The shared expert is this call on a one-expert stack with ids = 0 and
 *   top_k = 1.  Workspace as for q4k_moe_id_gemv. */
int moe_expert_ffn(const void *w_gate, const void *w_up, const void *w_down,
                   const float *h_post, const int32_t *ids, float *act, float *expert_out,
                   int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                   int64_t top_k, int bucket_flag, void *ws, int64_t ws_bytes, void *stream);

/* Whole MoE layer for a decode batch: routed experts, optional shared expert
 * and the weighted residual combine ([MF] gpu_batched_experts_forward and
 * emit_batched_experts: gate/up, SwiGLU, down for every selected expert and
 * the shared one, then moe_combine_residual), in the fewest launches:
 *   token mode (OFF, or AUTO below Q4K_AUTO_BUCKET_MIN_TOKENS tokens): fused
 *                gate/up+SiLU over routed and shared pairs, then the down
 *                projection fused with the combine (2 launches; when the
 *                token's top_k+1 activation rows of `inter` floats take more
 *                than 48 KB of a workgroup's LDS, down and the combine are 2
 *                launches -- the same bits either way);
 *   bucketed (ON, PREBUILT, or AUTO from Q4K_AUTO_BUCKET_MIN_TOKENS tokens):
 *                bucketed gate/up+SiLU and down (the shared expert as one more
 *                bucket holding every token), then the combine.  On the
 *                matrix cores with m*top_k <= 1024 and num_experts <= 1023
 *                the expert buckets are built inside the gate/up and down
 *                launches (each workgroup from the ids, in LDS); otherwise,
 *                or with Q4K_SCHED_BUCKET_LAUNCH, one bucketing launch writes
 *                them to the workspace.  The chunks, and so the bits, are
 *                the same either way.
 *   w_gate, w_up, w_down : routed stacks as in moe_expert_ffn
 *   sh_gate, sh_up, sh_down : one-expert stacks of the same row shapes, or
 *                all NULL with shared_mode == MOE_SHARED_NONE
 *   h_post [m,hidden], h_mid [m,hidden], ids [m*top_k], route_w [m*top_k],
 *   shared_gate_logit [m] (MOE_SHARED_SIGMOID only), out [m,hidden] fp32,
 *   all 4-byte aligned; weight stacks 16-byte aligned.
 *   ws: scratch of at least moe_layer_workspace_bytes(...) bytes, 16-byte
 *   aligned, no initial contents required; calls that may overlap in time must
 *   not share a workspace.  m*top_k <= Q4K_MAX_PAIRS.
 *   bucket_flag: as for q4k_moe_id_gemv.  The bits of `out` depend only on
 *   the arguments; token mode and vector-unit bucketing agree bit for bit, the
 *   matrix-core schedule within the band. */
int64_t moe_layer_workspace_bytes(int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                                  int64_t top_k);
int moe_layer_forward(const void *w_gate, const void *w_up, const void *w_down,
                      const void *sh_gate, const void *sh_up, const void *sh_down,
                      const float *h_post, const float *h_mid, const int32_t *ids,
                      const float *route_w, const float *shared_gate_logit, float *out,
                      int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                      int64_t top_k, int shared_mode, int bucket_flag, void *ws,
                      int64_t ws_bytes, void *stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The call allocates nothing: its scratch
 * (what moe_layer_workspace_bytes reports) is a static device array of
 * MOE_LAYER_NOALLOC_MAX_BYTES bytes that every GPU the library runs on holds
 * from the library's first use on it until the process ends.  Each device's
 * array is looked up once (on the first call with that device current); the
 * stream must belong to the current device.  Every call on one GPU uses the
 * same array, so calls on one GPU that may overlap in time (other streams,
 * other host threads) race and must be serialised by the caller; the array
 * keeps the last call's contents, and no call needs it cleared.  Arguments,
 * schedules and output bits are those of moe_layer_forward with the same
 * arguments.  Errors as moe_layer_forward, plus Q4K_ERR_SCRATCH when
 * moe_layer_workspace_bytes(hidden, inter, num_experts, m, top_k) exceeds
 * MOE_LAYER_NOALLOC_MAX_BYTES (e.g. hidden 7168, inter 2048, top_k 8 fits up
 * to m = 48) and Q4K_ERR_LAUNCH when the array's address cannot be found. */
#define MOE_LAYER_NOALLOC_MAX_BYTES (16 << 20)
int moe_layer_forward_noalloc(const void *w_gate, const void *w_up, const void *w_down,
                              const void *sh_gate, const void *sh_up, const void *sh_down,
                              const float *h_post, const float *h_mid, const int32_t *ids,
                              const float *route_w, const float *shared_gate_logit, float *out,
                              int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                              int64_t top_k, int shared_mode, int bucket_flag, void *stream);

/* The same layer with the next layer's input RMSNorm chained on ([MF]
 * ChainToNormed: after the combine, rms_norm_sum_sq and rms_norm_apply_bf16
 * with the next layer's input-norm weight and eps):
 *   out    as moe_layer_forward (bit for bit: the same launches),
 *   normed[t, i] = out[t, i] / sqrt(sum_j out[t, j]^2 / hidden + eps) * w[i],
 * norm_weight: [hidden] bf16, 2-byte aligned; normed: [m, hidden] fp32, not
 * `out`.  The few-token path adds one launch (a workgroup per token) after
 * down + combine; the bucketed path computes the combine and the norm in one
 * launch.  Errors as moe_layer_forward, plus Q4K_ERR_NULL (norm_weight or
 * normed missing or misaligned, normed == out) and Q4K_ERR_ARG (eps negative,
 * infinite or NaN). */
int moe_layer_forward_rmsnorm(const void *w_gate, const void *w_up, const void *w_down,
                              const void *sh_gate, const void *sh_up, const void *sh_down,
                              const float *h_post, const float *h_mid, const int32_t *ids,
                              const float *route_w, const float *shared_gate_logit, float *out,
                              const void *norm_weight, float eps, float *normed, int64_t hidden,
                              int64_t inter, int64_t num_experts, int64_t m, int64_t top_k,
                              int shared_mode, int bucket_flag, void *ws, int64_t ws_bytes,
                              void *stream);

/* Weighted combine with residual ([MF] module doc and
 * encode_moe_combine_residual_n_tokens):
 *   out[t,i] = h_mid[t,i] + sum_{s<top_k} route_w[t*top_k+s]*expert_out[t*top_k+s,i]
 *              + g_t*shared_out[t,i]
 * with g_t = sigmoid(shared_gate_logit[t]) (MOE_SHARED_SIGMOID), 1
 * (MOE_SHARED_UNSCALED) or no shared term (MOE_SHARED_NONE; shared_out and
 * shared_gate_logit may be NULL).  Slots are summed in order, so the result
 * does not depend on the batch.  `out` may alias `h_mid`. */
int moe_combine_residual(const float *h_mid, const float *expert_out, const float *route_w,
                         const float *shared_out, const float *shared_gate_logit, float *out,
                         int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                         void *stream);

/* moe_combine_residual followed by the chained RMSNorm of its rows, in one
 * launch of a workgroup per token: `out` is moe_combine_residual's result
 * bit for bit, normed[t, i] = out[t, i] / sqrt(sum_j out[t, j]^2 / hidden + eps)
 * * w[i] with norm_weight [hidden] bf16 (2-byte aligned).  normed must not be
 * `out` (out may alias h_mid).  1 <= m <= 65535.  Errors as
 * moe_combine_residual plus Q4K_ERR_NULL (norm_weight, normed) and
 * Q4K_ERR_ARG (eps negative, infinite or NaN). */
int moe_combine_residual_rmsnorm(const float *h_mid, const float *expert_out,
                                 const float *route_w, const float *shared_out,
                                 const float *shared_gate_logit, const void *norm_weight, float eps,
                                 float *out, float *normed, int64_t hidden, int64_t m,
                                 int64_t top_k, int shared_mode, void *stream);

/* Q4TiledP dense tensor ([CE] kernel `cur`): rows x cols, cols % 32 == 0,
 * gpr = cols/32 groups of 32 signed nibbles (value = nibble - 8, byte i of a
 * group holds elements 2i and 2i+1), 16 bytes per group at (r*gpr+g)*16; then
 * per row an fp16 pair (base, step); then per row ceil(5*gpr/8) bytes of 5-bit
 * group codes, least significant bit first.  Group scale = 2^(base+code*step).
 * q4tp_tensor_bytes returns the byte size, -1 on bad shape. */
int64_t q4tp_tensor_bytes(int64_t rows, int64_t cols);

/* y[r] = sum_g scale(r,g) * sum_j (nibble-8) * x[32g+j]  ([CE] kernel `cur`).
 * x: [cols] fp32, y: [rows] fp32.  1 <= cols <= Q4TP_MAX_COLS. */
int q4tp_matvec(const void *tensor, const float *x, float *y, int64_t rows, int64_t cols,
                void *stream);

/* The merged dispatch ([CE] main, walk mode `m`: q|k|v and gate|up each in
 * one dispatch; merged kernel `hlfm` over up to three tensors of the same
 * width): n_tensors (1..Q4TP_MAX_TENSORS) Q4TiledP tensors of the same cols
 * against the same x.  tensors[i] (device pointer, 16-byte aligned) has
 * rows[i] rows; tensors and rows are HOST arrays of n_tensors entries, read
 * during the call.  y receives the outputs one tensor after another: rows[0]
 * values of tensor 0, then tensor 1, ...  Each output equals that of a
 * separate q4tp_matvec call bit for bit.  Errors: Q4K_ERR_SHAPE (n_tensors,
 * any rows[i] < 1, the rows summing past 2^30, or cols as in q4tp_matvec),
 * Q4K_ERR_NULL (a null or misaligned pointer). */
int q4tp_matvec_multi(const void *const *tensors, const int64_t *rows, int n_tensors,
                      const float *x, float *y, int64_t cols, void *stream);

/* q4tp_quantize: fp32 [rows, cols] -> Q4TiledP.  The page prints no encoder;
 * reading: t_g = max|w|/7, lt_g = log2(t_g); base = fp16(min lt),
 * step = fp16((max lt - base)/31); code = rne((lt-base)/step);
 * nibble = clamp(rne(w/scale), -8, 7) + 8. */
int q4tp_quantize(const float *w, void *tensor, int64_t rows, int64_t cols, void *stream);

/* ---------------------------------------------------------------------- */
/* MLX affine 4-bit expert codec ([MF] module doc "4-bit only";             */
/* gpu_expert_forward / encode_matvec: GROUP_SIZE; encode_moe_gather_id_fuse */
/* and its gather call: expert blocks of expert_stride bytes (nb02) holding  */
/* packed weights (nb01_w = k/2 bytes per row), bf16 scales and bf16 biases  */
/* (nb01_s = (k/64)*2 bytes per row) at packed/scales/biases offsets).      */
/*                                                                          */
/* Bit layout (reading: the pages give the strides; this is MLX's affine    */
/* format): groups of MLX4_GROUP weights along a row; weight                 */
/* w = scale*q + bias with q the 4-bit code; byte j of a row holds weight   */
/* 2j in its low nibble and 2j+1 in its high nibble.                         */
/* ---------------------------------------------------------------------- */
#define MLX4_GROUP 64

/* Bytes of one n x k matrix: packed n*k/2 + scales and biases 2*(n*k/64)*2.
 * -1 when k is not a positive multiple of 64 or n < 0. */
int64_t mlx4_matrix_bytes(int64_t n, int64_t k);

/* packed [n, k/2] bytes, scales and biases [n, k/64] bf16 -> out fp32 [n, k].
 * w = scale*q + bias in fp32: scale*q is exact (8 + 4 significant bits) and
 * the sum rounds once, so the result is bit-identical to any correct
 * evaluation.  64 <= k <= Q4K_MAX_IN, k % 64 == 0; packed and out 16-byte
 * aligned, scales and biases 2-byte aligned.  Errors: Q4K_ERR_SHAPE,
 * Q4K_ERR_NULL. */
int mlx4_dequantize(const void *packed, const void *scales, const void *biases, float *out,
                    int64_t n, int64_t k, void *stream);

/* fp32 w [n, k] -> packed, scales, biases (layout above).  The pages print
 * no encoder; reading, a plain min/max affine code per group whose steps are
 * single IEEE float operations: lo = min w, hi = max w,
 * scale = bf16_rne((hi - lo)/15), bias = bf16_rne(lo),
 * q = clamp(rne((w - bias)/scale), 0, 15), q = 0 where scale is 0.
 * Same shape and alignment rules as mlx4_dequantize (w 4-byte aligned). */
int mlx4_quantize(const float *w, void *packed, void *scales, void *biases, int64_t n, int64_t k,
                  void *stream);

/* id-GEMV over MLX 4-bit experts ([MF] encode_moe_gather_id_fuse, one row of
 * src1 per (token, slot) pair as in [FK]'s 2-D walk):
 *   for p in [0, m*top_k): t = p / top_k, s = p % top_k, e = ids[p],
 *     x = src1 + t*src1_outer_stride + s*src1_inner_stride   (floats),
 *     blk = expert_base + e*expert_stride,
 *     dst[p, r] = sum_c (scale*q + bias)[r, c] * x[c]
 *   with the packed weights at blk + packed_off, scales at blk + scales_off,
 *   biases at blk + biases_off.  ids outside [0, num_experts) give zero rows.
 * dst: [m*top_k, n] fp32.  Shapes: n >= 1, 64 <= k <= Q4K_MAX_IN, k % 64 == 0,
 * m >= 1, 1 <= top_k <= Q4K_MAX_TOP_K, num_experts >= 1, m*top_k <= 65535,
 * each sub-tensor inside the block (offset + its bytes <= expert_stride),
 * else Q4K_ERR_SHAPE.  Negative activation strides: Q4K_ERR_STRIDE.
 * Alignment: expert_base, expert_stride and packed_off 16 bytes, scales_off and
 * biases_off 2 bytes, src1, ids and dst 4 bytes, else Q4K_ERR_NULL. */
int mlx4_moe_id_gemv(const void *expert_base, int64_t expert_stride, int64_t packed_off,
                     int64_t scales_off, int64_t biases_off, const float *src1,
                     const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                     int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                     int64_t num_experts, void *stream);

/* Fused gate/up + SiLU over MLX 4-bit experts ([MF] module doc: gate and up
 * matvecs then SwiGLU, and encode_moe_gather_id_fuse's gate and up gathers
 * over the same expert block): the gate matrix at the gate_* offsets and the
 * up matrix at the up_* offsets of each expert's block, both [n, k], against
 * the same activation row;
 *   dst[p, r] = silu(gate[p, r]) * up[p, r],  silu(z) = z / (1 + e^-z).
 * Arguments, walk, limits and errors as mlx4_moe_id_gemv, for both sets of
 * offsets. */
int mlx4_moe_gate_up_silu(const void *expert_base, int64_t expert_stride, int64_t gate_packed_off,
                          int64_t gate_scales_off, int64_t gate_biases_off, int64_t up_packed_off,
                          int64_t up_scales_off, int64_t up_biases_off, const float *src1,
                          const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                          int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                          int64_t num_experts, void *stream);

/* MLX affine 2-bit expert codec ([MF] module doc: g_use_2bit selects the
 * 2-bit matvec and expert layout).  Reading: MLX's 2-bit affine format, the
 * 4-bit layout above with 2-bit codes: groups of 64 weights, bf16 scale and
 * bias per group, w = scale*q + bias with q in 0..3, byte j of a row holding
 * weights 4j..4j+3 at bits 0-1, 2-3, 4-5 and 6-7; packed rows take k/4
 * bytes.  The encoder is the 4-bit one with scale = bf16_rne((hi - lo)/3)
 * and q clamped to 0..3.  Arguments, limits, alignment and errors as the
 * mlx4_* entry points (mlx2_matrix_bytes: n*k/4 + 2*(n*k/64)*2). */
int64_t mlx2_matrix_bytes(int64_t n, int64_t k);
int mlx2_dequantize(const void *packed, const void *scales, const void *biases, float *out,
                    int64_t n, int64_t k, void *stream);
int mlx2_quantize(const float *w, void *packed, void *scales, void *biases, int64_t n, int64_t k,
                  void *stream);
int mlx2_moe_id_gemv(const void *expert_base, int64_t expert_stride, int64_t packed_off,
                     int64_t scales_off, int64_t biases_off, const float *src1,
                     const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                     int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                     int64_t num_experts, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4KMOE_H */
