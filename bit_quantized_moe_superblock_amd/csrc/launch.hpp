// Internal launch interface between the C ABI (api.hip) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

struct GemvLaunch {
    const void *w0;            // stacked experts; the gate stack when fused_swiglu
    const void *w1;            // up stack (fused_swiglu only)
    const void *s0, *s1;       // shared expert (one-expert stacks) or null
    const float *src1;
    const float *src1_sh;      // shared activations, token t at src1_sh + t*outer_sh
    const int32_t *ids;
    const int32_t *bucket_ws;  // non-null selects the bucketed mode
    float *dst;
    float *dst_sh;             // [m_sh, n] shared-expert rows
    int64_t n, k, top_k, num_experts, n_pairs, m_sh;
    int64_t outer, inner, outer_sh;
    bool fused_swiglu;
    bool self_bucket;          // bucketed mode with the chunks built in-kernel from ids
    bool vector_units;         // bucketed mode on the vector units, not the matrix cores
};

// Largest pair count and bucket count (num_experts + 1) of self-bucketing.
constexpr int64_t kSelfBucketMaxPairs = 1024;
constexpr int64_t kSelfBucketMaxBuckets = 1024;

hipError_t launch_q4k_gemv(const GemvLaunch &L, hipStream_t st);
// Whether L may run bucketed with self_bucket set (the size limits above).
bool q4k_self_bucket_ok(const GemvLaunch &L);
// Whether the down projection fused with the combine fits one workgroup's
// LDS: the token's top_k (+ shared) activation rows of k floats are staged.
bool q4k_down_combine_ok(int64_t k, int64_t top_k, bool shared);
// Down projection fused with the weighted residual combine, one workgroup row
// of tiles per token (few tokens).  expert_out may be null.
hipError_t launch_q4k_down_combine(const GemvLaunch &L, const float *h_mid, const float *route_w,
                                   const float *shared_logit, float *out, float *expert_out,
                                   int shared_mode, hipStream_t st);
hipError_t launch_q4k_dequant(const void *blocks, float *out, int64_t n_blocks, hipStream_t st);
// n_mats matrices of n x k between GGUF row order and the tile layout
// (common.hpp); unpack reverses it.
hipError_t launch_q4k_pack_tiles(const void *src, void *dst, int64_t n_mats, int64_t n,
                                 int64_t k, bool unpack, hipStream_t st);
hipError_t launch_q4k_quant(const float *w, void *blocks, int64_t n_blocks, hipStream_t st);
hipError_t launch_moe_bucket(const int32_t *ids, int64_t n_pairs, int64_t num_experts,
                             int32_t *ws, hipStream_t st);
hipError_t launch_moe_combine(const float *h_mid, const float *expert_out, const float *route_w,
                              const float *shared_out, const float *shared_gate_logit, float *out,
                              int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                              hipStream_t st);
// RMSNorm of the rows of `out` into `normed` with a bf16 weight; with
// `combine` the rows are first computed by the combine and written to `out`.
hipError_t launch_combine_norm(const float *h_mid, const float *expert_out, const float *route_w,
                               const float *shared_out, const float *shared_gate_logit,
                               const void *norm_weight, float eps, float *out, float *normed,
                               int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                               bool combine, hipStream_t st);
hipError_t launch_q4tp_matvec_multi(const void *const *ts, const int64_t *rows, int nseg,
                                    const float *x, float *y, int64_t cols, hipStream_t st);
hipError_t launch_q4tp_matvec(const void *t, const float *x, float *y, int64_t rows,
                              int64_t cols, hipStream_t st);
hipError_t launch_q4tp_quant(const float *w, void *t, int64_t rows, int64_t cols,
                             hipStream_t st);

// MLX affine 4-bit id-GEMV (mlx4.hip): expert e's block at base + e*expert_stride,
// its packed weights, scales and biases at the offsets inside the block (a
// second set, the up matrix, for the fused gate/up + SiLU launch).
struct Mlx4Launch {
    const void *base;
    int64_t expert_stride, packed_off, scales_off, biases_off;
    int64_t packed_off1, scales_off1, biases_off1;   // up matrix (fused_swiglu)
    bool fused_swiglu;
    int bits;                                        // 4 (default when 0) or 2
    const float *src1;
    const int32_t *ids;
    float *dst;
    int64_t n, k, m, top_k, num_experts, outer, inner;
};
hipError_t launch_mlx4_gemv(const Mlx4Launch &L, hipStream_t st);
hipError_t launch_mlx4_dequant(const void *packed, const void *scales, const void *biases,
                               float *out, int64_t groups, int bits, hipStream_t st);
hipError_t launch_mlx4_quant(const float *w, void *packed, void *scales, void *biases,
                             int64_t groups, int bits, hipStream_t st);

// Workspace of the bucketing kernel in int32 words (layout in q4kmoe.h).
inline int64_t bucket_ws_words(int64_t n_pairs, int64_t num_experts) {
    return (num_experts + 1) + (num_experts + 2) + n_pairs + (num_experts + 1) + 1 + 1 +
           2 * n_pairs;
}

}  // namespace q4k
