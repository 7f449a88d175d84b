// C ABI of the library (declared and documented in include/q4kmoe.h).
// Validation happens here, on the host, before any HIP call; the kernels
// assume validated arguments.
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "q4kmoe.h"
#include "common.hpp"
#include "launch.hpp"

using namespace q4k;

namespace {

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned2(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH; }

bool k_ok(int64_t k) { return k >= 256 && k % 256 == 0 && k <= Q4K_MAX_IN; }

int check_gemv_shape(int64_t n, int64_t k, int64_t m, int64_t top_k, int64_t E) {
    if (!k_ok(k) || n < 1 || n > (1 << 30) || m < 1 || top_k < 1 || top_k > Q4K_MAX_TOP_K ||
        E < 1 || E > Q4K_MAX_EXPERTS)
        return Q4K_ERR_SHAPE;
    if (m * top_k > 65535)   // one workgroup row per pair in the grid
        return Q4K_ERR_SHAPE;
    return Q4K_OK;
}

// Splits a bucket_flag into its mode and schedule bits; Q4K_ERR_ARG for an
// unknown mode or bit.
int parse_flag(int flag, int *mode, bool *vector_units, bool *bucket_launch) {
    *mode = flag & Q4K_BUCKET_MODE_MASK;
    const int extra = flag & ~Q4K_BUCKET_MODE_MASK;
    if (*mode != Q4K_BUCKET_AUTO && *mode != Q4K_BUCKET_OFF && *mode != Q4K_BUCKET_ON &&
        *mode != Q4K_BUCKET_PREBUILT)
        return Q4K_ERR_ARG;
    if (extra & ~(Q4K_SCHED_VECTOR | Q4K_SCHED_BUCKET_LAUNCH))
        return Q4K_ERR_ARG;
    *vector_units = (extra & Q4K_SCHED_VECTOR) != 0;
    *bucket_launch = (extra & Q4K_SCHED_BUCKET_LAUNCH) != 0;
    return Q4K_OK;
}

bool bucketed_for(int mode, int64_t m) {
    return mode == Q4K_BUCKET_ON || mode == Q4K_BUCKET_PREBUILT ||
           (mode == Q4K_BUCKET_AUTO && m >= Q4K_AUTO_BUCKET_MIN_TOKENS);
}

// Bucketed mode decision and workspace check of the id-GEMV entry points;
// *use and *vec set on success.
int bucket_mode(int flag, int64_t m, int64_t P, int64_t E, void *ws, int64_t ws_bytes,
                bool *use, bool *vec, int *mode) {
    bool launch_bit = false;
    int rc = parse_flag(flag, mode, vec, &launch_bit);
    if (rc)
        return rc;
    *use = bucketed_for(*mode, m);
    if (!*use)
        return Q4K_OK;
    if (P > Q4K_MAX_PAIRS)
        return Q4K_ERR_SHAPE;
    if (!ws || !aligned4(ws) || ws_bytes < moe_bucket_workspace_bytes(P, E))
        return Q4K_ERR_WORKSPACE;
    return Q4K_OK;
}

}  // namespace

extern "C" {

const char *q4k_status_string(int status) {
    switch (status) {
    case Q4K_OK: return "ok";
    case Q4K_ERR_SHAPE: return "size out of range or not a required multiple";
    case Q4K_ERR_NULL: return "required pointer is NULL or misaligned";
    case Q4K_ERR_STRIDE: return "activation stride is negative";
    case Q4K_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4K_ERR_LAUNCH: return "HIP launch failed";
    case Q4K_ERR_ARG: return "unknown enum argument";
    case Q4K_ERR_SCRATCH: return "scratch needed exceeds the library's static scratch";
    default: return "unknown status";
    }
}

int q4k_abi_version(void) { return 4; }

int64_t q4k_matrix_bytes(int64_t n, int64_t k) {
    if (n < 0 || k <= 0 || k % Q4K_BLOCK_WEIGHTS)
        return -1;
    return n * (k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
}

int q4k_dequantize(const void *blocks, float *out, int64_t n_blocks, void *stream) {
    if (n_blocks < 0)
        return Q4K_ERR_SHAPE;
    if (n_blocks == 0)
        return Q4K_OK;
    if (!blocks || !out || !aligned16(blocks) || !aligned16(out))
        return Q4K_ERR_NULL;
    return launched(launch_q4k_dequant(blocks, out, n_blocks, as_stream(stream)));
}

int q4k_quantize(const float *w, void *blocks, int64_t n_rows, int64_t k, void *stream) {
    if (n_rows < 0 || k <= 0 || k % Q4K_BLOCK_WEIGHTS)
        return Q4K_ERR_SHAPE;
    if (n_rows == 0)
        return Q4K_OK;
    if (!w || !blocks || !aligned16(blocks) || !aligned4(w))
        return Q4K_ERR_NULL;
    return launched(launch_q4k_quant(w, blocks, n_rows * (k / Q4K_BLOCK_WEIGHTS),
                                     as_stream(stream)));
}

int64_t q4k_tiles_bytes(int64_t n, int64_t k) {
    if (n < 0 || k <= 0 || k % Q4K_BLOCK_WEIGHTS)
        return -1;
    return tiles_matrix_bytes(n, k);
}

namespace {

int pack_entry(const void *src, void *dst, int64_t n_mats, int64_t n, int64_t k, bool unpack,
               void *stream) {
    if (n_mats < 0 || n < 1 || n > (1 << 30) || k <= 0 || k % Q4K_BLOCK_WEIGHTS ||
        k > (1 << 20))
        return Q4K_ERR_SHAPE;
    // one launch of a thread per block: the grid must fit 2^31 - 1 workgroups
    if (n_mats > ((int64_t)1 << 38) / (tile_rows(n) * (k / Q4K_BLOCK_WEIGHTS)))
        return Q4K_ERR_SHAPE;
    if (n_mats == 0)
        return Q4K_OK;
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || src == dst)
        return Q4K_ERR_NULL;
    return launched(launch_q4k_pack_tiles(src, dst, n_mats, n, k, unpack, as_stream(stream)));
}

}  // namespace

int q4k_pack_tiles(const void *blocks, void *tiles, int64_t n_mats, int64_t n, int64_t k,
                   void *stream) {
    return pack_entry(blocks, tiles, n_mats, n, k, false, stream);
}

int q4k_unpack_tiles(const void *tiles, void *blocks, int64_t n_mats, int64_t n, int64_t k,
                     void *stream) {
    return pack_entry(tiles, blocks, n_mats, n, k, true, stream);
}

int64_t moe_bucket_workspace_bytes(int64_t n_pairs, int64_t num_experts) {
    if (n_pairs < 0 || num_experts < 1)
        return -1;
    return bucket_ws_words(n_pairs, num_experts) * 4;
}

int moe_bucket(const int32_t *ids, int64_t n_pairs, int64_t num_experts, void *ws,
               int64_t ws_bytes, void *stream) {
    if (n_pairs < 1 || n_pairs > Q4K_MAX_PAIRS || num_experts < 1 ||
        num_experts > Q4K_MAX_EXPERTS)
        return Q4K_ERR_SHAPE;
    if (!ids || !aligned4(ids))
        return Q4K_ERR_NULL;
    if (!ws || !aligned4(ws) || ws_bytes < moe_bucket_workspace_bytes(n_pairs, num_experts))
        return Q4K_ERR_WORKSPACE;
    return launched(launch_moe_bucket(ids, n_pairs, num_experts, (int32_t *)ws,
                                      as_stream(stream)));
}

}  // extern "C"

namespace {

int id_gemv_entry(const void *w0, const void *w1, const float *src1, const int32_t *ids,
                  float *dst, int64_t n, int64_t k, int64_t m, int64_t top_k,
                  int64_t src1_outer_stride, int64_t src1_inner_stride, int64_t num_experts,
                  const void *s0, const void *s1, float *sh_out,
                  int bucket_flag, void *ws, int64_t ws_bytes, void *stream) {
    const void *w_stacked = w0;
    int rc = check_gemv_shape(n, k, m, top_k, num_experts);
    if (rc)
        return rc;
    if (!w_stacked || !src1 || !ids || !dst || !aligned16(w_stacked) || !aligned4(src1) ||
        !aligned4(ids) || !aligned4(dst))
        return Q4K_ERR_NULL;
    if (w1 && !aligned16(w1))
        return Q4K_ERR_NULL;
    const bool has_sh = s0 != nullptr;
    if (has_sh && (!sh_out || !aligned16(s0) || !aligned4(sh_out) || (w1 && !s1) ||
                   (s1 && !aligned16(s1))))
        return Q4K_ERR_NULL;
    if (src1_outer_stride < 0 || src1_inner_stride < 0)
        return Q4K_ERR_STRIDE;
    const int64_t P = m * top_k;
    bool use = false, vec_units = false;
    int mode = 0;
    rc = bucket_mode(bucket_flag, m, P, num_experts, ws, ws_bytes, &use, &vec_units, &mode);
    if (rc)
        return rc;
    hipStream_t st = as_stream(stream);
    if (use && mode != Q4K_BUCKET_PREBUILT) {
        rc = launched(launch_moe_bucket(ids, P, num_experts, (int32_t *)ws, st));
        if (rc)
            return rc;
    }
    GemvLaunch L{};
    L.vector_units = vec_units;
    L.w0 = w_stacked;
    L.w1 = w1;
    L.src1 = src1;
    L.ids = ids;
    L.bucket_ws = use ? (const int32_t *)ws : nullptr;
    L.dst = dst;
    L.n = n;
    L.k = k;
    L.top_k = top_k;
    L.num_experts = num_experts;
    L.n_pairs = P;
    L.outer = src1_outer_stride;
    L.inner = src1_inner_stride;
    L.s0 = s0;
    L.s1 = has_sh ? s1 : nullptr;
    L.src1_sh = src1;
    L.outer_sh = src1_outer_stride;
    L.dst_sh = sh_out;
    L.m_sh = has_sh ? m : 0;
    L.fused_swiglu = w1 != nullptr;
    return launched(launch_q4k_gemv(L, st));
}

}  // namespace

extern "C" {

int q4k_moe_id_gemv(const void *w_stacked, const float *src1, const int32_t *ids, float *dst,
                    int64_t n, int64_t k, int64_t m, int64_t top_k,
                    int64_t src1_outer_stride, int64_t src1_inner_stride,
                    int64_t num_experts, int bucket_flag, void *ws, int64_t ws_bytes,
                    void *stream) {
    return id_gemv_entry(w_stacked, nullptr, src1, ids, dst, n, k, m, top_k, src1_outer_stride,
                         src1_inner_stride, num_experts, nullptr, nullptr, nullptr, bucket_flag,
                         ws, ws_bytes, stream);
}

int q4k_moe_gate_up_silu(const void *w_gate, const void *w_up, const float *src1,
                         const int32_t *ids, float *out, int64_t n, int64_t k, int64_t m,
                         int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                         int64_t num_experts, const void *sh_gate, const void *sh_up,
                         float *sh_out, int bucket_flag, void *ws, int64_t ws_bytes,
                         void *stream) {
    if (!w_up)
        return Q4K_ERR_NULL;
    if ((sh_gate == nullptr) != (sh_up == nullptr))
        return Q4K_ERR_NULL;
    return id_gemv_entry(w_gate, w_up, src1, ids, out, n, k, m, top_k, src1_outer_stride,
                         src1_inner_stride, num_experts, sh_gate, sh_up, sh_out, bucket_flag, ws,
                         ws_bytes, stream);
}

int moe_expert_ffn(const void *w_gate, const void *w_up, const void *w_down,
                   const float *h_post, const int32_t *ids, float *act, float *expert_out,
                   int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                   int64_t top_k, int bucket_flag, void *ws, int64_t ws_bytes, void *stream) {
    int rc = check_gemv_shape(inter, hidden, m, top_k, num_experts);
    if (rc)
        return rc;
    rc = check_gemv_shape(hidden, inter, m, top_k, num_experts);
    if (rc)
        return rc;
    if (!w_gate || !w_up || !w_down || !h_post || !ids || !act || !expert_out ||
        !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned4(h_post) ||
        !aligned4(ids) || !aligned4(act) || !aligned4(expert_out))
        return Q4K_ERR_NULL;
    const int64_t P = m * top_k;
    bool use = false, vec_units = false;
    int mode = 0;
    rc = bucket_mode(bucket_flag, m, P, num_experts, ws, ws_bytes, &use, &vec_units, &mode);
    if (rc)
        return rc;
    hipStream_t st = as_stream(stream);
    if (use && mode != Q4K_BUCKET_PREBUILT) {
        rc = launched(launch_moe_bucket(ids, P, num_experts, (int32_t *)ws, st));
        if (rc)
            return rc;
    }
    GemvLaunch L{};
    L.vector_units = vec_units;
    L.w0 = w_gate;
    L.w1 = w_up;
    L.src1 = h_post;
    L.ids = ids;
    L.bucket_ws = use ? (const int32_t *)ws : nullptr;
    L.dst = act;
    L.n = inter;
    L.k = hidden;
    L.top_k = top_k;
    L.num_experts = num_experts;
    L.n_pairs = P;
    L.outer = hidden;
    L.inner = 0;
    L.fused_swiglu = true;
    rc = launched(launch_q4k_gemv(L, st));
    if (rc)
        return rc;
    GemvLaunch D = L;
    D.w0 = w_down;
    D.w1 = nullptr;
    D.src1 = act;
    D.dst = expert_out;
    D.n = hidden;
    D.k = inter;
    D.outer = top_k * inter;
    D.inner = inter;
    D.fused_swiglu = false;
    return launched(launch_q4k_gemv(D, st));
}

int64_t moe_layer_workspace_bytes(int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                                  int64_t top_k) {
    if (hidden < 1 || inter < 1 || num_experts < 1 || m < 1 || top_k < 1)
        return -1;
    const int64_t P = m * top_k;
    auto up256 = [](int64_t b) { return (b + 255) / 256 * 256; };
    // act [P+m, inter] | expert_out [P, hidden] | shared_out [m, hidden] | buckets
    return up256((P + m) * inter * 4) + up256(P * hidden * 4) + up256(m * hidden * 4) +
           up256(moe_bucket_workspace_bytes(P, num_experts));
}

}  // extern "C"

namespace {

int layer_forward_impl(const void *w_gate, const void *w_up, const void *w_down,
                       const void *sh_gate, const void *sh_up, const void *sh_down,
                       const float *h_post, const float *h_mid, const int32_t *ids,
                       const float *route_w, const float *shared_gate_logit, float *out,
                       int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                       int64_t top_k, int shared_mode, int bucket_flag, void *ws,
                       int64_t ws_bytes, void *stream, const void *norm_weight, float eps,
                       float *normed) {
    int rc = check_gemv_shape(inter, hidden, m, top_k, num_experts);
    if (rc)
        return rc;
    rc = check_gemv_shape(hidden, inter, m, top_k, num_experts);
    if (rc)
        return rc;
    if (shared_mode != MOE_SHARED_NONE && shared_mode != MOE_SHARED_SIGMOID &&
        shared_mode != MOE_SHARED_UNSCALED)
        return Q4K_ERR_ARG;
    int mode = 0;
    bool vec_units = false, bucket_launch = false;
    rc = parse_flag(bucket_flag, &mode, &vec_units, &bucket_launch);
    if (rc)
        return rc;
    if (!w_gate || !w_up || !w_down || !h_post || !h_mid || !ids || !route_w || !out ||
        !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned4(h_post) ||
        !aligned4(h_mid) || !aligned4(ids) || !aligned4(route_w) || !aligned4(out))
        return Q4K_ERR_NULL;
    const bool has_sh = shared_mode != MOE_SHARED_NONE;
    if (has_sh && (!sh_gate || !sh_up || !sh_down || !aligned16(sh_gate) ||
                   !aligned16(sh_up) || !aligned16(sh_down)))
        return Q4K_ERR_NULL;
    if (shared_mode == MOE_SHARED_SIGMOID && !shared_gate_logit)
        return Q4K_ERR_NULL;
    const int64_t P = m * top_k;
    if (P > Q4K_MAX_PAIRS)
        return Q4K_ERR_SHAPE;
    const int64_t need = moe_layer_workspace_bytes(hidden, inter, num_experts, m, top_k);
    if (!ws || !aligned16(ws) || ws_bytes < need)
        return Q4K_ERR_WORKSPACE;
    auto up256 = [](int64_t b) { return (b + 255) / 256 * 256; };
    char *base = (char *)ws;
    float *act = (float *)base;
    float *eo = (float *)(base + up256((P + m) * inter * 4));
    float *s_out = (float *)((char *)eo + up256(P * hidden * 4));
    int32_t *bws = (int32_t *)((char *)s_out + up256(m * hidden * 4));
    const int64_t m_sh = has_sh ? m : 0;
    const bool bucketed = bucketed_for(mode, m);
    hipStream_t st = as_stream(stream);
    GemvLaunch G{};
    G.w0 = w_gate;
    G.w1 = w_up;
    G.s0 = has_sh ? sh_gate : nullptr;
    G.s1 = has_sh ? sh_up : nullptr;
    G.src1 = h_post;
    G.src1_sh = h_post;
    G.ids = ids;
    G.bucket_ws = bucketed ? bws : nullptr;
    G.dst = act;
    G.dst_sh = act + P * inter;
    G.n = inter;
    G.k = hidden;
    G.top_k = top_k;
    G.num_experts = num_experts;
    G.n_pairs = P;
    G.m_sh = m_sh;
    G.outer = hidden;
    G.inner = 0;
    G.outer_sh = hidden;
    G.fused_swiglu = true;
    G.vector_units = vec_units;
    GemvLaunch D = G;
    D.w0 = w_down;
    D.w1 = nullptr;
    D.s0 = has_sh ? sh_down : nullptr;
    D.s1 = nullptr;
    D.src1 = act;
    D.src1_sh = act + P * inter;
    D.dst = eo;
    D.dst_sh = s_out;
    D.n = hidden;
    D.k = inter;
    D.outer = top_k * inter;
    D.inner = inter;
    D.outer_sh = inter;
    D.fused_swiglu = false;
    // Bucketed layers on the matrix cores build their chunk lists inside the
    // two launches when the sizes allow; otherwise (or when asked) one
    // bucketing launch writes the list to the layer workspace (PREBUILT is
    // treated as ON here).
    if (bucketed && !vec_units && !bucket_launch && q4k_self_bucket_ok(G) &&
        q4k_self_bucket_ok(D)) {
        G.bucket_ws = D.bucket_ws = nullptr;
        G.self_bucket = D.self_bucket = true;
    } else if (bucketed) {
        rc = launched(launch_moe_bucket(ids, P, num_experts, bws, st));
        if (rc)
            return rc;
    }
    rc = launched(launch_q4k_gemv(G, st));
    if (rc)
        return rc;
    if (!bucketed && q4k_down_combine_ok(inter, top_k, has_sh)) {
        // few tokens: down fused with the combine, expert_out never written
        rc = launched(launch_q4k_down_combine(D, h_mid, route_w, shared_gate_logit, out, nullptr,
                                              shared_mode, st));
        if (rc || !norm_weight)
            return rc;
        return launched(launch_combine_norm(nullptr, nullptr, nullptr, nullptr, nullptr,
                                            norm_weight, eps, out, normed, hidden, m, top_k,
                                            shared_mode, false, st));
    }
    rc = launched(launch_q4k_gemv(D, st));
    if (rc)
        return rc;
    if (norm_weight)   // the combine and the norm in one launch, a workgroup per token
        return launched(launch_combine_norm(h_mid, eo, route_w, has_sh ? s_out : nullptr,
                                            shared_gate_logit, norm_weight, eps, out, normed,
                                            hidden, m, top_k, shared_mode, true, st));
    return launched(launch_moe_combine(h_mid, eo, route_w, has_sh ? s_out : nullptr,
                                       shared_gate_logit, out, hidden, m, top_k, shared_mode, st));
}

}  // namespace

extern "C" {

int moe_layer_forward(const void *w_gate, const void *w_up, const void *w_down,
                      const void *sh_gate, const void *sh_up, const void *sh_down,
                      const float *h_post, const float *h_mid, const int32_t *ids,
                      const float *route_w, const float *shared_gate_logit, float *out,
                      int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                      int64_t top_k, int shared_mode, int bucket_flag, void *ws,
                      int64_t ws_bytes, void *stream) {
    return layer_forward_impl(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids,
                              route_w, shared_gate_logit, out, hidden, inter, num_experts, m,
                              top_k, shared_mode, bucket_flag, ws, ws_bytes, stream, nullptr,
                              0.0f, nullptr);
}

}  // extern "C"

// ------------------------------------------------ no-allocation layer ----
// Device scratch of the no-allocation layer: one array per GPU, loaded with
// the library's code and held until the process ends.  Host code never uses
// the name as an address (on the host it is a stand-in for the symbol);
// kernels get the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[MOE_LAYER_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device

// Address of the current device's scratch, looked up once per device with
// that device current; nullptr when the lookup fails.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const void *w_gate, const void *w_up, const void *w_down,
                              const void *sh_gate, const void *sh_up, const void *sh_down,
                              const float *h_post, const float *h_mid, const int32_t *ids,
                              const float *route_w, const float *shared_gate_logit, float *out,
                              int64_t hidden, int64_t inter, int64_t num_experts, int64_t m,
                              int64_t top_k, int shared_mode, int bucket_flag, void *stream) {
    const int64_t need = moe_layer_workspace_bytes(hidden, inter, num_experts, m, top_k);
    if (need < 0)
        return Q4K_ERR_SHAPE;
    if (need > MOE_LAYER_NOALLOC_MAX_BYTES)
        return Q4K_ERR_SCRATCH;
    void *ws = device_scratch();
    if (!ws)
        return Q4K_ERR_LAUNCH;
    // the workspace needs no initial contents: every word is written before
    // it is read within the call
    return layer_forward_impl(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids,
                              route_w, shared_gate_logit, out, hidden, inter, num_experts, m,
                              top_k, shared_mode, bucket_flag, ws, MOE_LAYER_NOALLOC_MAX_BYTES,
                              stream, nullptr, 0.0f, nullptr);
}

int moe_layer_forward_rmsnorm(const void *w_gate, const void *w_up, const void *w_down,
                              const void *sh_gate, const void *sh_up, const void *sh_down,
                              const float *h_post, const float *h_mid, const int32_t *ids,
                              const float *route_w, const float *shared_gate_logit, float *out,
                              const void *norm_weight, float eps, float *normed, int64_t hidden,
                              int64_t inter, int64_t num_experts, int64_t m, int64_t top_k,
                              int shared_mode, int bucket_flag, void *ws, int64_t ws_bytes,
                              void *stream) {
    if (!norm_weight || !normed || !aligned2(norm_weight) || !aligned4(normed) || normed == out)
        return Q4K_ERR_NULL;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return Q4K_ERR_ARG;
    return layer_forward_impl(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids,
                              route_w, shared_gate_logit, out, hidden, inter, num_experts, m,
                              top_k, shared_mode, bucket_flag, ws, ws_bytes, stream, norm_weight,
                              eps, normed);
}

int moe_combine_residual(const float *h_mid, const float *expert_out, const float *route_w,
                         const float *shared_out, const float *shared_gate_logit, float *out,
                         int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                         void *stream) {
    if (hidden < 1 || m < 1 || top_k < 1 || top_k > Q4K_MAX_TOP_K)
        return Q4K_ERR_SHAPE;
    if (shared_mode != MOE_SHARED_NONE && shared_mode != MOE_SHARED_SIGMOID &&
        shared_mode != MOE_SHARED_UNSCALED)
        return Q4K_ERR_ARG;
    if (!h_mid || !expert_out || !route_w || !out)
        return Q4K_ERR_NULL;
    if (shared_mode != MOE_SHARED_NONE && !shared_out)
        return Q4K_ERR_NULL;
    if (shared_mode == MOE_SHARED_SIGMOID && !shared_gate_logit)
        return Q4K_ERR_NULL;
    return launched(launch_moe_combine(h_mid, expert_out, route_w, shared_out, shared_gate_logit,
                                       out, hidden, m, top_k, shared_mode, as_stream(stream)));
}

int moe_combine_residual_rmsnorm(const float *h_mid, const float *expert_out,
                                 const float *route_w, const float *shared_out,
                                 const float *shared_gate_logit, const void *norm_weight, float eps,
                                 float *out, float *normed, int64_t hidden, int64_t m,
                                 int64_t top_k, int shared_mode, void *stream) {
    if (hidden < 1 || m < 1 || m > 65535 || top_k < 1 || top_k > Q4K_MAX_TOP_K)
        return Q4K_ERR_SHAPE;
    if (shared_mode != MOE_SHARED_NONE && shared_mode != MOE_SHARED_SIGMOID &&
        shared_mode != MOE_SHARED_UNSCALED)
        return Q4K_ERR_ARG;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return Q4K_ERR_ARG;
    if (!h_mid || !expert_out || !route_w || !out || !normed || !norm_weight ||
        !aligned2(norm_weight) || normed == out)
        return Q4K_ERR_NULL;
    if (shared_mode != MOE_SHARED_NONE && !shared_out)
        return Q4K_ERR_NULL;
    if (shared_mode == MOE_SHARED_SIGMOID && !shared_gate_logit)
        return Q4K_ERR_NULL;
    return launched(launch_combine_norm(h_mid, expert_out, route_w, shared_out, shared_gate_logit,
                                        norm_weight, eps, out, normed, hidden, m, top_k,
                                        shared_mode, true, as_stream(stream)));
}

int64_t q4tp_tensor_bytes(int64_t rows, int64_t cols) {
    if (rows < 1 || cols < 32 || cols % 32)
        return -1;
    const int64_t gpr = cols / 32;
    return rows * gpr * 16 + rows * 4 + rows * ((5 * gpr + 7) / 8);
}

int q4tp_matvec(const void *tensor, const float *x, float *y, int64_t rows, int64_t cols,
                void *stream) {
    if (rows < 1 || rows > (1 << 30) || cols < 32 || cols % 32 || cols > Q4TP_MAX_COLS)
        return Q4K_ERR_SHAPE;
    if (!tensor || !x || !y || !aligned16(tensor) || !aligned4(x) || !aligned4(y))
        return Q4K_ERR_NULL;
    return launched(launch_q4tp_matvec(tensor, x, y, rows, cols, as_stream(stream)));
}

int q4tp_matvec_multi(const void *const *tensors, const int64_t *rows, int n_tensors,
                      const float *x, float *y, int64_t cols, void *stream) {
    if (n_tensors < 1 || n_tensors > Q4TP_MAX_TENSORS || cols < 32 || cols % 32 ||
        cols > Q4TP_MAX_COLS)
        return Q4K_ERR_SHAPE;
    if (!tensors || !rows || !x || !y || !aligned4(x) || !aligned4(y))
        return Q4K_ERR_NULL;
    int64_t total = 0;
    for (int i = 0; i < n_tensors; i++) {
        if (rows[i] < 1 || rows[i] > (1 << 30))
            return Q4K_ERR_SHAPE;
        total += rows[i];
        if (!tensors[i] || !aligned16(tensors[i]))
            return Q4K_ERR_NULL;
    }
    if (total > (1 << 30))
        return Q4K_ERR_SHAPE;
    return launched(launch_q4tp_matvec_multi(tensors, rows, n_tensors, x, y, cols,
                                             as_stream(stream)));
}

int q4tp_quantize(const float *w, void *tensor, int64_t rows, int64_t cols, void *stream) {
    if (rows < 1 || rows > (1 << 30) || cols < 32 || cols % 32 || cols > Q4TP_MAX_COLS)
        return Q4K_ERR_SHAPE;
    if (!w || !tensor || !aligned16(tensor) || !aligned4(w))
        return Q4K_ERR_NULL;
    return launched(launch_q4tp_quant(w, tensor, rows, cols, as_stream(stream)));
}

int64_t mlx4_matrix_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < MLX4_GROUP || k % MLX4_GROUP)
        return -1;
    return n * k / 2 + 2 * (n * (k / MLX4_GROUP) * 2);
}

int mlx4_dequantize(const void *packed, const void *scales, const void *biases, float *out,
                    int64_t n, int64_t k, void *stream) {
    if (n < 0 || n > (1 << 30) || k < MLX4_GROUP || k % MLX4_GROUP || k > Q4K_MAX_IN)
        return Q4K_ERR_SHAPE;
    if (n == 0)
        return Q4K_OK;
    if (!packed || !scales || !biases || !out || !aligned16(packed) || !aligned2(scales) ||
        !aligned2(biases) || !aligned16(out))
        return Q4K_ERR_NULL;
    return launched(launch_mlx4_dequant(packed, scales, biases, out, n * (k / MLX4_GROUP), 4,
                                        as_stream(stream)));
}

int mlx4_quantize(const float *w, void *packed, void *scales, void *biases, int64_t n, int64_t k,
                  void *stream) {
    if (n < 0 || n > (1 << 30) || k < MLX4_GROUP || k % MLX4_GROUP || k > Q4K_MAX_IN)
        return Q4K_ERR_SHAPE;
    if (n == 0)
        return Q4K_OK;
    if (!w || !packed || !scales || !biases || !aligned4(w) || !aligned16(packed) ||
        !aligned2(scales) || !aligned2(biases))
        return Q4K_ERR_NULL;
    return launched(launch_mlx4_quant(w, packed, scales, biases, n * (k / MLX4_GROUP), 4,
                                      as_stream(stream)));
}

}  // extern "C"

namespace {

// Shape, block and alignment checks shared by the MLX 4-bit id-GEMV entry
// points; offs holds (packed, scales, biases) offsets of n_mats matrices.
int mlx4_check(const void *expert_base, int64_t expert_stride, const int64_t *offs, int n_mats,
               const float *src1, const int32_t *ids, const float *dst, int64_t n, int64_t k,
               int64_t m, int64_t top_k, int64_t outer, int64_t inner, int64_t num_experts,
               int bits = 4) {
    if (n < 1 || n > (1 << 30) || k < MLX4_GROUP || k % MLX4_GROUP || k > Q4K_MAX_IN || m < 1 ||
        top_k < 1 || top_k > Q4K_MAX_TOP_K || num_experts < 1 || m * top_k > 65535)
        return Q4K_ERR_SHAPE;
    // every sub-tensor inside one expert block
    const int64_t pbytes = n * k * bits / 8, sbytes = n * (k / MLX4_GROUP) * 2;
    if (expert_stride < 0)
        return Q4K_ERR_SHAPE;
    for (int i = 0; i < n_mats; i++) {
        const int64_t po = offs[3 * i], so = offs[3 * i + 1], bo = offs[3 * i + 2];
        if (po < 0 || so < 0 || bo < 0 || po + pbytes > expert_stride ||
            so + sbytes > expert_stride || bo + sbytes > expert_stride)
            return Q4K_ERR_SHAPE;
    }
    if (outer < 0 || inner < 0)
        return Q4K_ERR_STRIDE;
    if (!expert_base || !src1 || !ids || !dst || !aligned16(expert_base) || expert_stride % 16 ||
        !aligned4(src1) || !aligned4(ids) || !aligned4(dst))
        return Q4K_ERR_NULL;
    for (int i = 0; i < n_mats; i++)
        if (offs[3 * i] % 16 || offs[3 * i + 1] % 2 || offs[3 * i + 2] % 2)
            return Q4K_ERR_NULL;
    return Q4K_OK;
}

}  // namespace

extern "C" {

int mlx4_moe_id_gemv(const void *expert_base, int64_t expert_stride, int64_t packed_off,
                     int64_t scales_off, int64_t biases_off, const float *src1,
                     const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                     int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                     int64_t num_experts, void *stream) {
    const int64_t offs[3] = {packed_off, scales_off, biases_off};
    const int rc = mlx4_check(expert_base, expert_stride, offs, 1, src1, ids, dst, n, k, m, top_k,
                              src1_outer_stride, src1_inner_stride, num_experts);
    if (rc)
        return rc;
    Mlx4Launch L{};
    L.base = expert_base;
    L.expert_stride = expert_stride;
    L.packed_off = packed_off;
    L.scales_off = scales_off;
    L.biases_off = biases_off;
    L.src1 = src1;
    L.ids = ids;
    L.dst = dst;
    L.n = n;
    L.k = k;
    L.m = m;
    L.top_k = top_k;
    L.num_experts = num_experts;
    L.outer = src1_outer_stride;
    L.inner = src1_inner_stride;
    return launched(launch_mlx4_gemv(L, as_stream(stream)));
}

int mlx4_moe_gate_up_silu(const void *expert_base, int64_t expert_stride, int64_t gate_packed_off,
                          int64_t gate_scales_off, int64_t gate_biases_off, int64_t up_packed_off,
                          int64_t up_scales_off, int64_t up_biases_off, const float *src1,
                          const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                          int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                          int64_t num_experts, void *stream) {
    const int64_t offs[6] = {gate_packed_off, gate_scales_off, gate_biases_off,
                             up_packed_off,   up_scales_off,   up_biases_off};
    const int rc = mlx4_check(expert_base, expert_stride, offs, 2, src1, ids, dst, n, k, m, top_k,
                              src1_outer_stride, src1_inner_stride, num_experts);
    if (rc)
        return rc;
    Mlx4Launch L{};
    L.base = expert_base;
    L.expert_stride = expert_stride;
    L.packed_off = gate_packed_off;
    L.scales_off = gate_scales_off;
    L.biases_off = gate_biases_off;
    L.packed_off1 = up_packed_off;
    L.scales_off1 = up_scales_off;
    L.biases_off1 = up_biases_off;
    L.fused_swiglu = true;
    L.src1 = src1;
    L.ids = ids;
    L.dst = dst;
    L.n = n;
    L.k = k;
    L.m = m;
    L.top_k = top_k;
    L.num_experts = num_experts;
    L.outer = src1_outer_stride;
    L.inner = src1_inner_stride;
    return launched(launch_mlx4_gemv(L, as_stream(stream)));
}

int64_t mlx2_matrix_bytes(int64_t n, int64_t k) {
    if (n < 0 || k < MLX4_GROUP || k % MLX4_GROUP)
        return -1;
    return n * k / 4 + 2 * (n * (k / MLX4_GROUP) * 2);
}

int mlx2_dequantize(const void *packed, const void *scales, const void *biases, float *out,
                    int64_t n, int64_t k, void *stream) {
    if (n < 0 || n > (1 << 30) || k < MLX4_GROUP || k % MLX4_GROUP || k > Q4K_MAX_IN)
        return Q4K_ERR_SHAPE;
    if (n == 0)
        return Q4K_OK;
    if (!packed || !scales || !biases || !out || !aligned16(packed) || !aligned2(scales) ||
        !aligned2(biases) || !aligned16(out))
        return Q4K_ERR_NULL;
    return launched(launch_mlx4_dequant(packed, scales, biases, out, n * (k / MLX4_GROUP), 2,
                                        as_stream(stream)));
}

int mlx2_quantize(const float *w, void *packed, void *scales, void *biases, int64_t n, int64_t k,
                  void *stream) {
    if (n < 0 || n > (1 << 30) || k < MLX4_GROUP || k % MLX4_GROUP || k > Q4K_MAX_IN)
        return Q4K_ERR_SHAPE;
    if (n == 0)
        return Q4K_OK;
    if (!w || !packed || !scales || !biases || !aligned4(w) || !aligned16(packed) ||
        !aligned2(scales) || !aligned2(biases))
        return Q4K_ERR_NULL;
    return launched(launch_mlx4_quant(w, packed, scales, biases, n * (k / MLX4_GROUP), 2,
                                      as_stream(stream)));
}

int mlx2_moe_id_gemv(const void *expert_base, int64_t expert_stride, int64_t packed_off,
                     int64_t scales_off, int64_t biases_off, const float *src1,
                     const int32_t *ids, float *dst, int64_t n, int64_t k, int64_t m,
                     int64_t top_k, int64_t src1_outer_stride, int64_t src1_inner_stride,
                     int64_t num_experts, void *stream) {
    const int64_t offs[3] = {packed_off, scales_off, biases_off};
    const int rc = mlx4_check(expert_base, expert_stride, offs, 1, src1, ids, dst, n, k, m, top_k,
                              src1_outer_stride, src1_inner_stride, num_experts, 2);
    if (rc)
        return rc;
    Mlx4Launch L{};
    L.base = expert_base;
    L.expert_stride = expert_stride;
    L.packed_off = packed_off;
    L.scales_off = scales_off;
    L.biases_off = biases_off;
    L.bits = 2;
    L.src1 = src1;
    L.ids = ids;
    L.dst = dst;
    L.n = n;
    L.k = k;
    L.m = m;
    L.top_k = top_k;
    L.num_experts = num_experts;
    L.outer = src1_outer_stride;
    L.inner = src1_inner_stride;
    return launched(launch_mlx4_gemv(L, as_stream(stream)));
}

}  // extern "C"
