// Expert bucketing and the weighted residual combine.
//
// Bucketing (moeflux expert_forward.rs, encode_moe_gather_id_fuse step 1 and
// the ExpertBuckets CSR): one workgroup of 1024 threads counts pairs per
// expert, scans the counts, lists the non-empty buckets and the work chunks
// (at most kBucketChunk pairs of one bucket each), and places the pairs in
// pair order: one wave takes 64 pairs at a time, finds the lanes that share a
// bucket by ballots over the bucket's bits, and writes each pair at its
// bucket's running cursor plus its rank among those lanes.  Each bucket thus
// lists its pairs in ascending pair order (a stable counting sort), the same on
// every run.  Bucket E collects ids outside [0, E).
//
// Combine (moeflux module doc and encode_moe_combine_residual_n_tokens):
// out[t,i] = h_mid[t,i] + sum_s w[t,s]*expert_out[t,s,i] + g_t*shared_out[t,i],
// slots in order, one thread per output element.
#include "common.hpp"
#include "launch.hpp"

namespace q4k {

constexpr int kBucketThreads = 1024;
constexpr int kMaxPairs = 8192;

__global__ __launch_bounds__(kBucketThreads) void k_moe_bucket(const int32_t *__restrict__ ids,
                                                               int P, int E, int32_t *ws) {
    __shared__ int cnt[kBucketThreads];
    __shared__ int bk[kMaxPairs];   // bucket of each pair
    __shared__ int wsum_c[16], wsum_f[16], wsum_h[16];
    const int tid = threadIdx.x;
    int32_t *counts = ws;
    int32_t *offsets = counts + (E + 1);
    int32_t *pairs = offsets + (E + 2);
    int32_t *active = pairs + P;
    int32_t *n_active = active + (E + 1);
    int32_t *n_chunks = n_active + 1;
    int32_t *chunks = n_chunks + 1;

    cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kBucketThreads) {
        const int e = ids[p];
        const int b = ((unsigned)e < (unsigned)E) ? e : E;
        atomicAdd(&cnt[b], 1);
        bk[p] = b;
    }
    __syncthreads();

    // Exclusive scans of the counts and of the non-empty flags over buckets.
    // Exclusive scans over buckets of the counts, of the non-empty flags and of
    // the chunk counts (kBucketChunk pairs per chunk).
    const int c = tid <= E ? cnt[tid] : 0;
    const int f = c > 0 ? 1 : 0;
    const int h = (c + kBucketChunk - 1) / kBucketChunk;
    int ic = c, iff = f, ih = h;   // inclusive wave scans
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int tc = __shfl_up(ic, off, 64);
        const int tf = __shfl_up(iff, off, 64);
        const int th = __shfl_up(ih, off, 64);
        if (lane >= off) {
            ic += tc;
            iff += tf;
            ih += th;
        }
    }
    if (lane == 63) {
        wsum_c[wave] = ic;
        wsum_f[wave] = iff;
        wsum_h[wave] = ih;
    }
    __syncthreads();
    int base_c = 0, base_f = 0, base_h = 0;
    for (int w = 0; w < wave; w++) {
        base_c += wsum_c[w];
        base_f += wsum_f[w];
        base_h += wsum_h[w];
    }
    const int ex_c = base_c + ic - c;
    const int ex_f = base_f + iff - f;
    const int ex_h = base_h + ih - h;
    if (tid <= E) {
        counts[tid] = c;
        offsets[tid] = ex_c;
        if (f)
            active[ex_f] = tid;
        for (int i = 0; i < h; i++) {
            const int n = c - i * kBucketChunk < kBucketChunk ? c - i * kBucketChunk : kBucketChunk;
            chunks[2 * (ex_h + i)] = tid;
            chunks[2 * (ex_h + i) + 1] = (ex_c + i * kBucketChunk) | (n << 24);
        }
    }
    if (tid == E) {
        offsets[E + 1] = ex_c + c;
        *n_active = ex_f + f;
        *n_chunks = ex_h + h;
    }

    // Stable placement, one wave.  The cursors start at the offsets (cnt is
    // reused; every wave has read its count above).
    __syncthreads();
    if (tid <= E)
        cnt[tid] = ex_c;
    __syncthreads();
    if (wave != 0)
        return;
    int nbits = 1;
    while ((1 << nbits) <= E)
        nbits++;
    const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;   // lanes under this one
    for (int p0 = 0; p0 < P; p0 += 64) {
        const int p = p0 + lane;
        const bool live = p < P;
        const int b = live ? bk[p] : 0;
        uint64_t same = __ballot(live);
        for (int bit = 0; bit < nbits; bit++) {
            const bool on = (b >> bit) & 1;
            const uint64_t m = __ballot(on);
            same &= on ? m : ~m;
        }
        if (live) {
            const int rank = __popcll(same & below);
            pairs[cnt[b] + rank] = p;
            if (rank == 0)   // one lane per bucket of this step
                cnt[b] += __popcll(same);
        }
    }
}

hipError_t launch_moe_bucket(const int32_t *ids, int64_t n_pairs, int64_t num_experts,
                             int32_t *ws, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_bucket, dim3(1), dim3(kBucketThreads), 0, st, ids, (int)n_pairs,
                       (int)num_experts, ws);
    return hipGetLastError();
}

// Combined value of output (t, i).  The top_k expert rows and weights are all
// loaded before the first use (slots past top_k re-load the last one, clamped,
// and are skipped), so the loads are in flight together; the sum then runs in
// slot order, one fma per slot, as the pages' combine does.
template <int KMAX>
__device__ __forceinline__ float combine_one(const float *__restrict__ h_mid,
                                             const float *__restrict__ eo,
                                             const float *__restrict__ w,
                                             const float *__restrict__ shared,
                                             const float *__restrict__ logit, int64_t H,
                                             int64_t t, int64_t i, int K, int mode) {
    const int64_t idx = t * H + i;
    float e[KMAX], wv[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; s++) {
        const int sc = s < K ? s : K - 1;
        e[s] = eo[(t * K + sc) * H + i];
        wv[s] = w[t * K + sc];
    }
    const float sh = mode != 0 ? shared[idx] : 0.0f;
    const float lg = mode == 1 ? logit[t] : 0.0f;
    float acc = h_mid[idx];
#pragma unroll
    for (int s = 0; s < KMAX; s++)
        if (s < K)
            acc = __builtin_fmaf(wv[s], e[s], acc);
    if (mode == 1) {
        const float g = 1.0f / (1.0f + expf(-lg));
        acc = __builtin_fmaf(g, sh, acc);
    } else if (mode == 2) {
        acc += sh;
    }
    return acc;
}

// One thread per output element.
template <int KMAX>
__global__ __launch_bounds__(256) void k_moe_combine(const float *__restrict__ h_mid,
                                                     const float *__restrict__ eo,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ shared,
                                                     const float *__restrict__ logit,
                                                     float *out, int64_t H, int64_t m, int K,
                                                     int mode) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= H * m)
        return;
    const int64_t t = idx / H, i = idx - t * H;
    out[idx] = combine_one<KMAX>(h_mid, eo, w, shared, logit, H, t, i, K, mode);
}

// RMSNorm of each row of `out` into `normed` (moeflux's chain appendix after
// the combine: sum of squares, then the bf16-weighted apply), one workgroup
// per token of kNormThreads threads (a few outputs per thread, so a token's
// loads are in flight together); with COMBINE the row is first computed by
// the combine (same arithmetic as k_moe_combine) and written to `out`.
//   normed[t, i] = out[t, i] / sqrt(sum_j out[t, j]^2 / H + eps) * w[i]
// Each thread re-reads only the outputs it wrote itself.
constexpr int kNormThreads = 1024;

template <int KMAX, bool COMBINE>
__global__ __launch_bounds__(kNormThreads) void k_combine_norm(const float *__restrict__ h_mid,
                                                      const float *__restrict__ eo,
                                                      const float *__restrict__ w,
                                                      const float *__restrict__ shared,
                                                      const float *__restrict__ logit,
                                                      const uint16_t *__restrict__ nw, float eps,
                                                      float *out, float *__restrict__ normed,
                                                      int64_t H, int K, int mode) {
    __shared__ float part[kNormThreads / 64];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    float ss = 0.0f;
    for (int64_t i = tid; i < H; i += kNormThreads) {
        float v;
        if constexpr (COMBINE) {
            v = combine_one<KMAX>(h_mid, eo, w, shared, logit, H, t, i, K, mode);
            out[t * H + i] = v;
        } else {
            v = out[t * H + i];
        }
        ss = __builtin_fmaf(v, v, ss);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        ss += __shfl_xor(ss, off, 64);
    if ((tid & 63) == 0)
        part[tid >> 6] = ss;
    __syncthreads();
    float total = 0.0f;
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; w++)
        total += part[w];
    const float inv = 1.0f / sqrtf(total / (float)H + eps);
    for (int64_t i = tid; i < H; i += kNormThreads) {
        const float wi = __uint_as_float((uint32_t)nw[i] << 16);
        normed[t * H + i] = out[t * H + i] * inv * wi;
    }
}

hipError_t launch_combine_norm(const float *h_mid, const float *expert_out, const float *route_w,
                               const float *shared_out, const float *shared_gate_logit,
                               const void *norm_weight, float eps, float *out, float *normed,
                               int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                               bool combine, hipStream_t st) {
    if (m == 0)
        return hipSuccess;
    const uint16_t *nw = (const uint16_t *)norm_weight;
    const dim3 grid((unsigned)m);
    if (!combine)
        hipLaunchKernelGGL((k_combine_norm<1, false>), grid, dim3(kNormThreads), 0, st, h_mid, expert_out,
                           route_w, shared_out, shared_gate_logit, nw, eps, out, normed, hidden,
                           (int)top_k, shared_mode);
    else if (top_k <= 8)
        hipLaunchKernelGGL((k_combine_norm<8, true>), grid, dim3(kNormThreads), 0, st, h_mid, expert_out,
                           route_w, shared_out, shared_gate_logit, nw, eps, out, normed, hidden,
                           (int)top_k, shared_mode);
    else
        hipLaunchKernelGGL((k_combine_norm<kMaxTopK, true>), grid, dim3(kNormThreads), 0, st, h_mid,
                           expert_out, route_w, shared_out, shared_gate_logit, nw, eps, out,
                           normed, hidden, (int)top_k, shared_mode);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float *h_mid, const float *expert_out, const float *route_w,
                              const float *shared_out, const float *shared_gate_logit, float *out,
                              int64_t hidden, int64_t m, int64_t top_k, int shared_mode,
                              hipStream_t st) {
    const int64_t n = hidden * m;
    if (n == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (top_k <= 8)
        hipLaunchKernelGGL(k_moe_combine<8>, grid, dim3(256), 0, st, h_mid, expert_out, route_w,
                           shared_out, shared_gate_logit, out, hidden, m, (int)top_k, shared_mode);
    else
        hipLaunchKernelGGL(k_moe_combine<kMaxTopK>, grid, dim3(256), 0, st, h_mid, expert_out,
                           route_w, shared_out, shared_gate_logit, out, hidden, m, (int)top_k,
                           shared_mode);
    return hipGetLastError();
}

}  // namespace q4k
