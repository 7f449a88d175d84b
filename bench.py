#!/usr/bin/env python3
"""Benchmark of the Q4_K MoE decode layer on one MI355X.

A step is one whole MoE layer on one batch of synthetic decode input: the
fused gate/up id-GEMV with SiLU over the routed experts and the shared expert,
the down id-GEMV, and the weighted residual combine (with expert bucketing
when the batch is large enough) -- every kernel of the hot path.

Headline workload (the JSON line's `value`): hidden 2048, expert intermediate
768, 128 experts, top_k 8, m = 1 token, sigmoid-gated shared expert of the
same shape (a Qwen3-30B-A3B-class layer; ferrum-kernels
q4_k_moe_id_gemv_batched.rs microbench shape, moeflux expert_forward.rs
combine).  value = unique expert-weight bytes per layer (distinct routed
experts plus the shared expert, three matrices each) / wall time per layer.

Further objects on the same line:
  m16      the same layer at m = 16 with Zipf(1.1) routing (bucketed), and its
           gate/up and down launches alone;
  sweep    m in {1, 2, 4, 8, 16}: the layer in AUTO, token mode, bucketed on
           the matrix cores and bucketed on the vector units, with the pages'
           batching criterion (ferrum moe_gemv_scaling_microbench: m = 16 in
           less than 0.6 x 16 x the m = 1 time);
  cfg4     hidden 7168, inter 2048, 256 experts, top_k 8 at m = 1 and m = 32;
  walk     the dense Q4TiledP decode walk (cortiq-engine mv_lab.rs) over
           several layers plus the head;
  mlx4     the MLX affine 4-bit / 2-bit id-GEMV at the single-token shapes;
  roofline the dominant kernel of the headline layer against HBM peak, with
           `ceiling` = the read rate of the same bytes by a plain coalesced
           read of the same expert matrices (q4k_ceiling_read);
  cpu_baseline  the CPU oracle's layer on one thread and on all host cores.

Protocol: weights live as R device-encoded replicas and G routing draws; step
i uses replica i mod R and draw i mod G, so consecutive steps read different
bytes and a graph of steps touches far more than the 256 MB Infinity Cache.
Steps are captured into HIP graphs.  Warm-up steps use draws disjoint from
the timed ones.  Every figure is timed in R rounds, figures round-robin (the
pages' lab protocol, cortiq-engine mv_lab.rs `main`), and reported as the
median with the quartiles; each headline round times exactly --steps layers
between device synchronisations, with HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE id-GEMV effective HBM GB/s (% of peak) + µs/MoE layer at M=1,16"
HBM_PEAK_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gate_up_silu_m1_hbm_traffic.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quartiles(vals):
    v = sorted(vals)
    n = len(v)

    def q(p):
        x = p * (n - 1)
        lo = int(x)
        hi = min(lo + 1, n - 1)
        return v[lo] + (v[hi] - v[lo]) * (x - lo)
    return q(0.25), q(0.5), q(0.75)


# ------------------------------------------------------------ timing ----

class Figure:
    """A HIP graph of `n` steps and the bytes those steps read; timed once
    per round."""

    def __init__(self, torch, name, fn, idx, bytes_of, warm_idx=None):
        self.torch, self.name, self.n = torch, name, len(idx)
        # the graph holds raw device pointers of whatever fn launches with: keep
        # fn (and the tensors its closure owns) alive as long as the graph
        self.fn = fn
        self.bytes = sum(bytes_of(i) for i in idx)
        log(f"capturing {name} ({self.n} steps)")
        self.graph = capture(torch, fn, idx)
        self.warm = capture(torch, fn, warm_idx) if warm_idx else None
        self.secs = []

    def run(self):
        torch = self.torch
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        self.graph.replay()
        e1.record()
        torch.cuda.synchronize()
        self.secs.append(e0.elapsed_time(e1) / 1e3)

    def summary(self):
        q1, med, q3 = quartiles([s / self.n * 1e6 for s in self.secs])
        return dict(us=round(med, 3), us_q1=round(q1, 3), us_q3=round(q3, 3),
                    gbs=round(self.bytes / self.n / med / 1e3, 2),
                    frac_hbm_peak=round(self.bytes / self.n / med / 1e3 / HBM_PEAK_GBS, 4),
                    bytes_per_step=int(self.bytes / self.n), steps=self.n, rounds=len(self.secs))


def capture(torch, fn, idx):
    """HIP graph of fn(i) for i in idx, run once on a side stream first."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in idx:
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in idx:
            fn(i)
    torch.cuda.synchronize()
    return g


def run_rounds(figs, rounds):
    for f in figs:
        if f.warm is not None:
            f.warm.replay()
    for _ in range(rounds):
        for f in figs:
            f.run()


# ---------------------------------------------------------- workload ----

class Moe:
    """Device-resident expert replicas and per-step inputs of one MoE
    workload (config cfg), plus the byte ranges each step reads."""

    def __init__(self, torch, q4, wl, cfg, replicas, n_sets, stacks=None, shared=None,
                 shared_replicas=None):
        self.torch, self.q4, self.cfg = torch, q4, cfg
        dev = torch.device("cuda")
        H, I, E = cfg.hidden, cfg.inter, cfg.num_experts
        self.mat = q4.q4k_tiles_bytes(I, H)           # gate/up and down matrices alike
        if stacks is None:
            stacks = [[self._encode(wl, E, rows, cols, cfg.w_std, 1000 * r + t)
                       for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)])]
                      for r in range(replicas)]
        if shared is None:
            shared = [[self._encode(wl, 1, rows, cols, cfg.w_std, 1000 * r + 3 + t)
                       for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)])]
                      for r in range(shared_replicas or len(stacks))]
        self.stacks, self.shared = stacks, shared
        torch.cuda.synchronize()
        m, K = cfg.m, cfg.top_k
        P = m * K
        self.sets, self.unique, self.ws_sets, self.ranges = [], [], [], []
        for s in range(n_sets):
            a = wl.moe_activations(cfg, index=s)
            self.sets.append(dict(h_post=torch.from_numpy(a.h_post).to(dev),
                                  h_mid=torch.from_numpy(a.h_mid).to(dev),
                                  ids=torch.from_numpy(a.ids).to(dev),
                                  route_w=torch.from_numpy(a.route_w).to(dev),
                                  logit=torch.from_numpy(a.shared_logit).to(dev)))
            self.unique.append(sorted(set(int(e) for e in a.ids if 0 <= e < E)))
            wsb = q4.moe_bucket_workspace_bytes(P, E)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
            q4.moe_bucket(self.sets[-1]["ids"], P, E, ws, wsb)
            self.ws_sets.append(ws)
        self.wsb = q4.moe_bucket_workspace_bytes(P, E)
        self.act = torch.randn(P + m, I, device=dev)
        self.eo = torch.empty(P, H, device=dev)
        self.s_act = torch.empty(m, I, device=dev)
        self.out = torch.empty(m, H, device=dev)
        self.normed = torch.empty(m, H, device=dev)
        self.norm_w = torch.ones(H, device=dev).to(torch.bfloat16)
        self.lwsb = q4.moe_layer_workspace_bytes(H, I, E, m, K)
        self.lws = torch.empty(self.lwsb, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self.ceiling_offsets = []
        torch.cuda.synchronize()

    def _encode(self, wl, n_exp, rows, cols, std, seed):
        """n_exp experts of rows x cols: N(0, std^2) on the device, Q4_K
        encoded, then packed into the tile layout the GEMV kernels read."""
        torch, q4 = self.torch, self.q4
        mb, tb = q4.q4k_matrix_bytes(rows, cols), q4.q4k_tiles_bytes(rows, cols)
        b = torch.empty(n_exp * tb, dtype=torch.uint8, device="cuda")
        per = max(1, (1 << 28) // (rows * cols * 4))     # experts per encoding batch (<= 256 MB fp32)
        for e0 in range(0, n_exp, per):
            ne = min(per, n_exp - e0)
            w = wl.device_normal((ne * rows, cols), std, seed=seed * 4099 + e0)
            gguf = torch.empty(ne * mb, dtype=torch.uint8, device="cuda")
            q4.q4k_quantize(w, gguf, ne * rows, cols)
            q4.q4k_pack_tiles(gguf, b[e0 * tb:(e0 + ne) * tb], ne, rows, cols)
            del w, gguf
        return b

    def pick(self, i):
        return self.stacks[i % len(self.stacks)], self.shared[i % len(self.shared)], \
            i % len(self.sets)

    def key(self, i):
        return i % len(self.stacks), i % len(self.shared), i % len(self.sets)

    def layer(self, i, flag=None):
        q4, c = self.q4, self.cfg
        st, sh, s = self.pick(i)
        x = self.sets[s]
        q4.moe_layer_forward(*st, *sh, x["h_post"], x["h_mid"], x["ids"], x["route_w"],
                             x["logit"], self.out, c.hidden, c.inter, c.num_experts, c.m,
                             c.top_k, c.shared_mode,
                             q4.Q4K_BUCKET_AUTO if flag is None else flag, self.lws, self.lwsb)

    def layer_norm(self, i):
        q4, c = self.q4, self.cfg
        st, sh, s = self.pick(i)
        x = self.sets[s]
        q4.moe_layer_forward_rmsnorm(*st, *sh, x["h_post"], x["h_mid"], x["ids"], x["route_w"],
                                     x["logit"], self.out, self.norm_w, 1e-6, self.normed,
                                     c.hidden, c.inter, c.num_experts, c.m, c.top_k,
                                     c.shared_mode, q4.Q4K_BUCKET_AUTO, self.lws, self.lwsb)

    def bucketed(self):
        return self.cfg.m >= self.q4.Q4K_AUTO_BUCKET_MIN_TOKENS

    def gate_up(self, i):
        """The layer's first launch alone (buckets pre-built when bucketed)."""
        q4, c = self.q4, self.cfg
        st, sh, s = self.pick(i)
        x = self.sets[s]
        flag = q4.Q4K_BUCKET_PREBUILT if self.bucketed() else q4.Q4K_BUCKET_OFF
        q4.q4k_moe_gate_up_silu(st[0], st[1], x["h_post"], x["ids"], self.act, c.inter,
                                c.hidden, c.m, c.top_k, c.hidden, 0, c.num_experts, sh[0], sh[1],
                                self.s_act, flag, self.ws_sets[s], self.wsb)

    def down(self, i):
        """The routed down projection alone (the bucketed id-GEMV on pre-built
        buckets, one activation row per pair)."""
        q4, c = self.q4, self.cfg
        st, sh, s = self.pick(i)
        x = self.sets[s]
        q4.q4k_moe_id_gemv(st[2], self.act, x["ids"], self.eo, c.hidden, c.inter, c.m, c.top_k,
                           c.top_k * c.inter, c.inter, c.num_experts, q4.Q4K_BUCKET_PREBUILT,
                           self.ws_sets[s], self.wsb)

    def ceiling(self, mats):
        """fn(i): a plain read of the matrices `mats` (0 gate, 1 up, 2 down)
        of the experts step i touches (and the shared expert's)."""
        torch, q4 = self.torch, self.q4
        base = self.stacks[0][0]
        b0 = base.data_ptr()
        offs = {}
        for r in range(max(len(self.stacks), len(self.shared))):
            for s in range(len(self.sets)):
                ks = (r % len(self.stacks), r % len(self.shared), s)
                st, sh = self.stacks[ks[0]], self.shared[ks[1]]
                o = [st[t].data_ptr() + e * self.mat - b0 for e in self.unique[s] for t in mats]
                o += [sh[t].data_ptr() - b0 for t in mats]
                offs[ks] = torch.tensor(o, dtype=torch.int64, device="cuda")

        # owned by the workload too: captured graphs replay with these pointers
        self.ceiling_offsets.append(offs)

        def fn(i):
            t = offs[self.key(i)]
            q4.q4k_ceiling_read(base, t, t.numel(), self.mat, self.sink)
        return fn

    def bytes_of(self, n_mats):
        return lambda i: (len(self.unique[i % len(self.sets)]) + 1) * n_mats * self.mat


# --------------------------------------------------------- sections ----

def section_walk(torch, q4, wl, n_layers, rounds):
    """The dense Q4TiledP decode walk: n_layers distinct layers of q, k, v, o
    (4096x4096), gate, up (14336x4096), down (4096x14336), then the head
    (32000x4096), merged dispatches q|k|v and gate|up (the pages' mode `m`),
    and one launch per tensor; 2 replicas of the whole walk alternate."""
    dev = torch.device("cuda")
    shapes = [(r, c) for _, r, c, _ in wl.walk_tensors(n_layers, True)]
    reps = []
    for rep in range(2):
        ts = []
        for i, (rows, cols) in enumerate(shapes):
            w = wl.device_normal((rows, cols), 0.02, seed=50000 + 1000 * rep + i)
            t = torch.empty(q4.q4tp_tensor_bytes(rows, cols), dtype=torch.uint8, device=dev)
            q4.q4tp_quantize(w, t, rows, cols)
            del w
            ts.append(t)
        reps.append(ts)
    x = wl.device_normal((wl.WALK_X_LEN,), 1.0, seed=59999)
    ys = [torch.empty(r, device=dev) for r, _ in shapes]
    groups = []
    for layer in range(n_layers):
        b = 7 * layer
        groups += [[b, b + 1, b + 2], [b + 3], [b + 4, b + 5], [b + 6]]
    groups.append([7 * n_layers])
    ym = [torch.empty(sum(shapes[j][0] for j in g), device=dev) for g in groups]
    torch.cuda.synchronize()

    def merged(i):
        ts = reps[i % 2]
        for g, y in zip(groups, ym):
            q4.q4tp_matvec_multi([ts[j] for j in g], [shapes[j][0] for j in g], x, y,
                                 shapes[g[0]][1])

    def single(i):
        ts = reps[i % 2]
        for (r, c), t, y in zip(shapes, ts, ys):
            q4.q4tp_matvec(t, x, y, r, c)

    # the read ceiling of the same access pattern: a plain read of each merged
    # group's tensors, one launch per group, in the same order
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    reads = []
    for ts in reps:
        reads.append([(ts[g[0]], torch.tensor([ts[j].data_ptr() - ts[g[0]].data_ptr() for j in g],
                                               dtype=torch.int64, device=dev),
                       len(g), q4.q4tp_tensor_bytes(*shapes[g[0]])) for g in groups])

    def ceiling(i):
        for base, offs, n, nb in reads[i % 2]:
            q4.q4k_ceiling_read(base, offs, n, nb, sink)

    nbytes = sum(q4.q4tp_tensor_bytes(r, c) for r, c in shapes)
    figs = [Figure(torch, "walk merged", merged, range(4), lambda i: nbytes),
            Figure(torch, "walk single", single, range(4), lambda i: nbytes),
            Figure(torch, "walk ceiling", ceiling, range(4), lambda i: nbytes)]
    run_rounds(figs, rounds)
    m, s, c = figs[0].summary(), figs[1].summary(), figs[2].summary()
    return {
        "workload": f"dense Q4TiledP decode walk: {n_layers} layers of q, k, v, o 4096x4096, "
                    "gate and up 14336x4096, down 4096x14336, then the head 32000x4096, "
                    "5-bit log-scale ladder, 2 walk replicas alternating",
        "kernel": "k_q4tp_matvec", "launches": "q|k|v, o, gate|up, down per layer, head",
        "bytes_per_walk": int(nbytes), "us_per_walk": m["us"], "us_q1": m["us_q1"],
        "us_q3": m["us_q3"], "gbs": m["gbs"], "frac_hbm_peak": m["frac_hbm_peak"],
        "us_per_walk_one_launch_per_tensor": s["us"], "gbs_one_launch_per_tensor": s["gbs"],
        "ceiling_gbs": c["gbs"], "us_per_walk_ceiling": c["us"],
        "frac_of_ceiling": round(m["gbs"] / c["gbs"], 4),
    }


def section_mlx4(torch, q4, wl, rounds):
    """MLX affine 4-bit expert path at the single-token decode shapes (moeflux
    expert_forward.rs 4-bit experts, bf16 scale and bias per 64 weights), 128
    experts, top_k 8, m = 1: the fused gate/up + SiLU over expert blocks
    holding the 768x2048 gate and up matrices, the down-shaped 2048x768
    id-GEMV, and the latter in the 2-bit variant; 8 replicas rotate."""
    dev = torch.device("cuda")
    cfg = wl.CFG2
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.top_k
    draws = [wl.moe_activations(cfg, index=s) for s in range(64)]
    ids = [torch.from_numpy(a.ids).to(dev) for a in draws]
    uniq = [len(set(a.ids.tolist())) for a in draws]
    res = {}
    for name, n, k, outer, inner, nmat, bits in [("gate_up_silu", I, H, H, 0, 2, 4),
                                                 ("down", H, I, K * I, I, 1, 4),
                                                 ("down_2bit", H, I, K * I, I, 1, 2)]:
        mat = q4.mlx4_matrix_bytes(n, k) if bits == 4 else q4.mlx2_matrix_bytes(n, k)
        pb = n * k * bits // 8
        stride = nmat * mat
        offs = [(j * mat, j * mat + pb, j * mat + pb + n * k // 32) for j in range(nmat)]
        quantize = q4.mlx4_quantize if bits == 4 else q4.mlx2_quantize
        blobs = []
        for r in range(8):
            blob = torch.empty(E * stride, dtype=torch.uint8, device=dev)
            for j in range(nmat):
                w = wl.device_normal((E * n, k), cfg.w_std, seed=70000 + 100 * r + 10 * j + nmat + 3 * bits)
                po, so, bo = offs[j]
                for e in range(E):
                    b0 = e * stride
                    quantize(w[e * n:(e + 1) * n], blob[b0 + po:b0 + so],
                             blob[b0 + so:b0 + bo], blob[b0 + bo:b0 + po + mat], n, k)
                del w
            blobs.append(blob)
        x = wl.device_normal((K, k), 1.0, seed=79999)
        out = torch.empty(K, n, device=dev)
        torch.cuda.synchronize()

        def launch(i, n=n, k=k, stride=stride, outer=outer, inner=inner, blobs=blobs, x=x,
                   out=out, offs=offs, nmat=nmat, bits=bits):
            blob, d_ids = blobs[i % 8], ids[i % 64]
            if bits == 2:
                q4.mlx2_moe_id_gemv(blob, stride, *offs[0], x, d_ids, out, n, k, 1, K, outer,
                                    inner, E)
            elif nmat == 2:
                q4.mlx4_moe_gate_up_silu(blob, stride, offs[0], offs[1], x, d_ids, out, n, k, 1,
                                         K, outer, inner, E)
            else:
                q4.mlx4_moe_id_gemv(blob, stride, *offs[0], x, d_ids, out, n, k, 1, K, outer,
                                    inner, E)

        f = Figure(torch, name, launch, range(64), lambda i, stride=stride: uniq[i % 64] * stride)
        run_rounds([f], rounds)
        sm = f.summary()
        res[name] = {"us_per_launch": sm["us"], "us_q1": sm["us_q1"], "us_q3": sm["us_q3"],
                     "bytes_per_launch": sm["bytes_per_step"], "gbs": sm["gbs"],
                     "frac_hbm_peak": sm["frac_hbm_peak"]}
        del blobs
        torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, cfg, seconds):
    """The oracle's layer forward (routed FFN, shared expert, combine) on one
    id set: on one host thread, and with the layer's independent expert FFNs
    (each routed pair and the shared expert) on a pool of threads, whose
    results are the same bits (each pair is computed alone either way)."""
    import numpy as np

    import oracle
    a = wl.moe_activations(cfg, index=0)
    H, I, E, K, m = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.m
    experts = sorted(set(a.ids.tolist()))
    mb = oracle.q4k_matrix_bytes(I, H)
    stk = [np.zeros(E * mb, np.uint8) for _ in range(3)]
    for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
        for e in experts:
            stk[t][e * mb:(e + 1) * mb] = oracle.q4k_quantize(wl.expert_weight(cfg, t, e, rows, cols))
    sh = [oracle.q4k_quantize(wl.expert_weight(cfg, wl.T_SH_GATE + t, 0, rows, cols))
          for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)])]
    zeros = np.zeros(m, np.int32)
    layer_bytes = (len(experts) + 1) * 3 * mb
    ids = a.ids.reshape(m, K)

    def one_thread():
        _, _, _, eo = oracle.moe_expert_ffn(*stk, E, H, I, a.h_post, a.ids, m, K)
        _, _, _, so = oracle.moe_expert_ffn(*sh, 1, H, I, a.h_post, zeros, m, 1)
        return oracle.moe_combine_residual(a.h_mid, eo, a.route_w, so, a.shared_logit, H, m, K,
                                           cfg.shared_mode)

    share = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    n_tasks = m * K + 1
    threads = max(1, min(n_tasks, share, 16))
    pool = cf.ThreadPoolExecutor(max_workers=threads)

    def pair(p):
        t, s = divmod(p, K)
        if p == m * K:
            return oracle.moe_expert_ffn(*sh, 1, H, I, a.h_post, zeros, m, 1)[3]
        return oracle.moe_expert_ffn(*stk, E, H, I, a.h_post[t:t + 1], ids[t, s:s + 1], 1, 1)[3]

    def all_cores():
        res = list(pool.map(pair, range(n_tasks)))
        eo = np.concatenate(res[:m * K])
        return oracle.moe_combine_residual(a.h_mid, eo, a.route_w, res[-1], a.shared_logit, H,
                                           m, K, cfg.shared_mode)

    assert np.array_equal(one_thread().view(np.uint32), all_cores().view(np.uint32))
    out = {}
    for name, fn in (("one_thread", one_thread), ("all_cores", all_cores)):
        n = 0
        t0 = time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds or n >= 10000:
                break
        out[name] = (n, el)
    pool.shutdown()
    n1, e1 = out["one_thread"]
    na, ea = out["all_cores"]
    return {
        "value": round(layer_bytes * na / ea / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{na} layer forwards of {cfg.name} (id set 0: {len(experts)} routed + 1 "
                  f"shared expert, oracle-encoded weights) in {ea:.1f} s on {threads} threads "
                  f"(one per expert FFN), {ea / na * 1e6:.0f} us/layer",
        "one_thread": {"value": round(layer_bytes * n1 / e1 / 1e9, 4), "unit": "GB/s",
                       "us_per_layer": round(e1 / n1 * 1e6, 1), "layers": n1},
        "all_cores": {"value": round(layer_bytes * na / ea / 1e9, 4), "unit": "GB/s",
                      "us_per_layer": round(ea / na * 1e6, 1), "layers": na,
                      "threads": threads},
        "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity": share},
    }


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(path):
    """HBM bytes per launch of the dominant kernel from a profile summary
    (lines `traffic_bytes_per_launch: N`, `source_files: F...` and
    `source_sha256: H`), or None when absent or taken on other sources."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for ln in text.splitlines():
        if ":" in ln:
            k, v = ln.split(":", 1)
            fields[k.strip().strip("-* `")] = v.strip().strip("`")
    files = fields.get("source_files", "").split()
    try:
        if not files or fields.get("source_sha256") != source_digest(files):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(torch, mib):
    """A plain device copy of a known size: the yardstick for HBM counters."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 10}), flush=True)


def eager(torch, fn, steps, warmup):
    """fn(i) launched one by one (counter passes)."""
    for i in range(warmup):
        fn(steps + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32, help="timed layers per headline round")
    ap.add_argument("--warmup", type=int, default=16, help="untimed layers before the rounds")
    ap.add_argument("--rounds", type=int, default=5, help="timed rounds per figure")
    ap.add_argument("--replicas", type=int, default=16, help="weight replicas rotated")
    ap.add_argument("--id-sets", type=int, default=128,
                    help="routing draws rotated (warm-up draws are disjoint from the timed "
                         "ones while steps + warmup <= id-sets)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="per CPU-baseline variant")
    ap.add_argument("--only", default="", help="comma list of sections: m1,m16,sweep,cfg4,walk,"
                                               "mlx4,cpu (default: all)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the headline and m16 kernels one by one, no graphs (counters)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter yardstick)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the path has no multi-GPU mode (asked for --gpus "
              f"{args.gpus}).", file=sys.stderr)
        sys.exit(2)
    want = set(s for s in args.only.split(",") if s) or \
        {"m1", "m16", "sweep", "cfg4", "walk", "mlx4", "cpu"}

    import torch

    import bit_quantized_moe_superblock_amd as q4
    from bit_quantized_moe_superblock_amd import workloads as wl
    q4._lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        copy_calibration(torch, args.calibrate_copy)
        return

    K, W, R = args.steps, args.warmup, args.rounds
    t_start = time.perf_counter()
    log(f"encoding {args.replicas} replicas of the hidden-2048 layer")
    m1 = Moe(torch, q4, wl, wl.CFG2, args.replicas, args.id_sets)
    line = {}
    if args.eager:
        for name, mo in (("m1", m1),
                         ("m16", Moe(torch, q4, wl, wl.CFG3, 0, args.id_sets, m1.stacks,
                                     m1.shared))):
            for kern in (mo.layer, mo.gate_up, mo.down):
                sec = eager(torch, kern, K, W)
                log(f"{name} {kern.__name__}: {sec / K * 1e6:.2f} us per call (eager)")
        return

    # ---- headline: m = 1 layer, its gate/up launch, and the ceiling
    timed = list(range(K))
    warm = list(range(K, K + W)) if W else None
    figs = {"m1": Figure(torch, "m1 layer", m1.layer, timed, m1.bytes_of(3), warm),
            "m1_gu": Figure(torch, "m1 gate/up", m1.gate_up, range(64), m1.bytes_of(2)),
            "m1_norm": Figure(torch, "m1 layer + rmsnorm", m1.layer_norm, range(64),
                              m1.bytes_of(3)),
            "m1_ceil": Figure(torch, "m1 ceiling", m1.ceiling([0, 1, 2]), range(64),
                              m1.bytes_of(3)),
            "m1_gu_ceil": Figure(torch, "m1 gate/up ceiling", m1.ceiling([0, 1]), range(64),
                                 m1.bytes_of(2))}
    m16 = None
    if "m16" in want or "sweep" in want:
        m16 = Moe(torch, q4, wl, wl.CFG3, 0, args.id_sets, m1.stacks, m1.shared)
    if "m16" in want:
        figs.update({
            "m16": Figure(torch, "m16 layer", m16.layer, range(32), m16.bytes_of(3)),
            "m16_norm": Figure(torch, "m16 layer + rmsnorm", m16.layer_norm, range(32),
                               m16.bytes_of(3)),
            "m16_gu": Figure(torch, "m16 gate/up", m16.gate_up, range(32), m16.bytes_of(2)),
            "m16_down": Figure(torch, "m16 down", m16.down, range(32),
                               lambda i: len(m16.unique[i % len(m16.sets)]) * m16.mat),
            "m16_ceil": Figure(torch, "m16 ceiling", m16.ceiling([0, 1, 2]), range(32),
                               m16.bytes_of(3)),
            "m16_gu_ceil": Figure(torch, "m16 gate/up ceiling", m16.ceiling([0, 1]), range(32),
                                  m16.bytes_of(2))})
    sweep = {}
    if "sweep" in want:
        import dataclasses
        flags = {"auto": q4.Q4K_BUCKET_AUTO, "token": q4.Q4K_BUCKET_OFF,
                 "matrix_cores": q4.Q4K_BUCKET_ON,
                 "vector_bucketed": q4.Q4K_BUCKET_ON | q4.Q4K_SCHED_VECTOR}
        for m in (1, 2, 4, 8, 16):
            cfg = wl.CFG2 if m == 1 else dataclasses.replace(
                wl.CFG3, name=f"decode_m{m}_zipf", m=m)
            mo = m1 if m == 1 else (m16 if m == 16 else
                                    Moe(torch, q4, wl, cfg, 0, args.id_sets, m1.stacks, m1.shared))
            for fname, fl in flags.items():
                figs[f"sweep_{m}_{fname}"] = Figure(
                    torch, f"m={m} {fname}", (lambda i, mo=mo, fl=fl: mo.layer(i, fl)),
                    range(32), mo.bytes_of(3))
            sweep[m] = mo
    log(f"timing {len(figs)} figures, {R} rounds round-robin")
    run_rounds(list(figs.values()), R)
    S = {k: f.summary() for k, f in figs.items()}

    hl = S["m1"]
    gu, gu_ceil = S["m1_gu"], S["m1_gu_ceil"]
    per_round = [s / K * 1e6 for s in figs["m1"].secs]
    line.update({
        "metric": METRIC,
        "value": hl["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(hl["us"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "single-token MoE FFN decode layer: hidden 2048, expert intermediate "
                        "768, 128 experts, top_k 8, m=1, Q4_K weights N(0,0.02^2), "
                        "sigmoid-gated shared expert, weighted residual combine",
            "hidden": 2048, "inter": 768, "experts": 128, "top_k": 8, "m": 1,
            "weight_replicas": args.replicas, "id_sets": args.id_sets,
            "launch": f"HIP graph of {K} layers per round, {R} rounds",
            "bytes_per_layer": hl["bytes_per_step"],
        },
        "us_per_layer": hl["us"], "us_per_layer_q1": hl["us_q1"],
        "us_per_layer_q3": hl["us_q3"],
        "us_per_layer_rounds": [round(x, 3) for x in per_round],
        "frac_hbm_peak": hl["frac_hbm_peak"],
        "ceiling_gbs": S["m1_ceil"]["gbs"],
        "us_per_layer_with_next_rmsnorm": S["m1_norm"]["us"],
        "roofline": {
            "bound": "hbm",
            "kernel": "fused gate/up id-GEMV + SiLU (routed + shared experts)",
            "achieved": gu["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gu["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(TRAFFIC_PROFILE),
            "us_per_launch": gu["us"], "us_q1": gu["us_q1"], "us_q3": gu["us_q3"],
            "bytes_per_launch": gu["bytes_per_step"],
            "ceiling": gu_ceil["gbs"],
            "frac_of_ceiling": round(gu["gbs"] / gu_ceil["gbs"], 4),
        },
    })
    if "m16" in want:
        L, G, D = S["m16"], S["m16_gu"], S["m16_down"]
        line["m16"] = {
            "workload": "same layer, m=16 tokens, Zipf(1.1) routing, bucketed",
            "value": L["gbs"], "unit": "GB/s", "us_per_layer": L["us"],
            "us_q1": L["us_q1"], "us_q3": L["us_q3"], "frac_hbm_peak": L["frac_hbm_peak"],
            "bytes_per_layer": L["bytes_per_step"], "ceiling_gbs": S["m16_ceil"]["gbs"],
            "us_per_layer_with_next_rmsnorm": S["m16_norm"]["us"],
            "roofline": {"bound": "hbm", "kernel": "bucketed gate/up + SiLU (matrix cores, "
                                                   "pre-built buckets)",
                         "achieved": G["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(G["gbs"] / HBM_PEAK_GBS, 4), "us_per_launch": G["us"],
                         "bytes_per_launch": G["bytes_per_step"],
                         "ceiling": S["m16_gu_ceil"]["gbs"],
                         "frac_of_ceiling": round(G["gbs"] / S["m16_gu_ceil"]["gbs"], 4)},
            "down": {"us_per_launch": D["us"], "gbs": D["gbs"],
                     "bytes_per_launch": D["bytes_per_step"]},
        }
    if sweep:
        t1 = S["sweep_1_auto"]["us"]
        rows = {}
        for m in sweep:
            rows[str(m)] = {f: {"us": S[f"sweep_{m}_{f}"]["us"], "gbs": S[f"sweep_{m}_{f}"]["gbs"]}
                            for f in ("auto", "token", "matrix_cores", "vector_bucketed")}
            rows[str(m)]["scaling_vs_m1"] = round(S[f"sweep_{m}_auto"]["us"] / t1, 3)
        t16 = S["sweep_16_auto"]["us"]
        line["sweep"] = {
            "workload": "the hidden-2048 layer at m tokens (m=1: uniform distinct ids; m>1: "
                        "Zipf(1.1)), us per layer and unique-byte GB/s per schedule",
            "m": rows, "auto_bucket_min_tokens": q4.Q4K_AUTO_BUCKET_MIN_TOKENS,
            "batches_well": {"m16_us": t16, "bound_us": round(0.6 * 16 * t1, 3),
                             "ok": t16 < 0.6 * 16 * t1},
        }
    del figs
    torch.cuda.empty_cache()

    if "cfg4" in want:
        log("cfg4: encoding one 6.3 GB layer (256 experts, hidden 7168, inter 2048)")
        c4 = {}
        big = Moe(torch, q4, wl, wl.CFG4_M1, 1, 32, shared_replicas=8)
        big32 = Moe(torch, q4, wl, wl.CFG4_M32, 0, 8, big.stacks, big.shared)
        f4 = {"m1": Figure(torch, "cfg4 m1", big.layer, range(32), big.bytes_of(3)),
              "m1_ceil": Figure(torch, "cfg4 m1 ceiling", big.ceiling([0, 1, 2]), range(32),
                                big.bytes_of(3)),
              "m32": Figure(torch, "cfg4 m32", big32.layer, range(8), big32.bytes_of(3)),
              "m32_ceil": Figure(torch, "cfg4 m32 ceiling", big32.ceiling([0, 1, 2]), range(8),
                                 big32.bytes_of(3))}
        # the dominant launch of each (gate/up + SiLU) and the plain read of its bytes
        for k, mo, n in (("m1", big, 32), ("m32", big32, 8)):
            f4[k + "_gu"] = Figure(torch, f"cfg4 {k} gate/up", mo.gate_up, range(n),
                                   mo.bytes_of(2))
            f4[k + "_gu_ceil"] = Figure(torch, f"cfg4 {k} gate/up ceiling", mo.ceiling([0, 1]),
                                        range(n), mo.bytes_of(2))
        run_rounds(list(f4.values()), R)
        for k, kern in (("m1", "fused gate/up id-GEMV + SiLU (vector units, pair mode)"),
                        ("m32", "bucketed gate/up + SiLU (matrix cores, pre-built buckets)")):
            s, c = f4[k].summary(), f4[k + "_ceil"].summary()
            g, gc = f4[k + "_gu"].summary(), f4[k + "_gu_ceil"].summary()
            c4[k] = {"us_per_layer": s["us"], "us_q1": s["us_q1"], "us_q3": s["us_q3"],
                     "gbs": s["gbs"], "frac_hbm_peak": s["frac_hbm_peak"],
                     "bytes_per_layer": s["bytes_per_step"], "ceiling_gbs": c["gbs"],
                     "roofline": {"bound": "hbm", "kernel": kern, "achieved": g["gbs"],
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(g["gbs"] / HBM_PEAK_GBS, 4),
                                  "us_per_launch": g["us"], "us_q1": g["us_q1"],
                                  "us_q3": g["us_q3"], "bytes_per_launch": g["bytes_per_step"],
                                  "ceiling": gc["gbs"],
                                  "frac_of_ceiling": round(g["gbs"] / gc["gbs"], 4)}}
        c4["workload"] = ("large-expert layer: hidden 7168, inter 2048, 256 experts, top_k 8, "
                          "unscaled shared expert (8 replicas); m=1 over 32 uniform draws of "
                          "distinct experts (a graph reads ~4 GB), m=32 over 8 draws")
        line["cfg4"] = c4
        del f4, big, big32
        torch.cuda.empty_cache()
    if "walk" in want:
        log("walk: encoding 8 layers + head, 2 replicas")
        line["walk"] = section_walk(torch, q4, wl, 8, R)
        torch.cuda.empty_cache()
    if "mlx4" in want:
        line["mlx4"] = section_mlx4(torch, q4, wl, R)
    if "cpu" in want:
        log("cpu oracle baseline")
        line["cpu_baseline"] = cpu_baseline(wl, wl.CFG2, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    log(f"done in {time.perf_counter() - t_start:.0f} s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
