#!/usr/bin/env python3
"""Benchmark of one Q4_K MoE decode layer on one MI355X.

A step is one whole MoE layer on one batch of synthetic decode input:
expert bucketing (when m > 1), the fused gate/up id-GEMV with SiLU over the
routed experts, the down id-GEMV, the shared expert's gate/up and down, and the
weighted residual combine -- every kernel of the hot path.

Workload (the throughput line): hidden 2048, expert intermediate 768, 128
experts, top_k 8, m = 1 token, sigmoid-gated shared expert of the same shape
(a Qwen3-30B-A3B-class layer; ferrum-kernels q4_k_moe_id_gemv_batched.rs
microbench shape, moeflux expert_forward.rs combine).  A second object reports
m = 16 tokens with Zipf(1.1) routing, where bucketing lets tokens that share
an expert read it once.

Cold-cache protocol: the weights exist as R independent replicas (each a full
128-expert layer, 340 MB) and G id sets; consecutive steps use different
replicas, so a graph replay of G steps touches far more distinct bytes than the
256 MB Infinity Cache holds.  Steps are captured into HIP graphs (one launch
per G layers) so host overhead does not pace the GPU.

value = unique expert-weight bytes read per layer (distinct routed experts
plus the shared expert, three matrices each) / wall time per layer.
roofline = the layer's first kernel (fused gate/up + SiLU over the routed
experts with the shared expert in the same launch), timed by a graph of only
its launches over the same rotation (in-graph launches run back to back, so
the per-launch time is the kernel's duration), against the 8 TB/s HBM peak.
cpu_baseline = the CPU oracle's layer forward, single-threaded, on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE id-GEMV effective HBM GB/s (% of peak) + µs/MoE layer at M=1,16"
HBM_PEAK_GBS = 8000.0
# FETCH_SIZE + WRITE_SIZE of the dominant kernel, scaled by a plain copy
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gate_up_silu_m1_hbm_traffic.md")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Layer:
    """Device-resident weight replicas and per-step inputs of one MoE workload."""

    def __init__(self, torch, q4, wl, cfg, replicas, stacks=None):
        self.torch, self.q4, self.cfg = torch, q4, cfg
        dev = torch.device("cuda")
        H, I, E = cfg.hidden, cfg.inter, cfg.num_experts
        self.mat_bytes = q4.q4k_matrix_bytes(I, H)           # one expert matrix
        self.expert_bytes = 3 * self.mat_bytes
        if stacks is None:
            stacks = []
            for r in range(replicas):
                st = []
                for t, (rows, cols, n_exp) in enumerate([(I, H, E), (I, H, E), (H, I, E),
                                                          (I, H, 1), (I, H, 1), (H, I, 1)]):
                    w = wl.device_normal((n_exp * rows, cols), cfg.w_std, seed=1000 * r + t)
                    b = torch.empty(n_exp * q4.q4k_matrix_bytes(rows, cols), dtype=torch.uint8,
                                    device=dev)
                    q4.q4k_quantize(w, b, n_exp * rows, cols)
                    del w
                    st.append(b)
                stacks.append(st)
            torch.cuda.synchronize()
        self.stacks = stacks

    def inputs(self, wl, n_sets):
        torch, cfg = self.torch, self.cfg
        dev = torch.device("cuda")
        self.sets = []
        self.unique = []
        for s in range(n_sets):
            a = wl.moe_activations(cfg, index=s)
            self.sets.append(dict(
                h_post=torch.from_numpy(a.h_post).to(dev),
                h_mid=torch.from_numpy(a.h_mid).to(dev),
                ids=torch.from_numpy(a.ids).to(dev),
                route_w=torch.from_numpy(a.route_w).to(dev),
                logit=torch.from_numpy(a.shared_logit).to(dev)))
            self.unique.append(len(set(a.ids.tolist())))
        m, K, H, I = cfg.m, cfg.top_k, cfg.hidden, cfg.inter
        P = m * K
        self.act = torch.empty(P, I, device=dev)
        self.eo = torch.empty(P, H, device=dev)
        self.s_act = torch.empty(m, I, device=dev)
        self.s_out = torch.empty(m, H, device=dev)
        self.out = torch.empty(m, H, device=dev)
        self.normed = torch.empty(m, H, device=dev)
        self.norm_w = torch.ones(H, device=dev).to(torch.bfloat16)   # next layer's norm weight
        self.lwsb = self.q4.moe_layer_workspace_bytes(H, I, cfg.num_experts, m, K)
        self.lws = torch.zeros(self.lwsb, dtype=torch.uint8, device=dev)   # barrier words zero
        self.wsb = self.q4.moe_bucket_workspace_bytes(P, cfg.num_experts)
        # one bucket workspace per id set, filled here, so a graph of gate/up
        # launches alone still reads the buckets of its own routing
        self.ws_sets = []
        for x in self.sets:
            ws = torch.empty(self.wsb, dtype=torch.uint8, device=dev)
            if m > 1:
                self.q4.moe_bucket(x["ids"], P, cfg.num_experts, ws, self.wsb)
            self.ws_sets.append(ws)
        torch.cuda.synchronize()

    def step_of(self, i):
        return i % len(self.stacks), i % len(self.sets)

    def bucketed(self):
        return self.cfg.m > 2    # moe_layer_forward's AUTO rule

    def gate_up(self, i):
        """The layer's first kernel alone: fused gate/up + SiLU over the routed
        pairs with the shared expert in the same launch (buckets pre-built)."""
        q4, cfg = self.q4, self.cfg
        r, s = self.step_of(i)
        st, x = self.stacks[r], self.sets[s]
        flag = q4.Q4K_BUCKET_PREBUILT if self.bucketed() else q4.Q4K_BUCKET_OFF
        q4.q4k_moe_gate_up_silu(st[0], st[1], x["h_post"], x["ids"], self.act, cfg.inter,
                                cfg.hidden, cfg.m, cfg.top_k, cfg.hidden, 0, cfg.num_experts,
                                st[3], st[4], self.s_act, flag, self.ws_sets[s], self.wsb)

    def layer(self, i):
        """One whole MoE layer (every kernel of the hot path)."""
        q4, cfg = self.q4, self.cfg
        r, s = self.step_of(i)
        st, x = self.stacks[r], self.sets[s]
        q4.moe_layer_forward(st[0], st[1], st[2], st[3], st[4], st[5], x["h_post"], x["h_mid"],
                             x["ids"], x["route_w"], x["logit"], self.out, cfg.hidden, cfg.inter,
                             cfg.num_experts, cfg.m, cfg.top_k, cfg.shared_mode,
                             q4.Q4K_BUCKET_AUTO, self.lws, self.lwsb)

    def layer_norm(self, i):
        """The layer with the next layer's input RMSNorm chained on."""
        q4, cfg = self.q4, self.cfg
        r, s = self.step_of(i)
        st, x = self.stacks[r], self.sets[s]
        q4.moe_layer_forward_rmsnorm(st[0], st[1], st[2], st[3], st[4], st[5], x["h_post"],
                                     x["h_mid"], x["ids"], x["route_w"], x["logit"], self.out,
                                     self.norm_w, 1e-6, self.normed, cfg.hidden, cfg.inter,
                                     cfg.num_experts, cfg.m, cfg.top_k, cfg.shared_mode,
                                     q4.Q4K_BUCKET_AUTO, self.lws, self.lwsb)

    def layer_bytes(self, i):
        r, s = self.step_of(i)
        return (self.unique[s] + 1) * self.expert_bytes

    def gate_up_bytes(self, i):
        r, s = self.step_of(i)
        return (self.unique[s] + 1) * 2 * self.mat_bytes


def capture(torch, fn, n):
    """HIP graph of fn(0..n-1), warmed up on a side stream first."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, replays, warmup):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def largest_divisor_at_most(k, cap):
    for g in range(min(k, cap), 0, -1):
        if k % g == 0:
            return g
    return 1


def time_eager(torch, fn, steps, warmup, start=0):
    """fn(i) launched one by one (no graph), timed with events on the launch
    stream; used under hardware-counter profiling."""
    for i in range(warmup):
        fn(start + i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(start + warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3, time.perf_counter() - t0


def run_walk(torch, q4, wl, replicas, walks, warmup):
    """The dense Q4TiledP decode walk (one layer's q, k, v, o, gate, up and down
    matvecs, then the head) over `replicas` device-encoded copies of its
    tensors, rotated so that consecutive walks do not find them in cache.
    Timed twice: one launch per tensor, and with q|k|v and gate|up each merged
    into one launch.  Returns (us per walk merged, us per walk one launch per
    tensor, tensor bytes)."""
    dev = torch.device("cuda")
    shapes = [(rows, cols) for _, rows, cols, _ in wl.walk_tensors(1, True)]
    reps = []
    for r in range(replicas):
        ts = []
        for i, (rows, cols) in enumerate(shapes):
            w = wl.device_normal((rows, cols), 0.02, seed=50000 + 100 * r + i)
            t = torch.empty(q4.q4tp_tensor_bytes(rows, cols), dtype=torch.uint8, device=dev)
            q4.q4tp_quantize(w, t, rows, cols)
            del w
            ts.append(t)
        reps.append(ts)
    x = wl.device_normal((wl.WALK_X_LEN,), 1.0, seed=59999)
    ys = [torch.empty(rows, device=dev) for rows, _ in shapes]
    torch.cuda.synchronize()

    def walk(i):
        ts = reps[i % replicas]
        for (rows, cols), t, y in zip(shapes, ts, ys):
            q4.q4tp_matvec(t, x, y, rows, cols)

    # q|k|v, o, gate|up, down, head
    groups = [[0, 1, 2], [3], [4, 5], [6], [7]]
    ym = [torch.empty(sum(shapes[j][0] for j in grp), device=dev) for grp in groups]

    def walk_merged(i):
        ts = reps[i % replicas]
        for grp, y in zip(groups, ym):
            q4.q4tp_matvec_multi([ts[j] for j in grp], [shapes[j][0] for j in grp], x, y,
                                 shapes[grp[0]][1])

    # concurrent mode (cortiq-engine mv_lab.rs, mode 'c'): the tensors of a
    # group run on parallel graph branches, joined before the next group
    side = [torch.cuda.Stream() for _ in range(3)]   # default priority

    def walk_concurrent(i):
        ts = reps[i % replicas]
        main = torch.cuda.current_stream()
        for grp in groups:
            if len(grp) == 1:
                j = grp[0]
                q4.q4tp_matvec(ts[j], x, ys[j], *shapes[j])
                continue
            for b, j in enumerate(grp):
                side[b].wait_stream(main)
                with torch.cuda.stream(side[b]):
                    q4.q4tp_matvec(ts[j], x, ys[j], *shapes[j], stream=side[b])
            for b in range(len(grp)):
                main.wait_stream(side[b])

    g = capture(torch, walk, walks)
    sec, _ = time_graph(torch, g, 4, warmup)
    gm = capture(torch, walk_merged, walks)
    sec_m, _ = time_graph(torch, gm, 4, warmup)
    gc = capture(torch, walk_concurrent, walks)
    sec_c, _ = time_graph(torch, gc, 4, warmup)
    nbytes = sum(q4.q4tp_tensor_bytes(rows, cols) for rows, cols in shapes)
    return (sec_m / (4 * walks) * 1e6, sec / (4 * walks) * 1e6, nbytes,
            sec_c / (4 * walks) * 1e6)


def run_mlx4(torch, q4, wl, replicas, launches, warmup):
    """The MLX affine 4-bit expert path (moeflux expert_forward.rs 4-bit
    experts, bf16 scale and bias per 64 weights) at the single-token decode
    shapes, 128 experts, top_k 8, m = 1: the fused gate/up + SiLU launch over
    expert blocks holding the gate and up matrices (768 x 2048 each, one
    activation row per token), and the down-shaped id-GEMV (2048 x 768, one
    row per pair), that one also in the 2-bit variant (moeflux's g_use_2bit
    layout).  Each replica is a full 128-expert stack, device-encoded;
    launches rotate over replicas and 64 routing draws.  Returns
    {name: (us per launch, unique weight bytes per launch)}."""
    dev = torch.device("cuda")
    cfg = wl.CFG2
    E, H, I, K = cfg.num_experts, cfg.hidden, cfg.inter, cfg.top_k
    sets = [wl.moe_activations(cfg, index=s) for s in range(64)]
    ids = [torch.from_numpy(a.ids).to(dev) for a in sets]
    uniq = [len(set(a.ids.tolist())) for a in sets]
    res = {}
    for name, n, k, outer, inner, nmat, bits in [("gate_up_silu", I, H, H, 0, 2, 4),
                                                 ("down", H, I, K * I, I, 1, 4),
                                                 ("down_2bit", H, I, K * I, I, 1, 2)]:
        mat = q4.mlx4_matrix_bytes(n, k) if bits == 4 else q4.mlx2_matrix_bytes(n, k)
        pb = n * k * bits // 8                   # packed bytes of a matrix
        stride = nmat * mat
        # matrix j of a block: packed | scales | biases at j * mat
        offs = [(j * mat, j * mat + pb, j * mat + pb + n * k // 32) for j in range(nmat)]
        quantize = q4.mlx4_quantize if bits == 4 else q4.mlx2_quantize
        blobs = []
        for r in range(replicas):
            blob = torch.empty(E * stride, dtype=torch.uint8, device=dev)
            for j in range(nmat):
                w = wl.device_normal((E * n, k), cfg.w_std,
                                     seed=70000 + 100 * r + 10 * j + nmat + 3 * bits)
                po, so, bo = offs[j]
                for e in range(E):
                    b0 = e * stride
                    quantize(w[e * n:(e + 1) * n], blob[b0 + po:b0 + so],
                             blob[b0 + so:b0 + bo], blob[b0 + bo:b0 + po + mat], n, k)
                del w
            blobs.append(blob)
        x = wl.device_normal((K, k), 1.0, seed=79999)   # row 0 for gate/up, 8 rows for down
        out = torch.empty(K, n, device=dev)
        torch.cuda.synchronize()

        def launch(i, n=n, k=k, stride=stride, outer=outer, inner=inner, blobs=blobs, x=x,
                   out=out, offs=offs, nmat=nmat, bits=bits):
            blob, d_ids = blobs[i % replicas], ids[i % 64]
            if bits == 2:
                q4.mlx2_moe_id_gemv(blob, stride, *offs[0], x, d_ids, out, n, k, 1, K, outer,
                                    inner, E)
            elif nmat == 2:
                q4.mlx4_moe_gate_up_silu(blob, stride, offs[0], offs[1], x, d_ids, out, n, k, 1,
                                         K, outer, inner, E)
            else:
                q4.mlx4_moe_id_gemv(blob, stride, *offs[0], x, d_ids, out, n, k, 1, K, outer,
                                    inner, E)

        g = capture(torch, launch, launches)
        sec, _ = time_graph(torch, g, 4, warmup)
        nbytes = sum(uniq[i % 64] for i in range(launches)) / launches * stride
        res[name] = (sec / (4 * launches) * 1e6, nbytes)
        del blobs
    return res


def run_workload(torch, q4, wl, cfg, args, stacks=None):
    """Times exactly args.steps layers (and, separately, args.steps launches
    of the layer's first kernel) after args.warmup untimed ones."""
    steps = args.steps
    layer = Layer(torch, q4, wl, cfg, args.replicas, stacks)
    layer.inputs(wl, args.id_sets)
    if args.eager:
        log(f"{cfg.name}: {steps} eager layers timed")
        gpu_s, wall_s = time_eager(torch, layer.layer, steps, args.warmup)
        gu_s, _ = time_eager(torch, layer.gate_up, steps, args.warmup)
        norm_s, _ = time_eager(torch, layer.layer_norm, steps, args.warmup)
        G, warm = 1, args.warmup
        idx = range(steps)
        mode = "eager launches"
    else:
        G = largest_divisor_at_most(steps, args.group)
        replays = steps // G
        warm_replays = max(1, -(-args.warmup // G))
        warm = warm_replays * G
        log(f"{cfg.name}: capturing {G} layers per graph, {replays} replays timed")
        g_layer = capture(torch, layer.layer, G)
        gpu_s, wall_s = time_graph(torch, g_layer, replays, warm_replays)
        g_gu = capture(torch, layer.gate_up, G)
        gu_s, _ = time_graph(torch, g_gu, replays, warm_replays)
        g_norm = capture(torch, layer.layer_norm, G)
        norm_s, _ = time_graph(torch, g_norm, replays, warm_replays)
        del g_layer, g_gu, g_norm
        idx = [i % G for i in range(steps)]
        mode = f"HIP graphs of {G} layers"
    total_bytes = sum(layer.layer_bytes(i) for i in idx)
    gu_bytes = sum(layer.gate_up_bytes(i) for i in idx)
    res = dict(steps=steps, warmup=warm, gpu_s=gpu_s, wall_s=wall_s, mode=mode, group=G,
               us_per_layer=gpu_s / steps * 1e6, gbs=total_bytes / gpu_s / 1e9,
               bytes_per_layer=total_bytes / steps, gate_up_us=gu_s / steps * 1e6,
               gate_up_gbs=gu_bytes / gu_s / 1e9, gate_up_bytes=gu_bytes / steps,
               us_per_layer_rmsnorm=norm_s / steps * 1e6)
    return res, layer.stacks


def copy_calibration(torch, mib):
    """A plain device-to-device copy of a known size, the yardstick that the
    FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 10}), flush=True)


def source_digest(files):
    """sha256 over the named kernel sources (paths relative to the repository
    root): a stored counter figure is reported only while the code it was
    taken from is unchanged."""
    import hashlib
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(path):
    """HBM bytes per launch of the dominant kernel from a profile summary
    (lines `traffic_bytes_per_launch: N`, `source_files: F...` and
    `source_sha256: H`), or None when the summary is absent or was taken on
    other kernel sources."""
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
    except OSError:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, cfg, seconds):
    """The oracle's layer forward (routed FFN, shared expert, combine), one
    thread, repeated on one id set until `seconds` of work is done."""
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
    n = 0
    t0 = time.perf_counter()
    while True:
        _, _, _, eo = oracle.moe_expert_ffn(*stk, E, H, I, a.h_post, a.ids, m, K)
        _, _, _, so = oracle.moe_expert_ffn(*sh, 1, H, I, a.h_post, zeros, m, 1)
        oracle.moe_combine_residual(a.h_mid, eo, a.route_w, so, a.shared_logit, H, m, K,
                                    cfg.shared_mode)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 10000:
            break
    layer_bytes = (len(experts) + 1) * 3 * mb
    return dict(value=round(layer_bytes * n / el / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{n} layer forwards of {cfg.name} (id set 0: {len(experts)} routed + 1 "
                       f"shared expert, oracle-encoded weights), {el:.1f} s, one thread; "
                       f"{el / n * 1e6:.0f} us/layer")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024, help="timed layers")
    ap.add_argument("--warmup", type=int, default=128, help="untimed layers")
    ap.add_argument("--group", type=int, default=64,
                    help="layers captured per graph (a divisor of --steps)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel directly instead of through graphs")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter yardstick)")
    ap.add_argument("--replicas", type=int, default=16, help="weight replicas rotated")
    ap.add_argument("--id-sets", type=int, default=64, help="routing draws rotated")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-m16", action="store_true")
    ap.add_argument("--no-walk", action="store_true")
    ap.add_argument("--no-mlx4", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: every box here has one MI355X and this path has no "
              f"multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_moe_superblock_amd as q4
    from bit_quantized_moe_superblock_amd import workloads as wl
    q4._lib.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        copy_calibration(torch, args.calibrate_copy)
        return

    res1, stacks = run_workload(torch, q4, wl, wl.CFG2, args)
    log(f"m=1: {res1['us_per_layer']:.2f} us/layer, {res1['gbs']:.1f} GB/s; gate/up "
        f"{res1['gate_up_us']:.2f} us, {res1['gate_up_gbs']:.1f} GB/s; with the next "
        f"layer's RMSNorm {res1['us_per_layer_rmsnorm']:.2f} us")
    res16 = None
    if not args.no_m16:
        res16, _ = run_workload(torch, q4, wl, wl.CFG3, args, stacks)
        log(f"m=16: {res16['us_per_layer']:.2f} us/layer, {res16['gbs']:.1f} GB/s; gate/up "
            f"{res16['gate_up_us']:.2f} us, {res16['gate_up_gbs']:.1f} GB/s; with the next "
            f"layer's RMSNorm {res16['us_per_layer_rmsnorm']:.2f} us")
    walk_us = None
    if not args.no_walk:
        walk_us, walk_single_us, walk_bytes, walk_conc_us = run_walk(torch, q4, wl, 2, 32, 1)
        log(f"walk: {walk_us:.2f} us/walk merged ({walk_bytes / walk_us / 1e3:.1f} GB/s), "
            f"{walk_single_us:.2f} us one launch per tensor, {walk_conc_us:.2f} us concurrent "
            f"groups")
    mlx = None
    if not args.no_mlx4:
        mlx = run_mlx4(torch, q4, wl, 8, 64, 1)
        log("mlx4: " + ", ".join(f"{k} {us:.2f} us ({b / us / 1e3:.1f} GB/s)"
                                 for k, (us, b) in mlx.items()))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, wl.CFG2, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']} GB/s")

    cfg = wl.CFG2
    line = {
        "metric": METRIC,
        "value": round(res1["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": res1["steps"],
        "warmup": res1["warmup"],
        "ms_per_step": round(res1["us_per_layer"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "single-token MoE FFN decode layer: hidden 2048, expert intermediate 768, "
                        "128 experts, top_k 8, m=1, Q4_K weights N(0,0.02^2), sigmoid-gated "
                        "shared expert, weighted residual combine",
            "hidden": cfg.hidden, "inter": cfg.inter, "experts": cfg.num_experts,
            "top_k": cfg.top_k, "m": cfg.m, "weight_replicas": args.replicas,
            "id_sets": args.id_sets, "launch": res1["mode"],
            "bytes_per_layer": int(res1["bytes_per_layer"]),
        },
        "us_per_layer": round(res1["us_per_layer"], 3),
        "us_per_layer_with_next_rmsnorm": round(res1["us_per_layer_rmsnorm"], 3),
        "frac_hbm_peak": round(res1["gbs"] / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "fused gate/up id-GEMV + SiLU (routed + shared experts)",
            "achieved": round(res1["gate_up_gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(res1["gate_up_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(TRAFFIC_PROFILE),
            "us_per_launch": round(res1["gate_up_us"], 3),
            "bytes_per_launch": int(res1["gate_up_bytes"]),
        },
        "cpu_baseline": cpu,
    }
    if res16 is not None:
        line["m16"] = {
            "workload": "same layer, m=16 tokens, Zipf(1.1) routing, bucketed",
            "value": round(res16["gbs"], 2), "unit": "GB/s",
            "us_per_layer": round(res16["us_per_layer"], 3),
            "us_per_layer_with_next_rmsnorm": round(res16["us_per_layer_rmsnorm"], 3),
            "frac_hbm_peak": round(res16["gbs"] / HBM_PEAK_GBS, 4),
            "bytes_per_layer": int(res16["bytes_per_layer"]),
            "gate_up_gbs": round(res16["gate_up_gbs"], 2),
            "gate_up_us": round(res16["gate_up_us"], 3),
        }
    if mlx is not None:
        line["mlx4"] = {
            "workload": "MLX affine 4-bit experts (bf16 scale and bias per 64 weights), 128 "
                        "experts, top_k 8, m=1: fused gate/up + SiLU over 768x2048 gate and up "
                        "matrices, the down-shaped 2048x768 id-GEMV, and the same in the 2-bit "
                        "variant; 8 replicas rotated",
            "kernel": "k_mlx4_rows",
        }
        for k, (us, b) in mlx.items():
            line["mlx4"][k] = {"us_per_launch": round(us, 3), "bytes_per_launch": int(b),
                               "gbs": round(b / us / 1e3, 2),
                               "frac_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    if walk_us is not None:
        line["walk"] = {
            "workload": "dense Q4TiledP decode walk: one layer (q, k, v, o 4096x4096, gate and up "
                        "14336x4096, down 4096x14336) and the head 32000x4096, 5-bit log-scale "
                        "ladder, 2 tensor replicas rotated",
            "kernel": "k_q4tp_matvec",
            "launches": "q|k|v, o, gate|up, down, head (merged dispatches)",
            "us_per_walk": round(walk_us, 3),
            "us_per_walk_one_launch_per_tensor": round(walk_single_us, 3),
            "us_per_walk_concurrent_groups": round(walk_conc_us, 3),
            "bytes_per_walk": int(walk_bytes),
            "gbs": round(walk_bytes / walk_us / 1e3, 2),
            "frac_hbm_peak": round(walk_bytes / walk_us / 1e3 / HBM_PEAK_GBS, 4),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
