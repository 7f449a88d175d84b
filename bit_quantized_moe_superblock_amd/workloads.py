"""Seeded synthetic workloads for the Q4_K MoE path and the Q4TiledP walk.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, no GEMV, no combine).  The tests feed
the same arrays to the oracle and to the GPU library; the benchmark uses the
device-side generator for sizes the host would take too long to draw.

No trained weights or real model files exist here; every tensor is drawn from
the distribution the workload names.  Shapes follow the pages' decode
workloads: a Qwen3-30B-A3B-class MoE layer (hidden 2048, expert intermediate
768, 128 experts, top-8; ferrum-kernels q4_k_moe_id_gemv_batched.rs,
microbench doc), a DeepSeek-V3-class layer (hidden 7168, 256 experts; moeflux
expert_forward.rs, Cogito-V2 hidden size note) and a 7B-class dense decode walk
(cortiq-engine mv_lab.rs, the per-layer q/k/v/o/gate/up/down walk and head).

Seeds: numpy ``default_rng([config, tensor_id, index])``; tensor ids below.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids inside a config's seed tuple
T_GATE, T_UP, T_DOWN = 0, 1, 2
T_SH_GATE, T_SH_UP, T_SH_DOWN = 3, 4, 5
T_H_POST, T_H_MID, T_IDS, T_ROUTE, T_SH_LOGIT, T_X = 10, 11, 12, 13, 14, 15
T_PERM = 16
T_WALK = 20  # + tensor index in the walk


@dataclass(frozen=True)
class MoeConfig:
    name: str
    cfg_id: int
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    m: int
    w_std: float = 0.02
    w_mean: float = 0.0
    ids_kind: str = "uniform"      # "uniform" (distinct per token) or "zipf"
    zipf_s: float = 1.1
    shared_mode: int = 1           # 0 none, 1 sigmoid gate, 2 unscaled

    @property
    def n_pairs(self) -> int:
        return self.m * self.top_k


@dataclass(frozen=True)
class IdGemvConfig:
    """A bare id-GEMV case (gate/up mode: one activation row per token)."""
    name: str
    cfg_id: int
    num_experts: int
    n: int
    k: int
    m: int
    top_k: int
    w_std: float
    w_mean: float


# Tiny gate/up-mode id-GEMV (the ferrum-kernels equivalence-test shape).
CFG1 = IdGemvConfig("cfg1_tiny_id_gemv", 1, num_experts=4, n=64, k=256, m=3, top_k=2,
                    w_std=0.4, w_mean=0.05)
# Single-token decode, Qwen3-30B-A3B-class layer, sigmoid-gated shared expert.
CFG2 = MoeConfig("cfg2_decode_m1", 2, hidden=2048, inter=768, num_experts=128, top_k=8, m=1)
# Sixteen tokens (c=16), Zipf(1.1) routing so experts repeat across tokens.
CFG3 = MoeConfig("cfg3_decode_m16_zipf", 3, hidden=2048, inter=768, num_experts=128, top_k=8,
                 m=16, ids_kind="zipf")
# DeepSeek-V3-class layer, unscaled shared expert.
CFG4_M1 = MoeConfig("cfg4_large_m1", 4, hidden=7168, inter=2048, num_experts=256, top_k=8, m=1,
                    shared_mode=2)
CFG4_M32 = MoeConfig("cfg4_large_m32", 4, hidden=7168, inter=2048, num_experts=256, top_k=8,
                     m=32, shared_mode=2)

# Dense 7B-class decode walk (Q4TiledP): per layer q,k,v,o then gate,up then down; head last.
WALK_LAYER = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
              ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
WALK_HEAD = ("head", 32000, 4096)
WALK_X_LEN = 14336
CFG5_ID = 5


def rng(cfg_id: int, tensor_id: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg_id, tensor_id, index])


def normal_f32(cfg_id: int, tensor_id: int, index: int, shape, std: float = 1.0,
               mean: float = 0.0) -> np.ndarray:
    g = rng(cfg_id, tensor_id, index)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def expert_weight(cfg, tensor_id: int, expert: int, rows: int, cols: int) -> np.ndarray:
    """One expert's fp32 matrix [rows, cols] ~ N(mean, std^2)."""
    return normal_f32(cfg.cfg_id, tensor_id, expert, (rows, cols), cfg.w_std, cfg.w_mean)


def distinct_uniform_ids(cfg_id: int, m: int, top_k: int, num_experts: int,
                         index: int = 0) -> np.ndarray:
    """top_k distinct experts per token, uniform (a router never repeats an expert)."""
    g = rng(cfg_id, T_IDS, index)
    ids = np.stack([g.choice(num_experts, size=top_k, replace=False) for _ in range(m)])
    return ids.reshape(-1).astype(np.int32)


def zipf_ids(cfg_id: int, m: int, top_k: int, num_experts: int, s: float,
             index: int = 0) -> np.ndarray:
    """Zipf(s) over expert ranks, top_k drawn without replacement per token; ranks
    map to ids through a seeded permutation so hot experts are not adjacent."""
    g = rng(cfg_id, T_IDS, index)
    ranks = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = rng(cfg_id, T_PERM, 0).permutation(num_experts)
    ids = np.stack([perm[g.choice(num_experts, size=top_k, replace=False, p=p)]
                    for _ in range(m)])
    return ids.reshape(-1).astype(np.int32)


def moe_ids(cfg: MoeConfig, index: int = 0) -> np.ndarray:
    if cfg.ids_kind == "zipf":
        return zipf_ids(cfg.cfg_id, cfg.m, cfg.top_k, cfg.num_experts, cfg.zipf_s, index)
    return distinct_uniform_ids(cfg.cfg_id, cfg.m, cfg.top_k, cfg.num_experts, index)


def route_weights(cfg: MoeConfig, index: int = 0) -> np.ndarray:
    """Softmax over top_k N(0,1) logits per token (sum-to-1 routing weights)."""
    z = normal_f32(cfg.cfg_id, T_ROUTE, index, (cfg.m, cfg.top_k)).astype(np.float64)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)


@dataclass
class MoeActivations:
    h_post: np.ndarray
    h_mid: np.ndarray
    ids: np.ndarray
    route_w: np.ndarray
    shared_logit: np.ndarray


def moe_activations(cfg: MoeConfig, index: int = 0) -> MoeActivations:
    return MoeActivations(
        h_post=normal_f32(cfg.cfg_id, T_H_POST, index, (cfg.m, cfg.hidden)),
        h_mid=normal_f32(cfg.cfg_id, T_H_MID, index, (cfg.m, cfg.hidden)),
        ids=moe_ids(cfg, index),
        route_w=route_weights(cfg, index),
        shared_logit=normal_f32(cfg.cfg_id, T_SH_LOGIT, index, (cfg.m,)),
    )


def id_gemv_inputs(cfg: IdGemvConfig):
    """fp32 expert weights [E, n, k], activations [m, k] and ids [m*top_k]."""
    w = np.stack([expert_weight(cfg, T_GATE, e, cfg.n, cfg.k) for e in range(cfg.num_experts)])
    x = normal_f32(cfg.cfg_id, T_X, 0, (cfg.m, cfg.k))
    ids = distinct_uniform_ids(cfg.cfg_id, cfg.m, cfg.top_k, cfg.num_experts)
    return w, x, ids


def walk_tensors(n_layers: int = 1, head: bool = True):
    """[(name, rows, cols, seed_index)] of the dense decode walk."""
    out = []
    idx = 0
    for layer in range(n_layers):
        for name, rows, cols in WALK_LAYER:
            out.append((f"L{layer}.{name}", rows, cols, idx))
            idx += 1
    if head:
        out.append((WALK_HEAD[0], WALK_HEAD[1], WALK_HEAD[2], idx))
    return out


def walk_weight(seed_index: int, rows: int, cols: int, std: float = 0.02) -> np.ndarray:
    return normal_f32(CFG5_ID, T_WALK, seed_index, (rows, cols), std)


def walk_x() -> np.ndarray:
    return normal_f32(CFG5_ID, T_X, 0, (WALK_X_LEN,))


# ------------------------------------------------------------ device side --

def device_normal(shape, std: float, seed: int, device="cuda"):
    """Device-side N(0, std^2) draw for benchmark-sized tensors (torch Philox).
    Not the numpy stream: used where the host would take minutes to draw."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x
