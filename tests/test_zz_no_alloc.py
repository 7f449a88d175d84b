"""The no-allocation layer entry point (moe_layer_forward_noalloc) against the
workspace entry point it stands in for (moe_layer_forward), through the C ABI:
two calls in a row on the library's static scratch, the second with a smaller
input, each equal bit for bit to the workspace call with the same arguments
(the same kernels run) and within the band of the oracle."""
import numpy as np
import pytest

import oracle
import bit_quantized_moe_superblock_amd as q4
from bit_quantized_moe_superblock_amd import workloads as wl
from _util import band, bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _stacks(cfg, ids, dev):
    """Device stacks of the routed experts (only the touched ones encoded)
    and the shared expert, plus their host bytes for the oracle."""
    H, I, E = cfg.hidden, cfg.inter, cfg.num_experts
    touched = sorted(set(int(e) for e in ids))
    d, h = [], []
    for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
        nb = oracle.q4k_matrix_bytes(rows, cols)
        host = np.zeros(E * nb, np.uint8)
        for e in touched:
            host[e * nb:(e + 1) * nb] = oracle.q4k_quantize(
                wl.expert_weight(cfg, t, e, rows, cols))
        h.append(host)
        d.append(_tiles(host, rows, cols))
    sh_h = [oracle.q4k_quantize(wl.expert_weight(cfg, wl.T_SH_GATE + t, 0, rows, cols))
            for t, (rows, cols) in enumerate([(I, H), (I, H), (H, I)])]
    sh_d = [_tiles(x, rows, cols) for x, (rows, cols) in zip(sh_h, [(I, H), (I, H), (H, I)])]
    return d, h, sh_d, sh_h


def _tiles(host, n, k):
    """GGUF-order matrices -> a device stack in the tile layout."""
    src = torch.from_numpy(host).to("cuda")
    n_mats = host.size // q4.q4k_matrix_bytes(n, k)
    out = torch.empty(n_mats * q4.q4k_tiles_bytes(n, k), dtype=torch.uint8, device="cuda")
    q4.q4k_pack_tiles(src, out, n_mats, n, k)
    return out


def _run(cfg, flag):
    H, I, E, K, m = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.m
    a = wl.moe_activations(cfg)
    d, h, sh_d, sh_h = _stacks(cfg, a.ids, "cuda")
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    args = (*d, *sh_d, T(a.h_post), T(a.h_mid), T(a.ids), T(a.route_w), T(a.shared_logit))
    out_na = torch.full((m, H), float("nan"), device="cuda")
    q4.moe_layer_forward_noalloc(*args, out_na, H, I, E, m, K, cfg.shared_mode, flag)
    wsb = q4.moe_layer_workspace_bytes(H, I, E, m, K)
    assert wsb <= q4.MOE_LAYER_NOALLOC_MAX_BYTES
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out_ws = torch.empty(m, H, device="cuda")
    q4.moe_layer_forward(*args, out_ws, H, I, E, m, K, cfg.shared_mode, flag, ws, wsb)
    torch.cuda.synchronize()
    got, ref = out_na.cpu().numpy(), out_ws.cpu().numpy()
    assert np.array_equal(bits(got), bits(ref)), f"{cfg.name}: no-alloc differs from workspace"
    _, _, _, eo = oracle.moe_expert_ffn(*h, E, H, I, a.h_post, a.ids, m, K)
    _, _, _, so = oracle.moe_expert_ffn(*sh_h, 1, H, I, a.h_post, np.zeros(m, np.int32), m, 1)
    want = oracle.moe_combine_residual(a.h_mid, eo, a.route_w, so, a.shared_logit, H, m, K,
                                       cfg.shared_mode)
    band(got, want, f"{cfg.name} no-alloc vs oracle")


def test_noalloc_layer_two_calls_second_smaller():
    q4._lib.load()
    print("[no-alloc] m=16 bucketed (matrix cores), then m=1 token mode", flush=True)
    _run(wl.CFG3, q4.Q4K_BUCKET_AUTO)    # 16 tokens: bucketed, in-kernel buckets
    _run(wl.CFG2, q4.Q4K_BUCKET_AUTO)    # 1 token: token mode, smaller scratch
