"""GPU parity of the schedules the bucket_flag selects, against the oracle:

- the matrix-core schedule at activation scales from 2^-24 to 2^18 (values
  far outside fp16's range included), and with tokens of very different
  scales sharing a work chunk, checked row by row;
- activation rows that are only 4-byte aligned (one float past an aligned
  base, strides of k + 1 floats) in pair mode, on the matrix cores and on the
  vector units, through every entry point that takes activations;
- vector-unit bucketing equal bit for bit to pair mode, and AUTO picking pair
  mode below Q4K_AUTO_BUCKET_MIN_TOKENS tokens and the matrix cores from there;
- the layer's token mode at two and three tokens of the decode shape (the
  fused down + combine with two row groups per workgroup) against vector-unit
  bucketing, bit for bit, and the oracle;
- the layer's token mode when the down + combine kernel's staged rows do not
  fit one workgroup, and a bucketed layer past the in-kernel bucketing limit
  (more than 1024 pairs) with unaligned activations.

The band is the pages' (moeflux expert_forward.rs, module doc, Tolerance
regime), applied here to every output row on its own, so that small rows next
to large ones are held to it too."""
import numpy as np
import pytest

import oracle
import bit_quantized_moe_superblock_amd as q4
from bit_quantized_moe_superblock_amd import workloads as wl
from _util import band, bits
from test_gpu_parity import (T, Ws, _ffn_case, _shared_stacks, quantize_many, say, sync_np)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ON, OFF, AUTO = q4.Q4K_BUCKET_ON, q4.Q4K_BUCKET_OFF, q4.Q4K_BUCKET_AUTO
VEC = q4.Q4K_BUCKET_ON | q4.Q4K_SCHED_VECTOR
ON_WS = q4.Q4K_BUCKET_ON | q4.Q4K_SCHED_BUCKET_LAUNCH


@pytest.fixture(scope="module")
def dev():
    q4._lib.load()
    return torch.device("cuda:0")


def band_rows(got, want, what):
    got = np.asarray(got).reshape(want.shape[0], -1)
    want = np.asarray(want).reshape(want.shape[0], -1)
    worst = 0.0
    for r in range(want.shape[0]):
        if not np.any(want[r]):
            assert not np.any(got[r]), f"{what}: row {r} should be zero"
            continue
        rel, _ = band(got[r], want[r], f"{what}, row {r}")
        worst = max(worst, rel)
    return worst


def _ws(dev, P, E):
    wsb = q4.moe_bucket_workspace_bytes(P, E)
    return torch.empty(wsb, dtype=torch.uint8, device=dev), wsb


def _gate_up(dev, st, x, ids, n, k, m, K, outer, inner, E, flag, sh=None):
    ws, wsb = _ws(dev, m * K, E)
    out = torch.empty(m * K, n, device=dev)
    sh_out = torch.empty(m, n, device=dev) if sh is not None else None
    q4.q4k_moe_gate_up_silu(st[0], st[1], x, ids, out, n, k, m, K, outer, inner, E,
                            sh[0] if sh else None, sh[1] if sh else None, sh_out, flag, ws, wsb)
    return sync_np(out), (sync_np(sh_out) if sh is not None else None)


def _id_gemv(dev, stack, x, ids, n, k, m, K, outer, inner, E, flag):
    ws, wsb = _ws(dev, m * K, E)
    out = torch.empty(m * K, n, device=dev)
    q4.q4k_moe_id_gemv(stack, x, ids, out, n, k, m, K, outer, inner, E, flag, ws, wsb)
    return sync_np(out)


def _layer(dev, d_st, sd, h_post, h_mid, ids, rw, lg, H, I, E, m, K, mode, flag):
    wsb = q4.moe_layer_workspace_bytes(H, I, E, m, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty(m, H, device=dev)
    q4.moe_layer_forward(*d_st, *sd, h_post, h_mid, ids, rw, lg, out, H, I, E, m, K, mode, flag,
                         ws, wsb)
    return sync_np(out)


def _oracle_layer(h_st, sh_h, h_post, h_mid, ids, rw, lg, H, I, E, m, K, mode):
    _, _, _, eo = oracle.moe_expert_ffn(*h_st, E, H, I, h_post, ids, m, K)
    so = None
    if mode:
        _, _, _, so = oracle.moe_expert_ffn(*sh_h, 1, H, I, h_post, np.zeros(m, np.int32), m, 1)
    return oracle.moe_combine_residual(h_mid, eo, rw, so, lg if mode == 1 else None, H, m, K,
                                       mode)


# ------------------------------------------------------- activation scale ----

@pytest.mark.parametrize("e", [-24, -18, -12, 0, 12, 18])
def test_matrix_cores_hold_the_band_at_any_activation_scale(dev, e):
    """The batched decode workload (hidden 2048, inter 768, 128 experts, top_k
    8, m = 16, Zipf ids) with every activation scaled by 2^e: the gate/up +
    SiLU launch, the down id-GEMV and the whole layer on the matrix cores,
    row by row against the oracle on the same scaled inputs."""
    cfg = wl.CFG3
    H, I, E, K, m = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.m
    say(f"matrix cores, activations x 2^{e}")
    a, ids, d_st, h_st = _ffn_case(cfg, dev)
    sd, sh = _shared_stacks(cfg, dev)
    s = np.float32(2.0 ** e)
    h = (a.h_post * s).astype(np.float32)
    if e == 18:
        assert np.abs(h).max() > 65504.0   # beyond fp16's range
    g_o, u_o, act_o, eo_o = oracle.moe_expert_ffn(*h_st, E, H, I, h, ids, m, K)
    d_h, d_ids = T(h, dev), T(ids, dev)
    act, _ = _gate_up(dev, d_st, d_h, d_ids, I, H, m, K, H, 0, E, ON)
    r1 = band_rows(act, act_o, f"gate/up x 2^{e}")
    # the down projection on the oracle's act (scaled the same way)
    down = _id_gemv(dev, d_st[2], T(act_o, dev), d_ids, H, I, m, K, K * I, I, E, ON)
    r2 = band_rows(down, eo_o, f"down x 2^{e}")
    # the layer: h_mid zero so the output is the experts' sum alone
    zeros = np.zeros((m, H), np.float32)
    out = _layer(dev, d_st, sd, d_h, T(zeros, dev), d_ids, T(a.route_w, dev),
                 T(a.shared_logit, dev), H, I, E, m, K, cfg.shared_mode, ON)
    want = _oracle_layer(h_st, sh, h, zeros, ids, a.route_w, a.shared_logit, H, I, E, m, K,
                         cfg.shared_mode)
    assert np.all(np.isfinite(out))
    r3 = band_rows(out, want, f"layer x 2^{e}")
    say(f"  worst row: gate/up {r1:.3g}, down {r2:.3g}, layer {r3:.3g}")


def test_matrix_cores_tokens_of_different_scales_share_chunks(dev):
    """Each token of the batched decode workload scaled by its own power of
    two (2^-24 .. 2^20), so the hot experts' chunks mix rows whose magnitudes
    differ by up to 2^44 and hold values past 65504; every output row meets
    the band on its own."""
    cfg = wl.CFG3
    H, I, E, K, m = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, cfg.m
    say("matrix cores, per-token scales 2^-24 .. 2^20")
    a, ids, d_st, h_st = _ffn_case(cfg, dev)
    exps = np.array([-24, 20, -12, 0, 7, -20, 16, 3, -6, 12, -16, 1, 18, -3, 9, -9])
    h = (a.h_post * (2.0 ** exps)[:, None]).astype(np.float32)
    _, _, act_o, eo_o = oracle.moe_expert_ffn(*h_st, E, H, I, h, ids, m, K)
    d_ids = T(ids, dev)
    act, _ = _gate_up(dev, d_st, T(h, dev), d_ids, I, H, m, K, H, 0, E, ON)
    band_rows(act, act_o, "gate/up, mixed scales")
    down = _id_gemv(dev, d_st[2], T(act_o, dev), d_ids, H, I, m, K, K * I, I, E, ON)
    band_rows(down, eo_o, "down, mixed scales")
    # a bucket that holds every token: one expert, 16 tokens, top_k 1
    one = np.full(m, int(ids[0]), np.int32)
    got = _id_gemv(dev, d_st[0], T(h, dev), T(one, dev), I, H, m, 1, H, 0, E, ON)
    want = oracle.q4k_moe_id_gemv(h_st[0], E, I, H, h, one, m, 1, H, 0)
    band_rows(got, want, "one bucket of 16 mixed-scale tokens")


# ------------------------------------------------------ unaligned rows ----

def _unaligned(x2d, stride):
    """Host buffer holding the rows of x2d one float past a 16-byte aligned
    base, `stride` floats apart; returns (host flat view from the first row,
    device tensor view with the same 4-byte offset)."""
    rows, k = x2d.shape
    buf = np.zeros(1 + rows * stride + 3, np.float32)
    for r in range(rows):
        buf[1 + r * stride:1 + r * stride + k] = x2d[r]
    return buf[1:], buf


@pytest.mark.parametrize("m", [1, 16])
def test_unaligned_activation_rows_every_schedule(dev, m):
    """src1 one float past an aligned base with strides of k + 1 floats (so no
    row is 16-byte aligned): id-GEMV in gate/up and down stride modes, the
    fused gate/up + SiLU with the shared expert, the FFN and the layer, in pair
    mode, on the matrix cores and on the vector units, against the oracle;
    vector-unit bucketing equal to pair mode bit for bit."""
    cfg = wl.CFG3
    H, I, E, K = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    say(f"unaligned activation rows, m={m}")
    a, ids_all, d_st, h_st = _ffn_case(cfg, dev)
    sd, sh = _shared_stacks(cfg, dev)
    ids = ids_all[:m * K].copy()
    h = a.h_post[:m]
    # gate/up stride mode: token rows H + 1 floats apart
    hx, hbuf = _unaligned(h, H + 1)
    d_hbuf = T(hbuf, dev)
    d_x = d_hbuf[1:]
    d_ids = T(ids, dev)
    want = oracle.q4k_moe_id_gemv(h_st[0], E, I, H, hx, ids, m, K, H + 1, 0)
    res = {f: _id_gemv(dev, d_st[0], d_x, d_ids, I, H, m, K, H + 1, 0, E, f)
           for f in (OFF, ON, VEC)}
    for f, o in res.items():
        band_rows(o, want, f"id-GEMV gate/up mode, flag {f:#x}")
    assert np.array_equal(bits(res[VEC]), bits(res[OFF]))
    # down stride mode: pair rows I + 1 floats apart
    act = np.random.default_rng(90 + m).standard_normal((m * K, I)).astype(np.float32)
    ax, abuf = _unaligned(act, I + 1)
    d_a = T(abuf, dev)[1:]
    want = oracle.q4k_moe_id_gemv(h_st[2], E, H, I, ax, ids, m, K, K * (I + 1), I + 1)
    res = {f: _id_gemv(dev, d_st[2], d_a, d_ids, H, I, m, K, K * (I + 1), I + 1, E, f)
           for f in (OFF, ON, VEC)}
    for f, o in res.items():
        band_rows(o, want, f"id-GEMV down mode, flag {f:#x}")
    assert np.array_equal(bits(res[VEC]), bits(res[OFF]))
    # fused gate/up + SiLU with the shared expert riding along
    _, _, act_o, _ = oracle.moe_expert_ffn(*h_st, E, H, I, h, ids, m, K)
    _, _, sact_o, _ = oracle.moe_expert_ffn(*sh, 1, H, I, h, np.zeros(m, np.int32), m, 1)
    res = {f: _gate_up(dev, d_st, d_x, d_ids, I, H, m, K, H + 1, 0, E, f, sh=sd)
           for f in (OFF, ON, VEC)}
    for f, (o, so) in res.items():
        band_rows(o, act_o, f"gate/up + SiLU, flag {f:#x}")
        band_rows(so, sact_o, f"shared gate/up + SiLU, flag {f:#x}")
    assert np.array_equal(bits(res[VEC][0]), bits(res[OFF][0]))
    assert np.array_equal(bits(res[VEC][1]), bits(res[OFF][1]))
    # FFN and layer: h_post [m, H] contiguous, one float past an aligned base
    hx2, hbuf2 = _unaligned(h, H)
    d_h2 = T(hbuf2, dev)[1:]
    _, _, _, eo_o = oracle.moe_expert_ffn(*h_st, E, H, I, hx2, ids, m, K)
    for f in (OFF, ON, VEC):
        ws, wsb = _ws(dev, m * K, E)
        d_act = torch.empty(m * K, I, device=dev)
        d_eo = torch.empty(m * K, H, device=dev)
        q4.moe_expert_ffn(*d_st, d_h2, d_ids, d_act, d_eo, H, I, E, m, K, f, ws, wsb)
        band_rows(sync_np(d_eo), eo_o, f"FFN, flag {f:#x}")
    hm = a.h_mid[:m]
    want = _oracle_layer(h_st, sh, hx2, hm, ids, a.route_w[:m * K], a.shared_logit[:m], H, I, E,
                         m, K, cfg.shared_mode)
    outs = {}
    for f in (OFF, ON, VEC, ON_WS):
        outs[f] = _layer(dev, d_st, sd, d_h2, T(hm, dev), d_ids, T(a.route_w[:m * K], dev),
                         T(a.shared_logit[:m], dev), H, I, E, m, K, cfg.shared_mode, f)
        band_rows(outs[f], want, f"layer, flag {f:#x}")
    assert np.array_equal(bits(outs[VEC]), bits(outs[OFF]))
    assert np.array_equal(bits(outs[ON_WS]), bits(outs[ON]))


# ---------------------------------------------------- schedule choices ----

def test_auto_threshold_and_vector_bucketing_bitwise(dev):
    """AUTO runs pair mode below Q4K_AUTO_BUCKET_MIN_TOKENS tokens and the
    matrix cores from there (same bits as the flag it stands for), in the
    id-GEMV and in the layer; vector-unit bucketing gives pair mode's bits."""
    cfg = wl.CFG3
    H, I, E, K = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    a, ids_all, d_st, h_st = _ffn_case(cfg, dev)
    sd, sh = _shared_stacks(cfg, dev)
    mt = q4.Q4K_AUTO_BUCKET_MIN_TOKENS
    for m in (mt - 1, mt):
        say(f"AUTO at m={m}")
        ids = ids_all[:m * K].copy()
        d_h, d_ids = T(a.h_post[:m], dev), T(ids, dev)
        res = {f: _id_gemv(dev, d_st[0], d_h, d_ids, I, H, m, K, H, 0, E, f)
               for f in (AUTO, OFF, ON, VEC)}
        same = OFF if m < mt else ON
        assert np.array_equal(bits(res[AUTO]), bits(res[same]))
        assert np.array_equal(bits(res[VEC]), bits(res[OFF]))
        want = oracle.q4k_moe_id_gemv(h_st[0], E, I, H, a.h_post[:m], ids, m, K, H, 0)
        band_rows(res[ON], want, f"id-GEMV m={m}, matrix cores")
        args = (d_st, sd, d_h, T(a.h_mid[:m], dev), d_ids, T(a.route_w[:m * K], dev),
                T(a.shared_logit[:m], dev), H, I, E, m, K, cfg.shared_mode)
        lay = {f: _layer(dev, *args, f) for f in (AUTO, OFF, ON, VEC)}
        assert np.array_equal(bits(lay[AUTO]), bits(lay[same]))
        assert np.array_equal(bits(lay[VEC]), bits(lay[OFF]))
        want = _oracle_layer(h_st, sh, a.h_post[:m], a.h_mid[:m], ids, a.route_w[:m * K],
                             a.shared_logit[:m], H, I, E, m, K, cfg.shared_mode)
        band_rows(lay[ON], want, f"layer m={m}, matrix cores")


@pytest.mark.parametrize("m,mode", [(2, q4.MOE_SHARED_SIGMOID), (3, q4.MOE_SHARED_NONE),
                                    (2, q4.MOE_SHARED_UNSCALED)])
def test_token_mode_two_row_groups_per_workgroup(dev, m, mode):
    """From two tokens on, the layer's fused down + combine covers two row
    groups per workgroup (eight waves at two tokens of the decode shape, four
    from three); at hidden 2048, inter 768 and top_k 8, with each shared-expert
    mode, it gives the bits of vector-unit bucketing (pair mode and the
    combine launch) and holds the band against the oracle."""
    cfg = wl.CFG3
    H, I, E, K = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    say(f"token mode, two row groups per workgroup: m={m} shared mode {mode}")
    a, ids_all, d_st, h_st = _ffn_case(cfg, dev)
    sd, sh = _shared_stacks(cfg, dev)
    if mode == q4.MOE_SHARED_NONE:
        sd = (None, None, None)
    ids = ids_all[:m * K].copy()
    args = (d_st, sd, T(a.h_post[:m], dev), T(a.h_mid[:m], dev), T(ids, dev),
            T(a.route_w[:m * K], dev), T(a.shared_logit[:m], dev), H, I, E, m, K, mode)
    tok = _layer(dev, *args, OFF)
    assert np.array_equal(bits(tok), bits(_layer(dev, *args, VEC)))
    assert np.array_equal(bits(tok), bits(_layer(dev, *args, AUTO)))
    want = _oracle_layer(h_st, sh, a.h_post[:m], a.h_mid[:m], ids, a.route_w[:m * K],
                         a.shared_logit[:m], H, I, E, m, K, mode)
    band_rows(tok, want, f"token mode m={m}")


def _random_stacks(g, E, H, I):
    st = [np.concatenate(quantize_many([(g.standard_normal((r, c)) * 0.05).astype(np.float32)
                                        for _ in range(E)]))
          for r, c in [(I, H), (I, H), (H, I)]]
    sh = [oracle.q4k_quantize((g.standard_normal((r, c)) * 0.05).astype(np.float32))
          for r, c in [(I, H), (I, H), (H, I)]]
    return st, sh


def test_layer_token_mode_when_down_rows_do_not_fit(dev):
    """inter 16384 and top_k 16 with a shared expert: the 17 staged activation
    rows of the fused down + combine (1.2 MB) exceed a workgroup's LDS, so
    token mode runs down and the combine as two launches; it still matches
    the oracle and vector-unit bucketing bit for bit."""
    g = np.random.default_rng(91)
    H, I, E, K, m = 256, 16384, 20, 16, 2
    say(f"layer token mode, unfused down: H={H} I={I} E={E} K={K} m={m}")
    st, sh = _random_stacks(g, E, H, I)
    h = g.standard_normal((m, H)).astype(np.float32)
    hm = g.standard_normal((m, H)).astype(np.float32)
    ids = g.integers(0, E, m * K).astype(np.int32)
    ids[5] = E + 2
    rw = g.random(m * K).astype(np.float32)
    lg = g.standard_normal(m).astype(np.float32)
    want = _oracle_layer(st, sh, h, hm, ids, rw, lg, H, I, E, m, K, 1)
    args = (Ws(st, H, I, dev), Ws(sh, H, I, dev), T(h, dev), T(hm, dev), T(ids, dev),
            T(rw, dev), T(lg, dev), H, I, E, m, K, 1)
    off = _layer(dev, *args, OFF)
    band_rows(off, want, "token mode, unfused down")
    assert np.array_equal(bits(_layer(dev, *args, VEC)), bits(off))
    band_rows(_layer(dev, *args, ON), want, "matrix cores")


def test_layer_past_in_kernel_bucketing_limit_unaligned(dev):
    """160 tokens x top_k 8 = 1280 pairs (past the 1024 the matrix-core
    launches bucket in-kernel), h_post one float off alignment: the layer
    buckets with a separate launch, on the matrix cores and on the vector
    units, and matches the oracle."""
    g = np.random.default_rng(92)
    H, I, E, K, m = 256, 512, 64, 8, 160
    say(f"layer past the in-kernel bucketing limit: P={m * K}, unaligned h_post")
    st, sh = _random_stacks(g, E, H, I)
    h = g.standard_normal((m, H)).astype(np.float32)
    hx, hbuf = _unaligned(h, H)
    hm = g.standard_normal((m, H)).astype(np.float32)
    ids = np.stack([g.choice(E, K, replace=False) for _ in range(m)]).reshape(-1).astype(np.int32)
    rw = g.random(m * K).astype(np.float32)
    lg = g.standard_normal(m).astype(np.float32)
    want = _oracle_layer(st, sh, hx, hm, ids, rw, lg, H, I, E, m, K, 2)
    args = (Ws(st, H, I, dev), Ws(sh, H, I, dev), T(hbuf, dev)[1:], T(hm, dev),
            T(ids, dev), T(rw, dev), T(lg, dev), H, I, E, m, K, 2)
    outs = {f: _layer(dev, *args, f) for f in (ON, VEC, OFF)}
    for f, o in outs.items():
        band_rows(o, want, f"P=1280, flag {f:#x}")
    assert np.array_equal(bits(outs[VEC]), bits(outs[OFF]))
