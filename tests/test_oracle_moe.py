"""Pins of the oracle's id-GEMV, expert FFN, combine and bucketing against
facts fixed outside it: a dense float64 matmul (numpy) over the dequantized
experts, the pair index / stride rule of the batched dispatcher, unit-vector
probes, batched == per-token on the pages' own equivalence case, closed forms
of the combine, scipy's logistic function, and brute-force bucket lists."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from bit_quantized_moe_superblock_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, np.int64(-2 ** 31) - a, a)
    b = np.where(b < 0, np.int64(-2 ** 31) - b, b)
    return np.abs(a - b)


def _stack(ws):
    return np.concatenate([oracle.q4k_quantize(w) for w in ws])


def _dense(stack, E, n, k):
    return oracle.q4k_dequantize(stack).reshape(E, n, k).astype(np.float64)


def _dense_id_gemv(W, src1_flat, ids, m, top_k, outer, inner, k):
    out = np.zeros((m * top_k, W.shape[1]))
    for p in range(m * top_k):
        t, s = divmod(p, top_k)
        e = ids[p]
        if 0 <= e < W.shape[0]:
            x = src1_flat[t * outer + s * inner: t * outer + s * inner + k].astype(np.float64)
            out[p] = W[e] @ x
    return out.astype(np.float32)


# -------------------------------------------------------------- id-GEMV ----

def test_id_gemv_equals_dense_matmul_cfg1():
    cfg = wl.CFG1
    w, x, ids = wl.id_gemv_inputs(cfg)
    stack = _stack(w)
    assert stack.size == cfg.num_experts * cfg.n * (cfg.k // 256) * 144
    got = oracle.q4k_moe_id_gemv(stack, cfg.num_experts, cfg.n, cfg.k, x, ids, cfg.m, cfg.top_k,
                                 cfg.k, 0)
    want = _dense_id_gemv(_dense(stack, cfg.num_experts, cfg.n, cfg.k), x.reshape(-1), ids,
                          cfg.m, cfg.top_k, cfg.k, 0, cfg.k)
    assert _ulp_diff(got, want).max() <= 1


@pytest.mark.parametrize("mode", ["gate_up", "down"])
def test_id_gemv_pair_index_and_strides(mode):
    """Row p comes from expert ids[p] applied to the activation row at
    token*outer + slot*inner (pair = token*top_k + slot)."""
    g = np.random.default_rng(3)
    E, n, k, m, K = 5, 16, 512, 4, 3
    stack = _stack([(g.standard_normal((n, k)) * 0.1).astype(np.float32) for _ in range(E)])
    W = _dense(stack, E, n, k)
    ids = g.integers(0, E, m * K).astype(np.int32)
    if mode == "gate_up":
        outer, inner = k, 0
        src1 = g.standard_normal(m * k).astype(np.float32)
    else:
        outer, inner = K * k, k
        src1 = g.standard_normal(m * K * k).astype(np.float32)
    got = oracle.q4k_moe_id_gemv(stack, E, n, k, src1, ids, m, K, outer, inner)
    for p in range(m * K):
        t, s = p // K, p % K
        x = src1[t * outer + s * inner:t * outer + s * inner + k].astype(np.float64)
        assert _ulp_diff(got[p], (W[ids[p]] @ x).astype(np.float32)).max() <= 1
    if mode == "down":   # distinct rows per slot: swapping two slots' rows swaps outputs
        src2 = src1.reshape(m, K, k).copy()
        src2[:, [0, 1]] = src2[:, [1, 0]]
        ids2 = ids.reshape(m, K).copy()
        ids2[:, [0, 1]] = ids2[:, [1, 0]]
        got2 = oracle.q4k_moe_id_gemv(stack, E, n, k, src2.reshape(-1), ids2.reshape(-1), m, K,
                                      outer, inner).reshape(m, K, n)
        g1 = got.reshape(m, K, n)
        assert np.array_equal(got2[:, 0], g1[:, 1]) and np.array_equal(got2[:, 1], g1[:, 0])


def test_id_gemv_unit_vector_probe_returns_columns_exactly():
    g = np.random.default_rng(4)
    E, n, k = 3, 8, 768
    stack = _stack([(g.standard_normal((n, k)) * 0.02).astype(np.float32) for _ in range(E)])
    W = oracle.q4k_dequantize(stack).reshape(E, n, k)
    for c in [0, 1, 31, 32, 63, 64, 255, 256, 300, 767]:
        x = np.zeros(k, np.float32)
        x[c] = 1.0
        ids = np.array([2, 0, 1], np.int32)
        got = oracle.q4k_moe_id_gemv(stack, E, n, k, x, ids, 1, 3, k, 0)
        for p in range(3):
            assert np.array_equal(got[p], W[ids[p], :, c])


def test_id_gemv_invalid_ids_give_zero_rows():
    g = np.random.default_rng(6)
    E, n, k = 2, 4, 256
    stack = _stack([(g.standard_normal((n, k))).astype(np.float32) for _ in range(E)])
    x = g.standard_normal(k).astype(np.float32)
    got = oracle.q4k_moe_id_gemv(stack, E, n, k, x, np.array([1, -1, 2, 0], np.int32), 1, 4, k, 0)
    assert np.all(got[1] == 0) and np.all(got[2] == 0)
    assert np.any(got[0] != 0) and np.any(got[3] != 0)


def test_id_gemv_one_matches_full():
    cfg = wl.CFG1
    w, x, ids = wl.id_gemv_inputs(cfg)
    stack = _stack(w)
    full = oracle.q4k_moe_id_gemv(stack, cfg.num_experts, cfg.n, cfg.k, x, ids, cfg.m, cfg.top_k,
                                  cfg.k, 0)
    for p, r in [(0, 0), (3, 17), (5, 63)]:
        assert oracle.q4k_moe_id_gemv_one(stack, cfg.num_experts, cfg.n, cfg.k, x, ids, cfg.top_k,
                                          cfg.k, 0, p, r) == full[p, r]


def _golden_case():
    with open(os.path.join(GOLDEN, "ferrum_equivalence_case.json")) as f:
        c = json.load(f)
    E, n, k, m, K = c["num_experts"], c["n"], c["k"], c["m"], c["top_k"]
    i = np.arange(n * k)
    wg = [(np.sin(((i + e * 313) % 251).astype(np.float32) * np.float32(0.013)) * np.float32(0.4)
           + np.float32(0.05)).astype(np.float32).reshape(n, k) for e in range(E)]
    wd = [(np.cos(((i + e * 251) % 199).astype(np.float32) * np.float32(0.011)) * np.float32(0.3)
           - np.float32(0.1)).astype(np.float32).reshape(n, k) for e in range(E)]
    ag = (np.cos(np.arange(m * k, dtype=np.float32) * np.float32(0.0021)) * np.float32(0.7)).astype(np.float32)
    ad = (np.sin(np.arange(m * K * k, dtype=np.float32) * np.float32(0.0017)) * np.float32(0.5)).astype(np.float32)
    return c, E, n, k, m, K, np.array(c["ids"], np.int32), wg, wd, ag, ad


def test_batched_equals_per_token_on_pages_case():
    """The pages' equivalence test, run on the oracle: one batched call over all
    m*top_k pairs equals m per-token calls, in both stride modes, bit for bit."""
    c, E, n, k, m, K, ids, wg, wd, ag, ad = _golden_case()
    for wts, act, outer, inner in [(wg, ag, k, 0), (wd, ad, K * k, k)]:
        stack = _stack(wts)
        batched = oracle.q4k_moe_id_gemv(stack, E, n, k, act, ids, m, K, outer, inner)
        per_tok = np.concatenate([
            oracle.q4k_moe_id_gemv(stack, E, n, k, act[t * outer:], ids[t * K:(t + 1) * K], 1, K,
                                   outer, inner) for t in range(m)])
        assert np.array_equal(batched.view(np.uint32), per_tok.view(np.uint32))


# ------------------------------------------------------------------ FFN ----

def test_expert_ffn_matches_dense_pipeline():
    g = np.random.default_rng(8)
    E, H, I, m, K = 4, 512, 256, 3, 2
    wgate = [(g.standard_normal((I, H)) * 0.05).astype(np.float32) for _ in range(E)]
    wup = [(g.standard_normal((I, H)) * 0.05).astype(np.float32) for _ in range(E)]
    wdown = [(g.standard_normal((H, I)) * 0.05).astype(np.float32) for _ in range(E)]
    sg, su, sd = _stack(wgate), _stack(wup), _stack(wdown)
    h = g.standard_normal((m, H)).astype(np.float32)
    ids = np.array([0, 3, 2, 3, 1, 0], np.int32)
    gate, up, act, out = oracle.moe_expert_ffn(sg, su, sd, E, H, I, h, ids, m, K)
    Wg, Wu, Wd = _dense(sg, E, I, H), _dense(su, E, I, H), _dense(sd, E, H, I)
    for p in range(m * K):
        t = p // K
        gg = (Wg[ids[p]] @ h[t].astype(np.float64)).astype(np.float32)
        uu = (Wu[ids[p]] @ h[t].astype(np.float64)).astype(np.float32)
        assert _ulp_diff(gate[p], gg).max() <= 1 and _ulp_diff(up[p], uu).max() <= 1
        # SiLU against scipy's logistic: z * expit(z)
        a = (gate[p].astype(np.float64) * expit(gate[p].astype(np.float64)) * up[p]).astype(np.float32)
        assert _ulp_diff(act[p], a).max() <= 1
        oo = (Wd[ids[p]] @ act[p].astype(np.float64)).astype(np.float32)
        assert _ulp_diff(out[p], oo).max() <= 1


def test_silu_and_sigmoid_special_values():
    assert oracle.silu(0.0) == 0.0
    assert math.isclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert oracle.silu(-800.0) == 0.0 and oracle.silu(800.0) == 800.0
    assert oracle.sigmoid(0.0) == 0.5
    for z in np.linspace(-30, 30, 61):
        assert math.isclose(oracle.sigmoid(z), float(expit(z)), rel_tol=1e-14)


# -------------------------------------------------------------- combine ----

def _combine_inputs(g, m, K, H):
    return (g.standard_normal((m, H)).astype(np.float32),
            g.standard_normal((m * K, H)).astype(np.float32),
            g.standard_normal((m, H)).astype(np.float32))


def test_combine_one_hot_weights_no_shared():
    g = np.random.default_rng(10)
    m, K, H = 3, 4, 64
    h_mid, eo, so = _combine_inputs(g, m, K, H)
    for s in range(K):
        w = np.zeros(m * K, np.float32)
        w[s::K] = 1.0
        out = oracle.moe_combine_residual(h_mid, eo, w, so, None, H, m, K, oracle.SHARED_NONE)
        assert np.array_equal(out, h_mid + eo.reshape(m, K, H)[:, s])


def test_combine_unscaled_and_half_gate_closed_forms():
    g = np.random.default_rng(12)
    m, K, H = 2, 8, 128
    h_mid, eo, so = _combine_inputs(g, m, K, H)
    w0 = np.zeros(m * K, np.float32)
    out = oracle.moe_combine_residual(h_mid, eo, w0, so, None, H, m, K, oracle.SHARED_UNSCALED)
    assert np.array_equal(out, h_mid + so)
    # sigmoid(0) = 1/2 exactly
    out = oracle.moe_combine_residual(h_mid, eo, w0, so, np.zeros(m, np.float32), H, m, K,
                                      oracle.SHARED_SIGMOID)
    assert np.array_equal(out, h_mid + np.float32(0.5) * so)
    # a very negative logit switches the shared expert off
    w = wl.route_weights(wl.CFG3)[:m * K]
    a = oracle.moe_combine_residual(h_mid, eo, w, so, np.full(m, -200.0, np.float32), H, m, K,
                                    oracle.SHARED_SIGMOID)
    b = oracle.moe_combine_residual(h_mid, eo, w, so, None, H, m, K, oracle.SHARED_NONE)
    assert np.array_equal(a, b)


def test_combine_general_matches_einsum():
    g = np.random.default_rng(13)
    m, K, H = 4, 8, 256
    h_mid, eo, so = _combine_inputs(g, m, K, H)
    w = g.random(m * K).astype(np.float32)
    logit = g.standard_normal(m).astype(np.float32)
    out = oracle.moe_combine_residual(h_mid, eo, w, so, logit, H, m, K, oracle.SHARED_SIGMOID)
    want = (h_mid.astype(np.float64)
            + np.einsum("ts,tsh->th", w.reshape(m, K).astype(np.float64),
                        eo.reshape(m, K, H).astype(np.float64))
            + expit(logit.astype(np.float64))[:, None] * so)
    assert _ulp_diff(out, want.astype(np.float32)).max() <= 1


# ------------------------------------------------------------ bucketing ----

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bucket_brute_force(seed):
    g = np.random.default_rng(seed)
    E = 16
    ids = g.integers(-2, E + 2, 64).astype(np.int32)   # includes invalid ids
    counts, offsets, pairs = oracle.moe_bucket(ids, E)
    for e in range(E + 1):
        if e < E:
            want = [p for p in range(ids.size) if ids[p] == e]
        else:
            want = [p for p in range(ids.size) if not (0 <= ids[p] < E)]
        assert counts[e] == len(want)
        assert list(pairs[offsets[e]:offsets[e + 1]]) == want
    assert offsets[0] == 0 and offsets[-1] == ids.size
    assert sorted(pairs.tolist()) == list(range(ids.size))


def test_bucket_zipf_config_shape():
    cfg = wl.CFG3
    ids = wl.moe_ids(cfg)
    counts, offsets, pairs = oracle.moe_bucket(ids, cfg.num_experts)
    used = int((counts[:cfg.num_experts] > 0).sum())
    assert counts[cfg.num_experts] == 0
    # a token never repeats an expert, so no bucket exceeds m
    assert counts.max() <= cfg.m
    assert 30 <= used <= 80
    for t in range(cfg.m):
        assert len(set(ids[t * cfg.top_k:(t + 1) * cfg.top_k])) == cfg.top_k


# ------------------------------------------------------- chained RMSNorm ----

def _bf16(vals):
    return np.array([oracle.f32_to_bf16(float(v)) for v in vals], np.uint16)


def test_rmsnorm_hand_values_and_closed_forms():
    # [1, 7]: mean square 25, rms 5 -> [0.2, 1.4] (by hand); weights 1 and 2
    got = oracle.rmsnorm_bf16(np.array([[1.0, 7.0]], np.float32), _bf16([1.0, 2.0]), 0.0)
    assert got[0].tolist() == [np.float32(0.2), np.float32(2.8)]
    # a constant row c with eps = 0 normalises to sign(c) * w
    w = _bf16(np.linspace(-3, 3, 64))
    wf = np.array([oracle.bf16_to_f32(int(h)) for h in w], np.float32)
    for c in (-2.5, 0.125, 7.0):
        got = oracle.rmsnorm_bf16(np.full((1, 64), c, np.float32), w, 0.0)
        assert np.array_equal(got[0], np.sign(c) * wf)
    # zero row with eps > 0 stays zero; eps enters under the root: x = 0.5
    # everywhere, eps = 0.75 -> rms 1 -> 0.5 * w
    assert np.all(oracle.rmsnorm_bf16(np.zeros((2, 8), np.float32), _bf16([1.0] * 8), 1e-6) == 0)
    got = oracle.rmsnorm_bf16(np.full((1, 8), 0.5, np.float32), _bf16([3.0] * 8), 0.75)
    assert np.all(got == 1.5)


def test_rmsnorm_scale_invariance_and_rows_independent():
    g = np.random.default_rng(11)
    x = g.standard_normal((3, 2048)).astype(np.float32)
    w = _bf16(g.standard_normal(2048))
    base = oracle.rmsnorm_bf16(x, w, 0.0)
    for a in (0.5, 4.0, 1024.0):   # powers of two scale exactly
        assert np.array_equal(oracle.rmsnorm_bf16(x * np.float32(a), w, 0.0), base)
    # each row normalises on its own: the batch equals row-by-row calls
    for t in range(3):
        assert np.array_equal(oracle.rmsnorm_bf16(x[t:t + 1], w, 0.0)[0], base[t])
    # unit mean square: the output is x * w (to float rounding)
    xs = x[0] / np.sqrt(np.mean(x[0].astype(np.float64) ** 2))
    wf = np.array([oracle.bf16_to_f32(int(h)) for h in w])
    np.testing.assert_allclose(oracle.rmsnorm_bf16(xs[None].astype(np.float32), w, 0.0)[0],
                               xs * wf, rtol=1e-6, atol=1e-7)
