"""Pins of the oracle's MLX affine 4-bit codec (moeflux expert_forward.rs:
4-bit experts, group of 64 weights, bf16 scales and biases at K/64 per row,
packed weights at K/2 bytes per row) against facts fixed outside it: torch's
bfloat16 conversion, hand-built groups, the single rounding of
scale*q + bias checked in float64, a dense float64 matmul (numpy) over the
dequantized experts, unit-vector probes and the pair index / stride rule."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
G = oracle.MLX_GROUP


def _bf16_torch(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_conversion_matches_torch():
    g = np.random.default_rng(0)
    xs = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38, 1.0 + 2 ** -8,
                  1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], np.float32),
    ]).astype(np.float32)
    want = _bf16_torch(xs)
    got = np.array([oracle.f32_to_bf16(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want)
    # widening is exact: back to float32 equals torch's
    back = np.array([oracle.bf16_to_f32(int(h)) for h in want[:2000]], np.float32)
    ref = torch.from_numpy(want[:2000].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), ref.view(np.uint32))
    # NaN stays NaN
    assert np.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(float("nan"))))


def test_nibble_order_low_then_high():
    # byte j holds weight 2j (low nibble) and 2j+1 (high nibble)
    packed = np.array([[0x21, 0x43, 0x65, 0x87] + [0xF0] * 28], np.uint8)
    assert [oracle.mlx4_nibble(packed[0], c) for c in range(8)] == [1, 2, 3, 4, 5, 6, 7, 8]
    one = oracle.f32_to_bf16(1.0)
    out = oracle.mlx4_dequantize(packed, np.array([[one]], np.uint16),
                                 np.array([[0]], np.uint16), 1, G)
    assert out[0, :8].tolist() == [1, 2, 3, 4, 5, 6, 7, 8]
    assert out[0, 8:].tolist() == [0.0, 15.0] * 28


def test_dequant_zero_scale_and_zero_codes_give_bias():
    g = np.random.default_rng(1)
    packed = g.integers(0, 256, (3, 2 * G // 2), dtype=np.uint8)
    b = np.array([oracle.f32_to_bf16(v) for v in (-0.75, 0.125, 3.5, -2.0, 0.0, 1.0)],
                 np.uint16).reshape(3, 2)
    out = oracle.mlx4_dequantize(packed, np.zeros((3, 2), np.uint16), b, 3, 2 * G)
    for r in range(3):
        for gi in range(2):
            assert np.all(out[r, gi * G:(gi + 1) * G] == oracle.bf16_to_f32(int(b[r, gi])))
    s = np.full((3, 2), oracle.f32_to_bf16(0.3), np.uint16)
    out = oracle.mlx4_dequantize(np.zeros_like(packed), s, b, 3, 2 * G)
    assert np.array_equal(out, np.repeat(np.array([[oracle.bf16_to_f32(int(v)) for v in row]
                                                   for row in b], np.float32), G, axis=1))


def test_dequant_single_rounding_of_exact_value():
    # scale*q is exact in float32 (8 + 4 significant bits), so the result is the
    # correctly rounded float32 of the exact scale*q + bias, which float64
    # holds exactly for these magnitudes
    g = np.random.default_rng(2)
    n, k = 16, 4 * G
    packed = g.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sv = (g.standard_normal((n, k // G)) * 10.0 ** g.integers(-6, 3, (n, k // G)))
    bv = (g.standard_normal((n, k // G)) * 10.0 ** g.integers(-6, 3, (n, k // G)))
    s = _bf16_torch(sv.astype(np.float32)).reshape(n, -1)
    b = _bf16_torch(bv.astype(np.float32)).reshape(n, -1)
    out = oracle.mlx4_dequantize(packed, s, b, n, k)
    sf = torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).double().numpy()
    bf = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    q = np.stack([packed & 15, packed >> 4], axis=-1).reshape(n, k).astype(np.float64)
    exact = np.repeat(sf, G, axis=1) * q + np.repeat(bf, G, axis=1)
    assert np.array_equal(out, exact.astype(np.float32))


def test_quantizer_bytes_on_grid_and_error_bound():
    g = np.random.default_rng(3)
    # weights already on a bf16 affine grid come back exactly
    n, k = 8, 2 * G
    s_true = np.float32(2.0 ** -5)
    b_true = np.float32(-0.25)
    q = g.integers(0, 16, (n, k))
    q[:, 0], q[:, G] = 0, 0          # every group spans the full code range
    q[:, 1], q[:, G + 1] = 15, 15
    w = (b_true + s_true * q).astype(np.float32)
    packed, s, b = oracle.mlx4_quantize(w)
    assert np.all(s == oracle.f32_to_bf16(float(s_true)))
    assert np.all(b == oracle.f32_to_bf16(float(b_true)))
    assert np.array_equal(oracle.mlx4_dequantize(packed, s, b, n, k), w)
    # general weights: error within half a step plus the bf16 rounding of the
    # group's scale (15 steps) and bias
    w = (g.standard_normal((32, 8 * G)) * 0.5 + 0.1).astype(np.float32)
    packed, s, b = oracle.mlx4_quantize(w)
    d = oracle.mlx4_dequantize(packed, s, b, 32, 8 * G)
    wg = w.reshape(32, 8, G).astype(np.float64)
    lo, hi = wg.min(-1), wg.max(-1)
    sf = np.array([[oracle.bf16_to_f32(int(v)) for v in row] for row in s])
    bf = np.array([[oracle.bf16_to_f32(int(v)) for v in row] for row in b])
    bound = 0.5 * sf + 15 * np.abs(sf - (hi - lo) / 15) + np.abs(bf - lo) + 1e-6
    err = np.abs(d.reshape(32, 8, G) - wg).max(-1)
    assert np.all(err <= bound)
    # constant groups: scale 0, every weight the bias
    p0, s0, b0 = oracle.mlx4_quantize(np.full((2, G), 0.7, np.float32))
    assert np.all(s0 == 0) and np.all(p0 == 0)


def _blob(mats):
    """Expert blocks of several sub-tensors: per expert, each matrix's packed,
    scales and biases one after another (16-byte aligned), like an expert
    block holding gate, up and down."""
    parts, offs = [], []
    off = 0
    for packed, s, b in mats[0]:
        o = []
        for a in (packed, s.view(np.uint8), b.view(np.uint8)):
            o.append(off)
            off += (a.nbytes + 15) // 16 * 16
        offs.append(tuple(o))
    stride = off
    blob = np.zeros(len(mats) * stride, np.uint8)
    for e, expert in enumerate(mats):
        for (packed, s, b), (po, so, bo) in zip(expert, offs):
            for a, o in ((packed, po), (s.view(np.uint8), so), (b.view(np.uint8), bo)):
                flat = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
                blob[e * stride + o: e * stride + o + flat.size] = flat
    return blob, stride, offs


def _dense_id_gemv(W, src1_flat, ids, m, top_k, outer, inner, k):
    out = np.zeros((m * top_k, W.shape[1]))
    for p in range(m * top_k):
        t, s = divmod(p, top_k)
        e = ids[p]
        if 0 <= e < W.shape[0]:
            x = src1_flat[t * outer + s * inner: t * outer + s * inner + k].astype(np.float64)
            out[p] = W[e] @ x
    return out.astype(np.float32)


@pytest.mark.parametrize("mode", ["gate_up", "down"])
def test_id_gemv_equals_dense_matmul_and_pair_walk(mode):
    g = np.random.default_rng(4)
    E, n, k, m, K = 5, 40, 3 * G, 3, 2
    mats = [[oracle.mlx4_quantize((g.standard_normal((n, k)) * 0.3).astype(np.float32)),
             oracle.mlx4_quantize((g.standard_normal((16, G)) * 0.3).astype(np.float32))]
            for _ in range(E)]
    blob, stride, offs = _blob(mats)
    W = np.stack([oracle.mlx4_dequantize(*mats[e][0], n, k) for e in range(E)]).astype(np.float64)
    ids = np.array([4, 1, 0, 4, 2, 3], np.int32)
    if mode == "gate_up":
        x = g.standard_normal((m, k)).astype(np.float32)
        outer, inner = k, 0
    else:
        x = g.standard_normal((m * K, k)).astype(np.float32)
        outer, inner = K * k, k
    got = oracle.mlx4_moe_id_gemv(blob, stride, *offs[0], E, n, k, x, ids, m, K, outer, inner)
    want = _dense_id_gemv(W, x.reshape(-1), ids, m, K, outer, inner, k)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)
    # row p comes from (token p // K, slot p % K): permuting the pairs permutes the rows
    perm = np.array([1, 0, 3, 2, 5, 4])
    if mode == "down":
        xp = x.reshape(m, K, k)[:, ::-1].reshape(m * K, k)
        got2 = oracle.mlx4_moe_id_gemv(blob, stride, *offs[0], E, n, k, xp, ids[perm], m, K,
                                       outer, inner)
        assert np.array_equal(got2, got[perm])


def test_id_gemv_unit_vector_probe_and_invalid_ids():
    g = np.random.default_rng(5)
    E, n, k = 3, 24, 4 * G
    mats = [[oracle.mlx4_quantize((g.standard_normal((n, k)) * 0.2).astype(np.float32))]
            for _ in range(E)]
    blob, stride, offs = _blob(mats)
    for c in (0, 1, 63, 64, 200, k - 1):
        x = np.zeros((1, k), np.float32)
        x[0, c] = 1.0
        ids = np.array([2, 0, 7, -1], np.int32)
        got = oracle.mlx4_moe_id_gemv(blob, stride, *offs[0], E, n, k, x, ids, 1, 4, k, 0)
        assert np.array_equal(got[0], oracle.mlx4_dequantize(*mats[2][0], n, k)[:, c])
        assert np.array_equal(got[1], oracle.mlx4_dequantize(*mats[0][0], n, k)[:, c])
        assert np.all(got[2:] == 0.0)


# ------------------------------------------------------------- 2-bit ----

def test_mlx2_code_order_and_hand_group():
    # byte j holds weights 4j..4j+3 at bits 0-1, 2-3, 4-5, 6-7
    packed = np.array([[0b11100100, 0b00011011] + [0] * 14], np.uint8)
    assert [oracle.mlx2_code(packed[0], c) for c in range(8)] == [0, 1, 2, 3, 3, 2, 1, 0]
    s = np.array([[oracle.f32_to_bf16(0.5)]], np.uint16)
    b = np.array([[oracle.f32_to_bf16(-1.0)]], np.uint16)
    out = oracle.mlx2_dequantize(packed, s, b, 1, G)
    assert out[0, :8].tolist() == [-1.0, -0.5, 0.0, 0.5, 0.5, 0.0, -0.5, -1.0]
    assert np.all(out[0, 8:] == -1.0)


def test_mlx2_quantizer_grid_and_bound():
    g = np.random.default_rng(6)
    q = g.integers(0, 4, (6, 2 * G))
    q[:, 0], q[:, G], q[:, 1], q[:, G + 1] = 0, 0, 3, 3
    w = (np.float32(0.75) + np.float32(0.125) * q).astype(np.float32)
    packed, s, b = oracle.mlx2_quantize(w)
    assert np.array_equal(oracle.mlx2_dequantize(packed, s, b, 6, 2 * G), w)
    w = (g.standard_normal((16, 4 * G)) * 0.3).astype(np.float32)
    packed, s, b = oracle.mlx2_quantize(w)
    d = oracle.mlx2_dequantize(packed, s, b, 16, 4 * G)
    wg = w.reshape(16, 4, G).astype(np.float64)
    lo, hi = wg.min(-1), wg.max(-1)
    sf = np.array([[oracle.bf16_to_f32(int(v)) for v in row] for row in s])
    bf = np.array([[oracle.bf16_to_f32(int(v)) for v in row] for row in b])
    bound = 0.5 * sf + 3 * np.abs(sf - (hi - lo) / 3) + np.abs(bf - lo) + 1e-6
    assert np.all(np.abs(d.reshape(16, 4, G) - wg).max(-1) <= bound)


def test_mlx2_id_gemv_equals_dense_matmul():
    g = np.random.default_rng(7)
    E, n, k, m, K = 4, 24, 3 * G, 2, 2
    mats = [oracle.mlx2_quantize((g.standard_normal((n, k)) * 0.3).astype(np.float32))
            for _ in range(E)]
    stride = n * k // 4 + 2 * (n * k // 32)
    blob = np.concatenate([np.concatenate([p.reshape(-1), s.reshape(-1).view(np.uint8),
                                           b.reshape(-1).view(np.uint8)]) for p, s, b in mats])
    offs = (0, n * k // 4, n * k // 4 + n * k // 32)
    W = np.stack([oracle.mlx2_dequantize(*mats[e], n, k) for e in range(E)]).astype(np.float64)
    x = g.standard_normal((m * K, k)).astype(np.float32)
    ids = np.array([3, 0, 9, 2], np.int32)
    got = oracle.mlx2_moe_id_gemv(blob, stride, *offs, E, n, k, x, ids, m, K, K * k, k)
    want = _dense_id_gemv(W, x.reshape(-1), ids, m, K, K * k, k, k)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)
    assert np.all(got[2] == 0.0)
