"""Pins of the oracle's Q4TiledP codec and matvec: byte counts from the page's
offsets, code extraction against an independent big-integer bit string, an
independent vectorized decode of the byte layout, the single-scale (step = 0)
reduction to a plain q4 GEMV, unit-vector probes, and encoder bounds."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, np.int64(-2 ** 31) - a, a)
    b = np.where(b < 0, np.int64(-2 ** 31) - b, b)
    return np.abs(a - b)


def _assemble(nib, codes, base16, step16):
    """Build a tensor from fields with Python integers (independent of the
    oracle): nibbles [rows, cols] in 0..15, codes [rows, gpr] in 0..31."""
    rows, cols = nib.shape
    gpr = cols // 32
    grp = nib.reshape(rows, gpr, 16, 2)
    body = (grp[..., 0] | (grp[..., 1] << 4)).astype(np.uint8).reshape(-1)
    params = np.zeros((rows, 4), np.uint8)
    params[:, 0] = base16 & 255
    params[:, 1] = base16 >> 8
    params[:, 2] = step16 & 255
    params[:, 3] = step16 >> 8
    stride = (5 * gpr + 7) // 8
    code_bytes = np.zeros((rows, stride), np.uint8)
    for r in range(rows):
        big = 0
        for g_ in range(gpr):
            big |= int(codes[r, g_]) << (5 * g_)
        code_bytes[r] = np.frombuffer(big.to_bytes(stride, "little"), np.uint8)
    return np.concatenate([body, params.reshape(-1), code_bytes.reshape(-1)])


def _decode_numpy(t, rows, cols):
    """Vectorized decode of the layout, written from the page's offsets."""
    gpr = cols // 32
    body = t[:rows * gpr * 16].reshape(rows, gpr, 16)
    nib = np.stack([body & 15, body >> 4], axis=-1).reshape(rows, cols).astype(np.int64)
    p = t[rows * gpr * 16: rows * gpr * 16 + rows * 4].reshape(rows, 4)
    base = p[:, 0:2].copy().view(np.float16).astype(np.float32).reshape(-1)
    step = p[:, 2:4].copy().view(np.float16).astype(np.float32).reshape(-1)
    stride = (5 * gpr + 7) // 8
    cb = t[rows * gpr * 16 + rows * 4:].reshape(rows, stride)
    bits = np.unpackbits(cb, axis=1, bitorder="little")[:, :5 * gpr].reshape(rows, gpr, 5)
    codes = (bits * (1 << np.arange(5))).sum(-1)
    expo = base[:, None] + codes.astype(np.float32) * step[:, None]   # float32, exact product
    L = np.exp2(expo.astype(np.float64)).astype(np.float32)
    return nib, codes, L


def test_row_bytes_match_layout():
    with open(os.path.join(GOLDEN, "format_constants.json")) as f:
        fmt = json.load(f)
    assert oracle.q4tp_bytes(1, 4096) == fmt["q4tp_row_bytes_at_4096_cols"]["value"]
    assert oracle.q4tp_bytes(1, 14336) == fmt["q4tp_row_bytes_at_14336_cols"]["value"]
    assert oracle.q4tp_bytes(4096, 4096) == 4096 * 2132


def test_code_extraction_brute_force_all_group_counts():
    g = np.random.default_rng(0)
    for gpr in range(1, 65):
        rows = 3
        codes = g.integers(0, 32, (rows, gpr))
        nib = g.integers(0, 16, (rows, 32 * gpr))
        t = _assemble(nib, codes, np.full(rows, 0x3C00), np.full(rows, 0))
        for r in range(rows):
            for gg in range(gpr):
                assert oracle.q4tp_code(t, rows, 32 * gpr, r, gg) == codes[r, gg]


def test_dequant_matches_independent_decode():
    g = np.random.default_rng(1)
    rows, cols = 7, 32 * 13
    codes = g.integers(0, 32, (rows, cols // 32))
    nib = g.integers(0, 16, (rows, cols))
    base = np.array([oracle.f32_to_f16(v) for v in g.uniform(-9, -3, rows)], np.int64)
    step = np.array([oracle.f32_to_f16(v) for v in g.uniform(0.01, 0.3, rows)], np.int64)
    t = _assemble(nib, codes, base, step)
    got = oracle.q4tp_dequantize(t, rows, cols)
    n2, c2, L = _decode_numpy(t, rows, cols)
    assert np.array_equal(n2, nib) and np.array_equal(c2, codes)
    want = np.repeat(L, 32, axis=1) * (nib - 8).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32))
    # nibble order: byte i of a group holds element 2i (low) and 2i+1 (high)
    for r, c in [(0, 0), (0, 1), (3, 33), (6, cols - 1)]:
        assert oracle.q4tp_nibble(t, cols, r, c) == nib[r, c]


def test_step_zero_reduces_to_single_scale_gemv():
    g = np.random.default_rng(2)
    rows, cols = 16, 256
    codes = g.integers(0, 32, (rows, cols // 32))   # ignored when step = 0
    nib = g.integers(0, 16, (rows, cols))
    base16 = oracle.f32_to_f16(-6.5)
    t = _assemble(nib, codes, np.full(rows, base16), np.zeros(rows, np.int64))
    x = g.standard_normal(cols).astype(np.float32)
    y = oracle.q4tp_matvec(t, rows, cols, x)
    s = 2.0 ** -6.5
    want = (s * ((nib - 8).astype(np.float64) @ x.astype(np.float64))).astype(np.float32)
    assert _ulp_diff(y, want).max() <= 1


def test_matvec_matches_dense_and_unit_probe():
    g = np.random.default_rng(3)
    rows, cols = 40, 4096
    w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    t = oracle.q4tp_quantize(w)
    assert t.size == oracle.q4tp_bytes(rows, cols)
    D = oracle.q4tp_dequantize(t, rows, cols)
    x = g.standard_normal(cols).astype(np.float32)
    y = oracle.q4tp_matvec(t, rows, cols, x)
    # scale*(nib-8) needs up to 27 bits, so the dense reference keeps the exact
    # weights in float64 (the stored fp32 dequant rounds them)
    nib, codes, L = _decode_numpy(t, rows, cols)
    W64 = np.repeat(L.astype(np.float64), 32, axis=1) * (nib - 8)
    assert _ulp_diff(y, (W64 @ x.astype(np.float64)).astype(np.float32)).max() <= 1
    for c in [0, 1, 31, 32, 2049, 4095]:
        e = np.zeros(cols, np.float32)
        e[c] = 1.0
        assert np.array_equal(oracle.q4tp_matvec(t, rows, cols, e), D[:, c])
    assert oracle.q4tp_matvec_one(t, rows, cols, x, 17) == y[17]


def test_quantizer_bounds_and_zero_groups():
    g = np.random.default_rng(4)
    rows, cols = 24, 1024
    w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w[5] = 0.0                       # all-zero row
    w[6, 64:96] = 0.0                # one all-zero group
    t = oracle.q4tp_quantize(w)
    nib, codes, L = _decode_numpy(t, rows, cols)
    assert np.all(nib[5] == 8) and np.all(codes[5] == 0)
    p = t[rows * cols // 2: rows * cols // 2 + rows * 4].reshape(rows, 4)
    assert p[5].tolist() == [0, 0, 0, 0]
    assert np.all(nib[6, 64:96] == 8)
    back = oracle.q4tp_dequantize(t, rows, cols)
    # the chosen rung covers its group's max|w| within the ladder spacing,
    # so every weight lands within about one rung of its value
    grp_w = w.reshape(rows, -1, 32)
    err = np.abs(back - w).reshape(rows, -1, 32).max(-1)
    assert np.all(err <= L * 1.0 + 1e-7)
    rel = np.sqrt(np.mean((back - w) ** 2)) / np.sqrt(np.mean(w ** 2))
    assert rel < 0.2
    assert np.all(grp_w.shape[1] == cols // 32)
