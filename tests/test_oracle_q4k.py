"""Pins of the oracle's fp16 conversion and Q4_K codec against facts fixed
outside the oracle: numpy's IEEE binary16, hand-built blocks, brute force over
the 6-bit scale packing, exactness of the fp32 dequant, and exact re-encoding of
blocks whose weights lie on the Q4_K grid."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fmt():
    with open(os.path.join(GOLDEN, "format_constants.json")) as f:
        return json.load(f)


# ----------------------------------------------------------------- fp16 ----

def test_f16_to_f32_all_patterns_match_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(h)) for h in pats], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_round_trip_and_rne_match_numpy():
    # every finite half survives f16 -> f32 -> f16
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16)
    fin = np.isfinite(vals)
    for h in pats[fin][::7]:
        assert oracle.f32_to_f16(oracle.f16_to_f32(int(h))) == int(h)
    # random floats across the whole half range, ties included
    g = np.random.default_rng(123)
    xs = np.concatenate([
        g.standard_normal(4000).astype(np.float32),
        (g.standard_normal(2000) * 3e4).astype(np.float32),
        (g.standard_normal(2000) * 1e-5).astype(np.float32),    # subnormal halves
        (g.standard_normal(1000) * 1e-8).astype(np.float32),    # underflow to 0
        np.array([65504, 65519.99, 65520, 65536, 1e9, -65520, 2.0 ** -25, 2.0 ** -24 * 1.5,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0, -0.0], dtype=np.float32),
    ])
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------- scale packing ----

def test_scale_min_unpack_hand_decoded_bytes():
    # Bytes chosen by hand; expected values read off the layout table:
    # j<4: sc=s[j]&63, m=s[j+4]&63; j>=4: sc=(s[j+4]&15)|(s[j-4]>>6)<<4,
    # m=(s[j+4]>>4)|(s[j]>>6)<<4.
    s = bytes([0xC5, 0x40, 0x3F, 0x81, 0x7F, 0xBE, 0x00, 0xC1, 0x9A, 0x0F, 0xF0, 0x66])
    want = {
        0: (0x05, 0x3F), 1: (0x00, 0x3E), 2: (0x3F, 0x00), 3: (0x01, 0x01),
        4: (0x0A | (3 << 4), 0x09 | (1 << 4)),
        5: (0x0F | (1 << 4), 0x00 | (2 << 4)),
        6: (0x00 | (0 << 4), 0x0F | (0 << 4)),
        7: (0x06 | (2 << 4), 0x06 | (3 << 4)),
    }
    for j, (sc, m) in want.items():
        assert oracle.q4k_get_scale_min(j, s) == (sc, m), j


def test_scale_min_pack_unpack_brute_force_all_values_every_slot():
    g = np.random.default_rng(7)
    combos = np.array([(sc, m) for sc in range(64) for m in range(64)])
    for j in range(8):
        for i in range(0, len(combos)):
            sc = g.integers(0, 64, 8)
            m = g.integers(0, 64, 8)
            sc[j], m[j] = combos[i]
            packed = oracle.q4k_set_scale_min(sc, m)
            got = oracle.q4k_get_scale_min(j, packed)
            assert got == (int(sc[j]), int(m[j]))
            if i % 512 == 0:   # the other slots must survive too
                for jj in range(8):
                    assert oracle.q4k_get_scale_min(jj, packed) == (int(sc[jj]), int(m[jj]))


# ------------------------------------------------------------- dequant ----

def _block(d16: int, dmin16: int, scales12: bytes, nibbles) -> np.ndarray:
    """Assemble one 144-byte block from fields; nibble order per the layout:
    byte 32c+l holds weight 64c+l (low) and 64c+32+l (high)."""
    nib = np.asarray(nibbles, dtype=np.int64)
    qs = np.zeros(128, dtype=np.uint8)
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = nib[64 * c + l] | (nib[64 * c + 32 + l] << 4)
    head = np.array([d16 & 255, d16 >> 8, dmin16 & 255, dmin16 >> 8], dtype=np.uint8)
    return np.concatenate([head, np.frombuffer(scales12, dtype=np.uint8), qs])


def test_block_size_constants():
    f = _fmt()
    assert f["q4k_weights_per_block"]["value"] == oracle.QK_K == 256
    assert f["q4k_block_bytes"]["value"] == oracle.BLOCK_BYTES == 144
    w = np.zeros((3, 512), np.float32)
    assert oracle.q4k_quantize(w).size == 3 * 2 * 144


def test_dequant_zero_scales_give_zero():
    blk = _block(0, 0, bytes(range(12)), np.arange(256) % 16)
    assert np.all(oracle.q4k_dequantize(blk) == 0.0)


def test_dequant_nibble_order_unit_scale():
    # d = 1, dmin = 0.5 (fp16 0x3C00 / 0x3800), every sc = 1 and m = 0:
    # w_i equals weight i's nibble, which pins the nibble order.
    sc = oracle.q4k_set_scale_min([1] * 8, [0] * 8)
    nib = (np.arange(256) * 7 + 3) % 16
    got = oracle.q4k_dequantize(_block(0x3C00, 0x3800, sc, nib))
    assert np.array_equal(got, nib.astype(np.float32))


def test_dequant_zero_nibbles_give_minus_dmin_m():
    m = [0, 1, 2, 13, 32, 47, 62, 63]
    sc = oracle.q4k_set_scale_min([63] * 8, m)
    got = oracle.q4k_dequantize(_block(0x3C00, 0x3400, sc, np.zeros(256, int)))  # dmin=0.25
    want = np.repeat(-0.25 * np.array(m, dtype=np.float64), 32).astype(np.float32)
    assert np.array_equal(got, want)


def test_dequant_max_fields_high_slot_path():
    # sc = m = 63 everywhere (exercises the two high bits of slots 4..7),
    # d = 2^-10 (0x1400), dmin = 2^-12 (0x0C00), nibbles 15:
    # w = 2^-10*63*15 - 2^-12*63
    sc = oracle.q4k_set_scale_min([63] * 8, [63] * 8)
    got = oracle.q4k_dequantize(_block(0x1400, 0x0C00, sc, np.full(256, 15)))
    assert np.all(got == np.float32(2.0 ** -10 * 63 * 15 - 2.0 ** -12 * 63))


def test_dequant_distinct_slots():
    scv = [3, 5, 7, 11, 17, 33, 49, 62]
    mv = [60, 2, 31, 1, 48, 16, 63, 9]
    sc = oracle.q4k_set_scale_min(scv, mv)
    nib = np.arange(256) % 16
    got = oracle.q4k_dequantize(_block(0x3C00, 0x3C00, sc, nib)).astype(np.float64)
    j = np.arange(256) // 32
    want = np.array(scv)[j] * nib - np.array(mv)[j]
    assert np.array_equal(got, want)


def test_dequant_is_exact_in_float32_any_order():
    """The fp32 value (d*sc)*q - dmin*m is exact, so a float-only evaluation
    equals the oracle's double evaluation rounded once, bit for bit."""
    g = np.random.default_rng(11)
    nblk = 400
    raw = g.integers(0, 256, (nblk, 144), dtype=np.uint8)
    # keep d and dmin finite (exponent field < 31)
    for off in (1, 3):
        raw[:, off] &= 0x7B
    got = oracle.q4k_dequantize(raw.reshape(-1)).reshape(nblk, 256)
    d = raw[:, 0:2].copy().view(np.float16).astype(np.float32).reshape(-1)
    dmin = raw[:, 2:4].copy().view(np.float16).astype(np.float32).reshape(-1)
    for b in range(0, nblk, 9):
        s = raw[b, 4:16].tobytes()
        # float32 two ways: (d*sc)*q - dmin*m and d*(sc*q) - (dmin*m)
        sc_m = np.array([oracle.q4k_get_scale_min(jj, s) for jj in range(8)], dtype=np.float32)
        qs = raw[b, 16:]
        nib = np.empty(256, np.float32)
        for c in range(4):
            nib[64 * c:64 * c + 32] = qs[32 * c:32 * c + 32] & 15
            nib[64 * c + 32:64 * c + 64] = qs[32 * c:32 * c + 32] >> 4
        scj = np.repeat(sc_m[:, 0], 32)
        mj = np.repeat(sc_m[:, 1], 32)
        a = (d[b] * scj) * nib - dmin[b] * mj
        c2 = d[b] * (scj * nib) - (mj * dmin[b])
        assert np.array_equal(a.view(np.uint32), got[b].view(np.uint32))
        assert np.array_equal(c2.view(np.uint32), got[b].view(np.uint32))


# ----------------------------------------------------------- quantizer ----

def _on_grid_block(g, d16, dmin16):
    d = float(np.uint16(d16).view(np.float16))
    dmin = float(np.uint16(dmin16).view(np.float16))
    sc = g.integers(1, 64, 8)
    sc[g.integers(0, 8)] = 63
    m = g.integers(0, 64, 8)
    m[g.integers(0, 8)] = 63
    q = g.integers(0, 16, 256)
    for j in range(8):   # each sub-block holds both q=0 and q=15
        i0, i1 = g.choice(32, 2, replace=False)
        q[32 * j + i0] = 0
        q[32 * j + i1] = 15
    w = (d * np.repeat(sc, 32) * q - dmin * np.repeat(m, 32)).astype(np.float32)
    blk = _block(d16, dmin16, oracle.q4k_set_scale_min(sc, m), q)
    return w, blk


def test_quantizer_reencodes_on_grid_blocks_exactly():
    """Weights built as d*sc*q - dmin*m with the extreme codes present come back
    as the same 144 bytes: pins d/dmin selection, scale packing and nibble order."""
    g = np.random.default_rng(5)
    for d16, dmin16 in [(0x1C00, 0x1800), (0x2000, 0x2400), (0x3C00, 0x3800), (0x0400, 0x0800)]:
        ws, blks = zip(*[_on_grid_block(g, d16, dmin16) for _ in range(16)])
        w = np.concatenate(ws).reshape(4, 1024)
        got = oracle.q4k_quantize(w)
        assert np.array_equal(got, np.concatenate(blks))


def test_quantizer_error_bound_and_zero_rows():
    g = np.random.default_rng(9)
    w = (g.standard_normal((32, 2048)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4, :256] = -0.5          # constant negative sub-blocks
    blocks = oracle.q4k_quantize(w)
    back = oracle.q4k_dequantize(blocks).reshape(w.shape)
    assert np.all(back[3] == 0)
    # per sub-block, error stays within one full quantization step of the range
    sub = w.reshape(-1, 32)
    rng_ = np.maximum(sub.max(1), 0) - np.minimum(sub.min(1), 0)
    err = np.abs(back - w).reshape(-1, 32).max(1)
    assert np.all(err <= rng_ / 15.0 * 1.0 + 1e-6)
    rel = np.sqrt(np.mean((back - w) ** 2)) / np.sqrt(np.mean(w ** 2))
    assert rel < 0.15


def test_row_and_expert_byte_counts():
    f = _fmt()
    assert "(k/256)*144" == f["q4k_row_bytes_formula"]["value"]
    assert oracle.q4k_matrix_bytes(768, 2048) == 884_736        # gate/up, hidden 2048
    assert oracle.q4k_matrix_bytes(2048, 768) == 884_736        # down
    assert oracle.q4k_matrix_bytes(2048, 7168) == 8_257_536     # gate/up, hidden 7168
    assert oracle.q4k_matrix_bytes(7168, 2048) == 8_257_536
    assert 3 * 884_736 == 2_654_208
