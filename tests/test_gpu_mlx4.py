"""GPU parity of the MLX affine 4-bit codec (moeflux expert_forward.rs: 4-bit
experts, bf16 scale and bias per 64 weights, packed / scales / biases at
offsets inside an expert block) against the CPU oracle on the same seeded
inputs: dequantized weights and encoded bytes bit for bit, the id-GEMV within
max_abs_diff <= 1e-3*max|out| and cosine >= 0.9999, unit-vector probes and
batched-vs-per-token calls bit for bit."""
import sys

import numpy as np
import pytest

import oracle
import bit_quantized_moe_superblock_amd as q4
from _util import band, bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
G = oracle.MLX_GROUP


def say(msg):
    print(f"[gpu-mlx4] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    q4._lib.load()
    return torch.device("cuda:0")


def T(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def sync_np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _blob(experts, extra=0):
    """Expert blocks: per expert the packed weights, scales and biases of one
    matrix, each sub-tensor 16-byte aligned, after `extra` leading bytes (room
    another tensor of the block would take)."""
    packed, s, b = experts[0]
    po = extra
    so = po + (packed.nbytes + 15) // 16 * 16
    bo = so + (s.nbytes + 15) // 16 * 16
    stride = bo + (b.nbytes + 15) // 16 * 16
    blob = np.zeros(len(experts) * stride, np.uint8)
    for e, (p, sc, bi) in enumerate(experts):
        for a, o in ((p, po), (sc, so), (bi, bo)):
            flat = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
            blob[e * stride + o: e * stride + o + flat.size] = flat
    return blob, stride, (po, so, bo)


def _experts(g, E, n, k, touched=None, std=0.02):
    """E experts; the touched ones hold oracle-encoded N(0, std^2) weights,
    the rest zero bytes (never read by a correct kernel)."""
    zero = (np.zeros((n, k // 2), np.uint8), np.zeros((n, k // G), np.uint16),
            np.zeros((n, k // G), np.uint16))
    touched = set(range(E)) if touched is None else set(int(e) for e in touched)
    return [oracle.mlx4_quantize((g.standard_normal((n, k)) * std).astype(np.float32))
            if e in touched else zero for e in range(E)]


def _gemv(dev, blob, stride, offs, x, ids, n, k, m, K, outer, inner, E):
    out = torch.empty(m * K, n, device=dev)
    q4.mlx4_moe_id_gemv(T(blob, dev), stride, *offs, T(x, dev), T(ids, dev), out, n, k, m, K,
                        outer, inner, E)
    return sync_np(out)


def test_mlx4_dequant_bit_exact(dev):
    g = np.random.default_rng(70)
    for n, k in [(37, 320), (5, 64), (2, 16384)]:
        say(f"dequant n={n} k={k}")
        packed = g.integers(0, 256, (n, k // 2), dtype=np.uint8)
        sv = g.standard_normal((n, k // G)) * 10.0 ** g.integers(-4, 2, (n, k // G))
        bv = g.standard_normal((n, k // G)) * 10.0 ** g.integers(-4, 2, (n, k // G))
        s = np.array([oracle.f32_to_bf16(float(v)) for v in sv.reshape(-1)], np.uint16)
        b = np.array([oracle.f32_to_bf16(float(v)) for v in bv.reshape(-1)], np.uint16)
        want = oracle.mlx4_dequantize(packed, s, b, n, k)
        out = torch.empty(n, k, device=dev)
        q4.mlx4_dequantize(T(packed, dev), T(s.view(np.int16), dev), T(b.view(np.int16), dev),
                           out, n, k)
        assert np.array_equal(bits(sync_np(out)), bits(want))


def test_mlx4_quantize_bytes_bit_exact(dev):
    g = np.random.default_rng(71)
    cases = [(g.standard_normal((96, 2048)) * 0.02).astype(np.float32),
             (g.standard_normal((33, 448)) + 0.3).astype(np.float32),
             np.full((3, 128), -1.25, np.float32)]
    for w in cases:
        n, k = w.shape
        say(f"quantize n={n} k={k}")
        p_o, s_o, b_o = oracle.mlx4_quantize(w)
        p = torch.empty(n, k // 2, dtype=torch.uint8, device=dev)
        s = torch.empty(n, k // G, dtype=torch.int16, device=dev)
        b = torch.empty(n, k // G, dtype=torch.int16, device=dev)
        q4.mlx4_quantize(T(w, dev), p, s, b, n, k)
        assert np.array_equal(sync_np(p), p_o)
        assert np.array_equal(sync_np(s).view(np.uint16), s_o)
        assert np.array_equal(sync_np(b).view(np.uint16), b_o)


CASES = [
    # name, E, n, k, m, K, mode, extra leading bytes in the block
    ("tiny gate/up", 4, 64, 256, 3, 2, "gate_up", 0),
    ("decode gate, m=1", 128, 768, 2048, 1, 8, "gate_up", 0),
    ("decode down, m=2", 128, 2048, 768, 2, 8, "down", 48),
    ("decode gate, m=16", 128, 768, 2048, 16, 8, "gate_up", 0),
    ("ragged n, one group", 5, 100, 64, 3, 3, "down", 16),
    ("widest row", 2, 8, 16384, 1, 2, "gate_up", 0),
    ("k=4096 two waves' rows", 3, 40, 4096, 2, 2, "gate_up", 1024),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mlx4_id_gemv_matches_oracle(dev, case):
    name, E, n, k, m, K, mode, extra = case
    say(f"id-GEMV {name}: E={E} n={n} k={k} m={m} K={K} {mode}")
    g = np.random.default_rng(80 + CASES.index(case))
    ids = np.stack([g.choice(E, K, replace=False) for _ in range(m)]).reshape(-1).astype(np.int32)
    experts = _experts(g, E, n, k, touched=ids)
    blob, stride, offs = _blob(experts, extra)
    if mode == "gate_up":
        x = g.standard_normal((m, k)).astype(np.float32)
        outer, inner = k, 0
    else:
        x = g.standard_normal((m * K, k)).astype(np.float32)
        outer, inner = K * k, k
    want = oracle.mlx4_moe_id_gemv(blob, stride, *offs, E, n, k, x, ids, m, K, outer, inner)
    got = _gemv(dev, blob, stride, offs, x, ids, n, k, m, K, outer, inner, E)
    r = band(got, want, name)
    say(f"  rel {r[0]:.3g} cos {r[1]:.9f}")
    # batched equals per-token calls bit for bit
    if m > 1:
        for t in range(m):
            xt = x[t:t + 1] if mode == "gate_up" else x[t * K:(t + 1) * K]
            one = _gemv(dev, blob, stride, offs, xt, ids[t * K:(t + 1) * K], n, k, 1, K, outer,
                        inner, E)
            assert np.array_equal(bits(one), bits(got[t * K:(t + 1) * K]))


def test_mlx4_invalid_ids_and_unit_vector_probe(dev):
    g = np.random.default_rng(72)
    E, n, k = 6, 48, 512
    experts = _experts(g, E, n, k, std=0.3)
    blob, stride, offs = _blob(experts, 32)
    ids = np.array([3, E, -1, 0], np.int32)
    for c in (0, 1, 63, 64, 130, k - 1):
        say(f"unit-vector probe column {c}")
        x = np.zeros((1, k), np.float32)
        x[0, c] = 1.0
        got = _gemv(dev, blob, stride, offs, x, ids, n, k, 1, 4, k, 0, E)
        for p, e in enumerate(ids):
            if 0 <= e < E:
                col = oracle.mlx4_dequantize(*experts[e], n, k)[:, c]
                assert np.array_equal(bits(got[p]), bits(col))
            else:
                assert np.all(got[p] == 0.0)


@pytest.mark.parametrize("shape", [(768, 2048, 1), (768, 2048, 16), (96, 448, 3)],
                         ids=["decode m=1", "decode m=16", "ragged"])
def test_mlx4_gate_up_silu_matches_oracle(dev, shape):
    """Fused gate/up + SiLU over one expert block holding the gate and up
    matrices: against silu(oracle gate) * oracle up, and bit for bit against
    per-token calls."""
    n, k, m = shape
    E, K = 128 if n == 768 else 9, 8
    say(f"gate/up + SiLU n={n} k={k} m={m}")
    g = np.random.default_rng(90 + m)
    ids = np.stack([g.choice(E, K, replace=False) for _ in range(m)]).reshape(-1).astype(np.int32)
    gate = _experts(g, E, n, k, touched=ids)
    up = _experts(g, E, n, k, touched=ids)
    # one block per expert: gate's packed | scales | biases, then up's
    gb, gstride, goffs = _blob(gate)
    ub, ustride, uoffs = _blob(up)
    stride = gstride + ustride
    blob = np.zeros(E * stride, np.uint8)
    for e in range(E):
        blob[e * stride:e * stride + gstride] = gb[e * gstride:(e + 1) * gstride]
        blob[e * stride + gstride:(e + 1) * stride] = ub[e * ustride:(e + 1) * ustride]
    uoffs = tuple(o + gstride for o in uoffs)
    x = g.standard_normal((m, k)).astype(np.float32)
    go = oracle.mlx4_moe_id_gemv(blob, stride, *goffs, E, n, k, x, ids, m, K, k, 0)
    uo = oracle.mlx4_moe_id_gemv(blob, stride, *uoffs, E, n, k, x, ids, m, K, k, 0)
    want = np.array([oracle.silu(float(a)) * float(b) for a, b in zip(go.reshape(-1),
                                                                       uo.reshape(-1))])
    d_blob, d_x, d_ids = T(blob, dev), T(x, dev), T(ids, dev)
    out = torch.empty(m * K, n, device=dev)
    q4.mlx4_moe_gate_up_silu(d_blob, stride, goffs, uoffs, d_x, d_ids, out, n, k, m, K, k, 0, E)
    got = sync_np(out)
    r = band(got, want.reshape(m * K, n), "gate/up + SiLU")
    say(f"  rel {r[0]:.3g} cos {r[1]:.9f}")
    for t in range(min(m, 4)):
        one = torch.empty(K, n, device=dev)
        q4.mlx4_moe_gate_up_silu(d_blob, stride, goffs, uoffs, d_x[t:t + 1], d_ids[t * K:(t + 1) * K],
                                 one, n, k, 1, K, k, 0, E)
        assert np.array_equal(bits(sync_np(one)), bits(got[t * K:(t + 1) * K]))


# ------------------------------------------------------------------ 2-bit ----

def _experts2(g, E, n, k, touched):
    zero = (np.zeros((n, k // 4), np.uint8), np.zeros((n, k // G), np.uint16),
            np.zeros((n, k // G), np.uint16))
    touched = set(int(e) for e in touched)
    return [oracle.mlx2_quantize((g.standard_normal((n, k)) * 0.02).astype(np.float32))
            if e in touched else zero for e in range(E)]


def test_mlx2_dequant_and_quantize_bit_exact(dev):
    g = np.random.default_rng(95)
    for n, k in [(37, 320), (3, 64), (2, 16384)]:
        say(f"2-bit dequant/quantize n={n} k={k}")
        packed = g.integers(0, 256, (n, k // 4), dtype=np.uint8)
        s = np.array([oracle.f32_to_bf16(float(v)) for v in g.standard_normal(n * k // G)],
                     np.uint16)
        b = np.array([oracle.f32_to_bf16(float(v)) for v in g.standard_normal(n * k // G)],
                     np.uint16)
        want = oracle.mlx2_dequantize(packed, s, b, n, k)
        out = torch.empty(n, k, device=dev)
        q4.mlx2_dequantize(T(packed, dev), T(s.view(np.int16), dev), T(b.view(np.int16), dev),
                           out, n, k)
        assert np.array_equal(bits(sync_np(out)), bits(want))
        w = (g.standard_normal((n, k)) * 0.02 + 0.01).astype(np.float32)
        p_o, s_o, b_o = oracle.mlx2_quantize(w)
        p = torch.empty(n, k // 4, dtype=torch.uint8, device=dev)
        sd = torch.empty(n, k // G, dtype=torch.int16, device=dev)
        bd = torch.empty(n, k // G, dtype=torch.int16, device=dev)
        q4.mlx2_quantize(T(w, dev), p, sd, bd, n, k)
        assert np.array_equal(sync_np(p), p_o)
        assert np.array_equal(sync_np(sd).view(np.uint16), s_o)
        assert np.array_equal(sync_np(bd).view(np.uint16), b_o)


CASES2 = [("decode gate, m=1", 128, 768, 2048, 1, 8, "gate_up", 0),
          ("decode down, m=4", 128, 2048, 768, 4, 8, "down", 32),
          ("ragged, one group", 5, 100, 64, 3, 3, "down", 16),
          ("widest row", 2, 8, 16384, 1, 2, "gate_up", 0)]


@pytest.mark.parametrize("case", CASES2, ids=[c[0] for c in CASES2])
def test_mlx2_id_gemv_matches_oracle(dev, case):
    name, E, n, k, m, K, mode, extra = case
    say(f"2-bit id-GEMV {name}")
    g = np.random.default_rng(96 + CASES2.index(case))
    ids = np.stack([g.choice(E, K, replace=False) for _ in range(m)]).reshape(-1).astype(np.int32)
    ids[-1] = E + 2   # an invalid id: zero row
    blob, stride, offs = _blob(_experts2(g, E, n, k, ids[:-1]), extra)
    if mode == "gate_up":
        x = g.standard_normal((m, k)).astype(np.float32)
        outer, inner = k, 0
    else:
        x = g.standard_normal((m * K, k)).astype(np.float32)
        outer, inner = K * k, k
    want = oracle.mlx2_moe_id_gemv(blob, stride, *offs, E, n, k, x, ids, m, K, outer, inner)
    out = torch.empty(m * K, n, device=dev)
    q4.mlx2_moe_id_gemv(T(blob, dev), stride, *offs, T(x, dev), T(ids, dev), out, n, k, m, K,
                        outer, inner, E)
    got = sync_np(out)
    assert np.all(got[-1] == 0.0)
    r = band(got, want, name)
    say(f"  rel {r[0]:.3g} cos {r[1]:.9f}")
