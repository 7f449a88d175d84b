"""The C-ABI library loads and exports every entry point include/q4kmoe.h
declares, and rejects bad arguments on the host before any HIP call (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

import bit_quantized_moe_superblock_amd as q4
from bit_quantized_moe_superblock_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4kmoe.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "q4kceil.h")]


def _declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no Python binding"
    assert set(_lib.SIGNATURES) == set(names)


def test_constants_match_header(lib):
    src = open(HEADER).read()
    for name, val in [("Q4K_BLOCK_WEIGHTS", 256), ("Q4K_BLOCK_BYTES", 144), ("Q4K_MAX_TOP_K", 16),
                      ("Q4K_MAX_IN", _lib.Q4K_MAX_IN), ("Q4K_MAX_EXPERTS", _lib.Q4K_MAX_EXPERTS),
                      ("Q4K_MAX_PAIRS", _lib.Q4K_MAX_PAIRS), ("Q4TP_MAX_COLS", _lib.Q4TP_MAX_COLS),
                      ("Q4K_BUCKET_CHUNK", 8), ("Q4K_BUCKET_MODE_MASK", "0xFF"),
                      ("Q4K_SCHED_VECTOR", "0x100"), ("Q4K_SCHED_BUCKET_LAUNCH", "0x200"),
                      ("Q4K_AUTO_BUCKET_MIN_TOKENS", _lib.Q4K_AUTO_BUCKET_MIN_TOKENS),
                      ("Q4TP_MAX_TENSORS", _lib.Q4TP_MAX_TENSORS), ("MLX4_GROUP", 64)]:
        assert re.search(rf"#define {name} {val}\b", src), name
    assert (_lib.Q4K_BUCKET_MODE_MASK, _lib.Q4K_SCHED_VECTOR, _lib.Q4K_SCHED_BUCKET_LAUNCH) == \
        (0xFF, 0x100, 0x200)
    assert q4.q4k_abi_version() == 4


def test_size_helpers(lib):
    assert q4.q4k_matrix_bytes(768, 2048) == 884_736
    assert q4.q4k_matrix_bytes(7168, 2048) == 8_257_536
    assert q4.q4k_matrix_bytes(4, 100) == -1
    assert q4.q4tp_tensor_bytes(1, 4096) == 2132
    assert q4.q4tp_tensor_bytes(1, 14336) == 7452
    assert q4.q4tp_tensor_bytes(3, 33) == -1
    # MLX 4-bit: k/2 packed bytes + 2 bf16 per 64 weights per row (the same
    # 4.5 bits per weight as Q4_K at these shapes)
    assert q4.mlx4_matrix_bytes(768, 2048) == 884_736
    assert q4.mlx4_matrix_bytes(2048, 768) == 884_736
    assert q4.mlx4_matrix_bytes(3, 96) == -1
    assert q4.mlx2_matrix_bytes(768, 2048) == 768 * 512 + 768 * 32 * 4
    assert q4.mlx2_matrix_bytes(3, 96) == -1
    assert q4.moe_bucket_workspace_bytes(128, 128) == 4 * (129 + 130 + 128 + 129 + 1 + 1 + 256)
    # act [9, 768] | expert_out [8, 2048] | shared_out [1, 2048] | buckets
    assert q4.moe_layer_workspace_bytes(2048, 768, 128, 1, 8) == 27648 + 65536 + 8192 + 1792


def test_status_strings(lib):
    for s in range(8):
        assert q4.status_string(s) and q4.status_string(s) != "unknown status"
    assert q4.status_string(99) == "unknown status"


FAKE = 1 << 20   # a non-null, 16-byte aligned address that is never dereferenced


def _err(fn, *args):
    with pytest.raises(q4.Q4KError) as e:
        fn(*args, stream=0)
    return e.value.status


def test_id_gemv_validation(lib):
    g = q4.q4k_moe_id_gemv
    ok = dict(n=64, k=256, m=3, top_k=2, outer=256, inner=0, E=4)

    def call(w=FAKE, x=FAKE, ids=FAKE, dst=FAKE, n=64, k=256, m=3, top_k=2, outer=256, inner=0,
             E=4, flag=q4.Q4K_BUCKET_OFF, ws=None, wsb=0):
        return _err(g, w, x, ids, dst, n, k, m, top_k, outer, inner, E, flag, ws, wsb)

    assert call(k=100) == _lib.Q4K_ERR_SHAPE
    assert call(k=0) == _lib.Q4K_ERR_SHAPE
    assert call(k=16384 + 256) == _lib.Q4K_ERR_SHAPE
    assert call(n=0) == _lib.Q4K_ERR_SHAPE
    assert call(m=0) == _lib.Q4K_ERR_SHAPE
    assert call(top_k=0) == _lib.Q4K_ERR_SHAPE
    assert call(top_k=17) == _lib.Q4K_ERR_SHAPE
    assert call(E=0) == _lib.Q4K_ERR_SHAPE
    assert call(E=1024) == _lib.Q4K_ERR_SHAPE
    assert call(w=None) == _lib.Q4K_ERR_NULL
    assert call(w=FAKE + 8) == _lib.Q4K_ERR_NULL       # weights need 16-byte alignment
    assert call(dst=None) == _lib.Q4K_ERR_NULL
    assert call(outer=-1) == _lib.Q4K_ERR_STRIDE
    assert call(inner=-5) == _lib.Q4K_ERR_STRIDE
    assert call(flag=7) == _lib.Q4K_ERR_ARG
    assert call(flag=q4.Q4K_BUCKET_ON | 0x400) == _lib.Q4K_ERR_ARG    # unknown schedule bit
    assert call(flag=q4.Q4K_BUCKET_ON) == _lib.Q4K_ERR_WORKSPACE
    assert call(flag=q4.Q4K_BUCKET_ON | q4.Q4K_SCHED_VECTOR) == _lib.Q4K_ERR_WORKSPACE
    assert call(flag=q4.Q4K_BUCKET_ON, ws=FAKE, wsb=8) == _lib.Q4K_ERR_WORKSPACE
    # AUTO buckets from Q4K_AUTO_BUCKET_MIN_TOKENS tokens on, so only then
    # does it need a workspace
    mt = q4.Q4K_AUTO_BUCKET_MIN_TOKENS
    assert call(m=mt, flag=q4.Q4K_BUCKET_AUTO) == _lib.Q4K_ERR_WORKSPACE
    assert call(m=mt - 1, flag=q4.Q4K_BUCKET_AUTO, x=None) == _lib.Q4K_ERR_NULL
    assert call(x=FAKE + 2) == _lib.Q4K_ERR_NULL      # activations need 4-byte alignment


def test_ffn_combine_bucket_q4tp_validation(lib):
    f = q4.moe_expert_ffn
    base = [FAKE] * 7
    assert _err(f, *base, 2048, 700, 8, 1, 8) == _lib.Q4K_ERR_SHAPE       # inter % 256
    assert _err(f, *base, 2048, 768, 8, 1, 0) == _lib.Q4K_ERR_SHAPE
    bad = list(base)
    bad[4] = None
    assert _err(f, *bad, 2048, 768, 8, 1, 8) == _lib.Q4K_ERR_NULL
    c = q4.moe_combine_residual
    assert _err(c, FAKE, FAKE, FAKE, None, None, FAKE, 64, 1, 8, 3) == _lib.Q4K_ERR_ARG
    assert _err(c, FAKE, FAKE, FAKE, None, None, FAKE, 64, 1, 8, 1) == _lib.Q4K_ERR_NULL
    assert _err(c, FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 1, 8, 1) == _lib.Q4K_ERR_NULL
    assert _err(c, FAKE, FAKE, FAKE, None, None, FAKE, 0, 1, 8, 0) == _lib.Q4K_ERR_SHAPE
    b = q4.moe_bucket
    assert _err(b, FAKE, 0, 8, FAKE, 1 << 20) == _lib.Q4K_ERR_SHAPE
    assert _err(b, FAKE, 8193, 8, FAKE, 1 << 20) == _lib.Q4K_ERR_SHAPE
    assert _err(b, FAKE, 16, 8, FAKE, 4) == _lib.Q4K_ERR_WORKSPACE
    m = q4.q4tp_matvec
    assert _err(m, FAKE, FAKE, FAKE, 4, 48) == _lib.Q4K_ERR_SHAPE
    assert _err(m, FAKE, FAKE, FAKE, 4, 16384 + 32) == _lib.Q4K_ERR_SHAPE
    assert _err(m, None, FAKE, FAKE, 4, 64) == _lib.Q4K_ERR_NULL
    mm = q4.q4tp_matvec_multi
    assert _err(mm, [], [], FAKE, FAKE, 64) == _lib.Q4K_ERR_SHAPE
    assert _err(mm, [FAKE] * 4, [4] * 4, FAKE, FAKE, 64) == _lib.Q4K_ERR_SHAPE
    assert _err(mm, [FAKE, FAKE], [4, 0], FAKE, FAKE, 64) == _lib.Q4K_ERR_SHAPE
    assert _err(mm, [FAKE, FAKE], [4, 4], FAKE, FAKE, 48) == _lib.Q4K_ERR_SHAPE
    assert _err(mm, [FAKE, FAKE], [1 << 30, 4], FAKE, FAKE, 64) == _lib.Q4K_ERR_SHAPE
    assert _err(mm, [FAKE, None], [4, 4], FAKE, FAKE, 64) == _lib.Q4K_ERR_NULL
    assert _err(mm, [FAKE, FAKE + 8], [4, 4], FAKE, FAKE, 64) == _lib.Q4K_ERR_NULL
    assert _err(mm, [FAKE], [4], FAKE + 2, FAKE, 64) == _lib.Q4K_ERR_NULL
    assert _err(q4.q4k_quantize, FAKE, FAKE, 2, 300) == _lib.Q4K_ERR_SHAPE
    assert _err(q4.q4k_dequantize, FAKE, FAKE, -1) == _lib.Q4K_ERR_SHAPE
    assert _err(q4.q4tp_quantize, FAKE, FAKE, 2, 40) == _lib.Q4K_ERR_SHAPE
    lf = q4.moe_layer_forward
    st = [FAKE] * 6
    io = [FAKE] * 6
    need = q4.moe_layer_workspace_bytes(512, 256, 4, 2, 2)
    assert _err(lf, *st, *io, 512, 256, 4, 2, 2, 1, 0x7, FAKE, need) == _lib.Q4K_ERR_ARG
    assert _err(lf, *st, *io, 512, 256, 4, 2, 2, 1, 0x802, FAKE, need) == _lib.Q4K_ERR_ARG
    assert _err(lf, *st, *io, 512, 256, 4, 2, 2, 1, 0, FAKE, need - 4) == _lib.Q4K_ERR_WORKSPACE
    assert _err(lf, *st, *io, 512, 256, 4, 2, 2, 1, 0, None, need) == _lib.Q4K_ERR_WORKSPACE
    # the no-allocation layer: sizes past its static scratch are refused
    # before any HIP call
    na = q4.moe_layer_forward_noalloc
    assert q4.moe_layer_workspace_bytes(7168, 2048, 256, 48, 8) <= q4.MOE_LAYER_NOALLOC_MAX_BYTES
    assert q4.moe_layer_workspace_bytes(7168, 2048, 256, 64, 8) > q4.MOE_LAYER_NOALLOC_MAX_BYTES
    assert _err(na, *st, *io, 7168, 2048, 256, 64, 8, 2, 0) == _lib.Q4K_ERR_SCRATCH
    assert _err(na, *st, *io, 7168, 2048, 256, 0, 8, 2, 0) == _lib.Q4K_ERR_SHAPE
    assert re.search(r"#define MOE_LAYER_NOALLOC_MAX_BYTES \(16 << 20\)", open(HEADER).read())


def test_binding_refuses_host_tensors(lib):
    import torch
    with pytest.raises(ValueError):
        q4.q4k_dequantize(torch.zeros(144, dtype=torch.uint8), FAKE, 1, stream=0)


def test_mlx4_validation(lib):
    g = q4.mlx4_moe_id_gemv
    n, k = 64, 256
    stride = q4.mlx4_matrix_bytes(n, k)
    so, bo = n * k // 2, n * k // 2 + n * k // 32

    def call(base=FAKE, st=stride, po=0, s_off=so, b_off=bo, x=FAKE, ids=FAKE, dst=FAKE, n=n,
             k=k, m=3, top_k=2, outer=k, inner=0, E=4):
        return _err(g, base, st, po, s_off, b_off, x, ids, dst, n, k, m, top_k, outer, inner, E)

    assert call(k=96) == _lib.Q4K_ERR_SHAPE
    assert call(k=0) == _lib.Q4K_ERR_SHAPE
    assert call(k=16384 + 64) == _lib.Q4K_ERR_SHAPE
    assert call(n=0) == _lib.Q4K_ERR_SHAPE
    assert call(m=0) == _lib.Q4K_ERR_SHAPE
    assert call(top_k=17) == _lib.Q4K_ERR_SHAPE
    assert call(E=0) == _lib.Q4K_ERR_SHAPE
    assert call(st=stride - 2) == _lib.Q4K_ERR_SHAPE      # biases past the block
    assert call(po=stride - n * k // 2 + 16) == _lib.Q4K_ERR_SHAPE   # packed past the block
    assert call(po=-16) == _lib.Q4K_ERR_SHAPE
    assert call(outer=-1) == _lib.Q4K_ERR_STRIDE
    assert call(base=None) == _lib.Q4K_ERR_NULL
    assert call(base=FAKE + 8) == _lib.Q4K_ERR_NULL
    assert call(st=stride + 8) == _lib.Q4K_ERR_NULL       # stride not 16-byte aligned
    assert call(s_off=so + 1) == _lib.Q4K_ERR_NULL
    assert call(dst=None) == _lib.Q4K_ERR_NULL
    f = q4.mlx4_moe_gate_up_silu
    goffs, uoffs = (0, so, bo), (0, so, bo)
    past = stride - n * k // 2 + 16
    assert _err(f, FAKE, stride, goffs, (past, so, bo), FAKE, FAKE, FAKE, n, k, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_SHAPE                                 # up's packed runs past the block
    assert _err(f, FAKE, stride, goffs, (0, so, bo + 1), FAKE, FAKE, FAKE, n, k, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_SHAPE                                 # up's biases run past the block
    assert _err(f, FAKE, stride, goffs, uoffs, FAKE, FAKE, None, n, k, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_NULL
    assert _err(f, FAKE, stride, goffs, uoffs, FAKE, FAKE, FAKE, n, k, 1, 2, -k, 0, 4) == \
        _lib.Q4K_ERR_STRIDE
    d = q4.mlx4_dequantize
    assert _err(d, FAKE, FAKE, FAKE, FAKE, 4, 100) == _lib.Q4K_ERR_SHAPE
    assert _err(d, FAKE, FAKE + 1, FAKE, FAKE, 4, 128) == _lib.Q4K_ERR_NULL
    qz = q4.mlx4_quantize
    assert _err(qz, FAKE, FAKE, FAKE, FAKE, 4, 32) == _lib.Q4K_ERR_SHAPE
    assert _err(qz, FAKE, FAKE + 4, FAKE, FAKE, 4, 64) == _lib.Q4K_ERR_NULL


def test_rmsnorm_chain_validation(lib):
    c = q4.moe_combine_residual_rmsnorm
    ok = [FAKE, FAKE, FAKE, None, None, FAKE, 1e-6, FAKE, FAKE + 4096, 64, 2, 2, 0]

    def call(i=None, v=None):
        args = list(ok)
        if i is not None:
            args[i] = v
        return _err(c, *args)

    assert call(9, 0) == _lib.Q4K_ERR_SHAPE          # hidden
    assert call(10, 0) == _lib.Q4K_ERR_SHAPE         # m
    assert call(11, 17) == _lib.Q4K_ERR_SHAPE        # top_k
    assert call(12, 5) == _lib.Q4K_ERR_ARG           # shared mode
    assert call(6, -1.0) == _lib.Q4K_ERR_ARG         # eps
    assert call(6, float("nan")) == _lib.Q4K_ERR_ARG
    assert call(5, None) == _lib.Q4K_ERR_NULL        # norm weight
    assert call(5, FAKE + 1) == _lib.Q4K_ERR_NULL
    assert call(8, FAKE) == _lib.Q4K_ERR_NULL        # normed == out
    assert call(12, 1) == _lib.Q4K_ERR_NULL          # sigmoid mode needs shared and logit
    f = q4.moe_layer_forward_rmsnorm
    base = [FAKE] * 12
    assert _err(f, *base, None, 1e-6, FAKE, 512, 256, 4, 1, 2, 0) == _lib.Q4K_ERR_NULL
    assert _err(f, *base, FAKE, -1.0, FAKE + 4096, 512, 256, 4, 1, 2, 0) == _lib.Q4K_ERR_ARG
    assert _err(f, *base, FAKE, 1e-6, FAKE, 512, 256, 4, 1, 2, 0) == _lib.Q4K_ERR_NULL


def test_mlx2_validation(lib):
    g = q4.mlx2_moe_id_gemv
    n, k = 64, 256
    stride = q4.mlx2_matrix_bytes(n, k)
    so, bo = n * k // 4, n * k // 4 + n * k // 32
    assert _err(g, FAKE, stride, 0, so, bo, FAKE, FAKE, FAKE, n, 96, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_SHAPE
    assert _err(g, FAKE, stride - 2, 0, so, bo, FAKE, FAKE, FAKE, n, k, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_SHAPE                              # biases run past the block
    assert _err(g, FAKE, stride, 8, so, bo, FAKE, FAKE, FAKE, n, k, 1, 2, k, 0, 4) == \
        _lib.Q4K_ERR_NULL                               # packed offset not 16-byte aligned
    assert _err(q4.mlx2_dequantize, FAKE, FAKE, FAKE, FAKE, 4, 100) == _lib.Q4K_ERR_SHAPE
    assert _err(q4.mlx2_quantize, FAKE, FAKE + 8, FAKE, FAKE, 4, 64) == _lib.Q4K_ERR_NULL
