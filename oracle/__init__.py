"""CPU oracle for the Q4_K MoE expert path, the Q4TiledP dense matvec and the
MLX affine 4-bit expert codec.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product library
never imports this package, and this package imports nothing from the product
package.  The arithmetic lives in ``q4k_oracle.c`` (plain scalar C, double
accumulation); this module only marshals numpy arrays through ctypes.

Parity status per function is stated in ``q4k_oracle.c``; every function is
pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4k_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_q4k.so")

QK_K = 256
BLOCK_BYTES = 144
SHARED_NONE, SHARED_SIGMOID, SHARED_UNSCALED = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sig = {
        "orc_f16_value": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_q4k_get_scale_min": (None, [ctypes.c_int, P, P, P]),
        "orc_q4k_set_scale_min": (None, [P, P, P]),
        "orc_q4k_nibble": (ctypes.c_int, [P, ctypes.c_int]),
        "orc_q4k_dequantize": (None, [P, I64, P]),
        "orc_q4k_quantize": (ctypes.c_int, [P, I64, I64, P]),
        "orc_q4k_moe_id_gemv": (ctypes.c_int, [P, I64, I64, I64, P, P, I64, I64, I64, I64, P]),
        "orc_q4k_moe_id_gemv_one": (ctypes.c_float, [P, I64, I64, I64, P, P, I64, I64, I64, I64, I64]),
        "orc_silu": (ctypes.c_double, [ctypes.c_double]),
        "orc_sigmoid": (ctypes.c_double, [ctypes.c_double]),
        "orc_moe_expert_ffn": (ctypes.c_int, [P, P, P, I64, I64, I64, P, P, I64, I64, P, P, P, P]),
        "orc_moe_combine_residual": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I64, ctypes.c_int]),
        "orc_moe_bucket": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "orc_q4tp_bytes": (I64, [I64, I64]),
        "orc_q4tp_code": (ctypes.c_int, [P, I64, I64, I64, I64]),
        "orc_q4tp_rung": (ctypes.c_float, [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int]),
        "orc_q4tp_nibble": (ctypes.c_int, [P, I64, I64, I64]),
        "orc_q4tp_dequantize": (None, [P, I64, I64, P]),
        "orc_q4tp_matvec": (ctypes.c_int, [P, I64, I64, P, P]),
        "orc_q4tp_matvec_one": (ctypes.c_float, [P, I64, I64, P, I64]),
        "orc_q4tp_quantize": (ctypes.c_int, [P, I64, I64, P]),
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_mlx4_nibble": (ctypes.c_int, [P, I64]),
        "orc_mlx4_dequantize": (None, [P, P, P, I64, I64, P]),
        "orc_mlx4_quantize": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "orc_mlx4_moe_id_gemv": (ctypes.c_int, [P, I64, I64, I64, I64, I64, I64, I64, P, P,
                                                I64, I64, I64, I64, P]),
        "orc_rmsnorm_bf16": (ctypes.c_int, [P, P, ctypes.c_float, I64, I64, P]),
        "orc_mlx2_code": (ctypes.c_int, [P, I64]),
        "orc_mlx2_dequantize": (None, [P, P, P, I64, I64, P]),
        "orc_mlx2_quantize": (ctypes.c_int, [P, I64, I64, P, P, P]),
        "orc_mlx2_moe_id_gemv": (ctypes.c_int, [P, I64, I64, I64, I64, I64, I64, I64, P, P,
                                                I64, I64, I64, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# ---------------------------------------------------------------- fp16 ----

def f16_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(int(h)))


def f32_to_f16(x: float) -> int:
    return int(_load().orc_f32_to_f16(float(x)))


# ---------------------------------------------------------------- Q4_K ----

def q4k_matrix_bytes(n: int, k: int) -> int:
    return n * (k // QK_K) * BLOCK_BYTES


def q4k_get_scale_min(j: int, scales12: bytes):
    s = np.frombuffer(bytes(scales12), dtype=np.uint8).copy()
    sc = ctypes.c_int()
    m = ctypes.c_int()
    _load().orc_q4k_get_scale_min(j, _ptr(s), ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def q4k_set_scale_min(sc, m) -> bytes:
    out = np.zeros(12, dtype=np.uint8)
    sca = _c(sc, np.int32)
    ma = _c(m, np.int32)
    _load().orc_q4k_set_scale_min(_ptr(out), _ptr(sca), _ptr(ma))
    return out.tobytes()


def q4k_quantize(w: np.ndarray) -> np.ndarray:
    """fp32 [..., n, k] -> uint8 Q4_K blocks (flat, n*(k/256)*144 bytes per matrix)."""
    w = _c(w, np.float32)
    k = w.shape[-1]
    rows = w.size // k
    out = np.zeros(rows * (k // QK_K) * BLOCK_BYTES, dtype=np.uint8)
    _check(_load().orc_q4k_quantize(_ptr(w), rows, k, _ptr(out)), "q4k_quantize")
    return out


def q4k_dequantize(blocks: np.ndarray) -> np.ndarray:
    blocks = _c(blocks, np.uint8).reshape(-1)
    nb = blocks.size // BLOCK_BYTES
    out = np.zeros(nb * QK_K, dtype=np.float32)
    _load().orc_q4k_dequantize(_ptr(blocks), nb, _ptr(out))
    return out


def q4k_moe_id_gemv(w_stacked: np.ndarray, num_experts: int, n: int, k: int, src1: np.ndarray,
                    ids: np.ndarray, m: int, top_k: int, outer: int, inner: int) -> np.ndarray:
    w_stacked = _c(w_stacked, np.uint8)
    src1 = _c(src1, np.float32)
    ids = _c(ids, np.int32)
    dst = np.zeros((m * top_k, n), dtype=np.float32)
    _check(_load().orc_q4k_moe_id_gemv(_ptr(w_stacked), num_experts, n, k, _ptr(src1), _ptr(ids),
                                       m, top_k, outer, inner, _ptr(dst)), "q4k_moe_id_gemv")
    return dst


def q4k_moe_id_gemv_one(w_stacked, num_experts, n, k, src1, ids, top_k, outer, inner, p, r) -> float:
    return float(_load().orc_q4k_moe_id_gemv_one(
        _ptr(w_stacked), num_experts, n, k, _ptr(src1), _ptr(ids), top_k, outer, inner, p, r))


def silu(z: float) -> float:
    return float(_load().orc_silu(float(z)))


def sigmoid(z: float) -> float:
    return float(_load().orc_sigmoid(float(z)))


def moe_expert_ffn(w_gate, w_up, w_down, num_experts: int, hidden: int, inter: int,
                   h_post, ids, m: int, top_k: int):
    """Returns (gate_out, up_out, act, expert_out), all float32."""
    w_gate = _c(w_gate, np.uint8)
    w_up = _c(w_up, np.uint8)
    w_down = _c(w_down, np.uint8)
    h_post = _c(h_post, np.float32)
    ids = _c(ids, np.int32)
    P = m * top_k
    g = np.zeros((P, inter), np.float32)
    u = np.zeros((P, inter), np.float32)
    act = np.zeros((P, inter), np.float32)
    out = np.zeros((P, hidden), np.float32)
    _check(_load().orc_moe_expert_ffn(_ptr(w_gate), _ptr(w_up), _ptr(w_down), num_experts, hidden,
                                      inter, _ptr(h_post), _ptr(ids), m, top_k, _ptr(g), _ptr(u),
                                      _ptr(act), _ptr(out)), "moe_expert_ffn")
    return g, u, act, out


def moe_combine_residual(h_mid, expert_out, route_w, shared_out, shared_gate_logit,
                         hidden: int, m: int, top_k: int, shared_mode: int) -> np.ndarray:
    h_mid = _c(h_mid, np.float32)
    expert_out = _c(expert_out, np.float32)
    route_w = _c(route_w, np.float32)
    so = _c(shared_out if shared_out is not None else np.zeros(1), np.float32)
    sg = _c(shared_gate_logit if shared_gate_logit is not None else np.zeros(1), np.float32)
    out = np.zeros((m, hidden), np.float32)
    _check(_load().orc_moe_combine_residual(_ptr(h_mid), _ptr(expert_out), _ptr(route_w), _ptr(so),
                                            _ptr(sg), _ptr(out), hidden, m, top_k, shared_mode),
           "moe_combine_residual")
    return out


def moe_bucket(ids, num_experts: int):
    """Returns (counts[E+1], offsets[E+2], pairs[P]); bucket E holds invalid ids."""
    ids = _c(ids, np.int32).reshape(-1)
    P = ids.size
    counts = np.zeros(num_experts + 1, np.int32)
    offsets = np.zeros(num_experts + 2, np.int32)
    pairs = np.zeros(max(P, 1), np.int32)
    _check(_load().orc_moe_bucket(_ptr(ids), P, num_experts, _ptr(counts), _ptr(offsets),
                                  _ptr(pairs)), "moe_bucket")
    return counts, offsets, pairs[:P]


# ------------------------------------------------------------- Q4TiledP ----

def q4tp_bytes(rows: int, cols: int) -> int:
    return int(_load().orc_q4tp_bytes(rows, cols))


def q4tp_quantize(w: np.ndarray) -> np.ndarray:
    w = _c(w, np.float32)
    rows, cols = w.shape
    out = np.zeros(q4tp_bytes(rows, cols), np.uint8)
    _check(_load().orc_q4tp_quantize(_ptr(w), rows, cols, _ptr(out)), "q4tp_quantize")
    return out


def q4tp_dequantize(t: np.ndarray, rows: int, cols: int) -> np.ndarray:
    t = _c(t, np.uint8)
    out = np.zeros((rows, cols), np.float32)
    _load().orc_q4tp_dequantize(_ptr(t), rows, cols, _ptr(out))
    return out


def q4tp_code(t: np.ndarray, rows: int, cols: int, r: int, g: int) -> int:
    return int(_load().orc_q4tp_code(_ptr(t), rows, cols, r, g))


def q4tp_rung(base: int, step: int, code: int) -> float:
    return float(_load().orc_q4tp_rung(base, step, code))


def q4tp_nibble(t: np.ndarray, cols: int, r: int, c: int) -> int:
    return int(_load().orc_q4tp_nibble(_ptr(t), cols, r, c))


def q4tp_matvec(t: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    t = _c(t, np.uint8)
    x = _c(x, np.float32)
    y = np.zeros(rows, np.float32)
    _check(_load().orc_q4tp_matvec(_ptr(t), rows, cols, _ptr(x), _ptr(y)), "q4tp_matvec")
    return y


def q4tp_matvec_one(t: np.ndarray, rows: int, cols: int, x: np.ndarray, r: int) -> float:
    return float(_load().orc_q4tp_matvec_one(_ptr(t), rows, cols, _ptr(x), r))


# ------------------------------------------------------ MLX affine 4-bit ----

MLX_GROUP = 64


def bf16_to_f32(h: int) -> float:
    return float(_load().orc_bf16_to_f32(int(h)))


def f32_to_bf16(x: float) -> int:
    return int(_load().orc_f32_to_bf16(float(x)))


def mlx4_nibble(packed_row: np.ndarray, c: int) -> int:
    return int(_load().orc_mlx4_nibble(_ptr(_c(packed_row, np.uint8)), c))


def mlx4_quantize(w: np.ndarray):
    """fp32 [n, k] -> (packed uint8 [n, k/2], scales uint16 [n, k/64], biases uint16 [n, k/64])."""
    w = _c(w, np.float32)
    n, k = w.shape
    packed = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // MLX_GROUP), np.uint16)
    biases = np.zeros((n, k // MLX_GROUP), np.uint16)
    _check(_load().orc_mlx4_quantize(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(biases)),
           "mlx4_quantize")
    return packed, scales, biases


def mlx4_dequantize(packed, scales, biases, n: int, k: int) -> np.ndarray:
    packed, scales, biases = _c(packed, np.uint8), _c(scales, np.uint16), _c(biases, np.uint16)
    out = np.zeros((n, k), np.float32)
    _load().orc_mlx4_dequantize(_ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(out))
    return out


def mlx4_moe_id_gemv(base: np.ndarray, expert_stride: int, packed_off: int, scales_off: int,
                     biases_off: int, num_experts: int, n: int, k: int, src1: np.ndarray,
                     ids: np.ndarray, m: int, top_k: int, outer: int, inner: int) -> np.ndarray:
    """dst [m*top_k, n] of the id-GEMV over MLX 4-bit experts laid out in blocks of
    expert_stride bytes at base (offsets of the sub-tensors inside a block)."""
    base, src1, ids = _c(base, np.uint8), _c(src1, np.float32), _c(ids, np.int32)
    out = np.zeros((m * top_k, n), np.float32)
    _check(_load().orc_mlx4_moe_id_gemv(_ptr(base), expert_stride, packed_off, scales_off,
                                        biases_off, num_experts, n, k, _ptr(src1), _ptr(ids), m,
                                        top_k, outer, inner, _ptr(out)), "mlx4_moe_id_gemv")
    return out


# ------------------------------------------------------ chained RMSNorm ----

def rmsnorm_bf16(x: np.ndarray, w_bf16: np.ndarray, eps: float) -> np.ndarray:
    """x [m, H] fp32, w [H] bf16 bit patterns (uint16) -> x / rms(x) * w, fp32."""
    x = _c(np.atleast_2d(x), np.float32)
    w = _c(w_bf16, np.uint16)
    m, H = x.shape
    out = np.zeros((m, H), np.float32)
    _check(_load().orc_rmsnorm_bf16(_ptr(x), _ptr(w), float(eps), m, H, _ptr(out)), "rmsnorm_bf16")
    return out


# ------------------------------------------------------ MLX affine 2-bit ----

def mlx2_code(packed_row: np.ndarray, c: int) -> int:
    return int(_load().orc_mlx2_code(_ptr(_c(packed_row, np.uint8)), c))


def mlx2_quantize(w: np.ndarray):
    """fp32 [n, k] -> (packed uint8 [n, k/4], scales uint16 [n, k/64], biases uint16 [n, k/64])."""
    w = _c(w, np.float32)
    n, k = w.shape
    packed = np.zeros((n, k // 4), np.uint8)
    scales = np.zeros((n, k // MLX_GROUP), np.uint16)
    biases = np.zeros((n, k // MLX_GROUP), np.uint16)
    _check(_load().orc_mlx2_quantize(_ptr(w), n, k, _ptr(packed), _ptr(scales), _ptr(biases)),
           "mlx2_quantize")
    return packed, scales, biases


def mlx2_dequantize(packed, scales, biases, n: int, k: int) -> np.ndarray:
    packed, scales, biases = _c(packed, np.uint8), _c(scales, np.uint16), _c(biases, np.uint16)
    out = np.zeros((n, k), np.float32)
    _load().orc_mlx2_dequantize(_ptr(packed), _ptr(scales), _ptr(biases), n, k, _ptr(out))
    return out


def mlx2_moe_id_gemv(base, expert_stride: int, packed_off: int, scales_off: int, biases_off: int,
                     num_experts: int, n: int, k: int, src1, ids, m: int, top_k: int, outer: int,
                     inner: int) -> np.ndarray:
    base, src1, ids = _c(base, np.uint8), _c(src1, np.float32), _c(ids, np.int32)
    out = np.zeros((m * top_k, n), np.float32)
    _check(_load().orc_mlx2_moe_id_gemv(_ptr(base), expert_stride, packed_off, scales_off,
                                        biases_off, num_experts, n, k, _ptr(src1), _ptr(ids), m,
                                        top_k, outer, inner, _ptr(out)), "mlx2_moe_id_gemv")
    return out
