"""ctypes binding of libq4kmoe.so (include/q4kmoe.h), same names as the C ABI.

Argument marshalling only: tensors are passed as device pointers
(``tensor.data_ptr()``), the stream defaults to torch's current stream, and a
nonzero status raises ``Q4KError``.  Every computation runs in the HIP
kernels; there is no host fallback, and a missing library raises at load time.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4kmoe.so")

Q4K_OK, Q4K_ERR_SHAPE, Q4K_ERR_NULL, Q4K_ERR_STRIDE, Q4K_ERR_WORKSPACE, Q4K_ERR_LAUNCH, \
    Q4K_ERR_ARG, Q4K_ERR_SCRATCH = range(8)
MOE_LAYER_NOALLOC_MAX_BYTES = 16 << 20
Q4K_BUCKET_AUTO, Q4K_BUCKET_OFF, Q4K_BUCKET_ON, Q4K_BUCKET_PREBUILT = 0, 1, 2, 3
Q4K_BUCKET_MODE_MASK, Q4K_SCHED_VECTOR, Q4K_SCHED_BUCKET_LAUNCH = 0xFF, 0x100, 0x200
Q4K_AUTO_BUCKET_MIN_TOKENS = 5
MOE_SHARED_NONE, MOE_SHARED_SIGMOID, MOE_SHARED_UNSCALED = 0, 1, 2
Q4K_BLOCK_WEIGHTS, Q4K_BLOCK_BYTES, Q4K_MAX_TOP_K = 256, 144, 16
Q4K_MAX_IN, Q4K_MAX_EXPERTS, Q4K_MAX_PAIRS, Q4TP_MAX_COLS = 16384, 1023, 8192, 16384
Q4TP_MAX_TENSORS = 3
MLX4_GROUP = 64

# name -> (restype, argtypes); mirrors include/q4kmoe.h
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "q4k_status_string": (ctypes.c_char_p, [_I]),
    "q4k_abi_version": (_I, []),
    "q4k_matrix_bytes": (_I64, [_I64, _I64]),
    "q4k_dequantize": (_I, [_P, _P, _I64, _P]),
    "q4k_quantize": (_I, [_P, _P, _I64, _I64, _P]),
    "q4k_tiles_bytes": (_I64, [_I64, _I64]),
    "q4k_pack_tiles": (_I, [_P, _P, _I64, _I64, _I64, _P]),
    "q4k_unpack_tiles": (_I, [_P, _P, _I64, _I64, _I64, _P]),
    "moe_bucket_workspace_bytes": (_I64, [_I64, _I64]),
    "moe_bucket": (_I, [_P, _I64, _I64, _P, _I64, _P]),
    "q4k_moe_id_gemv": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I, _P,
                             _I64, _P]),
    "q4k_moe_gate_up_silu": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                  _P, _P, _P, _I, _P, _I64, _P]),
    "moe_expert_ffn": (_I, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P,
                            _I64, _P]),
    "moe_layer_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64]),
    "moe_layer_forward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                               _I64, _I64, _I, _I, _P, _I64, _P]),
    "moe_layer_forward_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                       _I64, _I64, _I64, _I64, _I, _I, _P]),
    "moe_combine_residual": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P]),
    "moe_layer_forward_rmsnorm": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_float, _P, _I64, _I64, _I64, _I64, _I64, _I,
                                       _I, _P, _I64, _P]),
    "moe_combine_residual_rmsnorm": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _I64,
                                          _I64, _I64, _I, _P]),
    "q4tp_tensor_bytes": (_I64, [_I64, _I64]),
    "q4tp_matvec": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "q4tp_matvec_multi": (_I, [_P, _P, _I, _P, _P, _I64, _P]),
    "q4tp_quantize": (_I, [_P, _P, _I64, _I64, _P]),
    "mlx4_matrix_bytes": (_I64, [_I64, _I64]),
    "mlx4_dequantize": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "mlx4_quantize": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "mlx4_moe_id_gemv": (_I, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _I64,
                              _I64, _I64, _I64, _P]),
    "mlx4_moe_gate_up_silu": (_I, [_P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P,
                                   _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P]),
    "mlx2_matrix_bytes": (_I64, [_I64, _I64]),
    "mlx2_dequantize": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "mlx2_quantize": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "mlx2_moe_id_gemv": (_I, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _I64, _I64,
                              _I64, _I64, _I64, _P]),
    # include/q4kceil.h (measurement)
    "q4k_ceiling_read": (_I, [_P, _P, _I64, _I64, _P, _P]),
}


class Q4KError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return ctypes.c_void_p(x)
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("device tensor expected")
        if not x.is_contiguous():
            raise ValueError("contiguous tensor expected")
        return ctypes.c_void_p(x.data_ptr())
    raise TypeError(f"cannot pass {type(x)} as a device pointer")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != Q4K_OK:
        raise Q4KError(name, rc)


def status_string(status: int) -> str:
    return load().q4k_status_string(status).decode()


def q4k_abi_version() -> int:
    return load().q4k_abi_version()


def q4k_matrix_bytes(n: int, k: int) -> int:
    return load().q4k_matrix_bytes(n, k)


def q4tp_tensor_bytes(rows: int, cols: int) -> int:
    return load().q4tp_tensor_bytes(rows, cols)


def q4k_tiles_bytes(n: int, k: int) -> int:
    return load().q4k_tiles_bytes(n, k)


def q4k_pack_tiles(blocks, tiles, n_mats: int, n: int, k: int, stream=None):
    _call("q4k_pack_tiles", _ptr(blocks), _ptr(tiles), n_mats, n, k, _stream(stream))


def q4k_unpack_tiles(tiles, blocks, n_mats: int, n: int, k: int, stream=None):
    _call("q4k_unpack_tiles", _ptr(tiles), _ptr(blocks), n_mats, n, k, _stream(stream))


def moe_bucket_workspace_bytes(n_pairs: int, num_experts: int) -> int:
    return load().moe_bucket_workspace_bytes(n_pairs, num_experts)


def q4k_dequantize(blocks, out, n_blocks: int, stream=None):
    _call("q4k_dequantize", _ptr(blocks), _ptr(out), n_blocks, _stream(stream))


def q4k_quantize(w, blocks, n_rows: int, k: int, stream=None):
    _call("q4k_quantize", _ptr(w), _ptr(blocks), n_rows, k, _stream(stream))


def moe_bucket(ids, n_pairs: int, num_experts: int, ws, ws_bytes: int, stream=None):
    _call("moe_bucket", _ptr(ids), n_pairs, num_experts, _ptr(ws), ws_bytes, _stream(stream))


def q4k_moe_id_gemv(w_stacked, src1, ids, dst, n: int, k: int, m: int, top_k: int,
                    src1_outer_stride: int, src1_inner_stride: int, num_experts: int,
                    bucket_flag: int = Q4K_BUCKET_AUTO, ws=None, ws_bytes: int = 0, stream=None):
    _call("q4k_moe_id_gemv", _ptr(w_stacked), _ptr(src1), _ptr(ids), _ptr(dst), n, k, m, top_k,
          src1_outer_stride, src1_inner_stride, num_experts, bucket_flag, _ptr(ws), ws_bytes,
          _stream(stream))


def q4k_moe_gate_up_silu(w_gate, w_up, src1, ids, out, n: int, k: int, m: int, top_k: int,
                         src1_outer_stride: int, src1_inner_stride: int, num_experts: int,
                         sh_gate=None, sh_up=None, sh_out=None,
                         bucket_flag: int = Q4K_BUCKET_AUTO, ws=None, ws_bytes: int = 0,
                         stream=None):
    _call("q4k_moe_gate_up_silu", _ptr(w_gate), _ptr(w_up), _ptr(src1), _ptr(ids), _ptr(out), n,
          k, m, top_k, src1_outer_stride, src1_inner_stride, num_experts, _ptr(sh_gate),
          _ptr(sh_up), _ptr(sh_out), bucket_flag, _ptr(ws), ws_bytes, _stream(stream))


def moe_expert_ffn(w_gate, w_up, w_down, h_post, ids, act, expert_out, hidden: int, inter: int,
                   num_experts: int, m: int, top_k: int, bucket_flag: int = Q4K_BUCKET_AUTO,
                   ws=None, ws_bytes: int = 0, stream=None):
    _call("moe_expert_ffn", _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(h_post), _ptr(ids),
          _ptr(act), _ptr(expert_out), hidden, inter, num_experts, m, top_k, bucket_flag,
          _ptr(ws), ws_bytes, _stream(stream))


def moe_layer_workspace_bytes(hidden: int, inter: int, num_experts: int, m: int,
                              top_k: int) -> int:
    return load().moe_layer_workspace_bytes(hidden, inter, num_experts, m, top_k)


def moe_layer_forward(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids, route_w,
                      shared_gate_logit, out, hidden: int, inter: int, num_experts: int, m: int,
                      top_k: int, shared_mode: int, bucket_flag: int = Q4K_BUCKET_AUTO, ws=None,
                      ws_bytes: int = 0, stream=None):
    _call("moe_layer_forward", _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate),
          _ptr(sh_up), _ptr(sh_down), _ptr(h_post), _ptr(h_mid), _ptr(ids), _ptr(route_w),
          _ptr(shared_gate_logit), _ptr(out), hidden, inter, num_experts, m, top_k, shared_mode,
          bucket_flag, _ptr(ws), ws_bytes, _stream(stream))


def moe_layer_forward_noalloc(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids,
                              route_w, shared_gate_logit, out, hidden: int, inter: int,
                              num_experts: int, m: int, top_k: int, shared_mode: int,
                              bucket_flag: int = Q4K_BUCKET_AUTO, stream=None):
    _call("moe_layer_forward_noalloc", _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate),
          _ptr(sh_up), _ptr(sh_down), _ptr(h_post), _ptr(h_mid), _ptr(ids), _ptr(route_w),
          _ptr(shared_gate_logit), _ptr(out), hidden, inter, num_experts, m, top_k, shared_mode,
          bucket_flag, _stream(stream))


def moe_combine_residual(h_mid, expert_out, route_w, shared_out, shared_gate_logit, out,
                         hidden: int, m: int, top_k: int, shared_mode: int, stream=None):
    _call("moe_combine_residual", _ptr(h_mid), _ptr(expert_out), _ptr(route_w), _ptr(shared_out),
          _ptr(shared_gate_logit), _ptr(out), hidden, m, top_k, shared_mode, _stream(stream))


def q4tp_matvec(tensor, x, y, rows: int, cols: int, stream=None):
    _call("q4tp_matvec", _ptr(tensor), _ptr(x), _ptr(y), rows, cols, _stream(stream))


def q4tp_matvec_multi(tensors, rows, x, y, cols: int, stream=None):
    """Merged matvec of up to three tensors of the same width against x; y
    holds their outputs one after another.  `tensors` and `rows` are lists."""
    n = len(tensors)
    if len(rows) != n:
        raise ValueError("tensors and rows differ in length")
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in tensors])
    rws = (ctypes.c_int64 * max(n, 1))(*[int(r) for r in rows])
    _call("q4tp_matvec_multi", ctypes.cast(ptrs, ctypes.c_void_p),
          ctypes.cast(rws, ctypes.c_void_p), n, _ptr(x), _ptr(y), cols, _stream(stream))


def q4tp_quantize(w, tensor, rows: int, cols: int, stream=None):
    _call("q4tp_quantize", _ptr(w), _ptr(tensor), rows, cols, _stream(stream))


def mlx4_matrix_bytes(n: int, k: int) -> int:
    return load().mlx4_matrix_bytes(n, k)


def mlx4_dequantize(packed, scales, biases, out, n: int, k: int, stream=None):
    _call("mlx4_dequantize", _ptr(packed), _ptr(scales), _ptr(biases), _ptr(out), n, k,
          _stream(stream))


def mlx4_quantize(w, packed, scales, biases, n: int, k: int, stream=None):
    _call("mlx4_quantize", _ptr(w), _ptr(packed), _ptr(scales), _ptr(biases), n, k,
          _stream(stream))


def mlx4_moe_id_gemv(expert_base, expert_stride: int, packed_off: int, scales_off: int,
                     biases_off: int, src1, ids, dst, n: int, k: int, m: int, top_k: int,
                     src1_outer_stride: int, src1_inner_stride: int, num_experts: int,
                     stream=None):
    _call("mlx4_moe_id_gemv", _ptr(expert_base), expert_stride, packed_off, scales_off,
          biases_off, _ptr(src1), _ptr(ids), _ptr(dst), n, k, m, top_k, src1_outer_stride,
          src1_inner_stride, num_experts, _stream(stream))


def mlx4_moe_gate_up_silu(expert_base, expert_stride: int, gate_offs, up_offs, src1, ids, dst,
                          n: int, k: int, m: int, top_k: int, src1_outer_stride: int,
                          src1_inner_stride: int, num_experts: int, stream=None):
    """gate_offs and up_offs are (packed, scales, biases) byte offsets inside an expert block."""
    _call("mlx4_moe_gate_up_silu", _ptr(expert_base), expert_stride, *[int(o) for o in gate_offs],
          *[int(o) for o in up_offs], _ptr(src1), _ptr(ids), _ptr(dst), n, k, m, top_k,
          src1_outer_stride, src1_inner_stride, num_experts, _stream(stream))


def moe_layer_forward_rmsnorm(w_gate, w_up, w_down, sh_gate, sh_up, sh_down, h_post, h_mid, ids,
                              route_w, shared_gate_logit, out, norm_weight, eps: float, normed,
                              hidden: int, inter: int, num_experts: int, m: int, top_k: int,
                              shared_mode: int, bucket_flag: int = Q4K_BUCKET_AUTO, ws=None,
                              ws_bytes: int = 0, stream=None):
    _call("moe_layer_forward_rmsnorm", _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(sh_gate),
          _ptr(sh_up), _ptr(sh_down), _ptr(h_post), _ptr(h_mid), _ptr(ids), _ptr(route_w),
          _ptr(shared_gate_logit), _ptr(out), _ptr(norm_weight), float(eps), _ptr(normed),
          hidden, inter, num_experts, m, top_k, shared_mode, bucket_flag, _ptr(ws), ws_bytes,
          _stream(stream))


def moe_combine_residual_rmsnorm(h_mid, expert_out, route_w, shared_out, shared_gate_logit,
                                 norm_weight, eps: float, out, normed, hidden: int, m: int,
                                 top_k: int, shared_mode: int, stream=None):
    _call("moe_combine_residual_rmsnorm", _ptr(h_mid), _ptr(expert_out), _ptr(route_w),
          _ptr(shared_out), _ptr(shared_gate_logit), _ptr(norm_weight), float(eps), _ptr(out),
          _ptr(normed), hidden, m, top_k, shared_mode, _stream(stream))


def mlx2_matrix_bytes(n: int, k: int) -> int:
    return load().mlx2_matrix_bytes(n, k)


def mlx2_dequantize(packed, scales, biases, out, n: int, k: int, stream=None):
    _call("mlx2_dequantize", _ptr(packed), _ptr(scales), _ptr(biases), _ptr(out), n, k,
          _stream(stream))


def mlx2_quantize(w, packed, scales, biases, n: int, k: int, stream=None):
    _call("mlx2_quantize", _ptr(w), _ptr(packed), _ptr(scales), _ptr(biases), n, k,
          _stream(stream))


def mlx2_moe_id_gemv(expert_base, expert_stride: int, packed_off: int, scales_off: int,
                     biases_off: int, src1, ids, dst, n: int, k: int, m: int, top_k: int,
                     src1_outer_stride: int, src1_inner_stride: int, num_experts: int,
                     stream=None):
    _call("mlx2_moe_id_gemv", _ptr(expert_base), expert_stride, packed_off, scales_off,
          biases_off, _ptr(src1), _ptr(ids), _ptr(dst), n, k, m, top_k, src1_outer_stride,
          src1_inner_stride, num_experts, _stream(stream))


def q4k_ceiling_read(base, offsets, n_ranges: int, range_bytes: int, sink, stream=None):
    """Measurement only (include/q4kceil.h): read n_ranges ranges of
    range_bytes bytes at base + offsets[i] (offsets: a device int64 tensor)."""
    rc = load().q4k_ceiling_read(_ptr(base), _ptr(offsets), n_ranges, range_bytes, _ptr(sink),
                                 _stream(stream))
    if rc != 0:
        raise RuntimeError(f"q4k_ceiling_read: status {rc}")
