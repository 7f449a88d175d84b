"""Q4_K (and MLX affine 4-bit) MoE expert path for AMD MI355X (gfx950).

The compute lives in ``libq4kmoe.so`` (HIP kernels behind the C ABI in
``include/q4kmoe.h``); ``_lib`` is its ctypes binding with the same names.
Importing the package does not load the library; the first call does, and
raises if it has not been built.
"""
from . import _lib
from ._lib import (  # noqa: F401
    MLX4_GROUP, MOE_LAYER_NOALLOC_MAX_BYTES, MOE_SHARED_NONE, MOE_SHARED_SIGMOID,
    MOE_SHARED_UNSCALED, Q4K_AUTO_BUCKET_MIN_TOKENS, Q4K_BUCKET_AUTO, Q4K_BUCKET_MODE_MASK,
    Q4K_BUCKET_OFF, Q4K_BUCKET_ON, Q4K_BUCKET_PREBUILT, Q4K_SCHED_BUCKET_LAUNCH, Q4K_SCHED_VECTOR,
    Q4KError, mlx2_dequantize, mlx2_matrix_bytes, mlx2_moe_id_gemv, mlx2_quantize,
    mlx4_dequantize, mlx4_matrix_bytes, mlx4_moe_gate_up_silu, mlx4_moe_id_gemv, mlx4_quantize,
    moe_bucket, moe_bucket_workspace_bytes, moe_combine_residual, moe_combine_residual_rmsnorm,
    moe_expert_ffn, moe_layer_forward, moe_layer_forward_noalloc, moe_layer_forward_rmsnorm,
    moe_layer_workspace_bytes, q4k_abi_version, q4k_ceiling_read, q4k_dequantize,
    q4k_matrix_bytes, q4k_moe_gate_up_silu, q4k_moe_id_gemv, q4k_pack_tiles, q4k_quantize,
    q4k_tiles_bytes, q4k_unpack_tiles, q4tp_matvec, q4tp_matvec_multi, q4tp_quantize,
    q4tp_tensor_bytes, status_string,
)
