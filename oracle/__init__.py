"""fp64 CPU oracle of one tensor-parallel rank's Transformer-layer shard.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package's smoke check and the benchmark's
CPU-baseline leg, never by the product path.  Shares no code with the HIP library.
"""

from .tp_shard import *  # noqa: F401,F403
from .tp_shard import (shard_range, qkv_column_range, slice_qkv, slice_fc1, slice_fc2, gelu_tanh, gelu_tanh_grad,
                       slice_attn_out, attn_out_fwd, attn_out_bwd, gelu,
                       gelu_grad, attention_fwd, attention_bwd, qkv_fwd, qkv_bwd, mlp_fwd, mlp_bwd,
                       layer_fwd, tp_qkv_shard_fwd, tp_attn_heads_fwd, tp_mlp_shard_fwd,
                       tp_mlp_shard_bwd, tp_qkv_shard_bwd, tp_attn_heads_bwd,
                       tp_attn_out_shard_fwd, tp_attn_out_shard_bwd, dropout_add, layernorm,
                       layernorm_bwd, sp_rows, tp_residual_ln_fwd, tp_residual_ln_bwd,
                       tp_mlp_grouped_shard_fwd, moe_route, moe_combine, tp_moe_shard_fwd,
                       moe_combine_bwd, tp_mlp_grouped_shard_bwd, tp_moe_shard_bwd, moe_route_bwd,
                       e4m3_decode, e4m3_encode, fp8_decode, fp8_encode, fp8_quantize, fp8_gemm_nt,
                       FP8_EPI_NONE, FP8_EPI_GELU, FP8_EPI_GELU_TANH, FP8_EPI_DGELU, FP8_EPI_DGELU_TANH,
                       normwise_error, blockwise_error)
