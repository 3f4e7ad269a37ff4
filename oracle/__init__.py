"""fp64 CPU oracle for one tensor-parallel rank's share of a Megatron-style
Transformer layer (MLP block and causal self-attention block, forward and
backward), of the residual add + LayerNorm that follows each block, and of the
vocabulary-parallel logits + cross-entropy of the output layer; attention
dropout masks from a counter-based generator.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package. The product path (the HIP library and
its Python binding) never imports or calls it, and this package imports
nothing from the product path.

Every function is the plain definition written out in float64 with NumPy:
matrix products use `@`, everything else is elementwise code; attention
materialises the full score matrix of each head. Inputs are the exact values
the GPU receives (bf16-rounded where the storage type is bf16), widened to
float64; nothing is rounded inside.

Pinned against: torch float64 library routines (tanh-GeLU, scaled dot-product
attention, log-sum-exp, autograd) on the unsharded layer, central finite
differences, closed forms and the parameter counts the pages print. No
function here is "parity unpinned".
"""
from .tp_layer import (  # noqa: F401
    GELU_C, gelu, gelu_grad, column_shard, row_shard, qkv_weight_shard, qkv_bias_shard,
    layer_weight_shapes, mlp_fwd, mlp_bwd, alibi_slope, attn_core_fwd, attn_core_bwd, attn_fwd,
    attn_bwd, sum_partials,
)
from .ln_residual import ln_residual_fwd, ln_residual_bwd, ln_residual_bwd_dropout  # noqa: F401
from .vocab_ce import vocab_shard, logits_fwd, ce_partial_stats, ce_combine, ce_bwd  # noqa: F401
from .dropout import philox4x64_10, keep_threshold, keep_scale, attention_multipliers, residual_multipliers  # noqa: F401
