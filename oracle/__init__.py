"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import (attn_proj_shard, col_linear, col_shard, col_shard_uneven, combine_sum,
                        concat, f64, input_slice, layer_sharded, layer_unsharded, linear,
                        linear_entry, linear_fsum, mlp, mlp_shard, mlp_shards, qkv_rows,
                        qkv_segments, qkv_unreplicate, qkv_shard, rel_err, row_partial, row_shard, silu, swiglu,
                        gelu, ffn_gelu, ffn_gelu_shard, ffn_gelu_shards, kv_heads_of, blocks_of,
                        row_shard_uneven, input_slices_uneven, kv_group_of, attention_core_shard,
                        attention_decode_shard)
