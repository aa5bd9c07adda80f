"""fp64 CPU oracle for MLA decode with weight absorption.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and imports nothing from it.
"""
from .mla_oracle import (  # noqa: F401
    rope_inverse_frequencies,
    rope_rotate,
    absorb_query,
    reconstruct_keys,
    reconstruct_values,
    decode_sequence,
    merge_partials,
    value_up_projection,
    output_projection,
    fold_output,
    query_from_compressed,
    fold_query,
    e4m3_value,
    e4m3_encode,
    fp8_tile_scale,
    fp8_quantize_latent,
    fp8_dequantize_latent,
    FP8_TILE,
    FP8_MAX,
    mla_cache_elements_per_token,
    mla_cache_bytes_per_token,
    mha_cache_bytes_per_token,
    gqa_cache_bytes_per_token,
)
