"""MLA decode with weight absorption for MI355X (gfx950).

The computation lives in libmla.so (C ABI in include/mla.h, HIP kernels in
csrc/); this package is its thin Python binding.  Importing it does not load
the library; the first call does, and fails loudly if it is not built.
"""
from ._binding import (  # noqa: F401
    BF16,
    BlockPool,
    EXPORTED,
    F32,
    FP8_E4M3,
    LIB_PATH,
    Dims,
    LatentCache,
    MlaError,
    load_library,
    mla_absorb_q,
    mla_cache_append,
    mla_append_absorb_q,
    mla_combine,
    mla_decode,
    mla_num_partials,
    mla_out_proj,
    mla_combine_out_proj,
    mla_decode_out_noalloc,
    mla_fold_out,
    mla_out_proj_folded,
    mla_o_proj,
    mla_fold_q,
    mla_absorb_q_folded,
    mla_cache_row_bytes,
    mla_prefill_weights,
    mla_prefill_workspace_bytes,
    mla_prefill,
)

__version__ = "0.1.0"
