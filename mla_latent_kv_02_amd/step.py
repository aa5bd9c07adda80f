"""One MLA decode step as the sequence of library calls:

    [cache_append of the new tokens] -> absorb_q -> decode -> combine -> out_proj

The append and the absorption go through mla_append_absorb_q (one launch where
the library fuses them); with ``fused_tail`` the last two are the single
mla_combine_out_proj call (the merged u is then not stored).  ``DecodeStep`` owns the intermediate
buffers (q_lat, q_pe, the split-KV partials, u, lse) and the output, sized once
for a batch shape, so that a step allocates nothing.  Every call goes through
the C ABI.
"""
from __future__ import annotations

from ._binding import (Dims, LatentCache, mla_absorb_q, mla_append_absorb_q, mla_combine, mla_combine_out_proj,
                       mla_decode, mla_num_partials, mla_out_proj)


class DecodeStep:
    def __init__(self, dims: Dims, B: int, n_q: int, num_splits: int, dtype, device="cuda"):
        import torch
        self.dims, self.B, self.n_q, self.num_splits = dims, B, n_q, num_splits
        slots = mla_num_partials(B, num_splits)
        f32 = torch.float32
        self.q_lat = torch.empty((B, n_q, dims.n_h, dims.d_c), dtype=dtype, device=device)
        self.q_pe = torch.empty((B, n_q, dims.n_h, dims.d_rope), dtype=dtype, device=device)
        self.u_part = torch.empty((slots, n_q, dims.n_h, dims.d_c), dtype=f32, device=device)
        self.lse_part = torch.empty((slots, n_q, dims.n_h, 2), dtype=f32, device=device)
        self.u = torch.empty((B, n_q, dims.n_h, dims.d_c), dtype=f32, device=device)
        self.lse = torch.empty((B, n_q, dims.n_h), dtype=f32, device=device)
        self.out = torch.empty((B, n_q, dims.n_h, dims.d_v), dtype=f32, device=device)

    def run(self, q_nope, q_rope, positions, w_uk, w_uv, cache: LatentCache, new_tokens=None, stream=None,
            fused_tail: bool = False):
        """``new_tokens`` = (seq_ids, positions, c_kv_new, k_rope_new) appends the
        step's own latents to the cache first."""
        d = self.dims
        if new_tokens is not None:
            mla_append_absorb_q(d, cache, *new_tokens, q_nope, q_rope, positions, w_uk, self.q_lat, self.q_pe,
                                stream=stream)
        else:
            mla_absorb_q(d, q_nope, q_rope, positions, w_uk, self.q_lat, self.q_pe, stream=stream)
        mla_decode(d, self.q_lat, self.q_pe, cache, positions, self.num_splits, self.u_part,
                   self.lse_part, stream=stream)
        if fused_tail:
            mla_combine_out_proj(d, cache.ctx_lens, self.num_splits, self.u_part, self.lse_part, w_uv, self.out,
                                 self.lse, stream=stream)
        else:
            mla_combine(d, cache.ctx_lens, self.num_splits, self.u_part, self.lse_part, self.u, self.lse,
                        stream=stream)
            mla_out_proj(d, self.u, w_uv, self.out, stream=stream)
        return self.out

    def capture(self, q_nope, q_rope, positions, w_uk, w_uv, cache: LatentCache, new_tokens=None,
                fused_tail: bool = False):
        """Record one step into a HIP graph (torch.cuda.CUDAGraph) and return it;
        ``graph.replay()`` then launches the same kernels on the same buffers
        without the per-call host work.  The library's kernels enqueue no
        memset or allocation, so the step is capturable as it stands."""
        import torch
        self.run(q_nope, q_rope, positions, w_uk, w_uv, cache, new_tokens, fused_tail=fused_tail)   # warm-up
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(q_nope, q_rope, positions, w_uk, w_uv, cache, new_tokens, fused_tail=fused_tail)
        torch.cuda.synchronize()
        return graph
