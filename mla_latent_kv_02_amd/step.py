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

from ._binding import (BlockPool, Dims, LatentCache, mla_absorb_q, mla_append_absorb_q, mla_cache_append,
                       mla_combine, mla_combine_out_proj, mla_decode, mla_num_partials, mla_out_proj)


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


def fused_tail_ok(dims: Dims, dtype) -> bool:
    """Whether mla_combine_out_proj is compiled for these shapes (bf16 weights,
    d_c = 512, d_v = 128)."""
    import torch
    return dtype == torch.bfloat16 and dims.d_c == 512 and dims.d_v == 128


class DecodeSession:
    """Autoregressive decode over a paged latent cache that grows by n_q tokens
    per sequence per step.  Blocks come from the library's block pool as the
    sequences grow and go back when one is released (the PagedAttention scheme
    of [Paldyn] = "MQA와 GQA: KV 캐시 경량화 전략", section "PagedAttention과
    연속 배칭"); a released slot takes a new sequence with ``append``.

    Per step the host reserves blocks.  Positions and context lengths advance
    by n_q on every step, so the device copy [positions | ctx_lens] is just
    incremented in place; only after a block was added, or after ``append`` /
    ``release`` changed the host state, do the block table and that array go
    to the device, from pinned staging (two slots, each reused only after its
    previous copy is known done).  The step then runs as mla_append_absorb_q,
    mla_decode and the merge + up-projection."""

    def __init__(self, dims: Dims, B: int, n_q: int, num_splits: int, dtype, n_blocks: int, block_size: int,
                 max_blocks: int, device="cuda"):
        import numpy as np
        import torch
        self.dims, self.B, self.n_q, self.num_splits, self.dtype = dims, B, n_q, num_splits, dtype
        self.pool = BlockPool(n_blocks, block_size, B, max_blocks)
        row = dims.d_c + dims.d_rope
        self.data = torch.empty((n_blocks, block_size, row), dtype=dtype, device=device)
        self.ctx = np.zeros(B, dtype=np.int32)
        self.table_dev = torch.full((B, max_blocks), -1, dtype=torch.int32, device=device)
        self._meta_dev = torch.zeros(B * n_q + B, dtype=torch.int32, device=device)
        self.positions = self._meta_dev[: B * n_q].view(B, n_q)
        self.cache = LatentCache(data=self.data, ctx_lens=self._meta_dev[B * n_q:], block_table=self.table_dev,
                                 block_size=block_size)
        self.work = DecodeStep(dims, B, n_q, num_splits, dtype, device)
        self.seq_ids = torch.arange(B, dtype=torch.int32, device=device).repeat_interleave(n_q)
        n_stage = B * max_blocks + B * n_q + B
        self._stage = [torch.empty(n_stage, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._stage_done = [None, None]
        self._slot = 0
        self._table_dirty = True
        self._meta_stale = True     # the device [positions | ctx_lens] does not follow from the last step

    def _reserve(self, b: int, n_tokens: int) -> None:
        before = self.pool.free_count
        self.pool.reserve(b, n_tokens)
        self._table_dirty |= self.pool.free_count != before

    def _upload(self, positions, ctx, stream) -> None:
        import torch
        slot, self._slot = self._slot, self._slot ^ 1
        if self._stage_done[slot] is not None:
            self._stage_done[slot].synchronize()     # its previous copy has been read
        buf = self._stage[slot]
        host = buf.numpy()
        nt = self.pool.table.size
        nm = positions.size + ctx.size
        host[nt: nt + positions.size] = positions.reshape(-1)
        host[nt + positions.size: nt + nm] = ctx
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            if self._table_dirty:
                host[:nt] = self.pool.table.reshape(-1)
                self.table_dev.view(-1).copy_(buf[:nt], non_blocking=True)
                self._table_dirty = False
            self._meta_dev.copy_(buf[nt: nt + nm], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(s)
        self._stage_done[slot] = ev

    def append(self, seq_ids, positions, c_kv, k_rope, stream=None) -> None:
        """Write rows (e.g. a prompt's latents) into the cache: row k belongs to
        sequence seq_ids[k] (host int array) at position positions[k]; c_kv
        [n][d_c] and k_rope [n][d_rope] (raw, rotated on write) are device
        tensors.  Each sequence's context becomes max(context, position + 1)."""
        import numpy as np
        import torch
        seq_ids = np.asarray(seq_ids, dtype=np.int32)
        positions = np.asarray(positions, dtype=np.int32)
        for b in np.unique(seq_ids):
            top = int(positions[seq_ids == b].max()) + 1
            self._reserve(int(b), top)
            self.ctx[b] = max(int(self.ctx[b]), top)
        cur_pos = np.maximum(self.ctx[:, None] - self.n_q + np.arange(self.n_q, dtype=np.int32)[None, :], 0)
        self._upload(cur_pos, self.ctx, stream)
        self._meta_stale = True
        dev = self.data.device
        sid = torch.from_numpy(seq_ids).to(dev)
        pos = torch.from_numpy(positions).to(dev)
        mla_cache_append(self.dims, self.cache, sid, pos, c_kv, k_rope, stream=stream)
        if stream is None:
            torch.cuda.current_stream().synchronize()   # the index tensors above are temporaries
        else:
            stream.synchronize()

    def step(self, c_kv_new, k_rope_new, q_nope, q_rope, w_uk, w_uv, stream=None):
        """One decode step: appends the n_q new rows of every sequence (c_kv_new
        [B][n_q][d_c], k_rope_new [B][n_q][d_rope], raw) at positions ctx ..
        ctx + n_q - 1 and decodes the queries there.  Returns the output
        [B][n_q][n_h][d_v] (fp32, owned by the session, overwritten next step)."""
        import numpy as np
        d, B, n_q = self.dims, self.B, self.n_q
        before = self.pool.free_count
        self.pool.reserve_all(self.ctx + n_q)
        self._table_dirty |= self.pool.free_count != before
        pos = self.ctx[:, None] + np.arange(n_q, dtype=np.int32)[None, :]
        new_ctx = self.ctx + n_q
        if self._table_dirty or self._meta_stale:
            self._upload(pos, new_ctx, stream)
            self._meta_stale = False
        else:   # last step's positions and lengths, each + n_q
            import torch
            with torch.cuda.stream(torch.cuda.current_stream() if stream is None else stream):
                self._meta_dev.add_(n_q)
        w = self.work
        mla_append_absorb_q(d, self.cache, self.seq_ids, self.positions.view(-1),
                            c_kv_new.reshape(B * n_q, d.d_c), k_rope_new.reshape(B * n_q, d.d_rope), q_nope, q_rope,
                            self.positions, w_uk, w.q_lat, w.q_pe, stream=stream)
        mla_decode(d, w.q_lat, w.q_pe, self.cache, self.positions, self.num_splits, w.u_part, w.lse_part,
                   stream=stream)
        if fused_tail_ok(d, self.dtype):
            mla_combine_out_proj(d, self.cache.ctx_lens, self.num_splits, w.u_part, w.lse_part, w_uv, w.out,
                                 w.lse, stream=stream)
        else:
            mla_combine(d, self.cache.ctx_lens, self.num_splits, w.u_part, w.lse_part, w.u, w.lse, stream=stream)
            mla_out_proj(d, w.u, w_uv, w.out, stream=stream)
        self.ctx = new_ctx
        return w.out

    def release(self, b: int) -> None:
        """End sequence b: its blocks go back to the pool and its context to 0."""
        before = self.pool.free_count
        self.pool.release(b)
        self._table_dirty |= self.pool.free_count != before
        self.ctx[b] = 0
        self._meta_stale = True
