"""The host-side contract check (mla_latent_kv_02_amd.contract) on CPU tensors.

Each breach the library cannot see on the host (context lengths past the
cache, a missing or foreign block id inside a sequence's range, decode
positions that are not the last n_q tokens, append targets outside the cache
or written twice) must be named; everything inside the contract, including
the degenerate cases the kernels accept (empty contexts, -1 ids past a
sequence's range, shared blocks read by two sequences), must pass.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_02_amd import LatentCache
from mla_latent_kv_02_amd import _binding as bd
from mla_latent_kv_02_amd import contract as C


def _paged(ctx, bs=16, max_blocks=4, n_blocks=12, row=8):
    ctx = np.asarray(ctx, np.int32)
    table = np.full((len(ctx), max_blocks), -1, np.int32)
    nxt = 0
    for b, c in enumerate(ctx):
        for k in range(min(-(-int(c) // bs), max_blocks)):
            table[b, k] = nxt
            nxt += 1
    assert nxt <= n_blocks
    return LatentCache(data=torch.zeros((n_blocks, bs, row)), ctx_lens=torch.from_numpy(ctx),
                       block_table=torch.from_numpy(table), block_size=bs)


def _pos(ctx, n_q):
    ctx = np.asarray(ctx, np.int64)
    return torch.from_numpy((ctx[:, None] - n_q + np.arange(n_q)[None, :]).astype(np.int32))


def test_inside_the_contract_passes():
    cache = _paged([17, 0, 64, 1])               # ragged, an empty and a one-token context, a full row
    assert C.decode_errors(cache, _pos([17, 0, 64, 1], 1)) == []
    assert C.decode_errors(cache, _pos([17, 0, 64, 1], 2)) == []       # negative positions see nothing
    # two sequences reading one shared block is allowed
    cache.block_table[3, 0] = cache.block_table[0, 0]
    assert C.decode_errors(cache) == []
    contiguous = LatentCache(data=torch.zeros((3, 40, 8)), ctx_lens=torch.tensor([40, 0, 7], dtype=torch.int32))
    assert C.decode_errors(contiguous, _pos([40, 0, 7], 1)) == []


def test_context_lengths_outside_the_cache_are_named():
    cache = _paged([17, 65, 3])                  # 65 > max_blocks * bs = 64
    errs = C.decode_errors(cache)
    assert errs == ["ctx_lens[1] = 65 outside [0, 64]"]
    cache = _paged([17, 3])
    cache.ctx_lens[0] = -1
    assert C.decode_errors(cache) == ["ctx_lens[0] = -1 outside [0, 64]"]
    contiguous = LatentCache(data=torch.zeros((2, 40, 8)), ctx_lens=torch.tensor([41, 0], dtype=torch.int32))
    assert C.decode_errors(contiguous) == ["ctx_lens[0] = 41 outside [0, 40]"]


def test_block_ids_inside_a_range_must_exist():
    cache = _paged([40, 20])
    cache.block_table[0, 3] = -1                 # past sequence 0's 3 blocks: fine
    assert C.decode_errors(cache) == []
    cache.block_table[0, 2] = -1                 # its third block (tokens 32..47) missing
    errs = C.decode_errors(cache)
    assert len(errs) == 1 and errs[0].startswith("sequence 0: block 2 (tokens 32..47) has id -1")
    cache = _paged([40, 20])
    cache.block_table[1, 1] = 12                 # n_blocks = 12: one past the pool
    assert "sequence 1: block 1" in C.decode_errors(cache)[0]
    assert "outside [0, 12)" in C.decode_errors(cache)[0]


def test_decode_positions_must_be_the_last_tokens():
    ctx = [17, 5]
    cache = _paged(ctx)
    pos = _pos(ctx, 2)
    pos[1, 0] = 4                                 # should be 3
    assert C.decode_errors(cache, pos) == ["positions[1][0] = 4, the decode step puts it at 3"]
    with pytest.raises(C.ContractError, match=r"^mla_decode: positions\[1\]\[0\]"):
        C.check_decode(cache, pos)
    assert "must be [B][n_q]" in C.decode_errors(cache, pos[:1])[0]


def test_append_targets():
    cache = _paged([20, 10])                      # sequence 0: blocks 0, 1; sequence 1: block 2
    ok = C.cache_append_errors(cache, torch.tensor([0, 0, 1]), torch.tensor([20, 31, 10]))
    assert ok == []
    assert C.cache_append_errors(cache, torch.tensor([2]), torch.tensor([0])) == ["seq_ids[0] = 2 outside [0, 2)"]
    assert C.cache_append_errors(cache, torch.tensor([0]), torch.tensor([64])) == \
        ["positions[0] = 64 outside [0, 64)"]
    assert C.cache_append_errors(cache, torch.tensor([1]), torch.tensor([-1])) == \
        ["positions[0] = -1 outside [0, 64)"]
    errs = C.cache_append_errors(cache, torch.tensor([0, 1]), torch.tensor([5, 16]))
    assert errs == ["new token 1 (sequence 1, position 16) goes to block id -1, outside [0, 12)"]
    # the same row twice: once by one sequence, once through a block two sequences share
    assert "written to the same cache row" in C.cache_append_errors(cache, torch.tensor([0, 0]),
                                                                       torch.tensor([7, 7]))[0]
    cache.block_table[1, 1] = 0
    errs = C.cache_append_errors(cache, torch.tensor([0, 1]), torch.tensor([3, 19]))
    assert errs == ["new tokens 0 and 1 are written to the same cache row"]
    contiguous = LatentCache(data=torch.zeros((2, 40, 8)), ctx_lens=torch.tensor([3, 3], dtype=torch.int32))
    assert C.cache_append_errors(contiguous, torch.tensor([0, 1]), torch.tensor([39, 39])) == []
    assert C.cache_append_errors(contiguous, torch.tensor([1]), torch.tensor([40])) == \
        ["positions[0] = 40 outside [0, 40)"]


def test_binding_hook_is_opt_in(monkeypatch):
    cache = _paged([17, 65])
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "0")
    bd._contract("check_decode", cache, None, fn="mla_decode")
    monkeypatch.delenv("MLA_CHECK_CONTRACT")
    bd._contract("check_decode", cache, None, fn="mla_decode")
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "1")
    with pytest.raises(C.ContractError, match=r"mla_decode: ctx_lens\[1\] = 65"):
        bd._contract("check_decode", cache, None, fn="mla_decode")
    with pytest.raises(C.ContractError, match=r"mla_combine: ctx_lens\[0\] = -3"):
        bd._contract("check_ctx_lens", torch.tensor([-3, 4]), fn="mla_combine")
