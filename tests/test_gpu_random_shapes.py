"""Seeded random shapes through the GPU path against the oracle.

Decode over contiguous and paged caches (bf16 rows, and fp8 rows), and
prefill, with batch sizes, context lengths, query counts, block sizes and
split counts drawn from a fixed seeded generator (the same cases every run).
The shapes cover what the hand-picked cases of the other parity tests do not
combine: several query tokens with paged caches and many splits, odd block
sizes, contexts that end anywhere in a 32-token stage, prefill chunks whose
query block and context ends fall at arbitrary offsets.  Tolerance 1e-2 (bf16
operands, fp32 accumulation; fp8 rows are compared with the oracle's own
quantisation of the latents), the oracle on a subset of heads.
"""
import numpy as np
import pytest

import workloads as W
from tests import test_gpu_parity as par
from tests import test_gpu_prefill as pre

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HEADS = [0, 5, 77, 127]


BLOCKS = (0, 16, 40, 64, 128, 0, 96, 32, 256, 0)   # 0: contiguous; others: paged block sizes


def _decode_cases(n=len(BLOCKS)):
    rng = np.random.default_rng(0xA11CE)
    cases = []
    for k in range(n):
        batch = int(rng.integers(1, 5))
        n_q = int(rng.integers(1, 4))
        ctx = [int(rng.integers(n_q, 700)) for _ in range(batch)]
        block = BLOCKS[k]
        splits = int(rng.integers(1, 10))
        fp8 = bool(rng.random() < 0.3)
        cases.append(pytest.param(k, batch, n_q, ctx, block, splits, fp8,
                                  id=f"d{k}-B{batch}-q{n_q}-blk{block}-s{splits}{'-fp8' if fp8 else ''}"))
    return cases


# paged caches whose block size is a multiple of the 32-token stage, with many
# splits: most segments then start at tokens that are not multiples of 32
# (their first stage starts below the cut and masks the tokens before it)
MANY_SPLIT_BLOCKS = (32, 64, 96, 128, 64, 96)


def _many_split_cases():
    rng = np.random.default_rng(0x5EC7)
    cases = []
    for k, block in enumerate(MANY_SPLIT_BLOCKS):
        batch = int(rng.integers(2, 7))
        n_q = int(rng.integers(1, 4))
        ctx = [int(rng.integers(n_q, 900)) for _ in range(batch)]
        splits = int(rng.integers(10, 61))
        fp8 = k % 3 == 2
        cases.append(pytest.param(100 + k, batch, n_q, ctx, block, splits, fp8,
                                  id=f"m{k}-B{batch}-q{n_q}-blk{block}-s{splits}{'-fp8' if fp8 else ''}"))
    return cases


def _prefill_cases(n=5):
    rng = np.random.default_rng(0xBEE5)
    cases = []
    for k in range(n):
        batch = int(rng.integers(1, 4))
        n_q = int(rng.integers(1, 300))
        ctx = [int(rng.integers(n_q, 520)) for _ in range(batch)]
        cases.append(pytest.param(k, n_q, ctx, id=f"p{k}-B{batch}-q{n_q}"))
    return cases


@pytest.mark.parametrize("k,batch,n_q,ctx,block,splits,fp8", _decode_cases() + _many_split_cases())
def test_random_decode_shape(k, batch, n_q, ctx, block, splits, fp8):
    par._need_gpu()
    from workloads.device import stage
    w = W.custom(name=f"rand_dec{k}", seed=500 + k, batch=batch, n_q=n_q, ctx=None, ctx_range=(1, 1),
                 block_size=block)
    if fp8:
        w = W.with_fp8_cache(w)
    st = stage(w, ctx=np.array(ctx, np.int32))
    got = par._run(st, splits)
    par._check(w, st, got, heads=HEADS)


@pytest.mark.parametrize("k,n_q,ctx", _prefill_cases())
def test_random_prefill_shape(k, n_q, ctx):
    pre._need_gpu()
    from workloads.device import stage
    w = W.custom(name=f"rand_pf{k}", seed=600 + k, batch=len(ctx), n_q=n_q, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array(ctx, np.int32))
    pre._check(w, st, pre._prefill(st), heads=HEADS)
