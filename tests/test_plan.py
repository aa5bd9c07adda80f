"""The split-KV work plan (tests/plan_ref.py, the plan include/mla.h states
for mla_decode): every token in exactly one work unit, partial slots distinct
and within mla_num_partials, the plain token split when sequences start on
unit boundaries, and the same segment cost as the kernels' plan walk."""
import os
import re

import numpy as np
import pytest

from tests.plan_ref import SEGMENT_COST, Plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("seed", range(40))
def test_plan_covers_every_token_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 60))
    U = int(rng.integers(1, 300))
    ctx = rng.integers(0, 5000, size=B) * (rng.random(B) < 0.8)
    plan = Plan(ctx, U)
    seen = [np.zeros(int(n), np.int64) for n in ctx]
    slots = []
    for w in range(U):
        last_b = -1
        for b, t0, t1, slot in plan.segments(w):
            assert b > last_b and 0 <= t0 < t1 <= ctx[b]
            last_b = b
            seen[b][t0:t1] += 1
            slots.append(slot)
    assert all((s == 1).all() for s in seen)
    assert sorted(slots) == list(range(len(slots)))            # consecutive from 0, no gap
    assert len(slots) == sum(plan.parts) <= U + B - 1          # mla_num_partials
    for b in range(B):                                          # a sequence's slots in token order
        own = [(t0, slot) for w in range(U) for bb, t0, _, slot in plan.segments(w) if bb == b]
        assert [s for _, s in sorted(own)] == list(range(plan.slot0[b], plan.slot0[b] + plan.parts[b]))


def test_aligned_starts_give_the_token_split():
    # 64 sequences of 8192 tokens in 256 units: every sequence starts on a
    # multiple of q0 = 2048, so the units are the quarters of the sequences
    plan = Plan(np.full(64, 8192), 256)
    assert plan.q0 == plan.Q == 2048 and plan.cost_total == 64 * 8192
    assert all(plan.segments(w) == [(w // 4, 2048 * (w % 4), 2048 * (w % 4 + 1), w)] for w in range(256))


def test_inside_starts_move_the_cuts():
    # 3 sequences of 1000 tokens, 3 units: q0 = 1000 and every start is on a
    # cut, so nothing moves; with 4 units (q0 = 750) sequences 1 and 2 start
    # inside a unit and each adds SEGMENT_COST in front of its tokens
    plan = Plan([1000, 1000, 1000], 3)
    assert [plan.segments(w) for w in range(3)] == [[(0, 0, 1000, 0)], [(1, 0, 1000, 1)], [(2, 0, 1000, 2)]]
    plan = Plan([1000, 1000, 1000], 4)
    assert plan.cost_pos == [0, 1000 + SEGMENT_COST, 2000 + 2 * SEGMENT_COST]
    assert plan.Q == -(-(3000 + 2 * SEGMENT_COST) // 4)
    q = plan.Q
    assert plan.segments(0) == [(0, 0, q, 0)]
    assert plan.segments(1)[0] == (0, q, 1000, 1)


def test_kernel_plan_uses_the_same_segment_cost():
    src = open(os.path.join(ROOT, "mla_latent_kv_02_amd", "csrc", "mla_device.h")).read()
    assert int(re.search(r"kSegmentCost = (\d+);", src).group(1)) == SEGMENT_COST
    hdr = open(os.path.join(ROOT, "include", "mla.h")).read()
    assert f"preceded by {SEGMENT_COST} cost" in hdr and f"Q = ceil((T + {SEGMENT_COST} E) / U)" in hdr
