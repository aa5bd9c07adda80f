"""The split-KV work plan that include/mla.h documents for mla_decode, restated
in plain Python for the tests that build or read partials slot by slot.

The tokens of all sequences lie in order on a cost line.  A sequence whose
token prefix is not a multiple of the plain token cut q0 = ceil(T / U) starts
inside a work unit and is preceded by SEGMENT_COST cost positions (the price
of a second segment in that unit); work unit w covers cost positions
[w Q, (w + 1) Q) with Q = ceil((T + SEGMENT_COST * E) / U), E the number of
such starts.  Sequence b meets units C_b // Q .. (C_b + L_b - 1) // Q and owns
that many consecutive partial slots.
"""
from __future__ import annotations

SEGMENT_COST = 288


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class Plan:
    def __init__(self, ctx, num_splits: int, segment_cost: int = SEGMENT_COST):
        lens = [int(x) for x in ctx]
        T = sum(lens)
        self.q0 = max(1, _ceil_div(T, num_splits))
        self.cost_pos, self.parts, self.slot0 = [], [], []
        p = starts = slot = 0
        for L in lens:
            if L > 0 and p % self.q0 != 0:
                starts += 1
            self.cost_pos.append(p + segment_cost * starts)
            p += L
        self.cost_total = T + segment_cost * starts
        self.Q = max(1, _ceil_div(self.cost_total, num_splits))
        for c, L in zip(self.cost_pos, lens):
            n = (c + L - 1) // self.Q - c // self.Q + 1 if L > 0 else 0
            self.parts.append(n)
            self.slot0.append(slot)
            slot += n
        self.lens = lens
        self.num_splits = num_splits

    def segments(self, w: int):
        """(b, t0, t1, slot) of work unit w, in sequence order."""
        a, e = w * self.Q, min((w + 1) * self.Q, self.cost_total)
        out = []
        for b, (c, L) in enumerate(zip(self.cost_pos, self.lens)):
            if L > 0 and c < e and c + L > a:
                out.append((b, max(a, c) - c, min(e, c + L) - c, self.slot0[b] + w - c // self.Q))
        return out

    def cuts(self, b: int):
        """Token offsets inside sequence b where a unit boundary falls."""
        c, L = self.cost_pos[b], self.lens[b]
        return [m * self.Q - c for m in range(c // self.Q + 1, (c + L - 1) // self.Q + 1)] if L > 0 else []
