"""Choice of the split-KV work-unit count for a batch."""
from __future__ import annotations

import math

MI355X_CUS = 256

# Cost model of one mla_decode + merge on MI355X (V3 shapes, bf16 cache),
# measured on the kernels of this library:
#   - a work unit (one workgroup per 128 query rows) pays a fixed start-up
#     (query rows and the first stages in flight before any compute),
#   - then one 32-token stage after another,
#   - and each partial it leaves (128 rows x (d_c + 2) fp32) is written once
#     and read once by the merge, at HBM rate.
UNIT_STARTUP_US = 6.0
STAGE_US = 1.9
PARTIAL_US = 2 * 128 * 514 * 4 / 6.0e12 * 1e6     # 2 x 263 KB at 6 TB/s


def default_num_splits(total_tokens: int, n_q: int, n_h: int, num_cus: int = MI355X_CUS) -> int:
    """The work-unit count U <= num_cus / (row groups) that minimises
    start-up + ceil(tokens per unit / 32) stages + U x (row groups) partials."""
    groups = max(1, math.ceil(n_q * n_h / 128))
    by_cus = max(1, num_cus // groups)
    best_u, best_t = 1, float("inf")
    for u in range(1, by_cus + 1):
        stages = math.ceil(math.ceil(total_tokens / u) / 32)
        t = UNIT_STARTUP_US + stages * STAGE_US + u * groups * PARTIAL_US
        if t < best_t - 1e-9:
            best_u, best_t = u, t
    return best_u
