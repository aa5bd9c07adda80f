"""Choice of the split-KV work-unit count for a batch."""
from __future__ import annotations

import math

MI355X_CUS = 256


def default_num_splits(total_tokens: int, n_q: int, n_h: int, num_cus: int = MI355X_CUS,
                       min_tokens: int = 1024) -> int:
    """One work unit per CU for each group of 128 query rows, but no unit
    smaller than ``min_tokens`` tokens (a partial costs n_h*n_q*(d_c+1)*4
    bytes written and read again, worth ~200 cache rows at 128 heads)."""
    groups = max(1, math.ceil(n_q * n_h / 128))
    by_cus = max(1, num_cus // groups)
    by_len = max(1, math.ceil(total_tokens / min_tokens))
    return int(min(by_cus, by_len))
