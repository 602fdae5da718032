"""Oracle for the combine step around the routed kernel.

TEST INFRASTRUCTURE ONLY.  After the routed kernel, each token's k expert
outputs are summed back into one row (the benchmark write-up
"MetaX-TileLang工具链", section 2.7 item 7: the scatter_reduce that follows
the routed kernel).  The pages do not fix the precision of that sum; the
reading used here: the k fp16 rows are widened to fp32, added in slot order
j = 0..k-1 starting from +0, and the sum is rounded once to fp16 (IEEE,
nearest-even).
"""
from __future__ import annotations

import numpy as np


def combine(out_padded, padded_row_of_pair, num_tokens: int, top_k: int) -> np.ndarray:
    out = np.asarray(out_padded)
    H = out.shape[1]
    prow = np.asarray(padded_row_of_pair, dtype=np.int64).reshape(num_tokens, top_k) \
        if num_tokens * top_k else np.zeros((num_tokens, top_k), np.int64)
    acc = np.zeros((num_tokens, H), np.float32)
    for j in range(top_k):                      # slot order; fp32 adds
        acc = acc + out[prow[:, j]].astype(np.float32)
    return acc.astype(np.float16)
