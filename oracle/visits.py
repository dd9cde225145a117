"""Expected set of visited (query cell, key cell) pairs.

Test infrastructure only (see the package docstring).

Block-sparse FlashAttention evaluates only the blocks whose mask entry is 1
(FlashAttention reading guide, xyznot.com, "Ekstensi: Block-Sparse
FlashAttention"); a causal or padded block with no allowed entry is equally
all -inf and is skipped too.  Cells are 128 x 128.  Cell (i, j) of batch b is
visited iff
    block_mask[i][j] == 1  and  (not causal or j <= i)  and  128*j < kv_len[b]
with the mask taken as all ones when absent and kv_len[b] = N when absent.
Pure integer Python.
"""
from __future__ import annotations

import numpy as np

CELL = 128


def expected_visits(B, N, causal=False, block_mask=None, kv_len=None, cell=CELL):
    T = -(-N // cell)
    out = np.zeros((B, T, T), dtype=np.int64)
    for b in range(B):
        L = N if kv_len is None else int(kv_len[b])
        for i in range(T):
            for j in range(T):
                if block_mask is not None and int(block_mask[i][j]) == 0:
                    continue
                if causal and j > i:
                    continue
                if cell * j >= L:
                    continue
                out[b, i, j] = 1
    return out
