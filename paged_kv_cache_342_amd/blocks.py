"""Host-side slot assignment for the scatter: the block manager's side of the
block-table convention (position t of a sequence lives in row t mod bs of
physical block table[t // bs]; "PagedAttention in Production", section
"Core Principle", block-table figure)."""
from __future__ import annotations

import numpy as np


def slot_mapping(block_tables: np.ndarray, seqs, start, end, block_size: int) -> np.ndarray:
    """Slots (int64) of positions [start[i], end[i]) of sequence seqs[i], concatenated in order."""
    tables = np.asarray(block_tables)
    out = []
    for s, a, b in zip(np.asarray(seqs).tolist(), np.asarray(start).tolist(), np.asarray(end).tolist()):
        if b <= a:
            continue
        pos = np.arange(a, b, dtype=np.int64)
        blk = tables[s, pos // block_size].astype(np.int64)
        if (blk < 0).any():
            raise ValueError(f"sequence {s}: positions [{a}, {b}) reach an unmapped table entry")
        out.append(blk * block_size + pos % block_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)
