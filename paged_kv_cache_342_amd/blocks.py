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


class BlockManager:
    """The library's host block manager (pa_bm_* in pa.h): a pool of num_blocks
    physical blocks of block_size tokens, block tables grown on demand,
    forking with shared blocks, copy-on-write pairs for pa_copy_blocks."""

    def __init__(self, num_blocks: int, block_size: int):
        import ctypes

        from . import _check, library

        self._ct = ctypes
        self._check = _check
        lib = library()
        self._lib = lib
        self._h = lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError(lib.pa_last_error_message().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq: int):
        self._check(self._lib.pa_bm_add(self._h, int(seq)))

    def fork(self, parent: int, child: int):
        self._check(self._lib.pa_bm_fork(self._h, int(parent), int(child)))

    def append(self, seq: int, n: int):
        """Slots (int64 array) for n new tokens of seq, and the copy pairs (list of (src, dst))."""
        ct = self._ct
        slots = np.zeros(max(int(n), 1), np.int64)
        pair = np.zeros(2, np.int64)
        copied = ct.c_int32(0)
        self._check(self._lib.pa_bm_append(self._h, int(seq), int(n), slots.ctypes.data, pair.ctypes.data,
                                           ct.byref(copied)))
        return slots[:int(n)], ([(int(pair[0]), int(pair[1]))] if copied.value else [])

    def append_batch(self, seqs, n_tokens):
        """Append n_tokens[i] tokens to seqs[i] (all or nothing).  Returns (slots int64
        array, copy pairs int64 array [P, 2])."""
        ct = self._ct
        seqs = np.ascontiguousarray(seqs, np.int64)
        n_tokens = np.ascontiguousarray(n_tokens, np.int32)
        slots = np.zeros(max(int(n_tokens.sum()), 1), np.int64)
        pairs = np.zeros((max(len(seqs), 1), 2), np.int64)
        n_pairs = ct.c_int32(0)
        self._check(self._lib.pa_bm_append_batch(self._h, seqs.ctypes.data, len(seqs), n_tokens.ctypes.data,
                                                 slots.ctypes.data, pairs.ctypes.data, ct.byref(n_pairs)))
        return slots[:int(n_tokens.sum())], pairs[:n_pairs.value]

    def free(self, seq: int):
        self._check(self._lib.pa_bm_free(self._h, int(seq)))

    def evict(self, seq: int, sink_tokens: int, window_tokens: int) -> int:
        """Keep the blocks of the first sink_tokens and the last window_tokens positions of seq,
        release the whole blocks in between and close the gap; returns the positions dropped."""
        dropped = self._ct.c_int64(0)
        self._check(self._lib.pa_bm_evict(self._h, int(seq), int(sink_tokens), int(window_tokens),
                                          self._ct.byref(dropped)))
        return int(dropped.value)

    def table(self, seq: int) -> np.ndarray:
        n = self._lib.pa_bm_table(self._h, int(seq), None, 0)
        if n < 0:
            raise KeyError(seq)
        out = np.zeros(max(n, 1), np.int32)
        self._lib.pa_bm_table(self._h, int(seq), out.ctypes.data, n)
        return out[:n]

    def tables(self, seqs, width: int, out=None, lens_out=None, pad: bool = True):
        """Block tables [len(seqs), width] int32 padded with -1, and lengths [len(seqs)] int32.
        out / lens_out: C-contiguous int32 arrays of those shapes to write into (a caller that
        builds tables every step reuses them instead of faulting in new pages each time).
        pad=False leaves the entries past each sequence's blocks as they were in `out`."""
        seqs = np.ascontiguousarray(seqs, np.int64)
        n = len(seqs)
        if not pad and out is None:
            raise ValueError("pad=False writes only block ids: pass the table matrix to update as out")
        tables = np.empty((max(n, 1), width), np.int32) if out is None else out
        lens = np.empty(max(n, 1), np.int32) if lens_out is None else lens_out
        for arr, shape, name in ((out, (n, width), "out"), (lens_out, (n,), "lens_out")):
            if arr is not None and (arr.dtype != np.int32 or not arr.flags.c_contiguous or arr.shape != shape):
                raise ValueError(f"{name} must be a C-contiguous int32 array of shape {shape}")
        self._check(self._lib.pa_bm_tables(self._h, seqs.ctypes.data, n, tables.ctypes.data, int(width),
                                           lens.ctypes.data, 1 if pad else 0))
        return tables[:n], lens[:n]

    def length(self, seq: int) -> int:
        n = self._lib.pa_bm_length(self._h, int(seq))
        if n < 0:
            raise KeyError(seq)
        return int(n)

    def stats(self) -> dict:
        st = (self._ct.c_int64 * 6)()
        self._check(self._lib.pa_bm_get_stats(self._h, st))
        d = dict(zip(("blocks_in_use", "blocks_free", "shared_blocks", "slots_held", "tokens", "sequences"),
                     (int(x) for x in st)))
        d["tail_waste"] = (d["slots_held"] - d["tokens"]) / d["slots_held"] if d["slots_held"] else 0.0
        return d
