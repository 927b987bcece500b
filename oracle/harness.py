"""Replays a workload's pool-building steps with the oracle's own scatter and
copy, then evaluates the oracle decode (test infrastructure only).

The workload supplies token values, block tables and the order of appends and
copy-on-write copies; every address and byte written here comes from the
oracle's own functions.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from . import pa_oracle as O


def build_pools(w, seqs: Optional[Iterable[int]] = None, poison: bool = True):
    """Oracle K/V pools after all of the workload's write steps.

    With ``seqs`` given, only the writes that land in blocks those sequences'
    tables reference are replayed (enough to evaluate their outputs)."""
    kc = O.new_pool(w.num_blocks, w.Hkv, w.bs, w.D, w.cache_dtype, poison)
    vc = O.new_pool(w.num_blocks, w.Hkv, w.bs, w.D, w.cache_dtype, poison)
    needed = None
    if seqs is not None:
        needed = set()
        for s in seqs:
            n = (int(w.context_lens[s]) + w.bs - 1) // w.bs
            needed.update(int(b) for b in w.block_tables[s, :n])
    kv_cache = {}

    def kv(s):
        if s not in kv_cache:
            kv_cache[s] = w.seq_kv(s)
        return kv_cache[s]

    for op in w.ops:
        if op.kind == "copy":
            pairs = op.pairs if needed is None else np.array(
                [p for p in op.pairs if int(p[1]) in needed], np.int64).reshape(-1, 2)
            O.copy_blocks(kc, vc, pairs)
            continue
        for s, a, b in zip(op.seqs, op.start, op.end):
            s, a, b = int(s), int(a), int(b)
            if b <= a:
                continue
            row = w.block_tables[s]
            if needed is not None:
                blocks = {int(x) for x in row[a // w.bs:(b - 1) // w.bs + 1]}
                if not blocks & needed:
                    continue
            k, v = kv(s)
            O.reshape_and_cache(k[a:b], v[a:b], kc, vc, O.slots_for(row, a, b, w.bs), w.bs,
                                w.cache_dtype, w.k_scale, w.v_scale, src_dtype=w.src_dtype)
    return kc, vc


def decode(w, kc, vc, seqs=None, q=None):
    q = w.query() if q is None else q
    return O.decode(q, kc, vc, w.block_tables, w.context_lens, w.scale, w.group, w.cache_dtype,
                    w.q_dtype, w.k_scale, w.v_scale, seqs=seqs)


def decode_multi(w, kc, vc, seqs=None):
    """Oracle output [T, Hq, D] of a workload with several queries per sequence."""
    return O.decode_multi(w.query(), kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale, w.group,
                          w.cache_dtype, w.q_dtype, w.k_scale, w.v_scale, seqs=seqs)
