"""Plain fp64 CPU oracle for paged decode attention (test infrastructure).

This module is test infrastructure: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark may import it.  The GPU library never
calls it, and it shares no code with the GPU library.

What it computes, and where the pages fix it (pages: "Paged Attention and
Memory Efficiency in Production LLM Serving" on burnlayer.com = P1,
"PagedAttention in Production" on oh-bug.com = P2, "PagedAttention — The KV
Cache Problem" on infra.bea.ai = P3):

* A sequence's KV cache lives in fixed-size physical blocks; a per-sequence
  block table maps logical block j to a physical block (P1 "How PagedAttention
  borrows OS paging"; P2 "Core Principle", block-table figure; P3 "How It
  Works").  Position t of a sequence is row ``t mod bs`` of physical block
  ``table[t // bs]``.
* Attention over the gathered keys and values is ordinary attention: dot
  products, softmax, weighted sum of values, unchanged by the paging (P1 "How
  PagedAttention borrows OS paging": the math is that of a naive
  implementation).  The oracle therefore gathers each sequence into contiguous
  arrays and evaluates softmax attention directly in float64.
* New tokens' K/V rows are appended as decoding proceeds (P1 "Why KV cache
  memory was the bottleneck": the cache grows with every token); a sequence
  that diverges from a shared prefix gets its own copy of the shared block
  (P1 copy-on-write; P3 "Why This Matters": copy-on-write for parallel
  sampling).
* Per-token KV size is layers x kv_heads x head_dim x 2 (K and V) x bytes
  (P1 "Why KV cache memory was the bottleneck", 327,680 bytes for 80 x 8 x 128
  in FP16; P2 "Common Misconceptions", capacity formula).
* FP8 KV cache (P3 "What's Still Unsolved"): OCP E4M3FN codes, one fp32 scale
  per tensor; value = decode(code) x scale.
* FP4 KV cache (the same passage names FP4): OCP E2M1 codes (the element type
  of the OCP Microscaling formats: sign, 2 exponent bits, 1 mantissa bit,
  largest magnitude 6), two per byte, with one fp32 scale per (slot, kv head)
  row.

Readings where the pages are silent (each stated where it is used): block
layout [num_blocks, kv_heads, block_size, head_dim]; slot = block x bs +
offset, negative slot = skip; query head i reads KV head i // group;
context_lens include the just-appended token and nothing else is masked;
an empty context gives an all-zero output; FP8 encode = fp32 division by the
scale, round to nearest even, saturate to +-448, NaN kept as NaN.

Storage conventions: f16 = numpy.float16; bf16 = numpy.uint16 bit pattern;
fp8 = numpy.uint8 E4M3FN code; fp4 = numpy.uint8 holding two E2M1 codes,
element 2i in the low nibble and element 2i + 1 in the high one (a row of D
elements is D / 2 bytes).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ---------------------------------------------------------------------------
# sizing (P1 "Why KV cache memory was the bottleneck"; P2 capacity formula)
# ---------------------------------------------------------------------------

def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """Bytes of K plus V one token occupies across all layers."""
    return layers * kv_heads * head_dim * 2 * bytes_per_elem


def kv_cache_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem)


def tail_waste(context_lens, bs: int) -> float:
    """Fraction of allocated token slots left unused: only the tail of each
    sequence's last block is unused (P1 "How PagedAttention borrows OS paging")."""
    lens = np.asarray(context_lens, np.int64)
    alloc = ((lens + bs - 1) // bs) * bs
    total = int(alloc.sum())
    return float((alloc - lens).sum()) / total if total else 0.0


# ---------------------------------------------------------------------------
# block table addressing (P2 "Core Principle", block-table figure)
# ---------------------------------------------------------------------------

def slot_of(table_row, pos: int, bs: int) -> int:
    """Physical slot of logical position ``pos``: the block the table maps
    logical block pos // bs to, at row pos mod bs."""
    return int(table_row[pos // bs]) * bs + pos % bs


def slots_for(table_row, start: int, end: int, bs: int) -> np.ndarray:
    pos = np.arange(start, end, dtype=np.int64)
    return np.asarray(table_row, np.int64)[pos // bs] * bs + pos % bs


# ---------------------------------------------------------------------------
# FP8 E4M3FN codec (OCP 8-bit floating point spec; P3 "What's Still Unsolved")
# ---------------------------------------------------------------------------

def e4m3_values() -> np.ndarray:
    """Value of each of the 256 codes: sign, 4 exponent bits (bias 7), 3
    mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities."""
    out = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * 2.0 ** -6 * (m / 8.0)
        else:
            out[c] = s * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return out


_E4M3 = e4m3_values()
_POS_CODES = np.arange(0x7F)  # 0x00..0x7E: the non-negative finite codes, in increasing value order
_POS_VALS = _E4M3[:0x7F]


def e4m3_encode(x, scale: float) -> np.ndarray:
    """Quantise to E4M3FN codes: y = fp32(x) / fp32(scale) (correctly rounded
    fp32 division), then the nearest representable value with ties to the
    even code, magnitudes beyond 448 saturating to 448, NaN to the NaN code of
    the same sign."""
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = np.asarray(x, np.float32) / np.float32(scale)
    neg = np.signbit(y)
    a = np.abs(y).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALS, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_hi = _POS_VALS[hi] - a
    d_lo = a - _POS_VALS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def e4m3_decode(codes, scale: float = 1.0) -> np.ndarray:
    """fp64 value of each code times fp64(scale): both exact."""
    return _E4M3[np.asarray(codes, np.uint8)] * float(np.float32(scale))


# ---------------------------------------------------------------------------
# FP4 E2M1 codec (the element type of the OCP Microscaling formats spec;
# "PagedAttention - The KV Cache Problem", "What's Still Unsolved", names FP4
# KV caches)
# ---------------------------------------------------------------------------

def e2m1_values() -> np.ndarray:
    """Value of each of the 16 codes: sign (bit 3), 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (0 and 0.5); no infinities, no NaN."""
    out = np.empty(16, np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        out[c] = s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0))
    return out


_E2M1 = e2m1_values()
_E2M1_POS = _E2M1[:8]  # codes 0..7: the non-negative values, in increasing order


def e2m1_encode(x, scale) -> np.ndarray:
    """Quantise to E2M1 codes (one per uint8): y = fp32(x) / fp32(scale)
    (correctly rounded fp32 division), then the nearest of the eight
    magnitudes with ties to the even code (mantissa bit 0), magnitudes beyond
    6 saturating to 6, the sign kept (-0 stays -0).  E2M1 has no NaN: a NaN
    element is stored as +0 (reading: the row's scale ignores it, and zero
    keeps it out of the attention sums)."""
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = np.asarray(x, np.float32) / np.asarray(scale, np.float32)
    nan = np.isnan(y)
    neg = np.signbit(y) & ~nan
    a = np.where(nan, 0.0, np.minimum(np.abs(y).astype(np.float64), E2M1_MAX))
    hi = np.clip(np.searchsorted(_E2M1_POS, a, side="left"), 0, 7)  # first magnitude >= a
    lo = np.clip(hi - 1, 0, None)
    d_hi = _E2M1_POS[hi] - a
    d_lo = a - _E2M1_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return (code | np.where(neg, np.uint8(0x8), np.uint8(0))).astype(np.uint8)


def e2m1_pack(codes) -> np.ndarray:
    """Codes [..., D] (D even) -> bytes [..., D / 2]: element 2i in the low
    nibble, element 2i + 1 in the high nibble."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def e2m1_unpack(packed) -> np.ndarray:
    """Bytes [..., D / 2] -> codes [..., D]."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# widening of storage dtypes to fp64 (exact)
# ---------------------------------------------------------------------------

def widen(x, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Storage values -> float64, exactly.  f16 is IEEE binary16; bf16 is the
    upper half of an IEEE binary32 (1 sign, 8 exponent, 7 fraction bits), so
    its bit pattern shifted left by 16 is that binary32; fp8 goes through the
    E4M3FN code table times the scale."""
    if dtype == "f16":
        return np.asarray(x, np.float16).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_decode(x, scale)
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp64 values to a storage dtype with round-to-nearest-even (bf16
    through fp32, the path a fp32 kernel result takes)."""
    x = np.asarray(x, np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        f = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        bias = ((f >> 16) & 1) + 0x7FFF
        r = ((f + bias) >> 16).astype(np.uint16)
        return np.where(np.isnan(x), np.uint16(0x7FC0), r)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return {"f16": np.float16, "bf16": np.uint16, "fp8": np.uint8, "f32": np.float32}[dtype]


# ---------------------------------------------------------------------------
# the pool: [num_blocks, kv_heads, block_size, head_dim]
# ---------------------------------------------------------------------------

POISON = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}


def new_pool(num_blocks: int, kv_heads: int, bs: int, head_dim: int, dtype: str, poison: bool = True):
    """A pool whose every slot holds NaN until written, so that any read of
    an unwritten slot shows up in the output."""
    shape = (num_blocks, kv_heads, bs, head_dim)
    if dtype == "fp8":
        return np.full(shape, POISON["fp8"] if poison else 0, np.uint8)
    if dtype == "fp4":  # no NaN code: the row scales of an unwritten slot are NaN instead
        return np.full(shape[:-1] + (head_dim // 2,), 0x77 if poison else 0, np.uint8)
    bits = np.full(shape, POISON[dtype] if poison else 0, np.uint16)
    return bits.view(np.float16) if dtype == "f16" else bits


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, bs: int, cache_dtype: str,
                      k_scale: float = 1.0, v_scale: float = 1.0, src_dtype: Optional[str] = None):
    """Write token n's K/V rows [kv_heads, head_dim] into slot_mapping[n]
    (block slot // bs, row slot mod bs); a negative slot writes nothing.
    Same-dtype rows are copied bit for bit; an FP8 cache stores
    e4m3_encode(row, scale)."""
    slots = np.asarray(slot_mapping, np.int64)
    keep = slots >= 0
    b = slots[keep] // bs
    o = slots[keep] % bs
    k = np.asarray(key)[keep]
    v = np.asarray(value)[keep]
    if cache_dtype == "fp8":
        k = e4m3_encode(widen(k, src_dtype).astype(np.float32), k_scale)
        v = e4m3_encode(widen(v, src_dtype).astype(np.float32), v_scale)
    k_cache[b, :, o, :] = k
    v_cache[b, :, o, :] = v


# ---------------------------------------------------------------------------
# FP8 with one scale per (slot, kv head) row ("PagedAttention - The KV Cache
# Problem", section "What's Still Unsolved" names FP8/FP4 KV caches; the
# granularity is a reading: a row's scale is fixed when the row is written,
# which suits a cache that grows one token at a time)
# ---------------------------------------------------------------------------

def row_scale(rows32: np.ndarray, qmax: float = E4M3_MAX) -> np.ndarray:
    """Scale of each row (last axis = the row's elements, fp32): its largest
    magnitude, NaN elements left out, divided by qmax (448 for E4M3FN, 6 for
    E2M1) in fp32, so that element lands on the largest finite code; 1 for a
    row of zeros or one holding an infinity."""
    x = np.abs(np.asarray(rows32, np.float32))
    x = np.where(np.isnan(x), np.float32(0), x)
    amax = x.max(axis=-1)
    ok = (amax > 0) & np.isfinite(amax)
    return np.where(ok, amax / np.float32(qmax), np.float32(1)).astype(np.float32)


def reshape_and_cache_scaled(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping, bs: int,
                             src_dtype: str, cache_dtype: str = "fp8"):
    """Token n's rows into slot_mapping[n] of an FP8 (E4M3FN) or FP4 (E2M1,
    two codes per byte) cache, each (token, head) row encoded against its own
    scale -- largest magnitude / 448, or / 6 -- which goes to the scale pools
    [num_blocks, kv_heads, bs] (fp32); a negative slot writes nothing."""
    slots = np.asarray(slot_mapping, np.int64)
    keep = slots >= 0
    b = slots[keep] // bs
    o = slots[keep] % bs
    for src, cache, scales in ((key, k_cache, k_scales), (value, v_cache, v_scales)):
        x = widen(np.asarray(src)[keep], src_dtype).astype(np.float32)  # [n, kv_heads, D]
        if cache_dtype == "fp4":
            s = row_scale(x, E2M1_MAX)  # [n, kv_heads]
            cache[b, :, o, :] = e2m1_pack(e2m1_encode(x, s[..., None]))
        else:
            s = row_scale(x)
            cache[b, :, o, :] = e4m3_encode(x, s[..., None])
        scales[b, :, o] = s


def widen_rows(codes, scales, cache_dtype: str = "fp8") -> np.ndarray:
    """fp64 values of a cache's rows [..., D] (FP8 codes, or FP4 bytes
    [..., D / 2]) times their rows' scales [...]: exact."""
    s = np.asarray(scales, np.float32).astype(np.float64)[..., None]
    if cache_dtype == "fp4":
        return _E2M1[e2m1_unpack(codes)] * s
    return _E4M3[np.asarray(codes, np.uint8)] * s


def decode_scaled(q, k_cache, v_cache, k_scales, v_scales, block_tables, context_lens, scale: float,
                  group: int, q_dtype: str, seqs=None, cache_dtype: str = "fp8") -> np.ndarray:
    """fp64 decode over an FP8 or FP4 cache with a scale per row [B, Hq, D]."""
    q = np.asarray(q)
    out = []
    for s in (range(q.shape[0]) if seqs is None else seqs):
        L = int(context_lens[s])
        k = widen_rows(gather_kv(k_cache, block_tables[s], L), gather_kv(k_scales[..., None], block_tables[s], L)[..., 0],
                       cache_dtype)
        v = widen_rows(gather_kv(v_cache, block_tables[s], L), gather_kv(v_scales[..., None], block_tables[s], L)[..., 0],
                       cache_dtype)
        out.append(attend(widen(q[s], q_dtype), k, v, scale, group))
    return np.stack(out) if out else np.zeros((0,) + q.shape[1:])


def copy_blocks(k_cache, v_cache, pairs):
    """Copy-on-write duplication: block dst becomes a byte copy of block src,
    for K and V (P1 copy-on-write)."""
    for src, dst in np.asarray(pairs, np.int64).reshape(-1, 2):
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def gather_kv(cache, table_row, L: int) -> np.ndarray:
    """Contiguous rows [L, kv_heads, head_dim] of one sequence: position t is
    row t mod bs of block table_row[t // bs] (P3 "How It Works": the kernel
    reads the block table to gather from non-contiguous blocks)."""
    bs = cache.shape[2]
    pos = np.arange(L)
    blk = np.asarray(table_row, np.int64)[pos // bs]
    return cache[blk, :, pos % bs, :]


# ---------------------------------------------------------------------------
# decode attention (P1 "How PagedAttention borrows OS paging": dot products,
# softmax, weighted sum over values, as in a naive implementation)
# ---------------------------------------------------------------------------

def attend(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, scale: float, group: int) -> np.ndarray:
    """One sequence: q [Hq, D], k/v [L, Hkv, D] (fp64) -> [Hq, D].
    Query head i attends over KV head i // group."""
    Hq, D = q64.shape
    L, Hkv, _ = k64.shape
    if L == 0:
        return np.zeros((Hq, D))
    qg = q64.reshape(Hkv, group, D)
    kh = k64.transpose(1, 2, 0)  # [Hkv, D, L]
    scores = float(scale) * (qg @ kh)  # [Hkv, g, L]
    scores -= scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w /= w.sum(axis=-1, keepdims=True)
    return (w @ v64.transpose(1, 0, 2)).reshape(Hq, D)  # [Hkv, g, L] @ [Hkv, L, D]


def decode_one(q, k_cache, v_cache, table_row, L: int, scale: float, group: int, cache_dtype: str,
               q_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    k = widen(gather_kv(k_cache, table_row, L), cache_dtype, k_scale)
    v = widen(gather_kv(v_cache, table_row, L), cache_dtype, v_scale)
    return attend(widen(q, q_dtype), k, v, scale, group)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, group: int,
           cache_dtype: str, q_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
           seqs=None) -> np.ndarray:
    """fp64 decode output [B, Hq, D] (or only the rows of ``seqs``)."""
    q = np.asarray(q)
    seqs = range(q.shape[0]) if seqs is None else seqs
    out = []
    for s in seqs:
        out.append(decode_one(q[s], k_cache, v_cache, block_tables[s], int(context_lens[s]), scale,
                              group, cache_dtype, q_dtype, k_scale, v_scale))
    return np.stack(out) if out else np.zeros((0,) + q.shape[1:])


def window_positions(L: int, sink_tokens: int, window_tokens: int) -> np.ndarray:
    """Positions a query at the end of a sequence of L positions attends to
    under attention sinks plus a sliding window ("Paged Attention and Memory
    Efficiency in Production LLM Serving", section "Eviction, compression,
    and the challenge of fitting more KV cache into less memory": the first
    few tokens stay as attention sinks next to a window of the most recent
    ones): t < sink_tokens or t >= L - window_tokens, in order."""
    t = np.arange(L)
    return t[(t < sink_tokens) | (t >= L - window_tokens)]


def decode_window(q, k_cache, v_cache, block_tables, context_lens, scale: float, group: int, sink_tokens: int,
                  window_tokens: int, cache_dtype: str, q_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                  seqs=None) -> np.ndarray:
    """Decode attention over each sequence's sink and window positions only
    (window_positions), gathered through the block table like decode():
    fp64 [B, Hq, D] (or the rows of ``seqs``)."""
    q = np.asarray(q)
    seqs = range(q.shape[0]) if seqs is None else seqs
    out = []
    for s in seqs:
        L = int(context_lens[s])
        keep = window_positions(L, sink_tokens, window_tokens)
        k = widen(gather_kv(k_cache, block_tables[s], L), cache_dtype, k_scale)[keep]
        v = widen(gather_kv(v_cache, block_tables[s], L), cache_dtype, v_scale)[keep]
        out.append(attend(widen(q[s], q_dtype), k, v, scale, group))
    return np.stack(out) if out else np.zeros((0,) + q.shape[1:])


def decode_multi(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float, group: int,
                 cache_dtype: str, q_dtype: str, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None) -> np.ndarray:
    """Several query tokens per sequence, each seeing what a decode step at its
    own position would see ("Paged Attention and Memory Efficiency in
    Production LLM Serving", section "How vLLM turned PagedAttention into a
    production serving engine": speculative decoding and prefill run over the
    same paged cache).  Sequence s owns q rows query_start[s] .. query_start[s+1]-1,
    its last n positions; query j of them attends over positions
    0 .. L - n + j, i.e. the sequence cut just after its own position.
    Returns fp64 [T, Hq, D] (rows of sequences not in ``seqs`` stay zero)."""
    q = np.asarray(q)
    qs = np.asarray(query_start, np.int64)
    out = np.zeros(q.shape, np.float64)
    for s in (range(len(context_lens)) if seqs is None else seqs):
        L = int(context_lens[s])
        a, b = int(qs[s]), int(qs[s + 1])
        n = b - a
        if n == 0:
            continue
        k = widen(gather_kv(k_cache, block_tables[s], L), cache_dtype, k_scale)
        v = widen(gather_kv(v_cache, block_tables[s], L), cache_dtype, v_scale)
        for j in range(n):
            seen = L - n + j + 1  # positions 0 .. L - n + j
            out[a + j] = attend(widen(q[a + j], q_dtype), k[:seen], v[:seen], scale, group)
    return out


def decode_contiguous(q, keys, values, scale: float, group: int, cache_dtype: str, q_dtype: str,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """The same attention over per-sequence contiguous arrays (no paging):
    keys[s], values[s] are [L_s, kv_heads, head_dim] storage arrays."""
    return np.stack([
        attend(widen(q[s], q_dtype), widen(keys[s], cache_dtype, k_scale),
               widen(values[s], cache_dtype, v_scale), scale, group)
        for s in range(len(keys))
    ])
