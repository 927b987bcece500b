"""Seeded synthetic inputs for paged decode attention.

This module only *draws* inputs: context lengths, block tables built from a
seeded permutation of the physical pool, and N(0,1) key/value/query values cast
to their storage dtype.  It holds none of the attention, slot, gather or
quantisation arithmetic, so both the HIP path and the CPU oracle can take their
inputs from here without sharing any of the computation they are compared on.

Shapes follow the decode workloads on the PagedAttention pages: fixed-size
physical blocks (16 tokens in the pages' own example, "How It Works" on the
infra.bea.ai page), per-sequence block tables (the block-table figure in "Core
Principle" on the oh-bug.com page), shared prefixes with copy-on-write
("How PagedAttention borrows OS paging" on the burnlayer.com page) and an FP8
KV variant ("What's Still Unsolved" on the infra.bea.ai page).

Randomness: one ``numpy.random.PCG64`` stream per purpose, keyed by
``SeedSequence([seed, purpose, index])``, so any single sequence can be
regenerated on its own (the oracle samples a few sequences of a full-size batch
without generating the rest).

Storage dtypes: ``f16`` arrays are ``numpy.float16``; ``bf16`` arrays are
``numpy.uint16`` bit patterns (RNE cast from fp32 by torch on the CPU).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Tuple

import numpy as np

# purposes of the per-stream keys
_LENS, _KEY, _VAL, _Q, _TAIL_K, _TAIL_V, _DELTA = 0, 1, 2, 3, 4, 5, 6

DTYPES = ("f16", "bf16", "fp8")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 values to a 16-bit storage dtype with round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        import torch

        return torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    raise ValueError(f"not a 16-bit storage dtype: {dtype}")


def storage_to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 16-bit storage back to fp32 (exact)."""
    if dtype == "f16":
        return x.astype(np.float32)
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


@dataclass
class WriteOp:
    """One step of building the physical pool.

    kind == "append": write positions [start[i], end[i]) of sequence seqs[i]
    through that sequence's final block table.
    kind == "copy": duplicate whole blocks, pairs[n] = (src, dst).
    """

    kind: str
    seqs: Optional[np.ndarray] = None
    start: Optional[np.ndarray] = None
    end: Optional[np.ndarray] = None
    pairs: Optional[np.ndarray] = None


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    cache_dtype: str  # f16 | bf16 | fp8 | fp4 (fp4: two E2M1 codes per byte, row-scaled only)
    src_dtype: str  # dtype of the key/value rows handed to the scatter (f16 | bf16)
    q_dtype: str  # f16 | bf16
    scale: float
    context_lens: np.ndarray  # int32 [B], final lengths (the decode token included)
    block_tables: np.ndarray  # int32 [B, M], padded with -1
    num_blocks: int
    ops: List[WriteOp]  # how the pool is filled; the last op appends the decode token
    k_scale: float = 1.0
    v_scale: float = 1.0
    _kv: Callable[[int], Tuple[np.ndarray, np.ndarray]] = field(repr=False, default=None)
    _q: Callable[[], np.ndarray] = field(repr=False, default=None)
    meta: dict = field(default_factory=dict)
    # several queries per sequence: sequence s owns query rows
    # query_start[s] .. query_start[s+1]-1, its last positions (None = one each)
    query_start: Optional[np.ndarray] = None

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    def seq_kv(self, s: int) -> Tuple[np.ndarray, np.ndarray]:
        """Key and value rows of sequence s, positions 0..L_s-1, [L_s, Hkv, D] storage dtype."""
        return self._kv(s)

    def query(self) -> np.ndarray:
        """Queries in q_dtype storage: [B, Hq, D], or [T, Hq, D] with several per sequence."""
        return self._q()

    @property
    def max_queries(self) -> int:
        return int(np.diff(self.query_start).max()) if self.query_start is not None and self.B else 1

    def kv_bytes(self) -> int:
        """Bytes of K and V the decode batch attends over (each row once per KV head)."""
        bits = {"fp8": 8, "fp4": 4}.get(self.cache_dtype, 16)
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * bits // 8


def _deal_tables(rng, lens, bs, num_blocks):
    nblk = (lens + bs - 1) // bs
    M = max(1, int(nblk.max()))
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(lens), M), -1, np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[off:off + n]
        off += n
    assert off <= num_blocks
    return tables


def _plain_kv(seed, lens, Hkv, D, dtype):
    def kv(s):
        L = int(lens[s])
        k = _rng(seed, _KEY, s).standard_normal((L, Hkv, D), dtype=np.float32)
        v = _rng(seed, _VAL, s).standard_normal((L, Hkv, D), dtype=np.float32)
        return to_storage(k, dtype), to_storage(v, dtype)

    return kv


def _plain_q(seed, B, Hq, D, dtype):
    return lambda: to_storage(_rng(seed, _Q).standard_normal((B, Hq, D), dtype=np.float32), dtype)


def _prefill_ops(lens):
    B = len(lens)
    seqs = np.arange(B, dtype=np.int64)
    zero = np.zeros(B, np.int64)
    last = lens.astype(np.int64) - 1
    ops = [WriteOp("append", seqs, zero, np.maximum(last, 0))]
    live = lens > 0
    ops.append(WriteOp("append", seqs[live], last[live], last[live] + 1))
    return ops


def _uniform_batch(name, seed, B, Hq, Hkv, D, bs, dtype, lens, num_blocks, rng, scale=None):
    tables = _deal_tables(rng, lens, bs, num_blocks)
    return Workload(
        name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
        cache_dtype=dtype, src_dtype=dtype, q_dtype=dtype,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        context_lens=lens.astype(np.int32), block_tables=tables, num_blocks=int(num_blocks),
        ops=_prefill_ops(lens), _kv=_plain_kv(seed, lens, Hkv, D, dtype),
        _q=_plain_q(seed, B, Hq, D, dtype),
    )


def tiny(seed: int = 3421) -> Workload:
    """Two sequences of 37 and 100 tokens, 4 heads (no grouping), head_dim 64, fp16, 32-block pool."""
    rng = _rng(seed, _LENS)
    lens = np.array([37, 100], np.int32)
    return _uniform_batch("tiny", seed, 2, 4, 4, 64, 16, "f16", lens, 32, rng, scale=1.0 / 8.0)


def llama8b(seed: int = 3422, B: int = 64) -> Workload:
    """Llama-3-8B-shaped layer: 32 q / 8 KV heads, head_dim 128, bf16, lengths U{512..4096}."""
    rng = _rng(seed, _LENS)
    lens = rng.integers(512, 4096, size=B, endpoint=True).astype(np.int32)
    nblk = int(((lens + 15) // 16).sum())
    return _uniform_batch("llama8b", seed, B, 32, 8, 128, 16, "bf16", lens, math.ceil(1.1 * nblk), rng)


def llama70b(seed: int = 3423, B: int = 32, L: int = 8000) -> Workload:
    """70B-class layer: 64 q / 8 KV heads, head_dim 128, fp16, every context 8000, 16,000-block pool."""
    rng = _rng(seed, _LENS)
    lens = np.full(B, L, np.int32)
    pool = 16000 if (B, L) == (32, 8000) else int(((lens + 15) // 16).sum())
    return _uniform_batch("llama70b", seed, B, 64, 8, 128, 16, "f16", lens, pool, rng)


def shared_prefix(seed: int = 3424, prompts: int = 16, samples: int = 8, prefix: int = 2048,
                  max_tail: int = 512) -> Workload:
    """Parallel sampling over shared prompts with a copy-on-write tail block.

    Prompt k stores prefix + delta_k tokens once (delta_k in 1..15, so its last
    shared block is partially filled); every sample's table points at those
    blocks.  Samples 0..samples-2 get a private copy of the partial block (one
    copy pair each); the last sample keeps writing into the original.  Each
    sample then appends its own tail of U{0..max_tail} tokens plus one decode
    token.
    """
    bs, Hq, Hkv, D, dt = 16, 32, 8, 128, "bf16"
    rng = _rng(seed, _LENS)
    delta = rng.integers(1, 15, size=prompts, endpoint=True).astype(np.int64)
    plen = prefix + delta  # shared tokens per prompt
    B = prompts * samples
    tails = rng.integers(0, max_tail, size=B, endpoint=True).astype(np.int64)
    lens = np.repeat(plen, samples) + tails + 1
    shared_blocks = (plen + bs - 1) // bs  # the last one is partial
    # blocks needed: shared once per prompt, one CoW copy per non-last sample,
    # then private blocks for what no longer fits in the (copied) partial block
    priv = []
    for s in range(B):
        k = s // samples
        used_in_partial = plen[k] - (shared_blocks[k] - 1) * bs
        rest = max(0, int(lens[s] - plen[k] - (bs - used_in_partial)))
        priv.append((rest + bs - 1) // bs)
    total = int(shared_blocks.sum()) + prompts * (samples - 1) + int(sum(priv))
    num_blocks = math.ceil(1.1 * total)
    perm = rng.permutation(num_blocks).astype(np.int32)
    M = int(((lens + bs - 1) // bs).max())
    tables = np.full((B, M), -1, np.int32)
    pairs = []
    off = 0
    for k in range(prompts):
        nb = int(shared_blocks[k])
        shared = perm[off:off + nb]
        off += nb
        for j in range(samples):
            s = k * samples + j
            tables[s, :nb] = shared
            if j < samples - 1:
                dst = perm[off]
                off += 1
                tables[s, nb - 1] = dst
                pairs.append((int(shared[nb - 1]), int(dst)))
    for s in range(B):
        nb_total = int((lens[s] + bs - 1) // bs)
        nb_shared = int(shared_blocks[s // samples])
        n = nb_total - nb_shared
        tables[s, nb_shared:nb_total] = perm[off:off + n]
        off += n
    assert off <= num_blocks
    rep = np.arange(prompts, dtype=np.int64) * samples + (samples - 1)
    seqs = np.arange(B, dtype=np.int64)
    ops = [
        WriteOp("append", rep, np.zeros(prompts, np.int64), plen.copy()),
        WriteOp("copy", pairs=np.array(pairs, np.int64).reshape(-1, 2)),
        WriteOp("append", seqs, np.repeat(plen, samples), lens - 1),
        WriteOp("append", seqs, lens - 1, lens),
    ]

    def kv(s):
        k = s // samples
        n_tail = int(lens[s] - plen[k])
        pk = _rng(seed, _KEY, k).standard_normal((int(plen[k]), Hkv, D), dtype=np.float32)
        pv = _rng(seed, _VAL, k).standard_normal((int(plen[k]), Hkv, D), dtype=np.float32)
        tk = _rng(seed, _TAIL_K, s).standard_normal((n_tail, Hkv, D), dtype=np.float32)
        tv = _rng(seed, _TAIL_V, s).standard_normal((n_tail, Hkv, D), dtype=np.float32)
        return (to_storage(np.concatenate([pk, tk]), dt), to_storage(np.concatenate([pv, tv]), dt))

    return Workload(
        name="shared_prefix", seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
        cache_dtype=dt, src_dtype=dt, q_dtype=dt, scale=1.0 / math.sqrt(D),
        context_lens=lens.astype(np.int32), block_tables=tables, num_blocks=num_blocks,
        ops=ops, _kv=kv, _q=_plain_q(seed, B, Hq, D, dt),
        meta={"prompts": prompts, "samples": samples, "shared_len": plen.astype(np.int32),
              "cow_pairs": np.array(pairs, np.int64).reshape(-1, 2)},
    )


def heavy_tail_lengths(seed: int, B: int, median: float = 300.0, sigma: float = 1.5,
                       lo: int = 1, hi: int = 32768) -> np.ndarray:
    z = _rng(seed, _LENS).standard_normal(B)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int32)


def heavy_tail(seed: int = 3425, bs: int = 16, B: int = 256) -> Workload:
    """Log-normal lengths (median 300, clipped to [1, 32768]), fp8 e4m3 KV with per-tensor scales.

    Key/value rows are N(0,1) cast to bf16; the per-tensor scale is the largest
    magnitude over all rows that are written, divided by 448 (the largest
    finite E4M3FN value).  The same lengths and values are used for every
    block size.
    """
    lens = heavy_tail_lengths(seed, B)
    rng = _rng(seed, _LENS, 1)
    nblk = int(((lens + bs - 1) // bs).sum())
    w = _uniform_batch("heavy_tail", seed, B, 32, 8, 128, bs, "bf16", lens, math.ceil(1.1 * nblk), rng)
    w.cache_dtype = "fp8"
    w.name = f"heavy_tail_bs{bs}"
    kmax = vmax = 0.0
    for s in range(B):
        k, v = w.seq_kv(s)
        kmax = max(kmax, float(np.abs(storage_to_f32(k, "bf16")).max()))
        vmax = max(vmax, float(np.abs(storage_to_f32(v, "bf16")).max()))
    w.k_scale = float(np.float32(kmax) / np.float32(448.0))
    w.v_scale = float(np.float32(vmax) / np.float32(448.0))
    return w


def custom(name: str, seed: int, lens, Hq: int, Hkv: int, D: int, bs: int, cache_dtype: str,
           q_dtype: Optional[str] = None, num_blocks: Optional[int] = None,
           scale: Optional[float] = None, src_dtype: Optional[str] = None) -> Workload:
    """A plain batch with the given lengths (edge-case sweeps).  The rows handed
    to the scatter are in src_dtype: the cache dtype for 16-bit caches, bf16
    (or f16 when given) for fp8 and fp4 caches."""
    lens = np.asarray(lens, np.int32)
    rng = _rng(seed, _LENS)
    nblk = int(((lens + bs - 1) // bs).sum())
    pool = num_blocks if num_blocks is not None else max(1, math.ceil(1.1 * nblk) + 1)
    src = (src_dtype or "bf16") if cache_dtype in ("fp8", "fp4") else cache_dtype
    w = _uniform_batch(name, seed, len(lens), Hq, Hkv, D, bs, src, lens, pool, rng, scale)
    w.q_dtype = q_dtype or src
    w._q = _plain_q(seed, len(lens), Hq, D, w.q_dtype)
    if cache_dtype == "fp4":  # rows carry their own scales; no per-tensor scale
        w.cache_dtype = "fp4"
    if cache_dtype == "fp8":
        w.cache_dtype = "fp8"
        kmax = vmax = 1e-30
        for s in range(len(lens)):
            if lens[s]:
                k, v = w.seq_kv(s)
                kmax = max(kmax, float(np.abs(storage_to_f32(k, src)).max()))
                vmax = max(vmax, float(np.abs(storage_to_f32(v, src)).max()))
        w.k_scale = float(np.float32(kmax) / np.float32(448.0))
        w.v_scale = float(np.float32(vmax) / np.float32(448.0))
    return w


def multi_query(name: str, seed: int, lens, nqs, Hq: int, Hkv: int, D: int, bs: int, cache_dtype: str,
                q_dtype: Optional[str] = None) -> Workload:
    """Sequences whose last nqs[s] positions are queries (a chunk of a chunked
    prefill, or draft tokens to verify); the cache holds all of every
    sequence's rows, the chunk's included.  Queries are N(0,1) rows of its own
    stream, one per query token."""
    w = custom(name, seed, lens, Hq, Hkv, D, bs, cache_dtype, q_dtype)
    nqs = np.asarray(nqs, np.int64)
    assert len(nqs) == w.B and (nqs >= 0).all() and (nqs <= w.context_lens).all()
    w.query_start = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    T = int(w.query_start[-1])
    qd = w.q_dtype
    w._q = lambda: to_storage(_rng(seed, _Q, 7).standard_normal((T, Hq, D), dtype=np.float32), qd)
    return w


def spec_decode(seed: int = 3426, B: int = 64, draft: int = 4) -> Workload:
    """Speculative verification on the 8B-shaped layer: the 8B-shaped lengths,
    each sequence verifying `draft` tokens (its last positions)."""
    base = llama8b(B=B)
    w = multi_query("spec_decode", seed, base.context_lens, [draft] * B, 32, 8, 128, 16, "bf16")
    return w


def chunked_prefill(seed: int = 3427, B: int = 16, chunk: int = 64) -> Workload:
    """Chunked prefill on the 8B-shaped layer: contexts U{512..4096} whose last
    `chunk` positions are this step's queries."""
    lens = _rng(seed, _LENS).integers(512, 4096, size=B, endpoint=True)
    return multi_query("chunked_prefill", seed, lens, [chunk] * B, 32, 8, 128, 16, "bf16")


CONFIGS = {
    "tiny": tiny,
    "llama8b": llama8b,
    "llama70b": llama70b,
    "shared_prefix": shared_prefix,
    "heavy_tail": heavy_tail,
    "spec_decode": spec_decode,
    "chunked_prefill": chunked_prefill,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)
