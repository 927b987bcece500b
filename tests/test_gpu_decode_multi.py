"""pa_decode_multi (several query tokens per sequence, causal within them)
against the oracle: speculative verification and chunked prefill on the
8B-shaped layer, and a sweep over group sizes, head dims, block sizes,
dtypes, query counts (none, a few, the whole sequence) and lengths."""
import numpy as np
import pytest
import torch

import paged_kv_cache_342_amd as pa
import workloads as W
from oracle import harness as OH
from tests.gpu_util import GpuBatch, errors, log, set_variant, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_variant():
    set_variant(None)
    yield
    set_variant(None)


def _check_multi(w, seqs=None, label="", batch=None, **kw):
    log(f"[decode_multi {w.name}{label}] T={int(w.query_start[-1])} max_queries={w.max_queries}")
    g = batch or GpuBatch(w)
    out = g.decode_multi(**kw).cpu().numpy().astype(np.float64)
    kc, vc = OH.build_pools(w, seqs=seqs)
    ref = OH.decode_multi(w, kc, vc, seqs=seqs)
    if seqs is None:
        rows = np.arange(out.shape[0])
    else:
        rows = np.concatenate([np.arange(w.query_start[s], w.query_start[s + 1]) for s in seqs]).astype(np.int64)
    ma, rel = errors(out[rows], ref[rows])
    tol_abs, tol_rel = tolerance(w.cache_dtype)
    log(f"  max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.isfinite(out[rows]).all()
    assert ma <= tol_abs
    if tol_rel is not None:
        assert rel <= tol_rel
    return g, out


def test_spec_decode_reduced():
    _check_multi(W.spec_decode(B=6), label="[B=6]")


def test_spec_decode_full_size_sampled():
    w = W.spec_decode()
    _check_multi(w, seqs=[int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens)), 17, 40],
                 label="[full, sampled]")


def test_chunked_prefill_reduced():
    _check_multi(W.chunked_prefill(B=3), label="[B=3]")


def test_chunked_prefill_full_size_sampled():
    _check_multi(W.chunked_prefill(), seqs=[0, 7, 15], label="[full, sampled]")


@pytest.mark.parametrize("cache,q", [("f16", "f16"), ("bf16", "bf16"), ("fp8", "bf16")])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_multi_query_sweep(cache, q, D, bs):
    """Lengths around block and chunk boundaries with 0, 1, a few, and all of
    a sequence's positions as queries (a whole prefill), for groups 1 to 16
    (tiles of 16 (query, head) columns: one to several per KV head)."""
    lens = [1, 2, 17, 31, 33, 64, 65, 130, 300, 515, 9, 40]
    nqs = [1, 2, 5, 0, 33, 7, 1, 16, 3, 12, 9, 40]
    for g in (1, 2, 4, 8, 16):
        w = W.multi_query(f"mq_{cache}_{q}_D{D}_bs{bs}_g{g}", 300 + g, lens, nqs, 2 * g, 2, D, bs, cache, q)
        _check_multi(w)


def test_one_query_per_sequence_is_decode_bit_for_bit():
    """With one query per sequence the call computes what pa_decode's MFMA
    kernel computes, bit for bit."""
    lens = [int(x) for x in np.random.default_rng(41).integers(1, 900, size=40)]
    w = W.multi_query("mq_one", 42, lens, [1] * 40, 32, 8, 128, 16, "bf16")
    g, out = _check_multi(w)
    set_variant("mfma")
    dec = g.decode().cpu().numpy().astype(np.float64)
    assert np.array_equal(out, dec)


def test_multi_query_many_columns_per_kv_head():
    """256 queries of one sequence at group 4: 64 tiles of 16 columns per KV head."""
    w = W.multi_query("mq_wide", 43, [300, 700], [256, 100], 8, 2, 128, 16, "bf16")
    _check_multi(w)


def test_multi_query_batch_split_into_launches():
    lens = [int(x) for x in np.random.default_rng(44).integers(1, 500, size=120)]
    nqs = [min(L, int(n)) for L, n in zip(lens, np.random.default_rng(45).integers(0, 9, size=120))]
    w = W.multi_query("mq_sub_batches", 46, lens, nqs, 8, 2, 128, 16, "f16")
    _check_multi(w, max_context_len=1 << 30)


def test_multi_query_rejects_bad_arguments():
    w = W.multi_query("mq_bad", 47, [20, 30], [2, 3], 8, 2, 64, 16, "f16")
    g = GpuBatch(w)
    qs = torch.from_numpy(w.query_start).cuda()
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode_multi(g.q, g.kc, g.vc, g.tables, g.lens, qs, 2000, w.scale)
    assert e.value.status == pa.ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        pa.decode_multi(g.q, g.kc, g.vc, g.tables, g.lens, qs[:2], 3, w.scale)


def test_multi_query_more_sequences_than_one_launch_scans():
    """3,100 sequences: more than the 3,072 a multi-query launch scans (its
    query rows sit in LDS beside the lengths), so two launches share the call."""
    rng = np.random.default_rng(48)
    lens = [int(x) for x in rng.integers(0, 50, size=3100)]
    nqs = [min(L, int(n)) for L, n in zip(lens, rng.integers(0, 4, size=3100))]
    w = W.multi_query("mq_many_seqs", 49, lens, nqs, 4, 2, 64, 16, "f16")
    seqs = [0, 1, 3070, 3071, 3072, 3073, 3099] + [int(i) for i in np.nonzero(np.array(nqs) > 0)[0][:5]]
    _check_multi(w, seqs=sorted(set(seqs)))


def test_prefill_kernel_more_sequences_than_one_launch_takes():
    """600 sequences of up to 32 queries at G = 4 (128 columns a KV head, the
    prefill kernel): more than the 512 a prefill launch takes (its query rows
    and K/V stages fill the rest of LDS), so two launches share the call."""
    rng = np.random.default_rng(52)
    lens = [int(x) for x in rng.integers(32, 120, size=600)]
    nqs = [min(L, int(n)) for L, n in zip(lens, rng.integers(20, 33, size=600))]
    nqs[0] = 32
    w = W.multi_query("prefill_many_seqs", 53, lens, nqs, 8, 2, 128, 16, "bf16")
    _check_multi(w, seqs=[0, 1, 510, 511, 512, 513, 599], label="[two prefill launches]")


@pytest.mark.parametrize("cache,D,bs,G", [("bf16", 128, 16, 4), ("f16", 64, 8, 8), ("bf16", 128, 32, 4),
                                          ("f16", 128, 16, 16)])
@pytest.mark.parametrize("mode", ["1", "2", "3"])
def test_shared_chunk_kernel_equals_one_wave_kernel(cache, D, bs, G, mode, monkeypatch):
    """Queries spanning several tiles run a kernel whose waves share each K/V
    chunk through LDS: four waves of two tiles (mode 1), eight waves of one
    tile at two waves per SIMD (mode 2), or the prefill kernel's 32 x 32
    tiles (mode 3, the default).  Modes 1 and 2 read the bytes the one-wave
    kernel reads (PA_DECODE_MQ_SHARED=0) and do the same arithmetic per tile,
    so they must agree with it bit for bit; every mode agrees with the
    oracle.  Some sequences have fewer queries than the workgroup has
    columns, so some waves only load."""
    lens = [40, 300, 1031, 77, 513, 64, 129, 2050]
    nqs = [32, 64, 40, 5, 64, 64, 1, 48]
    w = W.multi_query(f"mq_shared_{cache}_D{D}_bs{bs}_g{G}", 330 + G, lens, nqs, 2 * G, 2, D, bs, cache)
    monkeypatch.setenv("PA_DECODE_MQ_SHARED", mode)
    g, out = _check_multi(w, label=f"[shared chunks, mode {mode}]")
    if mode != "3":
        monkeypatch.setenv("PA_DECODE_MQ_SHARED", "0")
        one = g.decode_multi().cpu().numpy()
        assert np.array_equal(out.astype(np.float32), one)


@pytest.mark.parametrize("seed", range(6))
def test_shared_chunk_kernels_on_random_shapes(seed, monkeypatch):
    """Seeded random batches (group 1-16, head_dim 64/128, block size 8/16/32,
    f16/bf16, empty sequences, sequences without queries, query counts up to
    the length): both 16-column shared-chunk kernels equal the one-wave
    kernel bit for bit, and the default (the prefill kernel) is within
    tolerance of the oracle and gives the same bits on every call."""
    rng = np.random.default_rng(900 + seed)
    G = [1, 2, 4, 8, 16, 4][seed]
    D = [64, 128][seed % 2]
    bs = int(rng.choice([8, 16, 32]))
    cache = str(rng.choice(["f16", "bf16"]))
    B = int(rng.integers(3, 12))
    lens = [int(x) for x in rng.integers(0, 1500, size=B)]
    lens[0] = max(lens[0], 160)  # at least one sequence with enough queries for the shared kernels
    lens[-1] = 0  # an empty sequence
    nqs = [int(rng.integers(0, min(L, 96) + 1)) for L in lens]
    nqs[0] = max(nqs[0], min(lens[0], -(-128 // G)))
    nqs[1] = 0  # a sequence without queries
    w = W.multi_query(f"mq_rand{seed}_{cache}_D{D}_bs{bs}_g{G}", 910 + seed, lens, nqs, 2 * G, 2, D, bs, cache)
    log(f"[random shapes seed={seed}] G={G} D={D} bs={bs} {cache} lens={lens} nqs={nqs}")
    g, out = _check_multi(w, label=f"[random {seed}]")
    res = {}
    for mode in ("0", "1", "2", "3"):
        monkeypatch.setenv("PA_DECODE_MQ_SHARED", mode)
        res[mode] = g.decode_multi().cpu().numpy()
    assert np.array_equal(res["1"], res["0"]) and np.array_equal(res["2"], res["0"])
    assert np.array_equal(out.astype(np.float32), res["3"])


@pytest.mark.parametrize("cache,D,bs,G,nq", [("bf16", 128, 16, 4, 64), ("f16", 128, 8, 8, 64), ("bf16", 64, 32, 4, 100),
                                             ("f16", 64, 16, 16, 40), ("bf16", 128, 32, 1, 300)])
def test_prefill_kernel_shapes(cache, D, bs, G, nq):
    """The prefill kernel (256 (query, head) columns per workgroup of eight
    waves, 32 x 32 tiles) on chunks that need one or several column groups
    (nq * G up to 512), query chunks shorter than the sequence and equal to
    it, ragged lengths around chunk and block boundaries, and sequences cut
    by slices (long ones)."""
    lens = [nq, nq + 1, 2 * nq + 31, 1000, 4097, 33, 0, 777]
    nqs = [min(L, n) for L, n in zip(lens, [nq, nq, nq, nq, nq, nq, 0, nq // 2])]
    w = W.multi_query(f"prefill_{cache}_D{D}_bs{bs}_g{G}_n{nq}", 950 + G + nq, lens, nqs, 2 * G, 2, D, bs, cache)
    _check_multi(w, label="[prefill kernel]")


@pytest.mark.parametrize("G,nq", [(3, 100), (5, 60), (6, 90)])
def test_prefill_kernel_groups_that_do_not_divide_its_columns(G, nq):
    """Group sizes 3, 5 and 6 through the prefill kernel: its 256 (query, head)
    columns per workgroup then end inside a query, whose heads fall into two
    column groups (and a group's last wave may hold dead columns)."""
    lens = [nq, 2 * nq + 7, 1000, 513, 0, 3000]
    nqs = [min(L, nq) for L in lens]
    w = W.multi_query(f"prefill_g{G}", 970 + G, lens, nqs, 2 * G, 2, 128, 16, "bf16")
    _check_multi(w, label=f"[prefill kernel, G={G}]")



def test_prefill_kernel_at_the_largest_query_count():
    """1,024 queries per sequence (the most pa_decode_multi takes) at group 4:
    4,096 (query, head) columns, sixteen 256-column groups of the prefill
    kernel per KV head, over a whole-sequence prefill and a chunk of a longer
    sequence."""
    w = W.multi_query("prefill_max_queries", 990, [1024, 1500, 40], [1024, 1024, 40], 8, 2, 128, 16, "bf16")
    _check_multi(w, label="[prefill kernel, 1024 queries]")


@pytest.mark.parametrize("seed", range(3))
def test_prefill_kernel_slices_of_many_short_sequences(seed):
    """300 short sequences (0-200 positions, 0-32 queries, some without
    queries and some empty) at group 4: a workgroup's slice then walks
    several sequences in a row, with one to seven 32-position chunks each,
    and requests a sequence's first chunks and query rows while it still
    works on the one before.  Every sequence against the oracle."""
    rng = np.random.default_rng(1200 + seed)
    lens = [int(x) for x in rng.integers(0, 201, size=300)]
    nqs = [min(L, int(n)) for L, n in zip(lens, rng.integers(0, 33, size=300))]
    for i in range(0, 300, 7):
        nqs[i] = 0
    lens[5] = 0
    nqs[5] = 0
    lens[1] = max(lens[1], 64)
    nqs[1] = 32  # 128 columns a KV head: the prefill kernel
    w = W.multi_query(f"prefill_short_seqs{seed}", 1210 + seed, lens, nqs, 8, 2, 128, 16, "bf16")
    g, out = _check_multi(w, label="[prefill kernel, many short sequences]")
    again = g.decode_multi().cpu().numpy()
    assert np.array_equal(out.astype(np.float32), again)


@pytest.mark.parametrize("scale", [0.0, -0.088, 1e-3, 0.5])
def test_prefill_shapes_at_any_scale(scale):
    """Query chunks the prefill kernel takes, at scales of either sign: the
    prefill kernel applies a positive scale inside its exponentials; a zero
    or negative one (the weights then favour the smallest scores, or are all
    equal) goes to the 16-column kernels.  Every case against the oracle."""
    lens = [64, 300, 1031, 2050]
    nqs = [64, 64, 40, 64]
    w = W.multi_query(f"prefill_scale_{scale}", 1300, lens, nqs, 8, 2, 128, 16, "bf16")
    w.scale = float(scale)
    _check_multi(w, label=f"[scale {scale}]")
