"""pa_decode_shared_prefix (each group's shared prefix read once, then each
sequence's own positions, combined) against the oracle's plain decode over
the same pools: the pages' sharing changes the reading, not the attention.

Cases: the shared-prefix parallel-sampling batch (reduced, and full size on
sampled sequences); random groups with prefixes of 0, of whole blocks, of
partial blocks and chunks, up to L - 1, groups of one; fp8 and fp16 caches,
both head_dims and block sizes; and a batch whose sequences all form groups
of one (prefix 0), which is plain decode."""
import numpy as np
import pytest
import torch

import paged_kv_cache_342_amd as pa
import workloads as W
from oracle import harness as OH
from oracle import pa_oracle as O
from tests.gpu_util import GpuBatch, errors, log, storage_to_torch, tolerance

pytestmark = pytest.mark.gpu


def _check_result(got, ref, cache_dtype, label):
    ma, rel = errors(got, ref)
    tol_abs, tol_rel = tolerance(cache_dtype)
    log(f"[shared prefix {label}] max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all()
    assert ma <= tol_abs
    if tol_rel is not None:
        assert rel <= tol_rel


def _run(b, w, group_start, prefix_lens, max_group):
    return pa.decode_shared_prefix(
        b.q, b.kc, b.vc, b.tables, b.lens, torch.tensor(group_start, dtype=torch.int32, device="cuda"),
        torch.tensor(prefix_lens, dtype=torch.int32, device="cuda"), max_group, w.scale,
        max_context_len=w.max_context_len, k_scale=w.k_scale, v_scale=w.v_scale, out_dtype=torch.float32)


def _sampling_groups(w):
    samples, plen = w.meta["samples"], w.meta["shared_len"]
    return [k * samples for k in range(len(plen) + 1)], [int(x) for x in plen], samples


@pytest.mark.parametrize("make,seqs", [
    (lambda: W.shared_prefix(prompts=2, samples=4, prefix=256, max_tail=100), None),
    (lambda: W.shared_prefix(prompts=3, samples=5, prefix=700, max_tail=40), None),
    (lambda: W.shared_prefix(), [0, 1, 7, 8, 63, 64, 120, 127]),
], ids=["2x4", "3x5", "full_sampled"])
def test_parallel_sampling_batch(make, seqs):
    w = make()
    b = GpuBatch(w)
    gs, pl, ng = _sampling_groups(w)
    got = _run(b, w, gs, pl, ng).cpu().numpy().astype(np.float64)
    kc, vc = OH.build_pools(w, seqs=seqs)
    ref = OH.decode(w, kc, vc, seqs=seqs)
    _check_result(got if seqs is None else got[seqs], ref, w.cache_dtype, w.name)
    # the same batch through pa_decode reads every prefix per sample; both agree
    plain = b.decode().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(plain - got)) <= 2 * tolerance(w.cache_dtype)[0]


def _grouped_case(seed, groups, cache, q, D, bs, Hkv=2, G=4):
    """Pools and tables for groups of sequences sharing prefixes.  groups: a
    list of (prefix, [member lengths]).  A group's whole prefix blocks are one
    set of blocks in every member's table; a partially filled prefix block is
    copied into a block of each member's own (copy-on-write), which then
    continues with the member's rows.  Returns the numpy pools (oracle
    storage), tables, lengths, group arrays and the query."""
    rng = np.random.default_rng(seed)
    lens = [L for _, ms in groups for L in ms]
    B = len(lens)
    M = max((L + bs - 1) // bs for L in lens)
    nb = sum((L + bs - 1) // bs for L in lens) + 4
    perm = list(rng.permutation(nb))
    kc, vc = O.new_pool(nb, Hkv, bs, D, cache), O.new_pool(nb, Hkv, bs, D, cache)
    tables = np.full((B, M), -1, np.int32)
    scale_k = scale_v = 1.0
    if cache == "fp8":
        scale_k, scale_v = 4.0 / 448, 4.0 / 448

    def rows(n):
        x = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        return W.to_storage(x, q if cache == "fp8" else cache)

    s = 0
    for prefix, members in groups:
        shared_k, shared_v = rows(prefix), rows(prefix)
        full = prefix // bs
        shared_ids = [perm.pop() for _ in range(full)]
        for L in members:
            own_k, own_v = rows(L - prefix), rows(L - prefix)
            k_all, v_all = np.concatenate([shared_k, own_k]), np.concatenate([shared_v, own_v])
            n = (L + bs - 1) // bs
            tables[s, :full] = shared_ids
            tables[s, full:n] = [perm.pop() for _ in range(n - full)]
            # every member writes all of its rows; the shared blocks receive
            # the same rows from each member
            src = q if cache == "fp8" else cache
            O.reshape_and_cache(k_all, v_all, kc, vc, O.slots_for(tables[s], 0, L, bs), bs, cache, scale_k, scale_v,
                                src_dtype=src)
            s += 1
    gs = np.concatenate([[0], np.cumsum([len(ms) for _, ms in groups])]).astype(np.int32)
    pl = np.array([p for p, _ in groups], np.int32)
    qv = W.to_storage(rng.standard_normal((B, Hkv * G, D)).astype(np.float32), q)
    return kc, vc, tables, np.array(lens, np.int32), gs, pl, qv, scale_k, scale_v


def _to_device_pool(pool, cache):
    t = torch.from_numpy(pool.view(np.uint8) if cache == "fp8" else pool.view(np.int16)).cuda()
    return t.view(torch.float8_e4m3fn if cache == "fp8" else (torch.float16 if cache == "f16" else torch.bfloat16))


GROUPS = [
    (0, [1, 40]),                 # no shared prefix
    (16, [17, 100, 33]),          # one whole block
    (37, [38, 39, 300]),          # a partial block, L = prefix + 1
    (64, [65, 1000]),             # two chunks exactly
    (513, [514, 700, 900, 2000, 519, 600, 601, 1031]),  # eight samples
    (200, [201]),                 # a group of one
    (1500, [1510, 1600, 1501]),   # a long prefix, short tails
]


@pytest.mark.parametrize("cache,q", [("f16", "f16"), ("bf16", "bf16"), ("fp8", "bf16"), ("fp8", "f16")])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_random_groups(cache, q, D, bs):
    G = 4
    kc, vc, tables, lens, gs, pl, qv, ks, vs = _grouped_case(500 + bs + D, GROUPS, cache, q, D, bs, G=G)
    Hkv = kc.shape[1]
    dkc, dvc = _to_device_pool(kc, cache), _to_device_pool(vc, cache)
    out = pa.decode_shared_prefix(storage_to_torch(qv, q).cuda(), dkc, dvc, torch.from_numpy(tables).cuda(),
                                  torch.from_numpy(lens).cuda(), torch.from_numpy(gs).cuda(),
                                  torch.from_numpy(pl).cuda(), 8, 1 / np.sqrt(D), k_scale=ks, v_scale=vs,
                                  out_dtype=torch.float32)
    got = out.cpu().numpy().astype(np.float64)
    ref = O.decode(qv, kc, vc, tables, lens, 1 / np.sqrt(D), G, cache, q, ks, vs)
    _check_result(got, ref, cache, f"groups {cache} q={q} D={D} bs={bs} Hkv={Hkv}")


def test_groups_of_one_without_prefix_are_decode():
    w = W.llama8b(B=12)
    b = GpuBatch(w)
    got = _run(b, w, list(range(w.B + 1)), [0] * w.B, 1).cpu().numpy().astype(np.float64)
    kc, vc = OH.build_pools(w)
    _check_result(got, OH.decode(w, kc, vc), w.cache_dtype, "groups of one")


def test_shared_prefix_rejects_bad_host_arguments():
    w = W.shared_prefix(prompts=2, samples=4, prefix=256, max_tail=100)
    b = GpuBatch(w)
    gs, pl, ng = _sampling_groups(w)
    with pytest.raises(pa.PagedAttentionError) as e:
        _run(b, w, gs, pl, 0)
    assert e.value.status == pa.ERR_UNSUPPORTED
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.decode_shared_prefix(b.q, b.kc, b.vc, b.tables, b.lens, torch.tensor(gs, dtype=torch.int32).cuda(),
                                torch.tensor(pl, dtype=torch.int32).cuda(), ng, w.scale, workspace=ws)
    assert e.value.status == pa.ERR_WORKSPACE
