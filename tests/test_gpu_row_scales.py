"""FP8 and FP4 caches with one scale per (slot, kv head) row: the scatter bit
for bit (codes and scales), the block copy bit for bit, and the decode
against the oracle.

Decode bound, from the kernel's arithmetic (fp32 output against the fp64
oracle over the same codes and scales):
  |out - ref| <= 3e-2 + (pv + 2 * (D + 8) * 2^-24 * A) * max|V|
* pv: PV takes each weight w = p * v_scale as two bf16 terms hi + lo with
  hi = RNE(w) and lo = RNE(w - hi), which hold w to 2^-18 relative; the
  products with the (exactly widened) codes are exact in fp32, and the
  accumulator rounds at most L/8 + 16 times (two MFMAs per 16 positions,
  rescales, the merge), 2^-24 each; 2^-21 covers the exp2 approximation of
  p, which the denominator shares only in part.  pv = 2^-17 + 2^-21 +
  (L_max / 8 + 16) * 2^-24, about 2^-16 at L_max = 1031.
* scores: q . k sums D exact products in fp32 and is then scaled twice;
  each of at most D + 8 roundings is within 2^-24 of A = max over heads and
  positions of scale * sum_d |q_d| |k_d| (K dequantised), so a score is off
  by at most (D + 8) 2^-24 A, and the normalised weights by twice that,
  relative.
Rows of unit magnitude meet the FP8 gate (max-abs 3e-2, relative L2 1e-3).
Rows whose K and V both spread over six decades have scores of ~1e4, where
the score term dominates; rows whose V alone spreads, with the query scaled
by 2^-4, leave the PV term alone, so a coarser PV (fp16 weights, 2^-11)
would fail there."""
import numpy as np
import pytest
import torch

import paged_kv_cache_342_amd as pa
import workloads as W
from oracle import pa_oracle as O
from tests.gpu_util import errors, log, storage_to_torch

pytestmark = pytest.mark.gpu


def _rows(w, spread, seed, k_spread=None):
    """Every sequence's K/V rows (bf16 storage), each (token, head) row scaled
    by 10^U(-spread, spread) so rows differ in magnitude (K by
    10^U(-k_spread, k_spread) when given); and their slots."""
    rng = np.random.default_rng(seed)
    ks, vs, slots = [], [], []
    k_spread = spread if k_spread is None else k_spread
    for s in range(w.B):
        L = int(w.context_lens[s])
        if L == 0:
            continue
        k, v = w.seq_kv(s)
        u = rng.uniform(-1.0, 1.0, size=(2, L, w.Hkv, 1))
        fk, fv = 10.0 ** (k_spread * u[0]), 10.0 ** (spread * u[1])
        ks.append(W.to_storage(W.storage_to_f32(k, "bf16") * fk.astype(np.float32), "bf16"))
        vs.append(W.to_storage(W.storage_to_f32(v, "bf16") * fv.astype(np.float32), "bf16"))
        slots.append(O.slots_for(w.block_tables[s], 0, L, w.bs))
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(slots).astype(np.int64)


def _pools(w, k, v, slots):
    nb, Hkv, bs, D = w.num_blocks, w.Hkv, w.bs, w.D
    cd = w.cache_dtype
    if cd == "fp4":
        kc = torch.full((nb, Hkv, bs, D // 2), 0x77, dtype=torch.uint8, device="cuda").view(torch.float4_e2m1fn_x2)
    else:
        kc = torch.full((nb, Hkv, bs, D), 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    vc = kc.clone()
    kss = torch.full((nb, Hkv, bs), float("nan"), dtype=torch.float32, device="cuda")
    vss = kss.clone()
    step = 1 << 15
    for i in range(0, len(slots), step):
        pa.reshape_and_cache_scaled(storage_to_torch(k[i:i + step], "bf16").cuda(),
                                    storage_to_torch(v[i:i + step], "bf16").cuda(), kc, vc, kss, vss,
                                    torch.from_numpy(slots[i:i + step]).cuda())
    okc, ovc = O.new_pool(nb, Hkv, bs, D, cd), O.new_pool(nb, Hkv, bs, D, cd)
    oks = np.full((nb, Hkv, bs), np.nan, np.float32)
    ovs = oks.copy()
    O.reshape_and_cache_scaled(k, v, okc, ovc, oks, ovs, slots, bs, "bf16", cd)
    return (kc, vc, kss, vss), (okc, ovc, oks, ovs)


def _same_bits(t, a):
    return np.array_equal(t.cpu().view(torch.uint8).numpy() if t.element_size() == 1 else
                          t.cpu().numpy().view(np.uint32), a.view(np.uint8) if a.dtype == np.uint8 else a.view(np.uint32))


@pytest.mark.parametrize("cd", ["fp8", "fp4"])
def test_scatter_with_row_scales_is_bit_exact(cd):
    w = W.custom(f"rs_scatter_{cd}", 61, [1, 15, 16, 17, 100, 300], 8, 4, 128, 16, cd)
    k, v, slots = _rows(w, 3.0, 62)
    # special rows: zeros, an infinity, NaN elements, a skipped token
    k[0] = 0
    k[1, 0, 5] = W.to_storage(np.array([np.inf], np.float32), "bf16")[0]
    v[2, 1, :3] = W.to_storage(np.array([np.nan] * 3, np.float32), "bf16")
    slots[3] = -1
    (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)
    assert np.array_equal(kss.cpu().numpy(), oks, equal_nan=True)
    assert np.array_equal(vss.cpu().numpy(), ovs, equal_nan=True)
    if cd == "fp4":  # E2M1 ties: every tie of the grid, both signs, through the same path
        t = np.arange(-24, 25, dtype=np.float32) * 0.25
        row = np.zeros((1, w.Hkv, 128), np.float32)
        row[0, 0, :49] = t
        row[0, 0, 49] = 6.0  # the row's scale is then exactly 1
        kt = W.to_storage(row, "bf16")
        kc = torch.zeros(tuple(kc.shape), dtype=torch.uint8, device="cuda").view(torch.float4_e2m1fn_x2)
        vc = kc.clone()
        pa.reshape_and_cache_scaled(storage_to_torch(kt, "bf16").cuda(), storage_to_torch(kt, "bf16").cuda(), kc, vc,
                                    kss, vss, torch.tensor([0], dtype=torch.int64, device="cuda"))
        assert float(kss[0, 0, 0]) == 1.0
        want = O.e2m1_pack(O.e2m1_encode(row[0, 0], 1.0))
        assert np.array_equal(kc[0, 0, 0].cpu().view(torch.uint8).numpy(), want)


def _bound(w, q, okc, oks, ovc, ovs, seqs=None):
    """The decode bound of the module docstring for these pools and queries
    (q in storage form), over the sequences `seqs` (default: all)."""
    cd, D = w.cache_dtype, w.D
    seqs = range(w.B) if seqs is None else seqs
    vmax = float(np.nanmax(np.abs(O.widen_rows(ovc, ovs, cd))))
    A, lmax = 0.0, 0
    for s in seqs:
        L = int(w.context_lens[s])
        if L == 0:
            continue
        lmax = max(lmax, L)
        k = O.widen_rows(O.gather_kv(okc, w.block_tables[s], L),
                         O.gather_kv(oks[..., None], w.block_tables[s], L)[..., 0], cd)  # [L, Hkv, D]
        qa = np.abs(O.widen(q[s], w.q_dtype)).reshape(w.Hkv, w.group, D)
        A = max(A, float(np.einsum("hgd,lhd->hgl", qa, np.abs(k)).max()) * abs(w.scale))
    pv = 2.0 ** -17 + 2.0 ** -21 + (lmax / 8 + 16) * 2.0 ** -24
    return 3e-2 + (pv + 2 * (D + 8) * 2.0 ** -24 * A) * vmax


def _scaled_query(w, factor):
    """The workload's queries times a power of two, in their storage dtype."""
    return W.to_storage(W.storage_to_f32(w.query(), w.q_dtype) * np.float32(factor), w.q_dtype)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("q", ["f16", "bf16"])
@pytest.mark.parametrize("spread", [0.0, 3.0])
@pytest.mark.parametrize("cd", ["fp8", "fp4"])
def test_decode_with_row_scales(D, bs, q, spread, cd):
    lens = [0, 1, 7, 31, 33, 64, 129, 300, 517, 1031]
    for g in (1, 2, 4, 8, 16):
        w = W.custom(f"rs_{cd}_D{D}_bs{bs}_{q}_g{g}", 70 + g, lens, 2 * g, 2, D, bs, cd, q)
        k, v, slots = _rows(w, spread, 80 + g)
        (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
        qd = storage_to_torch(w.query(), q).cuda()
        out = pa.decode_scaled(qd, kc, vc, kss, vss, torch.from_numpy(w.block_tables).cuda(),
                               torch.from_numpy(w.context_lens).cuda(), w.scale,
                               out_dtype=torch.float32).cpu().numpy().astype(np.float64)
        ref = O.decode_scaled(w.query(), okc, ovc, oks, ovs, w.block_tables, w.context_lens, w.scale, g, q,
                              cache_dtype=cd)
        ma, rel = errors(out, ref)
        bound = _bound(w, w.query(), okc, oks, ovc, ovs)
        log(f"[row scales {cd} D={D} bs={bs} q={q} g={g} spread={spread}] max_abs={ma:.2e} (bound {bound:.2e}) "
            f"rel_l2={rel:.2e}")
        assert np.isfinite(out).all() and ma <= bound and rel <= 1e-3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("q", ["f16", "bf16"])
@pytest.mark.parametrize("cd", ["fp8", "fp4"])
def test_decode_with_row_scales_pv_precision(D, q, cd):
    """V rows spread over six decades, K rows of unit magnitude and the query
    scaled by 2^-4: scores stay small, so the bound is about (2^-16 + 2^-19)
    max|V| and measures PV's precision."""
    lens = [1, 7, 33, 129, 517, 1031]
    for g in (1, 4, 8):
        w = W.custom(f"rs_pv_{cd}_D{D}_{q}_g{g}", 74 + g, lens, 2 * g, 2, D, 16, cd, q)
        k, v, slots = _rows(w, 3.0, 84 + g, k_spread=0.0)
        (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
        qs = _scaled_query(w, 2.0 ** -4)
        out = pa.decode_scaled(storage_to_torch(qs, q).cuda(), kc, vc, kss, vss,
                               torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(),
                               w.scale, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
        ref = O.decode_scaled(qs, okc, ovc, oks, ovs, w.block_tables, w.context_lens, w.scale, g, q, cache_dtype=cd)
        ma, rel = errors(out, ref)
        bound = _bound(w, qs, okc, oks, ovc, ovs)
        vmax = float(np.nanmax(np.abs(O.widen_rows(ovc, ovs, cd))))
        log(f"[row scales PV {cd} D={D} q={q} g={g}] max_abs={ma:.2e} = {ma / vmax:.2e} max|V| "
            f"(bound {bound:.2e} = {bound / vmax:.2e} max|V|) rel_l2={rel:.2e}")
        assert np.isfinite(out).all() and ma <= bound and rel <= 1e-3


@pytest.mark.parametrize("cd", ["fp8", "fp4"])
@pytest.mark.parametrize("base", ["heavy_tail", "llama8b"])
def test_decode_with_row_scales_full_size_sampled(base, cd):
    """The heavy-tailed batch (256 sequences, log-normal lengths) and the
    8B-shaped batch (64 sequences of 512 to 4,096 positions) at full size, as
    the row-scale and FP4 bench lines run them, with rows spread over six
    decades of magnitude, checked on sampled sequences."""
    w = W.heavy_tail(bs=16) if base == "heavy_tail" else W.llama8b()
    if cd == "fp4" or base == "llama8b":
        w = W.custom(f"{base}_{cd}", w.seed, w.context_lens, w.Hq, w.Hkv, w.D, w.bs, cd, w.q_dtype)
    k, v, slots = _rows(w, 3.0, 90)
    (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
    qd = storage_to_torch(w.query(), w.q_dtype).cuda()
    out = pa.decode_scaled(qd, kc, vc, kss, vss, torch.from_numpy(w.block_tables).cuda(),
                           torch.from_numpy(w.context_lens).cuda(), w.scale,
                           out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    order = np.argsort(w.context_lens)
    seqs = sorted({int(order[-1]), int(order[-2]), int(order[0]), int(order[len(order) // 2])})
    ref = O.decode_scaled(w.query(), okc, ovc, oks, ovs, w.block_tables, w.context_lens, w.scale, w.group,
                          w.q_dtype, seqs=seqs, cache_dtype=cd)
    ma, rel = errors(out[seqs], ref)
    bound = _bound(w, w.query(), okc, oks, ovc, ovs, seqs)
    log(f"[row scales {base} {cd}] max_abs={ma:.2e} (bound {bound:.2e}) rel_l2={rel:.2e}")
    assert np.isfinite(out).all() and ma <= bound and rel <= 1e-3


def test_row_scale_calls_reject_bad_arguments():
    w = W.custom("rs_bad", 63, [20], 4, 2, 64, 16, "fp8")
    k, v, slots = _rows(w, 1.0, 64)
    (kc, vc, kss, vss), _ = _pools(w, k, v, slots)
    with pytest.raises(ValueError):
        pa.reshape_and_cache_scaled(storage_to_torch(k, "bf16").cuda(), storage_to_torch(v, "bf16").cuda(), kc, vc,
                                    kss[:1], vss, torch.from_numpy(slots).cuda())
    f16cache = torch.zeros((w.num_blocks, 2, 16, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        pa.decode_scaled(torch.zeros((1, 4, 64), dtype=torch.float16, device="cuda"), f16cache, f16cache, kss, vss,
                         torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(), 0.1)


@pytest.mark.parametrize("cd", ["fp8", "fp4"])
def test_copy_blocks_scaled_is_bit_exact(cd):
    """Copy-on-write of a row-scaled cache copies the rows and their scales;
    the oracle's copy of the same pools agrees byte for byte."""
    w = W.custom(f"rs_copy_{cd}", 65, [40, 100, 7], 8, 4, 128, 16, cd)
    k, v, slots = _rows(w, 2.0, 66)
    (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
    used = [int(b) for b in w.block_tables[1][:5]]
    free = sorted(set(range(w.num_blocks)) - {int(b) for b in w.block_tables.ravel() if b >= 0})[:4]
    pairs = np.array([[used[0], free[0]], [used[3], free[1]], [used[3], free[2]], [used[1], used[1]]], np.int64)
    pa.copy_blocks_scaled(kc, vc, kss, vss, torch.from_numpy(pairs).cuda())
    O.copy_blocks(okc, ovc, pairs)
    O.copy_blocks(oks, ovs, pairs)
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)
    assert np.array_equal(kss.cpu().numpy(), oks, equal_nan=True)
    assert np.array_equal(vss.cpu().numpy(), ovs, equal_nan=True)
    assert np.isfinite(oks[free[1]]).all() and np.array_equal(oks[free[1]], oks[used[3]])


def test_fp4_cache_needs_row_scales():
    w = W.custom("fp4_plain", 67, [20], 4, 2, 64, 16, "fp4")
    k, v, slots = _rows(w, 1.0, 68)
    (kc, vc, kss, vss), _ = _pools(w, k, v, slots)
    lib = pa.library()
    # the plain calls refuse an FP4 cache on the host, before any launch
    st = lib.pa_reshape_and_cache(pa._ptr(storage_to_torch(k, "bf16").cuda()), pa._ptr(storage_to_torch(v, "bf16").cuda()),
                                  pa._ptr(kc), pa._ptr(vc), pa._ptr(torch.from_numpy(slots).cuda()), len(slots), 2, 64,
                                  16, w.num_blocks, pa.BF16, pa.FP4_E2M1, 1.0, 1.0, None)
    assert st == pa.ERR_UNSUPPORTED
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        pa.decode(q, kc, vc, torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(), 0.1)


@pytest.mark.parametrize("cd", ["fp8", "fp4"])
def test_row_scales_with_large_magnitudes_stay_finite(cd):
    """Rows near 1e5: a V weight p * scale then reaches 2^8 * 1e5 / 6 (FP4)
    or / 448 (FP8), beyond fp16; the kernel takes PV in bf16 for row-scaled
    caches, so the result stays finite and accurate."""
    w = W.custom(f"rs_big_{cd}", 69, [1, 40, 300, 1031], 16, 4, 128, 16, cd, "bf16")
    rng = np.random.default_rng(70)
    ks, vs, slots = [], [], []
    for s in range(w.B):
        L = int(w.context_lens[s])
        k, v = w.seq_kv(s)
        f = (1e5 * rng.uniform(0.5, 1.0, size=(2, L, w.Hkv, 1))).astype(np.float32)
        ks.append(W.to_storage(W.storage_to_f32(k, "bf16") * f[0] * 1e-5, "bf16"))  # K stays unit-sized
        vs.append(W.to_storage(W.storage_to_f32(v, "bf16") * f[1], "bf16"))
        slots.append(O.slots_for(w.block_tables[s], 0, L, w.bs))
    k, v, slots = np.concatenate(ks), np.concatenate(vs), np.concatenate(slots).astype(np.int64)
    (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
    out = pa.decode_scaled(storage_to_torch(w.query(), "bf16").cuda(), kc, vc, kss, vss,
                           torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(), w.scale,
                           out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    ref = O.decode_scaled(w.query(), okc, ovc, oks, ovs, w.block_tables, w.context_lens, w.scale, w.group, "bf16",
                          cache_dtype=cd)
    ma, rel = errors(out, ref)
    log(f"[row scales {cd}, |V| ~ 1e5] max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert np.isfinite(out).all() and rel <= 1e-3


def test_fp4_batch_across_launches():
    """FP4 kernels run two waves per SIMD and scan 2,048 sequences per launch:
    a batch of 2,100 short sequences is two launches.  Every sequence against
    the oracle."""
    rng = np.random.default_rng(71)
    lens = rng.integers(0, 48, size=2100)
    w = W.custom("rs_fp4_launches", 72, lens, 8, 2, 64, 16, "fp4", "bf16")
    k, v, slots = _rows(w, 1.0, 73)
    (kc, vc, kss, vss), (okc, ovc, oks, ovs) = _pools(w, k, v, slots)
    out = pa.decode_scaled(storage_to_torch(w.query(), "bf16").cuda(), kc, vc, kss, vss,
                           torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(), w.scale,
                           out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    ref = O.decode_scaled(w.query(), okc, ovc, oks, ovs, w.block_tables, w.context_lens, w.scale, w.group, "bf16",
                          cache_dtype="fp4")
    ma, rel = errors(out, ref)
    log(f"[fp4, 2100 sequences in two launches] max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert np.isfinite(out).all() and ma <= _bound(w, w.query(), okc, oks, ovc, ovs) and rel <= 1e-3
