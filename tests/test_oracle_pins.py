"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formulas: values printed
on the pages (tests/golden), closed forms, special cases, a library routine
(torch's scaled_dot_product_attention in float64), brute force with scalar
Python arithmetic, and invariants the pages state.  The last group plants
plausible mistakes in a copy of the oracle and checks that some pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import harness as OH
from oracle import pa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- sizing

def test_sizing_matches_printed_figures():
    g = _golden("sizing.json")
    m = g["model"]
    per_tok = O.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["bytes_per_elem"])
    assert per_tok == g["bytes_per_token"] == 327680
    prompt = O.kv_cache_bytes(g["prompt_tokens"], m["layers"], m["kv_heads"], m["head_dim"], m["bytes_per_elem"])
    assert prompt == 1_342_177_280
    assert round(prompt / 1e9, 2) == g["prompt_gb_decimal_2dp"]
    long = O.kv_cache_bytes(g["long_context_tokens"], m["layers"], m["kv_heads"], m["head_dim"], m["bytes_per_elem"])
    assert long / 2**30 == 39.0625
    assert round(long / 2**30, 2) == g["long_context_gib_2dp"]


def test_sizing_per_layer_and_dtype():
    # one layer of the decode configs: 8 KV heads x 128 dims
    assert O.kv_bytes_per_token(1, 8, 128, 2) == 4096
    assert O.kv_bytes_per_token(1, 8, 128, 1) == 2048
    assert O.kv_bytes_per_token(1, 4, 64, 2) == 1024


# ---------------------------------------------------------------- block table

def test_worked_block_table_example():
    g = _golden("block_table_example.json")
    bs = g["tokens_per_block"]
    table = [g["block_table"][str(j)] for j in range(len(g["logical_blocks"]))]
    pos = 0
    for j, toks in enumerate(g["logical_blocks"]):
        for r, name in enumerate(toks):
            assert name == f"t{pos}"
            slot = O.slot_of(table, pos, bs)
            assert slot // bs == g["block_table"][str(j)]
            assert slot % bs == r
            pos += 1
    assert O.slot_of(table, 9, bs) == 42 * 4 + 1 == 169


def test_gather_follows_the_table_of_the_worked_example():
    # a 50-block pool whose row r of block b holds the value 1000*b + r
    pool = np.zeros((50, 1, 4, 1), np.float16)
    for b in range(50):
        for r in range(4):
            pool[b, 0, r, 0] = b * 10 + r
    rows = O.gather_kv(pool, [17, 3, 42], 10)[:, 0, 0].astype(int).tolist()
    assert rows == [170, 171, 172, 173, 30, 31, 32, 33, 420, 421]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
def test_scatter_gather_round_trip_is_bit_exact(dtype):
    rng = np.random.default_rng(7)
    Hkv, D, bs = 3, 16, 8
    lens = [1, 7, 8, 9, 23]
    nblk = sum((L + bs - 1) // bs for L in lens)
    perm = rng.permutation(nblk + 5)
    kc = O.new_pool(nblk + 5, Hkv, bs, D, dtype)
    vc = O.new_pool(nblk + 5, Hkv, bs, D, dtype)
    src = []
    off = 0
    tables = []
    for L in lens:
        n = (L + bs - 1) // bs
        tables.append(perm[off:off + n])
        off += n
        if dtype == "fp8":
            k = rng.integers(0, 256, (L, Hkv, D)).astype(np.uint8)
            k[(k & 0x7F) == 0x7F] = 0  # keep NaN codes out of the source
            v = k[::-1].copy()
        else:
            k = W.to_storage(rng.standard_normal((L, Hkv, D), dtype=np.float32), dtype)
            v = W.to_storage(rng.standard_normal((L, Hkv, D), dtype=np.float32), dtype)
        src.append((k, v))
        slots = O.slots_for(tables[-1], 0, L, bs)
        # an fp8 source is already coded: store as bytes
        kc[slots // bs, :, slots % bs, :] = k
        vc[slots // bs, :, slots % bs, :] = v
    for (k, v), t, L in zip(src, tables, lens):
        assert O.gather_kv(kc, t, L).tobytes() == k.tobytes()
        assert O.gather_kv(vc, t, L).tobytes() == v.tobytes()


def test_reshape_and_cache_skips_negative_slots_and_writes_rows():
    kc = O.new_pool(4, 2, 4, 3, "f16")
    vc = O.new_pool(4, 2, 4, 3, "f16")
    key = np.arange(3 * 2 * 3, dtype=np.float16).reshape(3, 2, 3)
    val = -key
    O.reshape_and_cache(key, val, kc, vc, [5, -1, 12], 4, "f16")
    assert np.array_equal(kc[1, :, 1, :], key[0]) and np.array_equal(vc[1, :, 1, :], val[0])
    assert np.array_equal(kc[3, :, 0, :], key[2])
    assert int(np.isnan(kc).sum()) == kc.size - 2 * 2 * 3


def test_tail_waste_closed_form():
    lens = np.array([1, 15, 16, 17, 2304])
    w = O.tail_waste(lens, 16)
    assert w == (15 + 1 + 0 + 15 + 0) / (16 + 16 + 16 + 32 + 2304)
    # only the last block's tail: each sequence wastes < bs slots
    w2 = W.llama8b()
    assert O.tail_waste(w2.context_lens, 16) < 16 / 512
    assert O.tail_waste(w2.context_lens, 16) < 0.04


# ---------------------------------------------------------------- attention

def _tiny_pools():
    w = W.tiny()
    kc, vc = OH.build_pools(w)
    return w, kc, vc


def test_context_of_one_returns_that_value_row():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out = O.attend(q, k, v, 0.3, 2)
    assert np.array_equal(out, v[0].repeat(2, axis=0))


@pytest.mark.parametrize("zero", ["q", "scale"])
def test_uniform_weights_give_the_mean_of_values(zero):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 16))
    k = rng.standard_normal((37, 3, 16))
    v = rng.standard_normal((37, 3, 16))
    if zero == "q":
        q[:] = 0
        out = O.attend(q, k, v, 0.25, 2)
    else:
        out = O.attend(q, k, v, 0.0, 2)
    mean = v.mean(axis=0).repeat(2, axis=0)
    assert np.max(np.abs(out - mean)) <= 1e-15


def test_empty_context_gives_zeros():
    out = O.attend(np.ones((4, 8)), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 1.0, 2)
    assert np.array_equal(out, np.zeros((4, 8)))


def _sdpa(q, k, v, scale, group):
    """torch float64 scaled_dot_product_attention, KV heads repeated per group."""
    qt = torch.from_numpy(q)[:, None, :]  # [Hq, 1, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)  # [Hq, L, D]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :].numpy()


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_attention_matches_torch_sdpa_float64(group):
    rng = np.random.default_rng(10 + group)
    Hkv, D = 2, 32
    for L in (1, 5, 64, 301):
        q = rng.standard_normal((Hkv * group, D))
        k = rng.standard_normal((L, Hkv, D)) * 2
        v = rng.standard_normal((L, Hkv, D))
        out = O.attend(q, k, v, 1 / math.sqrt(D), group)
        ref = _sdpa(q, k, v, 1 / math.sqrt(D), group)
        assert np.max(np.abs(out - ref)) <= 1e-12


def test_tiny_decode_matches_sdpa_over_explicit_block_walk():
    w, kc, vc = _tiny_pools()
    out = OH.decode(w, kc, vc)
    q = O.widen(w.query(), w.q_dtype)
    for s in range(w.B):
        L = int(w.context_lens[s])
        # explicit walk: one row at a time through the table
        k = np.stack([kc[w.block_tables[s][t // w.bs], :, t % w.bs, :] for t in range(L)]).astype(np.float64)
        v = np.stack([vc[w.block_tables[s][t // w.bs], :, t % w.bs, :] for t in range(L)]).astype(np.float64)
        ref = _sdpa(q[s], k, v, w.scale, w.group)
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def _brute_force(q, k, v, scale, group):
    """Scalar Python: math.exp and math.fsum only."""
    Hq, D = len(q), len(q[0])
    L = len(k)
    out = []
    for i in range(Hq):
        h = i // group
        sc = [scale * math.fsum(q[i][d] * k[t][h][d] for d in range(D)) for t in range(L)]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = math.fsum(e)
        out.append([math.fsum(e[t] * v[t][h][d] for t in range(L)) / z for d in range(D)])
    return out


def test_tiny_decode_matches_brute_force():
    w, kc, vc = _tiny_pools()
    out = OH.decode(w, kc, vc)
    q = O.widen(w.query(), "f16").tolist()
    for s in range(w.B):
        L = int(w.context_lens[s])
        k = [[[float(x) for x in kc[w.block_tables[s][t // 16], h, t % 16, :]] for h in range(4)] for t in range(L)]
        v = [[[float(x) for x in vc[w.block_tables[s][t // 16], h, t % 16, :]] for h in range(4)] for t in range(L)]
        ref = np.array(_brute_force(q[s], k, v, w.scale, w.group))
        assert np.max(np.abs(out[s] - ref)) <= 1e-13


def test_tiny_pool_uses_a_permutation_without_reuse():
    w = W.tiny()
    assert w.num_blocks == 32
    used = np.concatenate([w.block_tables[s, :(int(L) + 15) // 16] for s, L in enumerate(w.context_lens)])
    assert len(used) == 3 + 7 and len(set(used.tolist())) == len(used)
    assert used.min() >= 0 and used.max() < 32


# ---------------------------------------------------------------- invariants the pages state

def test_paged_equals_contiguous_for_any_block_permutation():
    w = W.custom("perm", 11, [1, 16, 17, 50, 129], 8, 2, 32, 16, "bf16")
    kc, vc = OH.build_pools(w)
    paged = OH.decode(w, kc, vc)
    keys = [w.seq_kv(s)[0] for s in range(w.B)]
    vals = [w.seq_kv(s)[1] for s in range(w.B)]
    contig = O.decode_contiguous(w.query(), keys, vals, w.scale, w.group, "bf16", "bf16")
    assert np.array_equal(paged, contig)
    # a different permutation of the same pool: identical result
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.num_blocks)
    inv = np.argsort(perm)
    kc2, vc2 = kc[perm], vc[perm]
    tables2 = np.where(w.block_tables >= 0, inv[np.maximum(w.block_tables, 0)], -1)
    out2 = O.decode(w.query(), kc2, vc2, tables2, w.context_lens, w.scale, w.group, "bf16", "bf16")
    assert np.array_equal(out2, paged)


def _small_shared():
    return W.shared_prefix(seed=99, prompts=2, samples=3, prefix=64, max_tail=40)


def test_shared_prefix_tables_equal_private_copies():
    w = _small_shared()
    kc, vc = OH.build_pools(w)
    shared = OH.decode(w, kc, vc)
    keys = [w.seq_kv(s)[0] for s in range(w.B)]
    vals = [w.seq_kv(s)[1] for s in range(w.B)]
    private = O.decode_contiguous(w.query(), keys, vals, w.scale, w.group, "bf16", "bf16")
    assert np.array_equal(shared, private)
    # the prompt's full prefix blocks really are shared
    s0, s1 = 0, 1
    nfull = 64 // 16
    assert np.array_equal(w.block_tables[s0, :nfull], w.block_tables[s1, :nfull])


def test_copy_on_write_copies_bytes_and_leaves_source():
    w = _small_shared()
    kc, vc = OH.build_pools(w)
    pairs = w.meta["cow_pairs"]
    assert len(pairs) == 2 * 2
    kc2, vc2 = kc.copy(), vc.copy()
    src = int(pairs[0][0])
    before = kc2[src].tobytes()
    # copy again onto a fresh block and check it
    used = set(w.block_tables[w.block_tables >= 0].ravel().tolist())
    fresh = min(set(range(w.num_blocks)) - used)
    O.copy_blocks(kc2, vc2, [[src, fresh]])
    assert kc2[fresh].tobytes() == kc2[src].tobytes() == before
    assert vc2[fresh].tobytes() == vc2[src].tobytes()


def test_cow_isolates_samples_after_divergence():
    w = _small_shared()
    kc, vc = OH.build_pools(w)
    base = OH.decode(w, kc, vc)
    # overwrite the last sample's rows in its (original) partial block: the
    # other samples of that prompt hold copies and must not change
    s_last = w.meta["samples"] - 1
    nb = (int(w.meta["shared_len"][0]) + 15) // 16
    blk = w.block_tables[s_last, nb - 1]
    kc[blk, :, :, :] = np.float16(0).view(np.uint16)  # zero bits
    out = OH.decode(w, kc, vc)
    for s in range(w.meta["samples"] - 1):
        assert np.array_equal(out[s], base[s])
    assert not np.array_equal(out[s_last], base[s_last])


def test_poisoned_slots_are_never_read():
    for name in ("tiny",):
        w = W.make(name)
        kc, vc = OH.build_pools(w, poison=True)
        assert np.isnan(O.widen(kc, w.cache_dtype)).any()  # the poison is there
        out = OH.decode(w, kc, vc)
        assert np.isfinite(out).all()


# ---------------------------------------------------------------- fp8 codec

def test_e4m3_decode_table_against_torch_and_spec_points():
    vals = O.e4m3_values()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(vals), np.isnan(ref))
    ok = ~np.isnan(vals)
    assert np.array_equal(vals[ok], ref[ok])
    assert vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert vals[0x80] == 0.0 and math.copysign(1, vals[0x80]) == -1
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])


def _torch_encode(x_f32, scale):
    with np.errstate(over="ignore", invalid="ignore"):
        y = torch.from_numpy(np.asarray(x_f32, np.float32) / np.float32(scale))
    y = torch.where(torch.isnan(y), y, y.clamp(-448.0, 448.0))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 4.75 / 448.0, 2.0 ** -4])
def test_e4m3_encode_exhaustive_against_torch(src, scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32) if src == "f16" else W.storage_to_f32(bits, "bf16")
    ours = O.e4m3_encode(x, scale)
    ref = _torch_encode(x, scale)
    nan = np.isnan(x)
    # NaN: sign kept, NaN code
    assert np.array_equal(ours[nan] & 0x7F, np.full(nan.sum(), 0x7F, np.uint8))
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_encode_ties_and_saturation():
    enc = lambda v: int(O.e4m3_encode(np.array([v], np.float32), 1.0)[0])
    assert enc(448.0) == 0x7E and enc(464.0) == 0x7E and enc(1e30) == 0x7E and enc(np.inf) == 0x7E
    assert enc(-np.inf) == 0xFE
    assert enc(2.0 ** -10) == 0x00  # half of the smallest subnormal: tie to even (0)
    assert enc(3 * 2.0 ** -10) == 0x02  # 1.5 x smallest: tie to even code 2
    assert enc(1.0625) == 0x38  # halfway between 1 (0x38) and 1.125 (0x39): even
    assert enc(1.1875) == 0x3A  # halfway between 1.125 and 1.25: even (0x3A)
    assert enc(-0.0) == 0x80 and enc(-1e-9) == 0x80


def test_round_to_bf16_matches_torch():
    x = np.random.default_rng(3).standard_normal(10000) * 10.0 ** np.random.default_rng(4).integers(-30, 30, 10000)
    ours = O.round_to(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- widening of 16-bit storage

def _binary_format_value(bits, exp_bits, frac_bits):
    """Value of every bit pattern of an IEEE-style binary format, from its
    definition: (-1)^s 2^(e - bias) (1 + f / 2^frac_bits) for normal
    exponents, (-1)^s 2^(1 - bias) f / 2^frac_bits for e = 0, infinity or NaN
    for the all-ones exponent (Python integers and ldexp, no float casts)."""
    bias = (1 << (exp_bits - 1)) - 1
    out = []
    for b in bits.tolist():
        s = -1.0 if b >> (exp_bits + frac_bits) else 1.0
        e = (b >> frac_bits) & ((1 << exp_bits) - 1)
        f = b & ((1 << frac_bits) - 1)
        if e == (1 << exp_bits) - 1:
            out.append(s * math.inf if f == 0 else math.nan)
        elif e == 0:
            out.append(s * math.ldexp(f, 1 - bias - frac_bits))
        else:
            out.append(s * math.ldexp((1 << frac_bits) + f, e - bias - frac_bits))
    return np.array(out, np.float64)


def _same_values(a, b):
    """Equal as float64, NaN positions equal, and zeros of the same sign."""
    nan = np.isnan(a)
    if not np.array_equal(nan, np.isnan(b)):
        return False
    a, b = a[~nan], b[~nan]
    return np.array_equal(a, b) and np.array_equal(np.signbit(a), np.signbit(b))


ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_widen_bf16_every_bit_pattern():
    """bf16 -> fp64 over all 65,536 patterns against the format's definition
    (8 exponent bits, bias 127, 7 fraction bits) and against torch's
    bfloat16 -> float64 conversion."""
    ours = O.widen(ALL16, "bf16")
    assert _same_values(ours, _binary_format_value(ALL16, 8, 7))
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same_values(ours, ref)


def test_widen_f16_every_bit_pattern():
    """f16 -> fp64 over all 65,536 patterns against IEEE binary16 (5 exponent
    bits, bias 15, 10 fraction bits) and against torch's conversion."""
    ours = O.widen(ALL16.view(np.float16), "f16")
    assert _same_values(ours, _binary_format_value(ALL16, 5, 10))
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    assert _same_values(ours, ref)


@pytest.mark.parametrize("mistake", ["shift15", "as_f16", "byteswap", "low_half"])
def test_widen_pins_catch_planted_mistakes(mistake):
    bits = ALL16.astype(np.uint32)
    if mistake == "shift15":
        bad = (bits << 15).view(np.float32).astype(np.float64)
    elif mistake == "as_f16":
        bad = ALL16.view(np.float16).astype(np.float64)
    elif mistake == "byteswap":
        bad = (ALL16.byteswap().astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:  # the pattern in the low half of the binary32
        bad = bits.view(np.float32).astype(np.float64)
    assert not _same_values(bad, _binary_format_value(ALL16, 8, 7))


# ---------------------------------------------------------------- planted mistakes

def _pins_pass(attend):
    """Run the attention pins against an alternative attend(); True if all hold."""
    rng = np.random.default_rng(123)
    try:
        for group in (1, 4):
            q = rng.standard_normal((2 * group, 16))
            k = rng.standard_normal((21, 2, 16))
            v = rng.standard_normal((21, 2, 16))
            if np.max(np.abs(attend(q, k, v, 0.25, group) - _sdpa(q, k, v, 0.25, group))) > 1e-12:
                return False
            if not np.array_equal(attend(q, k[:1], v[:1], 0.25, group), v[0].repeat(group, axis=0)):
                return False
    except Exception:
        return False
    return True


def test_pins_accept_the_oracle():
    assert _pins_pass(O.attend)


@pytest.mark.parametrize("mistake", ["no_scale", "gqa_modulo", "no_normalize", "k_for_v", "sum_over_heads"])
def test_pins_catch_planted_mistakes(mistake):
    def bad(q, k, v, scale, group):
        Hq, D = q.shape
        L, Hkv, _ = k.shape
        out = np.zeros((Hq, D))
        for i in range(Hq):
            h = i // group
            if mistake == "gqa_modulo":
                h = i % Hkv
            kk = k[:, h, :]
            vv = (k if mistake == "k_for_v" else v)[:, h, :]
            sc = (1.0 if mistake == "no_scale" else scale) * kk @ q[i]
            sc = sc + sc.max() if mistake == "no_normalize" else sc - sc.max()
            e = np.exp(sc)
            if mistake == "sum_over_heads":
                e = np.exp(scale * k.sum(axis=1) @ q[i] - (scale * k.sum(axis=1) @ q[i]).max())
            out[i] = (e if mistake == "no_normalize" else e / e.sum()) @ vv
        return out

    assert not _pins_pass(bad)


# ---------------------------------------------------------------- several queries per sequence

def _causal_sdpa(q, k, v, scale, group):
    """torch float64 scaled_dot_product_attention with its own causal mask
    (is_causal: query row i sees key rows 0..i) over L queries and L keys."""
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, L, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=True).permute(1, 0, 2).numpy()


def _multi_case(seed, lens, nqs, group=4, Hkv=2, D=32, bs=8):
    """Pools holding each sequence's rows, plus one query row per position of
    every sequence (so the causal routine sees the whole sequence); the
    multi-query call takes the query rows of each sequence's last n positions."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    nb = int(sum((L + bs - 1) // bs for L in lens)) + 3
    perm = rng.permutation(nb)
    M = max((L + bs - 1) // bs for L in lens)
    tables = np.full((B, M), -1, np.int64)
    kc = O.new_pool(nb, Hkv, bs, D, "f16")
    vc = O.new_pool(nb, Hkv, bs, D, "f16")
    full_q, ks, vs, off = [], [], [], 0
    for s, L in enumerate(lens):
        n = (L + bs - 1) // bs
        tables[s, :n] = perm[off:off + n]
        off += n
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        O.reshape_and_cache(k, v, kc, vc, O.slots_for(tables[s], 0, L, bs), bs, "f16")
        full_q.append(rng.standard_normal((L, Hkv * group, D)).astype(np.float16))
        ks.append(k)
        vs.append(v)
    qs = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int64)
    q = np.concatenate([full_q[s][lens[s] - nqs[s]:] for s in range(B)])
    return tables, kc, vc, np.array(lens), qs, q, full_q, ks, vs


@pytest.mark.parametrize("group", [1, 4])
def test_multi_query_matches_torch_causal_attention(group):
    """The last n query rows of a sequence equal the last n rows of torch's
    causal attention over the whole sequence, for n = L (a whole prefill) and
    n < L (a chunk, or draft tokens)."""
    lens, nqs = [1, 9, 40, 75], [1, 9, 17, 3]
    tables, kc, vc, L, qs, q, full_q, ks, vs = _multi_case(5 + group, lens, nqs, group=group)
    scale = 0.2
    out = O.decode_multi(q, kc, vc, tables, L, qs, scale, group, "f16", "f16")
    for s in range(len(lens)):
        ref = _causal_sdpa(full_q[s].astype(np.float64), ks[s].astype(np.float64), vs[s].astype(np.float64),
                           scale, group)[lens[s] - nqs[s]:]
        assert np.max(np.abs(out[qs[s]:qs[s + 1]] - ref)) <= 1e-12


def test_multi_query_with_one_query_is_decode():
    lens, nqs = [5, 33, 64], [1, 1, 1]
    tables, kc, vc, L, qs, q, *_ = _multi_case(9, lens, nqs)
    out = O.decode_multi(q, kc, vc, tables, L, qs, 0.3, 4, "f16", "f16")
    ref = O.decode(q, kc, vc, tables, L, 0.3, 4, "f16", "f16")
    assert np.array_equal(out, ref)


def test_multi_query_matches_brute_force():
    """Scalar Python over the positions each query may see."""
    lens, nqs = [6, 11], [3, 11]
    tables, kc, vc, L, qs, q, full_q, ks, vs = _multi_case(13, lens, nqs, group=2, D=8)
    out = O.decode_multi(q, kc, vc, tables, L, qs, 0.5, 2, "f16", "f16")
    for s in range(len(lens)):
        for j in range(nqs[s]):
            seen = lens[s] - nqs[s] + j + 1
            k = [[[float(x) for x in ks[s][t, h]] for h in range(2)] for t in range(seen)]
            v = [[[float(x) for x in vs[s][t, h]] for h in range(2)] for t in range(seen)]
            ref = np.array(_brute_force([[float(x) for x in row] for row in q[qs[s] + j]], k, v, 0.5, 2))
            assert np.max(np.abs(out[qs[s] + j] - ref)) <= 1e-13


@pytest.mark.parametrize("mistake", ["mask_off_by_one", "mask_from_chunk_start", "row_by_sequence"])
def test_multi_query_pins_catch_planted_mistakes(mistake):
    def bad(q, kc, vc, tables, L, qs, scale, group, cd, qd):
        out = np.zeros(q.shape)
        for s in range(len(L)):
            a, b = int(qs[s]), int(qs[s + 1])
            n = b - a
            k = O.widen(O.gather_kv(kc, tables[s], int(L[s])), cd)
            v = O.widen(O.gather_kv(vc, tables[s], int(L[s])), cd)
            for j in range(n):
                seen = {"mask_off_by_one": L[s] - n + j, "mask_from_chunk_start": j + 1}.get(mistake, L[s] - n + j + 1)
                row = s + j if mistake == "row_by_sequence" else a + j
                out[a + j] = O.attend(O.widen(q[row], qd), k[:max(int(seen), 1)], v[:max(int(seen), 1)], scale, group)
        return out

    lens, nqs = [1, 9, 40, 75], [1, 9, 17, 3]
    tables, kc, vc, L, qs, q, full_q, ks, vs = _multi_case(5, lens, nqs)
    got = bad(q, kc, vc, tables, L, qs, 0.2, 4, "f16", "f16")
    ok = all(np.max(np.abs(got[qs[s]:qs[s + 1]] - _causal_sdpa(full_q[s].astype(np.float64), ks[s].astype(np.float64),
                                                                 vs[s].astype(np.float64), 0.2, 4)[lens[s] - nqs[s]:]))
             <= 1e-12 for s in range(len(lens)))
    assert not ok


# ---------------------------------------------------------------- FP8 with a scale per row

def _rows_of_many_magnitudes(seed, n=64, D=128):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-4, 4, size=(n, 1))
    return (rng.standard_normal((n, D)) * mag).astype(np.float32)


def test_row_scale_puts_each_rows_largest_magnitude_on_448():
    x = _rows_of_many_magnitudes(1)
    s = O.row_scale(x)
    codes = O.e4m3_encode(x, s[:, None])
    big = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(len(x)), big]
    assert set(np.unique(top & 0x7F).tolist()) == {0x7E}  # +-448, the largest finite code
    assert np.array_equal(top >> 7, (x[np.arange(len(x)), big] < 0).astype(np.uint8))


def test_row_scale_error_bounds():
    """Normal-range codes carry 3 mantissa bits: a relative error of at most
    2^-4 after the division by the scale (plus fp32 rounding); below 2^-6 the
    spacing is 2^-9, so the error is at most half of it, times the scale."""
    x = _rows_of_many_magnitudes(2)
    s = O.row_scale(x)
    back = O.widen_rows(O.e4m3_encode(x, s[:, None]), s)
    y = np.abs(x.astype(np.float64)) / s[:, None]
    err = np.abs(back - x)
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(x[normal]) * (2.0 ** -4) * (1 + 1e-6))
    assert np.all(err[~normal] <= (s[:, None] * np.ones_like(x))[~normal] * 2.0 ** -10 * (1 + 1e-6))


def test_row_scale_special_rows():
    rows = np.zeros((4, 8), np.float32)
    rows[1, 3] = np.inf
    rows[2, :] = [np.nan, 1.0, -3.0, 2.0, 0.0, 0.5, np.nan, 1.5]
    rows[3, 0] = -7.0
    s = O.row_scale(rows)
    assert s[0] == 1 and s[1] == 1  # zeros; an infinity
    assert s[2] == np.float32(3.0) / np.float32(448.0)  # NaN elements do not count
    assert s[3] == np.float32(7.0) / np.float32(448.0)
    codes = O.e4m3_encode(rows, s[:, None])
    assert (codes[0] == 0).all() and codes[1, 3] == 0x7E and codes[3, 0] == 0xFE
    assert codes[2, 0] == 0x7F and codes[2, 2] == 0xFE


def test_row_scales_keep_small_rows_that_one_tensor_scale_flushes():
    """Rows whose magnitudes span eight decades (more than the ~1e5 E4M3FN
    covers): one scale per tensor sends the small rows into the subnormal
    range or to zero, a scale per row keeps them."""
    x = _rows_of_many_magnitudes(3)
    t = np.float32(np.abs(x).max()) / np.float32(448.0)
    per_tensor = O.e4m3_decode(O.e4m3_encode(x, t), t)
    s = O.row_scale(x)
    per_row = O.widen_rows(O.e4m3_encode(x, s[:, None]), s)
    rel = lambda a: np.abs(a - x) / np.maximum(np.abs(x), 1e-30)
    assert (rel(per_row) > 0.5).mean() < 0.05 and (rel(per_tensor) > 0.5).mean() > 0.2


def test_scaled_decode_matches_attention_over_dequantised_rows():
    """Through the pool and the tables, against torch float64 attention over
    rows dequantised element by element from the code table."""
    rng = np.random.default_rng(4)
    Hkv, G, D, bs, L = 2, 4, 32, 8, 37
    k = (rng.standard_normal((L, Hkv, D)) * 10.0 ** rng.uniform(-2, 2, size=(L, Hkv, 1))).astype(np.float16)
    v = (rng.standard_normal((L, Hkv, D)) * 10.0 ** rng.uniform(-2, 2, size=(L, Hkv, 1))).astype(np.float16)
    nb = 8
    table = rng.permutation(nb)[:(L + bs - 1) // bs]
    kc = O.new_pool(nb, Hkv, bs, D, "fp8")
    vc = O.new_pool(nb, Hkv, bs, D, "fp8")
    ks = np.full((nb, Hkv, bs), np.nan, np.float32)
    vs = np.full((nb, Hkv, bs), np.nan, np.float32)
    O.reshape_and_cache_scaled(k, v, kc, vc, ks, vs, O.slots_for(table, 0, L, bs), bs, "f16")
    q = rng.standard_normal((1, Hkv * G, D)).astype(np.float16)
    out = O.decode_scaled(q, kc, vc, ks, vs, table[None], np.array([L]), 0.2, G, "f16")[0]
    table_vals = O.e4m3_values()
    kd = np.zeros((L, Hkv, D))
    vd = np.zeros((L, Hkv, D))
    for t in range(L):
        b, o = table[t // bs], t % bs
        for h in range(Hkv):
            kd[t, h] = [table_vals[c] * float(ks[b, h, o]) for c in kc[b, h, o]]
            vd[t, h] = [table_vals[c] * float(vs[b, h, o]) for c in vc[b, h, o]]
    ref = _sdpa(q[0].astype(np.float64), kd, vd, 0.2, G)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("mistake", ["fnuz_max", "signed_max"])
def test_row_scale_pins_catch_planted_mistakes(mistake):
    def bad_scale(rows):
        x = np.asarray(rows, np.float32)
        amax = (x.max(axis=-1) if mistake == "signed_max" else np.abs(x).max(axis=-1))
        div = np.float32(240.0) if mistake == "fnuz_max" else np.float32(448.0)
        return np.where(amax > 0, amax / div, np.float32(1)).astype(np.float32)

    x = _rows_of_many_magnitudes(1)
    s = bad_scale(x)
    codes = O.e4m3_encode(x, s[:, None])
    big = np.argmax(np.abs(x), axis=1)
    top_ok = set(np.unique(codes[np.arange(len(x)), big] & 0x7F).tolist()) == {0x7E}
    back = O.widen_rows(codes, s)
    bound_ok = np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 * (1 + 1e-6) + s[:, None] * 2.0 ** -10)
    assert not (top_ok and bound_ok)


# ---------------------------------------------------------------- FP4 E2M1 with a scale per row

# The eight magnitudes of the E2M1 element type as the OCP Microscaling
# formats spec lists them, by code 0b0000 .. 0b0111 (the sign is bit 3).
_E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_against_spec_values():
    vals = O.e2m1_values()
    assert vals[:8].tolist() == _E2M1_SPEC
    assert vals[8:].tolist() == [-v for v in _E2M1_SPEC]
    assert math.copysign(1.0, vals[8]) == -1.0  # 0b1000 is -0


def _e2m1_brute(y):
    """Nearest signed E2M1 value to each fp32 y by scanning all 16 codes; among
    equally near codes the one with mantissa bit 0; NaN -> 0."""
    out = []
    for v in np.asarray(y, np.float64).ravel():
        if math.isnan(v):
            out.append(0)
            continue
        best = None
        for c in range(16):
            cv = _E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0)
            if (c & 8) != (8 if math.copysign(1.0, v) < 0 else 0):
                continue  # the sign is kept, so only codes of v's sign compete
            d = abs(min(abs(v), 6.0) - abs(cv))
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        out.append(best[1])
    return np.array(out, np.uint8).reshape(np.shape(y))


def test_e2m1_encode_against_brute_force():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(4000) * 3, np.arange(-28, 29) * 0.25,  # every tie
                        [1e30, -1e30, 6.0000005, 5.9999995, 0.0, -0.0, 1e-30, np.inf, -np.inf]]).astype(np.float32)
    for scale in (1.0, 0.37, 2.0 ** -9, 1e4):
        ours = O.e2m1_encode(x, scale)
        with np.errstate(over="ignore"):
            ref = _e2m1_brute(x.astype(np.float32) / np.float32(scale))
        assert np.array_equal(ours, ref), scale


def test_e2m1_encode_ties_saturation_and_specials():
    enc = lambda v: int(O.e2m1_encode(np.array([v], np.float32), 1.0)[0])
    # ties go to the code whose mantissa bit is 0
    assert [enc(v) for v in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0, 2, 2, 4, 4, 6, 6]
    assert [enc(v) for v in (0.2500001, 0.7499999, 5.0000005)] == [1, 1, 7]
    assert enc(7.0) == 7 and enc(-1e30) == 0xF and enc(np.inf) == 7
    assert enc(-0.3) == 0x9 and enc(-0.0) == 0x8 and enc(np.nan) == 0


def test_e2m1_packing():
    assert O.e2m1_pack(np.array([1, 2], np.uint8)).tolist() == [0x21]
    assert O.e2m1_pack(np.array([0xF, 0x0, 0x7, 0x8], np.uint8)).tolist() == [0x0F, 0x87]
    rng = np.random.default_rng(22)
    c = rng.integers(0, 16, size=(5, 3, 64)).astype(np.uint8)
    p = O.e2m1_pack(c)
    assert p.shape == (5, 3, 32) and np.array_equal(O.e2m1_unpack(p), c)


def test_fp4_row_scale_puts_each_rows_largest_magnitude_on_6_and_bounds_the_error():
    x = _rows_of_many_magnitudes(23)
    s = O.row_scale(x, 6.0)
    codes = O.e2m1_encode(x, s[:, None])
    big = np.argmax(np.abs(x), axis=1)
    assert set(np.unique(codes[np.arange(len(x)), big] & 7).tolist()) == {7}
    back = O.widen_rows(O.e2m1_pack(codes), s, "fp4")
    y = np.abs(x) / s[:, None]
    # half the gap between neighbouring magnitudes: 0.25 up to 2, 0.5 up to 4, 1 up to 6
    half_gap = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, 1.0)) * s[:, None]
    assert np.all(np.abs(back - x) <= half_gap * (1 + 1e-6))
    assert np.array_equal(O.row_scale(np.array([[0.0, -3.0, np.nan]], np.float32), 6.0), [np.float32(0.5)])


def test_fp4_scaled_decode_matches_attention_over_dequantised_rows():
    """Through the pool and the tables, against torch float64 attention over
    rows dequantised nibble by nibble with the spec's values."""
    rng = np.random.default_rng(24)
    Hkv, G, D, bs, L = 2, 4, 32, 8, 37
    k = (rng.standard_normal((L, Hkv, D)) * 10.0 ** rng.uniform(-2, 2, size=(L, Hkv, 1))).astype(np.float16)
    v = (rng.standard_normal((L, Hkv, D)) * 10.0 ** rng.uniform(-2, 2, size=(L, Hkv, 1))).astype(np.float16)
    nb = 8
    table = rng.permutation(nb)[:(L + bs - 1) // bs]
    kc = O.new_pool(nb, Hkv, bs, D, "fp4")
    vc = O.new_pool(nb, Hkv, bs, D, "fp4")
    assert kc.shape == (nb, Hkv, bs, D // 2)
    ks = np.full((nb, Hkv, bs), np.nan, np.float32)
    vs = np.full((nb, Hkv, bs), np.nan, np.float32)
    O.reshape_and_cache_scaled(k, v, kc, vc, ks, vs, O.slots_for(table, 0, L, bs), bs, "f16", "fp4")
    q = rng.standard_normal((1, Hkv * G, D)).astype(np.float16)
    out = O.decode_scaled(q, kc, vc, ks, vs, table[None], np.array([L]), 0.2, G, "f16", cache_dtype="fp4")[0]

    def nibble_value(byte, hi):
        c = (int(byte) >> 4) & 0xF if hi else int(byte) & 0xF
        return _E2M1_SPEC[c & 7] * (-1.0 if c & 8 else 1.0)

    kd = np.zeros((L, Hkv, D))
    vd = np.zeros((L, Hkv, D))
    for t in range(L):
        b, o = table[t // bs], t % bs
        for h in range(Hkv):
            kd[t, h] = [nibble_value(kc[b, h, o, d // 2], d % 2) * float(ks[b, h, o]) for d in range(D)]
            vd[t, h] = [nibble_value(vc[b, h, o, d // 2], d % 2) * float(vs[b, h, o]) for d in range(D)]
    ref = _sdpa(q[0].astype(np.float64), kd, vd, 0.2, G)
    assert np.max(np.abs(out - ref)) <= 1e-12
    # and the dequantised rows are the source rows within the codec's bound
    assert np.all(np.abs(kd - k.astype(np.float64)) <= np.abs(k).max(axis=-1, keepdims=True) / 6 * (1 + 1e-6))


@pytest.mark.parametrize("mistake", ["tie_to_odd", "swapped_nibbles", "sign_dropped", "e4m3_max"])
def test_fp4_pins_catch_planted_mistakes(mistake):
    """Each plausible slip in an E2M1 encoder fails the brute-force pin or the
    bound pin above."""
    def bad_encode(x, scale):
        y = np.asarray(x, np.float32) / np.asarray(scale, np.float32)
        a = np.minimum(np.abs(y).astype(np.float64), 6.0)
        d = np.abs(a[..., None] - np.array(_E2M1_SPEC))
        if mistake == "tie_to_odd":
            d = d - 1e-12 * (np.arange(8) % 2)
        else:
            d = d + 1e-12 * (np.arange(8) % 2)
        code = np.argmin(d, axis=-1).astype(np.uint8)
        if mistake != "sign_dropped":
            code |= np.where(np.signbit(y), np.uint8(8), np.uint8(0))
        return code

    def bad_pack(c):
        p = O.e2m1_pack(c)
        return ((p >> 4) | (p << 4)) & 0xFF if mistake == "swapped_nibbles" else p

    x = np.concatenate([np.arange(-24, 25) * 0.25, np.random.default_rng(25).standard_normal(199)]).astype(np.float32)
    s = np.float32(np.abs(x).max()) / np.float32(448.0 if mistake == "e4m3_max" else 6.0)
    codes = bad_encode(x, s)
    brute_ok = np.array_equal(codes, _e2m1_brute(x / s))
    back = O.widen_rows(bad_pack(codes), s, "fp4")
    y = np.abs(x) / s
    half_gap = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, 1.0)) * s
    bound_ok = np.all(np.abs(back - x) <= half_gap * (1 + 1e-6))
    top_ok = codes[np.argmax(np.abs(x))] & 7 == 7
    assert not (brute_ok and bound_ok and top_ok)


# ---------------------------------------------------------------- attention sinks + sliding window

def test_window_positions_closed_forms():
    """Sink 4 and window 10 over 30 positions keep 0..3 and 20..29; a window
    (or sink) that covers the sequence keeps everything; window 1 keeps the
    newest position alone; overlapping ranges count each position once."""
    assert O.window_positions(30, 4, 10).tolist() == [0, 1, 2, 3] + list(range(20, 30))
    assert O.window_positions(30, 0, 30).tolist() == list(range(30))
    assert O.window_positions(30, 31, 1).tolist() == list(range(30))
    assert O.window_positions(30, 0, 1).tolist() == [29]
    assert O.window_positions(30, 12, 25).tolist() == list(range(30))
    for L in range(0, 40):
        for sink in (0, 1, 4, 17):
            for window in (1, 3, 16, 33):
                brute = sorted({t for t in range(L) if t < sink} | {t for t in range(L) if t >= L - window})
                assert O.window_positions(L, sink, window).tolist() == brute


def _window_case(seed, lens, group=2, Hkv=2, D=16, bs=4):
    """A permuted pool holding each sequence's rows (f16), tables and a query."""
    rng = np.random.default_rng(seed)
    nb = int(sum((L + bs - 1) // bs for L in lens)) + 2
    perm = rng.permutation(nb)
    M = max((L + bs - 1) // bs for L in lens)
    tables = np.full((len(lens), M), -1, np.int64)
    kc = O.new_pool(nb, Hkv, bs, D, "f16")
    vc = O.new_pool(nb, Hkv, bs, D, "f16")
    off = 0
    for s, L in enumerate(lens):
        n = (L + bs - 1) // bs
        tables[s, :n] = perm[off:off + n]
        off += n
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        O.reshape_and_cache(k, v, kc, vc, O.slots_for(tables[s], 0, L, bs), bs, "f16")
    q = rng.standard_normal((len(lens), Hkv * group, D)).astype(np.float16)
    return kc, vc, tables, np.array(lens), q


def test_window_decode_covering_everything_is_decode():
    kc, vc, tables, lens, q = _window_case(11, [1, 9, 30, 57])
    full = O.decode(q, kc, vc, tables, lens, 0.25, 2, "f16", "f16")
    for sink, window in ((0, 57), (57, 1), (3, 1000)):
        assert np.array_equal(O.decode_window(q, kc, vc, tables, lens, 0.25, 2, sink, window, "f16", "f16"), full)


def test_window_of_one_without_sink_is_the_newest_value_row():
    kc, vc, tables, lens, q = _window_case(12, [1, 9, 30, 57])
    out = O.decode_window(q, kc, vc, tables, lens, 0.25, 2, 0, 1, "f16", "f16")
    for s, L in enumerate(lens):
        v_last = O.widen(O.gather_kv(vc, tables[s], int(L)), "f16")[L - 1]  # [Hkv, D]
        assert np.array_equal(out[s], np.repeat(v_last, 2, axis=0))


def _masked_sdpa(q, k, v, keep, scale, group):
    """torch float64 scaled_dot_product_attention over the whole sequence with
    a boolean mask that admits only the kept positions."""
    L = k.shape[0]
    mask = torch.zeros((1, L), dtype=torch.bool)
    mask[0, torch.from_numpy(keep)] = True
    qt = torch.from_numpy(q)[:, None, :]  # [Hq, 1, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)[:, 0].numpy()


@pytest.mark.parametrize("sink,window", [(4, 10), (0, 7), (1, 1), (9, 3), (20, 20)])
def test_window_decode_matches_masked_torch_attention(sink, window):
    kc, vc, tables, lens, q = _window_case(13, [5, 23, 41, 64])
    out = O.decode_window(q, kc, vc, tables, lens, 0.25, 2, sink, window, "f16", "f16")
    for s, L in enumerate(lens):
        k = O.widen(O.gather_kv(kc, tables[s], int(L)), "f16")
        v = O.widen(O.gather_kv(vc, tables[s], int(L)), "f16")
        ref = _masked_sdpa(O.widen(q[s], "f16"), k, v, O.window_positions(int(L), sink, window), 0.25, 2)
        assert np.max(np.abs(out[s] - ref)) <= 1e-12


def test_window_decode_matches_brute_force():
    kc, vc, tables, lens, q = _window_case(14, [6, 19])
    out = O.decode_window(q, kc, vc, tables, lens, 0.25, 2, 2, 5, "f16", "f16")
    for s, L in enumerate(lens):
        keep = [t for t in range(int(L)) if t < 2 or t >= L - 5]
        for i in range(q.shape[1]):
            h = i // 2
            qi = [float(x) for x in q[s, i]]
            rows = [(int(tables[s][t // 4]), t % 4) for t in keep]
            sc = [0.25 * math.fsum(qi[d] * float(kc[b, h, r, d]) for d in range(16)) for b, r in rows]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            den = math.fsum(e)
            for d in range(16):
                want = math.fsum(e[u] * float(vc[b, h, r, d]) for u, (b, r) in enumerate(rows)) / den
                assert abs(out[s, i, d] - want) <= 1e-13


def test_window_decode_after_block_eviction_is_unchanged():
    """Whole-block eviction of what neither the sink nor the window holds,
    then the windowed decode over the shortened table, attends to the same
    rows in the same order as the windowed decode over the full table: the
    kept blocks keep the first positions, and the last positions stay last."""
    from oracle.block_manager import BlockManager

    rng = np.random.default_rng(15)
    bs, Hkv, D, group = 4, 2, 16, 2
    for L, sink, window in ((30, 4, 10), (57, 3, 9), (64, 0, 5), (13, 5, 20), (40, 9, 1)):
        bm = BlockManager(40, bs)
        bm.add(0)
        slots, _ = bm.append(0, L)
        kc, vc = O.new_pool(40, Hkv, bs, D, "f16"), O.new_pool(40, Hkv, bs, D, "f16")
        k = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((L, Hkv, D)).astype(np.float16)
        O.reshape_and_cache(k, v, kc, vc, np.array(slots), bs, "f16")
        q = rng.standard_normal((1, Hkv * group, D)).astype(np.float16)
        before = O.decode_window(q, kc, vc, np.array([bm.table(0)]), [L], 0.25, group, sink, window, "f16", "f16")
        bm.evict(0, sink, window)
        after = O.decode_window(q, kc, vc, np.array([bm.table(0)]), [bm.length(0)], 0.25, group, sink, window,
                                "f16", "f16")
        assert np.array_equal(before, after)


@pytest.mark.parametrize("mistake", ["window_one_short", "sink_inclusive", "window_after_sink"])
def test_window_pins_catch_planted_mistakes(mistake, monkeypatch):
    def bad(L, sink, window):
        t = np.arange(L)
        if mistake == "window_one_short":
            return t[(t < sink) | (t > L - window)]
        if mistake == "sink_inclusive":
            return t[(t <= sink) | (t >= L - window)]
        return t[t < sink + window]  # the window read as the positions right after the sink

    monkeypatch.setattr(O, "window_positions", bad)
    with pytest.raises(AssertionError):
        test_window_positions_closed_forms()
