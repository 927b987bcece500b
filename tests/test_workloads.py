"""The seeded input generators: determinism and the shapes of the workloads."""
import numpy as np

import workloads as W


def test_generators_are_deterministic():
    a, b = W.llama8b(B=4), W.llama8b(B=4)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    ka, va = a.seq_kv(2)
    kb, vb = b.seq_kv(2)
    assert ka.tobytes() == kb.tobytes() and va.tobytes() == vb.tobytes()
    assert a.query().tobytes() == b.query().tobytes()
    c = W.llama8b(seed=1, B=4)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_config_shapes():
    t = W.tiny()
    assert (t.B, t.Hq, t.Hkv, t.D, t.bs, t.cache_dtype) == (2, 4, 4, 64, 16, "f16")
    assert t.context_lens.tolist() == [37, 100] and t.scale == 0.125
    l8 = W.llama8b()
    assert (l8.B, l8.Hq, l8.Hkv, l8.D, l8.bs, l8.cache_dtype) == (64, 32, 8, 128, 16, "bf16")
    assert l8.context_lens.min() >= 512 and l8.context_lens.max() <= 4096
    nblk = int(((l8.context_lens + 15) // 16).sum())
    assert l8.num_blocks == int(np.ceil(1.1 * nblk))
    l70 = W.llama70b()
    assert (l70.B, l70.Hq, l70.Hkv, l70.num_blocks) == (32, 64, 8, 16000)
    assert (l70.context_lens == 8000).all() and l70.block_tables.shape == (32, 500)
    used = l70.block_tables.ravel()
    assert len(np.unique(used)) == 16000
    sp = W.shared_prefix()
    assert sp.B == 128 and len(sp.meta["cow_pairs"]) == 16 * 7
    assert ((sp.meta["shared_len"] - 2048 >= 1) & (sp.meta["shared_len"] - 2048 <= 15)).all()


def test_heavy_tail_lengths():
    lens = W.heavy_tail_lengths(3425, 256)
    assert lens.min() >= 1 and lens.max() <= 32768
    assert 150 < np.median(lens) < 600


def test_shared_prefix_tables_share_prompt_blocks():
    sp = W.shared_prefix(seed=5, prompts=2, samples=4, prefix=64, max_tail=30)
    nb = (sp.meta["shared_len"] + 15) // 16
    for k in range(2):
        rows = sp.block_tables[k * 4:(k + 1) * 4]
        full = int(nb[k]) - 1
        assert (rows[:, :full] == rows[0, :full]).all()
        last = rows[:, full]
        assert len(set(last.tolist())) == 4  # three copies + the original
    src = sp.meta["cow_pairs"][:, 0]
    assert set(src.tolist()) <= set(sp.block_tables.ravel().tolist())
