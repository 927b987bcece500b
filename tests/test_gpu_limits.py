"""Sizes at the limits: a pool larger than 2 GiB with the sequences' blocks
at its top (every row offset beyond 2^31 bytes), and the largest batch one
call takes (65,535 sequences, sixteen launches)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_342_amd as pa
import workloads as W
from oracle import pa_oracle as O
from tests.gpu_util import errors, log, storage_to_torch

pytestmark = pytest.mark.gpu


def test_pool_beyond_two_gib_uses_64_bit_offsets():
    Hkv, G, D, bs, dt = 8, 4, 128, 16, "bf16"
    num_blocks = 70_000  # 70,000 x 8 x 16 x 128 x 2 B = 2.29 GB per pool
    lens = [1, 17, 500, 1234, 4000]
    rng = np.random.default_rng(91)
    nblk = [(L + bs - 1) // bs for L in lens]
    top = rng.permutation(np.arange(num_blocks - 600, num_blocks))  # ids above 2^31 / (Hkv*bs*D*2) = 65,536
    tables = np.full((len(lens), max(nblk)), -1, np.int32)
    off = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = top[off:off + n]
        off += n
    assert (tables[tables >= 0].astype(np.int64) * Hkv * bs * D * 2 >= 2 ** 31).all()
    kc = torch.full((num_blocks, Hkv, bs, D), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = torch.full((num_blocks, Hkv, bs, D), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    keys, vals = [], []
    for s, L in enumerate(lens):
        k = W.to_storage(rng.standard_normal((L, Hkv, D), dtype=np.float32), dt)
        v = W.to_storage(rng.standard_normal((L, Hkv, D), dtype=np.float32), dt)
        keys.append(k)
        vals.append(v)
        slots = torch.from_numpy(O.slots_for(tables[s], 0, L, bs)).cuda()
        pa.reshape_and_cache(storage_to_torch(k, dt).cuda(), storage_to_torch(v, dt).cuda(), kc, vc, slots)
    q = W.to_storage(rng.standard_normal((len(lens), Hkv * G, D), dtype=np.float32), dt)
    out = pa.decode(storage_to_torch(q, dt).cuda(), kc, vc, torch.from_numpy(tables).cuda(),
                    torch.from_numpy(np.array(lens, np.int32)).cuda(), D ** -0.5,
                    out_dtype=torch.float32).cpu().numpy()
    ref = O.decode_contiguous(q, keys, vals, D ** -0.5, G, dt, dt)
    ma, rel = errors(out, ref)
    log(f"[pool > 2 GiB] max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert ma <= 2e-3 and rel <= 1e-3
    # the scatter wrote exactly the rows it was given at those offsets
    b, o = int(tables[3, 1233 // bs]), 1233 % bs
    assert np.array_equal(kc[b, :, o].cpu().view(torch.int16).numpy().view(np.uint16), keys[3][1233])


def test_largest_batch_one_call_takes():
    B = 65535
    rng = np.random.default_rng(92)
    lens = rng.integers(0, 20, size=B)
    w = W.custom("max_batch", 93, lens, 2, 1, 64, 16, "f16")
    from workloads.device import DeviceBatch
    g = DeviceBatch(w)
    out = g.decode().cpu().numpy().astype(np.float64)
    seqs = [0, 1, 4095, 4096, 40000, 65533, 65534]
    from oracle import harness as OH
    kc, vc = OH.build_pools(w, seqs=seqs)
    ref = OH.decode(w, kc, vc, seqs=seqs)
    ma, rel = errors(out[seqs], ref)
    log(f"[65,535 sequences] max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert np.isfinite(out).all() and ma <= 2e-3
    zero = np.nonzero(lens == 0)[0][:50]
    assert (out[zero] == 0).all()
    with pytest.raises(pa.PagedAttentionError):
        pa.decode(torch.zeros((B + 1, 2, 64), dtype=torch.float16, device="cuda"), g.kc, g.vc,
                  torch.zeros((B + 1, 2), dtype=torch.int32, device="cuda"),
                  torch.zeros((B + 1,), dtype=torch.int32, device="cuda"), 0.1)
