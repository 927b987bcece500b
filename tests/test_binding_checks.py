"""Host-side checks of the Python binding that need no GPU: a wrong-shaped
output or copy-pair tensor is refused with ValueError before anything is
launched (the kernels would otherwise write or read outside it), and a
max_context_len of 0 or below plans with every table entry, as the C calls
read it.

The binding's residency check (tensors must live on the GPU) is replaced by
one that accepts CPU tensors, so these shape checks run here; each case
fails before the library is called."""
import pytest
import torch

import paged_kv_cache_342_amd as pa


@pytest.fixture(autouse=True)
def cpu_tensors_pass_residency(monkeypatch):
    def require(t, name, dtype=None):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
            raise ValueError(f"{name} has dtype {t.dtype}")

    monkeypatch.setattr(pa, "_require", require)

    def no_library():
        raise AssertionError("the library was called")

    monkeypatch.setattr(pa, "library", no_library)


B, Hq, Hkv, D, bs, M, NB = 3, 8, 2, 64, 16, 4, 12


def _args(dtype=torch.float16):
    q = torch.zeros((B, Hq, D), dtype=dtype)
    kc = torch.zeros((NB, Hkv, bs, D), dtype=dtype)
    tables = torch.zeros((B, M), dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    return q, kc, kc.clone(), tables, lens


@pytest.mark.parametrize("shape", [(B, Hq, D - 1), (B - 1, Hq, D), (B, Hq), (B, Hq, D, 1), (B * Hq * D,)])
def test_decode_refuses_wrong_out_shape(shape):
    q, kc, vc, tables, lens = _args()
    out = torch.zeros(shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="out must have shape"):
        pa.decode(q, kc, vc, tables, lens, 0.125, out=out)


def test_decode_append_refuses_wrong_out_shape():
    q, kc, vc, tables, lens = _args()
    key = torch.zeros((B, Hkv, D), dtype=torch.float16)
    with pytest.raises(ValueError, match="out must have shape"):
        pa.decode_append(q, kc, vc, key, key.clone(), tables, lens, 0.125,
                         out=torch.zeros((B + 1, Hq, D), dtype=torch.float32))


def test_decode_scaled_refuses_wrong_out_shape():
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16)
    kc = torch.zeros((NB, Hkv, bs, D), dtype=torch.float8_e4m3fn)
    sc = torch.ones((NB, Hkv, bs), dtype=torch.float32)
    tables, lens = torch.zeros((B, M), dtype=torch.int32), torch.ones(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        pa.decode_scaled(q, kc, kc.clone(), sc, sc.clone(), tables, lens, 0.125,
                         out=torch.zeros((B, Hq // 2, D), dtype=torch.float32))


def test_decode_multi_refuses_wrong_out_shape():
    T = 7
    q = torch.zeros((T, Hq, D), dtype=torch.float16)
    _, kc, vc, tables, lens = _args()
    qs = torch.tensor([0, 2, 5, 7], dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        pa.decode_multi(q, kc, vc, tables, lens, qs, 3, 0.125, out=torch.zeros((B, Hq, D), dtype=torch.float32))


def test_out_dtype_must_be_a_result_dtype():
    q, kc, vc, tables, lens = _args()
    with pytest.raises(ValueError, match="out has dtype"):
        pa.decode(q, kc, vc, tables, lens, 0.125, out=torch.zeros((B, Hq, D), dtype=torch.int32))


@pytest.mark.parametrize("shape", [(4, 3), (8,), (2, 2, 2), (4, 1)])
def test_copy_blocks_refuses_pairs_not_n_by_2(shape):
    _, kc, vc, _, _ = _args()
    pairs = torch.zeros(shape, dtype=torch.int64)
    with pytest.raises(ValueError, match=r"block_mapping must be \[N, 2\]"):
        pa.copy_blocks(kc, vc, pairs)
    fp8 = torch.zeros((NB, Hkv, bs, D), dtype=torch.float8_e4m3fn)
    sc = torch.ones((NB, Hkv, bs), dtype=torch.float32)
    with pytest.raises(ValueError, match=r"block_mapping must be \[N, 2\]"):
        pa.copy_blocks_scaled(fp8, fp8.clone(), sc, sc.clone(), pairs)


@pytest.mark.parametrize("given, planned", [(None, M * bs), (0, M * bs), (-5, M * bs), (37, 37)])
def test_max_context_len_of_zero_or_less_means_every_table_entry(given, planned):
    assert pa._max_context(given, M, bs) == planned
