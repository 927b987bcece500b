"""The C-ABI library: it loads, exports every function include/pa.h declares,
and rejects bad arguments on the host before touching a GPU (these calls
never launch anything, so they run without one)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_342_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = pa.library()
    names = _declared()
    assert {"pa_reshape_and_cache", "pa_decode", "pa_decode_workspace_size", "pa_copy_blocks"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = pa.library()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.pa_status_string(code) != b"unknown status"
    assert b"gfx950" in lib.pa_version()
    assert lib.pa_is_checked_build() == 0


def test_checked_library_exports_the_same_symbols():
    """libpa_checked.so (device-side contract checks) declares the same ABI and
    says it is the checked build; switching back restores libpa.so."""
    pa.use_checked_library(True)
    try:
        lib = pa.library()
        assert lib.pa_is_checked_build() == 1
        for n in _declared():
            assert hasattr(lib, n), n
        # host validation is unchanged: this fails before any check kernel runs
        st = lib.pa_copy_blocks(FAKE, FAKE, FAKE, -1, 2, 128, 16, 10, pa.F16, None)
        assert st == pa.ERR_INVALID_ARG
    finally:
        pa.use_checked_library(False)
    assert pa.library().pa_is_checked_build() == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _decode(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, B=2, Hkv=2, G=2, D=128, bs=16, nb=10, M=4,
             mcl=64, scale=0.1, ks=1.0, vs=1.0, qd=pa.BF16, cd=pa.BF16, od=pa.F32, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return pa.library().pa_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["B"], a["Hkv"], a["G"], a["D"],
                                  a["bs"], a["nb"], a["M"], a["mcl"], a["scale"], a["ks"], a["vs"], a["qd"], a["cd"],
                                  a["od"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), pa.ERR_UNSUPPORTED),
    (dict(bs=12), pa.ERR_UNSUPPORTED),
    (dict(Hkv=0), pa.ERR_INVALID_ARG),
    (dict(G=0), pa.ERR_INVALID_ARG),
    (dict(B=-1), pa.ERR_INVALID_ARG),
    (dict(q=None), pa.ERR_INVALID_ARG),
    (dict(out=FAKE + 2), pa.ERR_INVALID_ARG),
    (dict(qd=pa.F16, cd=pa.BF16), pa.ERR_UNSUPPORTED),
    (dict(qd=pa.F32, cd=pa.F32), pa.ERR_UNSUPPORTED),
    (dict(od=pa.FP8_E4M3), pa.ERR_UNSUPPORTED),
    (dict(qd=7), pa.ERR_INVALID_ARG),
    (dict(cd=pa.FP8_E4M3, ks=0.0), pa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), pa.ERR_INVALID_ARG),
    (dict(M=0), pa.ERR_INVALID_ARG),
    (dict(B=70000), pa.ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_arguments(kw, status):
    assert _decode(**kw) == status
    assert pa.library().pa_last_error_message()


def _decode_append(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, key=FAKE, value=FAKE, sd=pa.BF16, bt=FAKE, cl=FAKE, B=2, Hkv=2, G=2,
             D=128, bs=16, nb=10, M=4, mcl=64, scale=0.1, ks=1.0, vs=1.0, qd=pa.BF16, cd=pa.BF16, od=pa.F32, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return pa.library().pa_decode_append(a["out"], a["q"], a["k"], a["v"], a["key"], a["value"], a["sd"], a["bt"],
                                         a["cl"], a["B"], a["Hkv"], a["G"], a["D"], a["bs"], a["nb"], a["M"], a["mcl"],
                                         a["scale"], a["ks"], a["vs"], a["qd"], a["cd"], a["od"], a["ws"], a["wsb"],
                                         None)


@pytest.mark.parametrize("kw,status", [
    (dict(sd=pa.F16), pa.ERR_UNSUPPORTED),          # 16-bit cache: rows must have its dtype
    (dict(cd=pa.FP8_E4M3, sd=pa.F32), pa.ERR_UNSUPPORTED),
    (dict(sd=9), pa.ERR_INVALID_ARG),
    (dict(key=None), pa.ERR_INVALID_ARG),
    (dict(value=FAKE + 8), pa.ERR_INVALID_ARG),
    (dict(D=96), pa.ERR_UNSUPPORTED),                # the checks of pa_decode apply as well
    (dict(ws=None, wsb=0), pa.ERR_WORKSPACE),
    (dict(qd=pa.F16, cd=pa.BF16), pa.ERR_UNSUPPORTED),
])
def test_decode_append_rejects_bad_arguments(kw, status):
    assert _decode_append(**kw) == status
    assert pa.library().pa_last_error_message()


def test_decode_append_empty_batch_is_a_no_op():
    assert _decode_append(B=0, out=None, q=None, bt=None, cl=None, key=None, value=None) == pa.OK


def test_decode_workspace_checks():
    need = pa.decode_workspace_size(64, 8, 4, 128, 16, 4096)
    assert need > 0
    assert _decode(B=64, Hkv=8, G=4, mcl=4096, M=256, ws=FAKE, wsb=need - 1) == pa.ERR_WORKSPACE
    assert _decode(B=64, Hkv=8, G=4, mcl=4096, M=256, ws=None, wsb=need) == pa.ERR_WORKSPACE
    assert _decode(B=64, Hkv=8, G=4, mcl=4096, M=256, ws=FAKE + 16, wsb=need) == pa.ERR_INVALID_ARG
    # every call needs the workspace (chunk prefix sum + partials), and its
    # size grows with the batch and with the query heads
    small = pa.decode_workspace_size(2, 4, 1, 64, 16, 64)
    assert small > 0
    assert _decode(B=2, Hkv=4, G=1, D=64, mcl=64, M=4, ws=None, wsb=0) == pa.ERR_WORKSPACE
    assert pa.decode_workspace_size(4, 4, 1, 64, 16, 64) > small
    assert pa.decode_workspace_size(2, 4, 2, 64, 16, 64) > small
    # sizes that describe no work give 0
    assert pa.decode_workspace_size(0, 4, 1, 64, 16, 100) == 0


def test_workspace_size_depends_on_the_arguments_alone():
    """The size covers every kernel choice and device: a process whose
    occupancy override differs gets the same sizes."""
    import subprocess
    import sys

    cases = [(64, 8, 4, 128, 16, 4096), (32, 8, 8, 128, 16, 8000), (256, 8, 4, 128, 8, 32768), (3, 2, 1, 64, 32, 100)]
    here = [pa.decode_workspace_size(*c) for c in cases]
    code = ("import sys; sys.path.insert(0, %r); import paged_kv_cache_342_amd as pa; "
            "print([pa.decode_workspace_size(*c) for c in %r])" % (ROOT, cases))
    for waves in ("1", "8", "32"):
        env = dict(os.environ, PA_DECODE_WAVES_PER_CU=waves)
        got = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
        assert eval(got.stdout.strip()) == here


def test_noalloc_refuses_sizes_beyond_its_scratch_on_the_host():
    """pa_decode_append_noalloc checks the partials against its 64 MiB scratch
    array before anything else, so an oversized batch is refused here, with
    no GPU; a batch that fits proceeds to the usual argument checks."""
    lib = pa.library()
    big = dict(B=4000, Hkv=8, G=8, D=128, bs=16, M=2, mcl=32)
    assert pa.decode_workspace_size(big["B"], big["Hkv"], big["G"], big["D"], big["bs"], big["mcl"]) > 64 << 20

    def call(B, Hkv, G, D, bs, M, mcl, key=FAKE):
        return lib.pa_decode_append_noalloc(FAKE, FAKE, FAKE, FAKE, key, key, pa.BF16, FAKE, FAKE, B, Hkv, G, D, bs,
                                            1000, M, mcl, 0.1, 1.0, 1.0, pa.BF16, pa.BF16, pa.F32, None)

    assert call(**big) == pa.ERR_WORKSPACE
    assert b"scratch" in lib.pa_last_error_message()
    assert call(**dict(big, mcl=0)) == pa.ERR_WORKSPACE  # <= 0 reads as M * bs
    # fits: the ordinary checks run next (a null key is refused before any launch)
    assert call(**dict(big, B=4), key=None) == pa.ERR_INVALID_ARG
    assert call(**dict(big, D=96)) == pa.ERR_UNSUPPORTED
    assert call(**dict(big, B=0)) == pa.OK


def test_empty_calls_are_no_ops():
    lib = pa.library()
    assert _decode(B=0, out=None, q=None, bt=None, cl=None) == pa.OK
    assert lib.pa_reshape_and_cache(None, None, FAKE, FAKE, None, 0, 8, 128, 16, 10, pa.BF16, pa.BF16, 1.0, 1.0, None) == pa.OK
    assert lib.pa_copy_blocks(FAKE, FAKE, None, 0, 8, 128, 16, 10, pa.BF16, None) == pa.OK


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, pa.BF16, pa.BF16, 1.0, 1.0), pa.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 80, 16, 10, pa.BF16, pa.BF16, 1.0, 1.0), pa.ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, pa.F16, pa.BF16, 1.0, 1.0), pa.ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, pa.BF16, pa.FP8_E4M3, -1.0, 1.0), pa.ERR_INVALID_ARG),
    ((FAKE, FAKE, None, FAKE, FAKE, 4, 8, 128, 16, 10, pa.BF16, pa.BF16, 1.0, 1.0), pa.ERR_INVALID_ARG),
    ((FAKE, FAKE, FAKE, FAKE, FAKE + 4, 4, 8, 128, 16, 10, pa.BF16, pa.BF16, 1.0, 1.0), pa.ERR_INVALID_ARG),
])
def test_reshape_and_cache_rejects_bad_arguments(args, status):
    assert pa.library().pa_reshape_and_cache(*args, None) == status


def test_copy_blocks_rejects_bad_arguments():
    lib = pa.library()
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, pa.BF16, None) == pa.ERR_INVALID_ARG
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, 2, 8, 128, 16, 10, pa.F32, None) == pa.ERR_UNSUPPORTED
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE + 4, 2, 8, 128, 16, 10, pa.BF16, None) == pa.ERR_INVALID_ARG


def test_slot_mapping_matches_the_block_table_convention():
    import numpy as np
    from oracle import pa_oracle as O
    tables = np.array([[17, 3, 42, -1], [5, 6, 7, 8]], np.int32)
    got = pa.slot_mapping(tables, [0, 1], [0, 3], [10, 16], 4)
    ref = np.concatenate([O.slots_for(tables[0], 0, 10, 4), O.slots_for(tables[1], 3, 16, 4)])
    assert np.array_equal(got, ref)
    with pytest.raises(ValueError):
        pa.slot_mapping(tables, [0], [0], [13], 4)
