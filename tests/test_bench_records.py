"""The bench's recorded profiler traffic: every bench line whose HBM bytes are
recorded finds its record under the name the bench looks it up by, and each
record points at a committed summary.  (The lookup itself returns nothing
once the decode sources change; that is checked too.)  No GPU is needed:
the workloads are built on the host and only their names are used."""
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (config, --row-scales, --fp4, --block-size) of the bench lines with profiler records
LINES = [
    ("llama8b", False, False, 0),
    ("llama70b", False, False, 0),
    ("heavy_tail", False, False, 0),
    ("heavy_tail", False, False, 8),
    ("heavy_tail", False, False, 32),
    ("shared_prefix", False, False, 0),
    ("spec_decode", False, False, 0),
    ("chunked_prefill", False, False, 0),
    ("heavy_tail", True, False, 0),
    ("llama8b", True, True, 0),
    ("heavy_tail", True, True, 0),
]


def _record():
    with open(bench.TRAFFIC_FILE) as f:
        return json.load(f)


@pytest.mark.parametrize("config,row_scales,fp4,block_size", LINES)
def test_every_profiled_line_finds_its_record(config, row_scales, fp4, block_size):
    w = bench.select_workload(config, 0, fp4, block_size)
    key = bench.traffic_key(w.name, row_scales or fp4)
    rec = _record()["workloads"]
    assert key in rec, f"no recorded traffic under {key!r}"
    r = rec[key]
    assert os.path.exists(os.path.join(ROOT, r["summary"]))
    # the record's algorithmic bytes are the bench's: K and V rows of every
    # position and KV head (plus two 4-byte scales per row with row scales)
    kv = w.kv_bytes() + (int(w.context_lens.sum()) * w.Hkv * 8 if (row_scales or fp4) else 0)
    assert r["algorithmic_kv_bytes"] == kv
    assert 0.5 * kv < r["hbm_bytes_per_call"] < 4 * kv


def test_records_are_dropped_when_the_sources_change(monkeypatch):
    key = bench.traffic_key("llama8b", False)
    if _record()["decode_source_sha256_16"] == bench.decode_source_hash():
        assert bench.recorded_traffic(key) == _record()["workloads"][key]["hbm_bytes_per_call"]
    monkeypatch.setattr(bench, "decode_source_hash", lambda: "0" * 16)
    assert bench.recorded_traffic(key) is None


def test_cascade_and_window_lines_find_their_records():
    """The shared-prefix cascade line (--cascade) and the sinks-plus-window
    line (--config llama70b --window 4,2048) are recorded under the workload
    name with the bench's suffix; the cascade reads each prompt's prefix once,
    so its bytes are well under the logical bytes of all samples' contexts,
    and the window line reads about the bytes of the positions it attends."""
    rec = _record()["workloads"]
    for key in ("shared_prefix+cascade", "llama70b+window4,2048"):
        assert key in rec, f"no recorded traffic under {key!r}"
        assert os.path.exists(os.path.join(ROOT, rec[key]["summary"]))
    w = bench.select_workload("shared_prefix", 0, False, 0)
    cas = rec["shared_prefix+cascade"]
    assert cas["algorithmic_kv_bytes"] == w.kv_bytes()
    assert cas["hbm_bytes_per_call"] < 0.5 * w.kv_bytes()
    win = rec["llama70b+window4,2048"]
    assert 0.9 * win["algorithmic_kv_bytes"] < win["hbm_bytes_per_call"] < 1.5 * win["algorithmic_kv_bytes"]
