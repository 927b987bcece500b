"""The decode calls captured in a HIP graph (as a serving loop would): each
replay, with eager work and synchronisations in between, equals the eager
call bit for bit.  The library records no memset and allocates nothing, so
its launches are all a graph holds besides what the test itself records."""
import numpy as np
import pytest
import torch

import paged_kv_cache_342_amd as pa
import workloads as W
from tests.gpu_util import GpuBatch, log

pytestmark = pytest.mark.gpu


def _replays_match(step, out, label, replays=4):
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for i in range(replays):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, eager)
        log(f"[graph {label}] replay {i}: {'equal' if same else 'DIFFERENT'}")
        assert same
        # eager work between replays
        torch.ones(1 << 20, device="cuda").sum()


def test_decode_append_step_in_a_graph():
    w = W.llama8b(B=16)
    g = GpuBatch(w, skip_last_append=True)
    k_new, v_new = g.last_rows()
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.decode_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len), dtype=torch.uint8,
                     device="cuda")

    def step():
        pa.decode_append(g.q, g.kc, g.vc, k_new, v_new, g.tables, g.lens, w.scale, max_context_len=w.max_context_len,
                         out=out, workspace=ws)

    _replays_match(step, out, "decode_append")


def test_decode_multi_in_a_graph():
    w = W.chunked_prefill(B=3)
    g = GpuBatch(w)
    qs = torch.from_numpy(w.query_start).cuda()
    out = torch.empty(tuple(g.q.shape), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.decode_multi_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len, w.max_queries),
                     dtype=torch.uint8, device="cuda")

    def step():
        pa.decode_multi(g.q, g.kc, g.vc, g.tables, g.lens, qs, w.max_queries, w.scale,
                        max_context_len=w.max_context_len, out=out, workspace=ws)

    _replays_match(step, out, "decode_multi")


def test_fp8_row_scale_decode_in_a_graph():
    w = W.heavy_tail(bs=16, B=24)
    g = GpuBatch(w, row_scales=True)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.decode_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len), dtype=torch.uint8,
                     device="cuda")

    def step():
        pa.decode_scaled(g.q, g.kc, g.vc, g.kss, g.vss, g.tables, g.lens, w.scale, max_context_len=w.max_context_len,
                         out=out, workspace=ws)

    _replays_match(step, out, "decode_scaled")
    assert np.isfinite(out.cpu().numpy()).all()


def test_window_decode_in_a_graph():
    w = W.llama70b(B=6)
    g = GpuBatch(w)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.decode_workspace_size(w.B, w.Hkv, w.group, w.D, w.bs, w.max_context_len), dtype=torch.uint8,
                     device="cuda")

    def step():
        pa.decode_window(g.q, g.kc, g.vc, g.tables, g.lens, w.scale, 4, 1024, max_context_len=w.max_context_len,
                         out=out, workspace=ws)

    _replays_match(step, out, "decode_window")


def test_shared_prefix_decode_in_a_graph():
    """Both passes, the merge between them and the final merge in one graph."""
    w = W.shared_prefix(prompts=3, samples=4, prefix=700, max_tail=100)
    g = GpuBatch(w)
    samples, plen = w.meta["samples"], w.meta["shared_len"]
    group_start = torch.tensor(np.arange(len(plen) + 1) * samples, dtype=torch.int32, device="cuda")
    prefix_lens = torch.tensor(np.asarray(plen), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pa.decode_shared_prefix_workspace_size(w.B, len(plen), samples, w.Hkv, w.group, w.D, w.bs,
                                                            w.max_context_len), dtype=torch.uint8, device="cuda")

    def step():
        pa.decode_shared_prefix(g.q, g.kc, g.vc, g.tables, g.lens, group_start, prefix_lens, samples, w.scale,
                                max_context_len=w.max_context_len, out=out, workspace=ws)

    _replays_match(step, out, "decode_shared_prefix")
