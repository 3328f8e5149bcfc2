"""Decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with the program's own eager work and synchronisations
between replays, gives bit for bit the eager call's output, and the fused
merge's counters are back at zero after each (the library records no memset;
the counters reset themselves).  Covers the one-workgroup and the parallel
fused merge, the separate combine and the allocation-free entry point."""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

from tests.gpu_env import need_gpu  # noqa: E402

need_gpu()
import torch  # noqa: E402

import paged_gqa_decode_attn_amd as pg  # noqa: E402
from tests.gpu_util import DeviceWorkload, new_counters  # noqa: E402

REPLAYS = 4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,splits,fused", [("C4", 3, True), ("C3", 128, True), ("C3", 128, False),
                                               ("PA", 8, True), ("C5W4096", 64, True)])
def test_decode_replays_from_a_graph(name, splits, fused):
    w = workloads.make(name)
    say(f"[gpu] graph {name} S={splits} {'fused' if fused else 'separate'}")
    dw = DeviceWorkload(w)
    out = torch.empty((w.rows, w.nh, w.hd), dtype=torch.int16, device="cuda")
    part = torch.empty(max(1, pg.decode_part_bytes(w.rows, w.nh, splits, w.hd)), dtype=torch.uint8, device="cuda")
    cnt = new_counters() if fused else None
    dw.run(splits, counters=cnt, out=out, part=part)
    ref = dw.host(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the capture's warm-up, on its own stream
        dw.run(splits, counters=cnt, out=out, part=part, sync=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dw.run(splits, counters=cnt, out=out, part=part, sync=False)
    for i in range(REPLAYS):
        out.fill_(0x1234)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dw.host(out), ref), f"{name}: replay {i} differs from the eager call"
        if cnt is not None:
            assert int(cnt.abs().sum().item()) == 0, f"{name}: counters not zero after replay {i}"
    del g


def test_noalloc_replays_from_a_graph():
    """The allocation-free entry point, for callers that capture: its partials
    live in the library's static scratch, so the capture holds no buffer of
    the caller's beyond the inputs and the output."""
    w = workloads.make("C5W4096")
    splits = 64
    dw = DeviceWorkload(w)
    out = torch.empty((w.rows, w.nh, w.hd), dtype=torch.int16, device="cuda")

    def call():
        pg.attn_decode_noalloc(out, dw.q, dw.k, dw.v, dw.bt, dw.off, dw.qpos, dw.last, w.rows, w.nh, w.nkv, w.hd,
                               w.window, splits, page_map=dw.pmap)

    call()
    torch.cuda.synchronize()
    ref = dw.host(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(REPLAYS):
        out.fill_(0x1234)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dw.host(out), ref), f"noalloc: replay {i} differs from the eager call"
    del g
