"""GPU parity of paged prefill (span-02 GPU test page, `run()`, the prefill
section): every context row attends causally (within the window) over the
same paged pool; rel-RMS < 1e-2 against the f64 oracle, and bit-identical
results for an identity pool and a permuted pool behind a page map."""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from tests.gpu_env import need_gpu  # noqa: E402

need_gpu()
import torch  # noqa: E402

import paged_gqa_decode_attn_amd as pg  # noqa: E402
from tests.gates import TOL, per_head  # noqa: E402
from tests.gpu_util import DeviceWorkload  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_workload(name, ctx, nh, nkv, hd, window):
    """All ctx rows of one sequence, at positions 0 .. ctx-1."""
    return workloads.single_sequence(name, ctx=ctx, rows=ctx, nh=nh, nkv=nkv, hd=hd, window=window)


CASES = [
    # the page's two prefill runs (its PA and PB shapes); at hd 256 a launch
    # of fewer than 512 (tile, kv head) units takes 64-column tiles
    ("pf_pa", 1500, 16, 8, 256, 1024),
    # hd 256 with 512 units: the wide 128-column form
    ("pf_wide256", 2048, 32, 16, 256, 128),
    ("pf_pb", 700, 16, 2, 512, 0),
    # the per-wave kernel (hd 64) and the shared-page kernel at hd 128, group 8
    ("pf_hd64", 300, 8, 2, 64, 50),
    ("pf_hd128", 257, 16, 2, 128, 0),
    # one head per kv head: the teams take alternate pages instead of
    # separate column blocks
    ("pf_mha", 200, 4, 4, 128, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_prefill_matches_oracle_and_page_map(case):
    name, ctx, nh, nkv, hd, window = case
    w = prefill_workload(*case)
    say(f"[gpu] prefill {name}: ctx={ctx} nh={nh} nkv={nkv} hd={hd} window={window}")
    dw = DeviceWorkload(w)
    got = dw.host(dw.prefill())
    ref = oracle.decode(w)
    whole, worst, at = per_head(got, ref)
    say(f"[gpu] prefill {name}: rel_rms={whole:.3e} worst (row, head) {at}: {worst:.3e}")
    assert worst < TOL, (name, at, worst)
    # the page's mapped pool for prefill keeps every page live
    wm = workloads.with_page_map(w, first_live=0)
    dm = DeviceWorkload(wm)
    assert np.array_equal(dm.host(dm.prefill()), got), f"{name}: page-map pool differs"
    # the same rows through decode agree within the bound too
    dec = dw.host(dw.run(1))
    assert per_head(dec, ref)[1] < TOL


def test_prefill_batched_sequences_and_tile_sizes():
    """Several sequences with distinct non-zero origins (tiles cut at every
    origin change), every row of each sequence, smaller caller tiles too."""
    b = workloads.batched("pfb", nseq=5, lmin=20, lmax=200, nh=8, nkv=2, hd=128, pad=16)
    lens = (b.kv_last + 1).astype(int)
    seq = np.repeat(np.arange(5), lens)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    rng = np.random.default_rng(9)
    q = (rng.standard_normal((len(seq), b.nh, b.hd)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = b.replace(name="pfb", rows=len(seq), q=q, page_origin=b.page_origin[seq].copy(), qpos=pos,
                  kv_last=pos.copy(), window=37)
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    full = dw.host(dw.prefill())
    assert per_head(full, ref)[1] < TOL
    for rpt in (1, 5, 16, 64):
        tiles = pg.make_tiles(w.page_origin, rpt)
        got = dw.host(dw.prefill(tiles=tiles))
        assert per_head(got, ref)[1] < TOL, rpt


def test_prefill_skips_tiles_outside_the_rows():
    """A tile that would reach past the last row is skipped (its rows are left
    as they were); the other tiles are computed."""
    w = prefill_workload("pf_bad", 100, 8, 2, 128, 0)
    dw = DeviceWorkload(w)
    t0 = np.array([0, 64, 90], np.int32)
    tn = np.array([64, 26, 20], np.int32)  # the last tile claims rows 90..109 of 100
    out = torch.full((w.rows, w.nh, w.hd), 0x1234, dtype=torch.int16, device="cuda")
    got = dw.host(dw.prefill(tiles=(t0, tn), out=out))
    ref = oracle.decode(w)
    assert per_head(got[:90], ref[:90])[1] < TOL
    assert np.all(got[90:] == 0x1234)


def test_prefill_full_8k_context_sampled_rows():
    """The 8192-row causal context (nh 16, nkv 8, hd 256) that the benchmark
    times, in the same launch (tiles from make_tiles): 72 rows -- both edges of
    several 64-row tiles, the first and last rows, and rows drawn at random --
    against the oracle computed for those rows alone; the permuted pool behind
    a page map gives the same bits."""
    w = prefill_workload("pf8k", 8192, 16, 8, 256, 0)
    say(f"[gpu] prefill 8K: rows={w.rows} nh={w.nh} nkv={w.nkv} hd={w.hd}")
    dw = DeviceWorkload(w)
    got = dw.host(dw.prefill())
    rng = np.random.default_rng(8192)
    edges = [0, 1, 62, 63, 64, 65, 4095, 4096, 8126, 8127, 8128, 8129, 8190, 8191]
    rows = sorted(set(edges) | set(int(r) for r in rng.choice(8192, 58, replace=False)))
    ref = oracle.decode(oracle.rows_subset(w, rows))
    whole, worst, at = per_head(got[rows], ref)
    say(f"[gpu] prefill 8K: {len(rows)} sampled rows, rel_rms={whole:.3e} worst {at}: {worst:.3e}")
    assert worst < TOL, (rows[at[0]], at[1], worst)
    wm = workloads.with_page_map(w, first_live=0)
    dm = DeviceWorkload(wm)
    assert np.array_equal(dm.host(dm.prefill()), got), "8K prefill: page-map pool differs"
