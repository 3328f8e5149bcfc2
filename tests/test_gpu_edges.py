"""GPU pins of the visibility boundary (span-02 GPU test page, ``reference``:
a key is visible to a row when it is at or before the row's last key and,
in a sliding layer, less than ``window`` positions before the query).

Every workload here carries window-edge sentinels (``workloads.plant_edges``):
NaN in each slot of a loaded page that no row of the sequence sees, and a
dominant key aimed at one head per kv group of row t at lo_t - 1 and
kv_last_t + 1 wherever another row of the sequence sees that slot.  A kernel
that takes in one key too many at either edge of any row makes that row's
output NaN, or turns the aimed-at head into the planted key's V row; either
fails the per-(row, head) gate by orders of magnitude.

Each case runs at 1, 3, the heuristic's and (pages + 3) splits, fused and
separate (bitwise equal), against the oracle per (row, head).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from tests.gpu_env import need_gpu  # noqa: E402

need_gpu()
from tests.gates import TOL, per_head  # noqa: E402
from tests.gpu_util import DeviceWorkload, new_counters  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def single_rows_cases():
    """Batches of one-row sequences: every edge slot is seen by no row, so it
    holds NaN.  Shapes reach the per-wave kernel at hd 64/128/256/512 and the
    shared-page kernel (group 8; and hd 512 below 64 splits)."""
    eb = workloads.edge_batch
    return [
        eb("eb256g2", nseq=8, lmin=300, lmax=3000, nh=16, nkv=8, hd=256, window=300),
        eb("eb128g4", nseq=16, lmin=200, lmax=2500, nh=32, nkv=8, hd=128, window=200),
        eb("eb64g4", nseq=5, lmin=100, lmax=900, nh=16, nkv=4, hd=64, window=100),
        eb("eb512g8", nseq=2, lmin=1200, lmax=4000, nh=16, nkv=2, hd=512, window=700),
        eb("eb256g8", nseq=6, lmin=300, lmax=3000, nh=8, nkv=1, hd=256, window=250),
        eb("eb128g4w0", nseq=7, lmin=100, lmax=2000, nh=32, nkv=8, hd=128, window=0),
    ]


def multi_row_cases():
    """Rows that share a sequence: row t's lo_t - 1 is seen by the rows before
    it and kv_last_t + 1 by the rows after it, so those slots hold dominant
    keys; the slots outside every row's range hold NaN."""
    seq = workloads.single_sequence
    cases = [workloads.plant_edges(workloads.make(n)) for n in ("PA", "C2")]
    cases.append(workloads.plant_edges(seq("c5w", ctx=9000, rows=8, nh=8, nkv=1, hd=256, window=4096,
                                           k_scale=8.0), name="c5w+edges"))
    cases.append(workloads.plant_edges(seq("mha", ctx=257, rows=19, nh=4, nkv=4, hd=128, window=100),
                                       name="mha+edges"))
    cases.append(workloads.plant_edges(seq("mr512", ctx=900, rows=3, nh=16, nkv=2, hd=512, window=250),
                                       name="mr512+edges"))
    wb = seq("blk", ctx=404, rows=4, nh=8, nkv=2, hd=128, window=50)
    cases.append(workloads.plant_edges(wb.replace(qpos=np.arange(396, 400, dtype=np.int32),
                                                  kv_last=np.full(4, 403, np.int32)), name="blockwin+edges"))
    # rows whose last visible keys are spread below their positions, window 0
    wk = seq("kvl", ctx=500, rows=4, nh=8, nkv=2, hd=256, window=0)
    cases.append(workloads.plant_edges(wk.replace(kv_last=np.array([100, 499, 300, 498], np.int32)),
                                       name="kvlast+edges"))
    return cases


@pytest.fixture(scope="module")
def counters():
    return new_counters()


def split_counts(dw):
    w = dw.w
    ctx = int(w.kv_last.max()) + 1
    pages = (ctx + 15) // 16
    rps = 1 if len(set(w.page_origin.tolist())) == w.rows else w.rows
    return sorted({1, 3, dw.heuristic_splits(rows_per_seq=rps), min(256, pages + 3)})


@pytest.mark.parametrize("w", single_rows_cases() + multi_row_cases(), ids=lambda w: w.name)
def test_window_edges_are_exact(counters, w):
    ref = oracle.decode(w)
    assert np.isfinite(workloads.bf16_bits_to_f32(ref)).all()
    dw = DeviceWorkload(w)
    for s in split_counts(dw):
        say(f"[gpu] edges {w.name} splits={s}")
        fused = dw.host(dw.run(s, counters=counters))
        assert int(counters.abs().sum().item()) == 0, "merge counters not restored to zero"
        sep = dw.host(dw.run(s, counters=None))
        assert np.array_equal(fused, sep), (w.name, s, "fused != separate")
        whole, worst, at = per_head(fused, ref)
        say(f"[gpu] edges {w.name} splits={s} rel_rms={whole:.3e} worst (row, head) {at}: {worst:.3e}")
        assert worst < TOL, (w.name, s, at, worst)
