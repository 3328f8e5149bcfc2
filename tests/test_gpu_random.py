"""A seeded sweep of random small decode shapes through the C ABI, so that
every kernel the plan can pick (per-wave, hd-sliced, shared-page; ranked and
plain launches; one-workgroup and parallel fused merges) meets the oracle on
shapes no other test names: rows, heads per kv head, hd, window, one
sequence or a batch of sequences, and the split count are drawn at random.
Each case: the per-(row, head) gate against the f64 oracle, fused merge ==
separate combine bit for bit, counters back at zero, and (every third case)
the permuted pool behind a page map gives the same bits (one sequence: with
the NaN null page below the first row's window)."""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from tests.gpu_env import need_gpu  # noqa: E402

need_gpu()
import torch  # noqa: E402

from tests.gates import TOL, per_head  # noqa: E402
from tests.gpu_util import DeviceWorkload, new_counters  # noqa: E402

N_CASES = 400


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw_case(i):
    """Case i of the sweep (a fixed function of i): (workload, splits, one
    sequence or not)."""
    r = np.random.default_rng(1000 + i)
    hd = int(r.choice([64, 128, 256, 512]))
    nkv = int(r.choice([1, 2, 4, 8]))
    group = int(r.choice([1, 2, 4, 8, 16]))
    if hd == 512:
        group = min(group, 8)
    nh = nkv * group
    window = int(r.choice([0, 0, 1, 7, 64, 333]))
    single = r.random() < 0.5
    if single:
        ctx = int(r.integers(1, 3000))
        rows = int(r.integers(1, min(ctx, 24) + 1))
        w = workloads.single_sequence(f"rand{i}", ctx=ctx, rows=rows, nh=nh, nkv=nkv, hd=hd, window=window,
                                      seed=77 + i)
        pages = (ctx + 15) // 16
    else:
        nseq = int(r.integers(2, 40))
        lmin = int(r.integers(1, 300))
        lmax = lmin + int(r.integers(0, 2500))
        # at most about 32M pool elements per pool
        while nseq > 2 and nseq * lmax * nkv * hd > (32 << 20):
            nseq -= 1
        while nseq * lmax * nkv * hd > (32 << 20):
            lmax = max(lmin, lmax // 2)
            if lmax == lmin:
                break
        w = workloads.batched(f"rand{i}", nseq=nseq, lmin=lmin, lmax=lmax, nh=nh, nkv=nkv, hd=hd,
                              window=window, len_seed=500 + i, data_seed=900 + i)
        pages = (lmax + 15) // 16
    splits = int(r.choice([1, 2, 3, 5, 8, 16, 33, 64]))
    splits = max(1, min(splits, 256, pages + 3))
    return w, splits, single


@pytest.fixture(scope="module")
def counters():
    return new_counters()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(counters, i):
    w, splits, single = draw_case(i)
    say(f"[gpu] random case {i}: rows={w.rows} nh={w.nh} nkv={w.nkv} hd={w.hd} window={w.window} "
        f"pages={w.npages} splits={splits}")
    units = w.rows * w.nkv * ((w.nh // w.nkv + 15) // 16)
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    sep = dw.host(dw.run(splits, counters=None))
    whole, worst, at = per_head(sep, ref)
    say(f"[gpu] random case {i}: rel_rms={whole:.3e} worst {at}: {worst:.3e}")
    assert worst < TOL, (i, at, worst)
    if units <= 4096:
        fused = dw.host(dw.run(splits, counters=counters))
        assert int(counters.abs().sum().item()) == 0, f"case {i}: counters not zero"
        assert np.array_equal(fused, sep), f"case {i}: fused merge != separate combine"
    if i % 3 == 0:
        # one sequence: the page's mapped pool, whose pages below the first
        # row's window map to the NaN null page; a batch: the permutation only
        # (its rows' windows start in different places)
        wm = workloads.with_page_map(w) if single else workloads.with_page_map(w, first_live=0)
        dm = DeviceWorkload(wm)
        assert np.array_equal(dm.host(dm.run(splits, counters=None)), sep), f"case {i}: page map differs"
