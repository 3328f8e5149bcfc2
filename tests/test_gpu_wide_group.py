"""Batches with more than 16 query heads per kv head, at the split count
pgqa_choose_splits_heads gives them (one round of the shared-page kernel's
workgroups): each (row, head) meets the f64 oracle, the fused merge equals
the separate combine bit for bit, and the counters end at zero.  The
lengths are spread like the batched workload's (a narrower range keeps the
oracle quick), so the tiles' split counts differ from row to row; the last
shapes launch more than the 256 workgroups the device holds at once, which
takes the rows longest first."""
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
from tests.gpu_util import DeviceWorkload, new_counters  # noqa: E402

SHAPES = [  # nseq, nh, nkv, hd, lmin, lmax
    (32, 32, 1, 128, 64, 3000),
    (12, 64, 2, 128, 1, 2500),
    (20, 32, 1, 256, 300, 2000),
    (6, 48, 2, 256, 16, 1200),
    (3, 32, 1, 512, 700, 900),
    # launches of more than 256 workgroups: rows taken longest first
    (64, 32, 1, 128, 16, 3000),
    (48, 64, 2, 256, 1, 1500),
    (40, 48, 1, 512, 100, 1100),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}_{s[2]}_{s[3]}" for s in SHAPES])
def test_wide_group_batch_at_the_chosen_count(shape):
    nseq, nh, nkv, hd, lmin, lmax = shape
    w = workloads.batched(f"wide{nseq}_{nh}_{nkv}_{hd}", nseq=nseq, lmin=lmin, lmax=lmax, nh=nh, nkv=nkv, hd=hd,
                          len_seed=31 + nseq, data_seed=4000 + hd)
    span = int(np.max(w.kv_last)) + 1
    splits = pg.choose_splits_heads(span, w.rows, nh, nkv, hd, 1)
    say(f"[gpu] wide group {shape}: splits {splits}")
    assert 1 <= splits <= 256
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    sep = dw.host(dw.run(splits, counters=None))
    whole, worst, at = per_head(sep, ref)
    say(f"[gpu] wide group {shape}: rel_rms={whole:.3e} worst {at}: {worst:.3e}")
    assert worst < TOL, (shape, at, worst)
    cnt = new_counters()
    fused = dw.host(dw.run(splits, counters=cnt))
    assert int(cnt.abs().sum().item()) == 0, "counters not back at zero"
    assert np.array_equal(fused, sep), "fused merge != separate combine"


N_RANDOM = 32


def draw_wide(i):
    """Random wide-group batch i (a fixed function of i) and its split count;
    large enough batches launch more than 256 workgroups."""
    r = np.random.default_rng(7000 + i)
    hd = int(r.choice([128, 256, 512]))
    nkv = int(r.choice([1, 2]))
    group = int(r.choice([24, 32, 48, 64]))
    nseq = int(r.integers(2, 81))
    lmin = int(r.integers(1, 400))
    lmax = lmin + int(r.integers(0, 1800))
    while nseq > 2 and nseq * lmax * nkv * hd > (24 << 20):
        nseq -= 1
    w = workloads.batched(f"widerand{i}", nseq=nseq, lmin=lmin, lmax=lmax, nh=nkv * group, nkv=nkv, hd=hd,
                          window=int(r.choice([0, 0, 300])), len_seed=800 + i, data_seed=1900 + i)
    splits = int(r.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    return w, splits


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_wide_group_batch(i):
    w, splits = draw_wide(i)
    say(f"[gpu] wide random {i}: rows={w.rows} nh={w.nh} nkv={w.nkv} hd={w.hd} window={w.window} splits={splits}")
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    sep = dw.host(dw.run(splits, counters=None))
    whole, worst, at = per_head(sep, ref)
    assert worst < TOL, (i, at, worst)
    cnt = new_counters()
    fused = dw.host(dw.run(splits, counters=cnt))
    assert int(cnt.abs().sum().item()) == 0, f"case {i}: counters not back at zero"
    assert np.array_equal(fused, sep), f"case {i}: fused merge != separate combine"


@pytest.mark.parametrize("kind,nh,nkv,hd,splits", [
    ("batch", 128, 1, 128, 4), ("batch", 96, 1, 256, 6), ("batch", 192, 2, 128, 16), ("batch", 80, 1, 512, 3),
    ("single", 128, 1, 128, 64), ("single", 96, 1, 256, 33), ("single", 160, 2, 128, 1), ("single", 72, 1, 512, 20),
    ("batch", 64, 1, 64, 5), ("single", 48, 1, 64, 40),
])
def test_groups_wider_than_a_tile(kind, nh, nkv, hd, splits):
    """More query heads per kv head than one tile holds (several head blocks
    per row, the last one partial where the group is not a multiple of the
    tile), in batches and on one multi-row sequence."""
    if kind == "batch":
        w = workloads.batched(f"hb_{nh}_{nkv}_{hd}", nseq=9, lmin=30, lmax=1400, nh=nh, nkv=nkv, hd=hd,
                              len_seed=55 + nh, data_seed=600 + hd)
    else:
        w = workloads.single_sequence(f"hb1_{nh}_{nkv}_{hd}", ctx=2100, rows=3, nh=nh, nkv=nkv, hd=hd, window=700,
                                      seed=91 + nh)
    say(f"[gpu] wide tile {kind} nh={nh} nkv={nkv} hd={hd} splits={splits}")
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    sep = dw.host(dw.run(splits, counters=None))
    whole, worst, at = per_head(sep, ref)
    assert worst < TOL, (kind, nh, hd, at, worst)
    cnt = new_counters()
    fused = dw.host(dw.run(splits, counters=cnt))
    assert int(cnt.abs().sum().item()) == 0, "counters not back at zero"
    assert np.array_equal(fused, sep), "fused merge != separate combine"
