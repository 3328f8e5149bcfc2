"""The two page steps of narrow tiles (at most 4 columns, i.e. rows of the
tile x heads per kv head, at hd 64 to 256): MFMA in 16-column blocks, and
the vector-ALU step with packed bf16 dot products and DPP sums.  Each case
runs with the step forced either way (``set_narrow_path``) and must pass the
per-(row, head) gate against the f64 oracle, give fused == separate bit for
bit with the counters back at zero, and, where the case has one, the same
bits from the permuted pool behind a page map.  The window-edge sentinel
workloads (NaN in slots no row sees, dominant keys at each row's edges) pin
the masking of both steps exactly.  The default choice is checked as well:
the 64-sequence batched decode (1536 workgroups) takes the vector-ALU step at
hd 64 and 128 and the MFMA step at hd 256, the one-row tiny decode (one
workgroup) the MFMA step."""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

from tests.gpu_env import need_gpu  # noqa: E402

need_gpu()
import paged_gqa_decode_attn_amd as pg  # noqa: E402
from tests.gates import TOL, per_head  # noqa: E402
from tests.gpu_util import DeviceWorkload, new_counters  # noqa: E402
from tests.test_gpu_edges import multi_row_cases, single_rows_cases, split_counts  # noqa: E402
from tests.test_gpu_random import N_CASES, draw_case  # noqa: E402

VALU, MFMA = 1, 2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def narrow(w):
    return w.hd in (64, 128, 256) and w.nh // w.nkv <= 4


@pytest.fixture(scope="module")
def counters():
    return new_counters()


@pytest.fixture
def path():
    """Sets the narrow-tile step for one test; restores the default after."""
    prev = pg.set_narrow_path(0)
    yield pg.set_narrow_path
    pg.set_narrow_path(prev)


def check(dw, ref, splits, counters, tag):
    fused = dw.host(dw.run(splits, counters=counters))
    assert int(counters.abs().sum().item()) == 0, f"{tag}: counters not zero"
    sep = dw.host(dw.run(splits, counters=None))
    assert np.array_equal(fused, sep), f"{tag}: fused != separate"
    whole, worst, at = per_head(sep, ref)
    say(f"[gpu] {tag}: rel_rms={whole:.3e} worst {at}: {worst:.3e}")
    assert worst < TOL, (tag, at, worst)
    return sep


def edge_cases():
    return [w for w in single_rows_cases() + multi_row_cases() if narrow(w)] + [
        workloads.plant_edges(workloads.single_sequence("g2hd64", ctx=700, rows=6, nh=8, nkv=4, hd=64, window=200),
                              name="g2hd64+edges"),
        workloads.plant_edges(workloads.single_sequence("g1hd64", ctx=333, rows=9, nh=2, nkv=2, hd=64, window=0),
                              name="g1hd64+edges"),
    ]


@pytest.mark.parametrize("w", edge_cases(), ids=lambda w: w.name)
@pytest.mark.parametrize("step", [VALU, MFMA], ids=["valu", "mfma"])
def test_narrow_window_edges(counters, path, w, step):
    path(step)
    ref = oracle.decode(w)
    dw = DeviceWorkload(w)
    for s in split_counts(dw):
        say(f"[gpu] narrow {w.name} step={step} splits={s}")
        check(dw, ref, s, counters, f"{w.name} step={step} S={s}")


RANDOM_NARROW = [i for i in range(N_CASES) if narrow(draw_case(i)[0])]


@pytest.mark.parametrize("i", RANDOM_NARROW)
def test_narrow_random_shapes(counters, path, i):
    w, splits, single = draw_case(i)
    ref = oracle.decode(w)
    dw = DeviceWorkload(w)
    outs = {}
    for step in (VALU, MFMA):
        path(step)
        say(f"[gpu] narrow random case {i} step={step}: rows={w.rows} nh={w.nh} nkv={w.nkv} hd={w.hd} "
            f"window={w.window} splits={splits}")
        outs[step] = check(dw, ref, splits, counters, f"random {i} step={step}")
        wm = workloads.with_page_map(w) if single else workloads.with_page_map(w, first_live=0)
        dm = DeviceWorkload(wm)
        assert np.array_equal(dm.host(dm.run(splits, counters=None)), outs[step]), f"case {i}: page map differs"


def narrow_workload(name):
    # 64-sequence batches at hd 64 and at hd 256 (2 heads per kv head)
    if name == "B64HD64":
        return workloads.batched("B64HD64", nseq=64, lmin=512, lmax=4096, nh=32, nkv=8, hd=64)
    if name == "B64HD256":
        return workloads.batched("B64HD256", nseq=64, lmin=512, lmax=4096, nh=16, nkv=8, hd=256)
    return workloads.make(name)


@pytest.mark.parametrize("name,splits", [("C1", 1), ("C1", 4), ("C4", 3), ("C4NAN", 3), ("B64HD64", 3),
                                         ("B64HD256", 3)])
def test_narrow_configurations(counters, path, name, splits):
    """Both steps on the named narrow configurations, and the default choice."""
    w = narrow_workload(name)
    ref = oracle.decode(w)
    dw = DeviceWorkload(w)
    outs = {}
    for step in (VALU, MFMA):
        path(step)
        say(f"[gpu] narrow {name} step={step} splits={splits}")
        outs[step] = check(dw, ref, splits, counters, f"{name} step={step}")
    path(0)
    auto = dw.host(dw.run(splits, counters=None))
    units = w.rows * w.nkv * splits
    want = VALU if units > 512 and narrow(w) and w.hd <= 128 else MFMA
    say(f"[gpu] narrow {name}: default step {want} over {units} workgroups")
    assert np.array_equal(auto, outs[want]), f"{name}: the default step is not the expected one"
