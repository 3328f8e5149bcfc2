"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, and the
bitwise gates of the span-02 GPU test page (fused merge == separate combine;
identity pool == permuted pool behind a page map with a NaN null page).

Tolerance: rel-RMS < 1e-2 against the oracle (the page's bound for decode),
required of every (row, head) output vector on its own.
"""
import functools
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def workload(name):
    return workloads.make(name)


@functools.lru_cache(maxsize=None)
def reference(name):
    return oracle.decode(workload(name))


@functools.lru_cache(maxsize=2)
def device(name):
    return DeviceWorkload(workload(name))


@pytest.fixture(scope="module")
def counters():
    return new_counters()


def check_counters_zero(cnt):
    assert int(cnt.abs().sum().item()) == 0, "merge counters not restored to zero"


def gate(name, dw, splits, cnt, ref):
    say(f"[gpu] {name} splits={splits}")
    fused = dw.host(dw.run(splits, counters=cnt))
    check_counters_zero(cnt)
    sep = dw.host(dw.run(splits, counters=None))
    assert np.array_equal(fused, sep), f"{name}: fused merge != separate combine at splits={splits}"
    whole, worst, at = per_head(fused, ref)
    say(f"[gpu] {name} splits={splits} rel_rms={whole:.3e} worst (row, head) {at}: {worst:.3e}")
    assert worst < TOL, (name, splits, "worst (row, head)", at, worst)
    return fused


@pytest.mark.parametrize("splits", [1, 4])
def test_c1_tiny(counters, splits):
    gate("C1", device("C1"), splits, counters, reference("C1"))


@pytest.mark.parametrize("name", ["PA", "PB", "C2"])
def test_page_configs_and_page_map(counters, name):
    dw = device(name)
    s = dw.heuristic_splits()
    a = gate(name, dw, s, counters, reference(name))
    wm = workloads.with_page_map(workload(name))
    dm = DeviceWorkload(wm)
    say(f"[gpu] {name}+pagemap splits={s}")
    b = dm.host(dm.run(s, counters=counters))
    check_counters_zero(counters)
    assert np.array_equal(a, b), f"{name}: page-map pool differs"
    for s2 in (1, 3, 16):
        x = dw.host(dw.run(s2, counters=counters))
        y = dm.host(dm.run(s2, counters=counters))
        assert np.array_equal(x, y), (name, s2)
        assert per_head(x, reference(name))[1] < TOL


def test_c3_global_wide_head(counters):
    """The heuristic's 128 splits (per-wave kernel at hd 512) and 32 (below
    64 splits the shared-page kernel takes hd 512); a permuted pool behind a
    page map gives the same bits in both."""
    dw = device("C3")
    s_h = dw.heuristic_splits()
    gate("C3", dw, s_h, counters, reference("C3"))
    gate("C3", dw, 32, counters, reference("C3"))
    dm = DeviceWorkload(workloads.with_page_map(workload("C3")))
    for s in (32, s_h):
        for cnt in (counters, None):
            a = dw.host(dw.run(s, counters=cnt))
            b = dm.host(dm.run(s, counters=cnt))
            assert np.array_equal(a, b), ("C3 page map", s, cnt is None)
    check_counters_zero(counters)


@pytest.mark.parametrize("name", ["C4", "C4NAN"])
def test_c4_batched(counters, name):
    dw = device(name)
    s = dw.heuristic_splits(rows_per_seq=1)
    ref = reference("C4")  # NaN tails are outside every window: same answer
    gate(name, dw, s, counters, ref)
    if s != 3:
        gate(name, dw, 3, counters, ref)


@pytest.mark.parametrize("name", ["C5W0", "C5W4096"])
def test_c5_long_multirow_split_sweep(counters, name):
    dw = device(name)
    ref = reference(name)
    s_h = dw.heuristic_splits()
    gate(name, dw, s_h, counters, ref)
    say(f"[gpu] {name} sweeping splits 1..256")
    for s in range(1, 257):
        fused = dw.host(dw.run(s, counters=counters))
        sep = dw.host(dw.run(s, counters=None))
        assert np.array_equal(fused, sep), (name, s)
        if s in (1, 2, 7, 64, 255, 256):
            assert per_head(fused, ref)[1] < TOL, (name, s)
    check_counters_zero(counters)
    if name == "C5W4096":
        dm = DeviceWorkload(workloads.with_page_map(workload(name)))
        for s in (1, s_h, 256):
            a = dw.host(dw.run(s, counters=counters))
            b = dm.host(dm.run(s, counters=counters))
            assert np.array_equal(a, b), ("page map", s)


@pytest.mark.parametrize("name,splits", [("PA", 1), ("PA", 2), ("PA", 7), ("PA", 64), ("C3", 7), ("C3", 64),
                                         ("C3", 128), ("C5W0", 1), ("C5W0", 256)])
def test_single_visible_key_is_exact(counters, name, splits):
    """window = 1: the output is the V row of the query position, bit for bit,
    in both merge modes (per-wave kernel: PA, and C3 from 64 splits;
    shared-page kernel: C3 below 64 splits, C5)."""
    w = workload(name).replace(window=1)
    dw = DeviceWorkload(w)
    g = w.nh // w.nkv
    for cnt in (counters, None):
        out = dw.host(dw.run(splits, counters=cnt))
        for t in range(w.rows):
            p = int(w.qpos[t])
            for h in range(w.nh):
                assert np.array_equal(out[t, h], w.v_pool[int(w.block_table[p // 16]), h // g, p % 16]), \
                    (name, splits, t, h)
    check_counters_zero(counters)


def bf16_within_one_ulp(a, b):
    """bf16 bit patterns a and b are equal or adjacent values of one sign."""
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    same_sign = (a >> 15) == (b >> 15)
    return bool(np.all(same_sign & (np.abs(a - b) <= 1)))


@pytest.mark.parametrize("name,splits", [("PA", 8), ("C3", 32), ("C3", 128), ("C5W0", 256), ("C4", 3)])
def test_constant_v_returns_that_row(counters, name, splits):
    """Every key of a kv head carries the same V row: the softmax weights sum
    to one, so every head of the group returns that row, whatever the scores
    (checked to within one bf16 ulp: the weighted sum is rounded in f32)."""
    w = workload(name)
    rng = np.random.default_rng(2024)
    vals = rng.uniform(0.25, 1.0, size=(w.nkv, w.hd)) * rng.choice([-1.0, 1.0], size=(w.nkv, w.hd))
    vrow = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    v = np.ascontiguousarray(np.broadcast_to(vrow[None, :, None, :], w.v_pool.shape))
    dw = DeviceWorkload(w.replace(v_pool=v))
    g = w.nh // w.nkv
    expect = np.broadcast_to(vrow[np.arange(w.nh) // g][None], (w.rows, w.nh, w.hd))
    for cnt in (counters, None):
        out = dw.host(dw.run(splits, counters=cnt))
        assert bf16_within_one_ulp(out, expect), (name, splits, cnt is None)
    check_counters_zero(counters)


def edge_workloads():
    rng_seq = workloads.single_sequence
    cases = []
    # rows of several sequences: runs of equal origin cut by origin changes and
    # by the tile size, distinct positions inside a run, ragged row count
    b = workloads.batched("mixed", nseq=4, lmin=40, lmax=300, nh=8, nkv=2, hd=128, pad=16)
    seq = np.array([0, 0, 1, 2, 2, 2, 2, 2, 3])
    back = np.array([1, 0, 0, 4, 3, 2, 1, 0, 0])
    qp = (b.qpos[seq] - back).astype(np.int32)
    cases.append(b.replace(name="mixed", rows=len(seq), q=np.concatenate([b.q, b.q, b.q])[:len(seq)],
                           page_origin=b.page_origin[seq].copy(), qpos=qp, kv_last=qp.copy()))
    # a large launch of multi-row tiles (16 sequences x 4 rows, MHA): with 5
    # splits it is big enough for the per-wave kernel to take rows longest first
    r = workloads.batched("ranked", nseq=16, lmin=20, lmax=3000, nh=8, nkv=8, hd=64, pad=16)
    seq = np.repeat(np.arange(16), 4)
    back = np.tile(np.arange(3, -1, -1), 16)
    qp = (r.qpos[seq] - back).astype(np.int32)
    rq = np.random.default_rng(3).standard_normal((len(seq), r.nh, r.hd)).astype(np.float32)
    rq = (rq.view(np.uint32) >> 16).astype(np.uint16)
    cases.append(r.replace(name="ranked", rows=len(seq), q=rq, page_origin=r.page_origin[seq].copy(),
                           qpos=qp, kv_last=qp.copy()))
    # wide group (32 heads per kv head -> two head blocks), nkv=1
    cases.append(rng_seq("g32", ctx=333, rows=2, nh=32, nkv=1, hd=64, window=0))
    # plain MHA (group 1): 16 rows share each page
    cases.append(rng_seq("mha", ctx=257, rows=19, nh=4, nkv=4, hd=128, window=100))
    # window larger than the context, partial first page, hd 512, 3 rows (group 8 -> 2 per tile)
    cases.append(rng_seq("wbig", ctx=181, rows=3, nh=16, nkv=2, hd=512, window=5000))
    # rows whose last visible key is below the query position (second position array)
    w2 = rng_seq("kvlast", ctx=500, rows=4, nh=8, nkv=2, hd=256, window=0)
    cases.append(w2.replace(name="kvlast", kv_last=np.array([100, 499, 300, 498], np.int32)))
    # shared-page kernel shapes: hd split in 2 slices (group 8, 3 rows, hd 128);
    # 64-column tiles with a ragged last tile (group 16, 5 rows; hd 512, 9 rows);
    # a group wider than a tile (128 heads -> two head blocks of 64)
    cases.append(rng_seq("sh128s2", ctx=300, rows=3, nh=16, nkv=2, hd=128, window=0))
    cases.append(rng_seq("sh128s1", ctx=400, rows=5, nh=16, nkv=1, hd=128, window=77))
    cases.append(rng_seq("sh512s1", ctx=150, rows=9, nh=8, nkv=1, hd=512, window=0))
    cases.append(rng_seq("sh256g128", ctx=260, rows=2, nh=128, nkv=1, hd=256, window=0))
    # block decode (non-causal inside the block): rows at positions 396..399
    # all see keys up to 403, with and without a window anchored at qpos
    for nm, win in (("block", 0), ("blockwin", 50)):
        wb = rng_seq(nm, ctx=404, rows=4, nh=8, nkv=2, hd=128, window=win)
        qb = np.arange(396, 400, dtype=np.int32)
        cases.append(wb.replace(name=nm, qpos=qb, kv_last=np.full(4, 403, np.int32)))
    # an empty visible set (last key below the window start) -> zeros
    w3 = rng_seq("empty", ctx=200, rows=2, nh=4, nkv=1, hd=64, window=8)
    cases.append(w3.replace(name="empty", kv_last=np.array([150, 199], np.int32)))
    return cases


@pytest.mark.parametrize("w", edge_workloads(), ids=lambda w: w.name)
def test_edge_cases(counters, w):
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    ctx = int(w.kv_last.max()) + 1
    pages = (ctx + 15) // 16
    for s in sorted({1, 2, 5, min(256, pages + 3)}):
        gate(w.name, dw, s, counters, ref)
    if w.name == "empty":
        out = dw.host(dw.run(4, counters=counters))
        assert not out[0].any()


def merge_layout_workloads():
    """Fused calls whose merge runs in parallel (64 KB or more of partials per
    merge unit) in other shapes than C3's and C5's: 300 units of 4 rows (hd
    512, group 8; shared-page kernel) in a launch larger than the device
    holds at once, so units complete one after another while their waiting
    workgroups hold CUs; units of one column (MHA, hd 512) with fewer blocks
    than workgroups; 4 units of 8 columns (2 rows x group 4, hd 512) in the
    hd-sliced kernel; and a batch of 8 sequences at hd 512, group 2, in the
    hd-sliced kernel (16 units, rows ranked from the scalar-cache metadata,
    several rounds of workgroups while earlier units wait for their merges).
    Split counts that are not powers of two are included; each tile uses
    pgqa_tile_splits of them."""
    rng_seq = workloads.single_sequence
    return [(rng_seq("units300", ctx=1200, rows=300, nh=8, nkv=1, hd=512, window=0), (32, 37, 64)),
            (rng_seq("col1", ctx=2000, rows=1, nh=2, nkv=2, hd=512, window=0), (64, 100, 125)),
            (rng_seq("g4x2", ctx=2100, rows=2, nh=16, nkv=4, hd=512, window=0), (32, 64, 131)),
            (workloads.batched("b512", nseq=8, lmin=600, lmax=3000, nh=4, nkv=2, hd=512, pad=16), (64, 100))]


@pytest.mark.parametrize("w,splits", merge_layout_workloads(), ids=lambda x: getattr(x, "name", None))
def test_parallel_merge_layouts(counters, w, splits):
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    for s in splits:
        gate(w.name, dw, s, counters, ref)


def test_counter_capacity_refusal():
    import paged_gqa_decode_attn_amd as pg
    w = workloads.single_sequence("cap", ctx=4200, rows=4097, nh=1, nkv=1, hd=64, window=0)
    dw = DeviceWorkload(w)
    with pytest.raises(pg.PgqaError) as ei:
        dw.run(2, counters=new_counters())
    assert ei.value.code == pg.ECAP


def test_counter_capacity_full(counters):
    """The largest fused call the counter buffer holds: 4096 rows x 1 kv head
    (one merge unit per row) uses every counter; fused == separate bit for
    bit, within the bound, counters zero afterwards."""
    w = workloads.single_sequence("capfull", ctx=4200, rows=4096, nh=1, nkv=1, hd=64, window=300)
    dw = DeviceWorkload(w)
    ref = oracle.decode(w)
    gate("capfull", dw, 3, counters, ref)


@pytest.mark.parametrize("name,splits", [("C3", 128), ("C5W0", 256), ("C5W4096", 64)])
def test_fused_merge_when_waiters_give_up(counters, name, splits):
    """The parallel fused merge with every wait bounded at one tick: the
    waiting workgroups leave almost at once and the last arrival merges what
    nobody took.  Same bits as the separate combine, counters back at zero,
    and the default bound restored afterwards."""
    import paged_gqa_decode_attn_amd as pg
    dw = device(name)
    sep = dw.host(dw.run(splits, counters=None))
    prev = pg.set_merge_wait_ticks(1)
    try:
        for _ in range(2):
            say(f"[gpu] {name} splits={splits} fused, waits of one tick")
            fused = dw.host(dw.run(splits, counters=counters))
            check_counters_zero(counters)
            assert np.array_equal(fused, sep), (name, splits)
    finally:
        pg.set_merge_wait_ticks(prev)
    assert per_head(sep, reference(name))[1] < TOL


@pytest.mark.parametrize("name,splits", [("C4", 16), ("C5W4096", 256), ("PA", 64), ("C3", 256)])
def test_tile_split_counts(name, splits):
    """Each tile works on pgqa_tile_splits(its pages, S) of the S splits: in
    the separate form, (row, head) slots below that count hold a split with
    visible keys (l > 0) and the others the empty (m, l) = (-inf, 0).  Each
    sequence here is one tile (its rows fit one tile of the call's plan)."""
    import paged_gqa_decode_attn_amd as pg
    w, dw = workload(name), device(name)
    part = torch.empty(pg.decode_part_bytes(w.rows, w.nh, splits, w.hd), dtype=torch.uint8, device="cuda")
    say(f"[gpu] {name} splits={splits}: partial slots")
    dw.run(splits, counters=None, part=part)
    ml = part.view(torch.float32)[w.rows * w.nh * splits * w.hd:].view(w.rows, w.nh, splits, 2).cpu().numpy()
    rr = workloads.row_ranges(w)
    lo = np.array([r[0] for r in rr])
    hi = np.array([r[1] for r in rr])
    for org in np.unique(w.page_origin):
        rows = np.flatnonzero(w.page_origin == org)
        assert np.all(np.diff(rows) == 1) and len(rows) <= 8
        pages = int(hi[rows].max()) // 16 - int(lo[rows].min()) // 16 + 1
        st = pg.tile_splits(pages, splits)
        assert 1 <= st <= splits
        used = ml[rows][:, :, :st]
        assert np.all(used[..., 1] > 0), (name, org, st)
        empty = ml[rows][:, :, st:]
        assert np.all(np.isneginf(empty[..., 0])) and np.all(empty[..., 1] == 0), (name, org, st)
