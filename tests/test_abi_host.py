"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every declared entry point; the split heuristic, buffer sizing and
refusals behave as documented in include/pgqa.h.  Refused calls return before
anything touches the HIP runtime, so they are safe without a device."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import paged_gqa_decode_attn_amd as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pgqa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pgqa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"pgqa_attn_decode", "pgqa_choose_splits", "pgqa_decode_part_bytes",
            "pgqa_counter_capacity", "pgqa_last_error", "pgqa_attn_prefill", "pgqa_make_tiles",
            "pgqa_prefill_rows_per_tile", "pgqa_qk_rope_prep", "pgqa_set_merge_wait_ticks",
            "pgqa_set_narrow_path", "pgqa_choose_splits_heads",
            "pgqa_attn_decode_noalloc", "pgqa_tile_splits"} <= set(names)
    h = ctypes.CDLL(pg.LIB_PATH)
    for n in names:
        assert getattr(h, n, None) is not None, n


def test_counter_capacity():
    assert pg.counter_capacity() == 4096


def test_part_bytes_formula():
    assert pg.decode_part_bytes(5, 16, 7, 256) == 5 * 16 * 7 * 258 * 4
    assert pg.decode_part_bytes(1, 16, 256, 512) == 16 * 256 * 514 * 4
    assert pg.decode_part_bytes(0, 16, 4, 64) == 0
    assert pg.decode_part_bytes(1, 1, 0, 64) == 0


def test_tile_splits_rule():
    """Splits a tile works on: ceil(pages / 4), at least 1, at most S (S
    clamped to 256); every count pgqa_choose_splits gives a one-sequence call
    is kept (it never gives fewer than 4 pages per split)."""
    for pages in (0, 1, 3, 4, 5, 16, 17, 32, 33, 240, 241, 1024, 1025, 4096, 1 << 20):
        for s in (1, 2, 3, 8, 16, 128, 256, 1000):
            want = max(1, min(min(s, 256), -(-pages // 4)))
            assert pg.tile_splits(pages, s) == want, (pages, s)
    assert pg.tile_splits(100, 0) == 1 and pg.tile_splits(-5, 8) == 1


def test_tile_splits_keep_the_heuristic_counts():
    for span in (16, 64, 700, 1024, 4096, 16384, 32768, 131072):
        for rows, nkv in ((1, 1), (1, 2), (4, 8), (8, 1), (5, 8)):
            s = pg.choose_splits(span, rows, nkv, rows)
            assert pg.tile_splits(-(-span // 16), s) == s, (span, rows, nkv, s)


def test_choose_splits_range_and_determinism():
    for span in (1, 16, 64, 700, 1024, 4096, 32768, 131072, 1 << 20):
        for rows in (1, 4, 8, 64, 512):
            for nkv in (1, 2, 8):
                for rps in (1, rows):
                    s = pg.choose_splits(span, rows, nkv, rps)
                    assert 1 <= s <= 256
                    assert s == pg.choose_splits(span, rows, nkv, rps)
                    # never more splits than pages
                    assert s <= max(1, (span + 15) // 16)
    # degenerate arguments fall back to one split
    assert pg.choose_splits(0, 1, 1, 1) == 1
    assert pg.choose_splits(100, 0, 1, 1) == 1
    # a long single sequence gets many splits, a big batch few
    assert pg.choose_splits(32768, 1, 2, 1) >= 64
    assert pg.choose_splits(16384, 64, 8, 1) <= 4


def test_choose_splits_on_the_measured_shapes():
    """The split counts the sweeps found fastest (or within a few percent):
    every target configuration, one-sequence calls at one workgroup per CU,
    and batches of 4 to 64 sequences."""
    # (kv_span, rows, nkv, rows_per_seq) -> splits
    cases = {
        (64, 1, 1, 1): 1,          # tiny decode
        (1024, 4, 8, 4): 8,        # local sliding layer, window 1024
        (32768, 1, 2, 1): 128,     # global layer, wide head (hd 512)
        (16384, 64, 8, 1): 3,      # batched decode, 64 sequences
        (131072, 8, 1, 8): 256,    # long multi-row, window 0
        (4096, 8, 1, 8): 64,       # long multi-row, window 4096
        (1024, 5, 8, 5): 8,        # the page's first parity shape
        (700, 1, 2, 1): 11,        # the page's second parity shape
        (16384, 1, 2, 1): 128,     # one row, hd 512, 16K: 31.6 us against 36.9 at 64
        (65536, 1, 2, 1): 128,     # one row, hd 512, 64K: 58.7 us against 72.0 at 256
        (32768, 1, 8, 1): 32,      # one row, hd 128, 8 kv heads: 34.8 us against 48.3 at 128
        (16384, 8, 1, 8): 128,     # 8 rows x 8 heads, 16K: 28.4 us against 29.6 at 64
        (16003, 4, 8, 1): 16,      # batch of 4: 37.8 us against 63.0 at 48
        (16384, 8, 8, 1): 16,      # batch of 8: 71.1 / 67.3 us against 72.8 / 70.9 at 12
        (16384, 16, 8, 1): 8,      # batch of 16: 115.8 / 114.1 us against 121.6 / 117.6 at 12
        (16384, 32, 8, 1): 4,      # batch of 32: 202.4 / 203.5 us against 206.9 / 205.1 at 6
        (16384, 32, 32, 1): 2,     # batch of 32, one head per kv head: 729.2 against 737.9 us at 1
    }
    for args, want in cases.items():
        assert pg.choose_splits(*args) == want, (args, pg.choose_splits(*args), want)


FAKE = 0x10000  # never dereferenced: every call below is refused first


def call(**kw):
    a = dict(out=FAKE, part=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, off=FAKE, qpos=FAKE,
             last=FAKE, rows=1, nh=4, nkv=1, hd=64, window=0, splits=1, cnt=None, pmap=None)
    a.update(kw)
    return pg.lib().pgqa_attn_decode(a["out"], a["part"], a["q"], a["k"], a["v"], a["bt"],
                                     a["off"], a["qpos"], a["last"], a["rows"], a["nh"],
                                     a["nkv"], a["hd"], a["window"], a["splits"], a["cnt"],
                                     a["pmap"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), pg.EINVAL),
    (dict(q=None), pg.EINVAL),
    (dict(k=None), pg.EINVAL),
    (dict(v=None), pg.EINVAL),
    (dict(bt=None), pg.EINVAL),
    (dict(off=None), pg.EINVAL),
    (dict(qpos=None), pg.EINVAL),
    (dict(last=None), pg.EINVAL),
    (dict(rows=0), pg.EINVAL),
    (dict(nh=6, nkv=4), pg.EINVAL),
    (dict(nkv=0), pg.EINVAL),
    (dict(hd=96), pg.EINVAL),
    (dict(hd=1024), pg.EINVAL),
    (dict(window=-1), pg.EINVAL),
    (dict(splits=0), pg.EINVAL),
    (dict(splits=257), pg.EINVAL),
    (dict(splits=4, part=None), pg.EINVAL),
    (dict(q=FAKE + 8), pg.EINVAL),
    (dict(splits=4, part=FAKE + 2), pg.EINVAL),
    (dict(rows=4097, nkv=1, splits=2, cnt=FAKE), pg.ECAP),
    (dict(rows=600, nh=64, nkv=8, splits=2, cnt=FAKE), pg.ECAP),
    # decode grid: 2^20 rows x 256 splits = 2^28 workgroups of 256 threads
    (dict(rows=1 << 20, nh=1, nkv=1, hd=64, splits=256), pg.EINVAL),
    # combine grid: 2^16 rows x 64 heads x 16 chunks = 2^26 workgroups of 256
    # threads, with a decode grid that fits
    (dict(rows=1 << 16, nh=64, nkv=64, hd=512, splits=2), pg.EINVAL),
])
def test_refusals(kw, code):
    assert call(**kw) == code
    assert pg.last_error() != ""


def test_large_grids_that_fit_are_not_refused_for_their_size():
    """The grid checks refuse nothing that fits: the fused form of the
    combine-grid case above needs no combine launch.  (Checked through the
    error text only: refused before launch for another reason.)"""
    rc = call(rows=1 << 16, nh=64, nkv=64, hd=512, splits=2, cnt=FAKE)
    assert rc == pg.ECAP and "grid" not in pg.last_error()


def test_noalloc_scratch_size_and_refusals():
    """The allocation-free entry point refuses partials beyond its scratch
    before it looks the scratch up (no HIP call), overflowing products
    included; the Python constant is the header's."""
    text = open(os.path.join(ROOT, "include", "pgqa.h")).read()
    m = re.search(r"#define PGQA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pg.NOALLOC_SCRATCH_BYTES
    f = pg.lib().pgqa_attn_decode_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64] * 6 + [ctypes.c_void_p] * 2
    # 16 heads x 256 splits x hd 512 is 8.4 MB a row: 4 rows exceed 32 MiB
    assert pg.decode_part_bytes(4, 16, 256, 512) > pg.NOALLOC_SCRATCH_BYTES
    for rows, nh, nkv, hd, splits in ((4, 16, 2, 512, 256), ((1 << 30) - 1, 65536, 1, 512, 256)):
        assert f(*[FAKE] * 8, rows, nh, nkv, hd, 0, splits, None, None) == pg.EINVAL
        assert "scratch" in pg.last_error()
    assert f(None, *[FAKE] * 7, 1, 4, 1, 64, 0, 2, None, None) == pg.EINVAL


def test_merge_wait_ticks_hook():
    prev = pg.set_merge_wait_ticks(7)
    try:
        assert pg.set_merge_wait_ticks(1) == 7
        with pytest.raises(pg.PgqaError):
            pg.set_merge_wait_ticks(-1)
    finally:
        pg.set_merge_wait_ticks(prev)


def test_narrow_path_hook():
    prev = pg.set_narrow_path(1)
    try:
        assert pg.set_narrow_path(2) == 1
        assert pg.set_narrow_path(0) == 2
        for bad in (-1, 3):
            with pytest.raises(pg.PgqaError):
                pg.set_narrow_path(bad)
        assert pg.set_narrow_path(0) == 0
    finally:
        pg.set_narrow_path(prev)


def test_library_loads_after_torch():
    """The library binds to torch's HIP runtime: loading it imports torch
    first (a fresh interpreter that touches only a host entry point)."""
    code = ("import sys, paged_gqa_decode_attn_amd as pg; assert 'torch' not in sys.modules; "
            "pg.choose_splits(4096, 1, 1, 1); print('torch' in sys.modules)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("True")


def test_missing_library_is_loud(tmp_path, monkeypatch):
    monkeypatch.setattr(pg, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(pg, "_lib", None)
    with pytest.raises(pg.PgqaError):
        pg.lib()


# ---- prefill (host side) ----

def test_prefill_rows_per_tile():
    for hd in (64, 128, 256, 512):
        assert pg.prefill_rows_per_tile(hd) == 64
    assert pg.prefill_rows_per_tile(96) == 0


def brute_tiles(origins, rpt):
    t0, tn = [], []
    r = 0
    while r < len(origins):
        e = r + 1
        while e < len(origins) and e - r < rpt and origins[e] == origins[r]:
            e += 1
        t0.append(r)
        tn.append(e - r)
        r = e
    return t0, tn


@pytest.mark.parametrize("origins,rpt", [
    ([0] * 200, 64),                       # one sequence: full tiles and a ragged one
    ([0] * 64, 64),                        # exactly one tile
    ([3], 64),                             # one row
    ([0, 0, 5, 5, 5, 9, 0, 0], 2),         # runs cut by origin changes and by size
    ([7] * 10 + [20] * 130 + [1] * 3, 64),
])
def test_make_tiles(origins, rpt):
    t0, tn = pg.make_tiles(origins, rpt)
    bt0, btn = brute_tiles(origins, rpt)
    assert t0.tolist() == bt0 and tn.tolist() == btn
    # the tiles cover every row once, and each tile keeps one origin
    covered = [r for a, n in zip(t0, tn) for r in range(a, a + n)]
    assert covered == list(range(len(origins)))
    for a, n in zip(t0, tn):
        assert len(set(origins[a:a + n])) == 1 and 1 <= n <= rpt


def test_make_tiles_refusals():
    import numpy as np
    org = np.zeros(10, np.int32)
    t0 = np.zeros(2, np.int32)
    tn = np.zeros(2, np.int32)
    assert pg.lib().pgqa_make_tiles(org.ctypes.data, 10, 4, t0.ctypes.data, tn.ctypes.data, 2) == pg.ECAP
    assert pg.lib().pgqa_make_tiles(org.ctypes.data, 10, 0, t0.ctypes.data, tn.ctypes.data, 2) == pg.EINVAL
    assert pg.lib().pgqa_make_tiles(org.ctypes.data, 10, 65, t0.ctypes.data, tn.ctypes.data, 2) == pg.EINVAL
    assert pg.lib().pgqa_make_tiles(None, 10, 4, t0.ctypes.data, tn.ctypes.data, 2) == pg.EINVAL


def pcall(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, off=FAKE, qpos=FAKE, last=FAKE, t0=FAKE,
             tn=FAKE, ntiles=1, rows=1, nh=4, nkv=1, hd=64, window=0, pmap=None)
    a.update(kw)
    return pg.lib().pgqa_attn_prefill(a["out"], a["q"], a["k"], a["v"], a["bt"], a["off"], a["qpos"],
                                      a["last"], a["t0"], a["tn"], a["ntiles"], a["rows"], a["nh"],
                                      a["nkv"], a["hd"], a["window"], a["pmap"], None)


@pytest.mark.parametrize("kw", [
    dict(out=None), dict(q=None), dict(t0=None), dict(tn=None), dict(last=None),
    dict(rows=0), dict(ntiles=0), dict(ntiles=2, rows=1), dict(nh=6, nkv=4), dict(hd=32),
    dict(window=-1), dict(k=FAKE + 4),
])
def test_prefill_refusals(kw):
    assert pcall(**kw) == pg.EINVAL
    assert pg.last_error() != ""


def rcall(**kw):
    a = dict(qo=FAKE, kp=FAKE, vp=FAKE, qi=FAKE, ki=FAKE, vi=None, qw=None, kw=None, cos=FAKE, sin=FAKE,
             pos=FAKE, bt=FAKE, off=FAKE, pmap=None, tokens=1, nh=4, nkv=1, hd=64, rd=64, eps=1e-6)
    a.update(kw)
    return pg.lib().pgqa_qk_rope_prep(a["qo"], a["kp"], a["vp"], a["qi"], a["ki"], a["vi"], a["qw"], a["kw"],
                                      a["cos"], a["sin"], a["pos"], a["bt"], a["off"], a["pmap"], a["tokens"],
                                      a["nh"], a["nkv"], a["hd"], a["rd"], a["eps"], None)


@pytest.mark.parametrize("kw", [
    dict(qo=None), dict(kp=None), dict(vp=None), dict(qi=None), dict(ki=None), dict(pos=None),
    dict(bt=None), dict(off=None), dict(cos=None), dict(sin=None), dict(tokens=-1), dict(nh=0),
    dict(nkv=0), dict(hd=96), dict(hd=1024), dict(rd=8), dict(rd=80), dict(rd=-16),
    dict(eps=-1.0), dict(eps=float("nan")), dict(eps=float("inf")), dict(qi=FAKE + 2),
    dict(vi=FAKE + 8), dict(qw=FAKE + 2), dict(cos=FAKE + 4), dict(kp=FAKE + 2),
])
def test_prep_refusals(kw):
    assert rcall(**kw) == pg.EINVAL
    assert pg.last_error() != ""


def test_prep_accepts_without_launch():
    # no tokens: nothing to enqueue (no device needed); no rotation: no tables needed
    assert rcall(tokens=0) == pg.OK
    assert rcall(tokens=0, rd=0, cos=None, sin=None) == pg.OK
    assert pg.last_error() == ""


def test_read_probe_refuses_bad_patterns():
    """The benchmark's streaming-read probe checks its arguments before it
    launches anything: a pattern outside 0..2, a buffer that is not whole 4 KB
    blocks or not 16-byte aligned, and scattered or paired patterns whose
    block count is not a power of two divisible by the grid are refused."""
    path = os.path.join(ROOT, "paged_gqa_decode_attn_amd", "libpgqa_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    h = ctypes.CDLL(path)
    f = h.pgqa_probe_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    buf, sink = 1 << 20, 1 << 21  # never dereferenced: every call below is refused first
    assert f(buf, 1 << 20, 16, 8, 3, sink, None) == -1   # no such pattern
    assert f(buf, 1 << 20, 16, 8, -1, sink, None) == -1
    assert f(buf, 5000, 1, 8, 0, sink, None) == -1       # not whole 4 KB blocks
    assert f(buf + 8, 1 << 20, 16, 8, 0, sink, None) == -1  # misaligned
    assert f(buf, 4096 * 3, 1, 8, 1, sink, None) == -1   # 3 blocks: not a power of two
    assert f(buf, 4096 * 3, 1, 8, 2, sink, None) == -1
    assert f(buf, 4096, 1, 8, 2, sink, None) == -1       # paired needs two blocks at least
    assert f(buf, 1 << 20, 3, 8, 2, sink, None) == -1    # 256 blocks not divisible by 3 workgroups
    assert f(buf, 1 << 20, 16, 3, 0, sink, None) == -1   # unroll 3 not built


def test_choose_splits_heads():
    """The head-aware count: batches whose tiles take the shared-page kernel
    (more than 16 query heads per kv head from hd 128) aim at one round of
    256 workgroups below 64 units and two rounds from 64, the counts measured
    best on batches with lengths 512..16384 (separate and fused merge);
    everything else keeps pgqa_choose_splits's count."""
    span = 16384
    for nseq, nh, nkv, hd, want in [(8, 32, 1, 128, 16), (16, 32, 1, 128, 16), (32, 32, 1, 128, 8),
                                    (64, 32, 1, 128, 8), (128, 32, 1, 128, 4), (32, 32, 1, 256, 8),
                                    (64, 32, 1, 256, 8), (16, 64, 2, 128, 8), (64, 64, 2, 128, 4),
                                    (256, 32, 1, 128, 2), (512, 32, 1, 128, 1)]:
        assert pg.choose_splits_heads(span, nseq, nh, nkv, hd, 1) == want, (nseq, nh, nkv, hd)
    # other kernels, one sequence, refused arguments: the plain count
    for span, rows, nh, nkv, hd, rps in [(16384, 64, 32, 8, 128, 1), (16384, 64, 32, 2, 128, 1),
                                         (16384, 64, 64, 1, 64, 1), (32768, 1, 16, 2, 512, 1),
                                         (131072, 8, 8, 1, 256, 8), (131072, 8, 64, 1, 128, 8),
                                         (4096, 4, 16, 8, 256, 4), (16384, 64, 33, 2, 128, 1),
                                         (16384, 64, 32, 1, 96, 1)]:
        assert pg.choose_splits_heads(span, rows, nh, nkv, hd, rps) == pg.choose_splits(span, rows, nkv, rps)
    # a short span keeps the short-span floor; degenerate input gives 1
    assert pg.choose_splits_heads(256, 64, 32, 1, 128, 1) == pg.choose_splits(256, 64, 1, 1)
    assert pg.choose_splits_heads(0, 1, 1, 1, 128, 1) == 1
    for span in (1, 17, 5000, 1 << 20):
        for nseq in (2, 3, 300, 5000):
            s = pg.choose_splits_heads(span, nseq, 48, 1, 256, 1)
            assert 1 <= s <= 256 and s == pg.choose_splits_heads(span, nseq, 48, 1, 256, 1)
            if nseq * 16 >= 64:  # no short-span floor above the round's count
                assert s <= 16
