"""Pins for the CPU oracle: it is checked against things other than itself.

* an arbitrary-precision brute force on tiny inputs, written from the visibility
  rule and softmax definition directly (``tests/brute.py``), over logical arrays
  that the test scatters into permuted pools with origins and page maps;
* closed forms (two keys with a known score gap; equal keys give the mean of V;
  one visible key returns that V row bit for bit);
* invariants of the definition (window 0 == a window covering everything; GQA
  group == separate single-head runs on the right kv head; permuting keys with
  their values; identity pool == permuted pool behind a page map);
* the bf16 rounding and the rel-RMS metric against hand-derived values.

Each was chosen so that a plausible slip in the oracle -- a dropped 1/z, a
1/sqrt(hd) scale, a window off by one, ``h % nkv`` for the kv head, a wrong
slot or page index, a transposed pool -- fails at least one of them.
"""
import math
import struct

import mpmath
import numpy as np
import pytest

import oracle
import workloads
from tests import brute

mpmath.mp.dps = 50


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_of_f32(x):
    """bf16 bits of a float that is exactly representable in bf16."""
    b = f32_bits(x)
    assert b & 0xFFFF == 0
    return b >> 16


def bf16_to_float(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def mp_to_bf16(x):
    """Round an mpf to bf16 (nearest even); also return the distance of the
    scaled value from a rounding tie, so callers can skip near-tie cases."""
    if x == 0:
        return 0, 1.0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = int(mpmath.floor(mpmath.log(a, 2)))
    # guard against log rounding at exact powers of two
    if mpmath.mpf(2) ** e > a:
        e -= 1
    if mpmath.mpf(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = mpmath.mpf(2) ** (e - 7)
    qv = a / ulp
    f = mpmath.floor(qv)
    r = qv - f
    n = int(f)
    if r > 0.5 or (r == 0.5 and n % 2 == 1):
        n += 1
    y = float(n * ulp)
    return sign | bf16_of_f32(y), float(abs(r - 0.5))


# --------------------------------------------------------------------------
# helpers that scatter logical data into pools (test-local, independent of the
# oracle's addressing code)
# --------------------------------------------------------------------------

def random_bits(rng, shape, lo=-1.0, hi=1.0):
    x = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def scatter_pool(seq_k, seq_v, nkv, hd, rng, pad=3):
    """seq_k[s]: [ctx_s][nkv][hd] bits.  Returns (k_pool, v_pool, table, origins)
    with a NaN null page 0, random physical placement and ``pad`` leading table
    entries that point at the null page."""
    pages = [(len(k) + 15) // 16 for k in seq_k]
    total = sum(pages)
    phys = rng.permutation(np.arange(1, total + 1))
    kp = np.full((total + 1, nkv, 16, hd), workloads.BF16_QNAN, np.uint16)
    vp = np.full((total + 1, nkv, 16, hd), workloads.BF16_QNAN, np.uint16)
    table = [0] * pad
    origins = []
    at = 0
    for s, (ks, vs) in enumerate(zip(seq_k, seq_v)):
        origins.append(len(table))
        for lp in range(pages[s]):
            pp = int(phys[at])
            at += 1
            table.append(pp)
            for slot in range(16):
                p = lp * 16 + slot
                if p < len(ks):
                    kp[pp, :, slot, :] = ks[p]
                    vp[pp, :, slot, :] = vs[p]
    return kp, vp, np.array(table, np.int32), np.array(origins, np.int32)


def brute_case(q, seq_k, seq_v, seq_of_row, qpos, last, nh, nkv, window):
    rows = q.shape[0]
    g = nh // nkv
    out = []
    for t in range(rows):
        s = seq_of_row[t]
        per_h = []
        for h in range(nh):
            kh = h // g
            kk = [seq_k[s][p][kh] for p in range(len(seq_k[s]))]
            vv = [seq_v[s][p][kh] for p in range(len(seq_v[s]))]
            per_h.append(brute.attend(q[t, h], kk, vv, int(qpos[t]), int(last[t]), window))
        out.append(per_h)
    return out


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 2, 15, 16, 17, 40, 53])
def test_brute_force_paged_multi_sequence(window):
    rng = np.random.default_rng(1000 + window)
    nh, nkv, hd = 4, 2, 8
    ctxs = [48, 33, 17]
    seq_k = [random_bits(rng, (c, nkv, hd), -2, 2) for c in ctxs]
    seq_v = [random_bits(rng, (c, nkv, hd)) for c in ctxs]
    # rows: two on sequence 0 (positions 46, 47), one on each other sequence
    seq_of_row = [0, 0, 1, 2]
    qpos = np.array([46, 47, 32, 16], np.int32)
    last = qpos.copy()
    q = random_bits(rng, (len(seq_of_row), nh, hd), -2, 2)
    kp, vp, table, origins = scatter_pool(seq_k, seq_v, nkv, hd, rng)
    row_origin = origins[seq_of_row]
    got, got64 = oracle.decode_arrays(q, kp, vp, table, row_origin, qpos, last, nh, nkv, hd,
                                      window, want_f64=True)
    want = brute_case(q, seq_k, seq_v, seq_of_row, qpos, last, nh, nkv, window)
    checked = 0
    for t in range(len(seq_of_row)):
        for h in range(nh):
            for d in range(hd):
                w = want[t][h][d]
                g = got64[t, h, d]
                assert abs(mpmath.mpf(g) - w) <= 1e-12 * max(abs(w), mpmath.mpf("1e-30")) + 1e-300, \
                    (t, h, d, g, w)
                bits, tie_dist = mp_to_bf16(w)
                if tie_dist > 1e-9:
                    assert got[t, h, d] == bits, (t, h, d, hex(got[t, h, d]), hex(bits))
                    checked += 1
    assert checked > 0.9 * len(seq_of_row) * nh * hd


def test_brute_force_page_map_and_kv_last_below_qpos():
    """A page map in front of the pool and a last visible key below the query
    position (the contract carries them as separate arrays)."""
    rng = np.random.default_rng(7)
    nh, nkv, hd, ctx = 2, 1, 4, 40
    k = random_bits(rng, (ctx, nkv, hd), -3, 3)
    v = random_bits(rng, (ctx, nkv, hd))
    kp, vp, table, origins = scatter_pool([k], [v], nkv, hd, rng, pad=0)
    # put a page map in front: table holds "virtual" ids, the map gives physical pages
    npg = kp.shape[0]
    virt = rng.permutation(np.arange(npg)).astype(np.int32)
    pmap = np.zeros(npg, np.int32)
    vtable = np.empty_like(table)
    for i, pp in enumerate(table):
        vtable[i] = virt[pp]
        pmap[virt[pp]] = pp
    q = random_bits(rng, (3, nh, hd), -3, 3)
    qpos = np.array([39, 39, 30], np.int32)
    last = np.array([39, 20, 30], np.int32)
    got, got64 = oracle.decode_arrays(q, kp, vp, vtable, origins[[0, 0, 0]], qpos, last, nh,
                                      nkv, hd, 8, page_map=pmap, want_f64=True)
    want = brute_case(q, [k], [v], [0, 0, 0], qpos, last, nh, nkv, 8)
    for t in range(3):
        for h in range(nh):
            for d in range(hd):
                w = want[t][h][d]
                assert abs(mpmath.mpf(got64[t, h, d]) - w) <= 1e-12 * max(abs(w), 1e-30) + 1e-300


@pytest.mark.parametrize("window", [0, 6])
def test_brute_force_block_decode_kv_last_above_qpos(window):
    """Block decode: rows at positions 36..39 of one sequence all see keys up to
    43 (the last visible key is a separate argument from the query position),
    with the window, when there is one, anchored at each row's own position."""
    rng = np.random.default_rng(11 + window)
    nh, nkv, hd, ctx = 4, 2, 8, 44
    k = random_bits(rng, (ctx, nkv, hd), -2, 2)
    v = random_bits(rng, (ctx, nkv, hd))
    kp, vp, table, origins = scatter_pool([k], [v], nkv, hd, rng)
    q = random_bits(rng, (4, nh, hd), -2, 2)
    qpos = np.arange(36, 40, dtype=np.int32)
    last = np.full(4, 43, np.int32)
    got, got64 = oracle.decode_arrays(q, kp, vp, table, origins[[0, 0, 0, 0]], qpos, last, nh, nkv, hd,
                                      window, want_f64=True)
    want = brute_case(q, [k], [v], [0, 0, 0, 0], qpos, last, nh, nkv, window)
    for t in range(4):
        for h in range(nh):
            for d in range(hd):
                w = want[t][h][d]
                assert abs(mpmath.mpf(got64[t, h, d]) - w) <= 1e-12 * max(abs(w), 1e-30) + 1e-300, (t, h, d)
                bits, tie_dist = mp_to_bf16(w)
                if tie_dist > 1e-9:
                    assert got[t, h, d] == bits, (t, h, d)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_two_keys_closed_form_scale_one():
    """Scores 0 and delta (scale 1.0): o = (v0 + e^delta v1) / (1 + e^delta)."""
    hd = 4
    delta = 1.5
    q = np.zeros((1, 1, hd), np.uint16)
    q[0, 0, 0] = bf16_of_f32(1.0)
    k = np.zeros((1, 1, 16, hd), np.uint16)
    k[0, 0, 1, 0] = bf16_of_f32(delta)  # key at position 1 scores delta, key 0 scores 0
    v = np.zeros((1, 1, 16, hd), np.uint16)
    v0 = [0.5, -1.0, 0.25, 2.0]
    v1 = [-0.75, 0.125, 1.0, 3.0]
    for d in range(hd):
        v[0, 0, 0, d] = bf16_of_f32(v0[d])
        v[0, 0, 1, d] = bf16_of_f32(v1[d])
    out, o64 = oracle.decode_arrays(q, k, v, [0], [0], [1], [1], 1, 1, hd, 0, want_f64=True)
    e = math.exp(delta)
    for d in range(hd):
        exact = (v0[d] + e * v1[d]) / (1 + e)
        assert o64[0, 0, d] == pytest.approx(exact, rel=1e-14, abs=1e-15)


def test_single_visible_key_returns_v_row_bitwise():
    """window = 1: only the query's own position is visible, weight exactly 1."""
    w = workloads.make("PA")
    w1 = w.replace(window=1)
    out = oracle.decode(w1)
    g = w.nh // w.nkv
    for t in range(w.rows):
        p = int(w.qpos[t])
        page = int(w.block_table[p // 16])
        for h in range(w.nh):
            assert np.array_equal(out[t, h], w.v_pool[page, h // g, p % 16])


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(3)
    nh, nkv, hd, ctx = 2, 1, 8, 37
    krow = random_bits(rng, (hd,))
    k = np.broadcast_to(krow, (ctx, nkv, hd)).copy()
    v = random_bits(rng, (ctx, nkv, hd))
    kp, vp, table, origins = scatter_pool([k], [v], nkv, hd, rng)
    q = random_bits(rng, (1, nh, hd), -4, 4)
    out, o64 = oracle.decode_arrays(q, kp, vp, table, origins, [ctx - 1], [ctx - 1], nh, nkv,
                                    hd, 0, want_f64=True)
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for d in range(hd):
        mean = mpmath.fsum(mpmath.mpf(float(x)) for x in vf[:, 0, d]) / ctx
        for h in range(nh):
            assert abs(mpmath.mpf(o64[0, h, d]) - mean) <= 1e-13 * max(abs(mean), 1e-30) + 1e-300
            bits, tie = mp_to_bf16(mean)
            if tie > 1e-9:
                assert out[0, h, d] == bits


def test_empty_visible_set_gives_zero():
    """last visible key below the window start: nothing visible, output 0."""
    w = workloads.make("C1")
    w2 = w.replace(window=4, kv_last=np.array([10], np.int32))
    out = oracle.decode(w2)
    assert not out.any()


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_window_zero_equals_window_covering_everything():
    w = workloads.make("PB")
    a = oracle.decode(w)
    for win in (int(w.qpos[0]) + 1, int(w.qpos[0]) + 1000):
        assert np.array_equal(a, oracle.decode(w.replace(window=win)))
    # and one key less is different
    assert not np.array_equal(a, oracle.decode(w.replace(window=int(w.qpos[0]))))


def test_gqa_group_equals_single_head_runs():
    """nh = nkv * g: query head h must read kv head h // g (not h % nkv)."""
    rng = np.random.default_rng(11)
    nkv, g, hd, ctx = 3, 2, 8, 40
    nh = nkv * g
    k = random_bits(rng, (ctx, nkv, hd), -2, 2)
    v = random_bits(rng, (ctx, nkv, hd))
    kp, vp, table, origins = scatter_pool([k], [v], nkv, hd, rng)
    q = random_bits(rng, (1, nh, hd), -2, 2)
    full = oracle.decode_arrays(q, kp, vp, table, origins, [ctx - 1], [ctx - 1], nh, nkv, hd, 0)
    for h in range(nh):
        kh = h // g
        k1 = np.ascontiguousarray(kp[:, kh:kh + 1])
        v1 = np.ascontiguousarray(vp[:, kh:kh + 1])
        one = oracle.decode_arrays(q[:, h:h + 1], k1, v1, table, origins, [ctx - 1], [ctx - 1],
                                   1, 1, hd, 0)
        assert np.array_equal(full[0, h], one[0, 0]), h


def test_permuting_keys_with_values():
    rng = np.random.default_rng(5)
    nh, nkv, hd, ctx = 2, 1, 8, 45
    k = random_bits(rng, (ctx, nkv, hd), -2, 2)
    v = random_bits(rng, (ctx, nkv, hd))
    perm = rng.permutation(ctx)
    q = random_bits(rng, (1, nh, hd), -2, 2)
    outs = []
    for kk, vv in ((k, v), (k[perm], v[perm])):
        kp, vp, table, origins = scatter_pool([kk], [vv], nkv, hd, np.random.default_rng(0))
        outs.append(oracle.decode_arrays(q, kp, vp, table, origins, [ctx - 1], [ctx - 1], nh,
                                         nkv, hd, 0, want_f64=True)[1])
    assert np.allclose(outs[0], outs[1], rtol=1e-12, atol=1e-15)


def test_identity_pool_equals_permuted_pool_with_page_map():
    for name in ("C2", "PA"):
        w = workloads.make(name)
        a = oracle.decode(w)
        wm = workloads.with_page_map(w)
        assert wm.page_map is not None and (wm.page_map == 0).any()
        assert np.array_equal(a, oracle.decode(wm)), name


def test_identity_pool_equals_scattered_pool_with_origins():
    w = workloads.make("PA")
    a = oracle.decode(w)
    ctx = int(w.qpos[-1]) + 1
    g_k = np.stack([w.k_pool[p // 16, :, p % 16] for p in range(ctx)])
    g_v = np.stack([w.v_pool[p // 16, :, p % 16] for p in range(ctx)])
    kp, vp, table, origins = scatter_pool([g_v[:5], g_k], [g_k[:5], g_v],
                                          w.nkv, w.hd, np.random.default_rng(9))
    b = oracle.decode_arrays(w.q, kp, vp, table, np.full(w.rows, origins[1], np.int32), w.qpos,
                             w.kv_last, w.nh, w.nkv, w.hd, w.window)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# rounding and the metric
# --------------------------------------------------------------------------

def test_bf16_rounding_hand_values():
    f = oracle.f64_to_bf16
    assert f(1.0) == 0x3F80
    assert f(-2.0) == 0xC000
    assert f(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # above the tie: up (no double rounding)
    assert f(1.0 + 2.0 ** -8 - 2.0 ** -40) == 0x3F80
    assert f(0.0) == 0 and f(-0.0) == 0x8000
    assert f(2.0 ** -133) == 0x0001                # smallest subnormal
    assert f(3.0e38) == 0x7F62 and f(4.0e38) == 0x7F80
    assert f(float("nan")) == 0x7FC0


def test_bf16_rounding_matches_f32_rne_on_f32_values():
    """For values exact in f32, direct rounding equals the usual f32->bf16 RNE."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    u = x.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, rne)


def test_rel_rms_hand_values():
    one = np.full(64, 0x3F80, np.uint16)           # 1.0
    assert oracle.rel_rms(one, one) == 0.0
    assert oracle.rel_rms(np.zeros(64, np.uint16), one) == pytest.approx(1.0)
    up = np.full(64, 0x3F81, np.uint16)            # 1 + 2^-7
    assert oracle.rel_rms(up, one) == pytest.approx(2.0 ** -7, rel=1e-12)
    zero = np.zeros(64, np.uint16)
    assert oracle.rel_rms(zero, zero) == 0.0                  # zero reference, matched
    assert oracle.rel_rms(one, zero) == math.inf               # zero reference, missed


def test_rel_rms_each_hand_values():
    """One value per last-axis vector: a vector of 1.0 with one element at
    1 + 2^-7 among n gives 2^-7 / sqrt(n); a vector of 2.0 against 1.0 gives 1;
    a NaN makes its own vector's value NaN and no other's."""
    one = np.full((3, 2, 8), 0x3F80, np.uint16)
    a = one.copy()
    a[0, 1, 5] = 0x3F81
    a[2, 0, :] = 0x4000                                 # 2.0
    a[1, 1, 3] = 0x7FC0                                 # NaN
    e = oracle.rel_rms_each(a, one)
    assert e.shape == (3, 2)
    assert e[0, 1] == pytest.approx(2.0 ** -7 / math.sqrt(8), rel=1e-12)
    assert e[2, 0] == pytest.approx(1.0, rel=1e-12)
    assert math.isnan(e[1, 1])
    ok = np.ones((3, 2), bool)
    ok[0, 1] = ok[2, 0] = ok[1, 1] = False
    assert np.all(e[ok] == 0.0)
