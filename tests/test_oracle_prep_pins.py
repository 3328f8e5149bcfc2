"""Pins for the QK-norm + RoPE prep oracle (``oracle.qk_rope_prep``), each
checked against something other than the oracle itself:

* 50-digit brute force per head (``tests/brute.py``: norm by the root mean
  square, rotation as complex multiplication), on every head of small calls;
* the addressing, through the decode oracle: a decode with window 1 at a
  token's position returns the V row stored at that token's slot bit for bit,
  so the prep must have written that token's V exactly where decode reads it;
* closed forms: a constant head normalises to +-1 (times the weight); a quarter
  turn maps (a, b) to (-b, a) and a half turn negates, bit for bit; a zero
  angle equals no rotation; the mean square after an unweighted norm is 1;
  doubling the input changes no bit (eps 0);
* structure: V is never rotated nor weighted; V = K when no V is given; the
  pools are untouched outside the tokens' slots.

Slips these catch: pairs taken as (2i, 2i + 1) instead of the two halves, a
sign flipped in the rotation, sum of squares over hd - 1 or without the mean,
the weight applied to V, V rotated, the slot or page of a token wrong, a write
outside the slot.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import brute


def f32(bits):
    return workloads.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def run(w, k_pool=None, v_pool=None, want_f64=True):
    kp, vp = w.zero_pools()
    if k_pool is not None:
        kp, vp = k_pool, v_pool
    return oracle.qk_rope_prep(w.q_in, w.k_in, w.v_in, w.q_w, w.k_w, w.rope_cos, w.rope_sin, w.pos,
                               w.block_table, w.page_origin, kp, vp, w.nh, w.nkv, w.hd, w.rotary_dim, w.eps,
                               page_map=w.page_map, want_f64=want_f64)


def slot_of(w, t):
    e = int(w.page_origin[t]) + int(w.pos[t]) // 16
    ph = int(w.block_table[e])
    if w.page_map is not None:
        ph = int(w.page_map[ph])
    return ph, int(w.pos[t]) % 16


def tiny(hd=16, rd=8, nh=2, nkv=1, tokens=5, p0=3, kv_equal=False, weights=True, eps=1e-6, seed=5):
    return workloads.prep_prefill("tiny", tokens=tokens, nh=nh, nkv=nkv, hd=hd, rotary_dim=rd, p0=p0,
                                  kv_equal=kv_equal, weights=weights, eps=eps, seed=seed)


@pytest.mark.parametrize("hd,rd,kv_equal,weights", [(16, 8, False, True), (16, 16, False, True),
                                                    (16, 0, True, False), (32, 16, True, True)])
def test_brute_force_every_head(hd, rd, kv_equal, weights):
    w = tiny(hd=hd, rd=rd, kv_equal=kv_equal, weights=weights)
    (_, _, _), (qf, kf, vf) = run(w)
    for t in range(w.tokens):
        p = int(w.pos[t])
        cr = w.rope_cos[p] if rd else None
        sr = w.rope_sin[p] if rd else None
        ph, sl = slot_of(w, t)
        for h in range(w.nh):
            ref = brute.prep_head(w.q_in[t, h], w.q_w, cr, sr, rd, w.eps)
            np.testing.assert_allclose(qf[t, h], [float(x) for x in ref], rtol=0, atol=1e-12)
        for kh in range(w.nkv):
            ref = brute.prep_head(w.k_in[t, kh], w.k_w, cr, sr, rd, w.eps)
            np.testing.assert_allclose(kf[ph, kh, sl], [float(x) for x in ref], rtol=0, atol=1e-12)
            vsrc = w.k_in if w.v_in is None else w.v_in
            ref = brute.prep_head(vsrc[t, kh], None, None, None, 0, w.eps, rotate=False)
            np.testing.assert_allclose(vf[ph, kh, sl], [float(x) for x in ref], rtol=0, atol=1e-12)


def test_rounding_is_nearest_even_of_the_f64_value():
    w = tiny(hd=32, rd=16)
    (q, kp, vp), (qf, kf, vf) = run(w)
    want = np.vectorize(oracle.f64_to_bf16, otypes=[np.uint16])
    assert np.array_equal(q, want(qf))
    assert np.array_equal(kp, want(kf))
    assert np.array_equal(vp, want(vf))


@pytest.mark.parametrize("make", ["decode", "compressed", "pagemap"])
def test_addressing_agrees_with_the_decode_oracle(make):
    """Decode with window 1 at a token's own position sees only that token's
    slot, and returns the V row there bit for bit (the decode oracle's own
    pinned addressing).  So prep's V for token t must come back from decode."""
    if make == "decode":
        w = workloads.prep_decode("d", nseq=7, lmin=1, lmax=90, nh=2, nkv=2, hd=16, rotary_dim=8, len_seed=3)
    elif make == "compressed":
        w = workloads.compress_windows(tiny(tokens=20, p0=9, nkv=2, nh=4))
    else:
        w = workloads.prep_with_page_map(workloads.prep_decode("m", nseq=5, lmin=1, lmax=60, nh=2, nkv=1,
                                                               hd=16, rotary_dim=16, len_seed=4))
    (_, kp, vp), _ = run(w)
    # V of every token computed alone, outside any pool
    vsrc = w.k_in if w.v_in is None else w.v_in
    q = np.zeros((w.tokens, w.nkv, w.hd), np.uint16)
    q[:, :, 0] = 0x3F80  # any query: one visible key gives that key's V
    out = oracle.decode_arrays(q, kp, vp, w.block_table, w.page_origin, w.pos, w.pos, w.nkv, w.nkv, w.hd,
                               window=1, page_map=w.page_map)
    for t in range(w.tokens):
        for kh in range(w.nkv):
            ref = [float(x) for x in brute.prep_head(vsrc[t, kh], None, None, None, 0, w.eps, rotate=False)]
            want = np.array([oracle.f64_to_bf16(x) for x in ref], np.uint16)
            assert np.array_equal(out[t, kh], want), (t, kh)


def test_pools_untouched_outside_the_slots():
    w = workloads.prep_decode("s", nseq=6, lmin=1, lmax=70, nh=2, nkv=2, hd=16, rotary_dim=8, len_seed=9)
    rng = np.random.default_rng(0)
    kp0 = rng.integers(0, 1 << 16, size=(w.npages, w.nkv, 16, w.hd), dtype=np.uint16)
    vp0 = rng.integers(0, 1 << 16, size=kp0.shape, dtype=np.uint16)
    (_, kp, vp), _ = run(w, kp0, vp0)
    written = np.zeros(kp0.shape[:3], bool)
    for t in range(w.tokens):
        ph, sl = slot_of(w, t)
        written[ph, :, sl] = True
    assert np.array_equal(kp[~written], kp0[~written])
    assert np.array_equal(vp[~written], vp0[~written])
    assert not np.array_equal(kp[written], kp0[written])


def _one_head(x_bits, w_bits=None, cos_row=None, sin_row=None, rd=0, eps=0.0, hd=None):
    hd = len(x_bits) if hd is None else hd
    x = np.asarray(x_bits, np.uint16).reshape(1, 1, hd)
    z = np.zeros((1, 1, hd), np.uint16)
    cos_t = np.zeros((1, max(rd // 2, 1)), np.float32) if cos_row is None else np.asarray(cos_row, np.float32)[None]
    sin_t = np.zeros((1, max(rd // 2, 1)), np.float32) if sin_row is None else np.asarray(sin_row, np.float32)[None]
    kp = np.zeros((2, 1, 16, hd), np.uint16)
    (q, _, _), (qf, _, _) = oracle.qk_rope_prep(x, z, z, w_bits, None, cos_t, sin_t, np.array([0], np.int32),
                                                np.array([1], np.int32), np.array([0], np.int32), kp, kp.copy(),
                                                1, 1, hd, rd, eps, want_f64=True)
    return q[0, 0], qf[0, 0]


@pytest.mark.parametrize("c", [0.375, -3.0, 2.0 ** -20])
def test_constant_head_normalises_to_sign_times_weight(c):
    hd = 64
    cb = workloads._bf16_trunc(np.float32(c))
    x = np.full(hd, cb, np.uint16)
    _, yf = _one_head(x)
    assert np.all(yf == np.sign(c))
    wts = workloads._bf16_trunc(np.linspace(0.5, 1.5, hd, dtype=np.float32))
    _, yf = _one_head(x, wts)
    assert np.array_equal(yf, np.sign(c) * f32(wts))


def test_unweighted_norm_has_unit_mean_square_and_ignores_scale():
    rng = workloads.Lcg(99)
    x = rng.uniform_bf16(128)
    y, yf = _one_head(x)
    assert abs(np.mean(yf ** 2) - 1.0) < 1e-12
    x2 = workloads._bf16_trunc(2.0 * workloads.bf16_bits_to_f32(x))  # exact doubling
    y2, yf2 = _one_head(x2)
    assert np.array_equal(yf2, yf) and np.array_equal(y2, y)


def test_eps_enters_under_the_root():
    x = workloads.Lcg(7).uniform_bf16(64)
    eps = 1e6
    _, yf = _one_head(x, eps=eps)
    xf = f32(x)
    ms = np.sum(xf * xf) / 64
    np.testing.assert_allclose(yf, xf / np.sqrt(ms + eps), rtol=1e-14)


def test_quarter_turn_half_turn_and_zero_angle():
    hd, rd = 64, 32
    x = workloads.Lcg(3).uniform_bf16(hd)
    _, n = _one_head(x)  # no rotation: the normalised head
    h = rd // 2
    _, y = _one_head(x, cos_row=np.zeros(h), sin_row=np.ones(h), rd=rd)
    assert np.array_equal(y[:h], -n[h:rd]) and np.array_equal(y[h:rd], n[:h]) and np.array_equal(y[rd:], n[rd:])
    _, y = _one_head(x, cos_row=-np.ones(h), sin_row=np.zeros(h), rd=rd)
    assert np.array_equal(y[:rd], -n[:rd]) and np.array_equal(y[rd:], n[rd:])
    _, y = _one_head(x, cos_row=np.ones(h), sin_row=np.zeros(h), rd=rd)
    assert np.array_equal(y, n)


def test_rotation_scales_pair_norms_by_the_table_modulus():
    hd = rd = 32
    h = rd // 2
    x = workloads.Lcg(4).uniform_bf16(hd)
    _, n = _one_head(x)
    cos_t, sin_t = workloads.rope_tables(40, rd)
    c, s = cos_t[37].astype(np.float64), sin_t[37].astype(np.float64)
    _, y = _one_head(x, cos_row=cos_t[37], sin_row=sin_t[37], rd=rd)
    got = y[:h] ** 2 + y[h:] ** 2
    np.testing.assert_allclose(got, (n[:h] ** 2 + n[h:] ** 2) * (c * c + s * s), rtol=1e-13)


def test_v_is_weightless_unrotated_and_defaults_to_k():
    w = tiny(hd=32, rd=32, nkv=2, nh=2)
    (_, kp, vp), (_, kf, vf) = run(w)
    (_, kp2, vp2), _ = run(w.replace(v_in=w.k_in))
    (_, kp3, vp3), _ = run(w.replace(v_in=None))
    assert np.array_equal(vp2, vp3) and np.array_equal(kp2, kp3)
    for t in range(w.tokens):
        ph, sl = slot_of(w, t)
        for kh in range(w.nkv):
            _, want = _one_head(w.v_in[t, kh], eps=w.eps)
            assert np.array_equal(vf[ph, kh, sl], want)
