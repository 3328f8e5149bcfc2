"""GPU parity of the QK-norm + RoPE prep (``pgqa_qk_rope_prep``), through the
C ABI, against the CPU oracle; and the two GPU-vs-GPU gates of the pegainfer
pull request page #1002:

* lands at layout addresses: pools start at zero; every slot the oracle
  writes must hold the oracle's value, every other element must still be
  exactly zero (the sentinel page 0 included);
* decode equals prefill: the same tokens written once with the prefill form
  (one table, origin 0) and once with per-token compressed windows (distinct,
  non-zero origins over separate table spans) give identical bits.

Tolerance (f32 arithmetic against the f64 oracle, both rounded once to
bf16): |gpu - exact| <= half a bf16 ulp of the exact value plus
(hd 2^-24 + 2^-20) times the head's largest magnitude -- the bound on the f32
sum of squares (hd terms), the reciprocal square root and the rotation's
few roundings.
"""
import numpy as np
import pytest

from tests.gpu_env import need_gpu

need_gpu()
import torch  # noqa: E402

import oracle  # noqa: E402
import paged_gqa_decode_attn_amd as pg  # noqa: E402
import workloads  # noqa: E402
from tests.gates import TOL, per_head  # noqa: E402
from tests.gpu_util import DevicePrep, DeviceWorkload  # noqa: E402

pytestmark = pytest.mark.gpu


def host(t):
    return t.cpu().numpy().view(np.uint16)


def oracle_prep(w):
    kp, vp = w.zero_pools()
    return oracle.qk_rope_prep(w.q_in, w.k_in, w.v_in, w.q_w, w.k_w, w.rope_cos, w.rope_sin, w.pos,
                               w.block_table, w.page_origin, kp, vp, w.nh, w.nkv, w.hd, w.rotary_dim, w.eps,
                               page_map=w.page_map, want_f64=True)


def written_rows(w):
    """(page, kv head, slot) rows the oracle writes: pools pre-filled with a
    marker, rows that changed."""
    kp = np.full((w.npages, w.nkv, 16, w.hd), 0xFFFF, np.uint16)
    _, k2, _ = oracle.qk_rope_prep(w.q_in, w.k_in, w.v_in, w.q_w, w.k_w, w.rope_cos, w.rope_sin, w.pos,
                                   w.block_table, w.page_origin, kp, kp.copy(), w.nh, w.nkv, w.hd, w.rotary_dim,
                                   w.eps, page_map=w.page_map)
    return np.any(k2 != 0xFFFF, axis=-1)


def within_bound(got_bits, exact, hd):
    """Elementwise check of the tolerance above over [..., hd] arrays."""
    g = workloads.bf16_bits_to_f32(got_bits).astype(np.float64)
    ax = np.abs(exact)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    ulp = np.where(ax > 0, 2.0 ** (np.maximum(e, -126) - 7), 2.0 ** -133)
    rowmax = np.max(ax, axis=-1, keepdims=True)
    bound = 0.5 * ulp + (hd * 2.0 ** -24 + 2.0 ** -20) * rowmax
    return np.abs(g - exact) <= bound


def check(w, q, kp, vp):
    (q_o, kp_o, vp_o), (qf, kf, vf) = oracle_prep(w)
    rows = written_rows(w)
    assert np.all(within_bound(q, qf, w.hd)), "q_out"
    for name, got, ref_bits, ref in (("k_pool", kp, kp_o, kf), ("v_pool", vp, vp_o, vf)):
        assert np.all(got[~rows] == 0), name + ": written outside the tokens' slots"
        ok = within_bound(got[rows], ref[rows], w.hd)
        assert np.all(ok), f"{name}: {np.count_nonzero(~ok)} elements outside the bound"
        # nearly every element is the oracle's bf16 exactly
        assert np.mean(got[rows] != ref_bits[rows]) < 0.01, name
    assert np.mean(q != q_o) < 0.01
    assert oracle.rel_rms(q, q_o) < 1e-2


CASES = list(workloads.PREP_NAMES) + ["R128D+pagemap", "R256F+pagemap", "R256P+rd0", "R128D+eps"]


def make_case(name):
    base, _, var = name.partition("+")
    w = workloads.make_prep(base)
    if var == "pagemap":
        w = workloads.prep_with_page_map(w)
    elif var == "rd0":
        w = w.replace(rotary_dim=0)
    elif var == "eps":
        w = w.replace(eps=0.25)
    return w


@pytest.mark.parametrize("name", CASES)
def test_prep_matches_oracle(name):
    w = make_case(name)
    print(f"prep {name}: tokens {w.tokens} nh {w.nh} nkv {w.nkv} hd {w.hd} rd {w.rotary_dim}", flush=True)
    q, kp, vp = DevicePrep(w).run()
    check(w, host(q), host(kp), host(vp))


@pytest.mark.parametrize("name", ["R256F", "R256P", "R512KV", "R128D"])
def test_prep_decode_equals_prefill(name):
    """One table at the tokens' shared origins versus per-token compressed
    windows: the same slots, so the same bits; page 0 stays zero in both."""
    w = workloads.make_prep(name)
    c = workloads.compress_windows(w)
    # origins that differ between tokens, from the prefill form's, and from 0
    assert len(set(c.page_origin.tolist())) > 1
    assert np.all(c.page_origin > 0) and np.all(c.page_origin != w.page_origin)
    print(f"prep decode==prefill {name}: tokens {w.tokens}", flush=True)
    q1, k1, v1 = (host(t) for t in DevicePrep(w).run())
    q2, k2, v2 = (host(t) for t in DevicePrep(c).run())
    assert np.array_equal(q1, q2)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.any(k2[0]) and not np.any(v2[0])


def test_prep_in_place_query():
    w = workloads.make_prep("R256P")
    d = DevicePrep(w)
    q_sep, _, _ = d.run()
    q_io = d.q_in.clone()
    d2 = DevicePrep(w)
    d2.q_in = q_io
    q_in_place, _, _ = d2.run(q_out=q_io)
    assert torch.equal(q_sep, q_in_place)


def test_prep_zero_tokens_touches_nothing():
    w = workloads.make_prep("R64D")
    d = DevicePrep(w)
    kp = torch.full((w.npages, w.nkv, 16, w.hd), 7, dtype=torch.int16, device="cuda")
    pg.qk_rope_prep(torch.empty(8, dtype=torch.int16, device="cuda"), kp, kp, d.q_in, d.k_in, None, None, None,
                    d.cos, d.sin, d.pos, d.bt, d.off, 0, w.nh, w.nkv, w.hd, w.rotary_dim, w.eps)
    torch.cuda.synchronize()
    assert bool(torch.all(kp == 7))


def test_prep_full_size_prefill_8k():
    """The measured prefill shape (8192 tokens, nh 32, nkv 8, hd 128) in the
    launch configuration the benchmark times, against the oracle in full."""
    w = workloads.make_prep("R128P8K")
    print("prep R128P8K full size", flush=True)
    q, kp, vp = DevicePrep(w).run()
    check(w, host(q), host(kp), host(vp))


def test_prep_then_decode():
    """The pool the prep fills is the pool decode reads: prep over a 300-token
    context, then decode of its last 4 rows with the prepped queries, against
    oracle prep followed by oracle decode."""
    w = workloads.prep_prefill("ctx", tokens=300, nh=8, nkv=2, hd=128, rotary_dim=64, seed=31)
    q, kp, vp = DevicePrep(w).run()
    (q_o, kp_o, vp_o) = oracle_prep(w)[0]
    rows = 4
    qpos = w.pos[-rows:]
    dw = workloads.Workload("ctx", rows, w.nh, w.nkv, w.hd, 0, host(q)[-rows:].copy(), host(kp), host(vp),
                            w.block_table, np.zeros(rows, np.int32), qpos, qpos.copy())
    d = DeviceWorkload(dw)
    d.q = q[-rows:].contiguous()
    d.k, d.v = kp, vp
    got = d.host(d.run(d.heuristic_splits()))
    ref = oracle.decode_arrays(q_o[-rows:], kp_o, vp_o, w.block_table, np.zeros(rows, np.int32), qpos, qpos,
                               w.nh, w.nkv, w.hd, 0)
    assert per_head(got, ref)[1] < TOL
