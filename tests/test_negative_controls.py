"""Negative controls: every gate the GPU path must pass has to turn red when a
plausible mistake is planted.  The mistakes are planted on the CPU -- in the
oracle's inputs or addressing, or in a plain model of the merge and its
counter protocol -- never in the HIP path.

Gates (span-02 GPU test page, engine/crates/kernels/tests/gpu.rs, `run()`):
rel-RMS < 1e-2 against the f64 reference, fused merge == separate combine bit
for bit, counters back to zero after a call.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gates import TOL, per_head


def red(ref, got):
    """The rel-RMS gate fails (a NaN counts as failing)."""
    e = oracle.rel_rms(got, ref)
    return not (e < TOL)


@pytest.fixture(scope="module")
def pa():
    w = workloads.make("PA")
    return w, oracle.decode(w)


def test_page_address_off_by_one_slot_is_caught(pa):
    """Reading token slot p % 16 + 1 instead of p % 16."""
    w, ref = pa
    shifted = w.replace(k_pool=np.roll(w.k_pool, -1, axis=2), v_pool=np.roll(w.v_pool, -1, axis=2))
    assert red(ref, oracle.decode(shifted))


def test_page_address_off_by_one_page_is_caught(pa):
    """Reading the block-table entry after the right one."""
    w, ref = pa
    bt = np.concatenate([w.block_table[1:], w.block_table[-1:]]).astype(np.int32)
    assert red(ref, oracle.decode(w.replace(block_table=bt)))


def test_origins_forced_to_zero_is_caught():
    """Row origins ignored in a batch: rows read the pad entries (NaN page 0)
    and other sequences' pages."""
    w = workloads.batched("neg", nseq=6, lmin=40, lmax=400, nh=4, nkv=2, hd=64, pad=16)
    ref = oracle.decode(w)
    bad = oracle.decode(w.replace(page_origin=np.zeros_like(w.page_origin)))
    assert red(ref, bad)


def test_rows_pinned_to_row_zero_window_is_caught():
    """Every row of a multi-row call using row 0's visible range."""
    w = workloads.single_sequence("neg2", ctx=300, rows=6, nh=4, nkv=1, hd=64, window=7)
    ref = oracle.decode(w)
    pinned = w.replace(qpos=np.full_like(w.qpos, w.qpos[0]), kv_last=np.full_like(w.kv_last, w.kv_last[0]))
    bad = oracle.decode(pinned)
    # row 0 itself is unchanged; every other row moves
    assert np.array_equal(bad[0], ref[0])
    assert red(ref[1:], bad[1:])


# ---- window edges, through the per-(row, head) gate the GPU tests use ----

def red_per_head(ref, got):
    return not (per_head(got, ref)[1] < TOL)


@pytest.fixture(scope="module")
def one_row_batch():
    w = workloads.edge_batch("neg_eb", nseq=6, lmin=200, lmax=1500, nh=8, nkv=4, hd=128, window=150)
    return w, oracle.decode(w)


def test_edge_slip_on_one_row_sequences_is_caught(one_row_batch):
    """One key too many below the window start (window + 1) or above the last
    key (kv_last + 1) reads a NaN sentinel."""
    w, ref = one_row_batch
    assert per_head(ref, ref)[1] == 0.0
    assert red_per_head(ref, oracle.decode(w.replace(window=w.window + 1)))
    assert red_per_head(ref, oracle.decode(w.replace(kv_last=w.kv_last + 1)))
    # one row alone slipping is enough
    last = w.kv_last.copy()
    last[3] += 1
    bad = oracle.decode(w.replace(kv_last=last))
    assert red_per_head(ref[3:4], bad[3:4]) and not red_per_head(np.delete(ref, 3, 0), np.delete(bad, 3, 0))


@pytest.mark.parametrize("name", ["PA", "C2"])
def test_edge_slip_inside_a_shared_sequence_is_caught(name):
    """Rows of one sequence at the page's window of 1024: row t taking in
    lo_t - 1 (seen legitimately by row t - 1) or kv_last_t + 1 (seen by row
    t + 1) picks up the key aimed at it, and the aimed-at head of every kv
    group turns red -- a one-key slip that a whole-output gate can average
    away."""
    w = workloads.plant_edges(workloads.make(name))
    ref = oracle.decode(w)
    g = w.nh // w.nkv
    for t in range(1, w.rows):  # lower edge: start one key early (same last key)
        qp = w.qpos.copy()
        qp[t] -= 1
        bad = oracle.decode(w.replace(qpos=qp))
        e = oracle.rel_rms_each(bad, ref)
        aimed = [kh * g + t % g for kh in range(w.nkv)]
        assert np.all(e[t, aimed] > 0.1), (name, "lower", t, e[t, aimed])
        assert np.all(np.delete(e, t, 0) == 0.0)
    for t in range(w.rows - 1):  # upper edge: one key past the last
        last = w.kv_last.copy()
        last[t] += 1
        bad = oracle.decode(w.replace(kv_last=last))
        e = oracle.rel_rms_each(bad, ref)
        aimed = [kh * g + t % g for kh in range(w.nkv)]
        assert np.all(e[t, aimed] > 0.1), (name, "upper", t, e[t, aimed])


def test_rows_pinned_to_row_zero_window_at_the_page_window_is_caught():
    """The C2 shape (window 1024): every row using row 0's range."""
    w = workloads.plant_edges(workloads.make("C2"))
    ref = oracle.decode(w)
    pinned = w.replace(qpos=np.full_like(w.qpos, w.qpos[0]), kv_last=np.full_like(w.kv_last, w.kv_last[0]))
    assert red_per_head(ref[1:], oracle.decode(pinned)[1:])


def test_window_off_by_one_is_caught():
    """lo = qpos - window (one key too many) instead of qpos + 1 - window, at
    window 1: the single visible key becomes two."""
    w = workloads.make("PA").replace(window=1)
    ref = oracle.decode(w)
    assert red(ref, oracle.decode(w.replace(window=2)))


# ---- merge and counter protocol (plain f32 model of the GPU's merge) ----

def merge_model(m, l, o, order):
    """Merge S partials of one output: M = max m over non-empty splits,
    w = exp2(m - M), num / den summed as 8 interleaved groups in the given
    group-internal order, groups added in order (all f32)."""
    f = np.float32
    S = len(m)
    live = l > 0
    M = np.max(np.where(live, m, -np.inf)).astype(f)
    w = np.where(live, np.exp2((m - M).astype(f)), f(0)).astype(f)
    num = np.zeros(o.shape[1], f)
    den = f(0)
    for g in range(8):
        idx = list(range(g, S, 8))
        if order == "reversed":
            idx = idx[::-1]
        ng = np.zeros(o.shape[1], f)
        dg = f(0)
        for s in idx:
            if w[s] != 0:
                ng = (w[s] * o[s] + ng).astype(f)
                dg = f(w[s] * l[s] + dg)
        num = (num + ng).astype(f)
        den = f(den + dg)
    return (num / den).astype(f)


def test_merge_order_reversed_in_one_mode_is_caught():
    rng = np.random.default_rng(11)
    S, hd = 64, 256
    m = rng.normal(0, 3, S).astype(np.float32)
    l = rng.uniform(0.5, 20, S).astype(np.float32)
    o = (rng.normal(0, 1, (S, hd)) * l[:, None]).astype(np.float32)
    a = merge_model(m, l, o, "forward")
    b = merge_model(m, l, o, "reversed")
    assert np.allclose(a, b, rtol=1e-5)  # the same value ...
    assert not np.array_equal(a.view(np.uint32), b.view(np.uint32))  # ... but not the same bits


def counter_protocol(counter, splits, reset):
    """One fused call: every split takes a ticket; the one drawing splits-1
    merges and (if reset) restores the counter.  Returns (merged, counter)."""
    merged = False
    for _ in range(splits):
        ticket = counter
        counter += 1
        if ticket == splits - 1:
            merged = True
            if reset:
                counter = 0
    return merged, counter


def test_missing_counter_reset_is_caught():
    c = 0
    for call in range(2):
        merged, c = counter_protocol(c, 7, reset=True)
        assert merged and c == 0
    c = 0
    merged1, c = counter_protocol(c, 7, reset=False)
    merged2, c = counter_protocol(c, 7, reset=False)
    assert merged1 and not merged2 and c != 0  # second call never merges; counters not zero


# ---- the QK-norm + RoPE prep gates (pegainfer pull request page #1002,
# its negative controls: a paged address off by one must fail the
# layout-address gate; every row pinned to row 0's window must fail the
# decode == prefill gate) ----

def _prep_pools(w):
    kp, vp = w.zero_pools()
    return oracle.qk_rope_prep(w.q_in, w.k_in, w.v_in, w.q_w, w.k_w, w.rope_cos, w.rope_sin, w.pos,
                               w.block_table, w.page_origin, kp, vp, w.nh, w.nkv, w.hd, w.rotary_dim, w.eps,
                               page_map=w.page_map)


def test_prep_slot_off_by_one_is_caught():
    """Writing each token one slot further (position + 1) lands values
    outside the expected rows: the layout-address gate (exact zeros
    elsewhere, the expected values in place) turns red."""
    w = workloads.prep_prefill("negp", tokens=20, nh=2, nkv=1, hd=64, rotary_dim=32, p0=3)
    _, kp, vp = _prep_pools(w)
    # the same values one slot on: shift the positions, keep the rotary rows
    shifted = w.replace(pos=(w.pos + 1).astype(np.int32),
                        rope_cos=np.concatenate([w.rope_cos[:1], w.rope_cos]),
                        rope_sin=np.concatenate([w.rope_sin[:1], w.rope_sin]))
    _, kp2, vp2 = _prep_pools(shifted)
    assert not np.array_equal(kp2, kp) and not np.array_equal(vp2, vp)
    written = np.any(kp != 0, axis=-1)
    assert np.any(np.any(kp2 != 0, axis=-1) & ~written)  # something landed outside the expected rows


def test_prep_rows_pinned_to_row_zero_window_is_caught():
    """The decode form with every token's origin pinned to token 0's (its
    compressed window read for all rows) no longer equals the prefill form."""
    w = workloads.prep_prefill("negq", tokens=40, nh=2, nkv=1, hd=64, rotary_dim=64, p0=5)
    c = workloads.compress_windows(w)
    q_ref, k_ref, v_ref = _prep_pools(w)
    q_ok, k_ok, v_ok = _prep_pools(c)
    assert np.array_equal(k_ok, k_ref) and np.array_equal(v_ok, v_ref)  # the gate passes when origins are read
    pinned = c.replace(page_origin=np.full_like(c.page_origin, c.page_origin[0]))
    _, k_bad, v_bad = _prep_pools(pinned)
    assert not np.array_equal(k_bad, k_ref) or not np.array_equal(v_bad, v_ref)
