"""The code against the values the span-02 GPU kernel test page prints
(tests/golden/span02_gpu_test_page.json): generator constants and seed, the
null-page fill, page size and spare page, the counter buffer, the rel-RMS
bounds the tests use, and the page's two parity configurations."""
import json
import os
import re

import numpy as np

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "span02_gpu_test_page.json")))


def val(key):
    return G[key]["value"]


def test_generator_constants_and_seed():
    assert workloads._MUL == val("lcg_multiplier")
    assert workloads._INC == val("lcg_increment")
    # the single-sequence fixtures seed with seed_base + hd: the first K value
    # of PA is the first draw of Lcg(seed_base + 256)
    w = workloads.make("PA")
    first = workloads.Lcg(val("seed_base") + w.hd).uniform_bf16(1)[0]
    assert w.k_pool.reshape(-1)[0] == first


def test_null_page_fill():
    assert workloads.BF16_QNAN == val("null_page_fill_bits")
    m = workloads.with_page_map(workloads.make("PA"))
    assert np.all(m.k_pool[0] == val("null_page_fill_bits"))
    assert np.all(m.v_pool[0] == val("null_page_fill_bits"))


def test_parity_configs_and_pool_size():
    for c in val("parity_configs"):
        w = workloads.make(c["name"])
        assert (w.nh, w.nkv, w.hd, w.window, w.rows) == (c["nh"], c["nkv"], c["hd"], c["window"], c["rows"])
        ctx = int(w.kv_last.max()) + 1
        assert ctx == c["ctx"]
        page = val("page_tokens")
        assert w.k_pool.shape == ((ctx + page - 1) // page + val("spare_pages"), w.nkv, page, w.hd)
        assert len(w.block_table) == (ctx + page - 1) // page
        assert list(w.qpos) == list(range(ctx - w.rows, ctx))


def test_counter_buffer_matches_the_page():
    import paged_gqa_decode_attn_amd as pg

    assert pg.counter_capacity() == val("counter_entries")
    assert pg.PAGE == val("page_tokens")


def test_tolerances_in_the_gpu_tests():
    """The GPU parity tests gate decode and prefill at the page's bounds: they
    take the gate's bound (tests/gates.py) and nothing looser."""
    text = open(os.path.join(HERE, "gates.py")).read()
    m = re.search(r"^TOL = ([0-9.e+-]+)$", text, re.M)
    assert m
    assert float(m.group(1)) == val("decode_rel_rms_bound") == val("prefill_rel_rms_bound")
    for fname in ("test_gpu_decode.py", "test_gpu_prefill.py", "test_gpu_edges.py"):
        src = open(os.path.join(HERE, fname)).read()
        assert "from tests.gates import TOL, per_head" in src, fname
        assert not re.search(r"^TOL = ", src, re.M), fname
