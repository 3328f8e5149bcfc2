"""The allocation-free decode entry point (pgqa_attn_decode_noalloc), through
the C ABI: it must give, bit for bit, what pgqa_attn_decode gives with the
caller's partial buffer and the separate combine, for the same split count
-- on two calls in a row, the second on a smaller input (the scratch keeps
the first call's contents) -- and stay within the parity bound against the
oracle.  A call whose partials exceed the scratch is refused."""
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
from tests.gpu_util import DeviceWorkload  # noqa: E402


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def noalloc(dw, splits):
    w = dw.w
    out = torch.empty((w.rows, w.nh, w.hd), dtype=torch.int16, device="cuda")
    pg.attn_decode_noalloc(out, dw.q, dw.k, dw.v, dw.bt, dw.off, dw.qpos, dw.last, w.rows, w.nh, w.nkv, w.hd,
                           w.window, splits, page_map=dw.pmap)
    torch.cuda.synchronize()
    return dw.host(out)


def test_noalloc_equals_the_partial_buffer_call_twice_in_a_row():
    cases = [(workloads.make("C5W4096"), 64),      # 8 rows x 8 heads x 64 splits: 4.2 MB of partials
             (workloads.with_page_map(workloads.make("PA")), 8)]  # then a smaller call
    for w, s in cases:
        need = pg.decode_part_bytes(w.rows, w.nh, s, w.hd)
        assert 0 < need <= pg.NOALLOC_SCRATCH_BYTES
        say(f"[gpu] noalloc {w.name} splits={s} partials={need} bytes")
        dw = DeviceWorkload(w)
        ref_call = dw.host(dw.run(s, counters=None))
        got = noalloc(dw, s)
        assert np.array_equal(got, ref_call), (w.name, s)
        whole, worst, at = per_head(got, oracle.decode(w))
        say(f"[gpu] noalloc {w.name}: rel_rms {whole:.3e} worst (row, head) {at}: {worst:.3e}")
        assert worst < TOL
    # one split: no scratch used at all
    dw = DeviceWorkload(workloads.make("C1"))
    assert np.array_equal(noalloc(dw, 1), dw.host(dw.run(1)))


def test_noalloc_refuses_partials_beyond_the_scratch():
    w = workloads.make("C3")  # 16 heads x 512: 256 splits need 8.4 MB -- fits; 64 rows would not
    dw = DeviceWorkload(w)
    rows = 64
    q = torch.zeros((rows, w.nh, w.hd), dtype=torch.int16, device="cuda")
    out = torch.empty_like(q)
    z = torch.zeros(rows, dtype=torch.int32, device="cuda")
    assert pg.decode_part_bytes(rows, w.nh, 256, w.hd) > pg.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pg.PgqaError) as ei:
        pg.attn_decode_noalloc(out, q, dw.k, dw.v, dw.bt, z, z, z, rows, w.nh, w.nkv, w.hd, 0, 256)
    assert ei.value.code == pg.EINVAL and "scratch" in str(ei.value)
