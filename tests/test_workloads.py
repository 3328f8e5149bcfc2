"""The seeded input generators (shared by the oracle and the HIP path)."""
import numpy as np

import workloads


def test_lcg_vectorised_equals_sequential():
    a = workloads.Lcg(12345)
    b = workloads.Lcg(12345)
    st = a.states(5000)
    for i in range(5000):
        assert int(st[i]) == b.step()
    assert a.state == b.state


def test_lcg_first_state_by_hand():
    # one step of s*6364136223846793005 + 1442695040888963407 mod 2^64 from 12345
    s = (12345 * 6364136223846793005 + 1442695040888963407) % (1 << 64)
    assert workloads.Lcg(12345).step() == s


def test_uniform_range_and_truncation():
    r = workloads.Lcg(99)
    bits = r.uniform_bf16(200000)
    x = workloads.bf16_bits_to_f32(bits)
    assert x.min() >= -1.0 and x.max() < 1.0
    assert x.min() < -0.99 and x.max() > 0.99          # covers [-1, 1)
    assert abs(float(x.mean())) < 0.01
    # truncation: recompute one value by hand from the state
    r2 = workloads.Lcg(99)
    s = r2.step()
    f = np.float32((s >> 40) * 2.0 ** -23 - 1.0)
    assert bits[0] == (int(f.view(np.uint32)) >> 16)
    k8 = workloads.Lcg(99).uniform_bf16(1000, 8.0)
    assert np.array_equal(workloads.bf16_bits_to_f32(k8), 8.0 * x[:1000])


def test_single_sequence_fixture_shapes():
    w = workloads.make("C1")
    assert w.k_pool.shape == (5, 1, 16, 64)
    assert list(w.block_table) == [0, 1, 2, 3]
    assert list(w.qpos) == [63] and list(w.kv_last) == [63] and list(w.page_origin) == [0]
    w = workloads.make("PA")
    assert w.k_pool.shape == ((1500 + 15) // 16 + 1, 8, 16, 256)
    assert list(w.qpos) == [1495, 1496, 1497, 1498, 1499]


def test_mapped_pool_layout():
    w = workloads.make("C2")
    fl = workloads.first_live_page(w)
    assert fl == (4092 + 1 - 1024) // 16 == 191
    m = workloads.with_page_map(w)
    npg = w.npages
    assert m.k_pool.shape[0] == npg + 1
    assert (m.k_pool[0] == workloads.BF16_QNAN).all() and (m.v_pool[0] == workloads.BF16_QNAN).all()
    for p in range(npg):
        if p < fl:
            assert m.page_map[p] == 0
        else:
            assert m.page_map[p] == npg - p
            assert np.array_equal(m.k_pool[npg - p], w.k_pool[p])
            assert np.array_equal(m.v_pool[npg - p], w.v_pool[p])


def test_batched_layout():
    w = workloads.batched("t", nseq=6, lmin=20, lmax=100, nh=4, nkv=2, hd=8, pad=16)
    lens = w.qpos + 1
    assert ((lens >= 20) & (lens <= 100)).all()
    pages = (lens + 15) // 16
    assert list(w.page_origin) == list(16 + np.concatenate([[0], np.cumsum(pages)[:-1]]))
    assert (w.block_table[:16] == 0).all()
    body = w.block_table[16:]
    assert sorted(body.tolist()) == list(range(1, pages.sum() + 1))   # a permutation
    assert (w.k_pool[0] == workloads.BF16_QNAN).all()
    assert len(set(w.page_origin.tolist())) == 6 and (w.page_origin > 0).all()
    wn = workloads.batched("t", nseq=6, lmin=20, lmax=100, nh=4, nkv=2, hd=8, pad=16, nan_tail=True)
    for s in range(6):
        used = int(lens[s]) % 16
        if used:
            phys = wn.block_table[wn.page_origin[s] + pages[s] - 1]
            assert (wn.k_pool[phys, :, used:] == workloads.BF16_QNAN).all()
            assert np.array_equal(wn.k_pool[phys, :, :used], w.k_pool[phys, :, :used])


def test_c4_lengths_in_range():
    r = workloads.Lcg(777)
    lens = [512 + r.u32() % 15873 for _ in range(64)]
    assert min(lens) >= 512 and max(lens) <= 16384
