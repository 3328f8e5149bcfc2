"""Upload helpers: put a workload's host arrays on the GPU and make calls of
the C ABI (through the binding) on them.  Nothing here computes attention;
the tests and the benchmark share it."""
import numpy as np
import torch

import paged_gqa_decode_attn_amd as pg


def dev_i16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


class DevicePrep:
    """A prep workload's inputs on the device; ``run`` makes one
    pgqa_qk_rope_prep call into zeroed (or given) pools."""

    def __init__(self, w):
        self.w = w
        self.q_in = dev_i16(w.q_in)
        self.k_in = dev_i16(w.k_in)
        self.v_in = None if w.v_in is None else dev_i16(w.v_in)
        self.q_w = None if w.q_w is None else dev_i16(w.q_w)
        self.k_w = None if w.k_w is None else dev_i16(w.k_w)
        self.cos = dev_f32(w.rope_cos) if w.rotary_dim else None
        self.sin = dev_f32(w.rope_sin) if w.rotary_dim else None
        self.pos = dev_i32(w.pos)
        self.bt = dev_i32(w.block_table)
        self.off = dev_i32(w.page_origin)
        self.pmap = None if w.page_map is None else dev_i32(w.page_map)

    def run(self, k_pool=None, v_pool=None, q_out=None, sync=True):
        w = self.w
        shape = (w.npages, w.nkv, 16, w.hd)
        kp = torch.zeros(shape, dtype=torch.int16, device="cuda") if k_pool is None else k_pool
        vp = torch.zeros(shape, dtype=torch.int16, device="cuda") if v_pool is None else v_pool
        qo = torch.empty((w.tokens, w.nh, w.hd), dtype=torch.int16, device="cuda") if q_out is None else q_out
        pg.qk_rope_prep(qo, kp, vp, self.q_in, self.k_in, self.v_in, self.q_w, self.k_w, self.cos, self.sin,
                        self.pos, self.bt, self.off, w.tokens, w.nh, w.nkv, w.hd, w.rotary_dim, w.eps,
                        page_map=self.pmap)
        if sync:
            torch.cuda.synchronize()
        return qo, kp, vp


class DeviceWorkload:
    """A decode workload's inputs on the device; ``run`` makes one
    pgqa_attn_decode call, ``prefill`` one pgqa_attn_prefill call."""

    def __init__(self, w):
        self.w = w
        self.q = dev_i16(w.q)
        self.k = dev_i16(w.k_pool)
        self.v = dev_i16(w.v_pool)
        self.bt = dev_i32(w.block_table)
        self.off = dev_i32(w.page_origin)
        self.qpos = dev_i32(w.qpos)
        self.last = dev_i32(w.kv_last)
        self.pmap = None if w.page_map is None else dev_i32(w.page_map)

    def span(self):
        w = self.w
        ctx = int(w.kv_last.max()) + 1
        return min(ctx, w.window) if w.window > 0 else ctx

    def heuristic_splits(self, rows_per_seq=None):
        w = self.w
        return pg.choose_splits(self.span(), w.rows, w.nkv, w.rows if rows_per_seq is None else rows_per_seq)

    def run(self, splits, counters=None, out=None, part=None, sync=True):
        w = self.w
        if out is None:
            out = torch.empty((w.rows, w.nh, w.hd), dtype=torch.int16, device="cuda")
        if part is None and splits > 1:
            part = torch.empty(pg.decode_part_bytes(w.rows, w.nh, splits, w.hd), dtype=torch.uint8,
                               device="cuda")
        pg.attn_decode(out, part, self.q, self.k, self.v, self.bt, self.off, self.qpos, self.last,
                       w.rows, w.nh, w.nkv, w.hd, w.window, splits, counters, self.pmap)
        if sync:
            torch.cuda.synchronize()
        return out

    def prefill(self, tiles=None, out=None, sync=True):
        """One pgqa_attn_prefill call over all rows; tiles default to
        make_tiles(page_origin, prefill_rows_per_tile(hd))."""
        w = self.w
        if tiles is None:
            tiles = pg.make_tiles(w.page_origin, pg.prefill_rows_per_tile(w.hd))
        t0, tn = tiles
        if not isinstance(t0, torch.Tensor):  # host arrays: upload
            t0, tn = dev_i32(t0), dev_i32(tn)
        if out is None:
            out = torch.empty((w.rows, w.nh, w.hd), dtype=torch.int16, device="cuda")
        pg.attn_prefill(out, self.q, self.k, self.v, self.bt, self.off, self.qpos, self.last, t0, tn,
                        len(t0), w.rows, w.nh, w.nkv, w.hd, w.window, self.pmap)
        if sync:
            torch.cuda.synchronize()
        return out

    def host(self, out):
        return out.cpu().numpy().view(np.uint16)


def new_counters():
    return torch.zeros(pg.counter_capacity(), dtype=torch.int32, device="cuda")
