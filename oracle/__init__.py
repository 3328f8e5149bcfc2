"""CPU oracle for paged GQA decode attention (f64, plain C, OpenMP over rows x heads).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``paged_gqa_decode_attn_amd``) and the library never calls
it: there is no CPU fallback.

Decode attention: what it computes is the f64 reference of the span-02 GPU test page
(engine/crates/kernels/tests/gpu.rs, function ``reference``), extended to the
full decode contract of that page's ``attn_decode`` call: per-row page origins
into the block table, an optional page map, and a separate last-visible-key
array.  See ``pgqa_oracle.c`` for the formulas and addressing.

QK-norm + RoPE prep (``qk_rope_prep``): RMSNorm, rotary embedding and the
paged-pool write of the step before decode, as the pegainfer pull request page
#1002 describes its QK-RoPE gates; ``qk_rope_oracle.c`` states the reading.

Every function here is pinned by ``tests/test_oracle_pins.py`` (arbitrary
precision brute force on tiny inputs, closed forms and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "pgqa_oracle.c"), os.path.join(_HERE, "qk_rope_oracle.c")]
_LIB = os.path.join(_HERE, "liboracle.so")

_handle = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3 -fopenmp, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp] + _SRCS + ["-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(_LIB):
            build(force=False)
        h = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        h.pgqa_oracle_decode.restype = ctypes.c_int
        h.pgqa_oracle_decode.argtypes = [p, p, p, p, p, p, i64, p, p, p, p, i64, i64,
                                         i64, i64, i64, i64, i64, ctypes.c_int]
        h.pgqa_oracle_rel_rms.restype = ctypes.c_double
        h.pgqa_oracle_rel_rms.argtypes = [p, p, i64]
        h.pgqa_oracle_rel_rms_each.restype = None
        h.pgqa_oracle_rel_rms_each.argtypes = [p, p, i64, i64, p]
        h.pgqa_oracle_qk_rope_prep.restype = ctypes.c_int
        h.pgqa_oracle_qk_rope_prep.argtypes = [p] * 13 + [i64, p, p, i64, p, p, i64, i64, i64, i64,
                                                          i64, i64, i64, ctypes.c_double]
        h.oracle_f64_to_bf16.restype = ctypes.c_uint16
        h.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        _handle = h
    return _handle


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def decode_arrays(q, k_pool, v_pool, block_table, page_origin, qpos, kv_last,
                  nh: int, nkv: int, hd: int, window: int, page_map=None,
                  threads: int = 0, want_f64: bool = False):
    """Decode attention over a paged pool; bf16 arrays are uint16 bit patterns.

    Returns ``out`` (uint16 [rows, nh, hd]) or ``(out, out_f64)``."""
    q = _c(q, np.uint16)
    k_pool = _c(k_pool, np.uint16)
    v_pool = _c(v_pool, np.uint16)
    bt = _c(block_table, np.int32)
    off = _c(page_origin, np.int32)
    qp = _c(qpos, np.int32)
    kl = _c(kv_last, np.int32)
    pm = None if page_map is None else _c(page_map, np.int32)
    rows = int(qp.shape[0])
    npages = int(k_pool.size // (nkv * 16 * hd))
    out = np.zeros((rows, nh, hd), dtype=np.uint16)
    of = np.zeros((rows, nh, hd), dtype=np.float64) if want_f64 else None
    rc = _lib().pgqa_oracle_decode(_ptr(out), _ptr(of), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                   _ptr(bt), bt.size, _ptr(off), _ptr(qp), _ptr(kl),
                                   _ptr(pm), 0 if pm is None else pm.size, npages,
                                   rows, nh, nkv, hd, window, threads)
    if rc != 0:
        raise ValueError(f"oracle refused its inputs (code {rc})")
    return (out, of) if want_f64 else out


def decode(w, threads: int = 0, want_f64: bool = False):
    """Oracle output for a ``workloads.Workload``."""
    return decode_arrays(w.q, w.k_pool, w.v_pool, w.block_table, w.page_origin, w.qpos,
                         w.kv_last, w.nh, w.nkv, w.hd, w.window, w.page_map,
                         threads=threads, want_f64=want_f64)


def rows_subset(w, rows):
    """The same workload restricted to a subset of query rows (for sampling)."""
    idx = np.asarray(rows, dtype=np.int64)
    return w.replace(rows=len(idx), q=w.q[idx], page_origin=w.page_origin[idx],
                     qpos=w.qpos[idx], kv_last=w.kv_last[idx])


def rel_rms(a: np.ndarray, b: np.ndarray) -> float:
    """Relative RMS difference of bf16 bit patterns ``a`` from the reference
    ``b``: rms(a - b) / rms(b), in f64 (0 or inf for an all-zero reference).
    The span-02 test page gates decode on this measure below 1e-2."""
    a = _c(a, np.uint16).ravel()
    b = _c(b, np.uint16).ravel()
    if a.size != b.size:
        raise ValueError("size mismatch")
    return float(_lib().pgqa_oracle_rel_rms(_ptr(a), _ptr(b), a.size))


def rel_rms_each(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """``rel_rms`` of every last-axis vector (for decode outputs
    ``[rows, nh, hd]``: one value per (row, head)), shaped like ``a[..., 0]``."""
    a = _c(a, np.uint16)
    b = _c(b, np.uint16)
    if a.shape != b.shape or a.ndim < 1:
        raise ValueError("shape mismatch")
    ln = a.shape[-1]
    nvec = a.size // max(ln, 1)
    out = np.zeros(nvec, np.float64)
    _lib().pgqa_oracle_rel_rms_each(_ptr(a), _ptr(b), nvec, ln, _ptr(out))
    return out.reshape(a.shape[:-1])


def f64_to_bf16(x: float) -> int:
    """Correctly rounded f64 -> bf16 bits (nearest, ties to even)."""
    return int(_lib().oracle_f64_to_bf16(float(x)))


def timed_decode(w, threads: int = 0) -> Tuple[np.ndarray, float]:
    t0 = time.perf_counter()
    out = decode(w, threads=threads)
    return out, time.perf_counter() - t0


def qk_rope_prep(q_in, k_in, v_in, q_w, k_w, rope_cos, rope_sin, pos, block_table, page_origin,
                 k_pool, v_pool, nh: int, nkv: int, hd: int, rotary_dim: int, eps: float,
                 page_map=None, want_f64: bool = False):
    """QK-norm + RoPE prep of ``tokens`` tokens (bf16 arrays as uint16 bits).

    ``k_pool`` / ``v_pool`` are copied and the copies written at the tokens'
    slots (everything else is left as given).  ``v_in`` None: V from ``k_in``;
    ``q_w`` / ``k_w`` None: weight 1.  ``rope_cos`` / ``rope_sin`` are f32
    ``[positions, rotary_dim / 2]``.

    Returns ``(q_out, k_pool, v_pool)``, or with ``want_f64`` also
    ``(q_f64, k_f64, v_f64)``: the unrounded values, the pool shadows zero
    wherever nothing was written."""
    q_in = _c(q_in, np.uint16)
    k_in = _c(k_in, np.uint16)
    v_in = None if v_in is None else _c(v_in, np.uint16)
    q_w = None if q_w is None else _c(q_w, np.uint16)
    k_w = None if k_w is None else _c(k_w, np.uint16)
    half = rotary_dim // 2
    cos_t = _c(rope_cos, np.float32).reshape(-1, max(half, 1)) if half else np.zeros((0, 1), np.float32)
    sin_t = _c(rope_sin, np.float32).reshape(-1, max(half, 1)) if half else np.zeros((0, 1), np.float32)
    ps = _c(pos, np.int32)
    bt = _c(block_table, np.int32)
    off = _c(page_origin, np.int32)
    pm = None if page_map is None else _c(page_map, np.int32)
    kp = np.array(k_pool, dtype=np.uint16, copy=True, order="C")
    vp = np.array(v_pool, dtype=np.uint16, copy=True, order="C")
    tokens = int(ps.shape[0])
    npages = int(kp.size // (nkv * 16 * hd))
    q_out = np.zeros((tokens, nh, hd), dtype=np.uint16)
    qf = kf = vf = None
    if want_f64:
        qf = np.zeros((tokens, nh, hd), dtype=np.float64)
        kf = np.zeros(kp.shape, dtype=np.float64)
        vf = np.zeros(vp.shape, dtype=np.float64)
    rc = _lib().pgqa_oracle_qk_rope_prep(
        _ptr(q_out), _ptr(qf), _ptr(kp), _ptr(vp), _ptr(kf), _ptr(vf), _ptr(q_in), _ptr(k_in), _ptr(v_in),
        _ptr(q_w), _ptr(k_w), _ptr(cos_t), _ptr(sin_t), cos_t.shape[0] if half else 0, _ptr(ps), _ptr(bt),
        bt.size, _ptr(off), _ptr(pm), 0 if pm is None else pm.size, npages, tokens, nh, nkv, hd, rotary_dim,
        float(eps))
    if rc != 0:
        raise ValueError(f"oracle refused its inputs (code {rc})")
    if want_f64:
        return (q_out, kp, vp), (qf, kf, vf)
    return q_out, kp, vp
