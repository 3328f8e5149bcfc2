"""Paged GQA decode attention on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libpgqa.so`` (declared in ``include/pgqa.h``).  It
only marshals arguments -- torch tensors (or raw device addresses) to pointers,
the current torch stream to a ``hipStream_t`` -- and raises on a non-zero
return.  Every step of the computation runs in the HIP kernels; there is no
CPU or framework fallback, and a missing library is an error.

Entry points (same names and argument order as the C ABI, after the span-02
GPU test page's ``attn`` calls): ``choose_splits`` (and ``choose_splits_heads``,
the same count with the head layout), ``decode_part_bytes``,
``counter_capacity``, ``attn_decode``, ``prefill_rows_per_tile``,
``make_tiles``, ``attn_prefill``; ``qk_rope_prep``, the QK-norm + RoPE step
that fills the pool before decode; ``attn_decode_noalloc``, decode for
callers that cannot allocate; ``set_merge_wait_ticks`` and
``set_narrow_path``, test hooks.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpgqa.so")

PAGE = 16
MAX_SPLITS = 256
OK, EINVAL, ECAP, ELAUNCH = 0, -1, -2, -3


class PgqaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pgqa error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PgqaError(EINVAL, f"{LIB_PATH} is not built; run __graft_entry__.build() "
                                    "or python -m paged_gqa_decode_attn_amd._build")
        # One HIP runtime per process: torch ships its own copy of the runtime
        # under the same soname, and the library must bind to that one.  Loaded
        # first, the library would pull in the system copy and torch would then
        # load its own beside it, with separate device state.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        h = ctypes.CDLL(LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        h.pgqa_choose_splits.restype = ctypes.c_int32
        h.pgqa_choose_splits.argtypes = [i64, i64, i64, i64]
        h.pgqa_choose_splits_heads.restype = ctypes.c_int32
        h.pgqa_choose_splits_heads.argtypes = [i64, i64, i64, i64, i64, i64]
        h.pgqa_tile_splits.restype = ctypes.c_int32
        h.pgqa_tile_splits.argtypes = [i64, i64]
        h.pgqa_decode_part_bytes.restype = ctypes.c_uint64
        h.pgqa_decode_part_bytes.argtypes = [i64, i64, i64, i64]
        h.pgqa_counter_capacity.restype = ctypes.c_int32
        h.pgqa_counter_capacity.argtypes = []
        h.pgqa_last_error.restype = ctypes.c_char_p
        h.pgqa_last_error.argtypes = []
        h.pgqa_attn_decode.restype = ctypes.c_int
        h.pgqa_attn_decode.argtypes = [p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                       p, p, p]
        h.pgqa_prefill_rows_per_tile.restype = ctypes.c_int32
        h.pgqa_prefill_rows_per_tile.argtypes = [i64]
        h.pgqa_make_tiles.restype = ctypes.c_int64
        h.pgqa_make_tiles.argtypes = [p, i64, i64, p, p, i64]
        h.pgqa_attn_prefill.restype = ctypes.c_int
        h.pgqa_attn_prefill.argtypes = [p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, p]
        h.pgqa_attn_decode_noalloc.restype = ctypes.c_int
        h.pgqa_attn_decode_noalloc.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, p]
        h.pgqa_set_merge_wait_ticks.restype = ctypes.c_int32
        h.pgqa_set_merge_wait_ticks.argtypes = [ctypes.c_int32]
        h.pgqa_set_narrow_path.restype = ctypes.c_int32
        h.pgqa_set_narrow_path.argtypes = [ctypes.c_int32]
        h.pgqa_qk_rope_prep.restype = ctypes.c_int
        h.pgqa_qk_rope_prep.argtypes = [p] * 14 + [i64, i64, i64, i64, i64, ctypes.c_float, p]
        _lib = h
    return _lib


def choose_splits(kv_span: int, rows: int, nkv: int, rows_per_seq: int) -> int:
    return int(lib().pgqa_choose_splits(kv_span, rows, nkv, rows_per_seq))


def choose_splits_heads(kv_span: int, rows: int, nh: int, nkv: int, hd: int, rows_per_seq: int) -> int:
    return int(lib().pgqa_choose_splits_heads(kv_span, rows, nh, nkv, hd, rows_per_seq))


def tile_splits(pages: int, splits: int) -> int:
    """Splits a tile of ``pages`` visible KV pages works on (``pgqa_tile_splits``)."""
    return int(lib().pgqa_tile_splits(pages, splits))


def decode_part_bytes(rows: int, nh: int, splits: int, hd: int) -> int:
    return int(lib().pgqa_decode_part_bytes(rows, nh, splits, hd))


def counter_capacity() -> int:
    return int(lib().pgqa_counter_capacity())


def set_narrow_path(mode: int) -> int:
    """Test hook (``pgqa_set_narrow_path``): page step of tiles of at most 4
    columns at hd 64-256 -- 0 the library's choice (default: the vector ALU
    at hd 64 and 128 in launches of more than 512 workgroups), 1 vector ALU,
    2 MFMA; returns the previous mode."""
    rc = int(lib().pgqa_set_narrow_path(mode))
    if rc < 0:
        raise PgqaError(rc, "mode must be 0, 1 or 2")
    return rc


def set_merge_wait_ticks(ticks: int) -> int:
    """Test hook (``pgqa_set_merge_wait_ticks``): bound of the fused merge's
    waits, in 100 MHz ticks (0 = default); returns the previous setting."""
    rc = int(lib().pgqa_set_merge_wait_ticks(ticks))
    if rc < 0:
        raise PgqaError(rc, "ticks must be >= 0")
    return rc


def last_error() -> str:
    return lib().pgqa_last_error().decode()


def _addr(x, name, dtypes=None, min_numel=None):
    """Device address of a tensor (checked) or of a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise PgqaError(EINVAL, f"{name} must be a device tensor")
    if not x.is_contiguous():
        raise PgqaError(EINVAL, f"{name} must be contiguous")
    if dtypes is not None and x.dtype not in dtypes:
        raise PgqaError(EINVAL, f"{name} has dtype {x.dtype}")
    if min_numel is not None and x.numel() < min_numel:
        raise PgqaError(EINVAL, f"{name} has {x.numel()} elements, needs {min_numel}")
    return x.data_ptr()


def attn_decode(out, part, q, k_pool, v_pool, block_table, page_origin, qpos, kv_last,
                rows: int, nh: int, nkv: int, hd: int, window: int, splits: int,
                counters=None, page_map=None, stream=None) -> None:
    """Enqueue one decode call (see ``pgqa_attn_decode`` in include/pgqa.h).

    Tensors: bf16 (or 16-bit integer views of bf16) ``out``/``q`` [rows][nh][hd],
    pools [npages][nkv][16][hd]; int32 ``block_table``, ``page_origin``,
    ``qpos``, ``kv_last``, ``counters``, ``page_map``; ``part`` any dtype with
    at least ``decode_part_bytes`` bytes.  ``stream`` defaults to torch's current
    stream on the tensors' device."""
    import torch

    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    i32 = (torch.int32,)
    n_out = rows * nh * hd
    args = [
        _addr(out, "out", b16, n_out),
        None,
        _addr(q, "q", b16, n_out),
        _addr(k_pool, "k_pool", b16),
        _addr(v_pool, "v_pool", b16),
        _addr(block_table, "block_table", i32),
        _addr(page_origin, "page_origin", i32, rows),
        _addr(qpos, "qpos", i32, rows),
        _addr(kv_last, "kv_last", i32, rows),
    ]
    if part is not None and not isinstance(part, int):
        need = decode_part_bytes(rows, nh, splits, hd) if splits > 1 else 0
        if not part.is_cuda or not part.is_contiguous() or part.numel() * part.element_size() < need:
            raise PgqaError(EINVAL, f"part must be a contiguous device buffer of >= {need} bytes")
        args[1] = part.data_ptr()
    elif isinstance(part, int):
        args[1] = part
    cnt = _addr(counters, "counters", i32, counter_capacity())
    pm = _addr(page_map, "page_map", i32)
    if stream is None:
        dev = out.device if hasattr(out, "device") else None
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = lib().pgqa_attn_decode(*args, rows, nh, nkv, hd, window, splits, cnt, pm, stream)
    if rc != OK:
        raise PgqaError(rc, last_error())


NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_decode_noalloc(out, q, k_pool, v_pool, block_table, page_origin, qpos, kv_last,
                        rows: int, nh: int, nkv: int, hd: int, window: int, splits: int,
                        page_map=None, stream=None) -> None:
    """Enqueue one decode call that allocates nothing (see
    ``pgqa_attn_decode_noalloc`` in include/pgqa.h): partials in the library's
    static device scratch, merged by the separate combine kernel.  Tensors as
    for ``attn_decode``."""
    import torch

    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    i32 = (torch.int32,)
    n_out = rows * nh * hd
    args = [
        _addr(out, "out", b16, n_out),
        _addr(q, "q", b16, n_out),
        _addr(k_pool, "k_pool", b16),
        _addr(v_pool, "v_pool", b16),
        _addr(block_table, "block_table", i32),
        _addr(page_origin, "page_origin", i32, rows),
        _addr(qpos, "qpos", i32, rows),
        _addr(kv_last, "kv_last", i32, rows),
    ]
    pm = _addr(page_map, "page_map", i32)
    if stream is None:
        stream = torch.cuda.current_stream(out.device if hasattr(out, "device") else None).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = lib().pgqa_attn_decode_noalloc(*args, rows, nh, nkv, hd, window, splits, pm, stream)
    if rc != OK:
        raise PgqaError(rc, last_error())


def prefill_rows_per_tile(hd: int) -> int:
    return int(lib().pgqa_prefill_rows_per_tile(hd))


def make_tiles(page_origin, rows_per_tile: int):
    """Prefill tiles from host page origins: (tile_row0, tile_rows) int32 numpy arrays."""
    import numpy as np

    org = np.ascontiguousarray(page_origin, dtype=np.int32)
    n = len(org)
    t0 = np.zeros(max(n, 1), np.int32)
    tn = np.zeros(max(n, 1), np.int32)
    rc = lib().pgqa_make_tiles(org.ctypes.data, n, rows_per_tile, t0.ctypes.data, tn.ctypes.data, len(t0))
    if rc < 0:
        raise PgqaError(int(rc), last_error())
    return t0[:rc].copy(), tn[:rc].copy()


def attn_prefill(out, q, k_pool, v_pool, block_table, page_origin, qpos, kv_last, tile_row0, tile_rows,
                 ntiles: int, rows: int, nh: int, nkv: int, hd: int, window: int, page_map=None,
                 stream=None) -> None:
    """Enqueue one prefill call (see ``pgqa_attn_prefill`` in include/pgqa.h).
    ``tile_row0`` / ``tile_rows`` are int32 device tensors of ``ntiles``."""
    import torch

    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    i32 = (torch.int32,)
    n_out = rows * nh * hd
    args = [
        _addr(out, "out", b16, n_out),
        _addr(q, "q", b16, n_out),
        _addr(k_pool, "k_pool", b16),
        _addr(v_pool, "v_pool", b16),
        _addr(block_table, "block_table", i32),
        _addr(page_origin, "page_origin", i32, rows),
        _addr(qpos, "qpos", i32, rows),
        _addr(kv_last, "kv_last", i32, rows),
        _addr(tile_row0, "tile_row0", i32, ntiles),
        _addr(tile_rows, "tile_rows", i32, ntiles),
    ]
    pm = _addr(page_map, "page_map", i32)
    if stream is None:
        stream = torch.cuda.current_stream(out.device if hasattr(out, "device") else None).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = lib().pgqa_attn_prefill(*args, ntiles, rows, nh, nkv, hd, window, pm, stream)
    if rc != OK:
        raise PgqaError(rc, last_error())


def qk_rope_prep(q_out, k_pool, v_pool, q_in, k_in, v_in, q_weight, k_weight, rope_cos, rope_sin, pos,
                 block_table, page_origin, tokens: int, nh: int, nkv: int, hd: int, rotary_dim: int,
                 eps: float, page_map=None, stream=None) -> None:
    """Enqueue one QK-norm + RoPE prep (see ``pgqa_qk_rope_prep`` in include/pgqa.h).

    bf16 (or 16-bit integer views) ``q_out`` / ``q_in`` [tokens][nh][hd],
    ``k_in`` / ``v_in`` [tokens][nkv][hd] (``v_in`` None: V from ``k_in``),
    pools [npages][nkv][16][hd], weights [hd] or None; f32 rotary tables
    [positions][rotary_dim / 2] (None when rotary_dim is 0); int32 ``pos``,
    ``block_table``, ``page_origin``, ``page_map``."""
    import torch

    b16 = (torch.bfloat16, torch.int16, torch.uint16)
    i32 = (torch.int32,)
    f32 = (torch.float32,)
    nq = tokens * nh * hd
    nk = tokens * nkv * hd
    args = [
        _addr(q_out, "q_out", b16, nq),
        _addr(k_pool, "k_pool", b16),
        _addr(v_pool, "v_pool", b16),
        _addr(q_in, "q_in", b16, nq),
        _addr(k_in, "k_in", b16, nk),
        _addr(v_in, "v_in", b16, nk),
        _addr(q_weight, "q_weight", b16, hd),
        _addr(k_weight, "k_weight", b16, hd),
        _addr(rope_cos, "rope_cos", f32),
        _addr(rope_sin, "rope_sin", f32),
        _addr(pos, "pos", i32, tokens),
        _addr(block_table, "block_table", i32),
        _addr(page_origin, "page_origin", i32, tokens),
        _addr(page_map, "page_map", i32),
    ]
    if stream is None:
        stream = torch.cuda.current_stream(q_out.device if hasattr(q_out, "device") else None).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    rc = lib().pgqa_qk_rope_prep(*args, tokens, nh, nkv, hd, rotary_dim, float(eps), stream)
    if rc != OK:
        raise PgqaError(rc, last_error())
