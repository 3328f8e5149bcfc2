"""Seeded synthetic inputs for paged GQA decode attention.

This module only *produces inputs*: random bf16 tensors, paged K/V pools, block
tables, per-row page origins, positions and page maps.  It holds none of the
attention arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``paged_gqa_decode_attn_amd``) can be fed from it without sharing any of the
method's code.

Generator.  The pages' GPU test for span-02 (``engine/crates/kernels/tests/gpu.rs``,
the ``Rng`` helper) draws test data from a 64-bit LCG with multiplier
6364136223846793005 and increment 1442695040888963407.  We keep that state
recurrence and the draw order (K pool, then V pool, then Q), but map the state
to ``x = (state >> 40) * 2^-23 - 1``, which lies exactly in [-1, 1): the page's
own mapping only reaches [-1, 0).  ``x`` is exact in f32 and is turned into
bf16 by truncation (the page's ``bf`` helper keeps the top 16 bits).

Pool layout (same page, ``reference`` and ``mapped_pool`` helpers): K and V are
separate bf16 pools ``[page][nkv][16][hd]``; token ``p`` of kv head ``kh`` for a
row whose table starts at ``origin`` sits in physical page
``block_table[origin + p // 16]`` (then through the page map, if any) at slot
``p % 16``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

PAGE = 16  # tokens per page (the pool layout fixes it)
BF16_QNAN = 0x7FC0  # bf16 quiet NaN the page fills its null page with

_MUL = 6364136223846793005
_INC = 1442695040888963407
_MASK = (1 << 64) - 1

_tables: dict = {}


def _jump_tables(n: int):
    """Affine maps s -> A[k]*s + C[k] (mod 2^64) for k = 1..n LCG steps."""
    best = _tables.get("t")
    if best is not None and len(best[0]) >= n:
        return best[0][:n], best[1][:n]
    a = np.array([_MUL], dtype=np.uint64)
    c = np.array([_INC], dtype=np.uint64)
    while len(a) < n:
        an, cn = np.uint64(int(a[-1])), np.uint64(int(c[-1]))
        # step k + m = (step k) o (step m):  A_{k+m} = A_k A_m,  C_{k+m} = A_k C_m + C_k
        a, c = np.concatenate([a, a * an]), np.concatenate([c, a * cn + c])
    _tables["t"] = (a, c)
    return a[:n], c[:n]


class Lcg:
    """64-bit LCG with the span-02 test's constants; vectorised by jump-ahead."""

    BLOCK = 1 << 22

    def __init__(self, seed: int):
        self.state = seed & _MASK

    def step(self) -> int:
        self.state = (self.state * _MUL + _INC) & _MASK
        return self.state

    def u32(self) -> int:
        """High 32 bits of the state after one step (integer draws)."""
        return self.step() >> 32

    def states(self, n: int) -> np.ndarray:
        """The next ``n`` states, as uint64, advancing the generator by ``n``."""
        out = np.empty(n, dtype=np.uint64)
        done = 0
        while done < n:
            m = min(self.BLOCK, n - done)
            a, c = _jump_tables(m)
            blk = a * np.uint64(self.state) + c
            out[done:done + m] = blk
            self.state = int(blk[-1])
            done += m
        return out

    def uniform_bf16(self, n: int, scale: float = 1.0) -> np.ndarray:
        """``n`` bf16 bit patterns of ``scale * x``, x uniform in [-1, 1)."""
        out = np.empty(n, dtype=np.uint16)
        done = 0
        sc = np.float32(scale)
        while done < n:
            m = min(self.BLOCK, n - done)
            a, c = _jump_tables(m)
            blk = a * np.uint64(self.state) + c
            self.state = int(blk[-1])
            x = (blk >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -23) - np.float32(1.0)
            if scale != 1.0:
                x = x * sc
            out[done:done + m] = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            done += m
        return out


@dataclasses.dataclass
class Workload:
    """One decode call's inputs, all host numpy arrays (bf16 as uint16 bits)."""

    name: str
    rows: int
    nh: int
    nkv: int
    hd: int
    window: int
    q: np.ndarray  # uint16 [rows, nh, hd]
    k_pool: np.ndarray  # uint16 [npages, nkv, 16, hd]
    v_pool: np.ndarray  # uint16 [npages, nkv, 16, hd]
    block_table: np.ndarray  # int32
    page_origin: np.ndarray  # int32 [rows]
    qpos: np.ndarray  # int32 [rows]
    kv_last: np.ndarray  # int32 [rows]
    page_map: Optional[np.ndarray] = None  # int32, indexed by block-table entry
    note: str = ""

    @property
    def npages(self) -> int:
        return int(self.k_pool.shape[0])

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _draw_pools(rng: Lcg, npages: int, nkv: int, hd: int, k_scale: float = 1.0):
    n = npages * nkv * PAGE * hd
    k = rng.uniform_bf16(n, k_scale).reshape(npages, nkv, PAGE, hd)
    v = rng.uniform_bf16(n).reshape(npages, nkv, PAGE, hd)
    return k, v


def single_sequence(name: str, ctx: int, rows: int, nh: int, nkv: int, hd: int,
                    window: int, seed: Optional[int] = None, k_scale: float = 1.0) -> Workload:
    """The span-02 ``run()`` fixture: rows at positions ctx-rows..ctx-1 of one
    sequence, ``ceil(ctx/16) + 1`` pool pages (one spare), identity block table,
    origin 0.  Seed defaults to ``12345 + hd`` as on the page."""
    rng = Lcg(12345 + hd if seed is None else seed)
    npg = (ctx + PAGE - 1) // PAGE + 1
    k, v = _draw_pools(rng, npg, nkv, hd, k_scale)
    q = rng.uniform_bf16(rows * nh * hd).reshape(rows, nh, hd)
    bt = np.arange((ctx + PAGE - 1) // PAGE, dtype=np.int32)
    qpos = np.arange(ctx - rows, ctx, dtype=np.int32)
    return Workload(name, rows, nh, nkv, hd, window, q, k, v, bt,
                    np.zeros(rows, np.int32), qpos, qpos.copy())


def first_live_page(w: Workload) -> int:
    """Lowest logical page any row can see (row 0's window start // 16), as the
    page's page-map fixture computes it; 0 for global (window 0) layers."""
    if w.window <= 0:
        return 0
    q0 = int(w.qpos[0])
    lo_row = q0 + 1 - min(w.window, q0 + 1)
    return lo_row // PAGE


def mapped_pool(k: np.ndarray, v: np.ndarray, first_live: int):
    """Permuted copy of a ``[npg][nkv][16][hd]`` pool behind a page map.

    The result has ``npg + 1`` pages.  Physical page 0 is a null page filled with
    bf16 NaN; logical page ``p >= first_live`` lives at physical page ``npg - p``;
    the map sends logical pages below ``first_live`` to the null page."""
    npg = k.shape[0]
    mk = np.full((npg + 1,) + k.shape[1:], BF16_QNAN, dtype=np.uint16)
    mv = np.full((npg + 1,) + v.shape[1:], BF16_QNAN, dtype=np.uint16)
    pmap = np.zeros(npg, dtype=np.int32)
    for p in range(first_live, npg):
        s = npg - p
        pmap[p] = s
        mk[s] = k[p]
        mv[s] = v[p]
    return mk, mv, pmap


def with_page_map(w: Workload, first_live: Optional[int] = None) -> Workload:
    """Same logical K/V as ``w`` (identity table) in a permuted pool + page map."""
    fl = first_live_page(w) if first_live is None else first_live
    mk, mv, pmap = mapped_pool(w.k_pool, w.v_pool, fl)
    return w.replace(name=w.name + "+pagemap", k_pool=mk, v_pool=mv, page_map=pmap,
                     note=f"permuted pool, first_live={fl}, null page 0 = NaN")


def batched(name: str = "C4", nseq: int = 64, lmin: int = 512, lmax: int = 16384,
            nh: int = 32, nkv: int = 8, hd: int = 128, window: int = 0,
            len_seed: int = 777, data_seed: int = 12345 + 128, pad: int = 16,
            nan_tail: bool = False) -> Workload:
    """Batched decode: ``nseq`` sequences, one query row each, at their last position.

    Lengths ``L_s = lmin + u32 % (lmax - lmin + 1)`` from ``Lcg(len_seed)``; each
    sequence holds ``ceil(L_s/16)`` pages.  Physical pages ``1..N`` are shuffled
    (Fisher-Yates, same generator) and dealt to the sequences in order, so each
    sequence is a random permutation inside one shared pool.  Physical page 0 is
    a NaN null page.  The block table starts with ``pad`` entries pointing at the
    null page, then every sequence's pages; row ``s`` has origin
    ``pad + sum(P_<s)`` (distinct, non-zero; reading a pad entry returns NaN).
    K, V (physical pages 1..N in order) and Q come from ``Lcg(data_seed)``.  With
    ``nan_tail`` the unused slots of each sequence's last page are NaN too."""
    r = Lcg(len_seed)
    lens = [lmin + r.u32() % (lmax - lmin + 1) for _ in range(nseq)]
    pages = [(L + PAGE - 1) // PAGE for L in lens]
    total = sum(pages)
    perm = list(range(1, total + 1))
    for i in range(total - 1, 0, -1):
        j = r.u32() % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    bt = np.array([0] * pad + perm, dtype=np.int32)
    origins = np.cumsum([0] + pages[:-1]).astype(np.int64) + pad
    rng = Lcg(data_seed)
    npages = total + 1
    k = np.empty((npages, nkv, PAGE, hd), dtype=np.uint16)
    v = np.empty((npages, nkv, PAGE, hd), dtype=np.uint16)
    k[0] = BF16_QNAN
    v[0] = BF16_QNAN
    n = total * nkv * PAGE * hd
    k[1:] = rng.uniform_bf16(n).reshape(total, nkv, PAGE, hd)
    v[1:] = rng.uniform_bf16(n).reshape(total, nkv, PAGE, hd)
    q = rng.uniform_bf16(nseq * nh * hd).reshape(nseq, nh, hd)
    if nan_tail:
        for s, L in enumerate(lens):
            used = L % PAGE
            if used:
                phys = bt[origins[s] + pages[s] - 1]
                k[phys, :, used:, :] = BF16_QNAN
                v[phys, :, used:, :] = BF16_QNAN
    qpos = np.array([L - 1 for L in lens], dtype=np.int32)
    return Workload(name, nseq, nh, nkv, hd, window, q, k, v, bt,
                    origins.astype(np.int32), qpos, qpos.copy(),
                    note=f"{nseq} seqs, lengths U[{lmin},{lmax}] seed {len_seed}")


# ---------------------------------------------------------------------------
# The named workloads.  C1..C5 are the decode shapes this project is measured
# on; PA and PB are the two shapes the span-02 test runs
# (``attention_matches_reference``).
# ---------------------------------------------------------------------------

def make(name: str) -> Workload:
    n = name.upper()
    if n == "C1":
        return single_sequence("C1", ctx=64, rows=1, nh=4, nkv=1, hd=64, window=0)
    if n == "C2":
        return single_sequence("C2", ctx=4096, rows=4, nh=16, nkv=8, hd=256, window=1024)
    if n == "C3":
        return single_sequence("C3", ctx=32768, rows=1, nh=16, nkv=2, hd=512, window=0)
    if n == "C4":
        return batched("C4")
    if n == "C4NAN":
        return batched("C4nan", nan_tail=True)
    if n in ("C5", "C5W0"):
        return single_sequence("C5w0", ctx=131072, rows=8, nh=8, nkv=1, hd=256, window=0, k_scale=8.0)
    if n == "C5W4096":
        return single_sequence("C5w4096", ctx=131072, rows=8, nh=8, nkv=1, hd=256, window=4096,
                               k_scale=8.0)
    if n == "PA":
        return single_sequence("PA", ctx=1500, rows=5, nh=16, nkv=8, hd=256, window=1024)
    if n == "PB":
        return single_sequence("PB", ctx=700, rows=1, nh=16, nkv=2, hd=512, window=0)
    raise KeyError(name)


NAMES = ("C1", "C2", "C3", "C4", "C4nan", "C5w0", "C5w4096", "PA", "PB")


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Inputs of the QK-norm + RoPE prep (the step that fills the pool before
# decode; pegainfer pull request page #1002).  Per token: raw query, key and
# value heads, the norm weights and the rotary tables, a position, and the
# page addressing of the decode workloads above.
# ---------------------------------------------------------------------------

def _bf16_trunc(x: np.ndarray) -> np.ndarray:
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rope_tables(positions: int, rotary_dim: int, base: float = 10000.0):
    """Rotary tables ``cos[p][i], sin[p][i]`` of the angle ``p * base^(-2i /
    rotary_dim)`` for ``i < rotary_dim / 2``: computed in f64, stored as f32
    (the prep takes the tables as inputs, as the page's fixtures build them)."""
    half = rotary_dim // 2
    if half == 0:
        return np.zeros((max(positions, 1), 1), np.float32), np.zeros((max(positions, 1), 1), np.float32)
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclasses.dataclass
class PrepWorkload:
    """One prep call's inputs (host numpy; bf16 as uint16 bits).  ``v_in``
    None is the K = V form; ``q_w`` / ``k_w`` None mean weight 1."""

    name: str
    nh: int
    nkv: int
    hd: int
    rotary_dim: int
    eps: float
    q_in: np.ndarray  # uint16 [tokens, nh, hd]
    k_in: np.ndarray  # uint16 [tokens, nkv, hd]
    v_in: Optional[np.ndarray]  # uint16 [tokens, nkv, hd] or None
    q_w: Optional[np.ndarray]  # uint16 [hd]
    k_w: Optional[np.ndarray]  # uint16 [hd]
    rope_cos: np.ndarray  # f32 [positions, max(rotary_dim / 2, 1)]
    rope_sin: np.ndarray
    pos: np.ndarray  # int32 [tokens]
    block_table: np.ndarray  # int32
    page_origin: np.ndarray  # int32 [tokens]
    npages: int
    page_map: Optional[np.ndarray] = None
    note: str = ""

    @property
    def tokens(self) -> int:
        return int(self.pos.shape[0])

    def zero_pools(self):
        shape = (self.npages, self.nkv, PAGE, self.hd)
        return np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)

    def replace(self, **kw) -> "PrepWorkload":
        return dataclasses.replace(self, **kw)


def _prep_data(rng: Lcg, tokens: int, nh: int, nkv: int, hd: int, kv_equal: bool, weights: bool):
    q = rng.uniform_bf16(tokens * nh * hd).reshape(tokens, nh, hd)
    k = rng.uniform_bf16(tokens * nkv * hd).reshape(tokens, nkv, hd)
    v = None if kv_equal else rng.uniform_bf16(tokens * nkv * hd).reshape(tokens, nkv, hd)
    qw = kw = None
    if weights:  # 1 + x / 2, x uniform in [-1, 1): weights in [0.5, 1.5)
        qw = _bf16_trunc(1.0 + 0.5 * bf16_bits_to_f32(rng.uniform_bf16(hd)))
        kw = _bf16_trunc(1.0 + 0.5 * bf16_bits_to_f32(rng.uniform_bf16(hd)))
    return q, k, v, qw, kw


def prep_prefill(name: str, tokens: int, nh: int, nkv: int, hd: int, rotary_dim: int, p0: int = 0,
                 kv_equal: bool = False, weights: bool = True, eps: float = 1e-6, base: float = 10000.0,
                 seed: Optional[int] = None, shuffle: bool = True) -> PrepWorkload:
    """Prefill form: positions ``p0 .. p0 + tokens - 1`` of one sequence, every
    token at origin 0 of a table of ``ceil((p0 + tokens) / 16)`` entries.  The
    sequence's pages are physical pages ``1..P``, shuffled (Fisher-Yates on
    ``Lcg(seed + 1)``) unless ``shuffle`` is False; physical page 0 is never
    in the table (a sentinel that must stay untouched).  Data from
    ``Lcg(seed)``, seed ``24680 + hd`` by default."""
    seed = 24680 + hd if seed is None else seed
    npg = (p0 + tokens + PAGE - 1) // PAGE
    perm = list(range(1, npg + 1))
    if shuffle:
        r = Lcg(seed + 1)
        for i in range(npg - 1, 0, -1):
            j = r.u32() % (i + 1)
            perm[i], perm[j] = perm[j], perm[i]
    q, k, v, qw, kw = _prep_data(Lcg(seed), tokens, nh, nkv, hd, kv_equal, weights)
    pos = np.arange(p0, p0 + tokens, dtype=np.int32)
    cos_t, sin_t = rope_tables(p0 + tokens, rotary_dim, base)
    return PrepWorkload(name, nh, nkv, hd, rotary_dim, eps, q, k, v, qw, kw, cos_t, sin_t, pos,
                        np.array(perm, np.int32), np.zeros(tokens, np.int32), npg + 1,
                        note=f"prefill positions {p0}..{p0 + tokens - 1}")


def prep_decode(name: str, nseq: int, lmin: int, lmax: int, nh: int, nkv: int, hd: int, rotary_dim: int,
                kv_equal: bool = False, weights: bool = True, eps: float = 1e-6, base: float = 10000.0,
                len_seed: int = 777, seed: Optional[int] = None, pad: int = 16) -> PrepWorkload:
    """Batched decode form: one new token per sequence, at position ``L_s - 1``
    of a sequence of length ``L_s`` (lengths and the page shuffle drawn as in
    ``batched``), so every token has its own distinct, non-zero origin into
    one concatenated table whose first ``pad`` entries point at physical page
    0 (a sentinel that must stay untouched)."""
    seed = 24680 + hd if seed is None else seed
    r = Lcg(len_seed)
    lens = [lmin + r.u32() % (lmax - lmin + 1) for _ in range(nseq)]
    pages = [(L + PAGE - 1) // PAGE for L in lens]
    total = sum(pages)
    perm = list(range(1, total + 1))
    for i in range(total - 1, 0, -1):
        j = r.u32() % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    bt = np.array([0] * pad + perm, dtype=np.int32)
    origins = (np.cumsum([0] + pages[:-1]) + pad).astype(np.int32)
    q, k, v, qw, kw = _prep_data(Lcg(seed), nseq, nh, nkv, hd, kv_equal, weights)
    pos = np.array([L - 1 for L in lens], dtype=np.int32)
    cos_t, sin_t = rope_tables(int(pos.max()) + 1, rotary_dim, base)
    return PrepWorkload(name, nh, nkv, hd, rotary_dim, eps, q, k, v, qw, kw, cos_t, sin_t, pos, bt,
                        origins, total + 1, note=f"{nseq} seqs, lengths U[{lmin},{lmax}] seed {len_seed}")


def compress_windows(w: PrepWorkload, pad: Optional[int] = None) -> PrepWorkload:
    """The same tokens, each behind its own table window that starts at the
    token's own page -- what a caller that released the front of a sequence
    passes.  Token t's window (the rest of its table from entry
    ``origin_t + pos_t // 16``) is copied to its own place in a new table after
    ``pad`` entries that point at physical page 0; its origin becomes
    ``place_t - pos_t // 16`` (distinct, non-zero).  Every token's slot resolves
    to the same physical page as before."""
    first = [int(w.page_origin[t]) + int(w.pos[t]) // PAGE for t in range(w.tokens)]
    pad = max(int(w.pos.max()) // PAGE + 1, 1) if pad is None else pad
    parts = [np.zeros(pad, np.int32)]
    origins = np.empty(w.tokens, np.int32)
    place = pad
    for t in range(w.tokens):
        span = w.block_table[first[t]:first[t] + 2]  # the token's page and the next
        origins[t] = place - int(w.pos[t]) // PAGE
        parts.append(np.asarray(span, np.int32))
        place += len(span)
    return w.replace(name=w.name + "+compressed", block_table=np.concatenate(parts),
                     page_origin=origins, note=w.note + ", per-token compressed windows")


def prep_with_page_map(w: PrepWorkload) -> PrepWorkload:
    """Every table entry ``e`` goes through a page map: the table is replaced
    by ``0..len-1`` (identity entries) and ``page_map[e]`` is the physical page
    the entry held; page 0 stays the untouched sentinel."""
    return w.replace(name=w.name + "+pagemap", page_map=np.asarray(w.block_table, np.int32).copy(),
                     block_table=np.arange(len(w.block_table), dtype=np.int32),
                     note=w.note + ", through a page map")


def make_prep(name: str) -> PrepWorkload:
    """Named prep shapes: hd 256 with full and partial rotation, hd 512 with
    V = K and rotary_dim 128 (the two gate families on the page), and the
    decode shapes' hd 128 / 64 with the batched decode form."""
    n = name.upper()
    if n == "R256F":
        return prep_prefill("R256F", tokens=48, nh=16, nkv=8, hd=256, rotary_dim=256, p0=5)
    if n == "R256P":
        return prep_prefill("R256P", tokens=40, nh=16, nkv=8, hd=256, rotary_dim=128, p0=21)
    if n == "R512KV":
        return prep_prefill("R512KV", tokens=36, nh=16, nkv=2, hd=512, rotary_dim=128, p0=3, kv_equal=True,
                            base=1000000.0)
    if n == "R128D":
        return prep_decode("R128D", nseq=64, lmin=17, lmax=2000, nh=32, nkv=8, hd=128, rotary_dim=128)
    if n == "R64D":
        return prep_decode("R64D", nseq=9, lmin=1, lmax=300, nh=4, nkv=1, hd=64, rotary_dim=32,
                           weights=False)
    if n == "R128P8K":
        return prep_prefill("R128P8K", tokens=8192, nh=32, nkv=8, hd=128, rotary_dim=128)
    raise KeyError(name)


PREP_NAMES = ("R256F", "R256P", "R512KV", "R128D", "R64D")


# ---------------------------------------------------------------------------
# Window-edge sentinels.  The visibility rule (span-02 GPU test page,
# ``reference``: causal, and inside a sliding window when one is set) decides
# which keys of a loaded page a row may read.  These inputs make a one-key slip
# at either edge of any row's visible range change that row's output by O(1):
#   * a slot of a loaded page that no row of the sequence can see holds NaN in
#     K and V (reading it, or multiplying its V by a zero weight, gives NaN);
#   * a slot just outside row t's range (lo_t - 1 or hi_t + 1) that another
#     row of the same sequence does see holds a key aimed at one head of row t
#     in every kv group: K = c * sign(q[t, h]), c = 4 * max|K| of the pool.
#     Row t's score for it would be c * sum|q[t, h]|, far above every real
#     score, so including it turns head h of row t into that key's V row.
# ---------------------------------------------------------------------------

def row_ranges(w: Workload):
    """Per row: (lo, hi) visible key range (hi < lo: nothing visible)."""
    lo = np.where(w.window > 0, np.maximum(0, w.qpos.astype(np.int64) + 1 - w.window), 0)
    return [(int(lo[t]), int(w.kv_last[t])) for t in range(w.rows)]


def plant_edges(w: Workload, name: Optional[str] = None) -> Workload:
    """``w`` with NaN in every slot of a loaded page that no row of its
    sequence sees and a dominant key at every window edge that another row of
    the sequence sees (see above).  Rows that share a page origin share a
    sequence; a sequence's loaded pages are those from its lowest visible key's
    page to its highest's.  Returns a new workload (pools copied)."""
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    g = w.nh // w.nkv
    kmag = float(np.abs(bf16_bits_to_f32(w.k_pool[np.isfinite(bf16_bits_to_f32(w.k_pool))])).max(initial=1.0))
    c = np.float32(2.0 ** np.ceil(np.log2(4.0 * kmag)))  # a power of two: exact in bf16
    rng = row_ranges(w)
    seqs = {}
    for t in range(w.rows):
        seqs.setdefault(int(w.page_origin[t]), []).append(t)

    def slot(origin, p):
        phys = int(w.block_table[origin + p // PAGE])
        if w.page_map is not None:
            phys = int(w.page_map[phys])
        return phys, p % PAGE

    for origin, rows in seqs.items():
        live = [(rng[t][0], rng[t][1]) for t in rows if rng[t][1] >= rng[t][0]]
        if not live:
            continue
        p_lo = min(a for a, _ in live) // PAGE * PAGE
        p_hi = (max(b for _, b in live) // PAGE + 1) * PAGE - 1
        seen = np.zeros(p_hi - p_lo + 1, bool)
        for a, b in live:
            seen[a - p_lo:b - p_lo + 1] = True
        for p in range(p_lo, p_hi + 1):
            if not seen[p - p_lo]:
                phys, s = slot(origin, p)
                k[phys, :, s, :] = BF16_QNAN
                v[phys, :, s, :] = BF16_QNAN
        taken = set()
        for t in rows:
            a, b = rng[t]
            if b < a:
                continue
            for e in (a - 1, b + 1):
                if e < p_lo or e > p_hi or not seen[e - p_lo] or e in taken:
                    continue
                taken.add(e)
                phys, s = slot(origin, e)
                for kh in range(w.nkv):
                    h = kh * g + t % g
                    neg = (w.q[t, h] & 0x8000) != 0
                    row = np.where(neg, -c, c).astype(np.float32)
                    k[phys, kh, s, :] = (row.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return w.replace(name=name or w.name + "+edges", k_pool=k, v_pool=v,
                     note=w.note + ", window-edge sentinels")


def edge_batch(name: str, nseq: int, lmin: int, lmax: int, nh: int, nkv: int, hd: int, window: int,
               len_seed: int = 4242) -> Workload:
    """A batch of one-row sequences whose visible ranges start and end inside a
    page (so the slots at lo - 1 and hi + 1 sit in pages the kernels load):
    row s sits a few keys before its sequence's last written slot, chosen so
    that hi % 16 != 15 and, with a window, lo % 16 != 0.  With window-edge
    sentinels planted."""
    b = batched(name, nseq=nseq, lmin=lmin, lmax=lmax, nh=nh, nkv=nkv, hd=hd, window=window,
                len_seed=len_seed, pad=16)
    qp = b.qpos.astype(np.int64).copy()
    for s in range(nseq):
        for back in range(1, 40):
            x = int(b.qpos[s]) - back
            lo = x + 1 - window if window > 0 else 1
            if x >= 0 and x % PAGE != PAGE - 1 and (window <= 0 or (lo > 0 and lo % PAGE != 0)):
                qp[s] = x
                break
    qp = qp.astype(np.int32)
    return plant_edges(b.replace(qpos=qp, kv_last=qp.copy()), name=name)
