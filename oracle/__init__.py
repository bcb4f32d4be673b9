"""TEST INFRASTRUCTURE - the CPU oracle for paged decode attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU path
(``paged_kv_cache_373_amd``) and imports nothing from it.

Sources (cited by title and section):
  [ITH] iThome ithelp article 10405755 on PagedAttention.
  [PU]  Fanyi Pu, "Infra: PagedAttention".
  [AK]  "只用了 8 格，為什麼占了 12 格？" (the paged-attention story page).
Everything here is a plain, direct statement of what those pages define:

* :func:`slot` / :func:`num_blocks_for` - where position t lives and how many
  blocks a length needs ([PU §按 Block 分配]: logical block t//B, offset t%B
  looked up through the table; a length T needs ceil(T/B) blocks).
* :class:`BlockPool` - the block manager the pages walk through: on-demand
  allocation that fills the tail block first and only then takes a free block,
  release back to the pool ([ITH §手動畫一次 block table]), reference counts,
  forks that share blocks and copy-on-write of a shared block before a write
  ([PU §共享前缀，分叉时 Copy-on-write]).
* :func:`write_cache` / :func:`copy_blocks` - the slot-mapped cache write and
  the whole-block copy, as numpy index assignment on bf16 bit patterns.
* :func:`swap_out` / :func:`swap_in` - whole blocks out to host memory and
  back ([AK §故事沒有說完的部分]: pages swapped out under memory pressure and
  swapped back in; a page may come back anywhere, the table finds it).
* :func:`merge_states` - the segment merge o = sum_r Z_r o_r / sum_r Z_r
  evaluated with every Z_r rescaled to the common maximum ([PU §按 Block 分配]).
* :func:`paged_decode` / :func:`dense_decode` - gather K,V into position order
  and run dense softmax attention in fp64 (the C file ``pkv_oracle.c``);
  :func:`paged_decode_py` is the same in pure Python for tiny inputs.
* :func:`paged_prefill` - the causal multi-query form: each new token of a
  sequence attends the positions up to its own ([PU §KV Cache 为什么会浪费
  显存]: causal attention; [PU §Continuous Batching]: paging keeps the dense
  attention semantics); :func:`paged_prefill_py` in pure Python.

Cache layout (the library's documented layout, restated independently):
k_cache bf16 [P, Hkv, B, D], v_cache bf16 [P, Hkv, D, B] (numpy C order).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv_oracle.so")
_lib = None


class PoolExhausted(RuntimeError):
    """No free block is left; the caller must wait or release blocks."""


# ----------------------------------------------------------------------------
# bf16 bit patterns


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# slots and block counts  [PU §按 Block 分配]


def slot(table_row: Sequence[int], t: int, block_size: int) -> int:
    """Slot of position t: physical block table_row[t // B] times B plus the
    in-block offset t % B."""
    return int(table_row[t // block_size]) * block_size + t % block_size


def num_blocks_for(length: int, block_size: int) -> int:
    """Blocks a sequence of `length` tokens occupies: ceil(length / B)."""
    return -(-int(length) // int(block_size))


# ----------------------------------------------------------------------------
# block manager model  [ITH §手動畫一次 block table; PU §共享前缀，分叉时 Copy-on-write]


class BlockPool:
    """Free list + per-sequence tables + reference counts.

    The free list is an ordered list; allocation takes its head and a released
    block is pushed back onto the head.  ``append`` reserves the slot of the
    next position of a sequence: a new block is taken only when the tail block
    is full (or there is none); if the tail block is shared (reference count
    above one) it is first copied to a fresh block and the writer's entry is
    pointed at the copy.  Every copy is reported as a (src, dst) pair."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free: List[int] = (list(range(num_blocks)) if free_order is None
                                else [int(x) for x in free_order])
        self.ref = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    def _take(self) -> int:
        if not self.free:
            raise PoolExhausted("block pool exhausted")
        blk = self.free.pop(0)
        self.ref[blk] = 1
        return blk

    def add(self, seq: int) -> None:
        self.tables[seq] = []
        self.lens[seq] = 0

    def append(self, seq: int) -> Tuple[int, List[Tuple[int, int]]]:
        """Reserve position lens[seq]; return (its slot, copy pairs)."""
        t = self.lens[seq]
        table = self.tables[seq]
        copies: List[Tuple[int, int]] = []
        if t % self.block_size == 0:
            # the tail block is full (or absent): take a new one
            table.append(self._take())
        else:
            tail = table[t // self.block_size]
            if self.ref[tail] > 1:
                new = self._take()
                copies.append((tail, new))
                self.ref[tail] -= 1
                table[t // self.block_size] = new
        self.lens[seq] = t + 1
        return slot(table, t, self.block_size), copies

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of parent (reference counts go up)."""
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.ref[blk] += 1

    def release(self, seq: int) -> None:
        """Drop the sequence's references; blocks nobody uses become free."""
        for blk in self.tables.pop(seq):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.insert(0, blk)
        del self.lens[seq]


# ----------------------------------------------------------------------------
# cache writers (bit copies)


def new_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
              fill: int = 0x7FC0) -> Tuple[np.ndarray, np.ndarray]:
    """(k_cache [P,Hkv,B,D], v_cache [P,Hkv,D,B]) as uint16, filled with `fill`
    (a bf16 NaN by default)."""
    k = np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=np.uint16)
    v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=np.uint16)
    return k, v


def write_cache(k_cache: np.ndarray, v_cache: np.ndarray, k_tok: np.ndarray,
                v_tok: np.ndarray, slots: np.ndarray) -> None:
    """Token n (rows k_tok[n], v_tok[n] of shape [Hkv, D]) goes to slot
    slots[n]: block slots[n] // B, offset slots[n] % B.  Negative slots are
    skipped."""
    block_size = k_cache.shape[2]
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    blk = slots[keep] // block_size
    off = slots[keep] % block_size
    k_cache[blk, :, off, :] = k_tok[keep]
    v_cache[blk, :, :, off] = v_tok[keep]


def copy_blocks(caches: Sequence[np.ndarray], pairs: Sequence[Tuple[int, int]]) -> None:
    """cache[dst] = cache[src] for every cache and every pair, pairs in order."""
    for cache in caches:
        for src, dst in pairs:
            cache[dst] = cache[src]


def swap_out(caches: Sequence[Tuple[np.ndarray, np.ndarray]],
             block_ids: Sequence[int]) -> np.ndarray:
    """Copy whole blocks out to host memory ([AK §故事沒有說完的部分]: when memory
    runs short some requests' pages are swapped out and later swapped back,
    which works because a page can live anywhere and is found through the
    table).  Returns uint16 [L, 2, n, Hkv*B*D]: [l, 0, i] is K block
    block_ids[i] of layer l and [l, 1, i] its V block, each block's elements in
    the cache's own order."""
    ids = np.asarray(block_ids, dtype=np.int64)
    n = ids.shape[0]
    return np.stack([np.stack([kc[ids].reshape(n, -1), vc[ids].reshape(n, -1)])
                     for kc, vc in caches])


def swap_in(caches: Sequence[Tuple[np.ndarray, np.ndarray]], block_ids: Sequence[int],
            buf: np.ndarray) -> None:
    """The way back: block i of ``buf`` (the layout :func:`swap_out` returns)
    becomes block ``block_ids[i]`` of every layer's K and V cache."""
    ids = np.asarray(block_ids, dtype=np.int64)
    for l, (kc, vc) in enumerate(caches):
        kc[ids] = buf[l, 0].reshape((ids.shape[0],) + kc.shape[1:])
        vc[ids] = buf[l, 1].reshape((ids.shape[0],) + vc.shape[1:])


def gather(k_cache: np.ndarray, v_cache: np.ndarray, table_row: Sequence[int],
           length: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows of positions 0..length-1 in position order, [T, Hkv, D]."""
    block_size = k_cache.shape[2]
    ks, vs = [], []
    for t in range(length):
        blk = int(table_row[t // block_size])
        off = t % block_size
        ks.append(k_cache[blk, :, off, :])
        vs.append(v_cache[blk, :, :, off])
    hkv, d = k_cache.shape[1], k_cache.shape[3]
    if not ks:
        return (np.zeros((0, hkv, d), np.uint16), np.zeros((0, hkv, d), np.uint16))
    return np.stack(ks), np.stack(vs)


# ----------------------------------------------------------------------------
# merge of segment results  [PU §按 Block 分配]


def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray) -> np.ndarray:
    """o = sum_r Z_r o_r / sum_r Z_r with ln Z_r = lse_parts[..., r].

    Every Z_r is rescaled by the common maximum M = max_r ln Z_r first
    (w_r = exp(ln Z_r - M)), which changes nothing algebraically and keeps the
    exponentials finite.  Segments with ln Z_r = -inf are empty; rows whose
    segments are all empty give 0.  Shapes: o_parts [..., R, D],
    lse_parts [..., R] -> [..., D], fp64."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isfinite(lse), np.exp(lse - m_safe), 0.0)
    num = np.sum(w[..., None] * np.where(np.isfinite(lse)[..., None], o_parts, 0.0), axis=-2)
    den = np.sum(w, axis=-1, keepdims=True)
    return np.where(empty, 0.0, num / np.where(empty, 1.0, den))


# ----------------------------------------------------------------------------
# attention


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        i32 = ctypes.c_int32
        lib.oracle_paged_decode.argtypes = [u16p, u16p, u16p, i32p, i32p, i32, i32, i32, i32,
                                            i32, i32, ctypes.c_double, f64p, i32]
        lib.oracle_paged_decode.restype = ctypes.c_int
        lib.oracle_dense_decode.argtypes = [u16p, u16p, u16p, i64p, i32, i32, i32, i32,
                                            ctypes.c_double, f64p, i32]
        lib.oracle_dense_decode.restype = ctypes.c_int
        lib.oracle_paged_prefill.argtypes = [u16p, u16p, u16p, i32p, i32p, i64p, i32, i32, i32,
                                             i32, i32, i32, ctypes.c_double, f64p, i32]
        lib.oracle_paged_prefill.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, seq_lens: np.ndarray, scale: float,
                 num_threads: int = 0) -> np.ndarray:
    """fp64 [S, Hq, D]: gather through the tables, then dense attention."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    s, hq, d = q.shape
    _, hkv, bs, d2 = k_cache.shape
    assert d2 == d and v_cache.shape == (k_cache.shape[0], hkv, d, bs)
    out = np.zeros((s, hq, d), dtype=np.float64)
    rc = lib.oracle_paged_decode(_ptr(q, ctypes.c_uint16), _ptr(k_cache, ctypes.c_uint16),
                                 _ptr(v_cache, ctypes.c_uint16), _ptr(bt, ctypes.c_int32),
                                 _ptr(lens, ctypes.c_int32), s, hq, hkv, d, bs, bt.shape[1],
                                 float(scale), _ptr(out, ctypes.c_double), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"oracle_paged_decode failed: {rc}")
    return out


def dense_decode(q: np.ndarray, k_tok: np.ndarray, v_tok: np.ndarray,
                 seq_lens: np.ndarray, scale: float, num_threads: int = 0) -> np.ndarray:
    """fp64 [S, Hq, D] from rows already in position order (sequence-major)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_tok = np.ascontiguousarray(k_tok, dtype=np.uint16)
    v_tok = np.ascontiguousarray(v_tok, dtype=np.uint16)
    lens = np.asarray(seq_lens, dtype=np.int64)
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    s, hq, d = q.shape
    hkv = k_tok.shape[1]
    out = np.zeros((s, hq, d), dtype=np.float64)
    rc = lib.oracle_dense_decode(_ptr(q, ctypes.c_uint16), _ptr(k_tok, ctypes.c_uint16),
                                 _ptr(v_tok, ctypes.c_uint16), _ptr(cu, ctypes.c_int64), s,
                                 hq, hkv, d, float(scale), _ptr(out, ctypes.c_double),
                                 int(num_threads))
    if rc != 0:
        raise RuntimeError(f"oracle_dense_decode failed: {rc}")
    return out


def paged_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  block_tables: np.ndarray, seq_lens: np.ndarray, q_lens: np.ndarray,
                  scale: float, num_threads: int = 0) -> np.ndarray:
    """fp64 [N, Hq, D]: causal multi-query attention of every sequence's new
    tokens (the last q_lens[b] of its seq_lens[b] cached tokens; q rows
    sequence-major) through the tables.  New token i of sequence b sits at
    position T_b - q_len_b + i and sees positions 0 .. that one ([PU §KV Cache
    为什么会浪费显存]: causal attention; [PU §Continuous Batching]: dense
    attention semantics are kept over the paged layout)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint16)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ql = np.asarray(q_lens, dtype=np.int64)
    cu = np.zeros(ql.shape[0] + 1, dtype=np.int64)
    np.cumsum(ql, out=cu[1:])
    n, hq, d = q.shape
    assert n == cu[-1]
    _, hkv, bs, d2 = k_cache.shape
    assert d2 == d and v_cache.shape == (k_cache.shape[0], hkv, d, bs)
    out = np.zeros((n, hq, d), dtype=np.float64)
    rc = lib.oracle_paged_prefill(_ptr(q, ctypes.c_uint16), _ptr(k_cache, ctypes.c_uint16),
                                  _ptr(v_cache, ctypes.c_uint16), _ptr(bt, ctypes.c_int32),
                                  _ptr(lens, ctypes.c_int32), _ptr(cu, ctypes.c_int64),
                                  lens.shape[0], hq, hkv, d, bs, bt.shape[1], float(scale),
                                  _ptr(out, ctypes.c_double), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"oracle_paged_prefill failed: {rc}")
    return out


def paged_prefill_py(q, k_cache, v_cache, block_tables, seq_lens, q_lens, scale) -> np.ndarray:
    """Pure-Python loops, for tiny inputs only: the causal prefill definition
    of :func:`paged_prefill` written a second time, each token's row from its
    own scores."""
    hq, d = q.shape[1], q.shape[2]
    hkv = k_cache.shape[1]
    group = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    row = 0
    for b in range(len(seq_lens)):
        length, nq = int(seq_lens[b]), int(q_lens[b])
        kb, vb = gather(k_cache, v_cache, block_tables[b], length)
        kf, vf = widen_bf16(kb), widen_bf16(vb)
        for i in range(nq):
            pos = length - nq + i
            qf = widen_bf16(q[row])
            for h in range(hq):
                kv = h // group
                scores = []
                for t in range(pos + 1):
                    acc = 0.0
                    for j in range(d):
                        acc += float(qf[h, j]) * float(kf[t, kv, j])
                    scores.append(scale * acc)
                m = max(scores)
                e = [math.exp(x - m) for x in scores]
                z = sum(e)
                for j in range(d):
                    out[row, h, j] = sum(e[t] * float(vf[t, kv, j]) for t in range(pos + 1)) / z
            row += 1
    return out


def paged_decode_py(q, k_cache, v_cache, block_tables, seq_lens, scale) -> np.ndarray:
    """Pure-Python loops, for tiny inputs only: the same definition as
    :func:`paged_decode`, written a second time without numpy vector maths."""
    s, hq, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    out = np.zeros((s, hq, d), dtype=np.float64)
    for b in range(s):
        length = int(seq_lens[b])
        kb, vb = gather(k_cache, v_cache, block_tables[b], length)
        kf, vf, qf = widen_bf16(kb), widen_bf16(vb), widen_bf16(q[b])
        for h in range(hq):
            kv = h // group
            if length == 0:
                continue
            scores = []
            for t in range(length):
                acc = 0.0
                for i in range(d):
                    acc += float(qf[h, i]) * float(kf[t, kv, i])
                scores.append(scale * acc)
            m = max(scores)
            e = [math.exp(x - m) for x in scores]
            z = sum(e)
            for i in range(d):
                out[b, h, i] = sum(e[t] * float(vf[t, kv, i]) for t in range(length)) / z
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (round half to even), returned as fp64.
    Rounds through fp32 first, the way an fp32 result is stored as bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    r = np.where(np.isnan(f), np.uint64(0x7FC00000), r).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)
