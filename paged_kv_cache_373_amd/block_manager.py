"""Host-side block manager for the paged KV cache.

It decides where tokens go; the GPU kernels only read and write where it
says.  The rules are the ones the pages walk through:

* [ITH §手動畫一次 block table] (iThome ithelp article 10405755 on
  PagedAttention): a growing sequence fills its last block first and only
  takes a fresh block from the pool when that block is full; nothing already
  cached moves; a finished sequence returns its blocks to the pool.
* [PU §按 Block 分配] (Fanyi Pu, "Infra: PagedAttention"): position t lives at
  offset t % B of the block the table gives for logical block t // B; a length
  T holds ceil(T / B) blocks.
* [PU §共享前缀，分叉时 Copy-on-write]: sequences sampled from one prompt point
  at the same blocks; a per-block reference count says how many sequences use
  a block; a write into a block used by more than one sequence first copies
  the block, re-points the writer's entry at the copy and then writes.  Full
  prefix blocks are never written again and so stay shared.

Pool policy: the free list is a FIFO/LIFO hybrid - blocks are handed out from
its front and released blocks are put back at its front (most recently freed
first).  Any free block would be correct; this one is deterministic given the
initial order.  Running out of blocks raises :class:`PoolExhaustedError`
without changing any state, so a scheduler can wait and retry.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class PoolExhaustedError(RuntimeError):
    pass


def slot_mapping_for(block_tables: np.ndarray, seq_ids: np.ndarray, positions: np.ndarray,
                     block_size: int) -> np.ndarray:
    """Vectorised slot lookup: for each i, the slot of position positions[i]
    of sequence seq_ids[i] (row of ``block_tables``), as int64; positions < 0
    give -1 (skipped by the cache writer)."""
    pos = np.asarray(positions, dtype=np.int64)
    rows = np.asarray(seq_ids, dtype=np.int64)
    out = np.full(pos.shape, -1, dtype=np.int64)
    ok = pos >= 0
    blk = np.asarray(block_tables)[rows[ok], pos[ok] // block_size].astype(np.int64)
    out[ok] = blk * block_size + pos[ok] % block_size
    return out


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(self.num_blocks) if free_order is None else free_order
        self._free = deque(int(b) for b in order)
        if len(self._free) != len(set(self._free)):
            raise ValueError("free_order repeats a block")
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)
        self._tables: Dict[object, List[int]] = {}
        self._lengths: Dict[object, int] = {}

    # -- queries -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def table(self, seq) -> List[int]:
        return list(self._tables[seq])

    def length(self, seq) -> int:
        return self._lengths[seq]

    def slot(self, seq, position: int) -> int:
        table = self._tables[seq]
        return table[position // self.block_size] * self.block_size + position % self.block_size

    def block_table_array(self, seqs: Sequence, width: Optional[int] = None,
                          pad: int = 0) -> np.ndarray:
        """int32 [len(seqs), width] of the tables, padded with ``pad``."""
        w = width if width is not None else max((len(self._tables[s]) for s in seqs), default=1)
        arr = np.full((len(seqs), max(w, 1)), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._tables[s]
            arr[i, :len(t)] = t
        return arr

    def shared_prefix_groups(self, seqs: Sequence) -> Tuple[np.ndarray, np.ndarray]:
        """Groups for shared-prefix decode over the batch ``seqs`` (in batch
        order): runs of consecutive sequences whose tables start with the same
        physical blocks ([PU §共享前缀，分叉时 Copy-on-write]: forks of one
        prompt point at the prompt's blocks).  A group's prefix is the leading
        blocks that every member holds, identical and full in every member
        (a partly filled block is never shared for long: the first divergent
        write copies it).  Returns (group_starts int32 [NG+1], prefix_lens
        int32 [NG], in tokens); a sequence sharing nothing with its neighbours
        is a group of one with prefix 0."""
        bs = self.block_size
        starts: List[int] = [0]
        plens: List[int] = []
        i, n = 0, len(seqs)
        while i < n:
            t0 = self._tables[seqs[i]]
            full0 = self._lengths[seqs[i]] // bs
            common = min(len(t0), full0)
            j = i + 1
            while j < n:
                tj = self._tables[seqs[j]]
                k = min(common, len(tj), self._lengths[seqs[j]] // bs)
                m = 0
                while m < k and tj[m] == t0[m]:
                    m += 1
                if m == 0:
                    break
                common = m
                j += 1
            plens.append(common * bs if j - i > 1 else 0)
            starts.append(j)
            i = j
        return np.asarray(starts, dtype=np.int32), np.asarray(plens, dtype=np.int32)

    # -- mutations -----------------------------------------------------------
    def _pop(self, n: int = 1) -> List[int]:
        if n > len(self._free):
            raise PoolExhaustedError(f"need {n} blocks, {len(self._free)} free")
        blocks = [self._free.popleft() for _ in range(n)]
        self.refcount[blocks] = 1
        return blocks

    def add_sequence(self, seq) -> None:
        if seq in self._tables:
            raise KeyError(f"sequence {seq!r} exists")
        self._tables[seq] = []
        self._lengths[seq] = 0

    def append_tokens(self, seq, count: int) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Reserve the next ``count`` positions of ``seq``.  Returns their
        slots (int64) and the (src, dst) block copies that must run before
        anything is written.  All-or-nothing on pool exhaustion."""
        table = self._tables[seq]
        start = self._lengths[seq]
        bs = self.block_size
        copies: List[Tuple[int, int]] = []
        if count <= 0:
            return np.zeros(0, dtype=np.int64), copies
        end = start + count
        have = len(table)
        need_new = -(-end // bs) - have
        tail_shared = start % bs != 0 and self.refcount[table[start // bs]] > 1
        if need_new + int(tail_shared) > len(self._free):
            raise PoolExhaustedError(
                f"need {need_new + int(tail_shared)} blocks, {len(self._free)} free")
        if tail_shared:
            old = table[start // bs]
            (new,) = self._pop(1)
            copies.append((old, new))
            self.refcount[old] -= 1
            table[start // bs] = new
        if need_new > 0:
            table.extend(self._pop(need_new))
        self._lengths[seq] = end
        pos = np.arange(start, end, dtype=np.int64)
        blk = np.asarray(table, dtype=np.int64)[pos // bs]
        return blk * bs + pos % bs, copies

    def append_token(self, seq) -> Tuple[int, List[Tuple[int, int]]]:
        slots, copies = self.append_tokens(seq, 1)
        return int(slots[0]), copies

    def fork(self, parent, child) -> None:
        """``child`` starts as a copy of ``parent``'s table: every block is
        shared and its reference count goes up by one."""
        if child in self._tables:
            raise KeyError(f"sequence {child!r} exists")
        table = list(self._tables[parent])
        self._tables[child] = table
        self._lengths[child] = self._lengths[parent]
        np.add.at(self.refcount, np.asarray(table, dtype=np.int64), 1)

    def release(self, seq) -> List[int]:
        """Drop ``seq``; returns the blocks that became free."""
        table = self._tables.pop(seq)
        del self._lengths[seq]
        freed = []
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self._free.appendleft(blk)
                freed.append(blk)
        return freed
