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

* [PU §共享前缀，分叉时 Copy-on-write], the paragraph on Automatic Prefix
  Caching: requests arriving at different times that start with the same
  tokens reuse the cached full prefix blocks; the lookup key of a block hashes
  the previous block's key, the block's tokens and context ids (a LoRA id, for
  instance), so only a whole matching prefix is reused; only full blocks are
  cached.  :meth:`BlockManager.add_prompt` does this; a cached block whose
  last user leaves stays findable until its space is needed.

Pool policy: the free list is a FIFO/LIFO hybrid - blocks are handed out from
its front and released blocks are put back at its front (most recently freed
first).  Cached blocks nobody uses wait in least-recently-released order and
are taken (forgetting their key) only when the free list is empty.  Any free
block would be correct; this policy is deterministic given the initial order.
Running out of blocks raises :class:`PoolExhaustedError` without changing any
state, so a scheduler can wait and retry.
"""
from __future__ import annotations

import hashlib
from collections import OrderedDict, deque
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


def block_key(prev: Optional[bytes], tokens: Sequence[int], extra: Sequence = ()) -> bytes:
    """Lookup key of a full block: sha256 over the previous block's key (32
    zero bytes for the first block), the block's token ids (int64, little
    endian) and the context ids ``extra``."""
    h = hashlib.sha256()
    h.update(prev if prev is not None else bytes(32))
    h.update(np.asarray(list(tokens), dtype="<i8").tobytes())
    h.update(repr(tuple(extra)).encode())
    return h.digest()


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
        # prefix caching: key <-> block for cached full blocks, cached blocks
        # nobody uses (least recently released first), and per sequence the
        # key of its last full block, its tail tokens and context ids
        self._index: Dict[bytes, int] = {}
        self._key_of: Dict[int, bytes] = {}
        self._idle: "OrderedDict[int, None]" = OrderedDict()
        self._chain: Dict[object, Tuple[Optional[bytes], List[int], tuple]] = {}

    # -- queries -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        """Blocks that can be handed out: free ones and cached ones nobody uses."""
        return len(self._free) + len(self._idle)

    @property
    def num_cached(self) -> int:
        """Full blocks findable by key (in use or not)."""
        return len(self._index)

    def has_sequence(self, seq) -> bool:
        return seq in self._tables

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
        if n > self.num_free:
            raise PoolExhaustedError(f"need {n} blocks, {self.num_free} free")
        blocks = []
        for _ in range(n):
            if self._free:
                blocks.append(self._free.popleft())
            else:  # the least recently released cached block loses its key
                blk, _ = self._idle.popitem(last=False)
                del self._index[self._key_of.pop(blk)]
                blocks.append(blk)
        self.refcount[blocks] = 1
        return blocks

    def _extend_chain(self, seq, new_tokens: Sequence[int]) -> None:
        """``seq`` has just grown by ``new_tokens`` (its length already counts
        them): every block they fill gets its key, chained from the previous
        block's, unless that key or that block is already keyed."""
        prev, tail, extra = self._chain[seq]
        tail = tail + list(new_tokens)
        table, bs = self._tables[seq], self.block_size
        start = self._lengths[seq] - len(tail)  # a block boundary
        while len(tail) >= bs:
            key = block_key(prev, tail[:bs], extra)
            blk = table[start // bs]
            if key not in self._index and blk not in self._key_of:
                self._index[key] = blk
                self._key_of[blk] = key
            prev, tail, start = key, tail[bs:], start + bs
        self._chain[seq] = (prev, tail, extra)

    def add_prompt(self, seq, token_ids: Sequence[int],
                   extra: Sequence = ()) -> Tuple[np.ndarray, int]:
        """Start ``seq`` with the prompt ``token_ids``, reusing cached full
        blocks for its longest prefix whose keys (chained from the first
        block, with context ids ``extra``) are known.  Returns the slots of
        the positions after that prefix, which the caller writes, and the
        number of cached tokens (a multiple of B) whose K/V are already there.
        The prompt's new full blocks become findable at once: the caller
        writes them before another request can read them.  Later tokens keep
        the chain going when :meth:`append_tokens` is given their ids.
        All-or-nothing on pool exhaustion."""
        if seq in self._tables:
            raise KeyError(f"sequence {seq!r} exists")
        toks, bs, extra = [int(t) for t in token_ids], self.block_size, tuple(extra)
        hits, prev = [], None
        for j in range(len(toks) // bs):
            key = block_key(prev, toks[j * bs:(j + 1) * bs], extra)
            blk = self._index.get(key)
            if blk is None:
                break
            hits.append(blk)
            prev = key
        need = -(-len(toks) // bs) - len(hits)
        available = self.num_free - sum(1 for b in hits if b in self._idle)
        if need > available:
            raise PoolExhaustedError(f"need {need} blocks, {available} free")
        for blk in hits:
            self._idle.pop(blk, None)
            self.refcount[blk] += 1
        cached = len(hits) * bs
        self._tables[seq] = hits + self._pop(need)
        self._lengths[seq] = len(toks)
        self._chain[seq] = (prev, [], extra)
        self._extend_chain(seq, toks[cached:])
        pos = np.arange(cached, len(toks), dtype=np.int64)
        blk = np.asarray(self._tables[seq], dtype=np.int64)[pos // bs]
        return blk * bs + pos % bs, cached

    def add_sequence(self, seq) -> None:
        if seq in self._tables:
            raise KeyError(f"sequence {seq!r} exists")
        self._tables[seq] = []
        self._lengths[seq] = 0

    def append_tokens(self, seq, count: int,
                      token_ids: Optional[Sequence[int]] = None
                      ) -> Tuple[np.ndarray, List[Tuple[int, int]]]:
        """Reserve the next ``count`` positions of ``seq``.  Returns their
        slots (int64) and the (src, dst) block copies that must run before
        anything is written.  For a sequence started by :meth:`add_prompt`,
        ``token_ids`` (the tokens placed there) keep its blocks findable as
        they fill; without them its later blocks are not cached.
        All-or-nothing on pool exhaustion."""
        if token_ids is not None and len(token_ids) != count:
            raise ValueError("token_ids must hold count ids")
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
        if need_new + int(tail_shared) > self.num_free:
            raise PoolExhaustedError(
                f"need {need_new + int(tail_shared)} blocks, {self.num_free} free")
        if tail_shared:
            old = table[start // bs]
            (new,) = self._pop(1)
            copies.append((old, new))
            self.refcount[old] -= 1
            table[start // bs] = new
        if need_new > 0:
            table.extend(self._pop(need_new))
        self._lengths[seq] = end
        if seq in self._chain:
            if token_ids is None:
                del self._chain[seq]
            else:
                self._extend_chain(seq, [int(t) for t in token_ids])
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
        if parent in self._chain:
            prev, tail, extra = self._chain[parent]
            self._chain[child] = (prev, list(tail), extra)
        np.add.at(self.refcount, np.asarray(table, dtype=np.int64), 1)

    def release(self, seq) -> List[int]:
        """Drop ``seq``; returns the blocks nobody uses any more.  A cached
        full block among them stays findable (and is handed out again only
        when the free list runs dry); the others go back to the free list."""
        table = self._tables.pop(seq)
        del self._lengths[seq]
        self._chain.pop(seq, None)
        freed = []
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                if blk in self._key_of:
                    self._idle[blk] = None
                else:
                    self._free.appendleft(blk)
                freed.append(blk)
        return freed
