"""Iteration-level batching of decode rounds over the block manager.

[PU §Continuous Batching] (Fanyi Pu, "Infra: PagedAttention"): a decode round
produces one token for every running sequence; with continuous batching the
batch is re-formed every round - finished requests leave at the end of a
round and waiting requests join at the start of the next one as far as slots
and memory allow - instead of a static batch that admits new requests only
once all of its members are done.

Host logic only: :class:`Batcher` decides which requests run in each round
and keeps their blocks in a :class:`BlockManager` (a prompt's blocks when it
joins, one more token per round, everything released when it finishes).
What the device computes in a round is the decode step of the running
sequences (``paged_attention_decode_append``).
"""
from __future__ import annotations

from collections import OrderedDict, deque
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

from .block_manager import BlockManager, PoolExhaustedError


@dataclass
class Request:
    """A request: its prompt length, the decode rounds it needs (tokens to
    generate) and the round after which it is ready (0: from the start)."""
    rid: object
    prompt_len: int
    rounds: int
    ready_after: int = 0
    prompt_tokens: Optional[Sequence[int]] = None  # enables prefix-cache reuse


class Batcher:
    """``policy`` "continuous" refills free slots every round; "static" admits
    only when the whole running batch has finished.  ``max_running`` is the
    number of slots.  A request joins only if the block manager can hold its
    prompt and every running sequence's next token, its own included;
    otherwise it waits (first come, first served: a request that does not fit
    holds back the ones behind it)."""

    def __init__(self, bm: BlockManager, max_running: int, policy: str = "continuous"):
        if policy not in ("continuous", "static") or max_running < 1:
            raise ValueError("policy is 'continuous' or 'static', max_running >= 1")
        self.bm, self.max_running, self.policy = bm, int(max_running), policy
        self.round = 0  # rounds completed
        self._waiting: deque = deque()
        self._running: "OrderedDict[object, int]" = OrderedDict()  # rid -> rounds left
        self.cached_tokens: Dict[object, int] = {}

    def add(self, req: Request) -> None:
        self._waiting.append(req)

    @property
    def running(self) -> List[object]:
        return list(self._running)

    @property
    def idle(self) -> bool:
        return not self._waiting and not self._running

    def _admit(self) -> None:
        if self.policy == "static" and self._running:
            return
        while self._waiting and len(self._running) < self.max_running:
            req = self._waiting[0]
            if req.ready_after > self.round:
                break
            try:
                if req.prompt_tokens is not None:
                    _, cached = self.bm.add_prompt(req.rid, req.prompt_tokens)
                else:
                    cached = 0
                    self.bm.add_sequence(req.rid)
                    self.bm.append_tokens(req.rid, req.prompt_len)
            except PoolExhaustedError:
                if self.bm.has_sequence(req.rid):
                    self.bm.release(req.rid)
                break
            # this round's tokens, the newcomer's included, must fit as well
            if self._round_blocks([*self._running, req.rid]) > self.bm.num_free:
                self.bm.release(req.rid)
                break
            self.cached_tokens[req.rid] = cached
            self._waiting.popleft()
            self._running[req.rid] = req.rounds

    def _round_blocks(self, rids) -> int:
        """Blocks a round's new tokens take: one per sequence whose next
        position starts a block."""
        bs = self.bm.block_size
        return sum(1 for rid in rids if self.bm.length(rid) % bs == 0)

    def step(self) -> List[object]:
        """One decode round: admit what may join, give every running request
        its new token's slot, retire those that are done.  Returns the
        requests that ran this round, in admission order."""
        self._admit()
        batch = list(self._running)
        for rid in batch:
            self.bm.append_tokens(rid, 1)
            self._running[rid] -= 1
        for rid in batch:
            if self._running[rid] == 0:
                del self._running[rid]
                self.bm.release(rid)
        self.round += 1
        return batch
