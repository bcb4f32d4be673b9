"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays out *inputs*: sequence
lengths, which physical blocks a sequence owns, and the bf16 bit patterns of
q, K and V for every logical token position.  It contains none of the
method's arithmetic (no slot computation, no cache write, no attention, no
merge), so both the CPU oracle and the GPU path can consume it without
sharing any code with each other.

Shapes follow the synthetic Llama-3.2-1B-shaped cache that the iThome ithelp
article 10405755 on PagedAttention sizes at about 32 KiB per token (bf16, GQA):
8 KV heads x head_dim 64 x 2 (K, V) x 2 bytes x 16 layers = 32768 bytes.

Every draw comes from ``np.random.SeedSequence([373, workload_id, role,
*index])`` so a single sequence (or layer) can be regenerated on its own,
which is how full-size parity tests sample outputs.  Values are fp32 N(0, 1)
rounded to bf16 with round-to-nearest-even (torch's CPU conversion).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

SEED = 373
BF16_NAN = 0x7FC0  # quiet NaN bit pattern used to poison unused cache bytes

# roles of the random streams
_ROLE_LENS, _ROLE_PERM, _ROLE_Q, _ROLE_K, _ROLE_V, _ROLE_PRIV_LEN = range(6)


def rng(workload_id: int, role: int, *index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, workload_id, role, *index]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(g: np.random.Generator, shape, mult: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return to_bf16_bits(x)


@dataclasses.dataclass
class Workload:
    """One decode step's inputs, in logical (per-token) form.

    k_tok / v_tok hold every cached token of every sequence, sequence-major:
    rows cu_seqlens[b] .. cu_seqlens[b+1]-1 are positions 0 .. T_b-1 of
    sequence b; the last row of each sequence is the token being decoded.
    ``block_tables`` is None when the blocks are handed out by an allocator
    from ``free_list`` (the shared-prefix and pool workloads)."""

    name: str
    workload_id: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray  # int32 [S]
    q: np.ndarray  # uint16 [S, Hq, D]
    scale: float
    partition_size: int = 0
    block_tables: Optional[np.ndarray] = None  # int32 [S, MB]
    k_tok: Optional[np.ndarray] = None  # uint16 [sum T, Hkv, D]
    v_tok: Optional[np.ndarray] = None
    free_list: Optional[np.ndarray] = None  # int32, head first
    poison_block: int = -1  # a block that holds only NaN (table padding target)
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int64)
        np.cumsum(self.seq_lens, out=cu[1:])
        return cu

    @property
    def total_tokens(self) -> int:
        return int(np.sum(self.seq_lens, dtype=np.int64))

    def kv_bytes(self) -> int:
        """Bytes of K and V that decode attention must read: every valid
        token's K and V row once per KV head."""
        return self.total_tokens * self.num_kv_heads * self.head_dim * 2 * 2


def _pad_tables(rows: List[List[int]], width: int, pad: int) -> np.ndarray:
    bt = np.full((len(rows), width), pad, dtype=np.int32)
    for b, r in enumerate(rows):
        bt[b, : len(r)] = r
    return bt


def tiny() -> Workload:
    """Three sequences of lengths 7, 9, 4 at B=4 in a pool of 8 blocks with
    tables [7,1], [3,0,4], [2] (the first two are the pages' worked tables);
    4 query heads over 2 KV heads, head_dim 16, scale 1/4.  Blocks 5 and 6
    stay free and hold NaN; table padding points at block 5."""
    wid = 1
    lens = np.array([7, 9, 4], dtype=np.int32)
    hq, hkv, d = 4, 2, 16
    rows = [[7, 1], [3, 0, 4], [2]]
    q = normal_bf16(rng(wid, _ROLE_Q), (3, hq, d))
    n = int(lens.sum())
    k = normal_bf16(rng(wid, _ROLE_K), (n, hkv, d))
    v = normal_bf16(rng(wid, _ROLE_V), (n, hkv, d))
    return Workload("tiny", wid, hq, hkv, d, 4, 8, lens, q, 1.0 / math.sqrt(d),
                    block_tables=_pad_tables(rows, 3, 5), k_tok=k, v_tok=v,
                    poison_block=5)


def _permuted_tables(wid: int, lens: np.ndarray, bs: int, slack: float = 1.1):
    need = [int(math.ceil(t / bs)) for t in lens]
    total = sum(need)
    pool = int(math.ceil(slack * total)) + 1  # +1 keeps a free poison block
    perm = rng(wid, _ROLE_PERM).permutation(pool).astype(np.int32)
    rows, pos = [], 0
    for nb in need:
        rows.append(perm[pos:pos + nb].tolist())
        pos += nb
    poison = int(perm[pos])  # first unused block of the permutation
    width = max(need) if need else 1
    return _pad_tables(rows, max(width, 1), poison), pool, poison


def _llama_shape_tokens(wid: int, lens: np.ndarray, hkv: int, d: int, k_mult: float = 1.0):
    n = int(lens.sum())
    k = normal_bf16(rng(wid, _ROLE_K), (n, hkv, d), mult=k_mult)
    v = normal_bf16(rng(wid, _ROLE_V), (n, hkv, d))
    return k, v


def llama_decode(num_seqs: int = 64, lo: int = 128, hi: int = 2048, wid: int = 2,
                 block_size: int = 16, with_kv: bool = True) -> Workload:
    """Llama-3.2-1B-shaped single-layer decode step: 32 q heads, 8 KV heads,
    head_dim 64, B=16, batch 64, lengths uniform on the integers [128, 2048],
    physical blocks a seeded permutation of a pool 10 % larger than needed."""
    hq, hkv, d = 32, 8, 64
    lens = rng(wid, _ROLE_LENS).integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int32)
    bt, pool, poison = _permuted_tables(wid, lens, block_size)
    q = normal_bf16(rng(wid, _ROLE_Q), (num_seqs, hq, d))
    k = v = None
    if with_kv:
        k, v = _llama_shape_tokens(wid, lens, hkv, d)
    return Workload("llama_b64", wid, hq, hkv, d, block_size, pool, lens, q,
                    1.0 / math.sqrt(d), block_tables=bt, k_tok=k, v_tok=v,
                    poison_block=poison)


def long_context(num_seqs: int = 8, lo: int = 16384, hi: int = 32768, wid: int = 3,
                 with_kv: bool = True) -> Workload:
    """Long-context split-KV: the Llama head shape, batch 8, lengths uniform on
    [16384, 32768], 512-token partitions, K multiplied by 3 before rounding."""
    hq, hkv, d, bs = 32, 8, 64, 16
    lens = rng(wid, _ROLE_LENS).integers(lo, hi, size=num_seqs, endpoint=True).astype(np.int32)
    bt, pool, poison = _permuted_tables(wid, lens, bs)
    q = normal_bf16(rng(wid, _ROLE_Q), (num_seqs, hq, d))
    k = v = None
    if with_kv:
        k, v = _llama_shape_tokens(wid, lens, hkv, d, k_mult=3.0)
    return Workload("long_splitkv", wid, hq, hkv, d, bs, pool, lens, q,
                    1.0 / math.sqrt(d), partition_size=512, block_tables=bt,
                    k_tok=k, v_tok=v, poison_block=poison)


def prefix_sharing(num_prompts: int = 4, prompt_len: int = 1000, forks: int = 16,
                   max_new: int = 300, wid: int = 4) -> Workload:
    """Shared prompts with copy-on-write forks: 4 prompts of 1000 tokens
    (B=16: 62 full blocks plus an 8-token tail), 16 forks per prompt that each
    append 1..300 private tokens.  Blocks come from a seeded shuffled free
    list; the sharing structure is built by the caller's block manager.

    k_tok/v_tok hold each fork's full logical sequence (prompt rows repeated
    per fork) so that consumers need no knowledge of the sharing; ``extra``
    records the geometry."""
    hq, hkv, d, bs = 32, 8, 64, 16
    s = num_prompts * forks
    n_priv = rng(wid, _ROLE_PRIV_LEN).integers(1, max_new, size=s, endpoint=True).astype(np.int32)
    lens = (prompt_len + n_priv).astype(np.int32)
    prompt_blocks = int(math.ceil(prompt_len / bs))
    # worst case: every fork copies its tail and grows by ceil(300/16)+1 blocks
    need = num_prompts * prompt_blocks + sum(int(math.ceil(t / bs)) for t in lens)
    pool = int(math.ceil(1.1 * need))
    free = rng(wid, _ROLE_PERM).permutation(pool).astype(np.int32)
    pk = normal_bf16(rng(wid, _ROLE_K), (num_prompts, prompt_len, hkv, d))
    pv = normal_bf16(rng(wid, _ROLE_V), (num_prompts, prompt_len, hkv, d))
    ks, vs = [], []
    for b in range(s):
        p = b // forks
        gk = rng(wid, _ROLE_K, 1, b)
        gv = rng(wid, _ROLE_V, 1, b)
        ks.append(pk[p]); ks.append(normal_bf16(gk, (int(n_priv[b]), hkv, d)))
        vs.append(pv[p]); vs.append(normal_bf16(gv, (int(n_priv[b]), hkv, d)))
    q = normal_bf16(rng(wid, _ROLE_Q), (s, hq, d))
    return Workload("prefix_cow", wid, hq, hkv, d, bs, pool, lens, q,
                    1.0 / math.sqrt(d), k_tok=np.concatenate(ks), v_tok=np.concatenate(vs),
                    free_list=free,
                    extra=dict(num_prompts=num_prompts, prompt_len=prompt_len,
                               forks=forks, n_private=n_priv))


POOL_SLOTS = 1 << 22
POOL_LAYERS = 16
POOL_SIGMA = 1.0  # the lognormal spread is not stated; 1.0 is the reading taken


def pool_lengths(num_seqs: int = 256, median: float = 1200.0, sigma: float = POOL_SIGMA,
                 cap: int = 8192, wid: int = 5) -> np.ndarray:
    x = rng(wid, _ROLE_LENS).lognormal(mean=math.log(median), sigma=sigma, size=num_seqs)
    return np.clip(np.ceil(x), 1, cap).astype(np.int32)


def pool_step(block_size: int, num_seqs: int = 256, wid: int = 5) -> Workload:
    """Full 16-layer decode step at pool scale: batch 256, lognormal lengths
    (median 1200, sigma 1.0, capped at 8192), 2^22 token slots per layer, a
    seeded shuffled free list (B in {8, 16, 32}).  K/V/q are drawn per
    (layer, sequence) by :func:`pool_layer_tokens` / :func:`pool_layer_q`
    because the full step holds ~15 GB of KV."""
    hq, hkv, d = 32, 8, 64
    lens = pool_lengths(num_seqs, wid=wid)
    pool = POOL_SLOTS // block_size
    free = rng(wid, _ROLE_PERM, block_size).permutation(pool).astype(np.int32)
    q0 = pool_layer_q(0, num_seqs, wid)
    return Workload(f"pool16_b{block_size}", wid, hq, hkv, d, block_size, pool, lens, q0,
                    1.0 / math.sqrt(d), free_list=free,
                    extra=dict(num_layers=POOL_LAYERS))


def pool_layer_q(layer: int, num_seqs: int = 256, wid: int = 5) -> np.ndarray:
    return normal_bf16(rng(wid, _ROLE_Q, layer), (num_seqs, 32, 64))


def pool_layer_tokens_device(layer: int, num_tokens: int, device, block_size: int,
                             wid: int = 5):
    """K and V (bf16 [num_tokens, 8, 64]) of every token of one layer of the
    pool workload, drawn on the device: the full step holds ~15 GB of KV,
    too much to draw on the host.  torch's seeded device generator, N(0, 1)
    rounded to bf16; sampled rows are copied back for the oracle."""
    import torch

    seed = int(np.random.SeedSequence([SEED, wid, _ROLE_K, layer, block_size]).generate_state(1)[0])
    g = torch.Generator(device=device).manual_seed(seed)
    k = torch.randn((num_tokens, 8, 64), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((num_tokens, 8, 64), generator=g, device=device, dtype=torch.float32)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def pool_layer_tokens(layer: int, seq: int, length: int, wid: int = 5):
    """K and V (bf16 bits, [length, 8, 64]) of one sequence in one layer."""
    k = normal_bf16(rng(wid, _ROLE_K, layer, seq), (length, 8, 64))
    v = normal_bf16(rng(wid, _ROLE_V, layer, seq), (length, 8, 64))
    return k, v


def random_small(seed: int, num_seqs: int, hq: int, hkv: int, d: int, bs: int,
                 max_len: int, min_len: int = 0, slack_blocks: int = 3,
                 k_mult: float = 1.0, lens=None) -> Workload:
    """Small random case for parity sweeps: lengths uniform on
    [min_len, max_len] (or the given ``lens``), blocks a random permutation
    of the pool."""
    wid = 100
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int32)
        assert len(lens) == num_seqs
    else:
        lens = rng(wid, _ROLE_LENS, seed).integers(min_len, max_len, size=num_seqs,
                                                   endpoint=True).astype(np.int32)
    need = [int(math.ceil(t / bs)) for t in lens]
    pool = sum(need) + slack_blocks
    perm = rng(wid, _ROLE_PERM, seed).permutation(pool).astype(np.int32)
    rows, pos = [], 0
    for nb in need:
        rows.append(perm[pos:pos + nb].tolist())
        pos += nb
    poison = int(perm[pos])
    width = max(max(need) if need else 1, 1)
    bt = _pad_tables(rows, width, poison)
    n = int(lens.sum())
    q = normal_bf16(rng(wid, _ROLE_Q, seed), (num_seqs, hq, d))
    k = normal_bf16(rng(wid, _ROLE_K, seed), (n, hkv, d), mult=k_mult)
    v = normal_bf16(rng(wid, _ROLE_V, seed), (n, hkv, d))
    return Workload(f"random{seed}", wid, hq, hkv, d, bs, pool, lens, q,
                    1.0 / math.sqrt(d), block_tables=bt, k_tok=k, v_tok=v,
                    poison_block=poison)


def shared_prefix_small(seed: int, group_sizes: List[int], prefix_blocks: List[int], hq: int,
                        hkv: int, d: int, bs: int, max_suffix: int, min_suffix: int = 0,
                        empty_tail: bool = False) -> Workload:
    """Small shared-prefix case: group g is group_sizes[g] consecutive
    sequences whose tables start with the same prefix_blocks[g] physical
    blocks (the group's prompt, drawn once), each followed by a private
    suffix of U{min_suffix..max_suffix} tokens in blocks of its own.  With
    ``empty_tail`` a last group of one empty sequence is appended.  Blocks are
    a seeded permutation of the pool.  k_tok/v_tok hold every sequence's full
    logical sequence (the prompt rows repeated per member); ``extra`` holds
    group_starts, prefix_lens and ``repeat_rows``, the k_tok rows that repeat a
    prompt row already held by the group's first member."""
    wid = 101
    sizes = list(group_sizes) + ([1] if empty_tail else [])
    pblocks = list(prefix_blocks) + ([0] if empty_tail else [])
    s = sum(sizes)
    suf = rng(wid, _ROLE_PRIV_LEN, seed).integers(min_suffix, max_suffix, size=s,
                                                  endpoint=True).astype(np.int32)
    if empty_tail:
        suf[-1] = 0
    owner = np.repeat(np.arange(len(sizes)), sizes)
    lens = (np.asarray(pblocks, dtype=np.int32)[owner] * bs + suf).astype(np.int32)
    need = sum(pblocks) + sum(int(math.ceil(int(x) / bs)) for x in suf)
    pool = need + 3
    perm = rng(wid, _ROLE_PERM, seed).permutation(pool).astype(np.int32)
    pos = 0
    rows: List[List[int]] = []
    prompts_k, prompts_v = [], []
    for g, (n, pb) in enumerate(zip(sizes, pblocks)):
        shared = perm[pos:pos + pb].tolist()
        pos += pb
        prompts_k.append(normal_bf16(rng(wid, _ROLE_K, seed, g), (pb * bs, hkv, d)))
        prompts_v.append(normal_bf16(rng(wid, _ROLE_V, seed, g), (pb * bs, hkv, d)))
        for _ in range(n):
            b = len(rows)
            nb = int(math.ceil(int(suf[b]) / bs))
            rows.append(shared + perm[pos:pos + nb].tolist())
            pos += nb
    poison = int(perm[pos])
    width = max(max(len(r) for r in rows), 1)
    bt = _pad_tables(rows, width, poison)
    ks, vs, repeat = [], [], []
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    for b in range(s):
        g = int(owner[b])
        ks.append(prompts_k[g])
        vs.append(prompts_v[g])
        repeat.append(np.full(len(prompts_k[g]), b != starts[g]))
        ks.append(normal_bf16(rng(wid, _ROLE_K, seed, 1000 + b), (int(suf[b]), hkv, d)))
        vs.append(normal_bf16(rng(wid, _ROLE_V, seed, 1000 + b), (int(suf[b]), hkv, d)))
        repeat.append(np.zeros(int(suf[b]), bool))
    q = normal_bf16(rng(wid, _ROLE_Q, seed), (s, hq, d))
    return Workload(f"shared_prefix{seed}", wid, hq, hkv, d, bs, pool, lens, q,
                    1.0 / math.sqrt(d), block_tables=bt, k_tok=np.concatenate(ks),
                    v_tok=np.concatenate(vs), poison_block=poison,
                    extra=dict(group_starts=starts,
                               prefix_lens=(np.asarray(pblocks) * bs).astype(np.int32),
                               repeat_rows=np.concatenate(repeat)))


def prefill_small(seed: int, num_seqs: int, hq: int, hkv: int, d: int, bs: int, max_ctx: int,
                  max_q: int, min_q: int = 1, min_ctx: int = 0, slack_blocks: int = 3,
                  wid: int = 102) -> Workload:
    """Prefill / chunked-prefill case: sequence b holds ctx_b cached tokens
    (U{min_ctx..max_ctx}) followed by q_len_b new ones (U{min_q..max_q}), all
    T_b = ctx_b + q_len_b of them in the cache; ``q`` holds the new tokens'
    queries, sequence-major ([sum q_len, Hq, D]); ``extra["q_lens"]`` their
    counts.  Blocks are a seeded permutation of the pool."""
    ctx = rng(wid, _ROLE_LENS, seed).integers(min_ctx, max_ctx, size=num_seqs,
                                              endpoint=True).astype(np.int32)
    ql = rng(wid, _ROLE_PRIV_LEN, seed).integers(min_q, max_q, size=num_seqs,
                                                 endpoint=True).astype(np.int32)
    lens = (ctx + ql).astype(np.int32)
    need = [int(math.ceil(t / bs)) for t in lens]
    pool = sum(need) + slack_blocks
    perm = rng(wid, _ROLE_PERM, seed).permutation(pool).astype(np.int32)
    rows, pos = [], 0
    for nb in need:
        rows.append(perm[pos:pos + nb].tolist())
        pos += nb
    poison = int(perm[pos])
    bt = _pad_tables(rows, max(max(need) if need else 1, 1), poison)
    n = int(lens.sum())
    q = normal_bf16(rng(wid, _ROLE_Q, seed), (int(ql.sum()), hq, d))
    k = normal_bf16(rng(wid, _ROLE_K, seed), (n, hkv, d))
    v = normal_bf16(rng(wid, _ROLE_V, seed), (n, hkv, d))
    return Workload(f"prefill{seed}", wid, hq, hkv, d, bs, pool, lens, q, 1.0 / math.sqrt(d),
                    block_tables=bt, k_tok=k, v_tok=v, poison_block=poison,
                    extra=dict(q_lens=ql))


def prefill_chunked(num_seqs: int = 8, q_len: int = 512, max_ctx: int = 2048,
                    wid: int = 7) -> Workload:
    """Llama-3.2-1B-shaped chunked prefill step of one layer: 8 sequences each
    adding a 512-token chunk after a cached context of U{0..2048} tokens (32 q
    heads, 8 KV heads, head_dim 64, B = 16), physical blocks a seeded
    permutation of a pool 10 % larger than needed."""
    hq, hkv, d, bs = 32, 8, 64, 16
    ctx = rng(wid, _ROLE_LENS).integers(0, max_ctx, size=num_seqs, endpoint=True).astype(np.int32)
    ql = np.full(num_seqs, q_len, dtype=np.int32)
    lens = (ctx + ql).astype(np.int32)
    bt, pool, poison = _permuted_tables(wid, lens, bs)
    q = normal_bf16(rng(wid, _ROLE_Q), (int(ql.sum()), hq, d))
    k, v = _llama_shape_tokens(wid, lens, hkv, d)
    return Workload("prefill_chunked", wid, hq, hkv, d, bs, pool, lens, q, 1.0 / math.sqrt(d),
                    block_tables=bt, k_tok=k, v_tok=v, poison_block=poison,
                    extra=dict(q_lens=ql))
