"""GPU parity of block swap-out/in (pkv_swap_out / pkv_swap_in): whole blocks
of every layer move to pinned host memory and back, possibly into other
blocks ([AK §故事沒有說完的部分]).  The oracle is numpy gather/scatter on the
same seeded cache contents; bit-exact."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import DEV, GpuSide, bf16_bits, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _caches(seed, layers, P, hkv, bs, d):
    r = workloads.rng(200, 0, seed)
    host = []
    dev = []
    for _ in range(layers):
        k = r.integers(0, 1 << 16, size=(P, hkv, bs, d), dtype=np.uint16)
        v = r.integers(0, 1 << 16, size=(P, hkv, d, bs), dtype=np.uint16)
        host.append((k, v))
        dev.append((torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).to(DEV),
                    torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(DEV)))
    return host, dev


@pytest.mark.parametrize("layers,P,hkv,bs,d,n", [(3, 40, 4, 16, 64, 17), (1, 9, 2, 8, 128, 9),
                                                 (16, 64, 8, 16, 64, 40)])
def test_swap_out_in(layers, P, hkv, bs, d, n):
    say(f"case swap layers={layers} P={P} B={bs} D={d} n={n}")
    host, dev = _caches(layers * 7 + n, layers, P, hkv, bs, d)
    r = workloads.rng(200, 1, n)
    out_ids = r.permutation(P)[:n].astype(np.int32)
    in_ids = r.permutation(P)[:n].astype(np.int32)
    kcs, vcs = [k for k, _ in dev], [v for _, v in dev]
    buf = pkv.swap_buffer(kcs, n)
    pkv.swap_out(kcs, vcs, torch.from_numpy(out_ids).to(DEV), buf)
    torch.cuda.synchronize()
    want = oracle.swap_out(host, out_ids)
    np.testing.assert_array_equal(buf.numpy().view(np.uint16), want)
    # back into other blocks
    pkv.swap_in(kcs, vcs, torch.from_numpy(in_ids).to(DEV), buf)
    torch.cuda.synchronize()
    oracle.swap_in(host, in_ids, want)
    for (k, v), (kd, vd) in zip(host, dev):
        np.testing.assert_array_equal(bf16_bits(kd), k)
        np.testing.assert_array_equal(bf16_bits(vd), v)


def test_swap_refuses_pageable_memory():
    say("case swap pageable host buffer")
    _, dev = _caches(1, 1, 8, 2, 16, 64)
    kc, vc = dev[0]
    ids = torch.arange(2, dtype=torch.int32, device=DEV)
    pageable = np.zeros(2 * 2 * kc[0].numel() + 64, dtype=np.uint16)
    ptr = (pageable.ctypes.data + 15) // 16 * 16
    karr = (ctypes.c_void_p * 1)(kc.data_ptr())
    varr = (ctypes.c_void_p * 1)(vc.data_ptr())
    st = pkv.lib().pkv_swap_out(karr, varr, 1, ids.data_ptr(), 2, kc[0].numel() * 2, ptr,
                                torch.cuda.current_stream().cuda_stream)
    assert st == pkv.PKV_ERR_INVALID
    torch.cuda.synchronize()  # and the stream is still usable


def test_swapped_blocks_found_through_the_table():
    """Swap out every block of a batch, bring the blocks back into other ids,
    re-point the tables: the decode output is the same, bit for bit."""
    say("case swap relocation decode")
    w = workloads.random_small(9, 6, 16, 4, 64, 16, 300, min_len=1, slack_blocks=80)
    g = GpuSide(w)
    before = g.decode(torch.float32).cpu().numpy()
    used = np.unique(np.concatenate([w.block_tables[b, :-(-int(w.seq_lens[b]) // 16)]
                                     for b in range(w.num_seqs)])).astype(np.int32)
    free = np.setdiff1d(np.arange(w.num_blocks), used)[:len(used)].astype(np.int32)
    assert len(free) == len(used)
    buf = pkv.swap_buffer([g.kc], len(used))
    pkv.swap_out([g.kc], [g.vc], torch.from_numpy(used).to(DEV), buf)
    g.kc[torch.from_numpy(used).long().to(DEV)] = float("nan")
    g.vc[torch.from_numpy(used).long().to(DEV)] = float("nan")
    pkv.swap_in([g.kc], [g.vc], torch.from_numpy(free).to(DEV), buf)
    moved = dict(zip(used.tolist(), free.tolist()))
    bt2 = w.block_tables.copy()
    for b in range(w.num_seqs):
        nb = -(-int(w.seq_lens[b]) // 16)
        bt2[b, :nb] = [moved[int(x)] for x in bt2[b, :nb]]
    g.bt = torch.from_numpy(bt2).to(DEV)
    after = g.decode(torch.float32).cpu().numpy()
    np.testing.assert_array_equal(after, before)
    compare(after, oracle.paged_decode(w.q, *_oracle_caches(w), w.block_tables, w.seq_lens,
                                       w.scale), strict_abs=True, what="relocated decode")


def _oracle_caches(w):
    from paritylib import OracleSide
    o = OracleSide(w)
    return o.kc, o.vc
