"""GPU tests of the input checkers (pkv_check_decode_inputs,
pkv_check_slot_mapping, pkv_check_block_pairs).  Consistent inputs give 0;
inputs made inconsistent on the host give exactly the documented bits.  The
checkers only compare values, so the inconsistent inputs here are never used
to address memory.  Table and slot rules: [ITH §手動畫一次 block table],
[PU §按 Block 分配]; copy pairs: [PU §共享前缀，分叉时 Copy-on-write]."""
import numpy as np
import pytest
import torch

import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _tables(w):
    return (torch.from_numpy(w.block_tables).to(DEV),
            torch.from_numpy(w.seq_lens.astype(np.int32)).to(DEV))


def test_decode_inputs():
    say("case check decode inputs")
    w = workloads.random_small(41, 40, 8, 2, 64, 16, 300, min_len=0)
    bt, lens = _tables(w)
    mx = int(w.seq_lens.max())
    assert pkv.check_decode_inputs(bt, lens, w.num_blocks, 16, mx) == 0
    # table padding past ceil(T/B) is never examined
    b = int(np.argmax(w.seq_lens < 16 * (w.block_tables.shape[1] - 1)))
    pad = w.block_tables.copy()
    pad[b, -1] = -7
    assert pkv.check_decode_inputs(torch.from_numpy(pad).to(DEV), lens, w.num_blocks, 16, mx) == 0
    # a used entry out of range
    b = int(np.argmax(w.seq_lens > 0))
    bad = w.block_tables.copy()
    bad[b, (int(w.seq_lens[b]) - 1) // 16] = w.num_blocks
    assert pkv.check_decode_inputs(torch.from_numpy(bad).to(DEV), lens, w.num_blocks, 16, mx) == 1
    # a length above the bound, and a negative one
    ll = w.seq_lens.astype(np.int32).copy()
    ll[3] = mx + 1
    assert pkv.check_decode_inputs(bt, torch.from_numpy(ll).to(DEV), w.num_blocks, 16, mx) == 2
    ll[3] = -1
    assert pkv.check_decode_inputs(bt, torch.from_numpy(ll).to(DEV), w.num_blocks, 16, mx) == 2
    # both at once
    assert pkv.check_decode_inputs(torch.from_numpy(bad).to(DEV), torch.from_numpy(ll).to(DEV),
                                   w.num_blocks, 16, mx) == 3
    # the flag word starts clear on every call
    assert pkv.check_decode_inputs(bt, lens, w.num_blocks, 16, mx) == 0


@pytest.mark.parametrize("n", [1, 255, 256, 257, 3000])
def test_slot_mapping(n):
    say(f"case check slot mapping n={n}")
    rng = np.random.default_rng(n)
    nslots = 16 * ((4 * n + 31) // 16)  # whole blocks of 16 slots
    slots = rng.permutation(nslots)[:n].astype(np.int64)
    if n > 2:
        slots[1] = -1
        slots[2] = -1  # padding may repeat
    t = torch.from_numpy(slots).to(DEV)
    assert pkv.check_slot_mapping(t, nslots // 16, 16) == 0
    if n > 1:
        dup = slots.copy()
        dup[-1] = dup[0]
        assert pkv.check_slot_mapping(torch.from_numpy(dup).to(DEV), nslots // 16, 16) == 2
    over = slots.copy()
    over[n // 2] = nslots
    assert pkv.check_slot_mapping(torch.from_numpy(over).to(DEV), nslots // 16, 16) & 1


@pytest.mark.parametrize("n", [1, 60, 300])
def test_block_pairs(n):
    say(f"case check block pairs n={n}")
    rng = np.random.default_rng(100 + n)
    P = 3 * n + 8
    ids = rng.permutation(P)[:2 * n].astype(np.int32)
    pairs = np.stack([ids[:n], ids[n:]], axis=1).copy()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    assert pkv.check_block_pairs(t(pairs), P) == 0
    out = pairs.copy()
    out[n - 1, 0] = P
    assert pkv.check_block_pairs(t(out), P) == 1
    if n > 1:
        dd = pairs.copy()
        dd[1, 1] = dd[0, 1]
        assert pkv.check_block_pairs(t(dd), P) == 2
        ds = pairs.copy()
        ds[1, 1] = ds[0, 0]  # pair 1 writes the block pair 0 reads
        assert pkv.check_block_pairs(t(ds), P) == 4
    # a pair copying a block onto itself: its dst is a src
    same = pairs.copy()
    same[0, 1] = same[0, 0]
    assert pkv.check_block_pairs(t(same), P) & 4


def test_workloads_pass_their_checks():
    """The tables, slot mappings and copy pairs the other tests and the
    benchmark build are consistent."""
    say("case check workloads")
    w = workloads.llama_decode()
    bt, lens = _tables(w)
    assert pkv.check_decode_inputs(bt, lens, w.num_blocks, w.block_size,
                                   int(w.seq_lens.max())) == 0
    from paged_kv_cache_373_amd.block_manager import slot_mapping_for
    seq = np.repeat(np.arange(w.num_seqs), w.seq_lens)
    pos = np.concatenate([np.arange(t) for t in w.seq_lens])
    slots = torch.from_numpy(slot_mapping_for(w.block_tables, seq, pos, w.block_size)).to(DEV)
    assert pkv.check_slot_mapping(slots, w.num_blocks, w.block_size) == 0
