"""Pins of the CPU oracle to facts that do not come from the oracle itself:
the pages' worked examples (tests/golden/*.json, each with its citation),
closed forms of softmax attention, a library routine (torch's
scaled_dot_product_attention in fp64 on the CPU) and pure-Python brute force.

A plausible slip in the oracle fails at least one of these:
  slot / table lookup (t//B vs t%B, wrong block)  -> page traces, SDPA check
  cache layout index                             -> layout golden, SDPA check
  GQA head mapping, scale, sign of the max shift -> SDPA check, closed forms
  merge weights                                  -> Z = 3, 1 pin
  allocation / copy-on-write / release           -> page traces
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import load_golden

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ---------------------------------------------------------------- page facts


def test_ith_block_table_trace():
    g = load_golden("ith_block_table_trace.json")
    pool = oracle.BlockPool(8, g["block_size"], free_order=g["free_list_head"])
    pool.add(0)
    for _ in range(g["prompt_tokens"]):
        pool.append(0)
    assert pool.tables[0] == g["table_after_prompt"]
    free_before = len(pool.free)
    s7, c7 = pool.append(0)
    assert (s7, pool.tables[0], c7) == (g["append_position_7"]["slot"],
                                        g["append_position_7"]["table"], [])
    assert len(pool.free) == free_before  # no new block
    s8, c8 = pool.append(0)
    assert (s8, pool.tables[0], c8) == (g["append_position_8"]["slot"],
                                        g["append_position_8"]["table"], [])
    assert len(pool.free) == free_before - 1
    pool.release(0)
    assert sorted(set(pool.free) & set(g["released_blocks"])) == g["released_blocks"]
    assert len(pool.free) == 8 and all(r == 0 for r in pool.ref)


def test_pu_table_lookup():
    g = load_golden("pu_table_lookup.json")
    b, t = g["block_size"], g["position"]
    assert t // b == g["logical_block"]
    assert g["table"][t // b] == g["physical_block"] and t % b == g["offset"]
    assert oracle.slot(g["table"], t, b) == g["slot"]
    nb = oracle.num_blocks_for(g["length"], b)
    assert nb == g["blocks"] and nb * b == g["slots"]
    assert nb * b - g["length"] == g["empty_tail_slots"]


def test_block_count_law_property():
    r = np.random.default_rng(7)
    for _ in range(2000):
        b = int(r.integers(1, 65))
        t = int(r.integers(0, 5000))
        nb = oracle.num_blocks_for(t, b)
        assert nb == math.ceil(t / b)
        assert 0 <= nb * b - t < b  # tail waste is below one block
        # an allocator run ends with exactly that many blocks
        if t <= 300:
            pool = oracle.BlockPool(nb + 2, b)
            pool.add(0)
            slots = [pool.append(0)[0] for _ in range(t)]
            assert len(pool.tables[0]) == nb
            assert len(set(slots)) == t


def test_pu_copy_on_write_trace():
    g = load_golden("pu_copy_on_write.json")
    pool = oracle.BlockPool(5, g["block_size"], free_order=g["free_list_head"])
    pool.add("B")
    for _ in range(g["shared_tokens"]):
        pool.append("B")
    assert pool.tables["B"] == g["table_before"]
    pool.fork("B", "A")
    s_a, pairs = pool.append("A")
    assert [list(p) for p in pairs] == g["copy_pairs_on_A_write"]
    s_b, pairs_b = pool.append("B")
    assert pairs_b == []  # B is now the only user of P0: writes in place
    assert pool.tables["A"] == g["table_A"] and pool.tables["B"] == g["table_B"]
    for blk, rc in g["refcount"].items():
        assert pool.ref[int(blk)] == rc
    assert s_a == g["slot_A_position_6"] and s_b == g["slot_B_position_6"]


def test_copy_blocks_then_write_keeps_prefix():
    # bytes: after the copy the new block equals the old one, and each writer's
    # token lands in its own block
    kc, vc = oracle.new_cache(5, 2, 4, 16)
    r = np.random.default_rng(3)
    toks = r.integers(0, 0x7F00, size=(7, 2, 16), dtype=np.uint16)
    pool = oracle.BlockPool(5, 4, free_order=[3, 0, 4, 1, 2])
    pool.add("B")
    slots = [pool.append("B")[0] for _ in range(6)]
    oracle.write_cache(kc, vc, toks[:6], toks[:6], np.array(slots))
    pool.fork("B", "A")
    s_a, pairs = pool.append("A")
    oracle.copy_blocks([kc, vc], pairs)
    np.testing.assert_array_equal(kc[4], kc[0])
    np.testing.assert_array_equal(vc[4], vc[0])
    oracle.write_cache(kc, vc, toks[6:7], toks[6:7], np.array([s_a]))
    ka, _ = oracle.gather(kc, vc, pool.tables["A"], 7)
    kb, _ = oracle.gather(kc, vc, pool.tables["B"], 6)
    np.testing.assert_array_equal(ka[:6], toks[:6])
    np.testing.assert_array_equal(ka[6], toks[6])
    np.testing.assert_array_equal(kb, toks[:6])


def test_pool_exhaustion_leaves_state():
    pool = oracle.BlockPool(2, 4)
    pool.add(0)
    for _ in range(8):
        pool.append(0)
    with pytest.raises(oracle.PoolExhausted):
        pool.append(0)


def test_merge_z_3_1():
    g = load_golden("pu_merge.json")
    z = np.array(g["Z"])
    o1 = np.array([1.0, -2.0, 0.5, 8.0])
    o2 = np.array([-3.0, 4.0, 0.25, 0.0])
    want = g["weights"][0] * o1 + g["weights"][1] * o2
    got = oracle.merge_states(np.stack([o1, o2])[None], np.log(z)[None])[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    # the page's literal form, computed directly
    literal = (z[0] * o1 + z[1] * o2) / (z[0] + z[1])
    np.testing.assert_allclose(got, literal, rtol=1e-15, atol=1e-15)
    # shifting every ln Z by the same amount changes nothing and cannot overflow
    for shift in (1e3, -1e3, 700.0):
        got2 = oracle.merge_states(np.stack([o1, o2])[None], (np.log(z) + shift)[None])[0]
        # (ln 3 + 1e3 carries ~1e-13 absolute rounding, hence the looser bound)
        np.testing.assert_allclose(got2, want, rtol=1e-12, atol=1e-12)


def test_merge_equals_unsplit_softmax():
    # splitting a softmax into segments and merging is the unsplit softmax
    r = np.random.default_rng(11)
    s = r.normal(size=50) * 4
    v = r.normal(size=(50, 8))
    p = np.exp(s - s.max())
    full = p @ v / p.sum()
    cuts = [0, 7, 8, 30, 50]
    os_, ls = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        e = np.exp(s[a:b])
        os_.append(e @ v[a:b] / e.sum())
        ls.append(np.log(e.sum()))
    got = oracle.merge_states(np.stack(os_)[None], np.array(ls)[None])[0]
    np.testing.assert_allclose(got, full, rtol=1e-12, atol=1e-13)


def test_merge_empty_segments():
    o = np.array([[[5.0, 5.0], [1.0, 2.0]]])
    lse = np.array([[-np.inf, 0.3]])
    np.testing.assert_array_equal(oracle.merge_states(o, lse)[0], [1.0, 2.0])
    lse2 = np.array([[-np.inf, -np.inf]])
    np.testing.assert_array_equal(oracle.merge_states(o, lse2)[0], [0.0, 0.0])


def test_layout_offsets():
    g = load_golden("layout_offsets.json")
    p, h, b, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    for c in g["cases"]:
        kc, vc = oracle.new_cache(p, h, b, d, fill=0)
        tok = np.zeros((1, h, d), np.uint16)
        tok[0, c["head"], c["dim"]] = 0x3F80  # 1.0
        oracle.write_cache(kc, vc, tok, tok, np.array([c["block"] * b + c["offset"]]))
        assert np.flatnonzero(kc.reshape(-1)).tolist() == [c["k_flat"]]
        assert np.flatnonzero(vc.reshape(-1)).tolist() == [c["v_flat"]]


def test_sizing_32kib_per_token():
    g = load_golden("sizing.json")
    w = workloads.llama_decode(num_seqs=2, with_kv=False)
    per_layer = w.num_kv_heads * w.head_dim * g["bytes_per_element"] * g["tensors"]
    assert per_layer * g["num_layers"] == g["bytes_per_token"] == 32768
    w.seq_lens[:] = [1, 0]
    assert w.kv_bytes() * g["num_layers"] == g["bytes_per_token"]


# ---------------------------------------------------------------- attention


def _oracle_cache(w):
    kc, vc = oracle.new_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    cu = w.cu_seqlens
    slots = np.concatenate([
        np.array([oracle.slot(w.block_tables[b], t, w.block_size) for t in range(w.seq_lens[b])],
                 dtype=np.int64) for b in range(w.num_seqs)])
    oracle.write_cache(kc, vc, w.k_tok, w.v_tok, slots)
    assert slots.shape[0] == cu[-1]
    return kc, vc


def _sdpa_f64(w):
    """torch's own attention routine, fp64 on the CPU, over the logical rows."""
    out = np.zeros((w.num_seqs, w.num_q_heads, w.head_dim))
    cu = w.cu_seqlens
    qf = oracle.widen_bf16(w.q)
    for b in range(w.num_seqs):
        if w.seq_lens[b] == 0:
            continue
        k = torch.from_numpy(oracle.widen_bf16(w.k_tok[cu[b]:cu[b + 1]])).permute(1, 0, 2)
        v = torch.from_numpy(oracle.widen_bf16(w.v_tok[cu[b]:cu[b + 1]])).permute(1, 0, 2)
        q = torch.from_numpy(qf[b])[:, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None].contiguous(), v[None].contiguous(), scale=w.scale, enable_gqa=True)
        out[b] = o[0, :, 0, :].numpy()
    return out


CASES = [
    lambda: workloads.tiny(),
    lambda: workloads.random_small(1, 5, 8, 2, 32, 4, 40),
    lambda: workloads.random_small(2, 4, 6, 6, 8, 3, 25, k_mult=3.0),
    lambda: workloads.random_small(3, 3, 16, 1, 64, 16, 70),
    lambda: workloads.random_small(4, 6, 4, 4, 24, 1, 9, min_len=0),
]


@pytest.mark.parametrize("make", CASES)
def test_paged_oracle_matches_torch_sdpa(make):
    w = make()
    kc, vc = _oracle_cache(w)
    got = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    want = _sdpa_f64(w)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    dense = oracle.dense_decode(w.q, w.k_tok, w.v_tok, w.seq_lens, w.scale)
    np.testing.assert_allclose(dense, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("make", CASES[:3])
def test_paged_oracle_matches_brute_force(make):
    w = make()
    kc, vc = _oracle_cache(w)
    got = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    want = oracle.paged_decode_py(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def _single(q, k, v, scale):
    """one sequence, Hq = Hkv = 1, rows given in position order (bf16 bits)."""
    t, d = k.shape
    kc, vc = oracle.new_cache(max(1, -(-t // 4)) + 1, 1, 4, d)
    table = np.arange(max(1, -(-t // 4)), dtype=np.int32)[None]
    slots = np.array([oracle.slot(table[0], i, 4) for i in range(t)], dtype=np.int64)
    oracle.write_cache(kc, vc, k[:, None], v[:, None], slots)
    return oracle.paged_decode(q[None, None], kc, vc, table, np.array([t], np.int32), scale)[0, 0]


def test_closed_form_single_token_returns_v():
    r = np.random.default_rng(5)
    q, k, v = (workloads.normal_bf16(r, (16,)), workloads.normal_bf16(r, (1, 16)),
               workloads.normal_bf16(r, (1, 16)))
    np.testing.assert_array_equal(_single(q, k, v, 0.25), oracle.widen_bf16(v[0]))


def test_closed_form_constant_v():
    r = np.random.default_rng(6)
    q, k = workloads.normal_bf16(r, (16,)), workloads.normal_bf16(r, (13, 16), mult=3.0)
    c = workloads.normal_bf16(r, (16,))
    v = np.repeat(c[None], 13, axis=0)
    np.testing.assert_allclose(_single(q, k, v, 0.25), oracle.widen_bf16(c), rtol=1e-14)


def test_closed_form_equal_keys_give_mean_of_v():
    r = np.random.default_rng(8)
    q = workloads.normal_bf16(r, (16,))
    k = np.repeat(workloads.normal_bf16(r, (1, 16)), 11, axis=0)
    v = workloads.normal_bf16(r, (11, 16))
    np.testing.assert_allclose(_single(q, k, v, 1.0), oracle.widen_bf16(v).mean(0), rtol=1e-13,
                               atol=1e-15)


def test_closed_form_large_scale_picks_argmax():
    r = np.random.default_rng(9)
    q, k = workloads.normal_bf16(r, (16,)), workloads.normal_bf16(r, (9, 16))
    v = workloads.normal_bf16(r, (9, 16))
    s = oracle.widen_bf16(k) @ oracle.widen_bf16(q)
    best = int(np.argmax(s))
    gap = np.sort(s)[-1] - np.sort(s)[-2]
    scale = 800.0 / gap  # second best weighs e^-800 relative
    out = _single(q, k, v, scale)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, oracle.widen_bf16(v[best]), rtol=0, atol=1e-300)


@pytest.mark.parametrize("scale", [1 / 8, 1.0, 10.0, 50.0])
def test_no_overflow_at_large_scores(scale):
    r = np.random.default_rng(10)
    q, k = workloads.normal_bf16(r, (16,), mult=8.0), workloads.normal_bf16(r, (20, 16), mult=8.0)
    v = workloads.normal_bf16(r, (20, 16))
    out = _single(q, k, v, scale)
    assert np.all(np.isfinite(out))
    vf = oracle.widen_bf16(v)
    assert np.all(out <= vf.max(0) + 1e-12) and np.all(out >= vf.min(0) - 1e-12)


def test_empty_sequence_gives_zero_row():
    w = workloads.random_small(12, 4, 4, 2, 16, 4, 10, min_len=0)
    w.seq_lens[1] = 0
    cu = np.zeros(5, np.int64)
    np.cumsum(w.seq_lens, out=cu[1:])
    # rebuild the token arrays for the shortened sequence 1
    full = workloads.random_small(12, 4, 4, 2, 16, 4, 10, min_len=0)
    keep = np.ones(full.k_tok.shape[0], bool)
    fcu = full.cu_seqlens
    keep[fcu[1]:fcu[2]] = False
    w.k_tok, w.v_tok = full.k_tok[keep], full.v_tok[keep]
    kc, vc = _oracle_cache(w)
    out = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    assert np.all(out[1] == 0.0)
    np.testing.assert_allclose(out, _sdpa_f64(w), rtol=1e-12, atol=1e-13)


def test_physical_permutation_invariance_is_bit_identical():
    w = workloads.random_small(13, 5, 8, 4, 32, 4, 30)
    kc, vc = _oracle_cache(w)
    base = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    perm = np.random.default_rng(1).permutation(w.num_blocks).astype(np.int32)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc  # block i moves to perm[i]
    bt2 = perm[w.block_tables]
    moved = oracle.paged_decode(w.q, kc2, vc2, bt2, w.seq_lens, w.scale)
    np.testing.assert_array_equal(moved, base)


def test_nan_in_unused_slots_is_never_read():
    w = workloads.tiny()
    kc, vc = _oracle_cache(w)  # free blocks 5, 6 and the tail slots are NaN
    assert np.isnan(oracle.widen_bf16(kc[5])).all()
    out = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    assert np.all(np.isfinite(out))


def test_bf16_round_matches_torch():
    r = np.random.default_rng(4)
    x = np.concatenate([r.normal(size=5000) * 10, [0.0, -0.0, 1e-40, 3.0e38]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x), want)


# ---------------------------------------------------------------- prefill


def _sdpa_prefill_f64(w):
    """torch's own attention routine (fp64, CPU) with an explicit causal mask
    aligned to the end of each sequence: new token i of sequence b may see
    positions 0 .. ctx_b + i."""
    ql = w.extra["q_lens"]
    out = np.zeros(w.q.shape, dtype=np.float64)
    cu = w.cu_seqlens
    qf = oracle.widen_bf16(w.q)
    row = 0
    for b in range(w.num_seqs):
        T, n = int(w.seq_lens[b]), int(ql[b])
        k = torch.from_numpy(oracle.widen_bf16(w.k_tok[cu[b]:cu[b + 1]])).permute(1, 0, 2)
        v = torch.from_numpy(oracle.widen_bf16(w.v_tok[cu[b]:cu[b + 1]])).permute(1, 0, 2)
        q = torch.from_numpy(qf[row:row + n]).permute(1, 0, 2)
        mask = torch.arange(T)[None, :] <= (T - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None].contiguous(), v[None].contiguous(), attn_mask=mask,
            scale=w.scale, enable_gqa=True)
        out[row:row + n] = o[0].permute(1, 0, 2).numpy()
        row += n
    return out


PREFILL_CASES = [
    lambda: workloads.prefill_small(1, 3, 4, 2, 16, 4, 20, 9),
    lambda: workloads.prefill_small(2, 4, 8, 2, 32, 8, 40, 17, min_ctx=0),
    lambda: workloads.prefill_small(3, 2, 6, 6, 8, 3, 0, 12),   # no context: a whole prompt
    lambda: workloads.prefill_small(4, 5, 16, 1, 24, 16, 70, 5),
]


@pytest.mark.parametrize("make", PREFILL_CASES)
def test_prefill_oracle_matches_torch_sdpa(make):
    w = make()
    kc, vc = _oracle_cache(w)
    got = oracle.paged_prefill(w.q, kc, vc, w.block_tables, w.seq_lens, w.extra["q_lens"],
                               w.scale)
    np.testing.assert_allclose(got, _sdpa_prefill_f64(w), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("make", PREFILL_CASES[:3])
def test_prefill_oracle_matches_brute_force(make):
    w = make()
    kc, vc = _oracle_cache(w)
    args = (w.q, kc, vc, w.block_tables, w.seq_lens, w.extra["q_lens"], w.scale)
    np.testing.assert_allclose(oracle.paged_prefill(*args), oracle.paged_prefill_py(*args),
                               rtol=1e-13, atol=1e-14)


def test_prefill_of_one_token_is_decode():
    """A chunk of one new token per sequence is the decode step."""
    w = workloads.random_small(5, 6, 8, 2, 32, 4, 30, min_len=1)
    kc, vc = _oracle_cache(w)
    got = oracle.paged_prefill(w.q, kc, vc, w.block_tables, w.seq_lens,
                               np.ones(w.num_seqs, np.int32), w.scale)
    want = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    np.testing.assert_array_equal(got, want)


def test_prefill_first_position_returns_v0_and_future_is_invisible():
    """With no context the first new token sees only itself (its output is
    v_0 exactly); changing the K/V of later positions leaves every earlier
    token's output unchanged, bit for bit."""
    w = workloads.prefill_small(6, 3, 4, 2, 16, 4, 0, 10, min_q=3)
    kc, vc = _oracle_cache(w)
    ql = w.extra["q_lens"]
    args = lambda kc_, vc_: (w.q, kc_, vc_, w.block_tables, w.seq_lens, ql, w.scale)
    out = oracle.paged_prefill(*args(kc, vc))
    cu_q = np.concatenate([[0], np.cumsum(ql)])
    cu = w.cu_seqlens
    for b in range(w.num_seqs):
        v0 = oracle.widen_bf16(w.v_tok[cu[b]])  # [Hkv, D]
        np.testing.assert_array_equal(out[cu_q[b]], np.repeat(v0, 2, axis=0))
    # perturb the last position of sequence 0: only its own last row may change
    kc2, vc2 = kc.copy(), vc.copy()
    last = int(w.seq_lens[0]) - 1
    s = oracle.slot(w.block_tables[0], last, w.block_size)
    kc2[s // w.block_size, :, s % w.block_size, :] ^= np.uint16(0x0040)
    vc2[s // w.block_size, :, :, s % w.block_size] ^= np.uint16(0x0040)
    out2 = oracle.paged_prefill(*args(kc2, vc2))
    np.testing.assert_array_equal(out2[:cu_q[1] - 1], out[:cu_q[1] - 1])
    np.testing.assert_array_equal(out2[cu_q[1]:], out[cu_q[1]:])
    assert not np.array_equal(out2[cu_q[1] - 1], out[cu_q[1] - 1])


# ---------------------------------------------------------------- swap


def test_swap_round_trip_and_relocation():
    """Blocks swapped out and back into the same ids leave every cache bit as
    it was; swapped back into other ids, with the tables re-pointed there,
    attention gives the same result bit for bit (the page is found through
    the table wherever it lives)."""
    w = workloads.random_small(8, 5, 8, 2, 32, 4, 30, min_len=1, slack_blocks=40)
    kc, vc = _oracle_cache(w)
    kc2, vc2 = _oracle_cache(w)
    caches = [(kc, vc), (kc2, vc2)]
    before = [(a.copy(), b.copy()) for a, b in caches]
    used = np.unique(np.concatenate([w.block_tables[b, :-(-int(w.seq_lens[b]) // 4)]
                                     for b in range(w.num_seqs)]))
    buf = oracle.swap_out(caches, used[::-1])
    assert buf.shape == (2, 2, len(used), kc[0].size)
    np.testing.assert_array_equal(buf[1, 0, 0], kc2[used[-1]].ravel())
    np.testing.assert_array_equal(buf[0, 1, 2], vc[used[-3]].ravel())
    ref = oracle.paged_decode(w.q, kc, vc, w.block_tables, w.seq_lens, w.scale)
    # scribble over the swapped-out blocks, then bring them back where they were
    for a, b in caches:
        a[used] = 0x7FC0
        b[used] = 0x7FC0
    oracle.swap_in(caches, used[::-1], buf)
    for (a, b), (a0, b0) in zip(caches, before):
        np.testing.assert_array_equal(a, a0)
        np.testing.assert_array_equal(b, b0)
    # relocate: the blocks come back into free ids, the tables follow them
    free = np.setdiff1d(np.arange(w.num_blocks), used)[:len(used)]
    assert len(free) == len(used)
    moved = dict(zip(used.tolist(), free.tolist()))
    oracle.swap_in(caches, [moved[int(x)] for x in used[::-1]], buf)
    bt2 = w.block_tables.copy()
    for b in range(w.num_seqs):
        nb = -(-int(w.seq_lens[b]) // 4)
        bt2[b, :nb] = [moved[int(x)] for x in bt2[b, :nb]]
    for a, b in caches:  # the old places are gone
        a[used] = 0x7FC0
        b[used] = 0x7FC0
    got = oracle.paged_decode(w.q, kc, vc, bt2, w.seq_lens, w.scale)
    np.testing.assert_array_equal(got, ref)
