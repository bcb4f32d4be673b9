"""GPU parity of the decode step with append (pkv_paged_attention_decode_append):
the cache holds every token of each sequence but its last; the call writes
the last one (position T_b - 1, the slot its block table names) and attends
over all T_b.  Caches must then equal the oracle's bit for bit, and the output
match the oracle's attention over the fully written cache."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_373_amd as pkv
import workloads
from paged_kv_cache_373_amd.block_manager import slot_mapping_for
from paritylib import DEV, OracleSide, bf16_bits, bits_to_bf16, compare, say, token_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _prefill_all_but_last(w, bt):
    """Product side: NaN caches holding every token but each sequence's last."""
    kc, vc = pkv.new_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                              fill=float("nan"))
    seq, pos = token_positions(w.seq_lens)
    last = np.zeros(len(pos), bool)
    cu = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int64)
    last[cu[1:][w.seq_lens > 0] - 1] = True
    slots = slot_mapping_for(bt, seq, pos, w.block_size)
    slots = np.where(last, -1, slots)
    pkv.reshape_and_cache(bits_to_bf16(w.k_tok).to(DEV), bits_to_bf16(w.v_tok).to(DEV),
                          torch.from_numpy(slots).to(DEV), kc, vc)
    k_new = np.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), np.uint16)
    v_new = np.zeros_like(k_new)
    has = w.seq_lens > 0
    k_new[has] = w.k_tok[cu[1:][has] - 1]
    v_new[has] = w.v_tok[cu[1:][has] - 1]
    return kc, vc, bits_to_bf16(k_new).to(DEV), bits_to_bf16(v_new).to(DEV)


def _run(w, kernel, out_dtype=torch.float32, **kw):
    bt = w.block_tables
    kc, vc, k_new, v_new = _prefill_all_but_last(w, bt)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=out_dtype, device=DEV)
    pkv.paged_attention_decode_append(
        bits_to_bf16(w.q).to(DEV), k_new, v_new, kc, vc, torch.from_numpy(bt).to(DEV),
        torch.from_numpy(w.seq_lens).to(DEV), w.block_size, w.scale, out,
        max_seq_len=int(w.seq_lens.max(initial=0)), kernel=kernel, **kw)
    return kc, vc, out


def _check(w, kernel, name, **kw):
    o = OracleSide(w)
    ref = o.decode()
    kc, vc, out = _run(w, kernel, **kw)
    np.testing.assert_array_equal(bf16_bits(kc), o.kc, err_msg=f"{name}: k_cache bits")
    np.testing.assert_array_equal(bf16_bits(vc), o.vc, err_msg=f"{name}: v_cache bits")
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"{name}/{kernel}")
    return out


CASES = {
    "g4_d64_b16": lambda: workloads.random_small(60, 7, 16, 4, 64, 16, 400, min_len=0),
    "g2_d64_b8": lambda: workloads.random_small(61, 9, 8, 4, 64, 8, 300, min_len=1),
    "g8_d128_b32": lambda: workloads.random_small(62, 5, 16, 2, 128, 32, 700, min_len=1),
    "g1_d64_b16": lambda: workloads.random_small(63, 6, 4, 4, 64, 16, 90, min_len=0),
    "g2_d16_b4": lambda: workloads.random_small(64, 5, 4, 2, 16, 4, 40, min_len=0),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("kernel", ["stream_wg", "stream", "mfma", "generic"])
def test_append_small(name, kernel):
    say(f"case append {name} kernel={kernel}")
    w = CASES[name]()
    g = w.num_q_heads // w.num_kv_heads
    if kernel != "generic" and not (w.head_dim in (64, 128) and w.block_size in (8, 16, 32)
                                    and g <= 16):
        pytest.skip("shape outside the matrix-core kernels")
    kw = dict(partition_size=64) if kernel == "mfma" else {}
    _check(w, kernel, name, **kw)


@pytest.mark.parametrize("waves", [4, 64, 2048])
@pytest.mark.parametrize("kernel", ["stream", "stream_wg"])
def test_append_token_positions(waves, kernel):
    """The new token at every position of a 32-token chunk and of a block:
    lengths 1..66 (block starts, block ends, chunk ends), and empty
    sequences, whose output is zero and whose cache is left alone."""
    say(f"case append positions waves={waves} kernel={kernel}")
    lens = list(range(0, 67))
    w = workloads.random_small(65, len(lens), 8, 2, 64, 16, 66, min_len=0)
    r = workloads.rng(100, 79)
    w.seq_lens = np.array(lens, dtype=np.int32)
    total = int(w.seq_lens.sum())
    w.k_tok = workloads.normal_bf16(r, (total, 2, 64))
    w.v_tok = workloads.normal_bf16(r, (total, 2, 64))
    need = [-(-t // 16) for t in lens]
    pool = sum(need) + 2
    perm = r.permutation(pool).astype(np.int32)
    bt = np.full((len(lens), 5), perm[-1], dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        bt[b, :nb] = perm[pos:pos + nb]
        pos += nb
    w.block_tables, w.num_blocks, w.poison_block = bt, pool, int(perm[-1])
    out = _check(w, kernel, f"positions w{waves}", stream_waves=waves)
    assert np.all(out[0].cpu().numpy() == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("waves", [4, 16])
@pytest.mark.parametrize("kernel", ["stream", "stream_wg"])
def test_append_more_units_than_wavefronts(d, waves, kernel):
    """Each wavefront writes the new tokens of units gw, gw + (all wavefronts),
    ...: with 40 sequences x 4 KV heads against 4 or 16 wavefronts (the
    workgroup kernel rounds up to whole workgroups) most wavefronts write
    several units, some after their chunks, the rest from the end loop."""
    say(f"case append units>waves d={d} waves={waves} kernel={kernel}")
    w = workloads.random_small(67, 40, 8, 4, d, 16, 150, min_len=0)
    _check(w, kernel, f"units>waves d{d} w{waves}", stream_waves=waves)


@pytest.mark.parametrize("hq,hkv,d", [(16, 1, 128), (16, 2, 128), (8, 4, 64)])
@pytest.mark.parametrize("waves", [4, 8])
def test_stream_held_back_stores(hq, hkv, d, waves):
    """The per-wavefront kernel holds whole units' output rows and its range's
    first piece in an LDS area of 2048 floats per wavefront, writing them
    after its last load: at G = 16, D = 128 the piece does not fit (published
    at once) and one unit's rows do; at G = 8, D = 128 the piece fits and no
    rows do; at G = 2, D = 64 many rows fit and the rest are stored at once.
    Few wavefronts, so each range holds several whole units and cut pieces."""
    say(f"case stream held-back stores hq={hq} hkv={hkv} d={d} waves={waves}")
    w = workloads.random_small(68, 24, hq, hkv, d, 16, 260, min_len=0)
    _check(w, "stream", f"held-back hq{hq} hkv{hkv} d{d} w{waves}", stream_waves=waves)


@pytest.mark.parametrize("kernel", ["stream", "stream_wg"])
def test_two_steps(kernel):
    """Two decode steps back to back: the second appends position T_b (one
    past the first step's), which for some sequences opens a new block."""
    say(f"case append two steps kernel={kernel}")
    w = workloads.random_small(66, 8, 16, 4, 64, 16, 200, min_len=1, slack_blocks=20)
    # the tables need room for one more token: give every sequence a spare block
    spare = w.num_blocks
    w.num_blocks += w.num_seqs
    bt = np.concatenate([w.block_tables, np.full((w.num_seqs, 1), w.poison_block, np.int32)], 1)
    for b in range(w.num_seqs):
        nb = -(-int(w.seq_lens[b]) // 16)
        if int(w.seq_lens[b]) % 16 == 0:  # the next token opens block nb
            bt[b, nb] = spare + b
    w.block_tables = bt
    # step 2 inputs: one more token per sequence
    r = workloads.rng(100, 80)
    k2 = workloads.normal_bf16(r, (w.num_seqs, 4, 64))
    v2 = workloads.normal_bf16(r, (w.num_seqs, 4, 64))
    q2 = workloads.normal_bf16(r, (w.num_seqs, 16, 64))
    kc, vc, out1 = _run(w, kernel)
    lens2 = w.seq_lens + 1
    out2 = torch.empty_like(out1)
    pkv.paged_attention_decode_append(
        bits_to_bf16(q2).to(DEV), bits_to_bf16(k2).to(DEV), bits_to_bf16(v2).to(DEV), kc, vc,
        torch.from_numpy(bt).to(DEV), torch.from_numpy(lens2.astype(np.int32)).to(DEV), 16,
        w.scale, out2, max_seq_len=int(lens2.max()), kernel=kernel)
    # oracle: every token of both steps, sequence-major
    ks, vs = [], []
    cu = np.concatenate([[0], np.cumsum(w.seq_lens)])
    for b in range(w.num_seqs):
        ks += [w.k_tok[cu[b]:cu[b + 1]], k2[b:b + 1]]
        vs += [w.v_tok[cu[b]:cu[b + 1]], v2[b:b + 1]]
    w2 = workloads.Workload("two_steps", 100, 16, 4, 64, 16, w.num_blocks, lens2.astype(np.int32),
                            q2, w.scale, block_tables=bt, k_tok=np.concatenate(ks),
                            v_tok=np.concatenate(vs), poison_block=w.poison_block)
    o = OracleSide(w2)
    np.testing.assert_array_equal(bf16_bits(kc), o.kc)
    np.testing.assert_array_equal(bf16_bits(vc), o.vc)
    compare(out2.cpu().numpy(), o.decode(), strict_abs=True, what="two steps / step 2")


def test_append_llama_b64():
    """The benchmark's step at full size: llama_b64, library choices, bf16 out."""
    say("case append llama_b64")
    w = workloads.llama_decode()
    o = OracleSide(w)
    ref = o.decode()
    kc, vc, out = _run(w, "auto", out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(bf16_bits(kc), o.kc)
    np.testing.assert_array_equal(bf16_bits(vc), o.vc)
    compare(out.float().cpu().numpy(), ref, strict_abs=False, what="llama_b64 append/bf16")
