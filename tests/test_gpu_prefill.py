"""GPU parity of paged prefill (pkv_paged_prefill): causal multi-query
attention of every sequence's new tokens over its cached tokens, read
through the block table ([PU §KV Cache 为什么会浪费显存]; [PU §Continuous
Batching]; [PU §按 Block 分配]).  The product writes the K/V with its own
reshape_and_cache into NaN-filled caches; the oracle writes its own cache and
runs fp64 causal attention.  Only the seeded inputs are shared."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import DEV, GpuSide, OracleSide, bits_to_bf16, compare, compare_bf16p, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _run(g, w, out_dtype, max_q_len=None, seq_lens=None, cu=None):
    ql = w.extra["q_lens"]
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32) if cu is None else cu
    lens = g.lens if seq_lens is None else torch.from_numpy(np.asarray(seq_lens, np.int32)).to(DEV)
    out = torch.empty(tuple(w.q.shape), dtype=out_dtype, device=DEV)
    pkv.paged_prefill(g.q, g.kc, g.vc, g.bt, lens, torch.from_numpy(cu).to(DEV), w.block_size,
                      w.scale, out, max_q_len=int(ql.max()) if max_q_len is None else max_q_len,
                      max_seq_len=int(w.seq_lens.max()))
    torch.cuda.synchronize()
    return out


def _oracle(w):
    o = OracleSide(w)
    return oracle.paged_prefill(w.q, o.kc, o.vc, o.bt, w.seq_lens, w.extra["q_lens"], w.scale)


# name: seed, S, Hq, Hkv, D, B, max ctx, max q, min q, min ctx
CASES = {
    "g4_d64_b16": (1, 3, 8, 2, 64, 16, 40, 20, 1, 0),
    "g4_d64_b8_long": (2, 4, 16, 4, 64, 8, 100, 37, 1, 0),
    "g16_d128_b32_prompt": (3, 2, 16, 1, 128, 32, 0, 64, 30, 0),   # no context
    "g1_d64_b16": (4, 5, 4, 4, 64, 16, 70, 5, 1, 0),
    "g16_d128_b16": (5, 3, 32, 2, 128, 16, 300, 50, 1, 0),
    "g1_d64_b32_one_token": (6, 6, 8, 8, 64, 32, 33, 1, 1, 0),       # the decode step
    "g2_d64_b16_ctx_batch": (7, 3, 4, 2, 64, 16, 1100, 20, 1, 1000),  # more than 64 blocks
    "g4_d64_b16_s64": (8, 64, 8, 2, 64, 16, 90, 12, 1, 0),   # sequences ranked by length
    "g4_d64_b16_s70": (9, 70, 8, 2, 64, 16, 90, 12, 1, 0),   # past 64: the batch's order
    # long contexts: items of >= 16 chunks near the longest are split between two wavefronts
    "g8_d128_b32_split": (10, 3, 16, 2, 128, 32, 700, 40, 20, 500),
    "g4_d64_b8_split": (11, 4, 16, 4, 64, 8, 900, 60, 30, 600),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_small(name):
    seed, s, hq, hkv, d, bs, mctx, mq, minq, minctx = CASES[name]
    say(f"case prefill {name}")
    w = workloads.prefill_small(seed, s, hq, hkv, d, bs, mctx, mq, min_q=minq, min_ctx=minctx)
    ref = _oracle(w)
    g = GpuSide(w)
    out = _run(g, w, torch.float32).cpu().numpy()
    compare(out, ref, strict_abs=True, what=f"{name}/f32")
    out16 = _run(g, w, torch.bfloat16).float().cpu().numpy()
    compare(out16, ref, strict_abs=False, what=f"{name}/bf16")
    # a grid sized for shorter chunks still covers every row, with the same bits
    short = _run(g, w, torch.float32, max_q_len=max(1, int(w.extra["q_lens"].max()) // 3))
    np.testing.assert_array_equal(short.cpu().numpy(), out)


def test_prefill_device_checks():
    """A sequence with more new tokens than cached ones gets NaN rows; the
    others are unaffected."""
    say("case prefill device-side checks")
    w = workloads.prefill_small(1, 3, 8, 2, 64, 16, 40, 20)
    g = GpuSide(w)
    ref = _oracle(w)
    lens = w.seq_lens.copy()
    lens[1] = int(w.extra["q_lens"][1]) - 1
    out = _run(g, w, torch.float32, seq_lens=lens).cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.extra["q_lens"])])
    assert np.all(np.isnan(out[cu[1]:cu[2]]))
    keep = np.r_[0:cu[1], cu[2]:cu[3]]
    compare(out[keep], ref[keep], strict_abs=True, what="other sequences")


def test_prefill_chunked_llama():
    """The Llama-shaped chunked prefill at full size: 8 sequences, 512 new
    tokens each after up to 2048 cached ones."""
    say("case prefill chunked llama")
    w = workloads.prefill_chunked()
    ref = _oracle(w)
    g = GpuSide(w)
    out = _run(g, w, torch.bfloat16).float().cpu().numpy()
    compare(out, ref, strict_abs=False, what="prefill_chunked/bf16")


# The regime the online softmax's rescaling exists for ([PU §按 Block 分配]:
# each block's maximum is kept and partial sums are rescaled to a common
# maximum), at the Llama head shape: 4 sequences of 40..120 new tokens after
# 200..1200 cached ones, so every (sequence, KV head) spans several items of
# tiles and up to two batches of block ids.
def _safety_base(seed):
    return workloads.prefill_small(seed, 4, 32, 8, 64, 16, 1200, 120, min_q=40, min_ctx=200)


def _visible(w):
    """(sequence, new token i, first cache row of b, rows visible to i)."""
    ql = w.extra["q_lens"]
    cu_tok = np.concatenate([[0], np.cumsum(w.seq_lens)])
    for b in range(w.num_seqs):
        ctx = int(w.seq_lens[b]) - int(ql[b])
        for i in range(int(ql[b])):
            yield b, i, int(cu_tok[b]), ctx + i + 1


def _bf16p_bound(w, ref):
    """Per element, the first-order error of forming the softmax weights in
    bf16 before the P.V product (both the numerator and the sum use the same
    rounded P_j = p_j (1 + d_j), |d_j| <= 2^-9): the output moves by
    sum_j w_j d_j (v_j - out), at most 2^-9 sum_j w_j |v_j - out|.  Twice that,
    from the oracle's own weights, bounds the kernel's deviation."""
    kf = oracle.widen_bf16(w.k_tok).astype(np.float64)
    vf = oracle.widen_bf16(w.v_tok).astype(np.float64)
    qf = oracle.widen_bf16(w.q).astype(np.float64)
    gq = w.num_q_heads // w.num_kv_heads
    ql = w.extra["q_lens"]
    cu_q = np.concatenate([[0], np.cumsum(ql)])
    cu_tok = np.concatenate([[0], np.cumsum(w.seq_lens)])
    bound = np.zeros_like(ref, dtype=np.float64)
    for b in range(w.num_seqs):
        T, nq = int(w.seq_lens[b]), int(ql[b])
        ctx = T - nq
        for h in range(w.num_q_heads):
            kv = h // gq
            s = qf[cu_q[b]:cu_q[b + 1], h] @ kf[cu_tok[b]:cu_tok[b + 1], kv].T * w.scale
            s[np.arange(T)[None, :] > (ctx + np.arange(nq))[:, None]] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            v = vf[cu_tok[b]:cu_tok[b + 1], kv]
            r = ref[cu_q[b]:cu_q[b + 1], h]
            for i in range(nq):
                bound[cu_q[b] + i, h] = p[i] @ np.abs(v - r[i])
    return 2.0 ** -8 * bound


@pytest.mark.parametrize("scale", [0.125, 1.0, 10.0, 50.0])
def test_prefill_softmax_scales(scale):
    import dataclasses
    say(f"case prefill softmax scale={scale}")
    w = dataclasses.replace(_safety_base(71), scale=scale)
    ref = _oracle(w)
    g = GpuSide(w)
    out = _run(g, w, torch.float32).cpu().numpy()
    out16 = _run(g, w, torch.bfloat16).float().cpu().numpy()
    if scale <= 0.125:  # the model's own scale, 1/sqrt(64): the spec rule
        compare(out, ref, strict_abs=True, what=f"prefill scale {scale}/f32")
        compare(out16, ref, strict_abs=False, what=f"prefill scale {scale}/bf16")
    else:  # sharper softmax: the rule, or the bf16-P bound where it is wider
        bound = _bf16p_bound(w, ref)
        compare_bf16p(out, ref, bound, f"prefill scale {scale}/f32")
        # the bf16 output adds its own rounding, half an ulp of |out|
        compare_bf16p(out16, ref, bound + 2.0 ** -8 * np.abs(ref), f"prefill scale {scale}/bf16")
    if scale == 50.0:
        # closed form: where a row's best visible score beats the second by a
        # wide margin the softmax is one-hot, and the output is that V row
        kf = oracle.widen_bf16(w.k_tok).astype(np.float64)
        vf = oracle.widen_bf16(w.v_tok).astype(np.float64)
        qf = oracle.widen_bf16(w.q).astype(np.float64)
        gq = w.num_q_heads // w.num_kv_heads
        cu_q = np.concatenate([[0], np.cumsum(w.extra["q_lens"])])
        checked = 0
        for b, i, t0, nvis in _visible(w):
            if nvis < 2:
                continue
            for h in range(0, w.num_q_heads, 5):
                kv = h // gq
                s = kf[t0:t0 + nvis, kv] @ qf[cu_q[b] + i, h] * scale
                top = np.argsort(s)[-2:]
                if s[top[1]] - s[top[0]] < 40.0:
                    continue
                assert np.max(np.abs(out[cu_q[b] + i, h] - vf[t0 + top[1], kv])) <= 1e-5, (b, i, h)
                checked += 1
        say(f"  one-hot rows checked against their argmax V row: {checked}")
        assert checked > 50


def test_prefill_constant_v():
    import dataclasses
    say("case prefill softmax V constant")
    base = _safety_base(72)
    c = 0.75
    bits = workloads.to_bf16_bits(np.float32(c))
    w = dataclasses.replace(base, v_tok=np.full_like(base.v_tok, bits), scale=10.0)
    g = GpuSide(w)
    out = _run(g, w, torch.float32).cpu().numpy()
    assert np.max(np.abs(out - c)) <= 1e-5
    out16 = _run(g, w, torch.bfloat16).float().cpu().numpy()
    assert np.all(out16 == c)


def test_prefill_equal_keys_give_causal_mean_of_v():
    import dataclasses
    say("case prefill softmax equal keys")
    base = _safety_base(73)
    k = base.k_tok.copy()
    cu_tok = np.concatenate([[0], np.cumsum(base.seq_lens)])
    for b in range(base.num_seqs):
        k[cu_tok[b]:cu_tok[b + 1]] = k[cu_tok[b]]  # every token: the sequence's first keys
    w = dataclasses.replace(base, k_tok=k, scale=50.0)
    ref = _oracle(w)
    g = GpuSide(w)
    out = _run(g, w, torch.float32).cpu().numpy()
    compare(out, ref, strict_abs=True, what="prefill equal K/f32")
    vf = oracle.widen_bf16(w.v_tok).astype(np.float64)
    gq = w.num_q_heads // w.num_kv_heads
    cu_q = np.concatenate([[0], np.cumsum(w.extra["q_lens"])])
    for b, i, t0, nvis in _visible(w):
        exp = np.repeat(vf[t0:t0 + nvis].mean(axis=0), gq, axis=0)  # [Hq, D]
        assert np.max(np.abs(out[cu_q[b] + i] - exp)) <= 1e-4, (b, i)
