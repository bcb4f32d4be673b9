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
from paritylib import DEV, GpuSide, OracleSide, bits_to_bf16, compare, say

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
