"""GPU parity in the regime the online softmax's rescaling exists for
([PU] "Infra: PagedAttention", section 按 Block 分配: each block's maximum
score is kept and partial sums are rescaled to a common maximum so nothing
overflows).

Every kernel family runs at the Llama head shape (32 q / 8 KV heads,
head_dim 64, B = 16) on sequences long enough that each (sequence, KV head)
is cut into many pieces (windows, wavefront ranges or partitions), with
  * scales 1/8, 1, 10 and 50 against the oracle;
  * V constant: the output is that constant (softmax weights sum to one);
  * all keys of a sequence equal: the output is the mean of its V rows;
  * scale 50: the output is the V row of the highest-scoring token wherever
    the two best scores are far apart.
The kernels form probabilities against a running maximum that is raised only
once a chunk's maximum exceeds it by 2^8, and round them to bf16 before the
P.V product; these cases stress exactly that.  Unused cache bytes are NaN."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import GpuSide, OracleSide, compare, say

pytestmark = pytest.mark.gpu

LENS = [3000, 1, 2100, 4096, 17, 1500, 33, 2600]
KERNELS = {
    "stream_wg": dict(kernel="stream_wg"),
    "stream": dict(kernel="stream"),
    "mfma": dict(kernel="mfma", partition_size=512),
    "generic": dict(kernel="generic", partition_size=512),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _base(seed=61):
    return workloads.random_small(seed, len(LENS), 32, 8, 64, 16, 0, lens=LENS)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return workloads.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _run(w, kernel):
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out32 = g.decode(torch.float32, **KERNELS[kernel]).cpu().numpy()
    out16 = g.decode(torch.bfloat16, **KERNELS[kernel]).float().cpu().numpy()
    return ref, out32, out16


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("scale", [0.125, 1.0, 10.0, 50.0])
def test_scales(kernel, scale):
    say(f"case softmax scale={scale} kernel={kernel}")
    w = dataclasses.replace(_base(), scale=scale)
    ref, out32, out16 = _run(w, kernel)
    compare(out32, ref, strict_abs=True, what=f"scale {scale}/{kernel}/f32")
    compare(out16, ref, strict_abs=False, what=f"scale {scale}/{kernel}/bf16")
    if scale == 50.0:
        # closed form: where the best score beats the second by a wide margin
        # the softmax is one-hot on it, so the output is that token's V row
        kf = oracle.widen_bf16(w.k_tok).astype(np.float64)
        vf = oracle.widen_bf16(w.v_tok).astype(np.float64)
        qf = oracle.widen_bf16(w.q).astype(np.float64)
        cu = w.cu_seqlens
        g = w.num_q_heads // w.num_kv_heads
        checked = 0
        for b in range(w.num_seqs):
            if w.seq_lens[b] < 2:
                continue
            for h in range(w.num_q_heads):
                kv = h // g
                s = kf[cu[b]:cu[b + 1], kv] @ qf[b, h] * scale
                top = np.argsort(s)[-2:]
                if s[top[1]] - s[top[0]] < 40.0:
                    continue
                vt = vf[cu[b] + top[1], kv]
                assert np.max(np.abs(out32[b, h] - vt)) <= 1e-5, (b, h)
                checked += 1
        say(f"  one-hot rows checked against their argmax V row: {checked}")
        assert checked > 20


@pytest.mark.parametrize("kernel", list(KERNELS))
def test_constant_v(kernel):
    say(f"case softmax V constant kernel={kernel}")
    base = _base(62)
    c = 0.75
    w = dataclasses.replace(base, v_tok=np.full_like(base.v_tok, _bf16_bits(np.float32(c))),
                            scale=10.0)
    ref, out32, out16 = _run(w, kernel)
    compare(out32, ref, strict_abs=True, what=f"V const/{kernel}/f32")
    live = w.seq_lens > 0
    assert np.max(np.abs(out32[live] - c)) <= 1e-5
    assert np.all(out16[live] == c)
    assert np.all(out32[~live] == 0.0)


@pytest.mark.parametrize("kernel", list(KERNELS))
def test_equal_keys_give_mean_of_v(kernel):
    say(f"case softmax equal keys kernel={kernel}")
    base = _base(63)
    k = base.k_tok.copy()
    cu = base.cu_seqlens
    for b in range(base.num_seqs):
        if base.seq_lens[b] > 0:
            k[cu[b]:cu[b + 1]] = k[cu[b]]  # every token of the sequence: the first one's keys
    w = dataclasses.replace(base, k_tok=k, scale=50.0)
    ref, out32, out16 = _run(w, kernel)
    compare(out32, ref, strict_abs=True, what=f"equal K/{kernel}/f32")
    compare(out16, ref, strict_abs=False, what=f"equal K/{kernel}/bf16")
    vf = oracle.widen_bf16(w.v_tok).astype(np.float64)
    g = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        if w.seq_lens[b] == 0:
            continue
        mean = vf[cu[b]:cu[b + 1]].mean(axis=0)  # [Hkv, D]
        exp = np.repeat(mean, g, axis=0)
        assert np.max(np.abs(out32[b] - exp)) <= 1e-4, b
