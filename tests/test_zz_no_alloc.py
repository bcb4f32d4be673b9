"""pkv_paged_attention_decode_noalloc (the decode call for callers that
cannot allocate) through the C ABI, against pkv_paged_attention_decode with
a workspace on the same inputs: the same kernels run, so the outputs must be
the same bits; both stay within the attention tolerance of the oracle.  Calls
follow one another on one device, so each finds the previous call's partial
results in the shared scratch array."""
import ctypes
import os

import pytest
import torch

import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import GpuSide, OracleSide, compare, say

pytestmark = pytest.mark.skipif(not os.path.exists(pkv.LIB_PATH),
                                reason="libpagedkv.so not built")


def _dims(**kw):
    base = dict(num_seqs=2048, num_q_heads=256, num_kv_heads=16, head_dim=128, num_blocks=1000,
                max_blocks_per_seq=4096, max_seq_len=65536, partition_size=0, out_dtype=1,
                kernel=0, waves_per_group=0, balance_partitions=0, stream_waves=0,
                no_shared_blocks=0)
    base.update(kw)
    return pkv.DecodeDims(**base)


def test_noalloc_rejects_a_call_beyond_the_array():
    """A shape whose workspace exceeds the array is refused with
    PKV_ERR_WORKSPACE before any HIP call (fake pointers, no GPU needed)."""
    d = _dims()
    need = pkv.lib().pkv_decode_workspace_size(ctypes.byref(d), 16)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(0x1000)
    st = pkv.lib().pkv_paged_attention_decode_noalloc(f, f, f, f, f, 16, 0.125, f,
                                                      ctypes.byref(d), None)
    assert st == pkv.PKV_ERR_WORKSPACE
    # invalid dims are still PKV_ERR_INVALID
    bad = _dims(num_q_heads=250)
    assert pkv.lib().pkv_paged_attention_decode_noalloc(f, f, f, f, f, 16, 0.125, f,
                                                        ctypes.byref(bad), None) == pkv.PKV_ERR_INVALID


def _one(w, kernel, **kw):
    g = GpuSide(w)
    args = dict(kernel=kernel, **kw)
    ref = g.decode(torch.float32, **args)
    out = torch.full_like(ref, float("nan"))
    pkv.paged_attention_decode_noalloc(g.q, g.kc, g.vc, g.bt, g.lens, w.block_size, w.scale, out,
                                       max_seq_len=int(w.seq_lens.max()), **args)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "no-alloc output differs from the workspace call's"
    compare(out.cpu().numpy(), OracleSide(w).decode(), strict_abs=True,
            what=f"noalloc/{kernel}/S={w.num_seqs}")


CASES = [("stream_wg", {}), ("stream", {}), ("mfma", {"partition_size": 128}),
         ("auto", {"no_shared_blocks": True})]


@pytest.mark.gpu
@pytest.mark.parametrize("kernel,kw", CASES, ids=[c[0] + ("_nt" if c[1].get("no_shared_blocks") else "")
                                                  for c in CASES])
def test_noalloc_two_calls_second_smaller(kernel, kw):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"case noalloc {kernel} {kw}: big, then small, then bigger")
    big = workloads.random_small(81, 40, 32, 8, 64, 16, 3000, min_len=1)
    small = workloads.random_small(82, 12, 32, 8, 64, 16, 700, min_len=1)
    _one(big, kernel, **kw)
    _one(small, kernel, **kw)
    # a counter region larger than the last call's, over its partial results
    bigger = workloads.random_small(83, 64, 32, 8, 64, 16, 4000, min_len=0)
    _one(bigger, kernel, **kw)
