"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark uses (library-chosen partition and waves, bf16
output) and with fp32 output for the strict bound."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_373_amd as pkv
import workloads
from paritylib import DEV, GpuSide, OracleSide, bf16_bits, bits_to_bf16, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _full(w, name, segments=None):
    """Caches bit-exact; attention in the benchmark's launch configuration
    (library choices: the stream kernel, bf16 output), with fp32 output for
    the strict bound, and - where the workload fixes its split-KV segment
    length - the partitioned kernel with exactly those segments."""
    g, o = GpuSide(w), OracleSide(w)
    say(f"  {name}: caches")
    np.testing.assert_array_equal(bf16_bits(g.kc), o.kc)
    np.testing.assert_array_equal(bf16_bits(g.vc), o.vc)
    ref = o.decode()
    outb = g.decode(torch.bfloat16, partition_size=0)  # the benchmark's configuration
    compare(outb.float().cpu().numpy(), ref, strict_abs=False, what=f"{name}/bf16")
    out = g.decode(torch.float32, partition_size=0)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"{name}/f32")
    if segments:
        out = g.decode(torch.float32, kernel="mfma", partition_size=segments)
        compare(out.cpu().numpy(), ref, strict_abs=True, what=f"{name}/f32/segments{segments}")


def test_tiny_workload():
    say("case workload tiny")
    _full(workloads.tiny(), "tiny")


def test_llama_b64_workload():
    say("case workload llama_b64 (S=64, 32q/8kv, d64, B16, T~U[128,2048])")
    _full(workloads.llama_decode(), "llama_b64")


def test_long_context_workload():
    say("case workload long_splitkv (S=8, T~U[16384,32768], PS=512, K*3)")
    _full(workloads.long_context(), "long_splitkv", segments=512)
