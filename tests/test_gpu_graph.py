"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: decode, the fused decode step, shared-prefix decode and prefill.
Each replay runs after eager work and a synchronisation of its own and must
give the eager result bit for bit.  The workspaces are prepared by an eager
call first, so nothing is cleared inside the graph (the kernels leave their
counters at zero themselves)."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import paged_kv_cache_373_amd as pkv
import workloads
from paged_kv_cache_373_amd.block_manager import slot_mapping_for
from paritylib import DEV, GpuSide, bits_to_bf16, say, token_positions

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.lib()


def _replays_match(fn, outs, n=4):
    """Eager reference, capture, then n replays separated by eager work."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    junk = torch.zeros(1 << 20, device=DEV)
    for k in range(n):
        for o in outs:
            o.fill_(float("nan"))
        junk.add_(1.0)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {k} differs from the eager call"


@pytest.mark.parametrize("kernel", ["stream_wg", "stream", "mfma"])
def test_decode_graph(kernel):
    say(f"case graph decode {kernel}")
    w = workloads.random_small(70, 12, 16, 4, 64, 16, 900, min_len=1)
    g = GpuSide(w)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    ws = pkv.DecodeWorkspace(device=DEV)
    kw = dict(max_seq_len=int(w.seq_lens.max()), kernel=kernel, workspace=ws)
    if kernel == "mfma":
        kw["partition_size"] = 128
    _replays_match(lambda: pkv.paged_attention_decode(g.q, g.kc, g.vc, g.bt, g.lens,
                                                      w.block_size, w.scale, out, **kw), [out])


def test_decode_append_graph():
    """The fused step writes the new tokens (the same bits every replay) and
    attends."""
    say("case graph decode append")
    w = workloads.random_small(71, 10, 8, 2, 64, 16, 500, min_len=1)
    g = GpuSide(w)
    cu = np.concatenate([[0], np.cumsum(w.seq_lens)])
    k_new = bits_to_bf16(w.k_tok[cu[1:] - 1]).to(DEV)
    v_new = bits_to_bf16(w.v_tok[cu[1:] - 1]).to(DEV)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    ws = pkv.DecodeWorkspace(device=DEV)
    _replays_match(lambda: pkv.paged_attention_decode_append(
        g.q, k_new, v_new, g.kc, g.vc, g.bt, g.lens, w.block_size, w.scale, out,
        max_seq_len=int(w.seq_lens.max()), workspace=ws), [out])


def test_cascade_and_prefill_graph():
    say("case graph cascade + prefill")
    w = workloads.shared_prefix_small(1, [3, 1, 5, 2], [4, 0, 6, 2], 16, 4, 64, 16, 150)
    # the shared prompt rows are written once (by each group's first member)
    seq, pos = token_positions(w.seq_lens)
    slots = np.where(w.extra["repeat_rows"], -1,
                     slot_mapping_for(w.block_tables, seq, pos, w.block_size))
    g = SimpleNamespace(bt=torch.from_numpy(w.block_tables).to(DEV),
                        lens=torch.from_numpy(w.seq_lens).to(DEV),
                        q=bits_to_bf16(w.q).to(DEV))
    g.kc, g.vc = pkv.new_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                                  fill=float("nan"))
    pkv.reshape_and_cache(bits_to_bf16(w.k_tok).to(DEV), bits_to_bf16(w.v_tok).to(DEV),
                          torch.from_numpy(slots).to(DEV), g.kc, g.vc)
    gs = torch.from_numpy(w.extra["group_starts"]).to(DEV)
    pl = torch.from_numpy(w.extra["prefix_lens"]).to(DEV)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=DEV)
    cws = torch.empty(pkv.cascade_workspace_size(g.q, g.kc, g.bt, len(pl),
                                                 int(w.extra["prefix_lens"].max()),
                                                 max_seq_len=int(w.seq_lens.max())),
                      dtype=torch.uint8, device=DEV)
    p = workloads.prefill_small(3, 3, 8, 2, 64, 16, 60, 24)
    gp = GpuSide(p)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(p.extra["q_lens"])]).astype(np.int32)).to(DEV)
    pout = torch.empty(tuple(p.q.shape), dtype=torch.float32, device=DEV)

    plmax = int(w.extra["prefix_lens"].max())  # host values: nothing reads the device in capture

    def both():
        pkv.cascade_decode(g.q, g.kc, g.vc, g.bt, g.lens, gs, pl, w.block_size, w.scale, out,
                           max_prefix_len=plmax, max_seq_len=int(w.seq_lens.max()),
                           workspace=cws)
        pkv.paged_prefill(gp.q, gp.kc, gp.vc, gp.bt, gp.lens, cu, p.block_size, p.scale, pout,
                          max_q_len=int(p.extra["q_lens"].max()),
                          max_seq_len=int(p.seq_lens.max()))
    _replays_match(both, [out, pout])
