"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Cache writers and copies: bit-exact.  Attention: per element
|d| <= 5e-3 or |d| <= 1e-2 |ref| against the fp64 oracle; with fp32 output
also max |d| <= 5e-3.  Every unused cache byte is NaN."""
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
    say(f"device: {torch.cuda.get_device_name(0)}")


def _check_caches(g: GpuSide, o: OracleSide, what: str):
    kg, vg = bf16_bits(g.kc), bf16_bits(g.vc)
    assert kg.shape == o.kc.shape and vg.shape == o.vc.shape
    np.testing.assert_array_equal(kg, o.kc, err_msg=f"{what}: k_cache bits")
    np.testing.assert_array_equal(vg, o.vc, err_msg=f"{what}: v_cache bits")


SMALL = {
    "tiny": lambda: workloads.tiny(),
    "g4_d64_b16": lambda: workloads.random_small(21, 6, 16, 4, 64, 16, 300),
    "g1_d64_b8": lambda: workloads.random_small(22, 5, 4, 4, 64, 8, 200, min_len=1),
    "g2_d64_b32": lambda: workloads.random_small(23, 4, 8, 4, 64, 32, 520),
    "g8_d128_b16": lambda: workloads.random_small(24, 3, 16, 2, 128, 16, 700),
    "g16_d64_b16": lambda: workloads.random_small(25, 3, 16, 1, 64, 16, 333),
    "g4_d64_b16_k3": lambda: workloads.random_small(26, 4, 8, 2, 64, 16, 900, k_mult=3.0),
    "g2_d16_b4": lambda: workloads.random_small(27, 5, 4, 2, 16, 4, 50, min_len=0),
    "g3_d40_b5": lambda: workloads.random_small(28, 4, 6, 2, 40, 5, 60, min_len=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_reshape_and_cache_bit_exact(name):
    say(f"case reshape_and_cache {name}")
    w = SMALL[name]()
    _check_caches(GpuSide(w), OracleSide(w), name)


def matrix_core_shape(w) -> bool:
    g = w.num_q_heads // w.num_kv_heads
    return w.head_dim in (64, 128) and w.block_size in (8, 16, 32) and g <= 16


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("kernel", ["auto", "stream_wg", "stream", "mfma", "generic"])
def test_decode_small(name, kernel):
    say(f"case decode {name} kernel={kernel}")
    w = SMALL[name]()
    if kernel in ("stream_wg", "stream", "mfma") and not matrix_core_shape(w):
        pytest.skip("shape outside the matrix-core kernels")
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    kw = dict(kernel=kernel)
    if kernel == "mfma":
        kw["partition_size"] = 64
    out = g.decode(torch.float32, **kw)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"{name}/{kernel}/f32")
    outb = g.decode(torch.bfloat16, **kw)
    compare(outb.float().cpu().numpy(), ref, strict_abs=False, what=f"{name}/{kernel}/bf16")


@pytest.mark.parametrize("waves", [4, 8, 12, 64, 256, 2048])
def test_stream_wave_counts(waves):
    """Fewer wavefronts than chunks (ranges over 64 chunks: several batches
    per wavefront), more wavefronts than chunks (one chunk each), units cut
    into many pieces; lengths include 0 and 1."""
    say(f"case stream waves={waves}")
    w = workloads.random_small(35, 9, 16, 4, 64, 16, 2100, min_len=0)
    w.seq_lens[2] = 0
    w.seq_lens[5] = 1
    w.k_tok = w.k_tok[: int(w.seq_lens.sum())]
    w.v_tok = w.v_tok[: int(w.seq_lens.sum())]
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out = g.decode(torch.float32, kernel="stream", stream_waves=waves)
    assert np.all(out[2].cpu().numpy() == 0)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"stream w{waves}")


@pytest.mark.parametrize("waves", [8, 16, 72, 400, 2048])
def test_stream_wg_group_counts(waves):
    """Workgroups of 8 wavefronts: one group (the 9 sequences' ~2000 chunks
    then need 14 windows in turn), two groups (7 windows each), 9, 50 and
    256 groups (one window each, units cut into many pieces, more windows
    than some units have chunks); lengths include 0 and 1."""
    say(f"case stream_wg waves={waves}")
    w = workloads.random_small(35, 9, 16, 4, 64, 16, 2100, min_len=0)
    w.seq_lens[2] = 0
    w.seq_lens[5] = 1
    w.k_tok = w.k_tok[: int(w.seq_lens.sum())]
    w.v_tok = w.v_tok[: int(w.seq_lens.sum())]
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out = g.decode(torch.float32, kernel="stream_wg", stream_waves=waves)
    assert np.all(out[2].cpu().numpy() == 0)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"stream_wg w{waves}")
    outb = g.decode(torch.bfloat16, kernel="stream_wg", stream_waves=waves)
    compare(outb.float().cpu().numpy(), ref, strict_abs=False, what=f"stream_wg w{waves} bf16")


@pytest.mark.parametrize("name", ["g8_d128_b16", "g16_d64_b16", "g1_d64_b8", "g2_d64_b32"])
def test_stream_wg_windows(name):
    """One workgroup walking several windows at each head shape and block
    size (head_dim 128: 4 wavefronts a group)."""
    say(f"case stream_wg windows {name}")
    w = SMALL[name]()
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    for waves in (4, 8):
        out = g.decode(torch.float32, kernel="stream_wg", stream_waves=waves)
        compare(out.cpu().numpy(), ref, strict_abs=True, what=f"{name} stream_wg w{waves}")


# Units of 8, 9, 16, 17, 64 and 65 chunks (the merge batches hold eight
# slots), single-chunk units and partial last chunks, over two KV heads.
MERGE_LENS = [8 * 32, 9 * 32 - 3, 16 * 32, 17 * 32 - 31, 64 * 32, 65 * 32 - 1, 1, 2, 31, 33,
              5 * 32]


@pytest.mark.parametrize("waves", [8, 16, 56, 200, 2048])
def test_stream_wg_merge_batches(waves):
    """The workgroup kernel's end of window: each unit's chunk slots merged
    in batches of eight, then the batches, for units whose chunk counts sit
    on and beside the batch edges; with 1 group (three windows in turn), 2,
    7, 25 and 256 groups the windows cut those units at many places,
    including windows inside one unit (cut at both ends).  Repeated calls
    give the same bits."""
    say(f"case stream_wg merge batches waves={waves}")
    w = workloads.random_small(38, len(MERGE_LENS), 8, 2, 64, 16, 0, lens=MERGE_LENS)
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out = g.decode(torch.float32, kernel="stream_wg", stream_waves=waves)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"merge batches w{waves}")
    again = g.decode(torch.float32, kernel="stream_wg", stream_waves=waves)
    np.testing.assert_array_equal(again.cpu().numpy(), out.cpu().numpy())


def test_stream_wg_lengths_over_bound_give_nan():
    """max_seq_len sizes the windows and the workspace; lengths far above it
    (a broken contract) fill the output with NaN instead of overrunning LDS."""
    say("case stream_wg over bound")
    w = workloads.random_small(37, 4, 16, 4, 64, 16, 2000, min_len=1500)
    g = GpuSide(w)
    out = g.decode(torch.float32, kernel="stream_wg", stream_waves=8, max_seq_len=32)
    assert torch.isnan(out).all()


@pytest.mark.parametrize("num_seqs", [64, 65, 300, 2048, 2100])
def test_many_short_sequences(num_seqs):
    """The stream kernel keeps every length in LDS up to 2048 sequences;
    beyond that AUTO runs the partitioned kernel.  64 sequences are the most
    the workgroup kernel holds in its wavefronts' lanes; 65 and 300 take its
    general set-up."""
    say(f"case many sequences S={num_seqs}")
    w = workloads.random_small(36, num_seqs, 8, 2, 64, 16, 40, min_len=0)
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out = g.decode(torch.float32)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"S{num_seqs} auto")
    if num_seqs <= 2048:
        for kernel in ("stream_wg", "stream"):
            out = g.decode(torch.float32, kernel=kernel)
            compare(out.cpu().numpy(), ref, strict_abs=True, what=f"S{num_seqs} {kernel}")


@pytest.mark.parametrize("ps", [32, 64, 96, 256, 512, 1024])
@pytest.mark.parametrize("waves", [1, 2, 4])
@pytest.mark.parametrize("balanced", [False, True])
def test_decode_partition_and_wave_sweep(ps, waves, balanced):
    say(f"case sweep ps={ps} waves={waves} balanced={balanced}")
    w = workloads.random_small(30, 6, 16, 4, 64, 16, 1100, min_len=1)
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    out = g.decode(torch.float32, kernel="mfma", partition_size=ps, waves_per_group=waves,
                   balance_partitions=balanced)
    compare(out.cpu().numpy(), ref, strict_abs=True, what=f"ps{ps}/w{waves}/bal{balanced}")


def test_decode_generic_partitions():
    say("case generic partitions")
    w = workloads.random_small(31, 5, 6, 3, 40, 5, 400, min_len=0)
    g, o = GpuSide(w), OracleSide(w)
    ref = o.decode()
    for ps in (5, 35, 100, 400):
        out = g.decode(torch.float32, kernel="generic", partition_size=ps)
        compare(out.cpu().numpy(), ref, strict_abs=True, what=f"generic ps{ps}")


def test_edge_lengths():
    """T = 0, 1, B-1, B, B+1, 31, 32, 33, partition boundaries, full table."""
    say("case edge lengths")
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1024]
    w2 = workloads.random_small(32, len(lens), 8, 2, 64, 16, 1024)
    total = sum(lens)
    r = workloads.rng(100, 77)
    w2.seq_lens = np.array(lens, dtype=np.int32)
    w2.k_tok = workloads.normal_bf16(r, (total, 2, 64))
    w2.v_tok = workloads.normal_bf16(r, (total, 2, 64))
    need = [-(-t // 16) for t in lens]
    pool = sum(need) + 2
    perm = r.permutation(pool).astype(np.int32)
    bt = np.full((len(lens), 64), perm[-1], dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    w2.block_tables, w2.num_blocks, w2.poison_block = bt, pool, int(perm[-1])
    g, o = GpuSide(w2), OracleSide(w2)
    ref = o.decode()
    assert np.all(ref[0] == 0)
    for kernel in ("mfma", "generic"):
        for ps in (32, 256):
            out = g.decode(torch.float32, kernel=kernel, partition_size=ps).cpu().numpy()
            assert np.all(out[0] == 0)
            compare(out, ref, strict_abs=True, what=f"edges {kernel} ps{ps}")
    for kernel in ("stream", "stream_wg"):
        for waves in (4, 16, 400):
            out = g.decode(torch.float32, kernel=kernel, stream_waves=waves).cpu().numpy()
            assert np.all(out[0] == 0)
            compare(out, ref, strict_abs=True, what=f"edges {kernel} w{waves}")
    # T = 1: the output is v_0 exactly (one weight of exactly 1)
    v0 = oracle.widen_bf16(w2.v_tok[0])  # sequence 1's only token (sequence 0 is empty)
    for kernel in ("stream_wg", "stream", "mfma", "generic"):
        out = g.decode(torch.float32, kernel=kernel).cpu().numpy()
        np.testing.assert_array_equal(out[1], np.repeat(v0, 4, axis=0))


@pytest.mark.parametrize("kernel", ["stream_wg", "stream", "mfma"])
def test_permutation_invariance_and_determinism(kernel):
    say(f"case permutation invariance {kernel}")
    w = workloads.random_small(33, 6, 16, 4, 64, 16, 700)
    g = GpuSide(w)
    kw = dict(kernel=kernel, partition_size=128 if kernel == "mfma" else 0)
    a = g.decode(torch.float32, **kw).cpu()
    b = g.decode(torch.float32, **kw).cpu()
    assert torch.equal(a, b), "repeated runs differ"
    perm = workloads.rng(100, 78).permutation(w.num_blocks).astype(np.int32)
    g2 = GpuSide(w, block_tables=perm[w.block_tables])
    c = g2.decode(torch.float32, **kw).cpu()
    assert torch.equal(a, c), "output depends on physical placement"


def test_merge_entry_point_z_3_1():
    say("case merge Z=3,1")
    o1 = torch.tensor([1.0, -2.0, 0.5, 8.0])
    o2 = torch.tensor([-3.0, 4.0, 0.25, 0.0])
    po = torch.stack([o1, o2])[None].to(DEV)
    lse = torch.log(torch.tensor([[3.0, 1.0]])).to(DEV)
    out = torch.empty((1, 4), device=DEV)
    pkv.merge_attention_states(po, lse, out)
    np.testing.assert_allclose(out.cpu().numpy()[0], (0.75 * o1 + 0.25 * o2).numpy(), rtol=1e-6,
                               atol=1e-6)


def test_merge_entry_point_random():
    say("case merge random")
    r = np.random.default_rng(5)
    o = r.normal(size=(300, 7, 128)).astype(np.float32)
    lse = (r.normal(size=(300, 7)) * 30).astype(np.float32)
    lse[::5, 2] = -np.inf
    o[::5, 2] = np.nan  # an empty segment's output must never be read
    lse[7, :] = -np.inf
    ref = oracle.merge_states(o.astype(np.float64), lse.astype(np.float64))
    out = torch.empty((300, 128), device=DEV)
    pkv.merge_attention_states(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV), out)
    got = out.cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=2e-5, atol=2e-6)
    assert np.all(got[7] == 0)


def test_copy_blocks_bit_exact():
    say("case copy_blocks")
    r = np.random.default_rng(6)
    layers, nb = 3, 40
    ks = [r.integers(0, 0xFFFF, size=(nb, 8, 16, 64), dtype=np.uint16) for _ in range(layers)]
    vs = [r.integers(0, 0xFFFF, size=(nb, 8, 64, 16), dtype=np.uint16) for _ in range(layers)]
    src = r.choice(20, 12, replace=False)
    dst = 20 + r.choice(20, 12, replace=False)
    pairs = np.stack([src, dst], 1).astype(np.int32)
    gk = [bits_to_bf16(k).to(DEV) for k in ks]
    gv = [bits_to_bf16(v).to(DEV) for v in vs]
    pkv.copy_blocks(gk, gv, torch.from_numpy(pairs).to(DEV))
    oracle.copy_blocks(ks + vs, [tuple(p) for p in pairs])
    for l in range(layers):
        np.testing.assert_array_equal(bf16_bits(gk[l]), ks[l])
        np.testing.assert_array_equal(bf16_bits(gv[l]), vs[l])


def test_negative_slots_are_skipped():
    say("case negative slots")
    kc, vc = pkv.new_kv_cache(4, 2, 16, 64, fill=1.0)
    k = torch.randn(3, 2, 64, device=DEV).to(torch.bfloat16)
    slots = torch.tensor([-1, 5, -7], dtype=torch.int64, device=DEV)
    pkv.reshape_and_cache(k, k, slots, kc, vc)
    ko, vo = oracle.new_cache(4, 2, 16, 64, fill=0x3F80)
    oracle.write_cache(ko, vo, bf16_bits(k), bf16_bits(k), slots.cpu().numpy())
    np.testing.assert_array_equal(bf16_bits(kc), ko)
    np.testing.assert_array_equal(bf16_bits(vc), vo)


def test_workspace_reuse_across_shapes():
    """One workspace serves split-KV calls of changing shapes back to back:
    leftover partial results of one shape land where the next shape keeps its
    counters.  A DecodeWorkspace wrapping a buffer of random bytes clears its
    counter region only when a call needs more of it; a raw tensor gets its
    counter region cleared before every call."""
    say("case workspace reuse across shapes")
    cases = [workloads.random_small(40, 5, 16, 4, 64, 16, 900, min_len=1),
             workloads.random_small(41, 9, 8, 2, 64, 16, 1500, min_len=1),
             workloads.random_small(42, 3, 16, 2, 128, 32, 1200, min_len=1),
             workloads.random_small(43, 12, 32, 8, 64, 8, 600, min_len=1)]
    sides = [(GpuSide(w), OracleSide(w)) for w in cases]
    refs = [o.decode() for _, o in sides]
    g = torch.Generator().manual_seed(44)
    raw = torch.randint(0, 256, (8 << 20,), dtype=torch.uint8, generator=g).to(DEV)
    tracked = pkv.DecodeWorkspace(raw.clone())
    for rnd in range(3):
        for i, (gs, _) in enumerate(sides):
            for label, ws in (("tracked", tracked), ("raw", raw)):
                for kw in (dict(kernel="mfma", partition_size=64),
                           dict(kernel="mfma", partition_size=64, balance_partitions=True),
                           dict(kernel="stream", stream_waves=32)):
                    out = gs.decode(torch.float32, workspace=ws, **kw)
                    compare(out.cpu().numpy(), refs[i], strict_abs=True,
                            what=f"ws {label} round {rnd} case {i} {kw}")
    # every counter region a call used is zero again afterwards
    for i, (gs, _) in enumerate(sides):
        w = gs.w
        dims = pkv._dims(gs.q, gs.kc, gs.bt, int(w.seq_lens.max()), 64, torch.float32, "mfma", 0,
                         False)
        z = pkv.lib().pkv_decode_workspace_zeroed_bytes(pkv.ctypes.byref(dims), w.block_size)
        assert int(raw[:z].count_nonzero()) == 0


@pytest.mark.parametrize("kernel", ["auto", "stream_wg", "stream"])
def test_no_shared_blocks_hint_is_bit_identical(kernel):
    """The streaming-load hint changes only how K/V are loaded: outputs are
    the same bits with and without it (plain decode and fused step), and
    within tolerance of the oracle."""
    say(f"case no_shared_blocks hint kernel={kernel}")
    w = workloads.random_small(91, 24, 32, 8, 64, 16, 2500, min_len=1)
    g, o = GpuSide(w), OracleSide(w)
    a = g.decode(torch.float32, kernel=kernel)
    b = g.decode(torch.float32, kernel=kernel, no_shared_blocks=True)
    assert torch.equal(a, b)
    compare(b.cpu().numpy(), o.decode(), strict_abs=True, what=f"hint/{kernel}")
    cu = w.cu_seqlens
    k_new = bits_to_bf16(w.k_tok[cu[1:] - 1]).to(DEV)
    v_new = bits_to_bf16(w.v_tok[cu[1:] - 1]).to(DEV)
    outs = []
    for hint in (False, True):
        out = torch.empty_like(a)
        pkv.paged_attention_decode_append(g.q, k_new, v_new, g.kc, g.vc, g.bt, g.lens,
                                          w.block_size, w.scale, out,
                                          max_seq_len=int(w.seq_lens.max()), kernel=kernel,
                                          no_shared_blocks=hint)
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], a)  # the new tokens are the cached ones: same result


def test_workspace_grown_on_a_side_stream():
    """A decode on a stream other than torch's current one, with a
    DecodeWorkspace that grows for it: the buffer is allocated and zeroed on
    that stream, so the counters are zero when the kernel starts.  Repeated
    with a larger call (the workspace grows again) and against the default
    per-stream workspace."""
    say("case workspace grown on a side stream")
    side = torch.cuda.Stream()
    ws = pkv.DecodeWorkspace(device=DEV)
    for seed, s_, mx in ((92, 6, 300), (93, 40, 3000)):
        w = workloads.random_small(seed, s_, 32, 8, 64, 16, mx, min_len=1)
        g, o = GpuSide(w), OracleSide(w)
        ref = o.decode()
        torch.cuda.synchronize()
        outs = []
        for wsp in (ws, None):
            out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32,
                              device=DEV)
            side.wait_stream(torch.cuda.current_stream())
            pkv.paged_attention_decode(g.q, g.kc, g.vc, g.bt, g.lens, w.block_size, w.scale, out,
                                       max_seq_len=int(w.seq_lens.max()), workspace=wsp,
                                       stream=side)
            side.synchronize()
            outs.append(out)
        for out in outs:
            compare(out.cpu().numpy(), ref, strict_abs=True, what=f"side stream S={s_}")
        assert torch.equal(outs[0], outs[1])
