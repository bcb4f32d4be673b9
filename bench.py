"""Benchmark of the paged decode-attention hot path on one MI355X.

One step = one decode step of one layer of the Llama-3.2-1B-shaped batch: the
new token of each of the 64 sequences is written into its slot and attention
runs over every cached token (32 q heads / 8 KV heads, head_dim 64, bf16,
B = 16, lengths U[128, 2048], physical blocks a seeded permutation).  By
default the step is one ``paged_attention_decode_append`` launch (write and
attention fused); ``--unfused`` runs ``reshape_and_cache`` then
``paged_attention_decode``.  There is no copy-on-write in this workload
(``copy_blocks`` has no pairs).

Metric: effective KV read GB/s = (sum_b T_b * Hkv * D * 2 tensors * 2 bytes)
/ step time.  The cache is rotated over enough independent copies (> 1 GiB in
total) that it cannot sit in the 256 MB Infinity Cache between steps.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

``--workload`` is llama_b64 (default, the headline line) or long_splitkv;
prefix_cow, pool16, prefill_chunked, swap and size_sweep print their own report
lines instead (logical and unique GB/s with the shared-prefix decode and the
copy_blocks time; the 16-layer pool step per block size, fused and unfused
writer; the chunked prefill's matrix-core rate; block swap-out/in against the
host link; the llama-shaped step at 16 .. 256 sequences and the read kernel at
32 MiB .. 1 GiB, each fitted to a fixed cost plus a streaming rate).

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one
GPU.  ``roofline.achieved`` is the decode launch alone (HIP events on the
stream it runs on); ``roofline.traffic`` is the HBM bytes per launch measured
with rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by the same counters
on a plain copy of known size) as recorded in profiles/pmc_traffic.json, and
null when the decode source has changed since then.

    python bench.py --calibrate-copy 256   # a plain 256 MiB copy, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
ROTATE_BYTES = 1 << 30
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_373_amd", "csrc", f)
                  for f in ("chunk.h", "decode.hip", "decode_wg.hip", "api.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bits_to_bf16(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def make_workload(name: str):
    import workloads

    if name == "llama_b64":
        return workloads.llama_decode()
    if name == "long_splitkv":
        return workloads.long_context()
    raise SystemExit(f"unknown workload {name!r}")


def source_digest() -> str:
    """sha256 over the decode kernels' sources, in a fixed order."""
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per decode launch from the committed counter records, if one
    was taken on this workload and kernel with the current decode source."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f).get("records", [])
    except (OSError, ValueError, AttributeError):
        return None
    digest = source_digest()
    for rec in recs:
        if (rec.get("workload"), rec.get("kernel")) == (workload, kernel) \
                and rec.get("decode_source_sha256") == digest:
            return rec.get("hbm_bytes_per_launch")
    return None


def calibrate_copy(mib: int, reps: int) -> int:
    """A plain device-to-device copy of `mib` MiB, `reps` times: the known-size
    reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "reps": reps}), flush=True)
    return 0


def host_cpu() -> str:
    """CPU model and logical CPU count of the host the oracle ran on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    """The oracle as it stands on the host cores: the paged path (each
    sequence's K/V gathered through its block table from the paged cache,
    then dense fp64 attention; OpenMP over (sequence, KV head)) over host
    copies of the workload's cache and tables, repeated for about budget_s
    seconds.  Building the host cache is not timed."""
    import oracle

    ko, vo = oracle.new_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    slots = np.array([oracle.slot(w.block_tables[b], t, w.block_size)
                      for b in range(w.num_seqs) for t in range(int(w.seq_lens[b]))],
                     dtype=np.int64)
    oracle.write_cache(ko, vo, w.k_tok, w.v_tok, slots)
    threads = oracle.max_threads()

    def run(nthreads, budget):
        reps, total = 0, 0.0
        while total < budget and reps < 5000:
            t0 = time.perf_counter()
            oracle.paged_decode(w.q, ko, vo, w.block_tables, w.seq_lens, w.scale,
                                num_threads=nthreads)
            total += time.perf_counter() - t0
            reps += 1
        return reps, total / reps

    reps, per = run(threads, budget_s)
    reps1, per1 = run(1, budget_s / 3)
    return {"value": round(w.kv_bytes() / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole {w.name} step ({w.total_tokens} tokens x {w.num_kv_heads} KV heads):"
                      f" oracle.paged_decode, K/V gathered through the block tables from the"
                      f" paged cache then fp64 dense attention, repeated {reps}x,"
                      f" {per * 1e3:.1f} ms each",
            "single_thread": {"value": round(w.kv_bytes() / per1 / 1e9, 3), "unit": "GB/s",
                              "sample": f"{reps1}x, {per1 * 1e3:.1f} ms each"},
            "host": host_cpu()}


PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_373_amd", "libpkv_probe.so")
_probe_lib = None


def probe_lib():
    """The benchmark's read-probe library (built beside libpagedkv.so by the
    package's build step; not part of the attention library's ABI)."""
    global _probe_lib
    if _probe_lib is None:
        import ctypes

        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: build with python -m "
                               "paged_kv_cache_373_amd.build")
        L = ctypes.CDLL(PROBE_LIB)
        L.pkv_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.pkv_probe_read_tiles.restype = ctypes.c_int
        _probe_lib = L
    return _probe_lib


def read_probe(src, order, sink, stream=None) -> None:
    """Reads order.numel() 2 KiB tiles of src (uint8 device tensor) in the
    given order; sink (int32, >= 8 words per tile) gets one folded word per
    thread.  Every order entry must name a tile inside src (the callers build
    the orders as permutations of src's tiles; they are not checked here, to
    keep device reads out of the timed loop)."""
    import torch

    n = order.numel()
    if (src.dtype != torch.uint8 or order.dtype != torch.int32 or sink.dtype != torch.int32
            or n % 32 != 0 or n * 2048 > src.numel() or sink.numel() < 8 * n):
        raise ValueError("probe: uint8 src holding the tiles, int32 order (a multiple of 32 "
                         "tiles) and int32 sink of 8 words per tile")
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = probe_lib().pkv_probe_read_tiles(src.data_ptr(), order.data_ptr(), n, sink.data_ptr(),
                                          st.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"pkv_probe_read_tiles returned {rc}")


def read_ceiling(pkv, torch, dev, stream, kv_bytes: int, launches: int) -> dict:
    """Context for the roofline: the library's trivial read kernel over the
    step's byte count as whole 2 KiB tiles in random order (the cache's access
    pattern), rotating over 8 regions so that none is cache resident."""
    tiles = (kv_bytes // 2048) // 32 * 32
    regions = 8
    src = torch.zeros(regions * tiles * 2048, dtype=torch.uint8, device=dev)
    g = torch.Generator().manual_seed(373)
    orders = [(torch.randperm(tiles, generator=g) + r * tiles).to(torch.int32).to(dev)
              for r in range(regions)]
    sink = torch.empty(tiles * 8, dtype=torch.int32, device=dev)
    for r in range(2 * regions):
        read_probe(src, orders[r % regions], sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    prime(stream)
    e0.record(stream)
    for r in range(launches):
        read_probe(src, orders[r % regions], sink)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    gbs = tiles * 2048 / (ms * 1e-3) / 1e9
    return {"value": round(gbs, 2), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "us_per_launch": round(ms * 1e3, 3), "bytes": tiles * 2048,
            "kind": "trivial read kernel (libpkv_probe.so): the step's byte count as 2 KiB "
                    "tiles in random order, 8 rotated regions, launches back to back"}


def prime(stream) -> None:
    """Hold `stream` with a short GPU-side sleep before a timed region opens,
    so that the host has enqueued the region's first steps by the time the
    start event runs: otherwise the GPU idles for the host's per-call cost of
    the first step inside every timed region (~13 us here, about 0.65 us per
    step over 20 steps)."""
    import torch

    with torch.cuda.stream(stream):
        torch.cuda._sleep(2_000_000)


def timed_graph(fn, calls: int, replays: int = 10) -> float:
    """Milliseconds per call of fn(i) on the GPU: `calls` calls captured in a
    HIP graph, replayed `replays` times between one pair of events.  For
    launches shorter than the host's per-call cost, where back-to-back eager
    calls would time the host."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(calls):
                fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (calls * replays)


def timed(stream, fn, launches: int, warmup: int = 3) -> float:
    """Milliseconds per call of fn(i), `launches` calls back to back between
    one pair of events on `stream` (after `warmup` untimed calls)."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    prime(stream)
    e0.record(stream)
    for i in range(launches):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / launches


def run_prefix_cow(args) -> int:
    """The shared-prefix workload: 4 prompts x 1000 tokens forked 16 ways
    (B = 16), 1..300 private tokens per fork, the shared 8-token tails copied
    with copy_blocks before the first private write.  Reports the decode and
    the shared-prefix (cascade) decode on logical bytes (every fork's tokens)
    and on unique bytes (each physical block once), and the copy_blocks
    launch on its own."""
    import torch

    import paged_kv_cache_373_amd as pkv
    import workloads

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    w = workloads.prefix_sharing()
    ex = w.extra
    P, L, F, bs = ex["num_prompts"], ex["prompt_len"], ex["forks"], w.block_size
    hkv, d = w.num_kv_heads, w.head_dim
    bm = pkv.BlockManager(w.num_blocks, bs, free_order=w.free_list)
    cu = w.cu_seqlens
    prompt_slots, private = [], []
    for p in range(P):
        bm.add_sequence(("prompt", p))
        prompt_slots.append(bm.append_tokens(("prompt", p), L)[0])
    for p in range(P):
        for f in range(F):
            bm.fork(("prompt", p), p * F + f)
        bm.release(("prompt", p))
    pairs = []
    for b in range(w.num_seqs):
        slots, copies = bm.append_tokens(b, int(ex["n_private"][b]))
        pairs += copies
        private.append((slots, cu[b] + L + np.arange(int(ex["n_private"][b]))))
    bt = torch.from_numpy(bm.block_table_array(list(range(w.num_seqs)), pad=0)).to(dev)
    used = sorted({blk for b in range(w.num_seqs) for blk in bm.table(b)})
    # unique bytes: each physical block's valid tokens once
    valid = {}
    for b in range(w.num_seqs):
        T = int(w.seq_lens[b])
        for j, blk in enumerate(bm.table(b)):
            valid[blk] = max(valid.get(blk, 0), min(bs, T - j * bs))
    unique_tokens = sum(valid.values())
    pool_bytes = 2 * w.num_blocks * hkv * bs * d * 2
    copies = args.copies or max(2, math.ceil(ROTATE_BYTES / pool_bytes))
    kt, vt = bits_to_bf16(w.k_tok).to(dev), bits_to_bf16(w.v_tok).to(dev)
    pairs_d = torch.tensor(pairs, dtype=torch.int32, device=dev)
    caches = []
    for _ in range(copies):
        kc, vc = pkv.new_kv_cache(w.num_blocks, hkv, bs, d, device=dev, fill=float("nan"))
        for p in range(P):
            rows = torch.from_numpy(cu[p * F] + np.arange(L)).to(dev)
            pkv.reshape_and_cache(kt[rows], vt[rows], torch.from_numpy(prompt_slots[p]).to(dev),
                                  kc, vc)
        pkv.copy_blocks([kc], [vc], pairs_d)
        for slots, rows in private:
            r = torch.from_numpy(rows).to(dev)
            pkv.reshape_and_cache(kt[r], vt[r], torch.from_numpy(slots).to(dev), kc, vc)
        caches.append((kc, vc))
    q = bits_to_bf16(w.q).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((w.num_seqs, w.num_q_heads, d), dtype=torch.bfloat16, device=dev)
    ws = pkv.DecodeWorkspace(device=dev)
    kw = dict(max_seq_len=int(w.seq_lens.max()), kernel=args.kernel, workspace=ws)

    def dec(i):
        kc, vc = caches[i % copies]
        pkv.paged_attention_decode(q, kc, vc, bt, lens, bs, w.scale, out, **kw)

    def cow(i):
        kc, vc = caches[i % copies]
        pkv.copy_blocks([kc], [vc], pairs_d)

    gs_np, pl_np = bm.shared_prefix_groups(list(range(w.num_seqs)))
    gs, pl = torch.from_numpy(gs_np).to(dev), torch.from_numpy(pl_np).to(dev)
    cws = torch.empty(pkv.cascade_workspace_size(q, caches[0][0], bt, len(pl_np),
                                                 int(pl_np.max()),
                                                 max_seq_len=kw["max_seq_len"]),
                      dtype=torch.uint8, device=dev)

    def casc_with(kernel):
        def casc(i):
            kc, vc = caches[i % copies]
            pkv.cascade_decode(q, kc, vc, bt, lens, gs, pl, bs, w.scale, out,
                               max_prefix_len=int(pl_np.max()), max_seq_len=kw["max_seq_len"],
                               workspace=cws, kernel=kernel)
        return casc

    ms = timed(stream, dec, args.steps, args.warmup)
    ms_casc = timed(stream, casc_with("auto"), args.steps, args.warmup)
    ms_casc2 = timed(stream, casc_with("mfma"), args.steps, args.warmup)
    ms_cow = timed(stream, cow, args.steps, args.warmup)
    ms_cow_gpu = timed_graph(cow, 50)
    logical = w.kv_bytes()
    unique = unique_tokens * hkv * d * 2 * 2
    print(json.dumps({
        "workload": "prefix_cow", "kernel": pkv.decode_plan_kernel(q, caches[0][0], bt,
                                                                    max_seq_len=kw["max_seq_len"],
                                                                    kernel=args.kernel),
        "decode_us": round(ms * 1e3, 3),
        "logical_kv_bytes": logical, "logical_gbs": round(logical / (ms * 1e-3) / 1e9, 1),
        "unique_kv_bytes": unique, "unique_gbs": round(unique / (ms * 1e-3) / 1e9, 1),
        "cascade_us": round(ms_casc * 1e3, 3),
        "cascade_kernel": pkv.cascade_plan_kernel(q, caches[0][0], bt, len(pl_np),
                                                  int(pl_np.max()),
                                                  max_seq_len=kw["max_seq_len"]),
        "cascade_two_launch_us": round(ms_casc2 * 1e3, 3),
        "cascade_logical_gbs": round(logical / (ms_casc * 1e-3) / 1e9, 1),
        "cascade_unique_gbs": round(unique / (ms_casc * 1e-3) / 1e9, 1),
        "cascade_groups": int(len(pl_np)), "cascade_prefix_tokens": int(pl_np.max()),
        "cascade_roofline": {"bound": "hbm", "achieved": round(unique / (ms_casc * 1e-3) / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(unique / (ms_casc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "note": "unique K/V bytes (each block once) per call"},
        "copy_blocks_pairs": len(pairs), "copy_blocks_bytes": 2 * len(pairs) * hkv * bs * d * 2,
        "copy_blocks_us": round(ms_cow_gpu * 1e3, 3),
        "copy_blocks_us_note": "GPU time per call, 50 calls replayed from a HIP graph; "
                               "eager calls back to back are host-bound",
        "copy_blocks_eager_call_us": round(ms_cow * 1e3, 3), "cache_copies_rotated": copies,
        "blocks_in_use": len(used), "steps": args.steps}), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def run_prefill(args) -> int:
    """The Llama-shaped chunked prefill of one layer: 8 sequences, each adding
    512 new tokens after U{0..2048} cached ones (their K/V written first, as a
    prefill step does); one pkv_paged_prefill launch per step.  Reports new
    tokens per second and the attention's algorithmic matrix-core rate: per
    new token and query head, 4 D flops per visible position (QK and PV)."""
    import torch

    import paged_kv_cache_373_amd as pkv
    import workloads

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    w = workloads.prefill_chunked()
    ql = w.extra["q_lens"]
    n = int(ql.sum())
    cu_np = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    ctx = w.seq_lens - ql
    visible = int(sum(int(ql[b]) * int(ctx[b]) + int(ql[b]) * (int(ql[b]) + 1) // 2
                      for b in range(w.num_seqs)))
    flops = 4 * w.head_dim * w.num_q_heads * visible
    pool_bytes = 2 * w.num_blocks * w.num_kv_heads * w.block_size * w.head_dim * 2
    copies = args.copies or max(2, math.ceil(ROTATE_BYTES / pool_bytes))
    seq = np.repeat(np.arange(w.num_seqs), w.seq_lens)
    pos = np.concatenate([np.arange(t) for t in w.seq_lens])
    from paged_kv_cache_373_amd.block_manager import slot_mapping_for
    slots = torch.from_numpy(slot_mapping_for(w.block_tables, seq, pos, w.block_size)).to(dev)
    kt, vt = bits_to_bf16(w.k_tok).to(dev), bits_to_bf16(w.v_tok).to(dev)
    caches = []
    for _ in range(copies):
        kc, vc = pkv.new_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim,
                                  device=dev, fill=float("nan"))
        pkv.reshape_and_cache(kt, vt, slots, kc, vc)
        caches.append((kc, vc))
    q = bits_to_bf16(w.q).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    cu = torch.from_numpy(cu_np).to(dev)
    out = torch.empty((n, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)

    def step(i):
        kc, vc = caches[i % copies]
        pkv.paged_prefill(q, kc, vc, bt, lens, cu, w.block_size, w.scale, out,
                          max_q_len=int(ql.max()), max_seq_len=int(w.seq_lens.max()))

    trials = [timed(stream, step, args.steps, args.warmup) for _ in range(max(1, args.trials))]
    ms = float(np.median(trials))
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "workload": "prefill_chunked", "metric": "paged prefill attention matrix-core rate",
        "us_per_step": round(ms * 1e3, 3), "new_tokens": n,
        "new_tokens_per_s": round(n / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_launch": flops,
                     "note": "4 D flops per (new token, q head, visible position)"},
        "kv_bytes_cached": w.kv_bytes(), "cache_copies_rotated": copies,
        "trials_us": [round(t * 1e3, 3) for t in trials], "steps": args.steps}), flush=True)
    return 0


def run_swap(args) -> int:
    """Block swap-out/in of the Llama-shaped pool: 16 layers of 2048 blocks
    (B = 16, 8 KV heads, head_dim 64: 16 KiB per block per cache), half of
    the blocks (a seeded random choice) swapped out to pinned host memory and
    back in.  Reports each direction's rate over the bytes moved, beside a
    plain contiguous copy of the same size between the device and pinned host
    memory (the host link's ceiling as the runtime reaches it)."""
    import torch

    import paged_kv_cache_373_amd as pkv

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    layers, P, hkv, bs, d = 16, 2048, 8, 16, 64
    n = P // 2
    kcs, vcs = [], []
    for _ in range(layers):
        kc, vc = pkv.new_kv_cache(P, hkv, bs, d, device=dev)
        kc.normal_()
        vc.normal_()
        kcs.append(kc)
        vcs.append(vc)
    ids = torch.from_numpy(np.random.default_rng(373).permutation(P)[:n].astype(np.int32)).to(dev)
    buf = pkv.swap_buffer(kcs, n)
    nbytes = buf.numel() * buf.element_size()
    flat = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    flat_host = buf.view(-1)

    steps = max(3, args.steps // 20)
    ms_out = timed(stream, lambda i: pkv.swap_out(kcs, vcs, ids, buf), steps, 2)
    ms_in = timed(stream, lambda i: pkv.swap_in(kcs, vcs, ids, buf), steps, 2)
    ms_d2h = timed(stream, lambda i: flat_host.copy_(flat, non_blocking=True), steps, 2)
    ms_h2d = timed(stream, lambda i: flat.copy_(flat_host, non_blocking=True), steps, 2)
    gbs = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    print(json.dumps({
        "workload": "swap", "layers": layers, "blocks_moved": n, "bytes_moved": nbytes,
        "swap_out_ms": round(ms_out, 4), "swap_out_gbs": gbs(ms_out),
        "swap_in_ms": round(ms_in, 4), "swap_in_gbs": gbs(ms_in),
        "link_ceiling": {"d2h_gbs": gbs(ms_d2h), "h2d_gbs": gbs(ms_h2d),
                         "kind": "contiguous device <-> pinned host copy of the same bytes"},
        "swap_out_frac_of_ceiling": round(ms_d2h / ms_out, 4),
        "swap_in_frac_of_ceiling": round(ms_h2d / ms_in, 4), "steps": steps}), flush=True)
    return 0


def run_pool16(args) -> int:
    """The 16-layer decode step at pool scale: 2^22 slots per layer (8 GiB of
    K+V per layer), 256 sequences with lognormal lengths (median 1200, capped
    at 8192), B in {8, 16, 32}.  One step = the 16 layers' decode launches in
    turn; with the writer each launch also stores its layer's new token
    (paged_attention_decode_append), without it only attends.  K/V values are
    drawn on the device (the timing does not depend on them)."""
    import torch

    import paged_kv_cache_373_amd as pkv
    import workloads

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    res = {"workload": "pool16", "layers": workloads.POOL_LAYERS, "by_block_size": {}}
    for bs in (8, 16, 32):
        w = workloads.pool_step(bs)
        S, hq, hkv, d = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
        bm = pkv.BlockManager(w.num_blocks, bs, free_order=w.free_list)
        slot_list = []
        for b in range(S):
            bm.add_sequence(b)
            slot_list.append(bm.append_tokens(b, int(w.seq_lens[b]))[0])
        slots = np.concatenate(slot_list)
        cu = w.cu_seqlens
        last = cu[1:] - 1
        pre = slots.copy()
        pre[last] = -1
        bt = torch.from_numpy(bm.block_table_array(list(range(S)), pad=0)).to(dev)
        lens = torch.from_numpy(w.seq_lens).to(dev)
        kt, vt = workloads.pool_layer_tokens_device(0, int(cu[-1]), dev, bs)
        pre_d = torch.from_numpy(pre).to(dev)
        lastd = torch.from_numpy(last).to(dev)
        layers = []
        for layer in range(workloads.POOL_LAYERS):
            kc, vc = pkv.new_kv_cache(w.num_blocks, hkv, bs, d, device=dev)
            pkv.reshape_and_cache(kt, vt, pre_d, kc, vc)
            q = bits_to_bf16(workloads.pool_layer_q(layer, S)).to(dev)
            layers.append((kc, vc, q))
        k_new, v_new = kt[lastd].contiguous(), vt[lastd].contiguous()
        del kt, vt
        new_slots = torch.from_numpy(slots[last]).to(dev)
        out = torch.empty((S, hq, d), dtype=torch.bfloat16, device=dev)
        ws = pkv.DecodeWorkspace(device=dev)
        # every block belongs to one sequence (the block manager hands each
        # out once), which the calls may declare
        no_shared = not args.plain_loads
        kw = dict(max_seq_len=int(w.seq_lens.max()), kernel=args.kernel, workspace=ws,
                  no_shared_blocks=no_shared)

        def step_append(i):
            for kc, vc, q in layers:
                pkv.paged_attention_decode_append(q, k_new, v_new, kc, vc, bt, lens, bs, w.scale,
                                                  out, **kw)

        def step_unfused(i):
            for kc, vc, q in layers:
                pkv.reshape_and_cache(k_new, v_new, new_slots, kc, vc)
                pkv.paged_attention_decode(q, kc, vc, bt, lens, bs, w.scale, out, **kw)

        def step_decode(i):
            for kc, vc, q in layers:
                pkv.paged_attention_decode(q, kc, vc, bt, lens, bs, w.scale, out, **kw)

        n = max(args.steps // 10, 5)
        ms_a = timed(stream, step_append, n, 2)
        ms_u = timed(stream, step_unfused, n, 2)
        ms_d = timed(stream, step_decode, n, 2)
        per_layer = w.kv_bytes()
        res["by_block_size"][str(bs)] = {
            "kernel": pkv.decode_plan_kernel(layers[0][2], layers[0][0], bt,
                                             max_seq_len=kw["max_seq_len"], kernel=args.kernel,
                                             no_shared_blocks=no_shared),
            "no_shared_blocks": no_shared,
            "tokens_per_layer": w.total_tokens, "kv_bytes_per_layer": per_layer,
            "step_ms_with_writer": round(ms_a, 4),
            "step_ms_writer_then_decode": round(ms_u, 4),
            "step_ms_without_writer": round(ms_d, 4),
            "per_layer_gbs_with_writer": round(16 * per_layer / (ms_a * 1e-3) / 1e9, 1),
            "per_layer_gbs_writer_then_decode": round(16 * per_layer / (ms_u * 1e-3) / 1e9, 1),
            "per_layer_gbs_without_writer": round(16 * per_layer / (ms_d * 1e-3) / 1e9, 1),
            "tokens_per_s": round(S / (ms_a * 1e-3), 1), "steps": n}
        log(f"pool16 B={bs}: step {ms_a:.3f} ms with the fused writer, {ms_u:.3f} ms with "
            f"reshape_and_cache then decode, {ms_d:.3f} ms without a writer")
        del layers, out
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)
    return 0


def run_size_sweep(args) -> int:
    """Separates the decode step's fixed cost from its streaming rate: the
    llama-shaped fused step (32 q / 8 KV heads, head_dim 64, block 16,
    lengths U[128, 2048]) at S = 16 .. 256 sequences, and the trivial read
    kernel over 32 MiB .. 1 GiB of 2 KiB tiles (random and sequential
    order), each fitted with time = intercept + bytes / rate.  K/V values are
    drawn on the device; regions rotate so that no launch reads a cache-
    resident one."""
    import torch

    import paged_kv_cache_373_amd as pkv
    import workloads

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    n = max(args.steps // 4, 20)
    trials = max(args.trials, 3)

    def med(fn):
        return float(np.median([timed(stream, fn, n, 3) for _ in range(trials)])) * 1e3

    def fit(rows):
        x = np.array([r["bytes"] for r in rows], float)
        y = np.array([r["us"] for r in rows], float)
        slope, icpt = np.linalg.lstsq(np.vstack([x, np.ones_like(x)]).T, y, rcond=None)[0]
        return {"intercept_us": round(float(icpt), 2), "rate_gbs": round(1e-3 / float(slope), 1)}

    res = {"workload": "size_sweep", "steps_per_trial": n, "trials": trials}
    dec = []
    for S in (16, 32, 64, 128, 256):
        w = workloads.llama_decode(num_seqs=S, with_kv=False)
        hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
        pool_bytes = 2 * w.num_blocks * hkv * bs * d * 2
        copies = max(2, math.ceil(ROTATE_BYTES / pool_bytes))
        caches = []
        for _ in range(copies):
            kc, vc = pkv.new_kv_cache(w.num_blocks, hkv, bs, d, device=dev)
            kc.normal_()
            vc.normal_()
            caches.append((kc, vc))
        bt = torch.from_numpy(w.block_tables).to(dev)
        lens = torch.from_numpy(w.seq_lens).to(dev)
        q = torch.randn((S, w.num_q_heads, d), device=dev).to(torch.bfloat16)
        kn = torch.randn((S, hkv, d), device=dev).to(torch.bfloat16)
        vn = torch.randn((S, hkv, d), device=dev).to(torch.bfloat16)
        out = torch.empty((S, w.num_q_heads, d), dtype=torch.bfloat16, device=dev)
        kw = dict(max_seq_len=int(w.seq_lens.max()), workspace=pkv.DecodeWorkspace(device=dev),
                  no_shared_blocks=not args.plain_loads)

        def step(i):
            kc, vc = caches[i % copies]
            pkv.paged_attention_decode_append(q, kn, vn, kc, vc, bt, lens, bs, w.scale, out, **kw)

        us = med(step)
        kvb = w.kv_bytes()
        dec.append({"num_seqs": S, "bytes": kvb, "us": round(us, 2),
                    "gbs": round(kvb / us / 1e3, 1), "frac": round(kvb / us / 1e3 / HBM_PEAK_GBS, 4)})
        log(f"decode S={S}: {kvb / 1e6:.1f} MB in {us:.2f} us ({kvb / us / 1e3:.0f} GB/s)")
        del caches
        torch.cuda.empty_cache()
    res["decode_step"] = {"rows": dec, "fit": fit(dec)}
    probe = {"random": [], "sequential": []}
    g = torch.Generator().manual_seed(373)
    for mib in (32, 64, 128, 256, 512, 1024):
        tiles = (mib << 20) // 2048 // 32 * 32
        regions = max(2, math.ceil(ROTATE_BYTES / (tiles * 2048)) + 1)
        src = torch.zeros(regions * tiles * 2048, dtype=torch.uint8, device=dev)
        sink = torch.empty(tiles * 8, dtype=torch.int32, device=dev)
        orders = {"random": [(torch.randperm(tiles, generator=g) + r * tiles).to(torch.int32)
                             .to(dev) for r in range(regions)],
                  "sequential": [(torch.arange(tiles) + r * tiles).to(torch.int32).to(dev)
                                 for r in range(regions)]}
        for kind, ords in orders.items():
            us = med(lambda i: read_probe(src, ords[i % regions], sink))
            b = tiles * 2048
            probe[kind].append({"mib": mib, "bytes": b, "us": round(us, 2),
                                "gbs": round(b / us / 1e3, 1),
                                "frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4)})
            log(f"read probe {kind} {mib} MiB: {us:.2f} us ({b / us / 1e3:.0f} GB/s)")
        del src, sink, orders
        torch.cuda.empty_cache()
    res["read_probe"] = {k: {"rows": v, "fit": fit(v)} for k, v in probe.items()}
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_b64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trials", type=int, default=5,
                    help="timed regions of --steps steps each; value is their median")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the trivial read kernel timed over the step's byte count")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: >1 GiB)")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "stream_wg", "stream", "mfma", "generic"])
    ap.add_argument("--stream-waves", type=int, default=0)
    ap.add_argument("--plain-loads", action="store_true",
                    help="do not pass no_shared_blocks (the workload's tables share no block, "
                         "so by default the call declares it and K/V stream non-temporally)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--unfused", action="store_true",
                    help="step = reshape_and_cache + paged_attention_decode (two launches)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(every kernel works on one GPU's share; see DESIGN.md for how it would shard).",
              file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, max(args.steps, 1))
    if args.workload == "prefix_cow":
        return run_prefix_cow(args)
    if args.workload == "pool16":
        return run_pool16(args)
    if args.workload == "prefill_chunked":
        return run_prefill(args)
    if args.workload == "swap":
        return run_swap(args)
    if args.workload == "size_sweep":
        return run_size_sweep(args)

    import torch

    import paged_kv_cache_373_amd as pkv
    from paged_kv_cache_373_amd.block_manager import slot_mapping_for

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"device {torch.cuda.get_device_name(0)}; generating {args.workload}")
    w = make_workload(args.workload)
    s, hq, hkv, d, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    cu = w.cu_seqlens
    kv_bytes = w.kv_bytes()
    pool_bytes = 2 * w.num_blocks * hkv * bs * d * 2
    copies = args.copies or max(2, math.ceil(ROTATE_BYTES / pool_bytes))
    log(f"{w.total_tokens} tokens, KV bytes/step {kv_bytes / 1e6:.1f} MB, pool "
        f"{pool_bytes / 1e6:.1f} MB x {copies} copies")

    # Prefill: every cached token except each sequence's last (the one the
    # step decodes) goes into every copy through the library's writer.
    seq_ids = np.repeat(np.arange(s), w.seq_lens)
    pos = np.concatenate([np.arange(t) for t in w.seq_lens])
    last = cu[1:] - 1
    slots_all = slot_mapping_for(w.block_tables, seq_ids, pos, bs)
    prefill = np.ones(len(pos), bool)
    prefill[last] = False
    k_all = bits_to_bf16(w.k_tok).to(dev)
    v_all = bits_to_bf16(w.v_tok).to(dev)
    slots_prefill = torch.from_numpy(np.where(prefill, slots_all, -1)).to(dev)
    k_new = k_all[torch.from_numpy(last).to(dev)].contiguous()
    v_new = v_all[torch.from_numpy(last).to(dev)].contiguous()
    slots_new = torch.from_numpy(slots_all[last]).to(dev)
    caches = []
    for _ in range(copies):
        kc, vc = pkv.new_kv_cache(w.num_blocks, hkv, bs, d, device=dev, fill=float("nan"))
        pkv.reshape_and_cache(k_all, v_all, slots_prefill, kc, vc)
        caches.append((kc, vc))
    del k_all, v_all
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q = bits_to_bf16(w.q).to(dev)
    out = torch.empty((s, hq, d), dtype=torch.bfloat16, device=dev)
    max_len = int(w.seq_lens.max())
    # the library chooses the split (the partitioned kernel with the
    # workload's own segment length is a parity case: --partition-size 512)
    ps = args.partition_size
    workspace = pkv.DecodeWorkspace(device=dev)
    stream = torch.cuda.current_stream()

    # every physical block of these workloads belongs to one sequence (the
    # tables are slices of one permutation), which the call may declare
    no_shared = not args.plain_loads
    assert len(np.unique(np.concatenate([w.block_tables[b, :-(-int(t) // bs)]
                                         for b, t in enumerate(w.seq_lens)]))) == \
        int(sum(-(-int(t) // bs) for t in w.seq_lens)), "a block is shared"
    kw = dict(max_seq_len=max_len, partition_size=ps, waves_per_group=args.waves,
              kernel=args.kernel, stream_waves=args.stream_waves, workspace=workspace,
              no_shared_blocks=no_shared)

    def step(i, ev=None):
        kc, vc = caches[i % copies]
        if args.unfused:
            pkv.reshape_and_cache(k_new, v_new, slots_new, kc, vc)
            if ev is not None:
                ev[0].record(stream)
            pkv.paged_attention_decode(q, kc, vc, bt, lens, bs, w.scale, out, **kw)
        else:
            if ev is not None:
                ev[0].record(stream)
            pkv.paged_attention_decode_append(q, k_new, v_new, kc, vc, bt, lens, bs, w.scale, out,
                                              **kw)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    # Each timed region: K steps back to back between one pair of events on
    # the stream the kernels run on, synchronised on both sides; the stream
    # is held by a short GPU sleep before the start event, so the host has
    # the first steps enqueued when the region opens.  The value is the
    # median over the trials.
    trial_ms = []
    nxt = args.warmup
    for _ in range(max(args.trials, 1)):
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        prime(stream)
        t_start.record(stream)
        for i in range(args.steps):
            step(nxt + i)
        t_end.record(stream)
        torch.cuda.synchronize()
        nxt += args.steps
        trial_ms.append(t_start.elapsed_time(t_end) / args.steps)
    ms_step = float(np.median(trial_ms))
    if args.unfused:
        # the decode launch on its own: one event pair around each launch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            step(nxt + i, evs[i])
        torch.cuda.synchronize()
        decode_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    else:
        decode_ms = ms_step  # the step is the one launch
    log(f"step {ms_step * 1e3:.2f} us (median of {len(trial_ms)} trials: "
        f"{', '.join(f'{t * 1e3:.2f}' for t in trial_ms)}), decode launch {decode_ms * 1e3:.2f} us")

    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = kv_bytes / (decode_ms * 1e-3) / 1e9
    kernel_name = pkv.decode_plan_kernel(q, caches[0][0], bt, **{
        k: v for k, v in kw.items() if k not in ("workspace",)})
    traffic = measured_traffic(w.name, kernel_name + ("" if args.unfused else "+append"))
    result = {
        "metric": "effective KV read GB/s (% of MI355X HBM peak) in paged decode attention",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": s, "num_q_heads": hq, "num_kv_heads": hkv,
            "head_dim": d, "block_size": bs, "total_tokens": w.total_tokens,
            "kv_bytes_per_step": kv_bytes, "cache_copies_rotated": copies,
            "partition_size": ps or "library", "kernel": kernel_name,
            "no_shared_blocks": no_shared,
            "step_launches": ("reshape_and_cache + paged_attention_decode" if args.unfused
                              else "paged_attention_decode_append (write + attention fused)"),
            "hbm_peak_frac_of_step": round(value / HBM_PEAK_GBS, 4),
            "tokens_per_s_per_layer_step": round(s / (ms_step * 1e-3), 1),
            # the step's other algorithmic bytes besides the K/V (the counters'
            # measured total is roofline.traffic): queries, outputs, the table
            # entries read, sequence lengths and the new tokens' rows written
            "other_bytes_per_step": {
                "q": s * hq * d * 2, "out_bf16": s * hq * d * 2,
                "table_entries": int(sum(-(-int(t) // bs) for t in w.seq_lens)) * 4,
                "seq_lens": s * 4,
                "new_token_rows_written": 0 if args.unfused else s * hkv * d * 2 * 2},
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": (f"paged_attention_decode ({kernel_name} kernel, one launch)" if args.unfused
                       else f"paged_attention_decode_append ({kernel_name} kernel, one launch)"),
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(decode_ms * 1e3, 3),
        },
    }
    result["device"] = {"name": torch.cuda.get_device_name(0),
                        "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                        "hip": torch.version.hip, "torch": torch.__version__}
    result["trials"] = {"ms_per_step": [round(t, 5) for t in trial_ms],
                        "median": round(ms_step, 5), "min": round(min(trial_ms), 5),
                        "max": round(max(trial_ms), 5)}
    if not args.no_read_ceiling:
        del caches
        torch.cuda.empty_cache()
        result["read_ceiling"] = read_ceiling(pkv, torch, dev, stream, kv_bytes, args.steps)
        log(f"read ceiling {result['read_ceiling']['value']} GB/s")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
