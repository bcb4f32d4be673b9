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
                  for f in ("chunk.h", "decode.hip", "decode_wg.hip")]
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
    """HBM bytes per decode launch from the committed counter record, if it
    was taken on this workload and kernel with the current decode source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("kernel") != kernel:
        return None
    if rec.get("decode_source_sha256") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


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


def cpu_baseline(w, budget_s: float = 12.0) -> dict:
    """The oracle as it stands (fp64 C, OpenMP over (sequence, KV head)) on
    the host cores, over repetitions of the whole step until ~budget_s."""
    import oracle

    threads = oracle.max_threads()
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 5000:
        t0 = time.perf_counter()
        oracle.dense_decode(w.q, w.k_tok, w.v_tok, w.seq_lens, w.scale, num_threads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
    per = t_total / reps
    return {"value": round(w.kv_bytes() / per / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole {w.name} step ({w.total_tokens} tokens x {w.num_kv_heads} KV heads)"
                      f" repeated {reps}x, {per * 1e3:.1f} ms each, fp64 gather + dense attention"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama_b64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: >1 GiB)")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "stream_wg", "stream", "mfma", "generic"])
    ap.add_argument("--stream-waves", type=int, default=0)
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
    ps = args.partition_size or w.partition_size
    workspace = pkv.DecodeWorkspace(device=dev)
    stream = torch.cuda.current_stream()

    kw = dict(max_seq_len=max_len, partition_size=ps, waves_per_group=args.waves,
              kernel=args.kernel, stream_waves=args.stream_waves, workspace=workspace)

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

    # The timed region: K steps back to back between one pair of events on the
    # stream the kernels run on.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    if args.unfused:
        # the decode launch on its own: one event pair around each launch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            step(args.warmup + args.steps + i, evs[i])
        torch.cuda.synchronize()
        decode_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    else:
        decode_ms = ms_step  # the step is the one launch
    log(f"step {ms_step * 1e3:.2f} us, decode launch {decode_ms * 1e3:.2f} us")

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
            "step_launches": ("reshape_and_cache + paged_attention_decode" if args.unfused
                              else "paged_attention_decode_append (write + attention fused)"),
            "hbm_peak_frac_of_step": round(value / HBM_PEAK_GBS, 4),
            "tokens_per_s_per_layer_step": round(s / (ms_step * 1e-3), 1),
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
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
