"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: compute the slots of this step's
new tokens (pa_slot_mapping), scatter their K/V rows into the paged cache
(pa_reshape_and_cache), and run decode attention over every sequence's cache
(pa_decode: the partitioned kernel and, when sequences are split, the
log-sum-exp merge).  Inputs are synthetic, seeded, and resident in HBM before
timing starts; the earlier context of every sequence is written before timing.

Default workload: Llama-3-8B decode layer, batch 64, context lengths uniform
in [1024, 8192], bf16 (32 query heads, 8 KV heads, head_dim 128, 16-token
blocks).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + seq-steps/s, 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
# Sources that define the decode kernels; the HBM traffic recorded under
# profiles/ is reported only while they hash to the value recorded with it.
DECODE_SOURCES = ["paged_kv_cache_432_amd/csrc/decode_kernel.hip", "paged_kv_cache_432_amd/csrc/device_common.h",
                  "paged_kv_cache_432_amd/csrc/launch.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama8b_b64_1k-8k_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="llama8b_decode",
                   choices=["llama8b_decode", "llama8b_decode_8k", "long_context", "continuous_batching"])
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probes", action="store_true")
    p.add_argument("--cpu-sample-seqs", type=int, default=16)
    return p.parse_args()


def decode_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per pa_decode call from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes recorded under profiles/ (already scaled by the copy-kernel
    factors), or None if they were taken on other kernel sources or another
    workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != decode_sources_sha256() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_call")


def probes(pa, torch, nbytes: int = 2 << 30, iters: int = 10):
    """The library's streaming read and copy probes on the same GPU: the
    achievable HBM rate the decode kernel is set against."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for name, fn, moved in (("stream_read", lambda: pa.pa_probe_stream_read(buf, sink, 16384), nbytes),
                            ("copy", lambda: pa.pa_probe_copy(buf[nbytes // 2:], buf[:nbytes // 2], 8192), nbytes)):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        out[name] = {"GBps": round(moved / us / 1e3, 1), "us": round(us, 1), "bytes": moved}
    del buf
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, nseq: int):
    """The oracle, untuned, on the host cores: the first `nseq` sequences of the
    workload (their K/V gathered through block tables into a compact pool built
    before timing), timed over the same step: slots and scatter of their new
    tokens, then attention."""
    import oracle
    import workloads as W
    idx = np.arange(min(nseq, w.num_seqs))
    sub = W._subset(w, idx, "cpu_sample")
    counts = W.blocks_needed(sub.seq_lens)
    table = np.full((len(idx), int(counts.max())), -1, np.int32)
    cursor = 0
    for i, c in enumerate(counts):
        table[i, :c] = np.arange(cursor, cursor + c)
        cursor += c
    sub = sub.with_block_table(table, num_blocks=int(cursor))
    kc, vc = oracle.build_cache(sub, "history")
    seq, pos = sub.tokens("new")
    k_new, v_new = (sub.encode(x) for x in sub.token_kv(seq, pos))
    q = sub.encode(sub.queries())
    oracle.lib()
    times = []
    for _ in range(3):                               # median of three runs of the step
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(sub.block_table, seq, pos)
        oracle.reshape_and_cache(k_new, v_new, kc, vc, slots)
        oracle.attention(q, kc, vc, sub.block_table, sub.cu_query_lens, sub.seq_lens, sub.num_heads,
                         sub.scale, sub.causal)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {
        "value": round(sub.kv_bytes() / dt / 1e9, 4),
        "unit": "GB/s",
        "seq_steps_per_s": round(len(idx) / dt, 3),
        "seconds": round(dt, 3),
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"first {len(idx)} of {w.num_seqs} sequences ({int(sub.seq_lens.sum())} KV tokens, "
                  f"{sub.kv_bytes() / 1e9:.3f} GB of KV), one step (slots + scatter + attention), fp64, median of 3",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(each GPU would run its own shard of sequences or KV heads).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import paged_kv_cache_432_amd as pa
    from paged_kv_cache_432_amd.staging import DeviceWorkload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pa.lib()
    w = W.CONFIGS[args.workload]()
    t_setup = time.perf_counter()
    dw = DeviceWorkload(w)
    pt = pa.pa_decode_partition_tokens(w.num_seqs, w.num_kv_heads, w.max_seq_len, args.partition_tokens)
    ws = dw.decode_workspace(args.partition_tokens)
    out = torch.empty_like(dw.query)
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s: {w.name}, {w.num_seqs} seqs, "
          f"{w.kv_bytes() / 1e9:.3f} GB KV, partition {pt} tokens (0: balanced stream)",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()

    def step(ev=None):
        dw.scatter_new(stream)
        if ev is not None:
            ev[0].record(stream)
        dw.decode(out, args.partition_tokens, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    dec_ms = np.array([a.elapsed_time(b) for a, b in events])
    dec_avg_ms = float(dec_ms.mean())

    kv = w.kv_bytes()
    gbps = kv / (ms_step * 1e-3) / 1e9
    dec_gbps = kv / (dec_avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic(w.name)
    probe = None if args.no_probes else probes(pa, torch)
    res = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)*sigma values, random block placement; no dataset)",
        "config": {
            "workload": w.name,
            "batch": w.num_seqs,
            "context_lens": f"min {int(w.seq_lens.min())} mean {float(w.seq_lens.mean()):.1f} "
                            f"max {int(w.seq_lens.max())}",
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "pool_blocks": w.num_blocks,
            "new_tokens_per_step": int(w.num_q_tokens),
            "decode_split": "balanced stream (equal block shares per workgroup)" if pt == 0
                            else f"partitions of {pt} tokens",
            "kv_bytes_per_step": kv,
        },
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": "pa_decode: decode_stream_kernel + merge_stream_kernel (one call)" if pt == 0
                      else "pa_decode: decode_partition_kernel + merge_partitions_kernel (one call)",
            "bound": "hbm",
            "achieved": round(dec_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(dec_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": kv,
        },
    }
    if probe is not None:
        res["probes"] = probe
        res["roofline"]["frac_of_read_probe"] = round(dec_gbps / probe["stream_read"]["GBps"], 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_seqs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
