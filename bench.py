"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: compute the slots of this step's
new tokens, scatter their K/V rows into the paged cache and run decode
attention over every sequence, in one pa_decode_append call (the balanced
stream kernel, which reads each newest token from its input row and writes it
to its slot, and the log-sum-exp merge of the sequences it splits).  The K
timed steps run with nothing else on the stream; K more steps with HIP events
around each call give the kernel's own rate, and K steps of the two-call form
(pa_slot_mapping_and_cache, then pa_decode; --step two-call to time it as the
step) are reported beside it.  Inputs are synthetic, seeded, and resident in HBM before
timing starts; the earlier context of every sequence is written before timing.

Default workload: Llama-3-8B decode layer, batch 64, context lengths uniform
in [1024, 8192], bf16 (32 query heads, 8 KV heads, head_dim 128, 16-token
blocks).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kv-cache bf16|fp8]
                  [--step append|two-call] [--no-cpu-baseline] [--no-probes]

With --workload chunked_prefill_mix a step is the scatter plus one
pa_chunked_prefill call over 4 prefill chunks and 96 decodes; the chunks are
also reported against the bf16 matrix peak.

With --kv-cache fp8 the caches hold E4M3 codes: the step is
pa_slot_mapping_and_cache_fp8 (slots and quantising scatter in one launch) and
pa_decode_fp8, and KV bytes count one byte per element.
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
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
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
                   choices=["llama8b_decode", "llama8b_decode_8k", "long_context", "continuous_batching",
                            "chunked_prefill_mix"])
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--kv-cache", default="bf16", choices=["bf16", "fp8"],
                   help="fp8: the caches hold E4M3 codes (pa_reshape_and_cache_fp8 / pa_decode_fp8)")
    p.add_argument("--step", default="append", choices=["append", "two-call"],
                   help="append: the step is one pa_decode_append call (bf16/fp32 caches, stream mode); "
                        "two-call: pa_slot_mapping_and_cache, then pa_decode")
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


def recorded_traffic(workload: str, call: str):
    """HBM bytes per decode call from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes recorded under profiles/ (already scaled by the copy-kernel
    factors), or None if they were taken on other kernel sources, another
    workload or another entry point."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("source_sha256") != decode_sources_sha256() or rec.get("workload") != workload
            or rec.get("call", "pa_decode") != call):
        return None
    return rec.get("hbm_bytes_per_call")


def probes(pa, torch, nbytes: int = 4 << 30, iters: int = 10):
    """The library's streaming read probe (all of a 4 GiB buffer, 16384
    workgroups) and copy probe (1 GiB each way) on the same GPU: the achievable
    HBM rates the decode kernel is set against.  The copy is also the transfer
    of known size that the traffic counters are scaled by."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    gib = 1 << 30
    out = {}
    for name, fn, moved in (("stream_read", lambda: pa.pa_probe_stream_read(buf, sink, 16384), nbytes),
                            ("copy", lambda: pa.pa_probe_copy(buf[gib:2 * gib], buf[:gib], 8192), 2 * gib)):
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


def rope_scatter_timing(pa, torch, token_counts=(64, 256, 2144, 16384), iters: int = 20, batch: int = 20):
    """The fused step before attention (pa_rope_reshape_and_cache: QKV split,
    RoPE on Q and K, K/V scatter) on Llama-3-8B shapes (32 Q heads, 8 KV heads,
    6144-column bf16 projection, rope_theta 5e5, rotary_dim 128), one call per
    count of new tokens.  Algorithmic bytes per token: the projection row read
    (12288 B) + Q, K, V written (12288 B) + the table row (512 B) + position
    and slot (16 B).  Each count is timed as a graph of `batch` calls back to
    back (per-call GPU time, free of the host launch path)."""
    hq, hkv, d, rot = 32, 8, 128, 128
    dev = "cuda"
    g = torch.Generator(device="cpu").manual_seed(21)
    max_pos = 8192
    inv = torch.pow(torch.tensor(500000.0, dtype=torch.float64),
                    -2.0 * torch.arange(rot // 2, dtype=torch.float64) / rot)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    table = torch.cat([ang.cos(), ang.sin()], 1).float().to(dev)
    per_token = (hq + 2 * hkv) * d * 2 * 2 + rot * 4 + 16
    rows = []
    for n in token_counts:
        nb = (n * 11 // 10 + 15) // 16 + 1
        qkv = torch.randn(n, (hq + 2 * hkv) * d, generator=g).to(torch.bfloat16).to(dev)
        qout = torch.empty(n, hq, d, dtype=torch.bfloat16, device=dev)
        pos = torch.randint(0, max_pos, (n,), generator=g).to(dev)
        slots = torch.randperm(nb * 16, generator=g)[:n].to(dev)
        kc = torch.zeros(nb, 16, hkv, d, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)

        def call():
            pa.pa_rope_reshape_and_cache(qout, qkv, pos, table, kc, vc, slots, hq, hkv)

        for _ in range(5):
            call()
        torch.cuda.synchronize()
        # a few small calls take less GPU time than their host launch path, so
        # the calls are captured back to back in a graph and its replay timed
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(batch):
                    call()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 / batch
        gbps = n * per_token / us / 1e3
        rows.append({"tokens": n, "us": round(us, 2), "GBps": round(gbps, 1),
                     "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2), "bytes": n * per_token})
        del qkv, qout, kc, vc, graph
    torch.cuda.empty_cache()
    return {"kernel": "rope_cache_kernel (pa_rope_reshape_and_cache)", "shapes": "Llama-3-8B, bf16",
            "bytes_per_token": per_token, "calls": rows}


def copy_blocks_timing(pa, torch, pair_counts=(1, 64, 1024), layers: int = 32, iters: int = 20, batch: int = 10):
    """Copy-on-write (pa_copy_blocks) over a Llama-3-8B cache of all 32 layers
    ([32, 2, 4096 blocks, 16, 8, 128] bf16, 8 GiB): each pair copies one
    32 KiB block of K and one of V in every layer.  Algorithmic bytes per pair:
    layers * 2 * 32 KiB read + as many written.  Timed as a graph of `batch`
    calls back to back."""
    nb, blk = 4096, 16 * 8 * 128
    kv = torch.zeros(layers, 2, nb, blk, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(5)
    rows = []
    for n in pair_counts:
        perm = torch.randperm(nb, generator=g)
        pairs = torch.stack([perm[:n], perm[n:2 * n]], 1).contiguous().to("cuda")

        def call():
            pa.pa_copy_blocks(kv, pairs)

        call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(batch):
                    call()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3 / batch
        moved = n * layers * 2 * blk * 2 * 2
        rows.append({"pairs": n, "us": round(us, 2), "GBps": round(moved / us / 1e3, 1),
                     "pct_hbm_peak": round(100.0 * moved / us / 1e3 / HBM_PEAK_GBPS, 2), "bytes": moved})
        del graph
    del kv
    torch.cuda.empty_cache()
    return {"kernel": "copy_blocks_kernel (pa_copy_blocks)", "shapes": "Llama-3-8B, 32 layers, bf16",
            "calls": rows}


def kv_manager_timing(pa, steps: int = 200):
    """Host cost of the block manager's step (pa_kvm_schedule + pa_kvm_commit,
    through the Python binding) for 256 running decode requests with the
    continuous-batching lengths (log-normal, median 900, clipped to [16,
    16384]); the pool is 110% of the blocks they need.  The prompts are first
    prefilled in chunks of at most 8192 tokens per step."""
    rng = np.random.default_rng(3)
    lens = np.clip(np.round(np.exp(rng.normal(np.log(900), 1.0, 256))), 16, 16384).astype(np.int64)
    need = int(((lens + 200 + 15) // 16).sum())
    m = pa.KvManager(int(need * 1.1), 256, 8192, 16384 + 256, prefix_caching=True)
    for i, n in enumerate(lens):
        m.add_request(i, rng.integers(0, 32000, int(n)))
    prefill_steps = 0
    while True:
        st = m.schedule()
        m.commit(np.full(st["num_seqs"], 11, np.int32))
        prefill_steps += 1
        if st["num_seqs"] == 256 and int(st["query_lens"].max()) == 1:
            break
    nxt = np.full(256, 11, np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        st = m.schedule()
        m.commit(nxt)
    us_py = (time.perf_counter() - t0) / steps * 1e6
    import ctypes
    L, raw = pa.lib(), pa._KvmStep()
    t0 = time.perf_counter()
    for _ in range(steps):
        L.pa_kvm_schedule(m._h, ctypes.byref(raw))
        L.pa_kvm_commit(m._h, nxt.ctypes.data, 256)
    us_c = (time.perf_counter() - t0) / steps * 1e6
    return {"what": "pa_kvm_schedule + pa_kvm_commit per decode step, host CPU", "requests": 256,
            "tokens_per_step": int(st["num_tokens"]), "block_table_width": int(raw.max_blocks_per_req),
            "us_per_step_c_abi": round(us_c, 1), "us_per_step_python_binding": round(us_py, 1),
            "prefill_steps": prefill_steps}


def mfma_probe(pa, torch, iters: int = 10):
    """The library's matrix-core probe (4 independent v_mfma_f32_32x32x16_bf16
    chains per wave, two 4-wave workgroups per compute unit): the matrix rate
    the prefill kernel is set against next to the nominal peak."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    wgs = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    flops = pa.pa_probe_mfma(sink, wgs, 4000)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        pa.pa_probe_mfma(sink, wgs, 4000)
        b.record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    return {"TFLOPs": round(flops / us / 1e6, 1), "us": round(us, 1), "flops": flops, "workgroups": wgs}


def device_info(torch) -> dict:
    """The GPU the figures were measured on: name, architecture, compute units,
    memory, the HIP runtime torch was built with, and the engine and memory
    clock levels the driver lists (read from sysfs; '*' marks the current one
    when the file is readable)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip}
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                sclk = [ln.strip() for ln in fh if ln.strip()]
            with open(f.replace("pp_dpm_sclk", "pp_dpm_mclk")) as fh:
                mclk = [ln.strip() for ln in fh if ln.strip()]
        except OSError:
            continue
        info["sclk_levels"], info["mclk_levels"] = sclk, mclk
        break
    return info


def cpu_baseline(w, nseq: int, fp8: bool = False):
    """The oracle, untuned, on the host cores: the first `nseq` sequences of the
    workload (their K/V gathered through block tables into a compact pool built
    before timing), timed over the same step: slots and scatter of their new
    tokens, then attention (over E4M3 codes when fp8)."""
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
    ks, vs = sub.fp8_scales()
    kc, vc = oracle.build_cache_fp8(sub, ks, vs, "history") if fp8 else oracle.build_cache(sub, "history")
    seq, pos = sub.tokens("new")
    k_new, v_new = (sub.encode(x) for x in sub.token_kv(seq, pos))
    q = sub.encode(sub.queries())
    oracle.lib()
    times = []
    for _ in range(3):                               # median of three runs of the step
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(sub.block_table, seq, pos)
        if fp8:
            oracle.reshape_and_cache_fp8(k_new, v_new, kc, vc, slots, ks, vs)
        else:
            oracle.reshape_and_cache(k_new, v_new, kc, vc, slots)
        oracle.attention(q, kc, vc, sub.block_table, sub.cu_query_lens, sub.seq_lens, sub.num_heads,
                         sub.scale, sub.causal, k_scale=ks if fp8 else 1.0, v_scale=vs if fp8 else 1.0)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    kvb = sub.kv_bytes(1 if fp8 else None)
    # one thread, on the first 4 of those sequences: a per-core figure
    one = W._subset(sub, np.arange(min(4, len(idx))), "cpu_sample_1t")
    kv1 = one.kv_bytes(1 if fp8 else None)
    threads = oracle.max_threads()
    oracle.set_threads(1)
    q1 = one.encode(one.queries())
    t1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.attention(q1, kc, vc, one.block_table, one.cu_query_lens, one.seq_lens, one.num_heads,
                         one.scale, one.causal, k_scale=ks if fp8 else 1.0, v_scale=vs if fp8 else 1.0)
        t1.append(time.perf_counter() - t0)
    oracle.set_threads(threads)
    dt1 = float(np.median(t1))
    return {
        "value": round(kvb / dt / 1e9, 4),
        "unit": "GB/s",
        "seq_steps_per_s": round(len(idx) / dt, 3),
        "seconds": round(dt, 3),
        "cores": threads,
        "kind": "oracle",
        "per_core": {"GBps": round(kv1 / dt1 / 1e9, 4), "seconds": round(dt1, 4),
                     "sample": f"attention only, first {one.num_seqs} sequences ({int(one.seq_lens.sum())} KV "
                               f"tokens), one thread, median of 3"},
        "sample": f"first {len(idx)} of {w.num_seqs} sequences ({int(sub.seq_lens.sum())} KV tokens, "
                  f"{kvb / 1e9:.3f} GB of KV), one step (slots + scatter + attention), fp64, median of 3",
    }


def event_timed(torch, fn, steps: int, warmup: int, stream):
    """Mean HIP-event time (ms) of fn() over `steps` calls on `stream`, after
    `warmup` untimed calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def causal_flops(w) -> int:
    """Algorithmic flops of the multi-row requests: 4 * head_dim per (query,
    key) pair each row attends, per query head (QK^T and PV)."""
    pairs = 0
    for b in range(w.num_seqs):
        q, L = int(w.query_lens[b]), int(w.seq_lens[b])
        if q < 2:
            continue
        pairs += sum(min(L, L - q + j + 1) for j in range(q)) if w.causal else q * L
    return pairs * w.num_heads * w.head_dim * 4


def main_mixed(args, w, torch, pa, W, DeviceWorkload):
    """The chunked-prefill + decode mix: one step is the scatter of every new
    row and one pa_chunked_prefill call over the whole batch.  The chunks and
    the decodes are also timed as the two calls of the split-call mode, the
    chunks against the bf16 matrix peak and the decodes against HBM."""
    stream = torch.cuda.current_stream()
    dw = DeviceWorkload(w)
    out = torch.empty_like(dw.query)
    ws = dw.prefill_workspace()
    torch.cuda.synchronize()

    def step(ev=None):
        dw.scatter_new(stream, fused=True)
        if ev is not None:
            ev[0].record(stream)
        dw.chunked_prefill(out, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    del dw, out, ws
    torch.cuda.empty_cache()

    pre, dec = W.prefill_part(w), W.decode_part(w)
    dpre = DeviceWorkload(pre)
    dpre.scatter_new(stream)
    opre, wspre = torch.empty_like(dpre.query), dpre.prefill_workspace()
    pre_ms = event_timed(torch, lambda: dpre.chunked_prefill(opre, wspre, stream), args.steps, args.warmup, stream)
    del dpre, opre, wspre
    torch.cuda.empty_cache()
    ddec = DeviceWorkload(dec)
    ddec.scatter_new(stream)
    odec, wsdec = torch.empty_like(ddec.query), ddec.decode_workspace(0)
    dec_ms = event_timed(torch, lambda: ddec.decode(odec, 0, wsdec, stream), args.steps, args.warmup, stream)
    del ddec, odec, wsdec
    torch.cuda.empty_cache()

    kv = w.kv_bytes()
    flops = causal_flops(pre)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    mprobe = None if args.no_probes else mfma_probe(pa, torch)
    res = {
        "metric": METRIC,
        "value": round(kv / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) values, random block placement; no dataset)",
        "config": {
            "workload": w.name, "batch": w.num_seqs, "query_rows": int(w.num_q_tokens),
            "chunks": int(np.sum(w.query_lens > 1)), "decodes": int(np.sum(w.query_lens == 1)),
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "pool_blocks": w.num_blocks, "kv_bytes_per_step": kv,
        },
        "unified_call_us": round(call_ms * 1e3, 2),
        "roofline": {
            "kernel": "pa_chunked_prefill over the chunks: prefill_kernel + prefill_merge_kernel",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "avg_launch_us": round(pre_ms * 1e3, 2),
            "algorithmic_flops_per_launch": flops,
        },
        "probes": {"mfma_32x32x16_bf16": mprobe} if mprobe else None,
        "decode_part": {
            "kernel": "pa_decode over the single-row requests",
            "bound": "hbm", "avg_launch_us": round(dec_ms * 1e3, 2),
            "GBps": round(dec.kv_bytes() / (dec_ms * 1e-3) / 1e9, 2),
            "frac": round(dec.kv_bytes() / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": dec.kv_bytes(),
        },
    }
    if mprobe:
        res["roofline"]["frac_of_mfma_probe"] = round(tflops / mprobe["TFLOPs"], 4)
    print(json.dumps(res), flush=True)


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
    if not w.is_decode:
        return main_mixed(args, w, torch, pa, W, DeviceWorkload)
    t_setup = time.perf_counter()
    fp8 = args.kv_cache == "fp8"
    if fp8 and args.partition_tokens != 0:
        print("an fp8 cache is read in the stream mode only (--partition-tokens 0)", file=sys.stderr)
        sys.exit(2)
    dw = DeviceWorkload(w, kv_fp8=fp8)
    pt = pa.pa_decode_partition_tokens(w.num_seqs, w.num_kv_heads, w.max_seq_len, args.partition_tokens)
    ws = dw.decode_workspace(args.partition_tokens)
    out = torch.empty_like(dw.query)
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s: {w.name}, {w.num_seqs} seqs, "
          f"{w.kv_bytes() / 1e9:.3f} GB KV, partition {pt} tokens (0: balanced stream)",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    append = args.step == "append" and not fp8 and pt == 0

    def two_call_step(ev=None):
        # slots and scatter of the step's tokens (one launch), then decode
        dw.scatter_new(stream, fused=True)
        if ev is not None:
            ev[0].record(stream)
        dw.decode(out, args.partition_tokens, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    def append_step(ev=None):
        # the newest tokens written to the cache and attended to, in one call
        if ev is not None:
            ev[0].record(stream)
        dw.decode_append(out, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    step = append_step if append else two_call_step

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the K timed steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    # then K more steps with HIP events around each pa_decode call, for the
    # kernel's own rate (the events' stream gaps stay out of the step time)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in events])
    dec_avg_ms = float(dec_ms.mean())
    two_call_ms = None
    if append:
        # the same step as two calls, for comparison (same values rewritten)
        for _ in range(args.warmup):
            two_call_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            two_call_step()
        torch.cuda.synchronize()
        two_call_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    kv = w.kv_bytes(1 if fp8 else None)
    gbps = kv / (ms_step * 1e-3) / 1e9
    dec_gbps = kv / (dec_avg_ms * 1e-3) / 1e9
    traffic = None if fp8 else recorded_traffic(w.name, "pa_decode_append" if append else "pa_decode")
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
        "dtype": "fp8_e4m3 KV, bf16 Q/out" if fp8 else w.dtype,
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
            "kv_cache": "fp8 E4M3 (1 byte/element), k_scale = v_scale = %.6g" % w.fp8_scales()[0] if fp8
                        else w.dtype,
            "step": "pa_decode_append (slots, scatter and decode in one call)" if append
                    else ("pa_slot_mapping_and_cache_fp8 + pa_decode_fp8" if fp8
                          else "pa_slot_mapping_and_cache + pa_decode"),
        },
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "roofline": {
            "kernel": "pa_decode_fp8: decode_stream_kernel<fp8> + merge_stream_kernel (one call)" if fp8
                      else "pa_decode_append: decode_stream_kernel<append> + merge_stream_kernel (one call)"
                      if append
                      else "pa_decode: decode_stream_kernel + merge_stream_kernel (one call)" if pt == 0
                      else "pa_decode: decode_partition_kernel + merge_partitions_kernel (one call)",
            "bound": "hbm",
            "achieved": round(dec_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(dec_avg_ms * 1e3, 2),
            "launch_us_median_p10_p90": [round(float(np.percentile(dec_ms, q)) * 1e3, 2) for q in (50, 10, 90)],
            "algorithmic_bytes_per_launch": kv,
        },
    }
    if two_call_ms is not None:
        res["two_call_step"] = {"what": "pa_slot_mapping_and_cache + pa_decode, same inputs, after the timed steps",
                                "ms_per_step": round(two_call_ms, 5),
                                "GBps": round(kv / (two_call_ms * 1e-3) / 1e9, 2)}
    if probe is not None:
        res["probes"] = probe
        res["roofline"]["frac_of_read_probe"] = round(dec_gbps / probe["stream_read"]["GBps"], 4)
        res["rope_reshape_and_cache"] = rope_scatter_timing(pa, torch)
        res["copy_blocks"] = copy_blocks_timing(pa, torch)
        res["kv_manager"] = kv_manager_timing(pa)
    res["device"] = device_info(torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_seqs, fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
