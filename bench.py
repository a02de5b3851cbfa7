"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: compute the slots of this step's
new tokens, scatter their K/V rows into the paged cache and run decode
attention over every sequence, in one pa_decode_append call (the balanced
stream kernel, which reads each newest token from its input row and writes it
to its slot, and the log-sum-exp merge of the sequences it splits).  The K
timed steps run with nothing else on the stream; K more steps with HIP events
around each call give the kernel's own rate, and K steps of the two-call form
(pa_slot_mapping_and_cache, then pa_decode; --step two-call to time it as the
step) are reported beside it.  Inputs are synthetic, seeded, and resident in
HBM before timing starts; the earlier context of every sequence is written
before timing.

Headline workload: Llama-3-8B decode layer, batch 64 with every context at 8192
tokens, bf16 (32 query heads, 8 KV heads, head_dim 128, 16-token blocks).
Prints one JSON line.  The same run also times, under "workloads": batch 64
with contexts uniform in [1024, 8192]; batch 16 at 32768; 256 sequences of
log-normal length with 64 query heads; the chunked-prefill mix (4 x 512-row
chunks + 96 decodes: the unified call, then the chunks against the bf16 matrix
peak and the decodes against HBM); and the headline batch over fp8 caches
(E4M3 and E5M2).  The CPU baseline runs the oracle over the whole headline workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kv-cache bf16|fp8|e5m2]
                  [--step append|two-call] [--no-cpu-baseline] [--no-probes] [--no-extra]

With --workload chunked_prefill_mix the headline step is the scatter plus one
pa_chunked_prefill call over 4 prefill chunks and 96 decodes.  With --kv-cache
fp8 the caches hold E4M3 codes (--kv-cache e5m2: E5M2 codes): the step is one
pa_decode_append_fp8 call (--step two-call: pa_slot_mapping_and_cache_fp8,
then pa_decode_fp8), and KV bytes count one byte per element.
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
# Sources that define the decode kernels and their launch (grid, shares,
# partition choice); the HBM traffic recorded under profiles/ is reported only
# while they hash to the value recorded with it.
DECODE_SOURCES = ["paged_kv_cache_432_amd/csrc/decode_kernel.hip", "paged_kv_cache_432_amd/csrc/device_common.h",
                  "paged_kv_cache_432_amd/csrc/launch.h", "paged_kv_cache_432_amd/csrc/abi.cpp"]
# HBM traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE of the decode call),
# one file per workload.
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "decode_*_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="llama8b_decode_8k",
                   choices=["llama8b_decode", "llama8b_decode_8k", "long_context", "continuous_batching",
                            "chunked_prefill_mix"])
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--kv-cache", default="bf16", choices=["bf16", "fp8", "e5m2"],
                   help="fp8: the caches hold E4M3 codes (pa_decode_append_fp8, or pa_slot_mapping_and_cache_fp8 "
                        "/ pa_decode_fp8); e5m2: E5M2 codes through the same calls' format argument")
    p.add_argument("--step", default="append", choices=["append", "two-call"],
                   help="append: the step is one pa_decode_append (fp8: pa_decode_append_fp8) call, stream mode; "
                        "two-call: pa_slot_mapping_and_cache(_fp8), then pa_decode(_fp8)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probes", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="time only the headline workload (not the other configurations and the fp8 caches)")
    return p.parse_args()


def decode_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_records() -> list:
    """Every HBM traffic record under profiles/, as (path, record)."""
    import glob
    out = []
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        try:
            with open(path) as f:
                out.append((path, json.load(f)))
        except (OSError, ValueError):
            continue
    return out


def recorded_traffic(workload: str, call: str):
    """HBM bytes per decode call from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes recorded under profiles/ for this workload and entry point (already
    scaled by the copy-kernel factors), or None if there is none or it was
    taken on other kernel or launch sources."""
    sha = decode_sources_sha256()
    for _, rec in traffic_records():
        if (rec.get("source_sha256") == sha and rec.get("workload") == workload
                and rec.get("call", "pa_decode") == call):
            return rec.get("hbm_bytes_per_call")
    return None


def probes(pa, torch, nbytes: int = 4 << 30, iters: int = 10):
    """The library's streaming read probe (all of a 4 GiB buffer; the best of
    16384, 32768 and 65536 workgroups, the grid that reads fastest differing
    from GPU to GPU) and copy probe (1 GiB each way) on the same GPU: the
    achievable HBM rates the decode kernel is set against.  The copy is also
    the transfer of known size that the traffic counters are scaled by."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    gib = 1 << 30
    out = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    grids = {g: timed(lambda: pa.pa_probe_stream_read(buf, sink, g)) for g in (16384, 32768, 65536)}
    g_best = min(grids, key=grids.get)
    us = grids[g_best]
    out["stream_read"] = {"GBps": round(nbytes / us / 1e3, 1), "us": round(us, 1), "bytes": nbytes,
                          "workgroups": g_best,
                          "GBps_by_workgroups": {str(g): round(nbytes / t / 1e3, 1) for g, t in grids.items()}}
    us = timed(lambda: pa.pa_probe_copy(buf[gib:2 * gib], buf[:gib], 8192))
    out["copy"] = {"GBps": round(2 * gib / us / 1e3, 1), "us": round(us, 1), "bytes": 2 * gib}
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


def cpu_info() -> dict:
    """The host the CPU baseline ran on: the CPU model (/proc/cpuinfo), the CPUs
    this process may run on (sched_getaffinity) and the OpenMP share of the job
    (OMP_NUM_THREADS), if set."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    env = os.environ.get("OMP_NUM_THREADS")
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "omp_num_threads_env": int(env) if env and env.isdigit() else None}


def cpu_baseline(w, fp8=None, one_thread_seqs: int = 4):
    """The oracle, untuned, on the host cores, over the WHOLE workload of the
    headline line: one step (slots and scatter of the step's new tokens, then
    attention over every sequence; over fp8 codes when fp8 names a format), its caches
    holding every sequence's earlier context (built before timing).  It runs
    with OpenMP over (query row, head) on the job's CPU share: every CPU the
    process may run on, capped by OMP_NUM_THREADS where the job sets it.  A
    per-core figure times the attention of the first few sequences on one
    thread."""
    import oracle
    import workloads as W
    info = cpu_info()
    threads = info["affinity_cores"]
    if info["omp_num_threads_env"]:
        threads = min(threads, info["omp_num_threads_env"])
    oracle.set_threads(threads)
    t_setup = time.perf_counter()
    ks, vs = w.fp8_scales()
    kc, vc = oracle.build_cache_fp8(w, ks, vs, "history", fp8) if fp8 else oracle.build_cache(w, "history")
    seq, pos = w.tokens("new")
    k_new, v_new = (w.encode(x) for x in w.token_kv(seq, pos))
    q = w.encode(w.queries())
    setup_s = time.perf_counter() - t_setup
    sc = dict(k_scale=ks, v_scale=vs, fp8_format=fp8) if fp8 else {}
    times = []
    for _ in range(3):                               # median of three runs of the step
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(w.block_table, seq, pos)
        if fp8:
            oracle.reshape_and_cache_fp8(k_new, v_new, kc, vc, slots, ks, vs, fp8_format=fp8)
        else:
            oracle.reshape_and_cache(k_new, v_new, kc, vc, slots)
        oracle.attention(q, kc, vc, w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads, w.scale,
                         w.causal, **sc)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    kvb = w.kv_bytes(1 if fp8 else None)
    # one thread, on the first few sequences: a per-core figure
    one = W._subset(w, np.arange(min(one_thread_seqs, w.num_seqs)), "cpu_sample_1t")
    kv1 = one.kv_bytes(1 if fp8 else None)
    q1 = one.encode(one.queries())
    oracle.set_threads(1)
    t1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.attention(q1, kc, vc, one.block_table, one.cu_query_lens, one.seq_lens, one.num_heads,
                         one.scale, one.causal, **sc)
        t1.append(time.perf_counter() - t0)
    oracle.set_threads(threads)
    dt1 = float(np.median(t1))
    del kc, vc
    return {
        "value": round(kvb / dt / 1e9, 4),
        "unit": "GB/s",
        "seq_steps_per_s": round(w.num_seqs / dt, 3),
        "seconds": round(dt, 3),
        "cores": int(oracle.max_threads()),
        "kind": "oracle",
        "cpu_model": info["cpu_model"],
        "affinity_cores": info["affinity_cores"],
        "omp_num_threads_env": info["omp_num_threads_env"],
        "setup_seconds": round(setup_s, 2),
        "per_core": {"GBps": round(kv1 / dt1 / 1e9, 4), "seconds": round(dt1, 4),
                     "sample": f"attention only, first {one.num_seqs} sequences ({int(one.seq_lens.sum())} KV "
                               f"tokens), one thread, median of 3"},
        "sample": f"the whole workload: all {w.num_seqs} sequences ({int(w.seq_lens.sum())} KV tokens, "
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


def measure_mixed(w, steps: int, warmup: int, torch, pa, W, DeviceWorkload, mfma: bool = True) -> dict:
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    del dw, out, ws
    torch.cuda.empty_cache()

    pre, dec = W.prefill_part(w), W.decode_part(w)
    dpre = DeviceWorkload(pre)
    dpre.scatter_new(stream)
    opre, wspre = torch.empty_like(dpre.query), dpre.prefill_workspace()
    pre_ms = event_timed(torch, lambda: dpre.chunked_prefill(opre, wspre, stream), steps, warmup, stream)
    del dpre, opre, wspre
    torch.cuda.empty_cache()
    ddec = DeviceWorkload(dec)
    ddec.scatter_new(stream)
    odec, wsdec = torch.empty_like(ddec.query), ddec.decode_workspace(0)
    dec_ms = event_timed(torch, lambda: ddec.decode(odec, 0, wsdec, stream), steps, warmup, stream)
    del ddec, odec, wsdec
    torch.cuda.empty_cache()

    kv = w.kv_bytes()
    flops = causal_flops(pre)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    mprobe = mfma_probe(pa, torch) if mfma else None
    r = {
        "workload": w.name, "kv_bytes_per_step": kv, "ms_per_step": round(ms_step, 5),
        "GBps": round(kv / (ms_step * 1e-3) / 1e9, 2),
        "step": "pa_slot_mapping_and_cache (2144 rows) + pa_chunked_prefill (chunks and decodes, one call)",
        "unified_call_us": round(call_ms * 1e3, 2),
        "chunks": {
            "kernel": "pa_chunked_prefill over the chunks: prefill_kernel + prefill_merge_kernel",
            "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
            "avg_launch_us": round(pre_ms * 1e3, 2), "algorithmic_flops_per_launch": flops,
        },
        "decodes": {
            "kernel": "pa_decode over the single-row requests",
            "bound": "hbm", "avg_launch_us": round(dec_ms * 1e3, 2),
            "GBps": round(dec.kv_bytes() / (dec_ms * 1e-3) / 1e9, 2),
            "frac": round(dec.kv_bytes() / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": dec.kv_bytes(),
        },
        "config": {
            "workload": w.name, "batch": w.num_seqs, "query_rows": int(w.num_q_tokens),
            "chunks": int(np.sum(w.query_lens > 1)), "decodes": int(np.sum(w.query_lens == 1)),
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "pool_blocks": w.num_blocks, "kv_bytes_per_step": kv,
        },
    }
    if mprobe:
        r["probes"] = {"mfma_32x32x16_bf16": mprobe}
        r["chunks"]["frac_of_mfma_probe"] = round(tflops / mprobe["TFLOPs"], 4)
    return r


def measure_decode(w, steps: int, warmup: int, torch, pa, DeviceWorkload, fp8=None,
                   step_kind: str = "append", partition_tokens: int = 0) -> dict:
    """One decode workload: K timed steps with nothing else on the stream (the
    step: pa_decode_append, or the two-call form / fp8 step), then K more with
    HIP events around each attention call (the kernel's own rate), then K
    steps of the two-call form for comparison when the step is the one call.
    fp8: None (a bf16 cache) or the fp8 format of the cache, "e4m3" / "e5m2"."""
    dw = DeviceWorkload(w, kv_fp8=bool(fp8), fp8_format=fp8 or "e4m3")
    pt = pa.pa_decode_partition_tokens(w.num_seqs, w.num_kv_heads, w.max_seq_len, partition_tokens)
    ws = dw.decode_workspace(partition_tokens)
    out = torch.empty_like(dw.query)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    append = step_kind == "append" and pt == 0

    def two_call_step(ev=None):
        # slots and scatter of the step's tokens (one launch), then decode
        dw.scatter_new(stream, fused=True)
        if ev is not None:
            ev[0].record(stream)
        dw.decode(out, partition_tokens, ws, stream)
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
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the K timed steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # then K more steps with HIP events around each attention call, for the
    # kernel's own rate (the events' stream gaps stay out of the step time)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in events])
    two_call_ms = None
    if append:
        # the same step as two calls, for comparison (same values rewritten)
        for _ in range(warmup):
            two_call_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            two_call_step()
        torch.cuda.synchronize()
        two_call_ms = (time.perf_counter() - t0) * 1e3 / steps
    del dw, ws, out
    torch.cuda.empty_cache()
    kv = w.kv_bytes(1 if fp8 else None)
    gbps = kv / (ms_step * 1e-3) / 1e9
    call_gbps = kv / (float(call_ms.mean()) * 1e-3) / 1e9
    r = {
        "workload": w.name,
        "kv_bytes_per_step": kv,
        "ms_per_step": round(ms_step, 5),
        "GBps": round(gbps, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "append": append,
        "partition_tokens": pt,
        "step": (f"pa_decode_append_fp8 ({fp8}): slots, quantising scatter and decode in one call" if fp8
                 else "pa_decode_append (slots, scatter and decode in one call)") if append
                else ((f"pa_slot_mapping_and_cache_fp8 + pa_decode_fp8 ({fp8})") if fp8
                      else "pa_slot_mapping_and_cache + pa_decode"),
        "kernel": (f"pa_decode_append_fp8 ({fp8}): decode_stream_kernel<fp8, append> + merge_stream_kernel "
                   "(one call)" if append else
                   f"pa_decode_fp8 ({fp8}): decode_stream_kernel<fp8> + merge_stream_kernel (one call)") if fp8
                  else "pa_decode_append: decode_stream_kernel<append> + merge_stream_kernel (one call)" if append
                  else "pa_decode: decode_stream_kernel + merge_stream_kernel (one call)" if pt == 0
                  else "pa_decode: decode_partition_kernel + merge_partitions_kernel (one call)",
        "call": ("pa_decode_append_fp8" if fp8 else "pa_decode_append") if append
                else ("pa_decode_fp8" if fp8 else "pa_decode"),
        "call_us_mean": round(float(call_ms.mean()) * 1e3, 2),
        "call_us_median_p10_p90": [round(float(np.percentile(call_ms, q)) * 1e3, 2) for q in (50, 10, 90)],
        "call_GBps": round(call_gbps, 2),
        "call_frac": round(call_gbps / HBM_PEAK_GBPS, 4),
    }
    if two_call_ms is not None:
        r["two_call_step"] = {"what": ("pa_slot_mapping_and_cache_fp8 + pa_decode_fp8" if fp8
                                       else "pa_slot_mapping_and_cache + pa_decode") +
                                      ", same inputs, after the timed steps",
                              "ms_per_step": round(two_call_ms, 5),
                              "GBps": round(kv / (two_call_ms * 1e-3) / 1e9, 2)}
    return r


def _brief(r: dict) -> dict:
    """The figures of an extra workload that go into the JSON line."""
    keys = ("workload", "step", "ms_per_step", "GBps", "pct_hbm_peak", "seq_steps_per_s", "call_us_mean",
            "call_GBps", "call_frac", "kv_bytes_per_step", "two_call_step", "unified_call_us", "chunks", "decodes")
    return {k: r[k] for k in keys if k in r}


# The workloads timed in the same run as the headline (bench.py --no-extra
# skips them): the other decode configurations, the chunked-prefill mix, and
# the headline workload over an fp8 cache.
EXTRA_DECODE = ["llama8b_decode", "long_context", "continuous_batching"]


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
    fp8 = {"bf16": None, "fp8": "e4m3", "e5m2": "e5m2"}[args.kv_cache]
    if fp8 and args.partition_tokens != 0:
        print("an fp8 cache is read in the stream mode only (--partition-tokens 0)", file=sys.stderr)
        sys.exit(2)
    t_setup = time.perf_counter()
    print(f"# {w.name}: {w.num_seqs} seqs, {w.kv_bytes() / 1e9:.3f} GB KV", file=sys.stderr, flush=True)
    common = {
        "metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "data": "synthetic (seeded N(0,1)*sigma values, random block placement; no dataset)",
    }
    if not w.is_decode:
        r = measure_mixed(w, args.steps, args.warmup, torch, pa, W, DeviceWorkload, mfma=not args.no_probes)
        res = dict(common, value=r["GBps"], ms_per_step=r["ms_per_step"], dtype=w.dtype, config=r["config"],
                   unified_call_us=r["unified_call_us"], roofline=r["chunks"], decode_part=r["decodes"])
        if "probes" in r:
            res["probes"] = r["probes"]
        res["device"] = device_info(torch)
        print(json.dumps(res), flush=True)
        return

    r = measure_decode(w, args.steps, args.warmup, torch, pa, DeviceWorkload, fp8, args.step, args.partition_tokens)
    print(f"# {w.name}: {r['ms_per_step'] * 1e3:.1f} us/step ({time.perf_counter() - t_setup:.1f}s)",
          file=sys.stderr, flush=True)
    traffic = None if fp8 else recorded_traffic(w.name, r["call"])
    res = dict(common)
    res.update({
        "value": r["GBps"],
        "ms_per_step": r["ms_per_step"],
        "dtype": f"fp8_{fp8} KV, bf16 Q/out" if fp8 else w.dtype,
        "config": {
            "workload": w.name,
            "batch": w.num_seqs,
            "context_lens": f"min {int(w.seq_lens.min())} mean {float(w.seq_lens.mean()):.1f} "
                            f"max {int(w.seq_lens.max())}",
            "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "pool_blocks": w.num_blocks,
            "new_tokens_per_step": int(w.num_q_tokens),
            "decode_split": "balanced stream (equal block shares per workgroup)" if r["partition_tokens"] == 0
                            else f"partitions of {r['partition_tokens']} tokens",
            "kv_bytes_per_step": r["kv_bytes_per_step"],
            "kv_cache": "fp8 %s (1 byte/element), k_scale = v_scale = %.6g" % (fp8.upper(), w.fp8_scales()[0])
                        if fp8 else w.dtype,
            "step": r["step"],
        },
        "pct_hbm_peak": r["pct_hbm_peak"],
        "seq_steps_per_s": r["seq_steps_per_s"],
        "roofline": {
            "kernel": r["kernel"],
            "bound": "hbm",
            "achieved": r["call_GBps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": r["call_frac"],
            "traffic": traffic,
            "avg_launch_us": r["call_us_mean"],
            "launch_us_median_p10_p90": r["call_us_median_p10_p90"],
            "algorithmic_bytes_per_launch": r["kv_bytes_per_step"],
        },
    })
    if "two_call_step" in r:
        res["two_call_step"] = r["two_call_step"]
    if not args.no_extra:
        extra_steps, extra_warmup = min(args.steps, 200), min(args.warmup, 20)
        extra = {}
        for name in EXTRA_DECODE:
            if name == args.workload:
                continue
            wx = W.CONFIGS[name]()
            extra[wx.name] = _brief(measure_decode(wx, extra_steps, extra_warmup, torch, pa, DeviceWorkload))
            print(f"# {wx.name}: {extra[wx.name]['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        wm = W.chunked_prefill_mix()
        extra[wm.name] = _brief(measure_mixed(wm, extra_steps, extra_warmup, torch, pa, W, DeviceWorkload,
                                              mfma=False))
        print(f"# {wm.name}: {extra[wm.name]['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        for fmt in ("e4m3", "e5m2"):
            if fmt == fp8:
                continue
            f = _brief(measure_decode(w, extra_steps, extra_warmup, torch, pa, DeviceWorkload, fp8=fmt))
            f["kv_cache"] = "fp8 %s (1 byte/element), k_scale = v_scale = %.6g" % (fmt.upper(), w.fp8_scales()[0])
            extra[w.name + ":" + fmt] = f
            print(f"# {w.name} {fmt}: {f['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
        res["workloads"] = extra
    if not args.no_probes:
        probe = probes(pa, torch)
        res["probes"] = probe
        res["roofline"]["frac_of_read_probe"] = round(r["call_GBps"] / probe["stream_read"]["GBps"], 4)
        res["rope_reshape_and_cache"] = rope_scatter_timing(pa, torch)
        res["copy_blocks"] = copy_blocks_timing(pa, torch)
        res["kv_manager"] = kv_manager_timing(pa)
    res["device"] = device_info(torch)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, fp8)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
