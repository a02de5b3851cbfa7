"""Whole-output parity at the workload sizes the benchmark runs.

The oracle's output for a whole workload is computed once per test session
(its caches built by the oracle's own slot function and scatter over the
workload's real block table, then its fp64 attention over that pool) and
shared by every test of that workload.  Device outputs, workspaces and caches
sit between guard zones (staging.Guarded): each check also asserts that no
kernel wrote outside the buffers it was given.
"""
from __future__ import annotations

import time

import numpy as np
import torch

import oracle
from parity import assert_parity, storage_bits, to_numpy

_OUT = {}


def _fmt(fp8):
    """False (a bf16/fp32 cache), True (E4M3) or a format name -> None or the name."""
    if fp8 is False or fp8 is None:
        return None
    return "e4m3" if fp8 is True else fp8


def _key(w, fp8):
    return (w.name, int(w.num_seqs), int(np.asarray(w.seq_lens, np.int64).sum()), _fmt(fp8))


def _attend(w, kc, vc, fmt):
    ks, vs = w.fp8_scales() if fmt else (1.0, 1.0)
    q = w.encode(w.queries())
    return oracle.attention(q, kc, vc, w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads, w.scale,
                            w.causal, k_scale=ks, v_scale=vs, fp8_format=fmt or "e4m3")


def oracle_cache(w, fp8=False):
    """The oracle's caches after every token of the workload (history and this
    step's) is scattered (fp8: False, True for E4M3, or "e4m3" / "e5m2"); the
    output over them is remembered for oracle_output()."""
    fmt = _fmt(fp8)
    t0 = time.perf_counter()
    kc, vc = oracle.build_cache_fp8(w, *w.fp8_scales(), "all", fmt) if fmt else oracle.build_cache(w, "all")
    t1 = time.perf_counter()
    key = _key(w, fp8)
    if key not in _OUT:
        _OUT[key] = _attend(w, kc, vc, fmt)
    print(f"  oracle {w.name}{' ' + fmt if fmt else ''}: cache {t1 - t0:.1f}s, attention "
          f"{time.perf_counter() - t1:.1f}s", flush=True)
    return kc, vc


def oracle_output(w, fp8=False) -> np.ndarray:
    """fp64 oracle output [num_q_tokens, Hq, D] of the whole workload."""
    key = _key(w, fp8)
    if key not in _OUT:
        oracle_cache(w, fp8)
    return _OUT[key]


def same_bytes(dev_tensor, host_storage) -> bool:
    if dev_tensor.dtype == torch.uint8:
        return np.array_equal(dev_tensor.cpu().numpy(), np.ascontiguousarray(host_storage))
    return np.array_equal(storage_bits(dev_tensor).view(np.uint8), np.ascontiguousarray(host_storage).view(np.uint8))


def assert_rows(gpu_out, ref, w, what: str):
    """Every output row against the oracle: the whole tensor, and each request's
    rows on their own, at the dtype's bar (max-abs and rel-L2)."""
    o = to_numpy(gpu_out) if isinstance(gpu_out, torch.Tensor) else gpu_out
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert_parity(o, ref, w.dtype, f"{what}: all {o.shape[0]} rows")
    cu = w.cu_query_lens
    worst = (0.0, 0.0, -1)
    from parity import TOL, errors
    tol_abs, tol_rel = TOL[w.dtype]
    for b in range(w.num_seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi == lo:
            continue
        mx, rel = errors(o[lo:hi], ref[lo:hi])
        assert mx <= tol_abs and rel <= tol_rel, (
            f"{what}: request {b} (L={int(w.seq_lens[b])}, {hi - lo} rows) max_abs {mx:.3e} rel_l2 {rel:.3e}")
        if rel > worst[1]:
            worst = (mx, rel, b)
    print(f"  {what}: worst request {worst[2]} max_abs={worst[0]:.3e} rel_l2={worst[1]:.3e}", flush=True)
