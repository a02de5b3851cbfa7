"""Row a10 on the GPU: chunked prefill (query_len > 1, causal, MFMA) mixed with
single-row decodes in one pa_chunked_prefill call, against the oracle, element
by element at small sizes and on sampled rows of the full mixed batch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_parity, to_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def staging():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    from paged_kv_cache_432_amd import staging
    return staging


def _run(staging, w):
    dw = staging.DeviceWorkload(w)
    dw.scatter_new()
    out = dw.chunked_prefill()
    torch.cuda.synchronize()
    return dw, out


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (8, 1)])
def test_chunks_and_decodes(staging, hq, hkv):
    """Chunks longer and shorter than a tile, with and without earlier
    context, next to decodes and a request with no rows this step."""
    lens = [300, 90, 700, 1, 64, 513, 40, 2]
    qlens = [300, 17, 260, 1, 0, 129, 1, 2]
    w = W.custom("mix", seq_lens=lens, query_lens=qlens, num_heads=hq, num_kv_heads=hkv,
                 dtype="bf16", seed=hq + 7 * hkv, causal=True)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", f"mixed G={hq // hkv} Hkv={hkv}")


def test_prefill_without_context_is_causal_self_attention(staging):
    w = W.custom("self", seq_lens=[256, 77], query_lens=[256, 77], dtype="bf16", seed=12, causal=True)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "causal self-attention")


def test_non_causal_chunks(staging):
    w = W.custom("full", seq_lens=[200, 65, 5], query_lens=[50, 65, 1], dtype="bf16", seed=13, causal=False)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "non-causal")


def test_deterministic(staging):
    w = W.custom("det", seq_lens=[400, 33, 1000], query_lens=[300, 1, 64], dtype="bf16", seed=14)
    dw, out1 = _run(staging, w)
    out2 = dw.chunked_prefill()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_split_call_mode_matches_unified(staging):
    """The mixed batch as two calls (chunks through pa_chunked_prefill, decodes
    through pa_decode) gives the same rows as the unified call."""
    w = W.custom("split", seq_lens=[500, 81, 1200, 9], query_lens=[128, 1, 200, 1], dtype="bf16", seed=15)
    dw, unified = _run(staging, w)
    ref = oracle.run(w)
    assert_parity(to_numpy(unified), ref, "bf16", "unified")
    pre = W.prefill_part(w)
    dec = W.decode_part(w)
    _, out_pre = _run(staging, pre)
    ddw = staging.DeviceWorkload(dec)
    ddw.scatter_new()
    out_dec = ddw.decode()
    torch.cuda.synchronize()
    cu = w.cu_query_lens
    rows_pre = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in range(w.num_seqs) if w.query_lens[b] > 1])
    rows_dec = np.array([cu[b] for b in range(w.num_seqs) if w.query_lens[b] == 1])
    assert_parity(to_numpy(out_pre), ref[rows_pre], "bf16", "split: chunks")
    assert_parity(to_numpy(out_dec), ref[rows_dec], "bf16", "split: decodes")


def _oracle_last_rows(w, b, k):
    """Oracle output of the last k query rows of request b: a request with the
    same context whose query is only those rows sits at the same positions."""
    L, q = int(w.seq_lens[b]), int(w.query_lens[b])
    sub = W._subset(w, np.array([b]), "rows")
    sub.query_lens = np.array([k], np.int32)
    sub.query = lambda _b: w.query(b)[q - k:]
    return oracle.run_sequences(sub, [0])[0]


def test_chunked_prefill_mix_full_size(staging):
    """The full mixed batch (4 x 512-row chunks at prior contexts 0, 2048,
    4096, 7680 plus 96 decodes) in the benchmark's launch configuration; the
    oracle recomputes whole short chunks, the last rows of the long ones, and
    sampled decodes."""
    w = W.chunked_prefill_mix()
    dw, out = _run(staging, w)
    o = to_numpy(out)
    assert np.all(np.isfinite(o))
    cu = w.cu_query_lens
    ref = oracle.run_sequences(w, [0, 1, 10, 57, 99])
    for b in (0, 1):
        assert_parity(o[cu[b]:cu[b + 1]], ref[b], "bf16", f"chunk {b} (L={int(w.seq_lens[b])})")
    for b in (2, 3):
        k = 64
        assert_parity(o[cu[b + 1] - k:cu[b + 1]], _oracle_last_rows(w, b, k), "bf16",
                      f"chunk {b} last {k} rows (L={int(w.seq_lens[b])})")
    for b in (10, 57, 99):
        assert_parity(o[cu[b]:cu[b + 1]], ref[b], "bf16", f"decode {b} (L={int(w.seq_lens[b])})")
