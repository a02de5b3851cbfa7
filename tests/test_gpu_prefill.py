"""Row a10 on the GPU: chunked prefill (query_len > 1, causal, MFMA) mixed with
single-row decodes in one pa_chunked_prefill call, against the oracle, element
by element at small sizes and on every row of the full mixed batch."""
import numpy as np
import pytest
import torch

import fullsize
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


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (8, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp32_chunks_and_decodes(staging, hq, hkv, causal):
    """fp32 caches: every query row runs as a decode row of its own (its key
    count under the mask, its request's table row), at the fp32 bar; chunks
    with and without earlier context, decodes, an empty request, and more rows
    than one stream-mode share."""
    lens = [300, 90, 700, 1, 64, 513, 40, 2]
    qlens = [300, 17, 260, 1, 0, 129, 1, 2]
    w = W.custom("mix32", seq_lens=lens, query_lens=qlens, num_heads=hq, num_kv_heads=hkv,
                 dtype="f32", seed=3 * hq + hkv, causal=causal)
    dw = staging.DeviceWorkload(w)
    dw.scatter_new()
    # output and workspace between guard zones: the row expansion and the
    # decode write nothing outside them
    import paged_kv_cache_432_amd as pa
    nbytes = pa.pa_chunked_prefill_workspace_bytes(w.num_seqs, w.num_q_tokens, w.max_query_len, w.max_seq_len,
                                                   w.num_heads, w.num_kv_heads, w.head_dim, torch.float32)
    out = staging.Guarded(dw.query.shape, torch.float32, dw.device)
    ws = staging.Guarded((nbytes,), torch.uint8, dw.device, 1 << 16)
    dw.chunked_prefill(out.t, ws.t)
    torch.cuda.synchronize()
    assert_parity(to_numpy(out.t), oracle.run(w), "f32", f"fp32 mixed G={hq // hkv} causal={causal}")
    assert out.intact() and ws.intact()


def test_fp32_more_rows_than_the_stream_mode_takes(staging):
    """4500 query rows (the decode's stream mode takes 4096 rows): the rows run
    in fixed partitions."""
    w = W.custom("rows32", seq_lens=[4600, 30], query_lens=[4490, 10], num_heads=2, num_kv_heads=2,
                 dtype="f32", seed=41, causal=True)
    assert w.num_q_tokens > 4096
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "f32", "fp32, 4500 rows")


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


def test_chunked_prefill_mix_full_size(staging):
    """The full mixed batch (4 x 512-row chunks at prior contexts 0, 2048,
    4096, 7680 plus 96 decodes) in the benchmark's launch configuration: the
    step's scatter of all 2144 new rows against the oracle's scatter (both
    whole caches byte for byte), and every one of the 2144 output rows of the
    unified call against the oracle; out, workspace and caches between guard
    zones.  Then the chunks alone (the split-call mode), every row."""
    w = W.chunked_prefill_mix()
    dw = staging.DeviceWorkload(w, guard_bytes=1 << 16)
    dw.scatter_new(fused=True)
    out = staging.Guarded(dw.query.shape, dw.query.dtype, dw.device)
    nbytes = dw.prefill_workspace().numel()
    ws = staging.Guarded((nbytes,), torch.uint8, dw.device, 1 << 16)
    dw.chunked_prefill(out.t, ws.t)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact() and dw.guards_intact(), "guard zone written"
    okc, ovc = fullsize.oracle_cache(w)
    assert fullsize.same_bytes(dw.key_cache, okc), "key cache"
    assert fullsize.same_bytes(dw.value_cache, ovc), "value cache"
    del okc, ovc, dw
    ref = fullsize.oracle_output(w)
    fullsize.assert_rows(out.t, ref, w, "chunked_prefill_mix unified")

    pre = W.prefill_part(w)
    dpre = staging.DeviceWorkload(pre, guard_bytes=1 << 16)
    dpre.scatter_new()
    out = staging.Guarded(dpre.query.shape, dpre.query.dtype, dpre.device)
    ws = staging.Guarded((dpre.prefill_workspace().numel(),), torch.uint8, dpre.device, 1 << 16)
    dpre.chunked_prefill(out.t, ws.t)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact() and dpre.guards_intact(), "guard zone written (chunks alone)"
    cu = w.cu_query_lens
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in range(w.num_seqs) if w.query_lens[b] > 1])
    fullsize.assert_rows(out.t, ref[rows], pre, "chunked_prefill_mix chunks, split mode")


def _with_values(w, kv_fn, q_fn=None):
    """w with K/V (and Q) of every sequence replaced by kv_fn(b, k, v) -> (k, v)
    of the drawn values; the oracle and the device staging read the same ones."""
    draw = w.kv
    memo = {}

    def kv(b, length=None):
        key = (b, length)
        if key not in memo:
            k, v = draw(b)
            k, v = kv_fn(b, k.copy(), v.copy())
            n = int(w.seq_lens[b]) if length is None else int(length)
            memo[key] = (k[:n], v[:n])
        return memo[key]

    w.kv = kv
    if q_fn is not None:
        drawq = w.query
        w.query = lambda b: q_fn(b, drawq(b).copy())
    return w


def test_tiny_probabilities_keep_their_weight(staging):
    """One key per sequence scores ~10.4 nats above all others, so every other
    probability is ~3e-5: below fp16's normal range.  The many small terms
    still carry ~9% of the weight at 3000 keys; dropping them (a flush of
    subnormals) moves the output by several hundredths."""
    w = W.custom("spike", seq_lens=[3000, 700], query_lens=[600, 700], dtype="bf16", seed=16)

    def kv_fn(b, k, v):
        rng = np.random.default_rng([16, b])
        k[:, :, 0] = W.bf16_round(0.05 * rng.standard_normal(k.shape[:2]).astype(np.float32))
        k[0, :, 0] = 14.75                             # the spike key: position 0
        v[:] = W.bf16_round(-1.0 + 0.1 * rng.standard_normal(v.shape).astype(np.float32))
        v[0] = 1.0
        return k, v

    def q_fn(b, q):
        q[:] = 0.0
        q[:, :, 0] = 8.0                               # score = scale * 8 * k[., 0]
        return q

    w = _with_values(w, kv_fn, q_fn)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "spike + subnormal tail")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8)])
def test_values_beyond_half_range(staging, hq, hkv):
    """V of one sequence scaled by 2^17 (exact in bf16): most of its values
    exceed fp16's range, while the other sequences' do not.  The scaled
    sequence's rows divided by 2^17 match the oracle on the unscaled values."""
    lens, qlens = [900, 300, 1200], [300, 300, 129]
    base = W.custom("big", seq_lens=lens, query_lens=qlens, num_heads=hq, num_kv_heads=hkv,
                    dtype="bf16", seed=17)
    ref = oracle.run(base)
    big = _with_values(W.custom("big", seq_lens=lens, query_lens=qlens, num_heads=hq, num_kv_heads=hkv,
                                dtype="bf16", seed=17),
                       lambda b, k, v: (k, v * np.float32(2.0 ** 17) if b == 0 else v))
    _, out = _run(staging, big)
    o = to_numpy(out)
    cu = base.cu_query_lens
    o[cu[0]:cu[1]] /= 2.0 ** 17
    assert_parity(o, ref, "bf16", f"V x 2^17 in sequence 0, G={hq // hkv}")


def test_mixed_record_formats(staging):
    """The tiles of one long chunk (6000 keys, 512 rows) are cut over several
    workgroups.  V of keys 4000 and up is scaled by 2^17, so the segments that
    stage those keys run the exact path and leave fp32 records, while the
    earlier segments of the same tiles leave fp16 ones; the merge combines
    both.  Those keys' K (dim 0 = -1000 against a query dim 0 of 10) puts
    their scores some 1300 log2 units down, so their probabilities are 0 in
    fp32 and fp64 alike and the outputs keep their usual magnitude."""
    w = W.custom("mixrec", seq_lens=[6000, 700], query_lens=[512, 700], dtype="bf16", seed=19, causal=True)

    def kv_fn(b, k, v):
        if b == 0:
            k[4000:, :, 0] = np.float32(-1000.0)
            v[4000:] = v[4000:] * np.float32(2.0 ** 17)
        return k, v

    def q_fn(b, q):
        if b == 0:
            q[:, :, 0] = np.float32(10.0)
        return q

    w = _with_values(w, kv_fn, q_fn)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "fp16 and fp32 records in one merge")


def test_rising_scores_rescale(staging):
    """Chunk rows whose scores rise along the keys (~40 log2 units over the
    context): the softmax reference is raised, and the accumulators rescaled,
    on many tiles, including across the pieces the merge combines."""
    w = W.custom("rise", seq_lens=[1800, 700], query_lens=[300, 700], dtype="bf16", seed=18)

    def kv_fn(b, k, v):
        k[:, :, 0] = W.bf16_round((0.05 * np.arange(k.shape[0], dtype=np.float32))[:, None]
                                  * np.ones(k.shape[1], np.float32)[None, :])
        return k, v

    def q_fn(b, q):
        q[:, :, 0] = 4.0
        return q

    w = _with_values(w, kv_fn, q_fn)
    _, out = _run(staging, w)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "rising scores")
