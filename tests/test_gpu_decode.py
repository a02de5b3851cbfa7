"""Rows a3-a9 on the GPU: paged decode attention (single pass and split +
merge) against the oracle, element by element, at small sizes and at the full
workload sizes (every output row), with guard zones around the output, the
workspace and the caches."""
import numpy as np
import pytest
import torch

import fullsize
import oracle
import workloads as W
from parity import assert_parity, storage_bits, to_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def staging():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    from paged_kv_cache_432_amd import staging
    return staging


def _run(staging, w, partition_tokens=0):
    dw = staging.DeviceWorkload(w)
    dw.scatter_new()
    out = dw.decode(partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return dw, out


@pytest.mark.parametrize("step", ["A", "B"])
@pytest.mark.parametrize("pt", [-1, 0, 16, 32])
def test_tiny_fp32(staging, step, pt):
    w = W.tiny(step)
    _, out = _run(staging, w, pt)
    assert_parity(to_numpy(out), oracle.run(w), "f32", f"tiny{step} pt={pt}")


RAGGED = [1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 1000, 1024, 2049, 4095]


@pytest.mark.parametrize("pt", [-1, 0, 16, 256, 512, 2048])
def test_ragged_bf16(staging, pt):
    w = W.custom("ragged", seq_lens=RAGGED, dtype="bf16", seed=31, sigma=1.0)
    _, out = _run(staging, w, pt)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", f"ragged pt={pt}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (32, 4), (64, 8), (16, 16)])
def test_group_sizes(staging, dtype, hq, hkv):
    w = W.custom("gqa", seq_lens=[5, 64, 130, 700], num_heads=hq, num_kv_heads=hkv, dtype=dtype,
                 seed=hq + hkv)
    for pt in (0, -1, 64):
        _, out = _run(staging, w, pt)
        assert_parity(to_numpy(out), oracle.run(w), dtype, f"G={hq // hkv} Hkv={hkv} pt={pt}")


def test_padding_sequences_output_zero(staging):
    w = W.custom("pad", seq_lens=[0, 40, 0, 300], dtype="bf16", seed=3)
    for pt in (0, -1, 64):
        _, out = _run(staging, w, pt)
        o = to_numpy(out)
        assert np.all(o[0] == 0) and np.all(o[2] == 0)
        assert_parity(o, oracle.run(w), "bf16", f"padding pt={pt}")


def test_deterministic_and_permutation_invariant(staging):
    w = W.custom("perm", seq_lens=[77, 300, 1234, 16], dtype="bf16", seed=5, num_blocks=200)
    dw, out1 = _run(staging, w, 128)
    out2 = dw.decode(partition_tokens=128)
    torch.cuda.synchronize()
    assert np.array_equal(storage_bits(out1), storage_bits(out2))
    perm = np.random.default_rng(1).permutation(300)
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    _, out3 = _run(staging, w.with_block_table(table, num_blocks=300), 128)
    assert np.array_equal(storage_bits(out1), storage_bits(out3))


@pytest.mark.parametrize("lens", [
    [5000, 3, 0, 17, 4096, 1, 2500],                # long and short neighbours, an empty one
    [33] * 600,                                     # many short sequences per workgroup
    [0] * 5 + [16] * 3 + [0] * 4,                   # empty sequences at both ends
])
def test_stream_mode_edges(staging, lens):
    """The automatic (balanced stream) mode: sequences cut between workgroups,
    workgroups spanning many sequences, empty sequences anywhere."""
    w = W.custom("stream", seq_lens=lens, dtype="bf16", seed=len(lens))
    _, out = _run(staging, w, 0)
    o = to_numpy(out)
    ref = oracle.run(w)
    for b in np.nonzero(np.asarray(lens) == 0)[0]:
        assert np.all(o[b] == 0)
    assert_parity(o, ref, "bf16", f"stream {len(lens)} seqs")


@pytest.mark.parametrize("dtype,form", [("bf16", "decode"), ("bf16", "append"), ("f32", "decode")])
def test_paired_merge(staging, dtype, form):
    """More (sequence, query head) pairs than one round of merge waves (32 per
    compute unit) with a group of 4: the split merge takes two heads of a KV
    head per wave.  Short sequences (one or two pieces) and empty ones, beside
    sequences cut into a few pieces, into 9-24 and into more than 64 (which
    the pair merges one head after the other)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = max(1100, 2 * cus + 64)
    rng = np.random.default_rng(99)
    lens = rng.integers(1, 300, n).astype(np.int32)
    lens[::53] = 0
    lens[7], lens[500], lens[900] = 65536, 6000, 2000
    assert n * 16 > 32 * cus
    w = W.custom("pairs", seq_lens=lens, num_heads=16, num_kv_heads=4, dtype=dtype, seed=99, sigma=0.5)
    dw = staging.DeviceWorkload(w)
    if form == "append":
        out = dw.decode_append()
    else:
        dw.scatter_new()
        out = dw.decode()
    torch.cuda.synchronize()
    o = to_numpy(out)
    for b in np.nonzero(lens == 0)[0]:
        assert np.all(o[b] == 0)
    assert_parity(o, oracle.run(w), dtype, f"paired merge, {dtype} {form}")


def test_many_sequences_use_partitions(staging):
    """Past 4096 sequences the automatic choice is fixed partitions."""
    import paged_kv_cache_432_amd as pa
    lens = (np.arange(4200) % 40 + 1).astype(np.int32)
    assert pa.pa_decode_partition_tokens(len(lens), 8, int(lens.max()), 0) > 0
    w = W.custom("many", seq_lens=lens, dtype="bf16", seed=77, num_heads=8, num_kv_heads=8)
    _, out = _run(staging, w, 0)
    assert_parity(to_numpy(out), oracle.run(w), "bf16", "4200 seqs")


def test_single_token_returns_value_row(staging):
    w = W.custom("one", seq_lens=[1, 1, 1], dtype="bf16", seed=8)
    _, out = _run(staging, w, 0)
    got = storage_bits(out)
    for b in range(3):
        _, v = w.kv(b)
        want = W.bf16_bits(np.repeat(v[0], w.group, axis=0))
        assert np.array_equal(got[b], want)


def _full(staging, w, pts=(0,)):
    """Full-size workload on the GPU in the benchmark's launch configuration,
    every output row against the oracle; out, workspace and caches between
    guard zones."""
    print(f"  full size {w.name}: B={w.num_seqs} Hq={w.num_heads} KV tokens {int(w.seq_lens.sum())}", flush=True)
    dw = staging.DeviceWorkload(w, guard_bytes=1 << 16)
    dw.scatter_new()
    ref = fullsize.oracle_output(w)
    for pt in pts:
        out = staging.Guarded(dw.query.shape, dw.query.dtype, dw.device)
        nbytes = dw.decode_workspace(pt).numel()
        ws = staging.Guarded((nbytes,), torch.uint8, dw.device, 1 << 16)
        dw.decode(out.t, pt, ws.t)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact() and dw.guards_intact(), f"{w.name} pt={pt}: guard zone written"
        fullsize.assert_rows(out.t, ref, w, f"{w.name} pt={pt}")


def test_llama8b_decode_full_size(staging):
    _full(staging, W.llama8b_decode())


def test_llama8b_decode_8k_full_size(staging):
    _full(staging, W.llama8b_decode_8k())


def test_long_context_full_size(staging):
    _full(staging, W.long_context(), pts=(0, 2048))


def test_continuous_batching_full_size(staging):
    _full(staging, W.continuous_batching(), pts=(0, 512))


def test_chunked_mix_decode_part_split_mode(staging):
    """The 96 decodes of the mixed batch, run through pa_decode (split-call
    mode), every row against the oracle's rows of the whole mixed batch."""
    mix = W.chunked_prefill_mix()
    w = W.decode_part(mix)
    print(f"  decodes of {mix.name}: {w.num_seqs}", flush=True)
    dw = staging.DeviceWorkload(w, guard_bytes=1 << 16)
    dw.scatter_new()
    out = staging.Guarded(dw.query.shape, dw.query.dtype, dw.device)
    nbytes = dw.decode_workspace(0).numel()
    ws = staging.Guarded((nbytes,), torch.uint8, dw.device, 1 << 16)
    dw.decode(out.t, 0, ws.t)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact() and dw.guards_intact()
    rows = mix.cu_query_lens[:-1][mix.query_lens == 1]
    fullsize.assert_rows(out.t, fullsize.oracle_output(mix)[rows], w, "mixed batch decodes, split mode")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (8, 8)])
def test_rising_scores_rescale(staging, hq, hkv):
    """Scores that rise along the sequence (~50 log2 units over 2000 tokens):
    the softmax reference is raised and the partial output rescaled many times
    within one wave's range, in every split mode."""
    w = W.custom("rise", seq_lens=[2000, 900, 37], num_heads=hq, num_kv_heads=hkv, dtype="bf16", seed=41)
    draw_kv, draw_q = w.kv, w.query
    memo = {}

    def kv(b, length=None):
        if (b, length) not in memo:
            k, v = draw_kv(b)
            k = k.copy()
            k[:, :, 0] = W.bf16_round((0.05 * np.arange(k.shape[0], dtype=np.float32))[:, None]
                                      * np.ones(k.shape[1], np.float32)[None, :])
            n = int(w.seq_lens[b]) if length is None else int(length)
            memo[(b, length)] = (k[:n], v[:n])
        return memo[(b, length)]

    def query(b):
        q = draw_q(b).copy()
        q[:, :, 0] = 4.0
        return q

    w.kv, w.query = kv, query
    ref = oracle.run(w)
    for pt in (0, -1, 256):
        _, out = _run(staging, w, pt)
        assert_parity(to_numpy(out), ref, "bf16", f"rising scores G={hq // hkv} pt={pt}")
