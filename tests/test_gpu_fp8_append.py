"""The fp8 decode step in one call on the GPU: pa_decode_append_fp8 stores each
sequence's newest token as fp8 codes in its slot (the page-table lookup of "AI
Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention"; the quantising
copy of section "Reshape & Cache") and attends over the whole sequence.

Against the two-call step (pa_slot_mapping_and_cache_fp8, then
pa_decode_fp8) on the same inputs: slots, both caches and the output bit for
bit, since the decode reads the newest token back from the cache like any
other.  Against the oracle: the slots and caches bit for bit, the output at the
bf16 bar over the codes; at the benchmark's full sizes every row, with guard
zones around the output, the workspace and the caches.  Both formats."""
import numpy as np
import pytest
import torch

import fullsize
import oracle
import workloads as W
from parity import assert_parity, to_numpy

pytestmark = pytest.mark.gpu
FORMATS = ["e4m3", "e5m2"]


@pytest.fixture(scope="module")
def staging():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    from paged_kv_cache_432_amd import staging
    return staging


def _expected_slots(w):
    out = np.full(w.num_seqs, -1, np.int64)
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        if L > 0:
            out[b] = oracle.slot(w.block_table[b], L - 1, w.block_size)
    return out


def _against_two_calls(staging, w, fmt, what):
    a = staging.DeviceWorkload(w, kv_fp8=True, fp8_format=fmt)
    out_a = a.decode_append()
    b = staging.DeviceWorkload(w, kv_fp8=True, fp8_format=fmt)
    b.scatter_new(fused=True)
    out_b = b.decode()
    torch.cuda.synchronize()
    _, _, slots = a.append_rows()
    assert np.array_equal(slots.cpu().numpy(), _expected_slots(w)), what
    assert torch.equal(a.key_cache, b.key_cache), f"{what}: key cache"
    assert torch.equal(a.value_cache, b.value_cache), f"{what}: value cache"
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"{what}: output"
    return a, out_a


@pytest.mark.parametrize("fmt", FORMATS)
def test_matches_two_call_step(staging, fmt):
    """Ragged lengths (one token, block edges, a new block for the newest
    token, empty sequences): identical to the two-call step, and the caches
    and output against the oracle."""
    lens = [1, 2, 15, 16, 17, 33, 0, 256, 257, 1000, 4097, 0, 77, 2049]
    w = W.custom("fp8_append", seq_lens=lens, dtype="bf16", seed=81, sigma=1.0)
    a, out = _against_two_calls(staging, w, fmt, f"{fmt} ragged")
    ks, vs = w.fp8_scales()
    okc, ovc = oracle.build_cache_fp8(w, ks, vs, "all", fmt)
    assert np.array_equal(a.key_cache.cpu().numpy(), okc)
    assert np.array_equal(a.value_cache.cpu().numpy(), ovc)
    o = to_numpy(out)
    for b in np.nonzero(np.asarray(lens) == 0)[0]:
        assert np.all(o[b] == 0)
    assert_parity(o, oracle.run_fp8(w, ks, vs, fmt), "bf16", f"{fmt} append ragged")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (32, 4), (64, 8), (16, 16)])
def test_group_sizes(staging, hq, hkv):
    """Every group size and workgroup width (several KV-head groups per
    sequence where W < Hkv), each group's newest rows stored by the workgroup
    that reads its last block."""
    w = W.custom("fp8_append_gqa", seq_lens=[5, 64, 130, 700, 16, 1], num_heads=hq, num_kv_heads=hkv,
                 dtype="bf16", seed=hq * 3 + hkv)
    _against_two_calls(staging, w, "e4m3", f"G={hq // hkv} Hkv={hkv}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_many_sequences_in_groups(staging, fmt):
    """8193 sequences: three launches over groups of 4096, 4096 and 1, each
    storing its own sequences' newest rows; identical to the two-call step."""
    rng = np.random.default_rng(82)
    lens = rng.integers(1, 60, 8193).astype(np.int32)
    lens[::97] = 0
    w = W.custom("fp8_append_many", seq_lens=lens, num_heads=8, num_kv_heads=8, dtype="bf16", seed=82, sigma=0.5)
    _against_two_calls(staging, w, fmt, f"{fmt} 8193 sequences")


def test_repeated_calls(staging):
    """A second call over the same inputs stores the same codes and gives the
    same output; stale codes in the newest slots before the first call make
    no difference."""
    w = W.custom("fp8_append_repeat", seq_lens=[33, 200, 1, 16], dtype="bf16", seed=83)
    dw = staging.DeviceWorkload(w, kv_fp8=True)
    for s in _expected_slots(w):                           # stale finite codes in the newest slots
        dw.key_cache.view(-1, w.num_kv_heads, w.head_dim)[int(s)] = 0x38
        dw.value_cache.view(-1, w.num_kv_heads, w.head_dim)[int(s)] = 0xB8
    out1 = dw.decode_append().clone()
    kc = dw.key_cache.clone()
    out2 = dw.decode_append()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(kc, dw.key_cache)
    assert_parity(to_numpy(out1), oracle.run_fp8(w, *w.fp8_scales()), "bf16", "fp8 append repeat")


def test_failed_workspace_check_writes_nothing(staging):
    """An undersized workspace is found before anything is enqueued: the call
    fails with PA_ERR_WORKSPACE and the caches and slot_mapping are unchanged
    byte for byte."""
    import paged_kv_cache_432_amd as pa
    w = W.custom("fp8_ws_check", seq_lens=[40, 700, 1300, 17], dtype="bf16", seed=84)
    dw = staging.DeviceWorkload(w, kv_fp8=True)
    _, _, slots = dw.append_rows()
    slots.fill_(-7)
    before = [t.clone() for t in (dw.key_cache, dw.value_cache, slots)]
    nbytes = dw.decode_workspace(0).numel()
    small = torch.empty(nbytes - 16, dtype=torch.uint8, device=dw.device)
    with pytest.raises(pa.PaError) as e:
        dw.decode_append(workspace=small)
    assert e.value.status == pa.PA_ERR_WORKSPACE, e.value
    torch.cuda.synchronize()
    for a, b in zip(before, (dw.key_cache, dw.value_cache, slots)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,fmt", [("llama8b_decode_8k", "e4m3"), ("llama8b_decode_8k", "e5m2"),
                                      ("continuous_batching", "e4m3")])
def test_full_size(staging, name, fmt):
    """The benchmark's fp8 step at full size: slots bit for bit, both whole
    caches byte for byte against the oracle's fp8 scatter of every token, every
    output row against the oracle's attention over the codes; out, workspace
    and caches between guard zones."""
    w = W.CONFIGS[name]()
    print(f"  full size {w.name} {fmt}: B={w.num_seqs} KV tokens {int(w.seq_lens.sum())}", flush=True)
    dw = staging.DeviceWorkload(w, kv_fp8=True, fp8_format=fmt, guard_bytes=1 << 16)
    out = staging.Guarded(dw.query.shape, dw.query.dtype, dw.device)
    ws = staging.Guarded((dw.decode_workspace(0).numel(),), torch.uint8, dw.device, 1 << 16)
    dw.decode_append(out.t, ws.t)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact() and dw.guards_intact(), "guard zone written"
    _, _, slots = dw.append_rows()
    assert np.array_equal(slots.cpu().numpy(), _expected_slots(w))
    okc, ovc = fullsize.oracle_cache(w, fp8=fmt)
    assert fullsize.same_bytes(dw.key_cache, okc), "key cache"
    assert fullsize.same_bytes(dw.value_cache, ovc), "value cache"
    del okc, ovc
    fullsize.assert_rows(out.t, fullsize.oracle_output(w, fp8=fmt), w, f"{fmt} append {name}")
