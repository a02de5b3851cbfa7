"""pa_decode_append_noalloc through the C ABI: on two calls in a row on one
device, the second with a smaller batch, its slots, caches and output equal
those of pa_decode_append with a caller workspace, bit for bit (the same
kernels on the same inputs), and meet the oracle; a call that needs more than
the library's scratch is refused before anything is written."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_parity, to_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    return pa


def _pair(pa, w):
    """The same step through both entry points, each on its own copy of the
    inputs; returns the two DeviceWorkloads and outputs."""
    from paged_kv_cache_432_amd.staging import DeviceWorkload
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    out_a = a.decode_append()                           # workspace from the caller
    k, v, slots = b.append_rows()
    out_b = torch.empty_like(b.query)
    pa.pa_decode_append_noalloc(out_b, b.query, k, v, b.key_cache, b.value_cache, b.block_table, b.seq_lens,
                                w.scale, w.max_seq_len, slots)
    torch.cuda.synchronize()
    return a, out_a, b, out_b


def _same(x, y) -> bool:
    return torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8))


@pytest.mark.parametrize("dtype,hq", [("bf16", 64), ("f32", 32)])
def test_noalloc_equals_workspace_entry_point_twice(pa, dtype, hq):
    """A wide call (300 sequences, nearly every one cut between workgroups, so
    the scratch holds many partial records; bf16 at G = 8, fp32 at G = 4 on its
    scatter-then-decode route), then a smaller one (5 sequences): the second
    call finds the first one's records in the scratch and must not depend on
    them."""
    rng = np.random.default_rng(70)
    big = W.custom("noalloc_big", seq_lens=rng.integers(1, 3000, 300), num_heads=hq, num_kv_heads=8,
                   dtype=dtype, seed=71)
    assert pa.pa_decode_workspace_bytes(big.num_seqs, hq, 8, 128, big.max_seq_len, 0) <= (32 << 20)
    small = W.custom("noalloc_small", seq_lens=[40, 1, 700, 0, 2500], num_heads=32, num_kv_heads=8,
                     dtype=dtype, seed=72)
    for w in (big, small):
        print(f"  {w.name} {dtype}: B={w.num_seqs} Hq={w.num_heads}", flush=True)
        a, out_a, b, out_b = _pair(pa, w)
        assert _same(out_a, out_b), f"{w.name}: outputs differ"
        assert _same(a.append_rows()[2], b.append_rows()[2]), f"{w.name}: slots differ"
        assert _same(a.key_cache, b.key_cache) and _same(a.value_cache, b.value_cache), f"{w.name}: caches differ"
        assert_parity(to_numpy(out_b), oracle.run(w), w.dtype, f"noalloc {w.name}")


def test_noalloc_refuses_a_call_beyond_its_scratch(pa):
    """More than 4096 sequences split into fixed partitions need
    B x Hq x partitions partial records: 5000 x 32 x 8 x 528 bytes, far above
    the 32 MiB scratch.  The host check refuses the call before any launch (the
    pointers are never dereferenced)."""
    L = pa.lib()
    need = pa.pa_decode_workspace_bytes(5000, 32, 8, 128, 8192, 0)
    assert need > (32 << 20)
    fake = 256
    st = L.pa_decode_append_noalloc(fake, fake, 4096, fake, 1024, fake, 1024, fake, fake, fake, fake, 512, fake,
                                    5000, 32, 8, 128, 16, 100000, ctypes.c_float(0.088), 8192, 1, None)
    assert st == pa.PA_ERR_WORKSPACE, pa.pa_last_error_message()
    assert "noalloc" in pa.pa_last_error_message()
