"""The measurement probes on the GPU: the copy probe moves bytes exactly, the
read probe and the matrix-core probe run to completion and leave their sinks
untouched (they write only if a fixed value comes out, which does not)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    return pa


def test_copy_probe_is_exact(pa):
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    pa.pa_probe_copy(dst, src, 64)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_read_probe_leaves_sink(pa):
    src = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_probe_stream_read(src, sink, 0)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_mfma_probe_runs(pa):
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    flops = pa.pa_probe_mfma(sink, 8, 16)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 16 * 4 * 32768
    assert int(sink.item()) == 0
