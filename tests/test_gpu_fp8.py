"""fp8 (OCP E4M3) KV cache on the GPU: the scatter against the oracle's
encoding, bit for bit (the code is an integer decided by float32 arithmetic
that both sides do the same way: a correctly rounded division, then the
nearest code), and decode over the codes against the oracle's fp64 attention
over the same codes (the bf16 bar: max-abs <= 1e-2, rel-L2 <= 2e-3)."""
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


@pytest.fixture(scope="module")
def staging(pa):
    from paged_kv_cache_432_amd import staging
    return staging


def _bf16_is_nan(bits):
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def _compare_codes(got, want, src_nan):
    """Bit-exact, except that a NaN input may come out as either NaN code."""
    got, want = got.reshape(-1), want.reshape(-1)
    nan = src_nan.reshape(-1)
    assert np.all(got[nan] & 0x7F == 0x7F) and np.all(want[nan] & 0x7F == 0x7F)
    bad = np.nonzero(got[~nan] != want[~nan])[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. got {got[~nan][bad[:5]]} want {want[~nan][bad[:5]]}"


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 3.1), (2.0 ** -6, 2.0 ** -3)])
def test_scatter_every_bf16_value(pa, scales):
    """All 65,536 bf16 bit patterns (zeros, subnormals, ties, values past 448,
    infinities, NaNs) as K, the same reversed as V."""
    ks, vs = scales
    hkv, d, nb = 8, 128, 8
    kbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(64, hkv, d)
    vbits = kbits[::-1].copy()
    slots = np.random.default_rng(1).choice(nb * 16, 64, replace=False).astype(np.int64)
    dev = "cuda"
    kc = torch.full((nb, 16, hkv, d), 0x5A, dtype=torch.uint8, device=dev)
    vc = kc.clone()
    as_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    pa.pa_reshape_and_cache_fp8(as_bf16(kbits), as_bf16(vbits), kc, vc, torch.from_numpy(slots).to(dev), ks, vs)
    torch.cuda.synchronize()
    okc = np.full((nb, 16, hkv, d), 0x5A, np.uint8)
    ovc = okc.copy()
    oracle.reshape_and_cache_fp8(kbits, vbits, okc, ovc, slots, ks, vs)
    gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
    flat = lambda a: a.reshape(nb * 16, hkv, d)
    _compare_codes(flat(gk)[slots], flat(okc)[slots], _bf16_is_nan(kbits))
    _compare_codes(flat(gv)[slots], flat(ovc)[slots], _bf16_is_nan(vbits))
    rest = np.setdiff1d(np.arange(nb * 16), slots)
    assert np.all(flat(gk)[rest] == 0x5A) and np.all(flat(gv)[rest] == 0x5A)


def test_scatter_f32_source_and_padding(pa):
    rng = np.random.default_rng(5)
    n, hkv, d, nb = 300, 2, 128, 40
    x = (rng.standard_normal((2, n, hkv, d)) * np.float32(50)).astype(np.float32)
    x[0, :, 0, :8] = np.float32(1e-6) * rng.standard_normal((n, 8)).astype(np.float32)   # deep underflow
    slots = rng.choice(nb * 16, n, replace=False).astype(np.int64)
    slots[::11] = -1
    slots[3::37] = nb * 16 + 5                         # past the pool: skipped
    dev = "cuda"
    kc = torch.zeros((nb, 16, hkv, d), dtype=torch.uint8, device=dev)
    vc = kc.clone()
    pa.pa_reshape_and_cache_fp8(torch.from_numpy(x[0]).to(dev), torch.from_numpy(x[1]).to(dev), kc, vc,
                                torch.from_numpy(slots).to(dev), 0.11, 0.29)
    torch.cuda.synchronize()
    okc = np.zeros((nb, 16, hkv, d), np.uint8)
    ovc = okc.copy()
    live = (slots >= 0) & (slots < nb * 16)
    oracle.reshape_and_cache_fp8(x[0], x[1], okc, ovc, np.where(live, slots, -1), 0.11, 0.29)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


def _decode(staging, w):
    dw = staging.DeviceWorkload(w, kv_fp8=True)
    dw.scatter_new()
    out = dw.decode()
    torch.cuda.synchronize()
    return dw, out


RAGGED = [1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 1000, 1024, 2049, 4095]


def test_decode_ragged_and_cache_bytes(staging):
    w = W.custom("ragged", seq_lens=RAGGED, dtype="bf16", seed=31, sigma=1.0)
    dw, out = _decode(staging, w)
    ks, vs = w.fp8_scales()
    okc, ovc = oracle.build_cache_fp8(w, ks, vs)
    assert np.array_equal(dw.key_cache.cpu().numpy(), okc)
    assert np.array_equal(dw.value_cache.cpu().numpy(), ovc)
    assert_parity(to_numpy(out), oracle.run_fp8(w, ks, vs), "bf16", "fp8 ragged")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (32, 4), (64, 8), (16, 16)])
def test_decode_group_sizes(staging, hq, hkv):
    w = W.custom("gqa", seq_lens=[5, 64, 130, 700], num_heads=hq, num_kv_heads=hkv, dtype="bf16", seed=hq + hkv)
    _, out = _decode(staging, w)
    assert_parity(to_numpy(out), oracle.run_fp8(w, *w.fp8_scales()), "bf16", f"fp8 G={hq // hkv} Hkv={hkv}")


@pytest.mark.parametrize("lens", [
    [5000, 3, 0, 17, 4096, 1, 2500],
    [33] * 600,
    [0] * 5 + [16] * 3 + [0] * 4,
])
def test_decode_stream_edges(staging, lens):
    w = W.custom("stream", seq_lens=lens, dtype="bf16", seed=len(lens))
    _, out = _decode(staging, w)
    o = to_numpy(out)
    for b in np.nonzero(np.asarray(lens) == 0)[0]:
        assert np.all(o[b] == 0)
    assert_parity(o, oracle.run_fp8(w, *w.fp8_scales()), "bf16", f"fp8 stream {len(lens)} seqs")


def test_decode_values_beyond_the_code_range(staging):
    """Scales of 1/512 for N(0, 1) values: every |x| > 448/512 = 0.875 (38% of
    them) saturates to +-0.875.  The oracle applies the same saturation, so
    the results agree (outputs stay below 1, where the bf16 bar is meant)."""
    w = W.custom("sat", seq_lens=[300, 1200, 47], dtype="bf16", seed=13, sigma=1.0)
    w.fp8_scales = lambda: (1.0 / 512, 1.0 / 512)
    dw, out = _decode(staging, w)
    assert np.mean((dw.key_cache.cpu().numpy() & 0x7F) == 0x7E) > 0.2
    assert_parity(to_numpy(out), oracle.run_fp8(w, 1.0 / 512, 1.0 / 512), "bf16", "fp8 saturated")


@pytest.mark.parametrize("name", ["llama8b_decode", "continuous_batching"])
def test_decode_full_size_sampled(staging, name):
    w = W.CONFIGS[name]()
    _, out = _decode(staging, w)
    o = to_numpy(out)
    assert np.all(np.isfinite(o))
    seqs = [int(np.argmax(w.seq_lens)), int(np.argmin(w.seq_lens)), 7, 33]
    ref = oracle.run_sequences(w, seqs, fp8_scales=w.fp8_scales())
    for b in seqs:
        assert_parity(o[b:b + 1], ref[b], "bf16", f"fp8 {name} seq {b} (L={int(w.seq_lens[b])})")
