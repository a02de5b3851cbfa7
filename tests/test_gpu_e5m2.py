"""fp8 KV cache in the other format the pages name, OCP E5M2, on the GPU: the
scatter against the oracle's encoding bit for bit (nearest code of the
float32 quotient, ties to even, saturating at 57344; both sides take the
integer decision in the same float32 arithmetic), and decode over the codes
against the oracle's fp64 attention over the same codes (the bf16 bar:
max-abs <= 1e-2, rel-L2 <= 2e-3)."""
import numpy as np
import pytest
import torch

import fullsize
import oracle
import workloads as W
from parity import assert_parity, to_numpy

pytestmark = pytest.mark.gpu
FMT = "e5m2"


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


def _is_e5m2_nan(codes):
    return ((codes & 0x7C) == 0x7C) & ((codes & 0x03) != 0)


def _compare_codes(got, want, src_nan):
    """Bit-exact, except that a NaN input may come out as any NaN code."""
    got, want = got.reshape(-1), want.reshape(-1)
    nan = src_nan.reshape(-1)
    assert np.all(_is_e5m2_nan(got[nan])) and np.all(_is_e5m2_nan(want[nan]))
    bad = np.nonzero(got[~nan] != want[~nan])[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. got {got[~nan][bad[:5]]} want {want[~nan][bad[:5]]}"


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 3.1), (2.0 ** -6, 2.0 ** -3), (2.0 ** 12, 1e-30)])
def test_scatter_every_bf16_value(pa, scales):
    """All 65,536 bf16 bit patterns (zeros, subnormals of both formats, ties,
    values past 57344, infinities, NaNs) as K, the same reversed as V."""
    ks, vs = scales
    hkv, d, nb = 8, 128, 8
    kbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(64, hkv, d)
    vbits = kbits[::-1].copy()
    slots = np.random.default_rng(2).choice(nb * 16, 64, replace=False).astype(np.int64)
    dev = "cuda"
    kc = torch.full((nb, 16, hkv, d), 0x5A, dtype=torch.uint8, device=dev)
    vc = kc.clone()
    as_bf16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    pa.pa_reshape_and_cache_fp8(as_bf16(kbits), as_bf16(vbits), kc, vc, torch.from_numpy(slots).to(dev), ks, vs,
                                fp8_format=FMT)
    torch.cuda.synchronize()
    okc = np.full((nb, 16, hkv, d), 0x5A, np.uint8)
    ovc = okc.copy()
    oracle.reshape_and_cache_fp8(kbits, vbits, okc, ovc, slots, ks, vs, fp8_format=FMT)
    gk, gv = kc.cpu().numpy(), vc.cpu().numpy()
    flat = lambda a: a.reshape(nb * 16, hkv, d)
    _compare_codes(flat(gk)[slots], flat(okc)[slots], _bf16_is_nan(kbits))
    _compare_codes(flat(gv)[slots], flat(ovc)[slots], _bf16_is_nan(vbits))
    rest = np.setdiff1d(np.arange(nb * 16), slots)
    assert np.all(flat(gk)[rest] == 0x5A) and np.all(flat(gv)[rest] == 0x5A)
    # the codes are E5M2, not E4M3: the two formats differ on most values
    e4 = np.full_like(okc, 0x5A)
    oracle.reshape_and_cache_fp8(kbits, vbits, e4, ovc.copy(), slots, ks, vs, fp8_format="e4m3")
    assert np.mean(flat(gk)[slots] != flat(e4)[slots]) > 0.5


def test_scatter_f32_source_and_padding(pa):
    rng = np.random.default_rng(6)
    n, hkv, d, nb = 300, 2, 128, 40
    x = (rng.standard_normal((2, n, hkv, d)) * np.float32(5e3)).astype(np.float32)
    x[0, :, 0, :8] = np.float32(1e-9) * rng.standard_normal((n, 8)).astype(np.float32)   # deep underflow
    x[1, :, 1, :4] = np.float32(1e6)                   # saturates
    slots = rng.choice(nb * 16, n, replace=False).astype(np.int64)
    slots[::11] = -1
    slots[3::37] = nb * 16 + 5                         # past the pool: skipped
    dev = "cuda"
    kc = torch.zeros((nb, 16, hkv, d), dtype=torch.uint8, device=dev)
    vc = kc.clone()
    pa.pa_reshape_and_cache_fp8(torch.from_numpy(x[0]).to(dev), torch.from_numpy(x[1]).to(dev), kc, vc,
                                torch.from_numpy(slots).to(dev), 0.11, 0.29, fp8_format=FMT)
    torch.cuda.synchronize()
    okc = np.zeros((nb, 16, hkv, d), np.uint8)
    ovc = okc.copy()
    live = (slots >= 0) & (slots < nb * 16)
    oracle.reshape_and_cache_fp8(x[0], x[1], okc, ovc, np.where(live, slots, -1), 0.11, 0.29, fp8_format=FMT)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_fused_slots_and_scatter(pa, src):
    """pa_slot_mapping_and_cache_fp8 in E5M2: slots equal the oracle's, codes
    equal the oracle's scatter through them; padding requests, positions past
    the table and unallocated entries give slot -1 and write nothing."""
    rng = np.random.default_rng(80)
    nb, hkv, d, n, B, width = 40, 8, 128, 160, 6, 8
    table = np.full((B, width), -1, np.int32)
    perm = rng.permutation(nb)
    for b in range(B):
        k = int(rng.integers(1, width))
        table[b, :k] = perm[b * 6:b * 6 + k]
    seq = rng.integers(-1, B + 1, n).astype(np.int32)
    pos = rng.integers(-2, width * 16 + 3, n).astype(np.int32)

    def expected():
        inside = (seq >= 0) & (seq < B) & (pos >= 0) & (pos // 16 < width)
        out = np.full(n, -1, np.int64)
        out[inside] = oracle.slot_mapping(table, seq[inside], pos[inside])
        return out

    seen = set()
    for i, sl in enumerate(expected()):                # distinct valid slots only
        if sl >= 0 and sl in seen:
            seq[i] = -1
        seen.add(int(sl))
    slots_o = expected()
    x = (rng.standard_normal((2, n, hkv, d)) * np.float32(30)).astype(np.float32)
    if src == "bf16":
        host = [W.bf16_bits(x[0]), W.bf16_bits(x[1])]
        dev_rows = [torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).cuda() for h in host]
    else:
        host = [x[0], x[1]]
        dev_rows = [torch.from_numpy(h).cuda() for h in host]
    kc = torch.full((nb, 16, hkv, d), 0x5A, dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    slots = torch.empty(n, dtype=torch.int64, device="cuda")
    pa.pa_slot_mapping_and_cache_fp8(slots, torch.from_numpy(table).cuda(), torch.from_numpy(seq).cuda(),
                                     torch.from_numpy(pos).cuda(), dev_rows[0], dev_rows[1], kc, vc, 0.021, 0.43,
                                     fp8_format=FMT)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), slots_o)
    okc = np.full((nb, 16, hkv, d), 0x5A, np.uint8)
    ovc = okc.copy()
    oracle.reshape_and_cache_fp8(host[0], host[1], okc, ovc, slots_o, 0.021, 0.43, fp8_format=FMT)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


def _decode(staging, w):
    dw = staging.DeviceWorkload(w, kv_fp8=True, fp8_format=FMT)
    dw.scatter_new(fused=True)
    out = dw.decode()
    torch.cuda.synchronize()
    return dw, out


RAGGED = [1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 1000, 1024, 2049, 4095]


def test_decode_ragged_and_cache_bytes(staging):
    w = W.custom("ragged", seq_lens=RAGGED, dtype="bf16", seed=32, sigma=1.0)
    dw, out = _decode(staging, w)
    ks, vs = w.fp8_scales()
    okc, ovc = oracle.build_cache_fp8(w, ks, vs, fp8_format=FMT)
    assert np.array_equal(dw.key_cache.cpu().numpy(), okc)
    assert np.array_equal(dw.value_cache.cpu().numpy(), ovc)
    assert_parity(to_numpy(out), oracle.run_fp8(w, ks, vs, FMT), "bf16", "e5m2 ragged")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (8, 1), (32, 4), (64, 8), (16, 16)])
def test_decode_group_sizes(staging, hq, hkv):
    w = W.custom("gqa", seq_lens=[5, 64, 130, 700], num_heads=hq, num_kv_heads=hkv, dtype="bf16", seed=hq + hkv + 1)
    _, out = _decode(staging, w)
    assert_parity(to_numpy(out), oracle.run_fp8(w, *w.fp8_scales(), FMT), "bf16", f"e5m2 G={hq // hkv} Hkv={hkv}")


@pytest.mark.parametrize("lens", [
    [5000, 3, 0, 17, 4096, 1, 2500],
    [33] * 600,
])
def test_decode_stream_edges(staging, lens):
    w = W.custom("stream", seq_lens=lens, dtype="bf16", seed=len(lens) + 1)
    _, out = _decode(staging, w)
    o = to_numpy(out)
    for b in np.nonzero(np.asarray(lens) == 0)[0]:
        assert np.all(o[b] == 0)
    assert_parity(o, oracle.run_fp8(w, *w.fp8_scales(), FMT), "bf16", f"e5m2 stream {len(lens)} seqs")


def test_decode_wide_range_values(staging):
    """V spread over many binades: N(0,1) times 2^(u - 12), u uniform in
    [-12, 12], stored with v_scale 2^-12, so that the codes (N(0,1) times 2^u)
    use most of E5M2's exponent range, subnormals included, while the values
    and outputs stay below a few units, where the bf16 bar is meant; the
    oracle attends over the same codes."""
    w = W.custom("wide", seq_lens=[300, 1200, 47], dtype="bf16", seed=14, sigma=1.0)
    draw = w.kv
    memo = {}

    def kv(b, length=None):
        if (b, length) not in memo:
            k, v = draw(b, length)
            rng = np.random.default_rng([14, b])
            u = rng.uniform(-12, 12, v.shape).astype(np.float32)
            memo[(b, length)] = (k * np.float32(0.25), W.bf16_round(v * np.exp2(u - 12)))
        return memo[(b, length)]

    w.kv = kv
    w.fp8_scales = lambda: (1.0, 2.0 ** -12)
    dw, out = _decode(staging, w)
    codes = dw.value_cache.cpu().numpy()
    used = codes[codes != 0x7F]
    assert np.any((used & 0x7C) == 0) and np.any((used & 0x7C) >= 0x60)     # subnormals and large exponents
    assert_parity(to_numpy(out), oracle.run_fp8(w, 1.0, 2.0 ** -12, FMT), "bf16", "e5m2 wide range")


def test_decode_full_size(staging):
    """Batch 64 x U[1K, 8K] over an E5M2 cache: the fused scatter's whole
    caches byte for byte against the oracle's, every output row against the
    oracle; out, workspace and caches between guard zones."""
    w = W.llama8b_decode()
    dw = staging.DeviceWorkload(w, kv_fp8=True, guard_bytes=1 << 16, fp8_format=FMT)
    dw.scatter_new(fused=True)
    out = staging.Guarded(dw.query.shape, dw.query.dtype, dw.device)
    ws = staging.Guarded((dw.decode_workspace(0).numel(),), torch.uint8, dw.device, 1 << 16)
    dw.decode(out.t, 0, ws.t)
    torch.cuda.synchronize()
    assert out.intact() and ws.intact() and dw.guards_intact(), "guard zone written"
    okc, ovc = fullsize.oracle_cache(w, fp8=FMT)
    assert fullsize.same_bytes(dw.key_cache, okc), "key cache"
    assert fullsize.same_bytes(dw.value_cache, ovc), "value cache"
    del okc, ovc
    fullsize.assert_rows(out.t, fullsize.oracle_output(w, fp8=FMT), w, "e5m2 llama8b_decode")
