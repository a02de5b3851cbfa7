"""The step before attention on the GPU: QKV split + RoPE + scatter
(pa_rope_reshape_and_cache) against the oracle's fp64 definition.

Bar: V and every cache byte the call must not touch are bit-exact; each
turned Q/K element is within half a unit in the last place of the storage
dtype of the exact (fp64) value, plus the fp32 rounding of the two products
that make it, 2^-22 (|x_a| + |x_b|) for the pair (x_a, x_b).  That is, the
result is the exact value rounded to nearest unless the exact value lies
within fp32 arithmetic error of a rounding midpoint.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import storage_bits

pytestmark = pytest.mark.gpu
D = 128
BASE = 500000.0


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_432_amd as pa
    pa.lib()
    return pa


def _store(t):
    """torch CPU tensor -> numpy storage (uint16 bf16 bits or float32)."""
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _ulp(v, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - (7 if dtype == torch.bfloat16 else 23))


def _pair_mag(x, rotary_dim, neox):
    """|x_a| + |x_b| for both members of each turned pair, 0 past rotary_dim."""
    i = np.arange(rotary_dim // 2)
    a, b = (i, i + rotary_dim // 2) if neox else (2 * i, 2 * i + 1)
    m = np.zeros_like(x)
    s = np.abs(x[..., a]) + np.abs(x[..., b])
    m[..., a] = s
    m[..., b] = s
    return m


def _check_turned(got, exact, x, rotary_dim, neox, dtype, what):
    got = got.astype(np.float64)
    tol = 0.5 * _ulp(np.maximum(np.abs(exact), np.abs(got)), dtype) + 2.0 ** -22 * _pair_mag(x, rotary_dim, neox)
    err = np.abs(got - exact)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements off, worst err {err.max():.3g}; "
                           f"first at {np.argwhere(bad)[0].tolist()}")
    # dimensions past rotary_dim are copied, so exact
    assert np.array_equal(got[..., rotary_dim:], exact[..., rotary_dim:]), what


def _run(pa, n, hq, hkv, dtype, neox, rotary_dim, seed, nb=64, max_position=8192, positions=None,
         in_place=False, extra_cols=16):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    width = (hq + 2 * hkv) * D
    qkv_full = torch.randn(n, width + extra_cols, generator=g).to(dtype)
    qkv = qkv_full[:, :width + extra_cols]                 # row stride > width
    if positions is None:
        positions = rng.integers(0, max_position, n)
    positions = np.asarray(positions, np.int64)
    slots = rng.choice(nb * 16, size=n, replace=False).astype(np.int64) if n <= nb * 16 else \
        rng.integers(0, nb * 16, n).astype(np.int64)
    if n:
        slots[::13] = -1                                   # padding tokens
        slots[5::29] = nb * 16 + 3                         # past the pool: skipped too
    table = oracle.rope_table(max_position, rotary_dim, BASE).astype(np.float32)
    sentinel = torch.randn(nb, 16, hkv, D, generator=torch.Generator().manual_seed(seed + 1)).to(dtype)

    dev = "cuda"
    qkv_d = qkv.to(dev)
    kc, vc = sentinel.clone().to(dev), (-sentinel).to(dev)
    if in_place:
        qout = qkv_d[:, :hq * D].view(n, hq, D)
    else:
        qout_full = torch.full((n, hq * D + 64), float("nan"), dtype=dtype, device=dev)
        qout = qout_full[:, :hq * D].view(n, hq, D)       # token stride hq * D + 64
    pa.pa_rope_reshape_and_cache(qout, qkv_d, torch.from_numpy(positions).to(dev),
                                 torch.from_numpy(table).to(dev), kc, vc, torch.from_numpy(slots).to(dev),
                                 hq, hkv, neox_style=neox)
    torch.cuda.synchronize()

    # oracle on the same storage; out-of-table positions are the caller's
    # contract, and the library clamps them into the table
    x = _store(qkv)
    pos_c = np.clip(positions, 0, max_position - 1)
    q_ex, k_ex, v_ex = oracle.rope_qkv(x, pos_c, table, rotary_dim, neox, hq, hkv, D)
    xw = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if dtype == torch.bfloat16 \
        else x.astype(np.float64)
    qx = xw[:, :hq * D].reshape(n, hq, D)
    kx = xw[:, hq * D:(hq + hkv) * D].reshape(n, hkv, D)

    got_q = qout.float().cpu().numpy()
    _check_turned(got_q, q_ex, qx, rotary_dim, neox, dtype, "query_out")

    kcache = kc.float().cpu().numpy().reshape(nb * 16, hkv, D)
    vbits = storage_bits(vc)
    live = (slots >= 0) & (slots < nb * 16)
    _check_turned(kcache[slots[live]], k_ex[live], kx[live], rotary_dim, neox, dtype, "key_cache")
    # every other K slot keeps the sentinel, bit for bit
    untouched = np.setdiff1d(np.arange(nb * 16), slots[live])
    kbits = storage_bits(kc).view(np.uint8).reshape(nb * 16, -1)
    sbits = _store(sentinel).view(np.uint8).reshape(nb * 16, -1)
    assert np.array_equal(kbits[untouched], sbits[untouched])
    # V: the oracle's scatter of the V columns, whole cache bit-exact (the
    # oracle scatters every slot >= 0, so past-the-pool slots go in as padding)
    ovc = _store(-sentinel).copy()
    vcols = x[:, (hq + hkv) * D:width].reshape(n, hkv, D)
    oracle.reshape_and_cache(vcols, vcols, _store(sentinel).copy(), ovc, np.where(live, slots, -1))
    assert np.array_equal(vbits.view(np.uint8), ovc.view(np.uint8))
    assert np.allclose(v_ex, xw[:, (hq + hkv) * D:width].reshape(n, hkv, D))
    if in_place:
        # K and V columns (and the padding columns) of the projection are untouched
        after = _store(qkv_d.cpu())
        assert np.array_equal(after[:, hq * D:], x[:, hq * D:])
    return got_q


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("neox", [True, False], ids=["halves", "neighbours"])
@pytest.mark.parametrize("rotary_dim", [128, 64, 16])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (64, 8), (4, 1)])
def test_rope_cache_matches_oracle(pa, dtype, neox, rotary_dim, hq, hkv):
    _run(pa, 300, hq, hkv, dtype, neox, rotary_dim, seed=hq * 7 + rotary_dim + int(neox))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_rope_in_place(pa, dtype):
    _run(pa, 200, 32, 8, dtype, True, 128, seed=4, in_place=True, extra_cols=0)


def test_rope_positions_clamped_into_table(pa):
    pos = [-5, 0, 1, 8191, 8192, 100000, 77]
    _run(pa, len(pos), 32, 8, torch.bfloat16, True, 128, seed=6, positions=pos)


def test_rope_position_zero_is_a_plain_copy(pa):
    """Row 0 of the table is cos 1, sin 0: Q comes out bit for bit as it went in."""
    got = _run(pa, 40, 32, 8, torch.bfloat16, True, 128, seed=9, positions=np.zeros(40, np.int64),
               extra_cols=0)
    q_in = torch.randn(40, 48 * D, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    assert np.array_equal(got, q_in[:, :32 * D].float().numpy().reshape(40, 32, D))


def test_rope_llama_mixed_batch_size(pa):
    """2144 new tokens (four 512-token prefill chunks + 96 decodes) of the
    Llama-3-8B projection, 6144 columns, into a pool of 2200 blocks."""
    _run(pa, 2144, 32, 8, torch.bfloat16, True, 128, seed=12, nb=2200, extra_cols=0)


def test_rope_empty(pa):
    dev = "cuda"
    q = torch.empty(0, 32, D, dtype=torch.bfloat16, device=dev)
    pa.pa_rope_reshape_and_cache(q, torch.empty(0, 6144, dtype=torch.bfloat16, device=dev),
                                 torch.empty(0, dtype=torch.int64, device=dev),
                                 torch.zeros(16, 128, dtype=torch.float32, device=dev),
                                 torch.zeros(4, 16, 8, D, dtype=torch.bfloat16, device=dev),
                                 torch.zeros(4, 16, 8, D, dtype=torch.bfloat16, device=dev),
                                 torch.empty(0, dtype=torch.int64, device=dev), 32, 8)


def test_rope_graph_replays_match_eager(pa):
    """The call captured in a graph (as the timing harness runs it) gives, on
    every replay with fresh inputs copied in between, what an eager call on
    the same inputs gives."""
    dev = "cuda"
    hq, hkv, n, nb = 32, 8, 96, 16
    table = torch.from_numpy(oracle.rope_table(4096, 128, BASE).astype(np.float32)).to(dev)
    qkv = torch.empty(n, (hq + 2 * hkv) * D, dtype=torch.bfloat16, device=dev)
    pos = torch.empty(n, dtype=torch.int64, device=dev)
    slots = torch.empty(n, dtype=torch.int64, device=dev)
    qout = torch.empty(n, hq, D, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(nb, 16, hkv, D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)

    def call(q_o, k_c, v_c):
        pa.pa_rope_reshape_and_cache(q_o, qkv, pos, table, k_c, v_c, slots, hq, hkv)

    def fill(seed):
        g = torch.Generator().manual_seed(seed)
        qkv.copy_(torch.randn(n, (hq + 2 * hkv) * D, generator=g).to(torch.bfloat16))
        pos.copy_(torch.randint(0, 4096, (n,), generator=g))
        slots.copy_(torch.randperm(nb * 16, generator=g)[:n])

    fill(0)
    call(qout, kc, vc)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call(qout, kc, vc)
    torch.cuda.current_stream().wait_stream(side)
    for seed in (1, 2, 3):
        fill(seed)
        torch.cuda.synchronize()
        q_e = torch.empty_like(qout)
        k_e, v_e = kc.clone(), vc.clone()
        call(q_e, k_e, v_e)                            # eager, same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(qout.view(torch.int16), q_e.view(torch.int16)), seed
        assert torch.equal(kc.view(torch.int16), k_e.view(torch.int16)), seed
        assert torch.equal(vc.view(torch.int16), v_e.view(torch.int16)), seed


def test_rope_scatter_then_decode_matches_oracle(pa):
    """The input side end to end: a Llama-3-8B-shaped decode step whose 8 new
    tokens come out of one fused projection row each.  pa_rope_reshape_and_cache
    turns Q and K and scatters K, V next to the 8 sequences' earlier context;
    pa_decode attends with the turned Q.  The oracle turns the same rows in
    fp64 (rounded to bf16, as stored), writes them into its own cache and
    attends: the bf16 bar."""
    import workloads as W
    dev = "cuda"
    rng = np.random.default_rng(17)
    hq, hkv, B = 32, 8, 8
    lens = rng.integers(20, 700, B).astype(np.int32)
    w = W.custom("rope_decode", seq_lens=lens, dtype="bf16", seed=17, sigma=1.0)
    table = oracle.rope_table(1024, 128, BASE).astype(np.float32)
    # earlier context through the library's plain scatter, the new token through the fused one
    kc = torch.full((w.num_blocks, 16, hkv, D), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    okc, okv = w.poisoned_cache(), w.poisoned_cache()
    seq_h, pos_h = w.tokens("history")
    slots_h = oracle.slot_mapping(w.block_table, seq_h, pos_h)
    kh, vh = w.token_kv(seq_h, pos_h)
    pa.pa_reshape_and_cache(torch.from_numpy(kh).to(dev).to(torch.bfloat16),
                            torch.from_numpy(vh).to(dev).to(torch.bfloat16), kc, vc,
                            torch.from_numpy(slots_h).to(dev))
    oracle.reshape_and_cache(w.encode(kh), w.encode(vh), okc, okv, slots_h)
    seq_n, pos_n = w.tokens("new")
    slots_n = oracle.slot_mapping(w.block_table, seq_n, pos_n)
    qkv = W.bf16_round(rng.standard_normal((B, (hq + 2 * hkv) * D), dtype=np.float32))
    qkv_bits = W.bf16_bits(qkv)
    q_d = torch.empty(B, hq, D, dtype=torch.bfloat16, device=dev)
    pa.pa_rope_reshape_and_cache(q_d, torch.from_numpy(qkv).to(dev).to(torch.bfloat16),
                                 torch.from_numpy(pos_n.astype(np.int64)).to(dev), torch.from_numpy(table).to(dev),
                                 kc, vc, torch.from_numpy(slots_n).to(dev), hq, hkv)
    out = torch.empty_like(q_d)
    ws = pa.decode_workspace(B, hq, hkv, D, int(lens.max()), 0)
    pa.pa_decode(out, q_d, kc, vc, torch.from_numpy(w.block_table).to(dev),
                 torch.from_numpy(lens).to(dev), w.scale, int(lens.max()), 0, ws)
    torch.cuda.synchronize()
    # oracle: the same rows turned in fp64, stored as bf16, then attention
    q_ex, k_ex, v_ex = oracle.rope_qkv(qkv_bits, pos_n, table, 128, True, hq, hkv, D)
    oracle.reshape_and_cache(W.bf16_bits(k_ex.astype(np.float32)), W.bf16_bits(v_ex.astype(np.float32)),
                             okc, okv, slots_n)
    cu = np.arange(B + 1, dtype=np.int32)
    ref = oracle.attention(W.bf16_bits(q_ex.astype(np.float32)), okc, okv, w.block_table, cu, lens, hq, w.scale,
                           False)
    from parity import assert_parity, to_numpy
    assert_parity(to_numpy(out), ref, "bf16", "RoPE scatter then decode")
