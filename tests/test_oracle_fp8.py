"""Pins for the oracle's fp8 (OCP E4M3 and E5M2) KV cache (CPU only).

The pages fix only that fewer bits per KV entry mean proportionally fewer bytes
per decoded token, and that e4m3 and e5m2 are both in use; the format itself is
its published definition (OCP 8-bit floating point: E4M3 with bias 7, 3
mantissa bits, subnormals m * 2^-9, S.1111.111 NaN, no infinity, largest 448).
E5M2, the other format the pages name, has bias 15, 2 mantissa bits,
subnormals m * 2^-16, infinity at S.11111.00, NaN at S.11111.{01,10,11}, and
largest finite 57344; the oracle saturates magnitudes beyond it (infinity
included) to 57344, as for E4M3, so that a stored code is always finite.
Independent references: the specification's landmark values, torch's own
float8_e4m3fn / float8_e5m2 conversions (library routines, in range, where
they round to nearest even), and the float-cache attention path, already pinned
against scaled_dot_product_attention.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _torch_codes(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_landmark_values():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9                       # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9                   # largest subnormal
    assert v(0x08) == 2.0 ** -6                       # smallest normal
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x3C) == 1.5
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0     # largest finite
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x77) == 240.0 and v(0x78) == 256.0


def test_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    ours = np.array([oracle.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_encode_matches_torch_in_range():
    """Every bf16 value below 464 in magnitude, every midpoint between
    neighbouring codes, and random float32 values: the oracle's code equals
    torch's."""
    bf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) < 464)]
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    rnd = np.random.default_rng(2).standard_normal(20000).astype(np.float32) * np.float32(40)
    y = np.concatenate([bf, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
                        rnd])
    y = y[np.abs(y) < 464]
    assert np.array_equal(oracle.e4m3_encode(y), _torch_codes(y))


def test_encode_ties_go_to_even_mantissa():
    v = oracle.e4m3_value
    for c in range(0x7E):
        mid = np.float32((v(c) + v(c + 1)) / 2)
        got = int(oracle.e4m3_encode(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), hex(c)


def test_encode_round_trip_and_saturation():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert int(oracle.e4m3_encode(np.array([oracle.e4m3_value(c)], np.float32))[0]) == c
    sat = oracle.e4m3_encode(np.array([448, 464, 1e30, np.inf, -500, -np.inf], np.float32))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_fp8_scatter(src):
    rng = np.random.default_rng(3)
    n, hkv, d, nb = 40, 2, 128, 8
    x = (rng.standard_normal((n, 2, hkv, d)) * 3).astype(np.float32)
    store = (lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)) if src == "bf16" else (lambda a: a)
    widen = (lambda a: (a.astype(np.uint32) << 16).view(np.float32)) if src == "bf16" else (lambda a: a)
    k, v = store(np.ascontiguousarray(x[:, 0])), store(np.ascontiguousarray(x[:, 1]))
    slots = rng.choice(nb * 16, n, replace=False).astype(np.int64)
    slots[::7] = -1
    kc = np.full((nb, 16, hkv, d), 0x55, np.uint8)
    vc = kc.copy()
    ks, vs = np.float32(0.37), np.float32(1.9)
    oracle.reshape_and_cache_fp8(k, v, kc, vc, slots, ks, vs)
    live = slots >= 0
    flat_k, flat_v = kc.reshape(nb * 16, hkv, d), vc.reshape(nb * 16, hkv, d)
    assert np.array_equal(flat_k[slots[live]], _torch_codes(widen(k)[live] / ks))
    assert np.array_equal(flat_v[slots[live]], _torch_codes(widen(v)[live] / vs))
    rest = np.setdiff1d(np.arange(nb * 16), slots[live])
    assert np.all(flat_k[rest] == 0x55) and np.all(flat_v[rest] == 0x55)


@pytest.mark.parametrize("scales", [(0.25, 2.0), (0.37, 1.9)])
def test_attention_over_fp8_is_attention_over_decoded_values(scales):
    """The fp8 cache attends like a float32 cache holding code value * scale.
    Power-of-two scales make that float32 cache exact, and the two results
    are then identical; other scales agree to float32 rounding of the cache."""
    ks, vs = scales
    w = W.tiny("B")
    kc, vc = oracle.build_cache(w, "all")               # float32 cache of the tiny workload
    rng = np.random.default_rng(4)
    codes_k = rng.integers(0, 256, kc.shape).astype(np.uint8)
    codes_v = rng.integers(0, 256, vc.shape).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x38           # no NaN codes
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x38
    table = np.array([oracle.e4m3_value(c) for c in range(256)])
    fk = (table[codes_k] * ks).astype(np.float32)
    fv = (table[codes_v] * vs).astype(np.float32)
    q = w.encode(w.queries())
    args = (w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads, w.scale, w.causal)
    got = oracle.attention(q, codes_k, codes_v, *args, k_scale=ks, v_scale=vs)
    ref = oracle.attention(q, fk, fv, *args)
    if ks == 0.25:
        assert np.array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


# ------------------------------------------------------------------ E5M2 --
def _torch_codes_e5m2(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_landmark_values():
    v = oracle.e5m2_value
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -16                      # smallest subnormal
    assert v(0x03) == 3 * 2.0 ** -16                  # largest subnormal
    assert v(0x04) == 2.0 ** -14                      # smallest normal
    assert v(0x3C) == 1.0 and v(0x3D) == 1.25 and v(0x3E) == 1.5 and v(0x3F) == 1.75 and v(0x40) == 2.0
    assert v(0x7B) == 57344.0 and v(0xFB) == -57344.0  # largest finite
    assert v(0x7C) == np.inf and v(0xFC) == -np.inf
    assert all(np.isnan(v(c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))


def test_e5m2_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).float().numpy().astype(np.float64)
    ours = np.array([oracle.e5m2_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e5m2_encode_matches_torch_in_range():
    """Every bf16 value below 61440 in magnitude (the rounding boundary above
    the largest code), every midpoint between neighbouring codes with its two
    float32 neighbours, and random float32 values: the oracle's code equals
    torch's."""
    bf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) < 61440)]
    vals = np.array([oracle.e5m2_value(c) for c in range(0x7C)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    rnd = np.random.default_rng(12).standard_normal(20000).astype(np.float32) * np.float32(3000)
    y = np.concatenate([bf, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(7e4)),
                        rnd])
    y = y[np.abs(y) < 61440]
    assert np.array_equal(oracle.e5m2_encode(y), _torch_codes_e5m2(y))


def test_e5m2_encode_ties_go_to_even_mantissa():
    v = oracle.e5m2_value
    for c in range(0x7B):
        mid = np.float32((v(c) + v(c + 1)) / 2)
        got = int(oracle.e5m2_encode(np.array([mid]))[0])
        assert got == (c if c % 2 == 0 else c + 1), hex(c)


def test_e5m2_encode_round_trip_and_saturation():
    for c in range(256):
        if (c & 0x7F) >= 0x7C:
            continue
        assert int(oracle.e5m2_encode(np.array([oracle.e5m2_value(c)], np.float32))[0]) == c
    sat = oracle.e5m2_encode(np.array([57344, 61440, 1e30, np.inf, -6e4, -np.inf], np.float32))
    assert sat.tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB]
    nan = int(oracle.e5m2_encode(np.array([np.nan], np.float32))[0])
    assert np.isnan(oracle.e5m2_value(nan))


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_e5m2_scatter(src):
    rng = np.random.default_rng(13)
    n, hkv, d, nb = 40, 2, 128, 8
    x = (rng.standard_normal((n, 2, hkv, d)) * 3).astype(np.float32)
    store = (lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)) if src == "bf16" else (lambda a: a)
    widen = (lambda a: (a.astype(np.uint32) << 16).view(np.float32)) if src == "bf16" else (lambda a: a)
    k, v = store(np.ascontiguousarray(x[:, 0])), store(np.ascontiguousarray(x[:, 1]))
    slots = rng.choice(nb * 16, n, replace=False).astype(np.int64)
    slots[::7] = -1
    kc = np.full((nb, 16, hkv, d), 0x55, np.uint8)
    vc = kc.copy()
    ks, vs = np.float32(0.0037), np.float32(1.9)
    oracle.reshape_and_cache_fp8(k, v, kc, vc, slots, ks, vs, fp8_format="e5m2")
    live = slots >= 0
    flat_k, flat_v = kc.reshape(nb * 16, hkv, d), vc.reshape(nb * 16, hkv, d)
    assert np.array_equal(flat_k[slots[live]], _torch_codes_e5m2(widen(k)[live] / ks))
    assert np.array_equal(flat_v[slots[live]], _torch_codes_e5m2(widen(v)[live] / vs))
    rest = np.setdiff1d(np.arange(nb * 16), slots[live])
    assert np.all(flat_k[rest] == 0x55) and np.all(flat_v[rest] == 0x55)


@pytest.mark.parametrize("scales", [(0.25, 2.0), (0.37, 1.9)])
def test_attention_over_e5m2_is_attention_over_decoded_values(scales):
    ks, vs = scales
    w = W.tiny("B")
    kc, vc = oracle.build_cache(w, "all")
    rng = np.random.default_rng(14)
    codes_k = rng.integers(0, 256, kc.shape).astype(np.uint8)
    codes_v = rng.integers(0, 256, vc.shape).astype(np.uint8)
    codes_k[(codes_k & 0x7F) >= 0x7C] = 0x3C           # no infinity or NaN codes
    codes_v[(codes_v & 0x7F) >= 0x7C] = 0x3C
    codes_k[(codes_k & 0x7F) >= 0x50] &= 0xCF          # keep scores moderate: magnitudes below 2^5
    table = np.array([oracle.e5m2_value(c) for c in range(256)])
    fk = (table[codes_k] * ks).astype(np.float32)
    fv = (table[codes_v] * vs).astype(np.float32)
    q = w.encode(w.queries())
    args = (w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads, w.scale, w.causal)
    got = oracle.attention(q, codes_k, codes_v, *args, k_scale=ks, v_scale=vs, fp8_format="e5m2")
    ref = oracle.attention(q, fk, fv, *args)
    if ks == 0.25:
        assert np.array_equal(got, ref)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    assert not np.array_equal(got, oracle.attention(q, codes_k, codes_v, *args, k_scale=ks, v_scale=vs))
