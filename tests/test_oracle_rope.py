"""Pins for the oracle's RoPE + QKV split (CPU only).

What the pages fix ("AI Infra入门干货总结：大模型是如何高效推理的", the RoPE summary
near its opening, section "Reshape & Cache" and its table, and the model table
"附1" for rope_theta): each pair of dimensions is a complex number turned by the
angle position * theta, so <R_m q, R_n k> depends on m - n only; the cos/sin
values come from a [max_position, rotary_dim] table looked up by position; Q,
K and V are consecutive column ranges of the fused projection (4096 | 1024 |
1024 for Llama-3-8B).  The checks below use independent formulations: numpy
complex arithmetic, angles read back with atan2, composition of rotations,
norms, and the relative-position identity.
"""
import numpy as np
import pytest

import oracle

BASE = 500000.0                                       # rope_theta of Llama-3-8B (model table)


def _bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (test-side input encoding)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _table32(max_position, rotary_dim, base=BASE):
    return oracle.rope_table(max_position, rotary_dim, base).astype(np.float32)


def _pairs(rotary_dim, neox):
    i = np.arange(rotary_dim // 2)
    return (i, i + rotary_dim // 2) if neox else (2 * i, 2 * i + 1)


def _complex_reference(x, pos, table, rotary_dim, neox):
    """x [n, H, D] float64; turn each pair, read as the complex number
    x[a] + i x[b], by the unit complex number cos + i sin of its table row."""
    a, b = _pairs(rotary_dim, neox)
    half = rotary_dim // 2
    rows = table[pos].astype(np.float64)
    e = rows[:, None, :half] + 1j * rows[:, None, half:]
    z = (x[..., a] + 1j * x[..., b]) * e
    out = x.copy()
    out[..., a] = z.real
    out[..., b] = z.imag
    return out


def test_table_frequency_schedule():
    """Angles read back from row 1 with atan2: pair 0 turns by exactly one
    radian per position, and successive frequencies fall by the constant
    factor base^(-2/R) down to base^(-(R-2)/R)."""
    R = 128
    t = oracle.rope_table(2, R, BASE)
    theta = np.arctan2(t[1, R // 2:], t[1, :R // 2])
    assert theta[0] == pytest.approx(1.0, abs=1e-15)
    ratio = theta[1:] / theta[:-1]
    np.testing.assert_allclose(ratio, BASE ** (-2.0 / R), rtol=1e-12)
    assert theta[-1] == pytest.approx(BASE ** (-(R - 2) / R), rel=1e-12)
    assert np.array_equal(t[0], np.r_[np.ones(R // 2), np.zeros(R // 2)])


def test_table_angles_add():
    """Row p + q is the composition of rows p and q (angles linear in p)."""
    R = 64
    t = oracle.rope_table(4000, R, BASE)
    h = R // 2
    z = t[:, :h] + 1j * t[:, h:]
    rng = np.random.default_rng(5)
    for p, q in rng.integers(0, 2000, size=(20, 2)):
        np.testing.assert_allclose(z[p] * z[q], z[p + q], atol=1e-9)
    np.testing.assert_allclose(np.abs(z), 1.0, atol=1e-14)


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("rotary_dim", [128, 64])
def test_rotation_matches_complex_multiply(neox, rotary_dim):
    rng = np.random.default_rng(11)
    hq, hkv, d, n = 4, 2, 128, 9
    qkv = rng.standard_normal((n, (hq + 2 * hkv) * d)).astype(np.float32)
    pos = rng.integers(0, 8192, n)
    table = _table32(8192, rotary_dim)
    q, k, v = oracle.rope_qkv(qkv, pos, table, rotary_dim, neox, hq, hkv, d)
    x = qkv.astype(np.float64)
    qx = x[:, :hq * d].reshape(n, hq, d)
    kx = x[:, hq * d:(hq + hkv) * d].reshape(n, hkv, d)
    vx = x[:, (hq + hkv) * d:].reshape(n, hkv, d)
    np.testing.assert_allclose(q, _complex_reference(qx, pos, table, rotary_dim, neox), rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, _complex_reference(kx, pos, table, rotary_dim, neox), rtol=0, atol=1e-12)
    assert np.array_equal(v, vx)
    # dimensions from rotary_dim on pass through untouched
    assert np.array_equal(q[..., rotary_dim:], qx[..., rotary_dim:])


@pytest.mark.parametrize("neox", [True, False])
def test_relative_position(neox):
    """<R_m q, R_n k> = Re(sum_i q_i conj(k_i) e^{i (m - n) theta_i}) and is
    unchanged when both positions shift by the same amount."""
    R, d = 128, 128
    rng = np.random.default_rng(3)
    table = oracle.rope_table(6000, R, BASE)             # fp64 table: the identity is exact up to rounding
    a, b = _pairs(R, neox)
    theta = BASE ** (-2.0 * np.arange(R // 2) / R)
    for _ in range(6):
        qv = rng.standard_normal(d)
        kv = rng.standard_normal(d)
        m, nn, s = (int(x) for x in rng.integers(0, 2000, 3))
        qkv = np.concatenate([qv, kv, np.zeros(d)]).astype(np.float32)[None].repeat(2, 0)
        qx, kx = qkv[0, :d].astype(np.float64), qkv[0, d:2 * d].astype(np.float64)

        def dot(pq, pk):
            q1, _, _ = oracle.rope_qkv(qkv[:1], [pq], table.astype(np.float32), R, neox, 1, 1, d)
            _, k1, _ = oracle.rope_qkv(qkv[:1], [pk], table.astype(np.float32), R, neox, 1, 1, d)
            return float(np.dot(q1.ravel(), k1.ravel()))

        zq = qx[a] + 1j * qx[b]
        zk = kx[a] + 1j * kx[b]
        closed = float(np.real(np.sum(zq * np.conj(zk) * np.exp(1j * (m - nn) * theta))))
        scale = float(np.abs(qx).sum() * np.abs(kx).sum())
        assert dot(m, nn) == pytest.approx(closed, abs=1e-6 * scale)
        assert dot(m + s, nn + s) == pytest.approx(dot(m, nn), abs=1e-6 * scale)


def test_norm_preserved_and_position_zero_is_identity():
    rng = np.random.default_rng(8)
    hq, hkv, d, n = 8, 2, 128, 16
    bits = _bf16_bits(rng.standard_normal((n, (hq + 2 * hkv) * d)))
    pos = np.r_[0, rng.integers(1, 8192, n - 1)]
    table = _table32(8192, 128)
    q, k, _ = oracle.rope_qkv(bits, pos, table, 128, True, hq, hkv, d)
    x = _widen(bits)
    qx = x[:, :hq * d].reshape(n, hq, d)
    a, b = _pairs(128, True)
    # the table is float32, so |cos + i sin| = 1 only to float32 rounding
    np.testing.assert_allclose(np.hypot(q[..., a], q[..., b]), np.hypot(qx[..., a], qx[..., b]),
                               rtol=2e-7, atol=1e-30)
    assert np.array_equal(q[0], qx[0])
    assert np.array_equal(k[0], x[0, hq * d:(hq + hkv) * d].reshape(hkv, d))


def test_column_ranges_follow_the_pages_llama_split():
    """Llama-3-8B: 4096 Q columns, then 1024 K, then 1024 V (6144 in all).  A
    row whose Q, K and V ranges hold different constants shows each range
    read from its own columns."""
    hq, hkv, d = 32, 8, 128
    assert (hq + 2 * hkv) * d == 6144 and hkv * d == 1024
    row = np.r_[np.full(hq * d, 1.0), np.full(hkv * d, 2.0), np.full(hkv * d, 3.0)].astype(np.float32)
    q, k, v = oracle.rope_qkv(row[None], [0], _table32(1, 128), 128, True, hq, hkv, d)
    assert np.all(q == 1.0) and np.all(k == 2.0) and np.all(v == 3.0)


def test_quarter_turn_swaps_pair():
    """A row whose first angle is pi/2 sends (x, y) to (-y, x) in pair 0."""
    R, d = 16, 16
    table = np.zeros((1, R), np.float32)
    table[0, :R // 2] = 1.0
    table[0, 0], table[0, R // 2] = 0.0, 1.0             # cos = 0, sin = 1 for pair 0 only
    x = np.arange(1, 3 * d + 1, dtype=np.float32)[None]
    for neox in (True, False):
        q, _, _ = oracle.rope_qkv(x, [0], table, R, neox, 1, 1, d)
        a, b = _pairs(R, neox)
        assert q[0, 0, a[0]] == -x[0, b[0]] and q[0, 0, b[0]] == x[0, a[0]]
        others = np.setdiff1d(np.arange(d), [a[0], b[0]])
        assert np.array_equal(q[0, 0, others], x[0, others])
