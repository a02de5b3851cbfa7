"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (a value printed on the pages, a library routine, a closed form, an
invariant), so that a plausible slip in it fails here.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- slots --
def test_slot_worked_example():
    """The worked example printed in the 'Paged Attention' section."""
    g = _golden("slot_example.json")
    assert oracle.slot(g["block_table_row"], g["position"], g["block_size"]) == g["slot"]
    sm = oracle.slot_mapping(np.array([g["block_table_row"]]), [0], [g["position"]], g["block_size"])
    assert sm.tolist() == [g["slot"]]


def test_slot_brute_force_bijection():
    """Every position of every request lands in its own table's block at its own
    offset, and no two tokens of the pool share a slot."""
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 90, size=7)
    table = W.deal_block_table(rng, W.blocks_needed(lens), 64)
    seq = np.concatenate([np.full(n, b) for b, n in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    sm = oracle.slot_mapping(table, seq, pos)
    assert len(set(sm.tolist())) == len(sm)
    blocks, offs = np.divmod(sm, 16)
    assert np.array_equal(offs, pos % 16)
    assert np.array_equal(blocks, table[seq, pos // 16])
    # consecutive positions within a block occupy consecutive slots
    same_blk = (pos[1:] // 16 == pos[:-1] // 16) & (seq[1:] == seq[:-1])
    assert np.all(np.diff(sm)[same_blk] == 1)


def test_slot_padding_and_unallocated():
    table = np.array([[3, -1]], np.int32)
    sm = oracle.slot_mapping(table, [0, 0, -1, 0], [5, -1, 3, 20])
    assert sm.tolist() == [3 * 16 + 5, -1, -1, -1]


def test_slot_tiny_config_steps():
    """Tiny config: sequence 0 writes slot 136 in step A and slot 137 in step B."""
    for step, want in (("A", 136), ("B", 137)):
        w = W.tiny(step)
        seq, pos = w.tokens("new")
        sm = oracle.slot_mapping(w.block_table, seq, pos)
        assert sm[0] == want


# ------------------------------------------------------------- scatter --
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scatter_writes_exactly_the_slots(dtype):
    """Rows land at the flat slot index of the [num_blocks*block_size, Hkv, D]
    view (numpy's own layout arithmetic), bit for bit; all other slots keep the
    sentinel; negative slots are skipped; token rows may be strided (the K and V
    column slices of a fused QKV output)."""
    rng = np.random.default_rng(5)
    nb, hkv, d = 9, 4, 128
    store = np.uint16 if dtype == "bf16" else np.float32
    sentinel = (rng.integers(0, 2**16, size=(nb, 16, hkv, d)).astype(np.uint16) if dtype == "bf16"
                else rng.standard_normal((nb, 16, hkv, d)).astype(np.float32))
    kc, vc = sentinel.copy(), sentinel[::-1].copy()
    n = 11
    width = (4 + 2) * hkv * d                     # Q (4 kv widths here) | K | V, as in a fused QKV row
    qkv = (rng.integers(0, 2**16, size=(n, width)).astype(np.uint16) if dtype == "bf16"
           else rng.standard_normal((n, width)).astype(np.float32))
    key = qkv[:, 4 * hkv * d:5 * hkv * d].reshape(n, hkv, d)
    val = qkv[:, 5 * hkv * d:].reshape(n, hkv, d)
    slots = rng.choice(nb * 16, size=n, replace=False).astype(np.int64)
    slots[3] = -1
    slots[7] = -5
    kc0, vc0 = kc.copy(), vc.copy()
    oracle.reshape_and_cache(key, val, kc, vc, slots)
    flat_k, flat_v = kc.reshape(nb * 16, hkv, d), vc.reshape(nb * 16, hkv, d)
    written = slots >= 0
    assert np.array_equal(flat_k[slots[written]].view(np.uint8), key[written].view(np.uint8))
    assert np.array_equal(flat_v[slots[written]].view(np.uint8), val[written].view(np.uint8))
    untouched = np.setdiff1d(np.arange(nb * 16), slots[written])
    assert np.array_equal(flat_k[untouched].view(np.uint8), kc0.reshape(nb * 16, hkv, d)[untouched].view(np.uint8))
    assert np.array_equal(flat_v[untouched].view(np.uint8), vc0.reshape(nb * 16, hkv, d)[untouched].view(np.uint8))
    assert store == kc.dtype


# ----------------------------------------------------------- attention --
def _sdpa_reference(w, b):
    """torch's scaled_dot_product_attention in fp64 on the logical, contiguous
    K/V of sequence b (no paging): a library routine, independent of the
    oracle's gather and softmax.  Causal chunks with earlier context are the
    last query_len rows of a full causal self-attention over the sequence."""
    L, qlen = int(w.seq_lens[b]), int(w.query_lens[b])
    k, v = w.kv(b)
    q = w.query(b)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]      # [1, Hkv, L, D]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]      # [1, Hq, qlen, D]
    if w.causal and qlen > 1:
        qfull = torch.zeros(1, w.num_heads, L, w.head_dim, dtype=torch.float64)
        qfull[:, :, L - qlen:] = qt
        o = torch.nn.functional.scaled_dot_product_attention(
            qfull, kt, vt, is_causal=True, scale=w.scale, enable_gqa=True)[:, :, L - qlen:]
    else:
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=w.scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()                                     # [qlen, Hq, D]


@pytest.mark.parametrize("step", ["A", "B"])
def test_attention_tiny_matches_sdpa(step):
    w = W.tiny(step)
    out = oracle.run(w)
    cu = w.cu_query_lens
    for b in range(w.num_seqs):
        ref = _sdpa_reference(w, b)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 1), (16, 2), (64, 8)])
def test_attention_gqa_shapes_match_sdpa(hq, hkv):
    """MHA (G=1), MQA (one KV head), and grouped shapes."""
    w = W.custom(seq_lens=[1, 17, 33, 48], num_heads=hq, num_kv_heads=hkv, dtype="bf16",
                 seed=7, head_dim=64)
    out = oracle.run(w)
    for b in range(w.num_seqs):
        np.testing.assert_allclose(out[b:b + 1], _sdpa_reference(w, b), rtol=0, atol=1e-12)


def test_causal_chunks_match_sdpa():
    """Chunks with earlier context (query j at position L - qlen + j) and a
    chunk with no earlier context, plus decodes in the same batch."""
    w = W.custom(seq_lens=[40, 37, 16, 9, 70], query_lens=[40, 5, 1, 9, 33], dtype="bf16",
                 seed=9, num_heads=8, num_kv_heads=2, causal=True)
    out = oracle.run(w)
    cu = w.cu_query_lens
    for b in range(w.num_seqs):
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], _sdpa_reference(w, b), rtol=0, atol=1e-12)


def test_decode_is_last_row_of_causal_prefill():
    """A single-token decode at length L equals the last row of a causal
    prefill of the whole sequence."""
    pre = W.custom(seq_lens=[50], query_lens=[50], dtype="f32", seed=3, num_heads=4,
                   num_kv_heads=1, causal=True)
    dec = W.custom(seq_lens=[50], query_lens=[1], dtype="f32", seed=3, num_heads=4,
                   num_kv_heads=1, causal=False)
    dec.block_table = pre.block_table
    dec.num_blocks = pre.num_blocks
    dec.query = lambda b: pre.query(b)[-1:]
    assert np.allclose(oracle.run(pre)[-1:], oracle.run(dec), atol=1e-13, rtol=0)


def test_probability_rows_sum_to_one():
    w = W.tiny("B")
    _, probs = oracle.run(w, return_probs=True)
    for b in range(w.num_seqs):
        L = int(w.seq_lens[b])
        rows = probs[b, :, :L]
        assert np.all(rows >= 0)
        np.testing.assert_allclose(rows.sum(-1), 1.0, atol=1e-12)
        assert np.all(probs[b, :, L:] == 0)


def test_block_permutation_invariance():
    """Relabelling physical blocks (moving the data with them) changes nothing,
    bit for bit."""
    w = W.custom(seq_lens=[30, 64, 5, 100], dtype="bf16", seed=12, num_blocks=40)
    base = oracle.run(w)
    rng = np.random.default_rng(99)
    perm = rng.permutation(64)                              # a bigger pool, new ids
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    moved = w.with_block_table(table, num_blocks=64)
    assert np.array_equal(oracle.run(moved), base)


def test_single_token_returns_its_value_row():
    w = W.custom(seq_lens=[1, 1], dtype="bf16", seed=4)
    out = oracle.run(w)
    for b in range(2):
        _, v = w.kv(b)
        vv = np.repeat(v[0], w.group, axis=0)              # [Hq, D]
        assert np.array_equal(out[b], vv.astype(np.float64))


def test_zero_query_averages_values():
    w = W.custom(seq_lens=[23], dtype="f32", seed=6, num_heads=4, num_kv_heads=2)
    w.query = lambda b: np.zeros((1, 4, 128), np.float32)
    out = oracle.run(w)
    _, v = w.kv(0)
    mean = v.astype(np.float64).mean(axis=0)               # [Hkv, D]
    np.testing.assert_allclose(out[0], np.repeat(mean, 2, axis=0), atol=1e-13)


def test_constant_values_pass_through():
    w = W.custom(seq_lens=[45], dtype="f32", seed=8, num_heads=4, num_kv_heads=4)
    k, v = w.kv(0)
    v[:] = 0.75
    out = oracle.run(w)
    np.testing.assert_allclose(out, 0.75, atol=1e-14)


def test_dominant_key_selects_its_value():
    w = W.custom(seq_lens=[37], dtype="f32", seed=10, num_heads=2, num_kv_heads=1)
    k, v = w.kv(0)
    q = w.query(0)
    k[:] *= 0.01
    k[21, 0] = 40.0 * q[0, 0] / np.linalg.norm(q[0, 0])   # head 0 sees key 21 far above the rest
    out = oracle.run(w)
    np.testing.assert_allclose(out[0, 0], v[21, 0], atol=1e-6)


def test_empty_sequence_outputs_zero():
    w = W.custom(seq_lens=[0, 3], dtype="f32", seed=1, num_heads=4, num_kv_heads=2, width=1)
    out = oracle.run(w)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_poison_never_read():
    """Unwritten slots (NaN) past each sequence's end never reach the output."""
    w = W.custom(seq_lens=[17, 31, 2], dtype="bf16", seed=2)
    assert np.all(np.isfinite(oracle.run(w)))


# --------------------------------------------------------------- bytes --
def test_kv_byte_accounting_matches_pages():
    g = _golden("llama3_8b_kv_bytes.json")
    w = W.custom(seq_lens=[g["context"]], num_heads=32, num_kv_heads=g["num_kv_heads"],
                 head_dim=g["head_dim"], dtype="bf16")
    assert g["num_layers"] * w.kv_bytes() == g["kv_bytes_all_layers"]


def test_copy_blocks_copies_every_layer_and_nothing_else():
    """Copy-on-write: block dst of every layer's K and V equals block src
    afterwards, byte for byte; every other block is untouched; a pair outside
    the pool does nothing; pairs apply in order (a later pair sees an earlier
    copy)."""
    rng = np.random.default_rng(0)
    kv = rng.integers(0, 1 << 16, size=(3, 2, 10, 16, 2, 8), dtype=np.uint16)
    before = kv.copy()
    pairs = np.array([[1, 4], [7, 2], [4, 9], [3, 10], [-1, 5]], np.int64)
    oracle.copy_blocks(kv, pairs)
    want = before.copy()
    want[:, :, 4] = before[:, :, 1]
    want[:, :, 2] = before[:, :, 7]
    want[:, :, 9] = before[:, :, 1]                    # via block 4, already a copy of 1
    assert np.array_equal(kv, want)
