"""The seeded input generators: determinism, encodings and the stated recipe."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00781250, 3.0e-39], np.float32)])
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draws_are_deterministic_and_prefix_consistent():
    a, b = W.tiny("A"), W.tiny("B")
    for s in range(4):
        ka, va = a.kv(s)
        kb, vb = b.kv(s)
        assert np.array_equal(ka, kb[:len(ka)]) and np.array_equal(va, vb[:len(va)])
    assert np.array_equal(W.llama8b_decode().seq_lens, W.llama8b_decode().seq_lens)


def test_tiny_layout():
    w = W.tiny("B")
    assert w.block_table[0, :3].tolist() == [5, 8, 12]
    assert w.seq_lens.tolist() == [26, 41, 8, 65]
    used = w.block_table[w.block_table >= 0]
    assert len(set(used.tolist())) == len(used) and used.max() < 32
    assert (w.block_table >= 0).sum(1).tolist() == [3, 3, 1, 5]
    assert W.tiny("A").seq_lens.tolist() == [25, 40, 7, 64]


def test_config_shapes():
    c1 = W.llama8b_decode()
    assert c1.num_seqs == 64 and c1.seq_lens.min() >= 1024 and c1.seq_lens.max() <= 8192
    assert c1.num_blocks == int(np.ceil(1.1 * W.blocks_needed(c1.seq_lens).sum()))
    assert c1.dtype == "bf16" and c1.sigma == 0.5 and c1.group == 4
    c2 = W.long_context()
    assert c2.num_blocks == 40000 and np.all(c2.seq_lens == 32768)
    c3 = W.continuous_batching()
    assert c3.num_heads == 64 and c3.num_seqs == 256
    assert 16 <= c3.seq_lens.min() and c3.seq_lens.max() <= 16384
    assert 600 < np.median(c3.seq_lens) < 1300
    c4 = W.chunked_prefill_mix()
    assert c4.num_q_tokens == 4 * 512 + 96 and c4.causal
    assert c4.seq_lens[:4].tolist() == [512, 2560, 4608, 8192]
    for w in (c1, c2, c3, c4):
        used = w.block_table[w.block_table >= 0]
        assert len(np.unique(used)) == len(used) and used.max() < w.num_blocks
        assert np.array_equal((w.block_table >= 0).sum(1), W.blocks_needed(w.seq_lens))


def test_token_lists():
    w = W.chunked_prefill_mix()
    seq, pos = w.tokens("new")
    assert len(seq) == w.num_q_tokens
    assert pos[:512].tolist() == list(range(0, 512))
    assert pos[512:1024].tolist() == list(range(2048, 2560))
    assert np.all(pos[2048:] == w.seq_lens[4:] - 1)
