"""Seeded synthetic inputs for paged KV-cache attention.

This module is shared by the tests, the benchmark and the smoke check, on both
sides of the comparison (the CPU oracle and the HIP library).  It only *draws*
inputs: sequence lengths, physical block tables dealt from a pool, the list of
(sequence, position) pairs a step writes, and Q/K/V values.  It holds none of
the method's arithmetic: no slot computation, no gather, no softmax.  Each side
derives slots, caches and outputs from these inputs on its own.

Shapes follow the Llama-3-8B figures of "AI Infra入门干货总结：大模型是如何高效推理的"
(appendix 1, model configuration table: 32 query heads, 8 KV heads, head_dim 128)
and the default block size of 16 tokens from its "Paged Attention" section.

Value recipe (documented once here, used everywhere):
  * lengths and block tables come from ``numpy.random.default_rng(seed)``;
  * K and V of sequence ``b`` are one float32 standard-normal stream each,
    ``default_rng([seed, 1, b])`` for K and ``default_rng([seed, 2, b])`` for V,
    drawn position-major as ``[L_b, Hkv, D]`` and multiplied by ``sigma``; a
    shorter draw is a prefix of a longer one, so a later step extends an earlier
    one;
  * Q of sequence ``b`` at history length ``h`` is ``default_rng([seed, 3, b, h])``;
  * bf16 values are the float32 draw rounded to nearest-even.
"""
from __future__ import annotations

import math
import os
from collections import deque
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
BF16_NAN_BITS = 0x7FC0


# ------------------------------------------------------------ parallel draws --
def draw_threads() -> int:
    """Threads for drawing values: the OpenMP share of the job if one is set,
    else the CPUs this process may run on (at most 16)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def prefetch_map(fn, items, threads: int | None = None, depth: int | None = None):
    """Yield fn(item) for each item, in order, computed on a thread pool at most
    `depth` items ahead of the consumer (numpy's generators and array
    arithmetic release the GIL, so the draws of different sequences overlap).
    The bounded look-ahead keeps only a few sequences' values in memory."""
    items = list(items)
    threads = threads or draw_threads()
    depth = depth or 2 * threads
    if threads <= 1 or len(items) <= 1:
        for it in items:
            yield fn(it)
        return
    with ThreadPoolExecutor(threads) as ex:
        pending = deque()
        nxt = 0
        while nxt < len(items) and len(pending) < depth:
            pending.append(ex.submit(fn, items[nxt]))
            nxt += 1
        while pending:
            res = pending.popleft().result()
            if nxt < len(items):
                pending.append(ex.submit(fn, items[nxt]))
                nxt += 1
            yield res


# ---------------------------------------------------------------- encodings --
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Input encoding only; inputs here are finite and far from overflow.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(x))


# ---------------------------------------------------------------- workload --
@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "bf16" or "f32"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    seq_lens: np.ndarray            # int32 [B]: KV tokens attended, this step's tokens included
    query_lens: np.ndarray          # int32 [B]: tokens this step computes (1 for a decode)
    causal: bool
    num_blocks: int
    block_table: np.ndarray         # int32 [B, max_blocks_per_req], -1 where unused
    sigma: float = 1.0
    block_size: int = BLOCK_SIZE
    notes: str = ""
    _kv_cache: dict = field(default_factory=dict, repr=False)

    # ---- sizes
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_req(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim) as the float32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def history_lens(self) -> np.ndarray:
        # a padding sequence (seq_len 0 with one query row) has no history
        return np.maximum(self.seq_lens - self.query_lens, 0).astype(np.int32)

    @property
    def cu_query_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.query_lens)
        return cu

    @property
    def num_q_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.query_lens == 1))

    def fp8_scales(self):
        """(k_scale, v_scale) for an fp8 (E4M3) cache of this workload: sigma / 64,
        so that values up to 7 sigma are representable (E4M3 reaches 448) and
        values near sigma sit in the normal range."""
        s = float(np.float32(self.sigma) / np.float32(64))
        return s, s

    def kv_bytes(self, elem_bytes: int | None = None) -> int:
        """Algorithmic KV bytes one attention call reads: each attended token's
        K and V row for every KV head, counted once (grouped query heads share it)."""
        eb = self.elem_bytes if elem_bytes is None else elem_bytes
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * eb

    # ---- values
    def _round(self, x: np.ndarray) -> np.ndarray:
        return bf16_round(x) if self.dtype == "bf16" else x.astype(np.float32)

    def kv(self, b: int, length: int | None = None):
        """K and V of sequence b for positions [0, length): float32 [length, Hkv, D],
        already rounded to the workload dtype."""
        n = int(self.seq_lens[b]) if length is None else int(length)
        key = (b, n)
        if key in self._kv_cache:
            return self._kv_cache[key]
        shape = (n, self.num_kv_heads, self.head_dim)
        rk = np.random.default_rng([self.seed, 1, b])
        rv = np.random.default_rng([self.seed, 2, b])
        k = self._round(np.float32(self.sigma) * rk.standard_normal(shape, dtype=np.float32))
        v = self._round(np.float32(self.sigma) * rv.standard_normal(shape, dtype=np.float32))
        if n * self.num_kv_heads * self.head_dim <= (1 << 22):   # memoise small draws only
            self._kv_cache[key] = (k, v)
        return k, v

    def iter_kv(self, seqs=None, encode: bool = False):
        """Yield (b, k, v) for each sequence b of `seqs` (default: all), in order,
        with each sequence's K and V as kv(b) draws them (or their storage
        encoding if `encode`), drawn a few sequences ahead on worker threads."""
        seqs = range(self.num_seqs) if seqs is None else [int(b) for b in seqs]

        def one(b):
            k, v = self.kv(b)
            return (b, self.encode(k), self.encode(v)) if encode else (b, k, v)

        yield from prefetch_map(one, seqs)

    def query(self, b: int) -> np.ndarray:
        """Q rows of sequence b for this step: float32 [query_len_b, Hq, D]."""
        h = int(self.history_lens[b])
        r = np.random.default_rng([self.seed, 3, b, h])
        shape = (int(self.query_lens[b]), self.num_heads, self.head_dim)
        return self._round(np.float32(self.sigma) * r.standard_normal(shape, dtype=np.float32))

    def queries(self) -> np.ndarray:
        """All of this step's Q rows, flattened in sequence order: [num_q_tokens, Hq, D]."""
        if self.num_q_tokens == 0:
            return np.zeros((0, self.num_heads, self.head_dim), np.float32)
        return np.concatenate([self.query(b) for b in range(self.num_seqs)], axis=0)

    # ---- token lists
    def tokens(self, which: str = "new"):
        """(seq, pos) int32 arrays of the tokens to write.

        which = "new": this step's tokens (positions history_len .. seq_len-1);
                "history": the earlier context, written before the step;
                "all": both, history first.
        """
        seqs, poss = [], []
        for b in range(self.num_seqs):
            h, n = int(self.history_lens[b]), int(self.seq_lens[b])
            lo, hi = {"new": (h, n), "history": (0, h), "all": (0, n)}[which]
            seqs.append(np.full(hi - lo, b, np.int32))
            poss.append(np.arange(lo, hi, dtype=np.int32))
        if not seqs:
            return np.zeros(0, np.int32), np.zeros(0, np.int32)
        return np.concatenate(seqs), np.concatenate(poss)

    def token_kv(self, seq: np.ndarray, pos: np.ndarray):
        """K and V rows for a token list, in list order: float32 [n, Hkv, D] each."""
        n = len(seq)
        k = np.empty((n, self.num_kv_heads, self.head_dim), np.float32)
        v = np.empty_like(k)
        seq = np.asarray(seq)
        pos = np.asarray(pos)
        for b, kb, vb in self.iter_kv(np.unique(seq)):
            idx = np.nonzero(seq == b)[0]
            k[idx] = kb[pos[idx]]
            v[idx] = vb[pos[idx]]
        return k, v

    def encode(self, x: np.ndarray) -> np.ndarray:
        """Float32 values -> the storage the kernels and the oracle read
        (uint16 bf16 bit patterns, or float32)."""
        return bf16_bits(x) if self.dtype == "bf16" else np.ascontiguousarray(x, np.float32)

    def poisoned_cache(self) -> np.ndarray:
        """A cache pool [num_blocks, block_size, Hkv, D] in storage format, every
        element NaN, so that a read of an unwritten slot shows in the result."""
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if self.dtype == "bf16":
            return np.full(shape, BF16_NAN_BITS, np.uint16)
        return np.full(shape, np.nan, np.float32)

    def with_block_table(self, table: np.ndarray, num_blocks: int | None = None) -> "Workload":
        """Same values, different physical placement (used to check that the result
        does not depend on which physical blocks hold a sequence)."""
        w = Workload(**{k: getattr(self, k) for k in (
            "name", "seed", "dtype", "num_heads", "num_kv_heads", "head_dim", "seq_lens",
            "query_lens", "causal", "num_blocks", "block_table", "sigma", "block_size", "notes")})
        w.block_table = np.ascontiguousarray(table, np.int32)
        if num_blocks is not None:
            w.num_blocks = int(num_blocks)
        w._kv_cache = self._kv_cache
        for attr in ("kv", "query"):                 # keep per-instance value sources (subsets)
            if attr in self.__dict__:
                w.__dict__[attr] = self.__dict__[attr]
        return w


# ------------------------------------------------------------ block dealing --
def blocks_needed(seq_lens, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Number of pool blocks a sequence of each length occupies (ceil(L / bs))."""
    s = np.asarray(seq_lens, np.int64)
    return ((s + block_size - 1) // block_size).astype(np.int64)


def deal_block_table(rng, counts, num_blocks: int, width: int | None = None,
                     fixed: dict | None = None) -> np.ndarray:
    """Deal distinct physical blocks from a random permutation of the pool.

    counts[b] blocks go to sequence b (in order); ``fixed`` pins whole rows.
    Unused table entries are -1.
    """
    fixed = fixed or {}
    counts = [int(c) for c in counts]
    width = width or max([1] + counts + [len(v) for v in fixed.values()])
    taken = {int(x) for row in fixed.values() for x in row}
    free = np.array([x for x in rng.permutation(num_blocks) if int(x) not in taken], np.int64)
    need = sum(c for b, c in enumerate(counts) if b not in fixed)
    if need > len(free):
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need + len(taken)} blocks")
    table = np.full((len(counts), width), -1, np.int32)
    cursor = 0
    for b, c in enumerate(counts):
        if b in fixed:
            row = list(fixed[b])
            table[b, :len(row)] = row
        else:
            table[b, :c] = free[cursor:cursor + c]
            cursor += c
    return table


def pool_for(counts, headroom: float = 1.1) -> int:
    return int(math.ceil(headroom * int(np.sum(counts))))


# ------------------------------------------------------------------ configs --
def custom(name="custom", *, seq_lens, query_lens=None, num_heads=32, num_kv_heads=8,
           head_dim=128, dtype="bf16", seed=0, sigma=1.0, causal=None, num_blocks=None,
           headroom=1.1, width=None) -> Workload:
    seq_lens = np.asarray(seq_lens, np.int32)
    query_lens = np.ones_like(seq_lens) if query_lens is None else np.asarray(query_lens, np.int32)
    if causal is None:
        causal = bool(np.any(query_lens > 1))
    rng = np.random.default_rng(seed)
    counts = blocks_needed(seq_lens)
    nb = num_blocks if num_blocks is not None else max(1, pool_for(counts, headroom))
    table = deal_block_table(rng, counts, nb, width=width)
    return Workload(name, seed, dtype, num_heads, num_kv_heads, head_dim, seq_lens,
                    query_lens, causal, nb, table, sigma)


def tiny(step: str = "A") -> Workload:
    """Tiny fp32 check, seed 0: 4 sequences, 32/8 heads, D 128, pool of 32 blocks.

    Sequence 0 holds blocks [5, 8, 12], the table of the worked slot example in
    "AI Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention".
    Step A attends [25, 40, 7, 64] tokens, each sequence's newest token being
    written this step; step B appends one more token per sequence (at positions
    [25, 40, 7, 64], so sequence 0's token lands on slot 137) and attends
    [26, 41, 8, 65].
    """
    rng = np.random.default_rng(0)
    lens_b = np.array([26, 41, 8, 65], np.int32)
    counts = blocks_needed(lens_b)                 # 2, 3, 1, 5
    table = deal_block_table(rng, [3, counts[1], counts[2], counts[3]], 32,
                             fixed={0: [5, 8, 12]})
    lens = lens_b if step == "B" else lens_b - 1
    return Workload(f"tiny_f32_step{step}", 0, "f32", 32, 8, 128, lens.astype(np.int32),
                    np.ones(4, np.int32), False, 32, table, 1.0,
                    notes="4 seqs, fp32, pool 32, seq0 table [5,8,12]")


def llama8b_decode(seed: int = 1) -> Workload:
    """Llama-3-8B decode layer: batch 64, lengths uniform in [1024, 8192], bf16,
    pool 110% of the blocks used, values 0.5*N(0,1)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1024, 8192, size=64, endpoint=True).astype(np.int32)
    counts = blocks_needed(lens)
    nb = pool_for(counts)
    table = deal_block_table(rng, counts, nb)
    return Workload("llama3_8b_decode_b64_1k-8k", seed, "bf16", 32, 8, 128, lens,
                    np.ones(64, np.int32), False, nb, table, 0.5,
                    notes="B=64, L~U[1024,8192], Hq=32, Hkv=8, D=128, bf16, sigma 0.5")


def llama8b_decode_8k(seed: int = 1) -> Workload:
    """Batch 64 with every sequence at 8192 tokens (the 'batch 64 x 8K' target)."""
    rng = np.random.default_rng(seed)
    lens = np.full(64, 8192, np.int32)
    counts = blocks_needed(lens)
    nb = pool_for(counts)
    table = deal_block_table(rng, counts, nb)
    return Workload("llama3_8b_decode_b64_8k", seed, "bf16", 32, 8, 128, lens,
                    np.ones(64, np.int32), False, nb, table, 0.5,
                    notes="B=64, L=8192, Hq=32, Hkv=8, D=128, bf16, sigma 0.5")


def long_context(seed: int = 2) -> Workload:
    """Long-context decode: batch 16 at 32768 tokens over a 40,000-block pool, bf16."""
    rng = np.random.default_rng(seed)
    lens = np.full(16, 32768, np.int32)
    table = deal_block_table(rng, blocks_needed(lens), 40000)
    return Workload("long_context_b16_32k", seed, "bf16", 32, 8, 128, lens,
                    np.ones(16, np.int32), False, 40000, table, 1.0,
                    notes="B=16, L=32768, pool 40000 blocks, bf16, N(0,1)")


def continuous_batching(seed: int = 3) -> Workload:
    """256 decodes, lengths log-normal (median 900, sigma 1) clipped to [16, 16384],
    70B-style GQA (64 query heads over 8 KV heads), bf16; every sequence writes one
    new token this step."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(np.exp(rng.normal(math.log(900.0), 1.0, size=256))), 16, 16384)
    lens = lens.astype(np.int32)
    counts = blocks_needed(lens)
    nb = pool_for(counts)
    table = deal_block_table(rng, counts, nb)
    return Workload("cb_mix_b256_gqa8", seed, "bf16", 64, 8, 128, lens,
                    np.ones(256, np.int32), False, nb, table, 1.0,
                    notes="B=256, L~logN(ln 900, 1) clipped [16,16384], Hq=64, Hkv=8, bf16")


def chunked_prefill_mix(seed: int = 4) -> Workload:
    """4 prefill chunks of 512 queries at prior contexts [0, 2048, 4096, 7680]
    (causal within the chunk) plus 96 single-token decodes at contexts uniform in
    [512, 8192]; Llama-3-8B heads, bf16."""
    rng = np.random.default_rng(seed)
    prior = np.array([0, 2048, 4096, 7680], np.int64)
    dec = rng.integers(512, 8192, size=96, endpoint=True)
    lens = np.concatenate([prior + 512, dec]).astype(np.int32)
    qlens = np.concatenate([np.full(4, 512), np.ones(96)]).astype(np.int32)
    counts = blocks_needed(lens)
    nb = pool_for(counts)
    table = deal_block_table(rng, counts, nb)
    return Workload("chunked_prefill_mix", seed, "bf16", 32, 8, 128, lens, qlens, True,
                    nb, table, 1.0,
                    notes="4x512-query chunks at prior [0,2048,4096,7680] + 96 decodes U[512,8192]")


CONFIGS = {
    "tiny": tiny,
    "llama8b_decode": llama8b_decode,
    "llama8b_decode_8k": llama8b_decode_8k,
    "long_context": long_context,
    "continuous_batching": continuous_batching,
    "chunked_prefill_mix": chunked_prefill_mix,
}


def decode_part(w: Workload) -> Workload:
    """The single-token sequences of a mixed batch, as their own decode workload
    (same values, same placement)."""
    idx = np.nonzero(w.query_lens == 1)[0]
    return _subset(w, idx, "decode_part")


def prefill_part(w: Workload) -> Workload:
    idx = np.nonzero(w.query_lens > 1)[0]
    return _subset(w, idx, "prefill_part")


def _subset(w: Workload, idx, tag) -> Workload:
    sub = Workload(f"{w.name}:{tag}", w.seed, w.dtype, w.num_heads, w.num_kv_heads,
                   w.head_dim, w.seq_lens[idx].copy(), w.query_lens[idx].copy(), w.causal,
                   w.num_blocks, w.block_table[idx].copy(), w.sigma)
    sub._parent = (w, np.asarray(idx))
    orig_kv, orig_q = w.kv, w.query
    sub.kv = lambda b, length=None: orig_kv(int(idx[b]), length)          # type: ignore
    sub.query = lambda b: orig_q(int(idx[b]))                              # type: ignore
    return sub
