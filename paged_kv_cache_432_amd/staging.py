"""Caller-side staging of a synthetic workload on the GPU.

This plays the part of an inference engine around the library: it uploads a
workload's inputs (block tables, lengths, queries, the K/V rows of every
token) and builds the paged cache the way an engine does, by computing slots
with ``pa_slot_mapping`` and writing rows with ``pa_reshape_and_cache``.  The
earlier context of every sequence is written once, before any timing; the
step itself then scatters only this step's tokens and attends.  Torch is used
for allocation and uploads only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (chunked_prefill_workspace, decode_workspace, pa_chunked_prefill, pa_decode, pa_decode_append,
               pa_decode_append_fp8, pa_decode_fp8, pa_reshape_and_cache, pa_reshape_and_cache_fp8, pa_slot_mapping, pa_slot_mapping_and_cache,
               pa_slot_mapping_and_cache_fp8)

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _upload(x: np.ndarray, dtype, device) -> torch.Tensor:
    # values drawn for a bf16 workload are exactly representable: the cast is exact
    return torch.from_numpy(np.ascontiguousarray(x)).to(device).to(dtype)


GUARD_BYTE = 0xA5


class Guarded:
    """A contiguous device tensor placed inside a larger byte buffer whose
    margins (guard_bytes before and after it, rounded up to 256) hold a fixed
    byte pattern: a kernel that writes outside the tensor changes the pattern,
    which intact() reports.  The tensor starts 256-byte aligned."""

    def __init__(self, shape, dtype, device, guard_bytes: int = 4096):
        self.shape = tuple(int(x) for x in shape)
        itemsize = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = int(np.prod(self.shape, dtype=np.int64)) * itemsize
        self.guard = ((int(guard_bytes) + 255) // 256) * 256
        self.buf = torch.full((self.guard + self.nbytes + self.guard,), GUARD_BYTE, dtype=torch.uint8,
                              device=device)
        self.t = self.buf[self.guard:self.guard + self.nbytes].view(dtype).view(self.shape)

    def intact(self) -> bool:
        return bool(torch.all(self.buf[:self.guard] == GUARD_BYTE).item()
                    and torch.all(self.buf[self.guard + self.nbytes:] == GUARD_BYTE).item())


class DeviceWorkload:
    """Device-resident inputs and paged cache of one workload step."""

    def __init__(self, w, device="cuda", fill_history: bool = True, poison: bool = True, kv_fp8: bool = False,
                 guard_bytes: int = 0, fp8_format: str = "e4m3"):
        """kv_fp8: the caches hold fp8 codes (uint8, fp8_format "e4m3" or
        "e5m2") written by the fp8 scatter with the workload's fp8_scales();
        queries and outputs stay bf16.
        guard_bytes > 0: each cache sits between guard zones (Guarded), checked
        by guards_intact()."""
        self.w = w
        self.device = torch.device(device)
        self.dtype = _TORCH_DTYPE[w.dtype]
        self.kv_fp8 = kv_fp8
        self.fp8_format = fp8_format
        if kv_fp8:
            assert w.dtype == "bf16", "an fp8 cache goes with bf16 queries"
            self.k_scale, self.v_scale = w.fp8_scales()
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        cdt = torch.uint8 if kv_fp8 else self.dtype
        if guard_bytes > 0:
            self._guards = [Guarded(shape, cdt, self.device, guard_bytes) for _ in range(2)]
            self.key_cache, self.value_cache = (g.t for g in self._guards)
        else:
            self._guards = []
            self.key_cache = torch.empty(shape, dtype=cdt, device=self.device)
            self.value_cache = torch.empty(shape, dtype=cdt, device=self.device)
        if kv_fp8:
            self.key_cache.fill_(0x7F if poison else 0)
            self.value_cache.fill_(0x7F if poison else 0)
        else:
            self.key_cache.fill_(float("nan") if poison else 0.0)
            self.value_cache.fill_(float("nan") if poison else 0.0)
        self.block_table = torch.from_numpy(np.ascontiguousarray(w.block_table, np.int32)).to(self.device)
        self.seq_lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens, np.int32)).to(self.device)
        self.cu_query_lens = torch.from_numpy(w.cu_query_lens).to(self.device)
        self.query = _upload(w.queries(), self.dtype, self.device)
        seq, pos = w.tokens("new")
        self.new_seq = torch.from_numpy(seq).to(self.device)
        self.new_pos = torch.from_numpy(pos).to(self.device)
        self.slot_mapping = torch.empty(len(seq), dtype=torch.int64, device=self.device)
        n, hkv, d = len(seq), w.num_kv_heads, w.head_dim
        new_k = np.empty((n, hkv, d), np.float32)
        new_v = np.empty((n, hkv, d), np.float32)
        cursor = 0
        # values drawn a few sequences ahead on host threads; uploads and
        # scatters stay in order on this thread
        for b, k, v in w.iter_kv(np.flatnonzero(np.asarray(w.seq_lens) > 0)):
            h, L = int(w.history_lens[b]), int(w.seq_lens[b])
            if fill_history and h > 0:
                self._write(b, k[:h], v[:h], 0)
            q = L - h
            new_k[cursor:cursor + q] = k[h:L]
            new_v[cursor:cursor + q] = v[h:L]
            cursor += q
        assert cursor == n
        self.new_k = _upload(new_k, self.dtype, self.device)
        self.new_v = _upload(new_v, self.dtype, self.device)

    def guards_intact(self) -> bool:
        """True when the guard zones around both caches are unchanged (always
        True without guards)."""
        return all(g.intact() for g in self._guards)

    def _write(self, b: int, k: np.ndarray, v: np.ndarray, start: int) -> None:
        n = k.shape[0]
        seq = torch.full((n,), b, dtype=torch.int32, device=self.device)
        pos = torch.arange(start, start + n, dtype=torch.int32, device=self.device)
        slots = torch.empty(n, dtype=torch.int64, device=self.device)
        pa_slot_mapping(slots, self.block_table, seq, pos)
        self._scatter(_upload(k, self.dtype, self.device), _upload(v, self.dtype, self.device), slots)

    def _scatter(self, k, v, slots, stream=None) -> None:
        if self.kv_fp8:
            pa_reshape_and_cache_fp8(k, v, self.key_cache, self.value_cache, slots, self.k_scale, self.v_scale,
                                     stream=stream, fp8_format=self.fp8_format)
        else:
            pa_reshape_and_cache(k, v, self.key_cache, self.value_cache, slots, stream=stream)

    # ---- the step
    def scatter_new(self, stream=None, fused: bool = False) -> None:
        """Rows a1-a2 of the step: slots of this step's tokens, then their scatter
        (fused: both in one launch, pa_slot_mapping_and_cache, or
        pa_slot_mapping_and_cache_fp8 over an fp8 cache)."""
        if fused and self.kv_fp8:
            pa_slot_mapping_and_cache_fp8(self.slot_mapping, self.block_table, self.new_seq, self.new_pos,
                                          self.new_k, self.new_v, self.key_cache, self.value_cache, self.k_scale,
                                          self.v_scale, stream=stream, fp8_format=self.fp8_format)
            return
        if fused:
            pa_slot_mapping_and_cache(self.slot_mapping, self.block_table, self.new_seq, self.new_pos,
                                      self.new_k, self.new_v, self.key_cache, self.value_cache, stream=stream)
            return
        pa_slot_mapping(self.slot_mapping, self.block_table, self.new_seq, self.new_pos, stream=stream)
        self._scatter(self.new_k, self.new_v, self.slot_mapping, stream=stream)

    def decode_workspace(self, partition_tokens: int = 0):
        w = self.w
        return decode_workspace(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq_len,
                                partition_tokens, device=self.device)

    def decode(self, out=None, partition_tokens: int = 0, workspace=None, stream=None) -> torch.Tensor:
        w = self.w
        if out is None:
            out = torch.empty_like(self.query)
        if workspace is None:
            workspace = self.decode_workspace(partition_tokens)
        if self.kv_fp8:
            assert partition_tokens == 0, "an fp8 cache is read in the stream mode only"
            return pa_decode_fp8(out, self.query, self.key_cache, self.value_cache, self.block_table,
                                 self.seq_lens, w.scale, self.k_scale, self.v_scale, w.max_seq_len, workspace,
                                 stream, fp8_format=self.fp8_format)
        return pa_decode(out, self.query, self.key_cache, self.value_cache, self.block_table,
                         self.seq_lens, w.scale, w.max_seq_len, partition_tokens, workspace, stream)

    def append_rows(self):
        """This step's new K/V rows indexed by sequence ([num_seqs, Hkv, D], row b
        the newest token of sequence b; zeros for sequences without one), as
        pa_decode_append takes them."""
        if not hasattr(self, "_append"):
            w = self.w
            L = np.asarray(w.seq_lens)
            assert np.all((L == 0) | (L - np.asarray(w.history_lens) == 1)), "one new token per sequence"
            idx = torch.from_numpy(np.flatnonzero(L > 0)).to(self.device)
            k = torch.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), dtype=self.dtype, device=self.device)
            v = torch.zeros_like(k)
            k[idx] = self.new_k
            v[idx] = self.new_v
            self._append = (k, v, torch.empty(w.num_seqs, dtype=torch.int64, device=self.device))
        return self._append

    def decode_append(self, out=None, workspace=None, stream=None) -> torch.Tensor:
        """The whole decode step in one call (pa_decode_append, or
        pa_decode_append_fp8 over an fp8 cache): the newest token of every
        sequence written to the cache and attended to."""
        w = self.w
        k, v, slots = self.append_rows()
        if out is None:
            out = torch.empty_like(self.query)
        if workspace is None:
            workspace = self.decode_workspace(0)
        if self.kv_fp8:
            return pa_decode_append_fp8(out, self.query, k, v, self.key_cache, self.value_cache, self.block_table,
                                        self.seq_lens, w.scale, self.k_scale, self.v_scale, w.max_seq_len, slots,
                                        workspace, stream, fp8_format=self.fp8_format)
        return pa_decode_append(out, self.query, k, v, self.key_cache, self.value_cache, self.block_table,
                                self.seq_lens, w.scale, w.max_seq_len, slots, workspace, stream)

    def prefill_workspace(self):
        w = self.w
        return chunked_prefill_workspace(w.num_seqs, w.num_q_tokens, w.max_query_len, w.max_seq_len,
                                         w.num_heads, w.num_kv_heads, w.head_dim, device=self.device,
                                         dtype=self.dtype)

    def chunked_prefill(self, out=None, workspace=None, stream=None) -> torch.Tensor:
        """Row a10: one call over the whole mixed batch (chunks and decodes)."""
        w = self.w
        if out is None:
            out = torch.empty_like(self.query)
        if workspace is None:
            workspace = self.prefill_workspace()
        return pa_chunked_prefill(out, self.query, self.key_cache, self.value_cache, self.block_table,
                                  self.cu_query_lens, self.seq_lens, w.scale, w.max_query_len, w.max_seq_len,
                                  w.causal, workspace, stream)
