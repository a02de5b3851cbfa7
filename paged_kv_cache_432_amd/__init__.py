"""Python binding of libpa.so, the MI355X (gfx950) paged KV-cache attention library.

Argument marshalling only: every function here checks the tensors it is
handed, turns them into device pointers, sizes and the current HIP stream,
and calls the C entry point of the same name (declared in include/pa.h).  All
computation happens in the library's kernels; PyTorch only provides device
memory and streams.  There is no fallback: if libpa.so is missing the first
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

__all__ = [
    "PaError", "lib", "lib_path", "pa_abi_version", "pa_status_string", "pa_last_error_message",
    "pa_slot_mapping", "pa_reshape_and_cache", "pa_slot_mapping_and_cache", "pa_rope_reshape_and_cache", "pa_reshape_and_cache_fp8", "pa_slot_mapping_and_cache_fp8",
    "pa_decode_fp8", "pa_copy_blocks", "KvManager", "pa_decode_workspace_bytes",
    "pa_decode_partition_tokens", "pa_decode", "pa_decode_append", "pa_decode_append_noalloc", "pa_decode_append_fp8", "decode_workspace", "pa_chunked_prefill_workspace_bytes",
    "pa_chunked_prefill", "chunked_prefill_workspace", "pa_probe_stream_read", "pa_probe_copy", "pa_probe_mfma",
    "pa_validate_block_tables", "pa_validate_slot_mapping", "pa_validate_query_lens",
]

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_F32, PA_BF16 = 0, 1
PA_FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
BLOCK_SIZE = 16

_DIR = os.path.dirname(os.path.abspath(__file__))
_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class _KvmStep(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_tokens", _i64), ("max_blocks_per_req", _i32),
                ("request_ids", _vp), ("query_lens", _vp), ("cu_query_lens", _vp), ("seq_lens", _vp),
                ("block_table", _vp), ("token_ids", _vp), ("positions", _vp), ("slot_mapping", _vp),
                ("copy_pairs", _vp), ("num_copies", _i32), ("preempted", _vp), ("num_preempted", _i32)]


class PaError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")


def lib_path() -> str:
    """The in-tree libpa.so, or the build named by the PA_LIB environment
    variable (e.g. one whose host code carries sanitizers)."""
    return os.environ.get("PA_LIB") or os.path.join(_DIR, "libpa.so")


def lib():
    """Load libpa.so (built in tree by __graft_entry__.build())."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                               "(or python paged_kv_cache_432_amd/_build.py)")
        L = ctypes.CDLL(path)
        L.pa_abi_version.restype = _i32
        L.pa_abi_version.argtypes = []
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_last_error_message.restype = ctypes.c_char_p
        L.pa_last_error_message.argtypes = []
        L.pa_slot_mapping.restype = ctypes.c_int
        L.pa_slot_mapping.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _i64, _i32, _vp]
        L.pa_slot_mapping_and_cache.restype = ctypes.c_int
        L.pa_slot_mapping_and_cache.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp,
                                                _i64, _i64, _i32, _i32, _i32, ctypes.c_int, _vp]
        L.pa_reshape_and_cache.restype = ctypes.c_int
        L.pa_reshape_and_cache.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32,
                                           _i32, _i32, ctypes.c_int, _vp]
        L.pa_kvm_create.restype = _vp
        L.pa_kvm_create.argtypes = [_i32, _i32, _i32, _i32, _i32]
        L.pa_kvm_destroy.restype = None
        L.pa_kvm_destroy.argtypes = [_vp]
        L.pa_kvm_add_request.restype = ctypes.c_int
        L.pa_kvm_add_request.argtypes = [_vp, _i64, _vp, _i32]
        L.pa_kvm_fork.restype = ctypes.c_int
        L.pa_kvm_fork.argtypes = [_vp, _i64, _i64]
        L.pa_kvm_finish.restype = ctypes.c_int
        L.pa_kvm_finish.argtypes = [_vp, _i64]
        L.pa_kvm_schedule.restype = ctypes.c_int
        L.pa_kvm_schedule.argtypes = [_vp, ctypes.POINTER(_KvmStep)]
        L.pa_kvm_commit.restype = ctypes.c_int
        L.pa_kvm_commit.argtypes = [_vp, _vp, _i32]
        L.pa_kvm_num_free_blocks.restype = _i32
        L.pa_kvm_num_free_blocks.argtypes = [_vp]
        L.pa_kvm_num_cached_blocks.restype = _i32
        L.pa_kvm_num_cached_blocks.argtypes = [_vp]
        L.pa_kvm_block_ref.restype = _i32
        L.pa_kvm_block_ref.argtypes = [_vp, _i32]
        L.pa_kvm_request_info.restype = ctypes.c_int
        L.pa_kvm_request_info.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp]
        L.pa_copy_blocks.restype = ctypes.c_int
        L.pa_copy_blocks.argtypes = [_vp, _vp, _i64, _i32, _i64, _i64, _vp, _i64, _vp]
        L.pa_reshape_and_cache_fp8.restype = ctypes.c_int
        L.pa_reshape_and_cache_fp8.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32,
                                               _i32, _i32, ctypes.c_int, ctypes.c_float, ctypes.c_float, _vp]
        L.pa_slot_mapping_and_cache_fp8.restype = ctypes.c_int
        L.pa_slot_mapping_and_cache_fp8.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp,
                                                    _i64, _i64, _i32, _i32, _i32, ctypes.c_int, ctypes.c_float,
                                                    ctypes.c_float, _vp]
        L.pa_reshape_and_cache_fp8_ex.restype = ctypes.c_int
        L.pa_reshape_and_cache_fp8_ex.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i32,
                                                  _i32, _i32, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                  ctypes.c_float, _vp]
        L.pa_slot_mapping_and_cache_fp8_ex.restype = ctypes.c_int
        L.pa_slot_mapping_and_cache_fp8_ex.argtypes = [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                                       _vp, _i64, _i64, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_float, ctypes.c_float, _vp]
        L.pa_decode_fp8_ex.restype = ctypes.c_int
        L.pa_decode_fp8_ex.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _i64, ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float,
                                       _i32, _vp, ctypes.c_size_t, _vp]
        L.pa_decode_fp8.restype = ctypes.c_int
        L.pa_decode_fp8.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_float, _i32, _vp,
                                    ctypes.c_size_t, _vp]
        L.pa_rope_reshape_and_cache.restype = ctypes.c_int
        L.pa_rope_reshape_and_cache.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp,
                                                _i64, _i64, _i32, _i32, _i32, _i32, ctypes.c_int, _vp]
        L.pa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.pa_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
        L.pa_decode_partition_tokens.restype = _i32
        L.pa_decode_partition_tokens.argtypes = [_i32, _i32, _i32, _i32]
        L.pa_decode.restype = ctypes.c_int
        L.pa_decode.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                _i32, _i64, ctypes.c_float, _i32, _i32, _vp, ctypes.c_size_t,
                                ctypes.c_int, _vp]
        L.pa_decode_append.restype = ctypes.c_int
        L.pa_decode_append.argtypes = [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                       _i32, _i32, _i32, _i32, _i64, ctypes.c_float, _i32, _vp, ctypes.c_size_t,
                                       ctypes.c_int, _vp]
        L.pa_decode_append_fp8.restype = ctypes.c_int
        L.pa_decode_append_fp8.argtypes = [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp,
                                           _i32, _i32, _i32, _i32, _i32, _i64, ctypes.c_float, ctypes.c_int,
                                           ctypes.c_float, ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp]
        L.pa_decode_append_noalloc.restype = ctypes.c_int
        L.pa_decode_append_noalloc.argtypes = [_vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp,
                                               _i32, _i32, _i32, _i32, _i32, _i64, ctypes.c_float, _i32,
                                               ctypes.c_int, _vp]
        L.pa_chunked_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.pa_chunked_prefill_workspace_bytes.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32, _i32]
        L.pa_chunked_prefill_workspace_bytes_ex.restype = ctypes.c_size_t
        L.pa_chunked_prefill_workspace_bytes_ex.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
        L.pa_chunked_prefill.restype = ctypes.c_int
        L.pa_chunked_prefill.argtypes = [_vp, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _i64, ctypes.c_float, _i32, _vp,
                                         ctypes.c_size_t, ctypes.c_int, _vp]
        L.pa_validate_block_tables.restype = ctypes.c_int
        L.pa_validate_block_tables.argtypes = [_vp, _i32, _vp, _i32, _i64, _i32, _i32]
        L.pa_validate_slot_mapping.restype = ctypes.c_int
        L.pa_validate_slot_mapping.argtypes = [_vp, _i64, _i64, _i32]
        L.pa_validate_query_lens.restype = ctypes.c_int
        L.pa_validate_query_lens.argtypes = [_vp, _vp, _i32, _i64, _i32]
        L.pa_probe_stream_read.restype = ctypes.c_int
        L.pa_probe_stream_read.argtypes = [_vp, _i64, _vp, _i32, _vp]
        L.pa_probe_copy.restype = ctypes.c_int
        L.pa_probe_copy.argtypes = [_vp, _vp, _i64, _i32, _vp]
        L.pa_probe_mfma.restype = ctypes.c_int
        L.pa_probe_mfma.argtypes = [_vp, _i32, _i32, _vp]
        _lib = L
        return L


def _status_name(s: int) -> str:
    try:
        return lib().pa_status_string(int(s)).decode()
    except Exception:                                     # noqa: BLE001 -- message only
        return f"status {s}"


def _check(status: int, fn: str) -> None:
    if status != PA_OK:
        raise PaError(status, fn, lib().pa_last_error_message().decode())


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def pa_abi_version() -> int:
    return int(lib().pa_abi_version())


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def pa_last_error_message() -> str:
    return lib().pa_last_error_message().decode()


# ------------------------------------------------------------ entry points --
def pa_slot_mapping(slot_mapping: torch.Tensor, block_table: torch.Tensor, token_seq: torch.Tensor,
                    token_pos: torch.Tensor, block_size: int = BLOCK_SIZE, stream=None) -> torch.Tensor:
    """slot_mapping[i] = block_table[token_seq[i], token_pos[i] // 16] * 16 + token_pos[i] % 16
    (int64 out), -1 for padding or unallocated tokens."""
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous(), "slot_mapping: contiguous int64")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(token_seq.dtype == torch.int32 and token_pos.dtype == torch.int32, "token_seq/token_pos: int32")
    _need(token_seq.is_contiguous() and token_pos.is_contiguous(), "token_seq/token_pos: contiguous")
    n = slot_mapping.numel()
    _need(token_seq.numel() == n and token_pos.numel() == n, "token lists of different lengths")
    s = lib().pa_slot_mapping(_ptr(slot_mapping), _ptr(block_table), block_table.shape[1],
                              block_table.shape[0], _ptr(token_seq), _ptr(token_pos), n, block_size,
                              _stream(stream, slot_mapping.device))
    _check(s, "pa_slot_mapping")
    return slot_mapping


def pa_slot_mapping_and_cache(slot_mapping: torch.Tensor, block_table: torch.Tensor, token_seq: torch.Tensor,
                              token_pos: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                              key_cache: torch.Tensor, value_cache: torch.Tensor, stream=None) -> torch.Tensor:
    """pa_slot_mapping then pa_reshape_and_cache in one launch: slot_mapping
    (int64, out) is written and the K/V rows are scattered to it."""
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous(), "slot_mapping: contiguous int64")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(token_seq.dtype == torch.int32 and token_pos.dtype == torch.int32, "token_seq/token_pos: int32")
    _need(token_seq.is_contiguous() and token_pos.is_contiguous(), "token_seq/token_pos: contiguous")
    _need(key.dim() == 3 and value.dim() == 3 and key.shape == value.shape, "key/value: [num_tokens, Hkv, D]")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(key.dtype == value.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    n, hkv, d = key.shape
    _need(slot_mapping.numel() == n and token_seq.numel() == n and token_pos.numel() == n, "token lists differ")
    _need(key_cache.shape[2] == hkv and key_cache.shape[3] == d, "cache head shape differs from key")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1 and value.stride(1) == d,
          "key/value heads and dims must be contiguous")
    s = lib().pa_slot_mapping_and_cache(_ptr(slot_mapping), _ptr(block_table), block_table.shape[1],
                                        block_table.shape[0], _ptr(token_seq), _ptr(token_pos), _ptr(key),
                                        key.stride(0), _ptr(value), value.stride(0), _ptr(key_cache),
                                        _ptr(value_cache), n, key_cache.shape[0], key_cache.shape[1], hkv, d,
                                        _dtype_code(key), _stream(stream, key_cache.device))
    _check(s, "pa_slot_mapping_and_cache")
    return slot_mapping


def pa_reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Scatter key/value [num_tokens, Hkv, D] (token stride free, e.g. QKV column
    slices) into caches [num_blocks, 16, Hkv, D] at slot_mapping (int64)."""
    _need(key.dim() == 3 and value.dim() == 3 and key.shape == value.shape, "key/value: [num_tokens, Hkv, D]")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(key.dtype == value.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    n, hkv, d = key.shape
    _need(key_cache.shape[2] == hkv and key_cache.shape[3] == d, "cache head shape differs from key")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1 and value.stride(1) == d,
          "key/value heads and dims must be contiguous")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == n and slot_mapping.is_contiguous(),
          "slot_mapping: contiguous int64 [num_tokens]")
    s = lib().pa_reshape_and_cache(_ptr(key), key.stride(0), _ptr(value), value.stride(0),
                                   _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), n,
                                   key_cache.shape[0], key_cache.shape[1], hkv, d, _dtype_code(key),
                                   _stream(stream, key_cache.device))
    _check(s, "pa_reshape_and_cache")


def _host_array(ptr, n, dtype):
    if n == 0 or not ptr:
        return np.zeros(0, dtype)
    ct = {np.int32: ctypes.c_int32, np.int64: ctypes.c_int64}[dtype]
    return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ct)), shape=(n,)).copy()


class KvManager:
    """The host block manager and step scheduler (pa_kvm_*): see include/pa.h."""

    def __init__(self, num_blocks: int, max_num_seqs: int, max_num_batched_tokens: int, max_model_len: int,
                 prefix_caching: bool = True):
        self._L = lib()
        self._h = self._L.pa_kvm_create(num_blocks, max_num_seqs, max_num_batched_tokens, max_model_len,
                                        int(bool(prefix_caching)))
        if not self._h:
            raise PaError(PA_ERR_INVALID_ARG, "pa_kvm_create", pa_last_error_message())

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._L.pa_kvm_destroy(h)

    def add_request(self, request_id: int, prompt) -> None:
        p = np.ascontiguousarray(prompt, np.int32)
        _check(self._L.pa_kvm_add_request(self._h, int(request_id), p.ctypes.data, len(p)), "pa_kvm_add_request")

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(self._L.pa_kvm_fork(self._h, int(parent_id), int(child_id)), "pa_kvm_fork")

    def finish(self, request_id: int) -> None:
        _check(self._L.pa_kvm_finish(self._h, int(request_id)), "pa_kvm_finish")

    def schedule(self) -> dict:
        """One step: numpy copies of the step's arrays (block_table 2-D,
        copy_pairs [n, 2])."""
        st = _KvmStep()
        _check(self._L.pa_kvm_schedule(self._h, ctypes.byref(st)), "pa_kvm_schedule")
        n, t, w = st.num_seqs, st.num_tokens, st.max_blocks_per_req
        return {
            "num_seqs": n, "num_tokens": t, "max_blocks_per_req": w,
            "request_ids": _host_array(st.request_ids, n, np.int64),
            "query_lens": _host_array(st.query_lens, n, np.int32),
            "cu_query_lens": _host_array(st.cu_query_lens, n + 1, np.int32),
            "seq_lens": _host_array(st.seq_lens, n, np.int32),
            "block_table": _host_array(st.block_table, n * w, np.int32).reshape(n, w),
            "token_ids": _host_array(st.token_ids, t, np.int32),
            "positions": _host_array(st.positions, t, np.int32),
            "slot_mapping": _host_array(st.slot_mapping, t, np.int64),
            "copy_pairs": _host_array(st.copy_pairs, 2 * st.num_copies, np.int64).reshape(-1, 2),
            "preempted": _host_array(st.preempted, st.num_preempted, np.int64),
        }

    def commit(self, next_tokens) -> None:
        t = np.ascontiguousarray(next_tokens, np.int32)
        _check(self._L.pa_kvm_commit(self._h, t.ctypes.data if len(t) else None, len(t)), "pa_kvm_commit")

    def num_free_blocks(self) -> int:
        return int(self._L.pa_kvm_num_free_blocks(self._h))

    def num_cached_blocks(self) -> int:
        return int(self._L.pa_kvm_num_cached_blocks(self._h))

    def block_ref(self, block: int) -> int:
        return int(self._L.pa_kvm_block_ref(self._h, int(block)))

    def request(self, request_id: int) -> dict:
        nc, nt, run, nb = (ctypes.c_int32() for _ in range(4))
        _check(self._L.pa_kvm_request_info(self._h, int(request_id), ctypes.byref(nc), ctypes.byref(nt),
                                           ctypes.byref(run), None, 0, ctypes.byref(nb)), "pa_kvm_request_info")
        blocks = np.zeros(nb.value, np.int32)
        _check(self._L.pa_kvm_request_info(self._h, int(request_id), None, None, None, blocks.ctypes.data,
                                           len(blocks), None), "pa_kvm_request_info")
        return {"num_computed": nc.value, "num_tokens": nt.value, "running": bool(run.value), "blocks": blocks}


def pa_copy_blocks(kv_cache: torch.Tensor, block_mapping: torch.Tensor, stream=None) -> None:
    """Copy-on-write over the pages' unified cache kv_cache [num_layers, 2,
    num_blocks, ...] (contiguous, any dtype): for each (src, dst) row of
    block_mapping (int64 [n, 2]), block dst of every layer's K and V becomes a
    copy of block src."""
    _need(kv_cache.dim() >= 4 and kv_cache.shape[1] == 2 and kv_cache.is_contiguous(),
          "kv_cache: contiguous [num_layers, 2, num_blocks, ...]")
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2 and block_mapping.shape[1] == 2
          and block_mapping.is_contiguous(), "block_mapping: contiguous int64 [n, 2]")
    num_layers, _, num_blocks = kv_cache.shape[:3]
    block_bytes = kv_cache[0, 0, 0].numel() * kv_cache.element_size()
    s = lib().pa_copy_blocks(_ptr(kv_cache), _ptr(kv_cache) + num_blocks * block_bytes,
                             2 * num_blocks * block_bytes, num_layers, num_blocks, block_bytes,
                             _ptr(block_mapping), block_mapping.shape[0], _stream(stream, kv_cache.device))
    _check(s, "pa_copy_blocks")


def _fp8_format(name: str) -> int:
    _need(name in PA_FP8_FORMATS, f"fp8_format {name!r}: 'e4m3' or 'e5m2'")
    return PA_FP8_FORMATS[name]


def pa_reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float, v_scale: float,
                             stream=None, fp8_format: str = "e4m3") -> None:
    """Scatter key/value [num_tokens, Hkv, D] (bf16 or fp32, token stride free)
    into uint8 fp8 caches [num_blocks, 16, Hkv, D] as codes of x / scale, in
    fp8_format ("e4m3" or "e5m2")."""
    _need(key.dim() == 3 and value.dim() == 3 and key.shape == value.shape, "key/value: [num_tokens, Hkv, D]")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(key_cache.dtype == value_cache.dtype == torch.uint8, "fp8 caches are uint8 (E4M3 codes)")
    _need(key.dtype == value.dtype, "key/value dtype mismatch")
    n, hkv, d = key.shape
    _need(key_cache.shape[2] == hkv and key_cache.shape[3] == d, "cache head shape differs from key")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1 and value.stride(1) == d,
          "key/value heads and dims must be contiguous")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == n and slot_mapping.is_contiguous(),
          "slot_mapping: contiguous int64 [num_tokens]")
    s = lib().pa_reshape_and_cache_fp8_ex(_ptr(key), key.stride(0), _ptr(value), value.stride(0),
                                          _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping), n,
                                          key_cache.shape[0], key_cache.shape[1], hkv, d, _dtype_code(key),
                                          _fp8_format(fp8_format), float(k_scale), float(v_scale),
                                          _stream(stream, key_cache.device))
    _check(s, "pa_reshape_and_cache_fp8_ex")


def pa_slot_mapping_and_cache_fp8(slot_mapping: torch.Tensor, block_table: torch.Tensor, token_seq: torch.Tensor,
                                  token_pos: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                  key_cache: torch.Tensor, value_cache: torch.Tensor, k_scale: float, v_scale: float,
                                  stream=None, fp8_format: str = "e4m3") -> torch.Tensor:
    """pa_slot_mapping then pa_reshape_and_cache_fp8 in one launch: slot_mapping
    (int64, out) is written and the K/V rows are quantised into the fp8 caches
    (fp8_format "e4m3" or "e5m2")."""
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous(), "slot_mapping: contiguous int64")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(token_seq.dtype == torch.int32 and token_pos.dtype == torch.int32, "token_seq/token_pos: int32")
    _need(token_seq.is_contiguous() and token_pos.is_contiguous(), "token_seq/token_pos: contiguous")
    _need(key.dim() == 3 and value.dim() == 3 and key.shape == value.shape, "key/value: [num_tokens, Hkv, D]")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(key_cache.dtype == value_cache.dtype == torch.uint8, "fp8 caches are uint8 (E4M3 codes)")
    _need(key.dtype == value.dtype, "key/value dtype mismatch")
    n, hkv, d = key.shape
    _need(slot_mapping.numel() == n and token_seq.numel() == n and token_pos.numel() == n, "token lists differ")
    _need(key_cache.shape[2] == hkv and key_cache.shape[3] == d, "cache head shape differs from key")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1 and value.stride(1) == d,
          "key/value heads and dims must be contiguous")
    s = lib().pa_slot_mapping_and_cache_fp8_ex(_ptr(slot_mapping), _ptr(block_table), block_table.shape[1],
                                               block_table.shape[0], _ptr(token_seq), _ptr(token_pos), _ptr(key),
                                               key.stride(0), _ptr(value), value.stride(0), _ptr(key_cache),
                                               _ptr(value_cache), n, key_cache.shape[0], key_cache.shape[1], hkv, d,
                                               _dtype_code(key), _fp8_format(fp8_format), float(k_scale),
                                               float(v_scale), _stream(stream, key_cache.device))
    _check(s, "pa_slot_mapping_and_cache_fp8_ex")
    return slot_mapping


def pa_decode_fp8(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                  block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, k_scale: float, v_scale: float,
                  max_seq_len: int, workspace: torch.Tensor | None = None, stream=None,
                  fp8_format: str = "e4m3") -> torch.Tensor:
    """Decode attention over uint8 fp8 caches (fp8_format "e4m3" or "e5m2"):
    out [B, Hq, D] bf16 for query [B, Hq, D] bf16; cached codes stand for
    value * k_scale / v_scale."""
    _need(query.dim() == 3 and out.shape == query.shape and out.is_contiguous(),
          "query/out: [num_seqs, num_heads, head_dim], out contiguous")
    _need(query.stride(2) == 1 and query.stride(1) == query.shape[2], "query heads/dims must be contiguous")
    _need(query.dtype == out.dtype == torch.bfloat16, "query/out: bfloat16")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(key_cache.dtype == value_cache.dtype == torch.uint8, "fp8 caches are uint8 (E4M3 codes)")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens: contiguous int32")
    b, hq, d = query.shape
    _need(block_table.shape[0] >= b and seq_lens.numel() >= b, "block_table/seq_lens shorter than batch")
    nb, bs, hkv, _ = key_cache.shape
    ws = workspace
    s = lib().pa_decode_fp8_ex(_ptr(out), _ptr(query), query.stride(0), _ptr(key_cache), _ptr(value_cache),
                               _ptr(block_table), block_table.shape[1], _ptr(seq_lens), b, hq, hkv, d, bs, nb,
                               float(scale), _fp8_format(fp8_format), float(k_scale), float(v_scale),
                               int(max_seq_len), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream, out.device))
    _check(s, "pa_decode_fp8_ex")
    return out


def pa_rope_reshape_and_cache(query_out: torch.Tensor, qkv: torch.Tensor, positions: torch.Tensor,
                              cos_sin_cache: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                              slot_mapping: torch.Tensor, num_heads: int, num_kv_heads: int,
                              neox_style: bool = True, stream=None) -> torch.Tensor:
    """Split qkv [num_tokens, (Hq + 2 Hkv) * D] (token stride free), turn Q and K
    by positions (int64) through cos_sin_cache (float32 [max_position,
    rotary_dim]), write Q to query_out [num_tokens, Hq, D] (token stride free;
    may be the Q columns of qkv itself) and scatter K, V into the caches at
    slot_mapping (int64)."""
    _need(qkv.dim() == 2 and qkv.stride(1) == 1, "qkv: [num_tokens, width] with contiguous columns")
    n = qkv.shape[0]
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    d = key_cache.shape[3]
    _need(key_cache.shape[2] == num_kv_heads, "cache KV heads differ from num_kv_heads")
    _need(qkv.shape[1] >= (num_heads + 2 * num_kv_heads) * d, "qkv narrower than (Hq + 2 Hkv) * D")
    _need(query_out.dim() == 3 and tuple(query_out.shape) == (n, num_heads, d), "query_out: [num_tokens, Hq, D]")
    _need(query_out.stride(2) == 1 and query_out.stride(1) == d, "query_out heads and dims must be contiguous")
    _need(qkv.dtype == query_out.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    _need(cos_sin_cache.dtype == torch.float32 and cos_sin_cache.dim() == 2 and cos_sin_cache.is_contiguous(),
          "cos_sin_cache: contiguous float32 [max_position, rotary_dim]")
    _need(positions.dtype == torch.int64 and positions.numel() == n and positions.is_contiguous(),
          "positions: contiguous int64 [num_tokens]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.numel() == n and slot_mapping.is_contiguous(),
          "slot_mapping: contiguous int64 [num_tokens]")
    s = lib().pa_rope_reshape_and_cache(_ptr(query_out), query_out.stride(0), _ptr(qkv), qkv.stride(0),
                                        _ptr(positions), _ptr(cos_sin_cache), cos_sin_cache.shape[0],
                                        cos_sin_cache.shape[1], int(bool(neox_style)), _ptr(key_cache),
                                        _ptr(value_cache), _ptr(slot_mapping), n, key_cache.shape[0],
                                        key_cache.shape[1], num_heads, num_kv_heads, d, _dtype_code(qkv),
                                        _stream(stream, key_cache.device))
    _check(s, "pa_rope_reshape_and_cache")
    return query_out


def pa_decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                              max_seq_len: int, partition_tokens: int = 0) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                               max_seq_len, partition_tokens))


def pa_decode_partition_tokens(num_seqs: int, num_kv_heads: int, max_seq_len: int,
                               partition_tokens: int = 0) -> int:
    return int(lib().pa_decode_partition_tokens(num_seqs, num_kv_heads, max_seq_len, partition_tokens))


def decode_workspace(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                     max_seq_len: int, partition_tokens: int = 0, device="cuda") -> torch.Tensor | None:
    """Allocate (with torch) the scratch pa_decode needs, or None if it needs none."""
    nbytes = pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len,
                                       partition_tokens)
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def pa_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
              block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, max_seq_len: int,
              partition_tokens: int = 0, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode attention: out [B, Hq, D] for query [B, Hq, D] (one token per sequence)."""
    _need(query.dim() == 3 and out.shape == query.shape and out.is_contiguous(),
          "query/out: [num_seqs, num_heads, head_dim], out contiguous")
    _need(query.stride(2) == 1 and query.stride(1) == query.shape[2], "query heads/dims must be contiguous")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(query.dtype == out.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens: contiguous int32")
    b, hq, d = query.shape
    _need(block_table.shape[0] >= b and seq_lens.numel() >= b, "block_table/seq_lens shorter than batch")
    nb, bs, hkv, _ = key_cache.shape
    ws = workspace
    s = lib().pa_decode(_ptr(out), _ptr(query), query.stride(0), _ptr(key_cache), _ptr(value_cache),
                        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), b, hq, hkv, d, bs, nb,
                        float(scale), int(max_seq_len), int(partition_tokens), _ptr(ws),
                        0 if ws is None else ws.numel() * ws.element_size(), _dtype_code(query),
                        _stream(stream, out.device))
    _check(s, "pa_decode")
    return out


def _check_decode_append(out, query, key, value, key_cache, value_cache, block_table, seq_lens, slot_mapping,
                         fp8=False):
    """Tensor checks shared by pa_decode_append, pa_decode_append_noalloc and
    (fp8: bf16 rows, uint8 caches) pa_decode_append_fp8."""
    _need(query.dim() == 3 and out.shape == query.shape and out.is_contiguous(),
          "query/out: [num_seqs, num_heads, head_dim], out contiguous")
    _need(query.stride(2) == 1 and query.stride(1) == query.shape[2], "query heads/dims must be contiguous")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    if fp8:
        _need(query.dtype == out.dtype == key.dtype == value.dtype == torch.bfloat16,
              "query/out/key/value: bfloat16")
        _need(key_cache.dtype == value_cache.dtype == torch.uint8, "fp8 caches are uint8 codes")
    else:
        _need(query.dtype == out.dtype == key.dtype == value.dtype == key_cache.dtype == value_cache.dtype,
              "dtype mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens: contiguous int32")
    b, hq, d = query.shape
    nb, bs, hkv, _ = key_cache.shape
    _need(block_table.shape[0] >= b and seq_lens.numel() >= b, "block_table/seq_lens shorter than batch")
    _need(key.dim() == 3 and value.dim() == 3 and key.shape[0] >= b and value.shape[0] >= b and
          tuple(key.shape[1:]) == (hkv, d) and tuple(value.shape[1:]) == (hkv, d),
          "key/value: [num_seqs, num_kv_heads, head_dim]")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1 and value.stride(1) == d,
          "key/value heads and dims must be contiguous")
    if slot_mapping is not None:
        _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous() and slot_mapping.numel() >= b,
              "slot_mapping: contiguous int64 [num_seqs]")


def pa_decode_append(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                     key_cache: torch.Tensor, value_cache: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: torch.Tensor, scale: float, max_seq_len: int, slot_mapping: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: row b of key/value [B, Hkv, D] (sequence b's newest token,
    at position seq_lens[b] - 1) is written into the caches and attended to with
    the rest of the sequence; out [B, Hq, D].  slot_mapping (int64 [B], optional)
    receives the newest tokens' slots."""
    _check_decode_append(out, query, key, value, key_cache, value_cache, block_table, seq_lens, slot_mapping)
    b, hq, d = query.shape
    nb, bs, hkv, _ = key_cache.shape
    ws = workspace
    s = lib().pa_decode_append(_ptr(out), _ptr(query), query.stride(0), _ptr(key), key.stride(0), _ptr(value),
                               value.stride(0), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
                               _ptr(block_table), block_table.shape[1], _ptr(seq_lens), b, hq, hkv, d, bs, nb,
                               float(scale), int(max_seq_len), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _dtype_code(query),
                               _stream(stream, out.device))
    _check(s, "pa_decode_append")
    return out


def pa_decode_append_fp8(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         key_cache: torch.Tensor, value_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, scale: float, k_scale: float, v_scale: float, max_seq_len: int,
                         slot_mapping: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None, fp8_format: str = "e4m3") -> torch.Tensor:
    """The decode step over uint8 fp8 caches in one call: row b of key/value
    [B, Hkv, D] bf16 (sequence b's newest token) is stored as fp8 codes of
    x / k_scale (x / v_scale) in its slot and attended to with the rest of the
    sequence; out [B, Hq, D] bf16.  slot_mapping (int64 [B], optional) receives
    the newest tokens' slots."""
    _check_decode_append(out, query, key, value, key_cache, value_cache, block_table, seq_lens, slot_mapping,
                         fp8=True)
    b, hq, d = query.shape
    nb, bs, hkv, _ = key_cache.shape
    ws = workspace
    s = lib().pa_decode_append_fp8(_ptr(out), _ptr(query), query.stride(0), _ptr(key), key.stride(0), _ptr(value),
                                   value.stride(0), _ptr(key_cache), _ptr(value_cache), _ptr(slot_mapping),
                                   _ptr(block_table), block_table.shape[1], _ptr(seq_lens), b, hq, hkv, d, bs, nb,
                                   float(scale), _fp8_format(fp8_format), float(k_scale), float(v_scale),
                                   int(max_seq_len), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                   _stream(stream, out.device))
    _check(s, "pa_decode_append_fp8")
    return out


def pa_decode_append_noalloc(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                             key_cache: torch.Tensor, value_cache: torch.Tensor, block_table: torch.Tensor,
                             seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                             slot_mapping: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """pa_decode_append without a workspace: the library's own per-device
    scratch array serves instead, and nothing is allocated.  Calls that overlap
    on one device race on that array."""
    _check_decode_append(out, query, key, value, key_cache, value_cache, block_table, seq_lens, slot_mapping)
    b, hq, d = query.shape
    nb, bs, hkv, _ = key_cache.shape
    s = lib().pa_decode_append_noalloc(_ptr(out), _ptr(query), query.stride(0), _ptr(key), key.stride(0),
                                       _ptr(value), value.stride(0), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(slot_mapping), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                       b, hq, hkv, d, bs, nb, float(scale), int(max_seq_len), _dtype_code(query),
                                       _stream(stream, out.device))
    _check(s, "pa_decode_append_noalloc")
    return out


def pa_chunked_prefill_workspace_bytes(num_seqs: int, num_q_tokens: int, max_query_len: int, max_seq_len: int,
                                       num_heads: int, num_kv_heads: int, head_dim: int, dtype=None) -> int:
    """Workspace bytes of pa_chunked_prefill; dtype None or torch.bfloat16 gives
    the bf16 size, torch.float32 the fp32 route's."""
    code = PA_BF16 if dtype is None else _dtype_code(torch.empty(0, dtype=dtype))
    return int(lib().pa_chunked_prefill_workspace_bytes_ex(num_seqs, num_q_tokens, max_query_len, max_seq_len,
                                                           num_heads, num_kv_heads, head_dim, code))


def chunked_prefill_workspace(num_seqs: int, num_q_tokens: int, max_query_len: int, max_seq_len: int,
                              num_heads: int, num_kv_heads: int, head_dim: int, device="cuda",
                              dtype=None) -> torch.Tensor:
    nbytes = pa_chunked_prefill_workspace_bytes(num_seqs, num_q_tokens, max_query_len, max_seq_len, num_heads,
                                                num_kv_heads, head_dim, dtype)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def pa_chunked_prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, block_table: torch.Tensor, cu_query_lens: torch.Tensor,
                       seq_lens: torch.Tensor, scale: float, max_query_len: int, max_seq_len: int,
                       causal: bool = True, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Mixed-batch attention: out [num_q_tokens, Hq, D] for flattened query rows
    [num_q_tokens, Hq, D] (bf16 or fp32), requests delimited by cu_query_lens."""
    _need(query.dim() == 3 and out.shape == query.shape and out.is_contiguous(),
          "query/out: [num_q_tokens, num_heads, head_dim], out contiguous")
    _need(query.stride(2) == 1 and query.stride(1) == query.shape[2], "query heads/dims must be contiguous")
    _need(key_cache.dim() == 4 and key_cache.shape == value_cache.shape, "caches: [num_blocks, 16, Hkv, D]")
    _need(key_cache.is_contiguous() and value_cache.is_contiguous(), "caches must be contiguous")
    _need(query.dtype == out.dtype == key_cache.dtype == value_cache.dtype, "dtype mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.is_contiguous(),
          "block_table: contiguous int32 [num_seqs, max_blocks_per_req]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens: contiguous int32")
    _need(cu_query_lens.dtype == torch.int32 and cu_query_lens.is_contiguous(), "cu_query_lens: contiguous int32")
    b = seq_lens.numel()
    _need(cu_query_lens.numel() == b + 1 and block_table.shape[0] >= b, "cu_query_lens/block_table sizes")
    nq, hq, d = query.shape
    nb, bs, hkv, _ = key_cache.shape
    ws = workspace
    s = lib().pa_chunked_prefill(_ptr(out), _ptr(query), query.stride(0), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(block_table), block_table.shape[1], _ptr(cu_query_lens), _ptr(seq_lens),
                                 b, nq, int(max_query_len), int(max_seq_len), hq, hkv, d, bs, nb, float(scale),
                                 int(bool(causal)), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                 _dtype_code(query), _stream(stream, out.device))
    _check(s, "pa_chunked_prefill")
    return out


# ------------------------------------------------- contract checks (host) --
def _host(a, dtype):
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=dtype)


def pa_validate_block_tables(block_table, seq_lens, num_blocks: int, max_seq_len: int,
                             block_size: int = BLOCK_SIZE) -> None:
    """Check host copies of block_table [num_seqs, max_blocks_per_req] and
    seq_lens against the device-array contract; raises PaError naming the first
    offending entry."""
    bt = _host(block_table, np.int32)
    sl = _host(seq_lens, np.int32)
    _need(bt.ndim == 2 and bt.shape[0] >= sl.shape[0], "block_table: [num_seqs, max_blocks_per_req]")
    _check(lib().pa_validate_block_tables(bt.ctypes.data, bt.shape[1], sl.ctypes.data, sl.shape[0], int(num_blocks),
                                          int(block_size), int(max_seq_len)), "pa_validate_block_tables")


def pa_validate_slot_mapping(slot_mapping, num_blocks: int, block_size: int = BLOCK_SIZE) -> None:
    """No two tokens of one scatter write the same slot (host copy)."""
    sm = _host(slot_mapping, np.int64)
    _check(lib().pa_validate_slot_mapping(sm.ctypes.data, sm.shape[0], int(num_blocks), int(block_size)),
           "pa_validate_slot_mapping")


def pa_validate_query_lens(cu_query_lens, seq_lens, num_q_tokens: int, max_query_len: int) -> None:
    """cu_query_lens [num_seqs + 1] against seq_lens and the host bounds (host copies)."""
    cu = _host(cu_query_lens, np.int32)
    sl = _host(seq_lens, np.int32)
    _need(cu.shape[0] == sl.shape[0] + 1, "cu_query_lens: [num_seqs + 1]")
    _check(lib().pa_validate_query_lens(cu.ctypes.data, sl.ctypes.data, sl.shape[0], int(num_q_tokens),
                                        int(max_query_len)), "pa_validate_query_lens")


# ------------------------------------------------------------------ probes --
def pa_probe_stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, stream=None) -> None:
    """Read every byte of `src` once (HBM read-bandwidth probe); `sink` is a
    1-element int32/uint32 device tensor that is written only by a fluke."""
    _need(src.is_contiguous() and sink.numel() >= 1, "src contiguous, sink of one element")
    nbytes = src.numel() * src.element_size()
    s = lib().pa_probe_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink), workgroups,
                                   _stream(stream, src.device))
    _check(s, "pa_probe_stream_read")


def pa_probe_copy(dst: torch.Tensor, src: torch.Tensor, workgroups: int = 0, stream=None) -> None:
    """dst[:] = src[:] bytewise (copy-bandwidth probe, and the known-size
    transfer for scaling traffic counters)."""
    _need(src.is_contiguous() and dst.is_contiguous(), "contiguous tensors")
    nbytes = src.numel() * src.element_size()
    _need(dst.numel() * dst.element_size() >= nbytes, "dst smaller than src")
    s = lib().pa_probe_copy(_ptr(dst), _ptr(src), nbytes - nbytes % 16, workgroups, _stream(stream, src.device))
    _check(s, "pa_probe_copy")


def pa_probe_mfma(sink: torch.Tensor, workgroups: int, iters: int, stream=None) -> int:
    """Run the matrix-core rate probe; returns the flops it performs
    (workgroups * 4 waves * iters * 4 * 32768)."""
    _need(sink.numel() >= 1, "sink of one element")
    s = lib().pa_probe_mfma(_ptr(sink), int(workgroups), int(iters), _stream(stream, sink.device))
    _check(s, "pa_probe_mfma")
    return int(workgroups) * 4 * int(iters) * 4 * 32768
