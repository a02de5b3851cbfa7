"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and shares
no code with it.

The arithmetic lives in ``pa_oracle.c`` (plain C, fp64, two-pass softmax,
explicit per-token gather through the block table).  This file compiles it with
gcc, wraps it with ctypes and adds numpy-level helpers that build a cache the
way a caller would (poisoned pool, then scatter) before attending over it.

Every function here follows "AI Infra入门干货总结：大模型是如何高效推理的":
section "Paged Attention" for slots and the scatter, section "Attention
(FlashAttention, Scaled Dot-Product Attention)" for the attention itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_lib = None
_lock = threading.Lock()

F32, BF16, E4M3, E5M2 = 0, 1, 2, 3
FP8_FORMATS = {"e4m3": E4M3, "e5m2": E5M2}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into libpa_oracle.so with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out: str) -> str:
    """The oracle under gcc's ASan and UBSan (for the sanitizer tests, which load
    it through PA_ORACLE_LIB with gcc's runtimes preloaded)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC,
                    "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("PA_ORACLE_LIB")      # a deliberately broken build, for the pin tests
            if not path:
                build(force=False)
                path = _LIB_PATH
            L = ctypes.CDLL(path)
            L.oracle_max_threads.restype = ctypes.c_int32
            L.oracle_max_threads.argtypes = []
            L.oracle_set_threads.restype = None
            L.oracle_set_threads.argtypes = [ctypes.c_int32]
            L.oracle_slot.restype = ctypes.c_int64
            L.oracle_slot.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32]
            L.oracle_slot_mapping.restype = None
            L.oracle_slot_mapping.argtypes = [_i32p, ctypes.c_int64, _i32p, _i32p, ctypes.c_int64,
                                              ctypes.c_int32, _i64p]
            L.oracle_reshape_and_cache.restype = None
            L.oracle_reshape_and_cache.argtypes = [
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, _i64p, ctypes.c_int64,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
            L.oracle_attention.restype = None
            L.oracle_attention.argtypes = [
                _f64p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                _i32p, ctypes.c_int64, _i32p, _i32p, ctypes.c_int32,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.c_double, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                ctypes.c_double, _f64p, ctypes.c_int64]
            L.oracle_e4m3_value.restype = ctypes.c_double
            L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
            L.oracle_e4m3_encode.restype = ctypes.c_uint8
            L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
            L.oracle_e5m2_value.restype = ctypes.c_double
            L.oracle_e5m2_value.argtypes = [ctypes.c_uint8]
            L.oracle_e5m2_encode.restype = ctypes.c_uint8
            L.oracle_e5m2_encode.argtypes = [ctypes.c_float]
            L.oracle_reshape_and_cache_fp8.restype = None
            L.oracle_reshape_and_cache_fp8.argtypes = [
                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, _i64p, ctypes.c_int64,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                ctypes.c_int32]
            L.oracle_rope_table.restype = None
            L.oracle_rope_table.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
            L.oracle_rope_qkv.restype = None
            L.oracle_rope_qkv.argtypes = [
                _f64p, _f64p, _f64p, ctypes.c_void_p, ctypes.c_int64, _i64p,
                ctypes.POINTER(ctypes.c_float), ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
            L.oracle_copy_blocks.restype = None
            L.oracle_copy_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int64, ctypes.c_int64, _i64p, ctypes.c_int64]
            _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> None:
    """Threads the attention loop uses from now on (for timing only)."""
    lib().oracle_set_threads(int(n))


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ slots --
def slot(bt_row, pos: int, block_size: int = 16) -> int:
    row = _c(bt_row, np.int32)
    return int(lib().oracle_slot(_p(row, _i32p), int(pos), int(block_size)))


def slot_mapping(block_table, token_seq, token_pos, block_size: int = 16) -> np.ndarray:
    bt = _c(block_table, np.int32)
    seq = _c(token_seq, np.int32)
    pos = _c(token_pos, np.int32)
    out = np.empty(len(seq), np.int64)
    lib().oracle_slot_mapping(_p(bt, _i32p), bt.shape[1], _p(seq, _i32p), _p(pos, _i32p),
                              len(seq), int(block_size), _p(out, _i64p))
    return out


# ---------------------------------------------------------------- scatter --
def reshape_and_cache(key, value, key_cache, value_cache, slots, block_size: int = 16):
    """In-place scatter into numpy caches [num_blocks, block_size, Hkv, D].

    key/value: [num_tokens, Hkv, D] in the cache's storage dtype (uint16 bf16
    bits or float32); rows may be strided along the token axis."""
    assert key_cache.flags.c_contiguous and value_cache.flags.c_contiguous
    assert key.dtype == key_cache.dtype == value.dtype == value_cache.dtype
    n = key.shape[0]
    if n == 0:
        return
    hkv, d = key_cache.shape[2], key_cache.shape[3]
    assert key.strides[1:] == (d * key.itemsize, key.itemsize)
    assert value.strides[1:] == (d * value.itemsize, value.itemsize)
    sm = _c(slots, np.int64)
    lib().oracle_reshape_and_cache(
        key.ctypes.data, key.strides[0] // key.itemsize, value.ctypes.data,
        value.strides[0] // value.itemsize, key_cache.ctypes.data, value_cache.ctypes.data,
        _p(sm, _i64p), n, int(block_size), hkv, d, key.itemsize)


# -------------------------------------------------------------- attention --
def _dtype_of(a):
    return {np.dtype(np.uint16): BF16, np.dtype(np.float32): F32, np.dtype(np.uint8): E4M3}[a.dtype]


def attention(query, key_cache, value_cache, block_table, cu_query_lens, seq_lens,
              num_heads: int, scale: float, causal: bool, return_probs: bool = False,
              k_scale: float = 1.0, v_scale: float = 1.0, fp8_format: str = "e4m3"):
    """fp64 attention over the paged cache; returns out [num_q_tokens, Hq, D]
    (and the probability rows [num_q_tokens, Hq, max_seq_len] if asked).

    The query is bf16 bits (uint16) or float32; the caches are the same dtype,
    or fp8 codes (uint8, in fp8_format: "e4m3" or "e5m2") standing for code
    value * k_scale / v_scale."""
    dtype = _dtype_of(query)
    kv_dtype = _dtype_of(key_cache)
    if kv_dtype == E4M3:
        kv_dtype = FP8_FORMATS[fp8_format]
    assert value_cache.dtype == key_cache.dtype and dtype != E4M3
    assert kv_dtype == dtype or kv_dtype in (E4M3, E5M2)
    q = query
    assert q.strides[1:] == (q.shape[2] * q.itemsize, q.itemsize)
    bt = _c(block_table, np.int32)
    cu = _c(cu_query_lens, np.int32)
    sl = _c(seq_lens, np.int32)
    nq, _, d = q.shape
    hkv = key_cache.shape[2]
    out = np.zeros((nq, num_heads, d), np.float64)
    probs = None
    pstride = 0
    if return_probs:
        pstride = int(sl.max()) if len(sl) else 0
        probs = np.zeros((nq, num_heads, max(pstride, 1)), np.float64)
    if nq:
        lib().oracle_attention(
            _p(out, _f64p), q.ctypes.data, q.strides[0] // q.itemsize,
            key_cache.ctypes.data, value_cache.ctypes.data, _p(bt, _i32p), bt.shape[1],
            _p(cu, _i32p), _p(sl, _i32p), len(sl), num_heads, hkv, d, key_cache.shape[1],
            float(scale), int(bool(causal)), dtype, kv_dtype, float(k_scale), float(v_scale),
            _p(probs, _f64p) if probs is not None else None, pstride)
    return (out, probs) if return_probs else out


# --------------------------------------------------------- copy-on-write --
def copy_blocks(kv, block_mapping):
    """In place on a numpy cache kv [num_layers, 2, num_blocks, ...] (the
    pages' layout): for each (src, dst) pair in order, block dst of every
    layer's K and V becomes a copy of block src; pairs outside the pool are
    skipped."""
    assert kv.flags.c_contiguous and kv.ndim >= 3 and kv.shape[1] == 2
    num_layers, _, num_blocks = kv.shape[:3]
    block_bytes = kv[0, 0, 0].nbytes
    pairs = _c(block_mapping, np.int64).reshape(-1, 2)
    base = kv.ctypes.data
    lib().oracle_copy_blocks(base, base + num_blocks * block_bytes, 2 * num_blocks * block_bytes, num_layers,
                             num_blocks, block_bytes, _p(pairs, _i64p), len(pairs))


# -------------------------------------------------------------- fp8 cache --
def e4m3_value(code: int) -> float:
    """The number an OCP E4M3 code stands for (NaN for 0x7F / 0xFF)."""
    return float(lib().oracle_e4m3_value(int(code)))


def e4m3_encode(y) -> np.ndarray:
    """E4M3 codes of float32 values: nearest, ties to even, saturating at 448."""
    y = np.ascontiguousarray(y, np.float32)
    enc = lib().oracle_e4m3_encode
    return np.array([enc(float(v)) for v in y.ravel()], np.uint8).reshape(y.shape)


def e5m2_value(code: int) -> float:
    """The number an OCP E5M2 code stands for (+-inf for 0x7C / 0xFC, NaN for
    the other codes of exponent field 31)."""
    return float(lib().oracle_e5m2_value(int(code)))


def e5m2_encode(y) -> np.ndarray:
    """E5M2 codes of float32 values: nearest, ties to even, saturating at 57344."""
    y = np.ascontiguousarray(y, np.float32)
    enc = lib().oracle_e5m2_encode
    return np.array([enc(float(v)) for v in y.ravel()], np.uint8).reshape(y.shape)


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slots, k_scale: float, v_scale: float,
                          block_size: int = 16, fp8_format: str = "e4m3"):
    """In-place fp8 scatter into uint8 caches [num_blocks, block_size, Hkv, D]:
    code = encode(x / scale) in fp8_format ("e4m3" or "e5m2") with the
    division in float32.  key/value are bf16 bits (uint16) or float32, token
    rows may be strided."""
    assert key_cache.dtype == value_cache.dtype == np.uint8
    assert key_cache.flags.c_contiguous and value_cache.flags.c_contiguous
    assert key.dtype == value.dtype
    n = key.shape[0]
    if n == 0:
        return
    hkv, d = key_cache.shape[2], key_cache.shape[3]
    assert key.strides[1:] == (d * key.itemsize, key.itemsize)
    assert value.strides[1:] == (d * value.itemsize, value.itemsize)
    sm = _c(slots, np.int64)
    lib().oracle_reshape_and_cache_fp8(
        key.ctypes.data, key.strides[0] // key.itemsize, value.ctypes.data,
        value.strides[0] // value.itemsize, key_cache.ctypes.data, value_cache.ctypes.data,
        _p(sm, _i64p), n, int(block_size), hkv, d, _dtype_of(key), float(k_scale), float(v_scale),
        {"e4m3": 0, "e5m2": 1}[fp8_format])


# ------------------------------------------------------ RoPE + QKV split --
def rope_table(max_position: int, rotary_dim: int, base: float) -> np.ndarray:
    """fp64 [max_position, rotary_dim]: cos(p * theta_i) then sin(p * theta_i),
    theta_i = base^(-2i / rotary_dim)."""
    t = np.empty((max_position, rotary_dim), np.float64)
    lib().oracle_rope_table(_p(t, _f64p), int(max_position), int(rotary_dim), float(base))
    return t


def rope_qkv(qkv, positions, cos_sin, rotary_dim: int, neox_style: bool, num_heads: int,
             num_kv_heads: int, head_dim: int):
    """Split a fused projection qkv [num_tokens, (Hq + 2 Hkv) * D] (storage dtype:
    uint16 bf16 bits or float32; rows may be strided) and rotate Q and K.

    cos_sin is the float32 table the GPU reads.  Returns fp64 arrays
    (q [n, Hq, D], k [n, Hkv, D], v [n, Hkv, D])."""
    dtype = BF16 if qkv.dtype == np.uint16 else F32
    assert qkv.strides[1] == qkv.itemsize
    n = qkv.shape[0]
    assert qkv.shape[1] >= (num_heads + 2 * num_kv_heads) * head_dim
    pos = _c(positions, np.int64)
    assert n == 0 or (pos.min() >= 0 and pos.max() < cos_sin.shape[0])
    cs = _c(cos_sin, np.float32)
    assert cs.shape[1] == rotary_dim
    q = np.zeros((n, num_heads, head_dim), np.float64)
    k = np.zeros((n, num_kv_heads, head_dim), np.float64)
    v = np.zeros((n, num_kv_heads, head_dim), np.float64)
    if n:
        lib().oracle_rope_qkv(_p(q, _f64p), _p(k, _f64p), _p(v, _f64p), qkv.ctypes.data,
                              qkv.strides[0] // qkv.itemsize, _p(pos, _i64p),
                              cs.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(rotary_dim),
                              int(bool(neox_style)), n, num_heads, num_kv_heads, head_dim, dtype)
    return q, k, v


# ------------------------------------------------- whole-workload helpers --
def build_cache(w, which: str = "all", caches=None):
    """Caller-side cache construction for a workload: a NaN-poisoned pool, then
    the scatter of the chosen tokens through slots computed from the block
    table.  Returns (key_cache, value_cache) in storage format."""
    if caches is None:
        kc, vc = w.poisoned_cache(), w.poisoned_cache()
    else:
        kc, vc = caches
    for _, k, v, slots in _token_rows(w, which):
        reshape_and_cache(k, v, kc, vc, slots, w.block_size)
    return kc, vc


def _token_rows(w, which: str):
    """Per sequence with tokens to write: (b, K rows, V rows, slots), the rows
    in storage format, the slots from this module's slot function over the
    workload's block table.  Values are drawn a few sequences ahead on worker
    threads (workloads.iter_kv), so a full-size pool is built in seconds."""
    seq, pos = w.tokens(which)
    if not len(seq):
        return
    for b, k, v in w.iter_kv(np.unique(seq), encode=True):
        p = pos[seq == b]
        slots = slot_mapping(w.block_table, np.full(len(p), b, np.int32), p, w.block_size)
        yield b, k[p], v[p], slots


def build_cache_fp8(w, k_scale: float, v_scale: float, which: str = "all", fp8_format: str = "e4m3"):
    """As build_cache, into fp8 caches (uint8, every byte 0x7F first, a NaN code
    in both formats) through the fp8 scatter."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc, vc = np.full(shape, 0x7F, np.uint8), np.full(shape, 0x7F, np.uint8)
    for _, k, v, slots in _token_rows(w, which):
        reshape_and_cache_fp8(k, v, kc, vc, slots, k_scale, v_scale, w.block_size, fp8_format)
    return kc, vc


def run_fp8(w, k_scale: float, v_scale: float, fp8_format: str = "e4m3"):
    """Oracle output over an fp8 cache of the workload: [num_q_tokens, Hq, D] fp64."""
    kc, vc = build_cache_fp8(w, k_scale, v_scale, "all", fp8_format)
    q = w.encode(w.queries())
    return attention(q, kc, vc, w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads, w.scale, w.causal,
                     k_scale=k_scale, v_scale=v_scale, fp8_format=fp8_format)


def run(w, return_probs: bool = False):
    """Oracle output for a whole workload: [num_q_tokens, Hq, D] fp64."""
    kc, vc = build_cache(w, "all")
    q = w.encode(w.queries())
    return attention(q, kc, vc, w.block_table, w.cu_query_lens, w.seq_lens, w.num_heads,
                     w.scale, w.causal, return_probs)


def run_sequences(w, seqs, fp8_scales=None, fp8_format: str = "e4m3"):
    """Oracle output for a few sequences of a large workload.

    The chosen sequences' blocks are relabelled into a compact pool (the result
    does not depend on the physical block ids) so that the oracle never holds
    the whole pool.  With fp8_scales = (k_scale, v_scale) the cache is E4M3.
    Returns {seq: [query_len, Hq, D] fp64}."""
    res = {}
    for b, k, v in w.iter_kv(seqs, encode=True):
        L = int(w.seq_lens[b])
        nblk = (L + w.block_size - 1) // w.block_size
        table = np.arange(max(nblk, 1), dtype=np.int32)[None, :]
        shape = (max(nblk, 1), w.block_size, w.num_kv_heads, w.head_dim)
        if fp8_scales is not None:
            kc = np.full(shape, 0x7F, np.uint8)
        elif w.dtype == "bf16":
            kc = np.full(shape, 0x7FC0, np.uint16)
        else:
            kc = np.full(shape, np.nan, np.float32)
        vc = kc.copy()
        pos = np.arange(L, dtype=np.int32)
        slots = slot_mapping(table, np.zeros(L, np.int32), pos, w.block_size)
        if fp8_scales is not None:
            reshape_and_cache_fp8(k, v, kc, vc, slots, fp8_scales[0], fp8_scales[1], w.block_size, fp8_format)
        else:
            reshape_and_cache(k, v, kc, vc, slots, w.block_size)
        q = w.encode(w.query(b))
        cu = np.array([0, q.shape[0]], np.int32)
        ks, vs = fp8_scales if fp8_scales is not None else (1.0, 1.0)
        res[b] = attention(q, kc, vc, table, cu, np.array([L], np.int32), w.num_heads,
                           w.scale, w.causal, k_scale=ks, v_scale=vs, fp8_format=fp8_format)
    return res
