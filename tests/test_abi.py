"""The C ABI without a GPU: libpa.so loads, exports every function include/pa.h
declares, and its host-side argument checks answer before any launch."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_432_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pa.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return pa.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"pa_slot_mapping", "pa_reshape_and_cache", "pa_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libpa.so does not export {n}"
    assert pa.pa_abi_version() == 1


def test_status_strings(L):
    assert pa.pa_status_string(0) == "PA_OK"
    assert pa.pa_status_string(3) == "PA_ERR_WORKSPACE"


def _decode(L, **kw):
    args = dict(out=16, query=16, q_token_stride=4096, key_cache=16, value_cache=16, block_table=16,
                max_blocks_per_req=8, seq_lens=16, num_seqs=2, num_heads=32, num_kv_heads=8,
                head_dim=128, block_size=16, num_blocks=10, scale=0.088, max_seq_len=100,
                partition_tokens=0, workspace=None, workspace_bytes=0, dtype=1, stream=None)
    args.update(kw)
    return L.pa_decode(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=32), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=24, num_kv_heads=8), pa.PA_ERR_UNSUPPORTED),       # group 3
    (dict(num_heads=30, num_kv_heads=8), pa.PA_ERR_INVALID_ARG),       # not a multiple
    (dict(dtype=7), pa.PA_ERR_UNSUPPORTED),
    (dict(out=None), pa.PA_ERR_INVALID_ARG),
    (dict(partition_tokens=100), pa.PA_ERR_INVALID_ARG),               # not a multiple of 16
    (dict(max_seq_len=200), pa.PA_ERR_INVALID_ARG),                    # beyond the table
    (dict(q_token_stride=100), pa.PA_ERR_INVALID_ARG),
    (dict(query=24), pa.PA_ERR_INVALID_ARG),                           # misaligned
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(scale=0.0), pa.PA_ERR_INVALID_ARG),                          # the scale must be > 0
    (dict(scale=-0.088), pa.PA_ERR_INVALID_ARG),
    (dict(partition_tokens=32), pa.PA_ERR_WORKSPACE),                  # split without workspace
    (dict(num_seqs=-1), pa.PA_ERR_INVALID_ARG),
])
def test_decode_rejects_before_launch(L, kw, status):
    assert _decode(L, **kw) == status
    assert pa.pa_last_error_message()


def test_decode_empty_batch_is_ok(L):
    assert _decode(L, num_seqs=0) == pa.PA_OK


def _decode_append(L, **kw):
    args = dict(out=16, query=16, q_token_stride=4096, key=16, key_token_stride=1024, value=16,
                value_token_stride=1024, key_cache=16, value_cache=16, slot_mapping=16, block_table=16,
                max_blocks_per_req=8, seq_lens=16, num_seqs=2, num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=10, scale=0.088, max_seq_len=100, workspace=None, workspace_bytes=0,
                dtype=1, stream=None)
    args.update(kw)
    return L.pa_decode_append(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=32), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=24, num_kv_heads=8), pa.PA_ERR_UNSUPPORTED),       # group 3
    (dict(dtype=7), pa.PA_ERR_UNSUPPORTED),
    (dict(key=None), pa.PA_ERR_INVALID_ARG),
    (dict(value=None), pa.PA_ERR_INVALID_ARG),
    (dict(key_token_stride=1000), pa.PA_ERR_INVALID_ARG),              # shorter than a row
    (dict(value_token_stride=1028), pa.PA_ERR_INVALID_ARG),            # rows not 16-byte aligned
    (dict(key=24), pa.PA_ERR_INVALID_ARG),                             # misaligned
    (dict(max_seq_len=200), pa.PA_ERR_INVALID_ARG),                    # beyond the table
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(scale=0.0), pa.PA_ERR_INVALID_ARG),
    (dict(scale=-0.088), pa.PA_ERR_INVALID_ARG),
    (dict(num_seqs=-1), pa.PA_ERR_INVALID_ARG),
])
def test_decode_append_rejects_before_launch(L, kw, status):
    assert _decode_append(L, **kw) == status
    assert pa.pa_last_error_message()


def test_decode_append_empty_batch_is_ok(L):
    assert _decode_append(L, num_seqs=0) == pa.PA_OK


def _decode_append_fp8(L, **kw):
    args = dict(out=16, query=16, q_token_stride=4096, key=16, key_token_stride=1024, value=16,
                value_token_stride=1024, key_cache=16, value_cache=16, slot_mapping=16, block_table=16,
                max_blocks_per_req=8, seq_lens=16, num_seqs=2, num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=10, scale=0.088, format=0, k_scale=0.5, v_scale=0.5, max_seq_len=100,
                workspace=None, workspace_bytes=0, stream=None)
    args.update(kw)
    return L.pa_decode_append_fp8(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=32), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=24, num_kv_heads=8), pa.PA_ERR_UNSUPPORTED),       # group 3
    (dict(format=2), pa.PA_ERR_UNSUPPORTED),
    (dict(key=None), pa.PA_ERR_INVALID_ARG),
    (dict(value=None), pa.PA_ERR_INVALID_ARG),
    (dict(key_token_stride=1000), pa.PA_ERR_INVALID_ARG),              # shorter than a row
    (dict(value_token_stride=1028), pa.PA_ERR_INVALID_ARG),            # rows not 16-byte aligned
    (dict(key=24), pa.PA_ERR_INVALID_ARG),                             # misaligned
    (dict(max_seq_len=200), pa.PA_ERR_INVALID_ARG),                    # beyond the table
    (dict(scale=0.0), pa.PA_ERR_INVALID_ARG),
    (dict(k_scale=-1.0), pa.PA_ERR_INVALID_ARG),
    (dict(v_scale=float("inf")), pa.PA_ERR_INVALID_ARG),
    (dict(num_seqs=-1), pa.PA_ERR_INVALID_ARG),
])
def test_decode_append_fp8_rejects_before_launch(L, kw, status):
    assert _decode_append_fp8(L, **kw) == status
    assert pa.pa_last_error_message()


def test_decode_append_fp8_empty_batch_is_ok(L):
    assert _decode_append_fp8(L, num_seqs=0) == pa.PA_OK
    assert _decode_append_fp8(L, num_seqs=0, format=1) == pa.PA_OK


def test_fused_fp8_scatter_checks(L):
    args = dict(slot_mapping=16, block_table=16, max_blocks_per_req=4, num_seqs=2, token_seq=16, token_pos=16,
                key=16, key_token_stride=1024, value=16, value_token_stride=1024, key_cache=16, value_cache=16,
                num_tokens=3, num_blocks=10, block_size=16, num_kv_heads=8, head_dim=128, dtype=1, k_scale=0.5,
                v_scale=0.5, stream=None)
    call = lambda **kw: L.pa_slot_mapping_and_cache_fp8(*{**args, **kw}.values())
    assert call(num_tokens=0) == pa.PA_OK
    assert call(block_size=8) == pa.PA_ERR_UNSUPPORTED
    assert call(dtype=5) == pa.PA_ERR_UNSUPPORTED
    assert call(k_scale=0.0) == pa.PA_ERR_INVALID_ARG
    assert call(v_scale=float("inf")) == pa.PA_ERR_INVALID_ARG
    assert call(slot_mapping=None) == pa.PA_ERR_INVALID_ARG
    assert call(token_pos=None) == pa.PA_ERR_INVALID_ARG
    assert call(key_token_stride=1000) == pa.PA_ERR_INVALID_ARG
    assert call(num_kv_heads=1, head_dim=100, key_token_stride=100,
                value_token_stride=100) == pa.PA_ERR_UNSUPPORTED   # rows of 100: not a multiple of 16


def test_workspace_query(L):
    assert pa.pa_decode_workspace_bytes(4, 32, 8, 128, 100, -1) == 0
    assert pa.pa_decode_workspace_bytes(4, 32, 8, 128, 100, 16) > 0
    # explicit partitions: one 132-float record per (sequence, head, partition)
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 8192, 512) == 64 * 32 * 16 * 132 * 4
    assert pa.pa_decode_partition_tokens(4, 8, 100, -1) == 112
    assert pa.pa_decode_partition_tokens(64, 8, 8192, 256) == 256
    # automatic: the balanced stream mode (reported as 0 tokens per partition);
    # past 4096 sequences, automatic fixed partitions of 256..1024 tokens
    assert pa.pa_decode_partition_tokens(64, 8, 8192, 0) == 0
    pt = pa.pa_decode_partition_tokens(5000, 8, 8192, 0)
    assert pt % 16 == 0 and 256 <= pt <= 1024


def test_scatter_and_slot_checks(L):
    # every call here fails its checks (or is empty) and so launches nothing
    assert L.pa_reshape_and_cache(16, 1024, 16, 1024, 16, 16, 16, 0, 10, 16, 8, 128, 1, None) == pa.PA_OK
    assert L.pa_reshape_and_cache(16, 1000, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_reshape_and_cache(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 8, 8, 128, 1, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_reshape_and_cache(None, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_slot_mapping(16, 16, 4, 2, 16, 16, 0, 16, None) == pa.PA_OK
    assert L.pa_slot_mapping(16, 16, 4, 2, 16, 16, 3, 8, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_slot_mapping(None, 16, 4, 2, 16, 16, 3, 16, None) == pa.PA_ERR_INVALID_ARG


def _prefill(L, **kw):
    args = dict(out=16, query=16, q_token_stride=4096, key_cache=16, value_cache=16, block_table=16,
                max_blocks_per_req=8, cu_query_lens=16, seq_lens=16, num_seqs=2, num_q_tokens=40,
                max_query_len=39, max_seq_len=100, num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, num_blocks=10, scale=0.088, causal=1, workspace=None, workspace_bytes=0,
                dtype=1, stream=None)
    args.update(kw)
    return L.pa_chunked_prefill(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), pa.PA_ERR_UNSUPPORTED),                            # bf16 or fp32
    (dict(dtype=0), pa.PA_ERR_WORKSPACE),                              # fp32: its row table is needed
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=8), pa.PA_ERR_UNSUPPORTED),
    (dict(num_heads=24), pa.PA_ERR_UNSUPPORTED),
    (dict(causal=2), pa.PA_ERR_INVALID_ARG),
    (dict(cu_query_lens=None), pa.PA_ERR_INVALID_ARG),
    (dict(max_seq_len=200), pa.PA_ERR_INVALID_ARG),
    (dict(query=8), pa.PA_ERR_INVALID_ARG),
    (dict(num_q_tokens=-1), pa.PA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), pa.PA_ERR_INVALID_ARG),
    (dict(scale=0.0), pa.PA_ERR_INVALID_ARG),
    (dict(scale=-0.088), pa.PA_ERR_INVALID_ARG),
])
def test_chunked_prefill_rejects_before_launch(L, kw, status):
    assert _prefill(L, **kw) == status
    assert pa.pa_last_error_message()


def test_chunked_prefill_workspace_by_dtype(L):
    """The bf16 size is the plain query's; the fp32 route holds a key count and
    a block-table row (the blocks of max_seq_len) per query row, then a decode
    workspace for that many rows."""
    shape = (3, 700, 512, 4000, 32, 8, 128)
    bf = L.pa_chunked_prefill_workspace_bytes(*shape)
    assert bf > 0 and L.pa_chunked_prefill_workspace_bytes_ex(*shape, pa.PA_BF16) == bf
    f32 = L.pa_chunked_prefill_workspace_bytes_ex(*shape, pa.PA_F32)
    align = lambda n: (n + 255) // 256 * 256
    assert f32 >= align(4 * 700) + align(4 * 700 * 250) + L.pa_decode_workspace_bytes(700, 32, 8, 128, 4000, 0)
    assert L.pa_chunked_prefill_workspace_bytes_ex(0, 700, 512, 4000, 32, 8, 128, pa.PA_F32) == 0
    # a workspace of the fp32 size passes the workspace check (null data
    # pointers then fail the argument check, still before any launch)
    assert _prefill(L, dtype=0, workspace=256, workspace_bytes=f32, out=None) == pa.PA_ERR_INVALID_ARG


def test_chunked_prefill_empty_is_ok(L):
    assert _prefill(L, num_seqs=0) == pa.PA_OK
    assert _prefill(L, num_q_tokens=0) == pa.PA_OK


def test_probes_reject_before_launch(L):
    """Probe arguments are checked on the host; none of these launches."""
    assert L.pa_probe_mfma(None, 4, 10, None) == pa.PA_ERR_INVALID_ARG       # null sink
    assert L.pa_probe_mfma(8, 0, 10, None) == pa.PA_ERR_INVALID_ARG          # no workgroups
    assert L.pa_probe_mfma(8, 4, -1, None) == pa.PA_ERR_INVALID_ARG          # negative rounds
    assert L.pa_probe_stream_read(8, 24, 8, 0, None) == pa.PA_ERR_INVALID_ARG  # not a multiple of 16
    assert L.pa_probe_copy(16, 32, 16, -1, None) == pa.PA_ERR_INVALID_ARG      # negative grid
    assert L.pa_probe_stream_read(None, 0, None, 0, None) == pa.PA_OK         # nothing to read


def _rope(L, **kw):
    a = dict(query_out=16, q_stride=4096, qkv=16, qkv_stride=6144, positions=16, cos_sin=16, max_position=8192,
             rotary_dim=128, neox=1, key_cache=16, value_cache=16, slots=16, num_tokens=5, num_blocks=10,
             block_size=16, num_heads=32, num_kv_heads=8, head_dim=128, dtype=1)
    a.update(kw)
    return L.pa_rope_reshape_and_cache(a["query_out"], a["q_stride"], a["qkv"], a["qkv_stride"], a["positions"],
                                       a["cos_sin"], a["max_position"], a["rotary_dim"], a["neox"],
                                       a["key_cache"], a["value_cache"], a["slots"], a["num_tokens"],
                                       a["num_blocks"], a["block_size"], a["num_heads"], a["num_kv_heads"],
                                       a["head_dim"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(rotary_dim=120), pa.PA_ERR_UNSUPPORTED),           # not a multiple of 16
    (dict(rotary_dim=0), pa.PA_ERR_UNSUPPORTED),
    (dict(rotary_dim=144), pa.PA_ERR_UNSUPPORTED),           # beyond head_dim
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(block_size=32), pa.PA_ERR_UNSUPPORTED),
    (dict(dtype=7), pa.PA_ERR_UNSUPPORTED),
    (dict(qkv_stride=6000), pa.PA_ERR_INVALID_ARG),          # narrower than Q | K | V
    (dict(q_stride=4000), pa.PA_ERR_INVALID_ARG),
    (dict(qkv_stride=6148), pa.PA_ERR_INVALID_ARG),          # bf16 rows off 16-byte boundaries
    (dict(qkv=24), pa.PA_ERR_INVALID_ARG),
    (dict(cos_sin=None), pa.PA_ERR_INVALID_ARG),
    (dict(positions=None), pa.PA_ERR_INVALID_ARG),
    (dict(max_position=0), pa.PA_ERR_INVALID_ARG),
    (dict(num_tokens=-1), pa.PA_ERR_INVALID_ARG),
    (dict(query_out=16, qkv=16, q_stride=4096, qkv_stride=6144), pa.PA_ERR_INVALID_ARG),   # in place, other stride
])
def test_rope_rejects_before_launch(L, kw, status):
    assert _rope(L, **kw) == status
    assert pa.pa_last_error_message()


def test_rope_empty_is_ok(L):
    assert _rope(L, num_tokens=0) == pa.PA_OK


def test_fp8_entries_reject_before_launch(L):
    """fp8 scatter and decode argument checks; none of these launches."""
    sc = L.pa_reshape_and_cache_fp8
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 0, 10, 16, 8, 128, 1, 1.0, 1.0, None) == pa.PA_OK
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, 0.0, 1.0, None) == pa.PA_ERR_INVALID_ARG
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, 1.0, float("inf"), None) == pa.PA_ERR_INVALID_ARG
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 3, 1.0, 1.0, None) == pa.PA_ERR_UNSUPPORTED
    assert sc(16, 1000, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, 1.0, 1.0, None) == pa.PA_ERR_INVALID_ARG
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 32, 8, 128, 1, 1.0, 1.0, None) == pa.PA_ERR_UNSUPPORTED
    dc = L.pa_decode_fp8

    def dec(**kw):
        a = dict(out=16, q=16, qs=4096, kc=16, vc=16, bt=16, mbr=512, sl=16, b=4, hq=32, hkv=8, d=128, bs=16,
                 nb=100, scale=0.088, ks=1.0, vs=1.0, msl=8192)
        a.update(kw)
        return dc(a["out"], a["q"], a["qs"], a["kc"], a["vc"], a["bt"], a["mbr"], a["sl"], a["b"], a["hq"], a["hkv"],
                  a["d"], a["bs"], a["nb"], a["scale"], a["ks"], a["vs"], a["msl"], None, 0, None)

    assert dec(b=0) == pa.PA_OK
    assert dec(ks=-1.0) == pa.PA_ERR_INVALID_ARG
    assert dec(scale=-0.088) == pa.PA_ERR_INVALID_ARG        # the softmax scale must be > 0
    assert dec(scale=0.0) == pa.PA_ERR_INVALID_ARG
    assert dec(vs=float("nan")) == pa.PA_ERR_INVALID_ARG
    # past the stream mode's 4096 sequences: taken in groups of 4096; on a host
    # without a device the first group's grid cannot be sized (and nothing runs)
    assert dec(b=5000) in (pa.PA_ERR_HIP, pa.PA_ERR_WORKSPACE)
    assert dec(d=64) == pa.PA_ERR_UNSUPPORTED
    assert dec(qs=4000) == pa.PA_ERR_INVALID_ARG
    assert dec(msl=8193) == pa.PA_ERR_INVALID_ARG


def test_fp8_format_is_checked(L):
    """The _ex forms take the fp8 format: E4M3 (0) and E5M2 (1); anything else
    is refused before any launch."""
    sc = L.pa_reshape_and_cache_fp8_ex
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, 2, 1.0, 1.0, None) == pa.PA_ERR_UNSUPPORTED
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 5, 10, 16, 8, 128, 1, -1, 1.0, 1.0, None) == pa.PA_ERR_UNSUPPORTED
    assert sc(16, 1024, 16, 1024, 16, 16, 16, 0, 10, 16, 8, 128, 1, 1, 1.0, 1.0, None) == pa.PA_OK
    fs = L.pa_slot_mapping_and_cache_fp8_ex
    assert fs(16, 16, 4, 2, 16, 16, 16, 1024, 16, 1024, 16, 16, 3, 10, 16, 8, 128, 1, 7, 0.5, 0.5,
              None) == pa.PA_ERR_UNSUPPORTED
    dc = L.pa_decode_fp8_ex
    args = [16, 16, 4096, 16, 16, 16, 512, 16, 4, 32, 8, 128, 16, 100, 0.088]
    assert dc(*args, 5, 1.0, 1.0, 8192, None, 0, None) == pa.PA_ERR_UNSUPPORTED
    assert dc(*args, 1, -1.0, 1.0, 8192, None, 0, None) == pa.PA_ERR_INVALID_ARG    # scales checked as for E4M3
    with pytest.raises(ValueError):
        pa._fp8_format("e3m4")


def test_copy_blocks_rejects_before_launch(L):
    cb = L.pa_copy_blocks
    assert cb(16, 16, 0, 1, 10, 32768, 16, 0, None) == pa.PA_OK                 # no pairs
    assert cb(16, 16, 0, 0, 10, 32768, 16, 4, None) == pa.PA_OK                 # no layers
    assert cb(16, 16, 0, 1, 10, 32760, 16, 4, None) == pa.PA_ERR_INVALID_ARG    # block not 16-byte sized
    assert cb(16, 24, 0, 1, 10, 32768, 16, 4, None) == pa.PA_ERR_INVALID_ARG    # misaligned cache
    assert cb(16, 16, 1000, 2, 10, 32768, 16, 4, None) == pa.PA_ERR_INVALID_ARG  # layers overlap
    assert cb(16, 16, 0, 1, 10, 32768, None, 4, None) == pa.PA_ERR_INVALID_ARG  # null mapping
    assert cb(16, 16, 0, 1, 10, -1, 16, 4, None) == pa.PA_ERR_INVALID_ARG
