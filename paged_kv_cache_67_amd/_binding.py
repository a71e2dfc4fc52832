"""ctypes binding of libpa (include/pa.h).  Argument marshalling only.

Each function has the name of the C entry point it calls.  Tensors must be
device tensors (torch is used for device memory and streams, nothing else);
sizes are read from tensor shapes and a non-zero pa_status raises PAError.
There is no fallback: if libpa.so is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

PA_F32, PA_BF16, PA_F16 = 0, 1, 2
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
          4: "PA_ERR_ALIGN", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_CAPACITY",
          8: "PA_ERR_CONTRACT"}

_i32, _i64, _f32, _vp, _sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
_u64, _pi32 = C.c_uint64, C.POINTER(C.c_int32)

PA_COPY_MANY_MAX = 8


class CopyDesc(C.Structure):
    """pa_copy_desc: {src (NULL = zero fill), dst, bytes}."""
    _fields_ = [("src", _vp), ("dst", _vp), ("bytes", _i64)]


# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_version": (C.c_int, []),
    "pa_status_string": (C.c_char_p, [C.c_int]),
    "pa_last_error": (C.c_char_p, []),
    "pa_slot_mapping": (C.c_int, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_store_kv": (C.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                              C.c_int, _vp]),
    "pa_store_kv_paged": (C.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                    _i32, _i32, _i32, _i32, _i32, _i32, C.c_int, _vp, _vp]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                            _i32, _f32, C.c_int, _i32, _vp, _sz, _vp]),
    "pa_decode_partitions": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _f32, C.c_int, _i32, _vp, _sz, _vp]),
    "pa_decode_append": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _i32,
                                   _i32, _i32, _i32, _i32, _i32, _i32, _f32, C.c_int, _i32, _vp,
                                   _sz, _vp]),
    "pa_decode_append_partitions": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32,
                                              _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                              C.c_int, _i32, _vp, _sz, _vp]),
    "pa_decode_merge": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, C.c_int, _vp]),
    "pa_decode_noalloc": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _f32, C.c_int, _i32, _vp]),
    "pa_prefill_paged": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                   _i32, _i32, _i32, _i32, _i32, _f32, _i32, C.c_int, _vp]),
    "pa_mixed_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_attention_mixed": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _f32, C.c_int, _vp, _sz,
                                     _vp]),
    "pa_copy_blocks": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, C.c_int, _vp]),
    "pa_copy_many": (C.c_int, [C.POINTER(CopyDesc), _i32, _vp]),
    "pa_read_ceiling": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, C.c_int, _i32,
                                  _vp, _vp]),
    "pa_set_debug_checks": (C.c_int, [C.c_int]),
    "pa_check_store_inputs": (C.c_int, [_vp, _i32, _i32, _i32, _vp]),
    "pa_check_store_paged_inputs": (C.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_check_decode_inputs": (C.c_int, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_check_prefill_inputs": (C.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _vp]),
    "pa_chain_hash": (_u64, [_pi32, _i32, _i32, _u64]),
    "pa_bm_create": (_vp, [_i32, _i32]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_allocate": (_i64, [_vp, _pi32, _i32]),
    "pa_bm_append": (C.c_int, [_vp, _i64, _i32, _pi32, _pi32]),
    "pa_bm_fork": (_i64, [_vp, _i64]),
    "pa_bm_free": (C.c_int, [_vp, _i64]),
    "pa_bm_block_table": (_i32, [_vp, _i64, _pi32, _i32]),
    "pa_bm_seq_len": (_i32, [_vp, _i64]),
    "pa_bm_num_cached_tokens": (_i32, [_vp, _i64]),
    "pa_bm_ref_count": (_i32, [_vp, _i32]),
    "pa_bm_num_free_blocks": (_i32, [_vp]),
}


class PAError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libpa (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m paged_kv_cache_67_amd.build`")
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise PAError(fn, status, lib().pa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpa takes device tensors only")
    return t.data_ptr()


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.float16:
        return PA_F16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _i32_vec(t, n, name):
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] < n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 vector of at least {n} entries")


def pa_version() -> int:
    return lib().pa_version()


def pa_status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def pa_last_error() -> str:
    return lib().pa_last_error().decode()


def pa_slot_mapping(slot_mapping, block_table, cu_seqlens_q, seq_lens_k, block_size, num_blocks,
                    stream=None):
    B, maxb = block_table.shape
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(seq_lens_k, B, "seq_lens_k")
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _check("pa_slot_mapping", lib().pa_slot_mapping(
        _ptr(slot_mapping), _ptr(block_table), maxb, _ptr(cu_seqlens_q), _ptr(seq_lens_k), B,
        slot_mapping.shape[0], block_size, num_blocks, _stream(stream)))


def pa_store_kv(key, value, k_cache, v_cache, slot_mapping, stream=None):
    NB, BS, HKV, D = k_cache.shape
    assert v_cache.shape == k_cache.shape and k_cache.is_contiguous() and v_cache.is_contiguous()
    for t in (key, value):
        assert t.dim() == 3 and t.shape[1:] == (HKV, D) and t.stride(2) == 1 and t.stride(1) == D
        assert t.dtype == k_cache.dtype
    N = key.shape[0]
    _i32_vec(slot_mapping, N, "slot_mapping")
    _check("pa_store_kv", lib().pa_store_kv(
        _ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), N, NB, BS, HKV, D, _dtype(k_cache), _stream(stream)))


def pa_store_kv_paged(key, value, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens_k,
                      max_seqlen_q, slot_mapping=None, stream=None):
    """pa_slot_mapping followed by pa_store_kv in one launch; slot_mapping, if given,
    receives the slots."""
    NB, BS, HKV, D = k_cache.shape
    assert v_cache.shape == k_cache.shape and k_cache.is_contiguous() and v_cache.is_contiguous()
    for t in (key, value):
        assert t.dim() == 3 and t.shape[1:] == (HKV, D) and t.stride(2) == 1 and t.stride(1) == D
        assert t.dtype == k_cache.dtype
    assert value.shape[0] == key.shape[0]
    B, maxb = block_table.shape
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(seq_lens_k, B, "seq_lens_k")
    N = key.shape[0]
    if slot_mapping is not None:
        _i32_vec(slot_mapping, N, "slot_mapping")
    _check("pa_store_kv_paged", lib().pa_store_kv_paged(
        _ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), maxb, _ptr(cu_seqlens_q), _ptr(seq_lens_k), B, N, int(max_seqlen_q),
        NB, BS, HKV, D, _dtype(k_cache), _ptr(slot_mapping), _stream(stream)))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                             partition_size=0) -> int:
    return lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, partition_size)


def pa_decode(out, q, k_cache, v_cache, block_table, context_lens, scale, max_context_len=0,
              partition_size=0, workspace=None, stream=None):
    B, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    assert out.shape == q.shape and Dk == D and v_cache.shape == k_cache.shape
    assert q.is_contiguous() and out.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert out.dtype == q.dtype == k_cache.dtype == v_cache.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    _i32_vec(context_lens, B, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", lib().pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), B, int(max_context_len), NB, BS, HQ, HKV, D, float(scale),
        _dtype(q), int(partition_size), _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_noalloc(out, q, k_cache, v_cache, block_table, context_lens, scale, max_context_len=0,
                      partition_size=0, stream=None):
    B, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    assert out.shape == q.shape and Dk == D and v_cache.shape == k_cache.shape
    assert q.is_contiguous() and out.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert out.dtype == q.dtype == k_cache.dtype == v_cache.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    _i32_vec(context_lens, B, "context_lens")
    _check("pa_decode_noalloc", lib().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), B, int(max_context_len), NB, BS, HQ, HKV, D, float(scale), _dtype(q),
        int(partition_size), _stream(stream)))


def pa_decode_partitions(out, q, k_cache, v_cache, block_table, context_lens, scale, max_context_len,
                         partition_size, workspace, stream=None):
    B, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape and q.dtype == k_cache.dtype
    assert q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    if out is not None:
        assert out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
    _i32_vec(context_lens, B, "context_lens")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_partitions", lib().pa_decode_partitions(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), B, int(max_context_len), NB, BS, HQ, HKV, D, float(scale), _dtype(q),
        int(partition_size), _ptr(workspace), ws_bytes, _stream(stream)))


def _decode_append(name, out, q, key, value, k_cache, v_cache, block_table, context_lens, scale,
                   max_context_len, partition_size, workspace, stream):
    B, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    assert Dk == D and v_cache.shape == k_cache.shape and q.dtype == k_cache.dtype == v_cache.dtype
    assert q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    for t in (key, value):
        assert t.dim() == 3 and t.shape == (B, HKV, D) and t.stride(2) == 1 and t.stride(1) == D
        assert t.dtype == k_cache.dtype
    if out is not None:
        assert out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
    assert block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.shape[0] == B
    _i32_vec(context_lens, B, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(context_lens), B,
        int(max_context_len), NB, BS, HQ, HKV, D, float(scale), _dtype(q), int(partition_size),
        _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_append(out, q, key, value, k_cache, v_cache, block_table, context_lens, scale,
                     max_context_len=0, partition_size=0, workspace=None, stream=None):
    """The step's new rows key / value [B, HKV, D] (row b: key context_lens[b] - 1 of sequence
    b) stored to the cache, then pa_decode over every key; one first pass with the balanced
    split."""
    _decode_append("pa_decode_append", out, q, key, value, k_cache, v_cache, block_table,
                   context_lens, scale, max_context_len, partition_size, workspace, stream)


def pa_decode_append_partitions(out, q, key, value, k_cache, v_cache, block_table, context_lens,
                                scale, max_context_len, partition_size, workspace, stream=None):
    _decode_append("pa_decode_append_partitions", out, q, key, value, k_cache, v_cache,
                   block_table, context_lens, scale, max_context_len, partition_size, workspace,
                   stream)


def pa_decode_merge(out, workspace, context_lens, num_kv_heads, max_context_len, partition_size,
                    stream=None):
    B, HQ, D = out.shape
    _i32_vec(context_lens, B, "context_lens")
    _check("pa_decode_merge", lib().pa_decode_merge(
        _ptr(out), _ptr(workspace), _ptr(context_lens), B, HQ, int(num_kv_heads), D,
        int(max_context_len), int(partition_size), _dtype(out), _stream(stream)))


def pa_prefill_paged(out, q, k_cache, v_cache, block_table, cu_seqlens_q, cu_seqlens_k,
                     max_seqlen_q, max_seqlen_k, scale, causal=True, stream=None):
    T, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    B = block_table.shape[0]
    assert out.shape == q.shape and Dk == D and v_cache.shape == k_cache.shape
    assert q.is_contiguous() and out.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert out.dtype == q.dtype == k_cache.dtype == v_cache.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(cu_seqlens_k, B + 1, "cu_seqlens_k")
    _check("pa_prefill_paged", lib().pa_prefill_paged(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, T, int(max_seqlen_q), int(max_seqlen_k), NB, BS,
        HQ, HKV, D, float(scale), 1 if causal else 0, _dtype(q), _stream(stream)))


def pa_mixed_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seqlen_k) -> int:
    return lib().pa_mixed_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seqlen_k)


def pa_attention_mixed(out, q, k_cache, v_cache, block_table, cu_seqlens_q, cu_seqlens_k,
                       max_seqlen_q, max_seqlen_k, scale, workspace, stream=None):
    T, HQ, D = q.shape
    NB, BS, HKV, Dk = k_cache.shape
    B = block_table.shape[0]
    assert out.shape == q.shape and Dk == D and v_cache.shape == k_cache.shape
    assert q.is_contiguous() and out.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert out.dtype == q.dtype == k_cache.dtype == v_cache.dtype
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(cu_seqlens_k, B + 1, "cu_seqlens_k")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_attention_mixed", lib().pa_attention_mixed(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1],
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, T, int(max_seqlen_q), int(max_seqlen_k), NB, BS,
        HQ, HKV, D, float(scale), _dtype(q), _ptr(workspace), ws_bytes, _stream(stream)))


def pa_set_debug_checks(on: bool) -> bool:
    """Switch the debug checks of every launching entry point on or off for the process
    (each call then synchronises to check its metadata); returns the previous setting."""
    return bool(lib().pa_set_debug_checks(1 if on else 0))


def pa_check_store_inputs(slot_mapping, num_blocks, block_size, stream=None):
    """Debug check of a store's slots (synchronises): raises PAError naming the first
    slot outside {-1} and [0, num_blocks * block_size) or the first repeated slot."""
    _i32_vec(slot_mapping, slot_mapping.shape[0], "slot_mapping")
    _check("pa_check_store_inputs", lib().pa_check_store_inputs(
        _ptr(slot_mapping), slot_mapping.shape[0], num_blocks, block_size, _stream(stream)))


def pa_check_store_paged_inputs(block_table, cu_seqlens_q, seq_lens_k, num_tokens, num_blocks,
                                block_size, stream=None):
    """Debug check of a fused store's offsets and the slots it computes (synchronises):
    raises PAError naming the first decreasing offset or the first slot two tokens map to."""
    B = block_table.shape[0]
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(seq_lens_k, B, "seq_lens_k")
    _check("pa_check_store_paged_inputs", lib().pa_check_store_paged_inputs(
        _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_q), _ptr(seq_lens_k), B,
        int(num_tokens), num_blocks, block_size, _stream(stream)))


def pa_check_decode_inputs(block_table, context_lens, num_blocks, block_size, max_context_len=0,
                           stream=None):
    """Debug check of a decode batch's lengths and block ids (synchronises)."""
    B = block_table.shape[0]
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(context_lens, B, "context_lens")
    _check("pa_check_decode_inputs", lib().pa_check_decode_inputs(
        _ptr(block_table), block_table.shape[1], _ptr(context_lens), B, int(max_context_len),
        num_blocks, block_size, _stream(stream)))


def pa_check_prefill_inputs(block_table, cu_seqlens_q, cu_seqlens_k, total_q, max_seqlen_q,
                            max_seqlen_k, num_blocks, block_size, stream=None):
    """Debug check of a varlen batch's offsets, lengths and block ids (synchronises)."""
    B = block_table.shape[0]
    assert block_table.dtype == torch.int32 and block_table.is_contiguous()
    _i32_vec(cu_seqlens_q, B + 1, "cu_seqlens_q")
    _i32_vec(cu_seqlens_k, B + 1, "cu_seqlens_k")
    _check("pa_check_prefill_inputs", lib().pa_check_prefill_inputs(
        _ptr(block_table), block_table.shape[1], _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
        int(total_q), int(max_seqlen_q), int(max_seqlen_k), num_blocks, block_size,
        _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy blocks block_pairs[p, 0] -> block_pairs[p, 1] of both pools (device int32 [P, 2])."""
    NB, BS, HKV, D = k_cache.shape
    assert v_cache.shape == k_cache.shape and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert v_cache.dtype == k_cache.dtype
    assert block_pairs.dtype == torch.int32 and block_pairs.is_contiguous()
    assert block_pairs.dim() == 2 and block_pairs.shape[1] == 2
    _check("pa_copy_blocks", lib().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), block_pairs.shape[0], NB, BS, HKV, D,
        _dtype(k_cache), _stream(stream)))


def copy_descs(n=PA_COPY_MANY_MAX):
    """A reusable host array of n pa_copy_desc."""
    return (CopyDesc * n)()


def pa_copy_many(pairs, stream=None, descs=None):
    """Copies src -> dst for each (src, dst) in pairs (src None: zero dst) in one launch.
    Tensors are contiguous device tensors; src and dst of a pair have the same byte size.
    descs: an optional array from copy_descs() to fill instead of a new one."""
    if len(pairs) > PA_COPY_MANY_MAX:
        raise ValueError(f"at most {PA_COPY_MANY_MAX} copies per call")
    if descs is None:
        descs = copy_descs(len(pairs))
    for k, (src, dst) in enumerate(pairs):
        assert dst.is_contiguous() and dst.is_cuda
        nbytes = dst.numel() * dst.element_size()
        if src is not None:
            assert src.is_contiguous() and src.is_cuda
            assert src.numel() * src.element_size() == nbytes, "src and dst sizes differ"
        d = descs[k]
        d.src = src.data_ptr() if src is not None else None
        d.dst = dst.data_ptr()
        d.bytes = nbytes
    _check("pa_copy_many", lib().pa_copy_many(descs, len(pairs), _stream(stream)))


def pa_read_ceiling(k_cache, v_cache, block_ids, num_workgroups, sink, stream=None):
    """Read every K/V byte of the listed pool blocks once (the decode's loads, no arithmetic);
    sink: device uint32 [num_workgroups * 8] receives the XOR of what each wave read."""
    NB, BS, HKV, D = k_cache.shape
    assert v_cache.shape == k_cache.shape and k_cache.is_contiguous() and v_cache.is_contiguous()
    assert v_cache.dtype == k_cache.dtype
    assert block_ids.dtype == torch.int32 and block_ids.is_contiguous() and block_ids.dim() == 1
    assert sink.dtype in (torch.int32, torch.uint32) and sink.numel() >= 8 * num_workgroups
    _check("pa_read_ceiling", lib().pa_read_ceiling(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_ids), block_ids.numel(), NB, BS, HKV, D,
        _dtype(k_cache), int(num_workgroups), _ptr(sink), _stream(stream)))


def _host_i32(values):
    arr = (C.c_int32 * max(1, len(values)))(*values)
    return arr


def pa_chain_hash(token_ids, prefix=None) -> int:
    """Fingerprint of one block of token ids, chained on the previous block's (None: first)."""
    arr = _host_i32(list(token_ids))
    return lib().pa_chain_hash(arr, len(token_ids), 0 if prefix is None else 1,
                               0 if prefix is None else int(prefix))


class BlockManager:
    """Handle on the library's host-side block manager (pa_bm_*); marshalling only."""

    def __init__(self, num_blocks, block_size):
        self._h = lib().pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PAError("pa_bm_create", 2, pa_last_error())
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _seq(self, fn, r):
        if r < 0:
            raise PAError(fn, -r, pa_last_error())
        return r

    def allocate(self, token_ids) -> int:
        arr = _host_i32(list(token_ids))
        return self._seq("pa_bm_allocate", lib().pa_bm_allocate(self._h, arr, len(token_ids)))

    def append(self, seq, token_id):
        """Returns the (src, dst) copy-on-write pair, or None."""
        src, dst = C.c_int32(-1), C.c_int32(-1)
        _check("pa_bm_append", lib().pa_bm_append(self._h, seq, int(token_id), C.byref(src),
                                                  C.byref(dst)))
        return None if src.value < 0 else (src.value, dst.value)

    def fork(self, seq) -> int:
        return self._seq("pa_bm_fork", lib().pa_bm_fork(self._h, seq))

    def free(self, seq):
        _check("pa_bm_free", lib().pa_bm_free(self._h, seq))

    def block_table(self, seq):
        n = self._seq("pa_bm_block_table", lib().pa_bm_block_table(self._h, seq, None, 0))
        out = (C.c_int32 * max(1, n))()
        lib().pa_bm_block_table(self._h, seq, out, n)
        return list(out[:n])

    def seq_len(self, seq) -> int:
        return self._seq("pa_bm_seq_len", lib().pa_bm_seq_len(self._h, seq))

    def num_cached_tokens(self, seq) -> int:
        return self._seq("pa_bm_num_cached_tokens", lib().pa_bm_num_cached_tokens(self._h, seq))

    def ref_count(self, block_id) -> int:
        return self._seq("pa_bm_ref_count", lib().pa_bm_ref_count(self._h, int(block_id)))

    def num_free_blocks(self) -> int:
        return lib().pa_bm_num_free_blocks(self._h)
