"""ctypes binding of libpa.so (declared in include/pa.h).

Argument marshalling only: shapes are read off the tensors, pointers and the
current HIP stream are passed through, and a nonzero status becomes a
``PaError``.  Every step of the computation runs in the HIP kernels of the
library; there is no fallback.  If libpa.so is missing or cannot be loaded the
functions raise instead of computing anything.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_F32 = 0
PA_F16 = 1
PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_EXHAUSTED = -5

DEFAULT_PARTITION = 0  # 0: as many persistent waves as the GPU holds

_c_int32 = ctypes.c_int32
_c_int64 = ctypes.c_int64
_vp = ctypes.c_void_p

# name -> (restype, argtypes); must match include/pa.h
SIGNATURES = {
    "pa_cache_write": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32,
                                  _c_int64, _c_int32, _vp]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                                    _c_int32]),
    "pa_decode": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _c_int32, _c_int32,
                             _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int64, _c_int32,
                             _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_noalloc": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _c_int32, _c_int32,
                                     _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int64,
                                     _c_int32, _c_int32, _vp]),
    "pa_decode_shared_workspace_bytes": (ctypes.c_size_t, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]),
    "pa_decode_shared": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int32, ctypes.c_float,
                                    _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                    _c_int64, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_shared_partitions": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int32,
                                               ctypes.c_float, _c_int32, _c_int32, _c_int32, _c_int32,
                                               _c_int32, _c_int32, _c_int32, _c_int64, _vp, ctypes.c_size_t,
                                               _vp]),
    "pa_decode_partitions": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _c_int32,
                                        _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                        _c_int64, _c_int32, _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_reduce": (_c_int32, [_vp, _vp, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                    _c_int32, _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_append": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _c_int32,
                                    _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                    _c_int64, _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_append_partitions": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                               _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                               _c_int32, _c_int32, _c_int64, _c_int32, _vp,
                                               ctypes.c_size_t, _vp]),
    "pa_decode_fp8_append": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_float, _c_int32, _c_int32, _c_int32,
                                        _c_int32, _c_int32, _c_int32, _c_int32, _c_int64, _c_int32,
                                        _vp, ctypes.c_size_t, _vp]),
    "pa_decode_fp8_append_partitions": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                   ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                                   _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                                   _c_int32, _c_int32, _c_int64, _c_int32, _vp,
                                                   ctypes.c_size_t, _vp]),
    "pa_cache_write_fp8": (_c_int32, [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float,
                                      _c_int32, _c_int32, _c_int32, _c_int32, _c_int64, _vp]),
    "pa_decode_fp8": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_float, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                 _c_int32, _c_int32, _c_int64, _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_decode_fp8_partitions": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float,
                                            ctypes.c_float, ctypes.c_float, _c_int32, _c_int32,
                                            _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                                            _c_int64, _c_int32, _vp, ctypes.c_size_t, _vp]),
    "pa_prefill": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _c_int32, _c_int32,
                              _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int64,
                              _c_int32, _vp]),
    "pa_copy_blocks": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _c_int32, _c_int64, _c_int64, _c_int64,
                                  _vp]),
    "pa_allocator_create": (_vp, [_c_int32, _c_int32, _vp]),
    "pa_allocator_destroy": (None, [_vp]),
    "pa_allocator_num_free": (_c_int32, [_vp]),
    "pa_allocator_refcount": (_c_int32, [_vp, _c_int32]),
    "pa_allocator_allocate": (_c_int32, [_vp, _vp]),
    "pa_allocator_share": (_c_int32, [_vp, _c_int32]),
    "pa_allocator_release": (_c_int32, [_vp, _c_int32]),
    "pa_allocator_append_slot": (_c_int32, [_vp, _vp, _c_int32, _vp, _c_int32, _vp, _vp, _vp]),
    "pa_allocator_fork": (_c_int32, [_vp, _vp, _c_int32, _vp]),
    "pa_allocator_free_table": (_c_int32, [_vp, _vp, _c_int32]),
    "pa_allocator_move": (_c_int32, [_vp, _vp, _vp, _vp, _c_int32, _c_int32, _vp, _c_int32, _vp]),
    "pa_vkv_create": (_vp, [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int64]),
    "pa_vkv_destroy": (None, [_vp]),
    "pa_vkv_step": (_c_int32, [_vp, _vp, _c_int32, _vp]),
    "pa_vkv_free_seq": (_c_int32, [_vp, _c_int32]),
    "pa_vkv_write": (_c_int32, [_vp, _vp, _vp, _vp, _vp, _c_int32, _vp]),
    "pa_vkv_k": (_vp, [_vp]),
    "pa_vkv_v": (_vp, [_vp]),
    "pa_vkv_seq_bytes": (_c_int64, [_vp]),
    "pa_vkv_page_bytes": (_c_int64, [_vp]),
    "pa_vkv_mapped_bytes": (_c_int64, [_vp]),
    "pa_vkv_capacity": (_c_int32, [_vp, _c_int32]),
    "pa_decode_dense": (_c_int32, [_vp, _vp, _vp, ctypes.c_float, _c_int32, _c_int32, _vp,
                                   ctypes.c_size_t, _vp]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_abi_version": (_c_int32, []),
}

_lib = None


class PaError(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} returned {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libpa.so from the package directory (built by build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_167_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().pa_last_error().decode()


def _check(func: str, code: int) -> None:
    if code != PA_OK:
        raise PaError(func, code, last_error())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.float32:
        return PA_F32
    raise PaError("binding", PA_ERR_UNSUPPORTED, f"dtype {t.dtype} is not float16 or float32")


def _same_dtype(call, *tensors):
    """One element type for all of them: the C ABI takes one dtype code for the call."""
    kinds = {t.dtype for t in tensors}
    if len(kinds) > 1:
        raise PaError(call, PA_ERR_INVALID_ARG, f"mixed element types {sorted(str(k) for k in kinds)}")


def _ptr(t) -> int:
    if not t.is_contiguous():
        raise PaError("binding", PA_ERR_INVALID_ARG, "tensors must be contiguous")
    return t.data_ptr()


def _stream(t, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def pa_cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """k_cache[slot // B, :, slot % B] = k[t] (same for v) for every t with slot >= 0."""
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    _same_dtype("pa_cache_write", k, v, k_cache, v_cache)
    code = lib().pa_cache_write(
        _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), k.shape[0],
        num_kv_heads, head_dim, block_size, num_blocks, _dtype_code(k_cache),
        _stream(k_cache, stream))
    _check("pa_cache_write", code)


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size=DEFAULT_PARTITION) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               max_context_len, partition_size))


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                 num_kv_heads, max_context_len, partition_size, workspace, stream, pools_like_q=True):
    import torch
    _same_dtype("pa_decode", out, q, *((k_cache, v_cache) if pools_like_q else ()))
    num_seqs, num_q_heads, head_dim = q.shape
    num_blocks = k_cache.shape[0]
    max_blocks = block_tables.shape[1]
    if max_context_len is None:  # the table width bounds every context without a device sync
        max_context_len = max_blocks * block_size
    need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), float(scale), int(block_size), int(num_kv_heads), num_seqs,
            num_q_heads, head_dim, max_blocks, int(max_context_len), num_blocks,
            int(partition_size), _dtype_code(q), ws_ptr, ws_bytes, _stream(q, stream)), workspace


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
              num_kv_heads, max_context_len=None, partition_size=DEFAULT_PARTITION,
              workspace=None, stream=None):
    """out[s, h] = softmax(scale * K_s q[s, h]) V_s over the first context_lens[s] positions.

    Returns the workspace tensor used (allocated here if none was given).
    """
    args, workspace = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   block_size, num_kv_heads, max_context_len, partition_size,
                                   workspace, stream)
    _check("pa_decode", lib().pa_decode(*args))
    return workspace


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                      num_kv_heads, max_context_len=None, partition_size=DEFAULT_PARTITION,
                      stream=None) -> None:
    """pa_decode with no workspace: the library's static scratch serves as one, and nothing
    is allocated (neither here nor in the library)."""
    _same_dtype("pa_decode_noalloc", out, q, k_cache, v_cache)
    num_seqs, num_q_heads, head_dim = q.shape
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    code = lib().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), int(block_size), int(num_kv_heads), num_seqs, num_q_heads, head_dim, max_blocks,
        int(max_context_len), k_cache.shape[0], int(partition_size), _dtype_code(q), _stream(q, stream))
    _check("pa_decode_noalloc", code)


def pa_decode_shared_workspace_bytes(num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(lib().pa_decode_shared_workspace_bytes(num_seqs, num_groups, num_q_heads, num_kv_heads,
                                                      head_dim))


def _shared_args(out, q, k_cache, v_cache, block_tables, context_lens, seq_group, group_first,
                 group_size, group_prefix, scale, block_size, num_kv_heads, max_context_len, workspace,
                 stream):
    import torch
    num_seqs, num_q_heads, head_dim = q.shape
    num_groups = group_first.shape[0]
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    need = pa_decode_shared_workspace_bytes(num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
            _ptr(seq_group), _ptr(group_first), _ptr(group_size), _ptr(group_prefix), int(num_groups),
            float(scale), int(block_size), int(num_kv_heads), num_seqs, num_q_heads, head_dim, max_blocks,
            int(max_context_len), k_cache.shape[0], ws_ptr, ws_bytes, _stream(q, stream)), workspace


def pa_decode_shared(out, q, k_cache, v_cache, block_tables, context_lens, seq_group, group_first,
                     group_size, group_prefix, scale, block_size, num_kv_heads, max_context_len=None,
                     workspace=None, stream=None):
    """pa_decode (fp16) with each group's shared prefix read once for all its members.

    seq_group [S] int32 (-1: none); group_first, group_size, group_prefix [NG] int32 on the
    device.  Returns the workspace tensor used (allocated here if none was given).
    """
    args, workspace = _shared_args(out, q, k_cache, v_cache, block_tables, context_lens, seq_group,
                                   group_first, group_size, group_prefix, scale, block_size, num_kv_heads,
                                   max_context_len, workspace, stream)
    _check("pa_decode_shared", lib().pa_decode_shared(*args))
    return workspace


def pa_decode_shared_partitions(out, q, k_cache, v_cache, block_tables, context_lens, seq_group,
                                group_first, group_size, group_prefix, scale, block_size, num_kv_heads,
                                max_context_len=None, workspace=None, stream=None):
    """First launch of pa_decode_shared alone (the stream over the virtual sequences)."""
    args, workspace = _shared_args(out, q, k_cache, v_cache, block_tables, context_lens, seq_group,
                                   group_first, group_size, group_prefix, scale, block_size, num_kv_heads,
                                   max_context_len, workspace, stream)
    _check("pa_decode_shared_partitions", lib().pa_decode_shared_partitions(*args))
    return workspace


def pa_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                         num_kv_heads, max_context_len=None, partition_size=DEFAULT_PARTITION,
                         workspace=None, stream=None):
    """First launch of pa_decode; returns the workspace holding the pieces of split contexts."""
    args, workspace = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   block_size, num_kv_heads, max_context_len, partition_size,
                                   workspace, stream)
    _check("pa_decode_partitions", lib().pa_decode_partitions(*args))
    return workspace


def pa_decode_reduce(out, context_lens, num_kv_heads, max_context_len, partition_size, workspace,
                     stream=None):
    """Second launch of pa_decode: merge the pieces left in the workspace into out."""
    num_seqs, num_q_heads, head_dim = out.shape
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    code = lib().pa_decode_reduce(_ptr(out), _ptr(context_lens), num_seqs, num_q_heads,
                                  int(num_kv_heads), head_dim, int(max_context_len),
                                  int(partition_size), _dtype_code(out), ws_ptr, ws_bytes,
                                  _stream(out, stream))
    _check("pa_decode_reduce", code)


def _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                        block_size, num_kv_heads, max_context_len, partition_size, workspace, stream):
    import torch
    if q.dtype != torch.float16 or k_cache.dtype != torch.float16:
        raise PaError("binding", PA_ERR_UNSUPPORTED, "pa_decode_append takes float16 tensors")
    if k_new.shape != (q.shape[0], k_cache.shape[1], q.shape[2]) or v_new.shape != k_new.shape:
        raise PaError("binding", PA_ERR_INVALID_ARG, "k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    args, workspace = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   block_size, num_kv_heads, max_context_len, partition_size,
                                   workspace, stream)
    # (out, q, k_new, v_new, kc, vc, bt, ctx, scale, block_size, ...) without the dtype
    return args[:2] + (_ptr(k_new), _ptr(v_new)) + args[2:16] + args[17:], workspace


def pa_decode_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                     block_size, num_kv_heads, max_context_len=None,
                     partition_size=DEFAULT_PARTITION, workspace=None, stream=None):
    """One decode step: store k_new[s], v_new[s] at position context_lens[s] - 1 of each
    sequence (the slot its table gives) and attend over the whole context (fp16)."""
    args, workspace = _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                          context_lens, scale, block_size, num_kv_heads,
                                          max_context_len, partition_size, workspace, stream)
    _check("pa_decode_append", lib().pa_decode_append(*args))
    return workspace


def pa_decode_append_partitions(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                scale, block_size, num_kv_heads, max_context_len=None,
                                partition_size=DEFAULT_PARTITION, workspace=None, stream=None):
    """First launch of pa_decode_append alone (stores nothing); pa_decode_reduce merges."""
    args, workspace = _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                          context_lens, scale, block_size, num_kv_heads,
                                          max_context_len, partition_size, workspace, stream)
    _check("pa_decode_append_partitions", lib().pa_decode_append_partitions(*args))
    return workspace


def _require_codes(t, name):
    import torch
    if t.dtype != torch.uint8:
        raise PaError("binding", PA_ERR_UNSUPPORTED, f"{name} must hold E4M3 codes as uint8")


def pa_cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream=None) -> None:
    """E4M3 pools (uint8): k_cache[slot // B, :, slot % B] = code(k[t] / k_scale), same for v."""
    import torch
    _require_codes(k_cache, "k_cache")
    _require_codes(v_cache, "v_cache")
    if k.dtype != torch.float16 or v.dtype != torch.float16:
        raise PaError("binding", PA_ERR_UNSUPPORTED, "k and v must be float16")
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    code = lib().pa_cache_write_fp8(
        _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), float(k_scale),
        float(v_scale), k.shape[0], num_kv_heads, head_dim, block_size, num_blocks,
        _stream(k_cache, stream))
    _check("pa_cache_write_fp8", code)


def _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                     block_size, num_kv_heads, max_context_len, partition_size, workspace, stream):
    _require_codes(k_cache, "k_cache")
    _require_codes(v_cache, "v_cache")
    args, workspace = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   block_size, num_kv_heads, max_context_len, partition_size,
                                   workspace, stream, pools_like_q=False)
    if args[16] != PA_F16:
        raise PaError("binding", PA_ERR_UNSUPPORTED, "q and out must be float16 with E4M3 pools")
    # (out, q, kc, vc, bt, ctx, scale, k_scale, v_scale, block_size, ...) without the dtype
    return args[:7] + (float(k_scale), float(v_scale)) + args[7:16] + args[17:], workspace


def pa_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                  block_size, num_kv_heads, max_context_len=None, partition_size=DEFAULT_PARTITION,
                  workspace=None, stream=None):
    """pa_decode over E4M3 pools: attention over the codes times k_scale / v_scale."""
    args, workspace = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                       k_scale, v_scale, block_size, num_kv_heads, max_context_len,
                                       partition_size, workspace, stream)
    _check("pa_decode_fp8", lib().pa_decode_fp8(*args))
    return workspace


def pa_decode_fp8_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                             v_scale, block_size, num_kv_heads, max_context_len=None,
                             partition_size=DEFAULT_PARTITION, workspace=None, stream=None):
    """First launch of pa_decode_fp8; pa_decode_reduce (dtype float16) is the second."""
    args, workspace = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                       k_scale, v_scale, block_size, num_kv_heads, max_context_len,
                                       partition_size, workspace, stream)
    _check("pa_decode_fp8_partitions", lib().pa_decode_fp8_partitions(*args))
    return workspace


def _decode_fp8_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                            k_scale, v_scale, block_size, num_kv_heads, max_context_len,
                            partition_size, workspace, stream):
    import torch
    if k_new.dtype != torch.float16 or v_new.dtype != torch.float16:
        raise PaError("binding", PA_ERR_UNSUPPORTED, "k_new and v_new must be float16")
    if k_new.shape != (q.shape[0], k_cache.shape[1], q.shape[2]) or v_new.shape != k_new.shape:
        raise PaError("binding", PA_ERR_INVALID_ARG, "k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    args, workspace = _decode_fp8_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                       k_scale, v_scale, block_size, num_kv_heads, max_context_len,
                                       partition_size, workspace, stream)
    return args[:2] + (_ptr(k_new), _ptr(v_new)) + args[2:], workspace


def pa_decode_fp8_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                         k_scale, v_scale, block_size, num_kv_heads, max_context_len=None,
                         partition_size=DEFAULT_PARTITION, workspace=None, stream=None):
    """pa_decode_append over E4M3 pools: store the new tokens' codes, attend over the codes
    times k_scale / v_scale."""
    args, workspace = _decode_fp8_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                              context_lens, scale, k_scale, v_scale, block_size,
                                              num_kv_heads, max_context_len, partition_size, workspace,
                                              stream)
    _check("pa_decode_fp8_append", lib().pa_decode_fp8_append(*args))
    return workspace


def pa_decode_fp8_append_partitions(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                    scale, k_scale, v_scale, block_size, num_kv_heads,
                                    max_context_len=None, partition_size=DEFAULT_PARTITION,
                                    workspace=None, stream=None):
    """First launch of pa_decode_fp8_append alone (stores nothing)."""
    args, workspace = _decode_fp8_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                              context_lens, scale, k_scale, v_scale, block_size,
                                              num_kv_heads, max_context_len, partition_size, workspace,
                                              stream)
    _check("pa_decode_fp8_append_partitions", lib().pa_decode_fp8_append_partitions(*args))
    return workspace


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               block_size, num_kv_heads, max_query_len, max_context_len=None, stream=None):
    """Causal attention of each sequence's chunk of query tokens (rows query_start[s] ..
    query_start[s+1]-1, the last positions of its context) over the paged cache."""
    total_q, num_q_heads, head_dim = q.shape
    num_seqs = context_lens.shape[0]
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * block_size
    code = lib().pa_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), float(scale), int(block_size), int(num_kv_heads), num_seqs, num_q_heads,
        head_dim, max_blocks, int(max_query_len), int(max_context_len), k_cache.shape[0],
        _dtype_code(q), _stream(q, stream))
    _check("pa_prefill", code)


def pa_copy_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None) -> None:
    """dst[pairs[i, 1]] = src[pairs[i, 0]] for K and V, whole blocks; pools on the device or in
    pinned host memory; pairs an int32 [n, 2] tensor (device or pinned host)."""
    import torch
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise PaError("binding", PA_ERR_INVALID_ARG, "pairs must be an int32 [n, 2] tensor")
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise PaError("binding", PA_ERR_INVALID_ARG, "source and destination blocks differ in shape")
    block_bytes = src_k[0].numel() * src_k.element_size() if src_k.shape[0] else 0
    dev = dst_k if dst_k.is_cuda else (src_k if src_k.is_cuda else None)
    st = _stream(dev, stream) if dev is not None else (0 if stream is None else _stream(None, stream))
    code = lib().pa_copy_blocks(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(pairs),
                                pairs.shape[0], src_k.shape[0], dst_k.shape[0], block_bytes, st)
    _check("pa_copy_blocks", code)


class BlockAllocator:
    """The library's reference-counted block allocator (host side; see pa.h)."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.block_size = int(block_size)
        self._order = None
        if order is not None:
            self._order = (ctypes.c_int32 * num_blocks)(*[int(b) for b in order])
        h = lib().pa_allocator_create(int(num_blocks), self.block_size, self._order)
        if not h:
            raise PaError("pa_allocator_create", PA_ERR_INVALID_ARG, last_error())
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_allocator_destroy(h)
            self._h = None

    @property
    def num_free(self) -> int:
        return int(lib().pa_allocator_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib().pa_allocator_refcount(self._h, int(block)))

    def allocate(self) -> int:
        b = ctypes.c_int32()
        _check("pa_allocator_allocate", lib().pa_allocator_allocate(self._h, ctypes.byref(b)))
        return b.value

    def share(self, block: int) -> None:
        _check("pa_allocator_share", lib().pa_allocator_share(self._h, int(block)))

    def release(self, block: int) -> None:
        _check("pa_allocator_release", lib().pa_allocator_release(self._h, int(block)))

    def append_slot(self, table: list, ctx: int, capacity: int = 1 << 16):
        """Slot of position ctx of the sequence whose table (a list, updated in place) is given,
        and the (source, destination) copy to make first, or None."""
        buf = (ctypes.c_int32 * max(capacity, len(table) + 1))(*table)
        n = ctypes.c_int32(len(table))
        slot, cs, cd = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_allocator_append_slot", lib().pa_allocator_append_slot(
            self._h, buf, len(buf), ctypes.byref(n), int(ctx), ctypes.byref(slot), ctypes.byref(cs),
            ctypes.byref(cd)))
        table[:] = list(buf[:n.value])
        return slot.value, (None if cs.value < 0 else (cs.value, cd.value))

    def fork(self, table: list) -> list:
        src = (ctypes.c_int32 * max(len(table), 1))(*table)
        child = (ctypes.c_int32 * max(len(table), 1))()
        _check("pa_allocator_fork", lib().pa_allocator_fork(self._h, src, len(table), child))
        return list(child[:len(table)])

    def free_table(self, table: list) -> None:
        buf = (ctypes.c_int32 * max(len(table), 1))(*table)
        _check("pa_allocator_free_table", lib().pa_allocator_free_table(self._h, buf, len(table)))
        table.clear()

    def move(self, tables: list, dst: "BlockAllocator") -> list:
        """Rewrite the tables (lists, updated in place) onto dst's pool; returns the copies."""
        stride = max([len(t) for t in tables] + [1])
        flat = (ctypes.c_int32 * (stride * max(len(tables), 1)))()
        for i, t in enumerate(tables):
            for j, b in enumerate(t):
                flat[i * stride + j] = b
        lens = (ctypes.c_int32 * max(len(tables), 1))(*[len(t) for t in tables])
        cap = sum(len(t) for t in tables)
        pairs = (ctypes.c_int32 * max(2 * cap, 2))()
        n = ctypes.c_int32()
        _check("pa_allocator_move", lib().pa_allocator_move(
            self._h, dst._h, flat, lens, len(tables), stride, pairs, cap, ctypes.byref(n)))
        for i, t in enumerate(tables):
            t[:] = list(flat[i * stride:i * stride + len(t)])
        return [(pairs[2 * i], pairs[2 * i + 1]) for i in range(n.value)]


class DenseKV:
    """The library's virtually contiguous K/V cache (HIP virtual memory, no block tables)."""

    def __init__(self, max_seqs, max_context_len, num_kv_heads, head_dim, page_bytes=0):
        h = lib().pa_vkv_create(int(max_seqs), int(max_context_len), int(num_kv_heads),
                                int(head_dim), PA_F16, int(page_bytes))
        if not h:
            raise PaError("pa_vkv_create", PA_ERR_INVALID_ARG, last_error())
        self._h = h
        self.max_seqs, self.max_context_len = int(max_seqs), int(max_context_len)
        self.num_kv_heads, self.head_dim = int(num_kv_heads), int(head_dim)
        self.num_seqs = 0

    def close(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_vkv_destroy(h)
        self._h = None

    def __del__(self):
        self.close()

    @property
    def page_bytes(self) -> int:
        return int(lib().pa_vkv_page_bytes(self._h))

    @property
    def seq_bytes(self) -> int:
        return int(lib().pa_vkv_seq_bytes(self._h))

    @property
    def mapped_bytes(self) -> int:
        return int(lib().pa_vkv_mapped_bytes(self._h))

    def capacity(self, seq: int) -> int:
        return int(lib().pa_vkv_capacity(self._h, int(seq)))

    def step(self, context_lens, stream=None) -> None:
        """Back tokens [0, context_lens[s]) of every sequence; record the lengths for decode."""
        n = len(context_lens)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(c) for c in context_lens])
        st = 0 if stream is None else (int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))
        _check("pa_vkv_step", lib().pa_vkv_step(self._h, arr, n, st))
        self.num_seqs = n

    def free_seq(self, seq: int) -> None:
        _check("pa_vkv_free_seq", lib().pa_vkv_free_seq(self._h, int(seq)))

    def write(self, k, v, seq_ids, positions, stream=None) -> None:
        import torch
        if k.dtype != torch.float16 or v.dtype != torch.float16:
            raise PaError("binding", PA_ERR_UNSUPPORTED, "k and v must be float16")
        if seq_ids.dtype != torch.int32 or positions.dtype != torch.int32:
            raise PaError("binding", PA_ERR_INVALID_ARG, "seq_ids and positions must be int32")
        _check("pa_vkv_write", lib().pa_vkv_write(self._h, _ptr(k), _ptr(v), _ptr(seq_ids), _ptr(positions),
                                                  k.shape[0], _stream(k, stream)))

    def decode(self, out, q, scale, partition_size=DEFAULT_PARTITION, workspace=None, stream=None):
        """pa_decode over this cache for the sequences and lengths of the last step."""
        import torch
        num_seqs, num_q_heads, head_dim = q.shape
        if num_seqs != self.num_seqs:
            raise PaError("binding", PA_ERR_INVALID_ARG, f"q has {num_seqs} sequences, the last step {self.num_seqs}")
        need = pa_decode_workspace_bytes(num_seqs, num_q_heads, self.num_kv_heads, head_dim,
                                         self.max_context_len, partition_size)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() if workspace is not None else 0
        _check("pa_decode_dense", lib().pa_decode_dense(
            _ptr(out), _ptr(q), self._h, float(scale), num_q_heads, int(partition_size), ws_ptr,
            ws_bytes, _stream(q, stream)))
        return workspace
