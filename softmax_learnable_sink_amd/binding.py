"""Thin ctypes binding of libattn_sink.so (C ABI in include/attn_sink.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
outputs and workspaces are allocated with torch when the caller passes none,
and the pointers plus the current HIP stream go to the C entry points.  Every
step of the computation runs in the library's HIP kernels.  The functions
carry the C names.  A missing library raises; there is no fallback.
"""

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_sink.so")
# the same library with device-side precondition checks (a debug build)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_sink_debug.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, F32 = 0, 1

_lib = None
_debug_lib = None
_vp = ctypes.c_void_p
_pu = ctypes.POINTER(ctypes.c_uint)
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "attn_sink_abi_version": ([], _i),
    "attn_sink_last_error": ([], ctypes.c_char_p),
    "attn_sink_fwd_prefill": ([_vp, _vp, _vp, _vp, _vp, _vp] + [_i] * 6 + [_f, _i, _i, _i, _i, _vp], _i),
    "attn_sink_fwd_decode_paged": ([_vp] * 8 + [_i] * 7 + [_f, _i, _i, _i, _vp, _sz, _i, _vp], _i),
    "attn_sink_fwd_decode_paged_noalloc": ([_vp] * 8 + [_i] * 7 + [_f, _i, _i, _i, _i, _vp], _i),
    "attn_sink_fwd_extend_paged": ([_vp] * 9 + [_i] * 9 + [_f, _i, _i, _i, _vp], _i),
    "attn_sink_fwd_varlen": ([_vp] * 8 + [_i] * 7 + [_f, _i, _i, _i, _i, _vp], _i),
    "attn_sink_fwd_index_paged": ([_vp] * 11 + [_i] * 11 + [_f, _i, _vp], _i),
    "attn_sink_fwd_index_rows_paged": ([_vp] * 10 + [_i] * 9 + [_f, _vp, _sz, _i, _vp], _i),
    "attn_sink_index_rows_workspace_bytes": ([_i] * 5, _sz),
    "attn_sink_decode_workspace_bytes": ([_i] * 9, _sz),
    "attn_sink_bwd": ([_vp] * 11 + [_i] * 6 + [_f, _i, _i, _i, _vp, _sz, _i, _vp], _i),
    "attn_sink_bwd_workspace_bytes": ([_i] * 6, _sz),
    "attn_sink_bwd_varlen": ([_vp] * 13 + [_i] * 8 + [_f, _i, _i, _i, _vp, _sz, _i, _vp], _i),
    "attn_sink_bwd_varlen_workspace_bytes": ([_i] * 4, _sz),
    "attn_sink_decode_select_slots": ([_vp, _vp] + [_i] * 5 + [_vp, _vp, _i, _vp], _i),
    "attn_sink_gather_kv": ([_vp] * 4 + [_i] * 7 + [_vp, _vp, _i, _i, _vp], _i),
    "attn_sink_device_check_flags": ([_pu, _i, _vp], _i),
    "attn_sink_check_paged_inputs": ([_vp] * 3 + [_i] * 9 + [_pu], _i),
}

CHECK_SEQLEN, CHECK_PAGE, CHECK_CU_SEQLENS = 1, 2, 4


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m softmax_learnable_sink_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.argtypes = args
        fn.restype = res
    return handle


def lib():
    """Load libattn_sink.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib():
    """Load libattn_sink_debug.so (device-side precondition checks) once."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def attn_sink_device_check_flags(clear=True, handle=None, stream=None):
    """ATTN_SINK_CHECK_* bits recorded by a debug library's device checks (waits for
    the stream).  Raises AttnSinkError with the release library."""
    h = handle if handle is not None else lib()
    flags = ctypes.c_uint(0)
    st = stream if stream is not None else _stream(torch.cuda.current_device())
    status = h.attn_sink_device_check_flags(ctypes.byref(flags), int(bool(clear)), st)
    if status != OK:
        raise AttnSinkError(status, h.attn_sink_last_error().decode())
    return flags.value


def attn_sink_check_paged_inputs(block_table, seqlens_k, page_size, num_pages, cu_seqlens_q=None,
                                 total_q=0, max_seqlen_q=0, window=None, decode=True):
    """The device-side precondition checks applied to host (NumPy) arrays: the
    ATTN_SINK_CHECK_* bits of every violation."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    cu = None if cu_seqlens_q is None else np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    w1, w2 = _window(window)
    flags = ctypes.c_uint(0)
    _check(lib().attn_sink_check_paged_inputs(
        bt.ctypes.data, sl.ctypes.data, None if cu is None else cu.ctypes.data, bt.shape[0],
        total_q, max_seqlen_q, bt.shape[1], page_size, num_pages, w1, w2, int(bool(decode)),
        ctypes.byref(flags)))
    return flags.value


class AttnSinkError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"attn_sink status {status}: {message}")
        self.status = status


def _check(status):
    if status != OK:
        raise AttnSinkError(status, lib().attn_sink_last_error().decode())


def abi_version():
    return lib().attn_sink_abi_version()


def last_error():
    return lib().attn_sink_last_error().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _window(window):
    if window is None:
        return -1, -1
    w1, w2 = window
    return int(w1), int(w2)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def attn_sink_fwd_prefill(q, k, v, sink=None, causal=True, softmax_scale=None, window=None,
                          out=None, lse=None, return_lse=True):
    """O [B,Sq,Hq,D], LSE [B,Hq,Sq] for q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], sink [Hq] fp32."""
    dev = q.device
    _need(q, "q")
    _need(k, "k", q.dtype, dev)
    _need(v, "v", q.dtype, dev)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Sk, Hkv, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
        if sink.shape != (Hq,):
            raise ValueError(f"sink must have shape ({Hq},)")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    w1, w2 = _window(window)
    _check(lib().attn_sink_fwd_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(out), _ptr(lse),
                                       B, Sq, Sk, Hq, Hkv, D, scale, int(bool(causal)), w1, w2,
                                       _dtype_code(q), _stream(dev)))
    return out, lse


def attn_sink_decode_workspace_bytes(B, Hq, Hkv, D, page_size, max_pages_per_seq, window=None,
                                     num_splits=0):
    w1, w2 = _window(window)
    return lib().attn_sink_decode_workspace_bytes(B, Hq, Hkv, D, page_size, max_pages_per_seq,
                                                  w1, w2, num_splits)


def attn_sink_fwd_decode_paged(q, k_cache, v_cache, block_table, seqlens_k, sink=None,
                               softmax_scale=None, window=None, num_splits=0, out=None, lse=None,
                               workspace=None, return_lse=True):
    """O [B,Hq,D], LSE [B,Hq] for one new token per sequence against a paged KV cache."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (num_pages, page_size, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, Hkv, D]")
    if block_table.dim() != 2 or block_table.shape[0] != B or seqlens_k.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens_k [B]")
    max_pages = block_table.shape[1]
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    w1, w2 = _window(window)
    need = lib().attn_sink_decode_workspace_bytes(B, Hq, Hkv, D, page_size, max_pages, w1, w2,
                                                  num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seqlens_k), _ptr(sink),
        _ptr(out), _ptr(lse), B, Hq, Hkv, D, page_size, max_pages, num_pages, scale, w1, w2,
        num_splits, _ptr(workspace), workspace.numel() * workspace.element_size(), BF16,
        _stream(dev)))
    return out, lse


DECODE_SCRATCH_BYTES = 32 << 20  # ATTN_SINK_DECODE_SCRATCH_BYTES


def attn_sink_fwd_decode_paged_noalloc(q, k_cache, v_cache, block_table, seqlens_k, sink=None,
                                       softmax_scale=None, window=None, num_splits=0, out=None,
                                       lse=None):
    """attn_sink_fwd_decode_paged on the library's own scratch: with `out` (and `lse`, if
    wanted) given, nothing is allocated on the device."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    B, Hq, D = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (num_pages, page_size, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, Hkv, D]")
    if block_table.dim() != 2 or block_table.shape[0] != B or seqlens_k.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens_k [B]")
    max_pages = block_table.shape[1]
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    w1, w2 = _window(window)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seqlens_k), _ptr(sink),
        _ptr(out), _ptr(lse), B, Hq, Hkv, D, page_size, max_pages, num_pages, scale, w1, w2,
        num_splits, BF16, _stream(dev)))
    return out, lse


def attn_sink_fwd_extend_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k,
                               max_seqlen_q, sink=None, softmax_scale=None, window=None,
                               out=None, lse=None, return_lse=True):
    """O [total_q,Hq,D], LSE [Hq,total_q] for packed new queries q [total_q,Hq,D] (rows of
    sequence b: cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1) against a paged KV cache holding
    seqlens_k[b] tokens of sequence b, the new ones last.  max_seqlen_q bounds every
    sequence's number of new queries (host int)."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    total_q, Hq, D = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (num_pages, page_size, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, Hkv, D]")
    B = seqlens_k.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.shape != (B + 1,):
        raise ValueError("block_table must be [B, max_pages], cu_seqlens_q [B+1], seqlens_k [B]")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    w1, w2 = _window(window)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_extend_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
        _ptr(seqlens_k), _ptr(sink), _ptr(out), _ptr(lse), B, total_q, int(max_seqlen_q), Hq, Hkv,
        D, page_size, block_table.shape[1], num_pages, scale, w1, w2, BF16, _stream(dev)))
    return out, lse


def attn_sink_fwd_index_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k,
                              max_seqlen_q, kv_index, cu_blocks, block_q, sink=None,
                              softmax_scale=None, out=None, lse=None, return_lse=True):
    """O [total_q,Hq,D], LSE [Hq,total_q] for packed new queries against a paged KV cache,
    each block of block_q query rows of a sequence attending to the tokens of one row of
    kv_index [num_blocks, topk] (sequence b's rows start at cu_blocks[b]) at or before its
    position."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q),
                    ("seqlens_k", seqlens_k), ("kv_index", kv_index), ("cu_blocks", cu_blocks)):
        _need(t, name, torch.int32, dev)
    total_q, Hq, D = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (num_pages, page_size, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, Hkv, D]")
    B = seqlens_k.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.shape != (B + 1,) \
            or cu_blocks.shape != (B + 1,) or kv_index.dim() != 2:
        raise ValueError("block_table must be [B, max_pages], cu_seqlens_q and cu_blocks [B+1], "
                         "seqlens_k [B], kv_index [num_blocks, topk]")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_index_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
        _ptr(seqlens_k), _ptr(kv_index), _ptr(cu_blocks), _ptr(sink), _ptr(out), _ptr(lse), B,
        total_q, int(max_seqlen_q), Hq, Hkv, D, page_size, block_table.shape[1], num_pages,
        int(block_q), kv_index.shape[1], scale, BF16, _stream(dev)))
    return out, lse


def attn_sink_index_rows_workspace_bytes(total_q, Hq, Hkv, D, topk):
    return lib().attn_sink_index_rows_workspace_bytes(total_q, Hq, Hkv, D, topk)


def attn_sink_fwd_index_rows_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k,
                                   kv_index, sink=None, softmax_scale=None, out=None, lse=None,
                                   workspace=None, return_lse=True):
    """O [total_q,Hq,D], LSE [Hq,total_q] for packed new queries against a paged KV cache,
    packed row r attending to the tokens of kv_index [total_q, topk] row r at or before its
    position."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    for name, t in (("block_table", block_table), ("cu_seqlens_q", cu_seqlens_q),
                    ("seqlens_k", seqlens_k), ("kv_index", kv_index)):
        _need(t, name, torch.int32, dev)
    total_q, Hq, D = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (num_pages, page_size, Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [num_pages, page_size, Hkv, D]")
    B = seqlens_k.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.shape != (B + 1,) \
            or kv_index.dim() != 2 or kv_index.shape[0] != total_q:
        raise ValueError("block_table must be [B, max_pages], cu_seqlens_q [B+1], seqlens_k [B], "
                         "kv_index [total_q, topk]")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    topk = kv_index.shape[1]
    if workspace is None:
        need = lib().attn_sink_index_rows_workspace_bytes(total_q, Hq, Hkv, D, topk)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_index_rows_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
        _ptr(seqlens_k), _ptr(kv_index), _ptr(sink), _ptr(out), _ptr(lse), B, total_q, Hq, Hkv,
        D, page_size, block_table.shape[1], num_pages, topk, scale, _ptr(workspace),
        workspace.numel() * workspace.element_size(), BF16, _stream(dev)))
    return out, lse


def attn_sink_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, sink=None,
                         causal=True, softmax_scale=None, window=None, out=None, lse=None,
                         return_lse=True):
    """O [total_q,Hq,D], LSE [Hq,total_q] for packed sequences: sequence b's queries are rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q [total_q,Hq,D] and its keys rows
    cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k, v [total_k,Hkv,D].  max_seqlen_q bounds
    every sequence's number of queries (host int)."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if k.shape != (total_k, Hkv, D) or v.shape != k.shape:
        raise ValueError("k/v must be [total_k, Hkv, D]")
    B = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev)
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
    w1, w2 = _window(window)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib().attn_sink_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(sink),
        _ptr(out), _ptr(lse), B, total_q, total_k, int(max_seqlen_q), Hq, Hkv, D, scale,
        int(bool(causal)), w1, w2, BF16, _stream(dev)))
    return out, lse


def attn_sink_bwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D):
    return lib().attn_sink_bwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D)


def attn_sink_bwd(q, k, v, o, dout, lse, sink=None, causal=True, softmax_scale=None, window=None,
                  dq=None, dk=None, dv=None, dsink=None, workspace=None):
    """(dq, dk, dv, dsink) of sum(dout * O); dsink is None when sink is None."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
        if dsink is None:
            dsink = torch.empty_like(sink)
    need = lib().attn_sink_bwd_workspace_bytes(B, Sq, Sk, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    w1, w2 = _window(window)
    _check(lib().attn_sink_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(sink), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dsink), B, Sq, Sk, Hq, Hkv, D, scale, int(bool(causal)), w1, w2,
        _ptr(workspace), workspace.numel() * workspace.element_size(), BF16, _stream(dev)))
    return dq, dk, dv, dsink


def attn_sink_bwd_varlen_workspace_bytes(B, total_q, max_seqlen_q, Hq):
    return lib().attn_sink_bwd_varlen_workspace_bytes(B, total_q, max_seqlen_q, Hq)


def attn_sink_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                         max_seqlen_k, sink=None, causal=True, softmax_scale=None, window=None,
                         dq=None, dk=None, dv=None, dsink=None, workspace=None):
    """(dq, dk, dv, dsink) of sum(dout * O) for attn_sink_fwd_varlen; lse is [Hq, total_q];
    dsink is None when sink is None."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_q.dim() != 1 or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B+1]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if sink is not None:
        _need(sink, "sink", torch.float32, dev)
        if dsink is None:
            dsink = torch.empty_like(sink)
    need = lib().attn_sink_bwd_varlen_workspace_bytes(B, total_q, int(max_seqlen_q), Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    w1, w2 = _window(window)
    _check(lib().attn_sink_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(sink), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), B, total_q, total_k,
        int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D, scale, int(bool(causal)), w1, w2,
        _ptr(workspace), workspace.numel() * workspace.element_size(), BF16, _stream(dev)))
    return dq, dk, dv, dsink


def attn_sink_decode_select_slots(block_table, seqlens_k, page_size, max_sel, window=None):
    """(slots [B, max_sel] int64, counts [B] int32) from the decode kernel's index map."""
    dev = block_table.device
    _need(block_table, "block_table", torch.int32)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    B, max_pages = block_table.shape
    slots = torch.empty((B, max_sel), dtype=torch.int64, device=dev)
    counts = torch.empty((B,), dtype=torch.int32, device=dev)
    w1, w2 = _window(window)
    _check(lib().attn_sink_decode_select_slots(_ptr(block_table), _ptr(seqlens_k), B, max_pages,
                                               page_size, w1, w2, _ptr(slots), _ptr(counts),
                                               max_sel, _stream(dev)))
    return slots, counts


def attn_sink_gather_kv(k_cache, v_cache, block_table, seqlens_k, max_sel, window=None):
    """K/V rows [B, max_sel, Hkv, D] of the selected tokens (zero past the selection)."""
    dev = k_cache.device
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens_k, "seqlens_k", torch.int32, dev)
    num_pages, page_size, Hkv, D = k_cache.shape
    B, max_pages = block_table.shape
    k_out = torch.empty((B, max_sel, Hkv, D), dtype=k_cache.dtype, device=dev)
    v_out = torch.empty_like(k_out)
    w1, w2 = _window(window)
    _check(lib().attn_sink_gather_kv(_ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                     _ptr(seqlens_k), B, Hkv, D, page_size, max_pages, w1, w2,
                                     _ptr(k_out), _ptr(v_out), max_sel, _dtype_code(k_cache),
                                     _stream(dev)))
    return k_out, v_out
