"""paged_kv_cache_332_amd — paged-attention decode on AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libpa.so`` (declared in
``include/pa.h``).  It only marshals arguments: every step of the decode path
(block-table bookkeeping, KV append, copy-on-write copies, attention, split-K
merge) runs in the library.  PyTorch supplies device memory and streams.

The library must be built first (``python paged_kv_cache_332_amd/build.py``);
importing this package without it raises ImportError — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "PAError", "lib", "LIB_PATH", "PA_F32", "PA_F16", "PA_BF16",
    "PA_KERNEL_AUTO", "PA_KERNEL_VALU", "PA_KERNEL_MFMA", "PA_KERNEL_STREAM",
    "pa_write_kv", "pa_copy_blocks", "pa_decode", "pa_decode_variant", "pa_decode_phase",
    "PA_PHASE_PASS", "PA_PHASE_MERGE", "PA_PHASE_ALL",
    "pa_decode_workspace_bytes", "pa_decode_default_partition", "pa_check_tables",
    "BlockManager", "alloc_cache", "cache_shapes", "torch_dtype_code", "pa_version", "pa_step",
    "pa_decode_stream_grid", "pa_decode_noalloc", "step_record_words", "step_args", "step_call",
    "stream_class_finish", "pa_stream_plan", "pa_prefill", "pa_prefill_workspace_bytes", "pa_prefill_column_blocks",
    "pa_swap_blocks",
    "pa_step_layer",
    "STEP_KV", "STEP_PASS", "STEP_MERGE", "STEP_ALL",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python paged_kv_cache_332_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

PA_OK, PA_ERR_INVALID, PA_ERR_OOM, PA_ERR_HIP, PA_ERR_UNSUPPORTED = range(5)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_KERNEL_AUTO, PA_KERNEL_VALU, PA_KERNEL_MFMA, PA_KERNEL_STREAM = 0, 1, 2, 3
PA_PHASE_PASS, PA_PHASE_MERGE, PA_PHASE_ALL = 1, 2, 3
_STATUS = {1: "invalid", 2: "out of blocks", 3: "hip", 4: "unsupported"}

_i32, _i64, _vp, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)


def _sig(name, res, *args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("pa_last_error", ctypes.c_char_p)
_sig("pa_version", ctypes.c_char_p)
_sig("pa_write_kv", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp)
_sig("pa_copy_blocks", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp)
_sig("pa_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32, _i32)
_sig("pa_decode_default_partition", _i32, _i32, _i32, _i32, _i32)
_DECODE_ARGS = [_vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                _i32, _f32, _i32, _vp, _sz, _vp]
_sig("pa_decode", _i32, *_DECODE_ARGS)
_sig("pa_decode_variant", _i32, *_DECODE_ARGS, _i32)
_sig("pa_decode_phase", _i32, *_DECODE_ARGS, _i32, _i32)
_sig("pa_decode_noalloc", _i32, *_DECODE_ARGS[:18], _vp)
_sig("pa_prefill", _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
     _i32, _i32, _f32, _vp, _sz, _vp)
_sig("pa_prefill_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32, _i32)
_sig("pa_prefill_column_blocks", _i32, _i32, _i32, _i32, _i32)
_sig("pa_bm_create", _vp, _i32, _i32, _pi32)
_sig("pa_bm_destroy", None, _vp)
_sig("pa_bm_add_seq", _i32, _vp, _i64, _i32, _pi32)
_sig("pa_bm_append_slots", _i32, _vp, _pi64, _i32, _pi32, _pi32, _pi32)
_sig("pa_bm_fork", _i32, _vp, _i64, _i64)
_sig("pa_bm_free_seq", _i32, _vp, _i64)
_sig("pa_bm_export", _i32, _vp, _pi64, _i32, _i32, _pi32, _pi32)
_sig("pa_bm_num_free", _i32, _vp)
_sig("pa_bm_admit", _i32, _vp, _i64, _i32, _i32, _pi32)
_sig("pa_bm_swap_out", _i32, _vp, _i64, _pi32, _pi32)
_sig("pa_bm_swap_in", _i32, _vp, _i64, _pi32, _pi32)
_sig("pa_bm_swapped_len", _i32, _vp, _i64)
_sig("pa_bm_add_seq_cached", _i32, _vp, _i64, _pi32, _i32, _pi32, _pi32)
_sig("pa_bm_cache_stats", _i32, _vp, _pi64)
_sig("pa_bm_cache_clear", _i32, _vp)
_sig("pa_swap_blocks", _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp)
_sig("pa_bm_occupancy", _i32, _vp, _pi64)
_sig("pa_bm_refcount", _i32, _vp, _i32)
_sig("pa_bm_seq_len", _i32, _vp, _i64)
_sig("pa_bm_shared_blocks", _i32, _vp, _i64)
_sig("pa_bm_num_seqs", _i32, _vp)
_sig("pa_bm_free_list", _i32, _vp, _pi32, _i32)
_sig("pa_bm_stats", _i32, _vp, _pi64)
_sig("pa_check_tables", _i32, _pi32, _i32, _i32, _pi32, _i32, _i32)
_sig("pa_step", _i32, _vp, _pi64, _i32, _vp, _vp, _sz, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
     _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp, _vp, _pi32, _pi32, _i32, _vp)
_sig("pa_decode_stream_grid", _i32, _i32, _i32, _i32, _i32)
_sig("pa_step_layer", _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
     _i32, _f32, _i32, _vp, _sz, _i32, _vp, _i32, _vp, _vp, _vp)
_sig("pa_step_record_words", _sz, _i32, _i32, _i32)
_sig("pa_stream_class_finish", _i32, _vp, _i32, _i32, _vp)
_sig("pa_stream_plan", _i64, _pi32, _i32, _i32, _i32, _pi32, _pi32, _sz, _pi32)


class PAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{_STATUS.get(status, status)}] {msg}")
        self.status = status


class OutOfBlocks(PAError):
    pass


def _check(st: int):
    if st != PA_OK:
        msg = lib.pa_last_error().decode()
        raise (OutOfBlocks if st == PA_ERR_OOM else PAError)(st, msg)


def pa_version() -> str:
    return lib.pa_version().decode()


# ------------------------------------------------------------------ tensors
def torch_dtype_code(dtype) -> int:
    import torch
    return {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}[dtype]


def cache_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, elem_bytes: int):
    """Shapes of the K pool [N][Hkv][D/X][BS][X] and V pool [N][Hkv][D][BS]."""
    x = 16 // elem_bytes
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
            (num_blocks, num_kv_heads, head_dim, block_size))


def alloc_cache(num_blocks, num_kv_heads, head_dim, block_size, dtype, device="cuda", poison=True):
    """Allocate a K and a V pool with torch; optionally fill with quiet NaN."""
    import torch
    ks, vs = cache_shapes(num_blocks, num_kv_heads, head_dim, block_size, torch.empty((), dtype=dtype).element_size())
    k = torch.empty(ks, dtype=dtype, device=device)
    v = torch.empty(vs, dtype=dtype, device=device)
    if poison:
        k.fill_(float("nan"))
        v.fill_(float("nan"))
    return k, v


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _pool_dims(k_cache, v_cache):
    n, hkv, dx, bs, x = k_cache.shape
    d = dx * x
    assert tuple(v_cache.shape) == (n, hkv, d, bs), "V pool shape does not match K pool"
    assert k_cache.dtype == v_cache.dtype and k_cache.is_contiguous() and v_cache.is_contiguous()
    return n, hkv, d, bs


def pa_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None) -> None:
    """k_new/v_new [T][Hkv][D], slot_mapping int32 [T] (device tensors)."""
    n, hkv, d, bs = _pool_dims(k_cache, v_cache)
    t = int(slot_mapping.numel())
    assert k_new.is_contiguous() and v_new.is_contiguous() and slot_mapping.is_contiguous()
    assert tuple(k_new.shape) == (t, hkv, d) and tuple(v_new.shape) == (t, hkv, d)
    assert k_new.dtype == k_cache.dtype and str(slot_mapping.dtype) == "torch.int32"
    _check(lib.pa_write_kv(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                           slot_mapping.data_ptr(), t, hkv, d, bs, n, torch_dtype_code(k_cache.dtype),
                           _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pairs int32 [P][2] = (src, dst) (device tensor)."""
    n, hkv, d, bs = _pool_dims(k_cache, v_cache)
    assert pairs.is_contiguous() and str(pairs.dtype) == "torch.int32"
    _check(lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(), int(pairs.numel() // 2),
                              hkv, d, bs, n, torch_dtype_code(k_cache.dtype), _stream(stream)))


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size=0) -> int:
    """Bytes of decode workspace (256-byte aligned device memory, any contents)."""
    return int(lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                             partition_size))


def pa_decode_default_partition(num_seqs, num_kv_heads, max_context_len, block_size) -> int:
    return int(lib.pa_decode_default_partition(num_seqs, num_kv_heads, max_context_len, block_size))


def pa_decode_variant(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int,
                      scale: float, partition_size: int = 0, workspace=None, stream=None,
                      kernel: int = PA_KERNEL_AUTO, phase: int = PA_PHASE_ALL) -> None:
    """q/out [B][Hq][D]; block_tables int32 [B][stride]; context_lens int32 [B]."""
    n, hkv, d, bs = _pool_dims(k_cache, v_cache)
    b, hq, dq = q.shape
    assert dq == d and tuple(out.shape) == (b, hq, d) and q.is_contiguous() and out.is_contiguous()
    assert block_tables.is_contiguous() and block_tables.dim() == 2 and block_tables.shape[0] == b
    assert context_lens.is_contiguous() and context_lens.numel() == b
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                          workspace.numel() * workspace.element_size())
    _check(lib.pa_decode_phase(out.data_ptr(), torch_dtype_code(out.dtype), q.data_ptr(), k_cache.data_ptr(),
                               v_cache.data_ptr(), torch_dtype_code(k_cache.dtype), block_tables.data_ptr(),
                               int(block_tables.shape[1]), context_lens.data_ptr(), int(max_context_len),
                               b, hq, hkv, d, bs, n, float(scale), int(partition_size), ws_ptr, ws_bytes,
                               _stream(stream), int(kernel), int(phase)))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int, scale: float,
              partition_size: int = 0, workspace=None, stream=None) -> None:
    pa_decode_variant(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                      partition_size, workspace, stream, PA_KERNEL_AUTO)


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int, scale: float,
                      partition_size: int = 0, stream=None) -> None:
    """pa_decode with the library's static device scratch as its workspace
    (no allocation; see pa_decode_noalloc in pa.h)."""
    n, hkv, d, bs = _pool_dims(k_cache, v_cache)
    b, hq, dq = q.shape
    assert dq == d and tuple(out.shape) == (b, hq, d) and q.is_contiguous() and out.is_contiguous()
    assert block_tables.is_contiguous() and block_tables.dim() == 2 and block_tables.shape[0] == b
    assert context_lens.is_contiguous() and context_lens.numel() == b
    _check(lib.pa_decode_noalloc(out.data_ptr(), torch_dtype_code(out.dtype), q.data_ptr(), k_cache.data_ptr(),
                                 v_cache.data_ptr(), torch_dtype_code(k_cache.dtype), block_tables.data_ptr(),
                                 int(block_tables.shape[1]), context_lens.data_ptr(), int(max_context_len),
                                 b, hq, hkv, d, bs, n, float(scale), int(partition_size), _stream(stream)))


def pa_swap_blocks(k_cache, v_cache, host_k, host_v, blocks, to_host: bool, stream=None) -> None:
    """Whole blocks between the pools and pinned host tensors ([n][Hkv*D*BS]
    elements each); ``blocks`` is an int32 tensor, pinned or on the device."""
    import torch
    n_, hkv, d, bs = _pool_dims(k_cache, v_cache)
    per_block = hkv * d * bs
    if blocks.dtype != torch.int32 or not blocks.is_contiguous():
        raise PAError("pa_swap_blocks: blocks must be a contiguous int32 tensor")
    for name, h in (("host_k", host_k), ("host_v", host_v)):
        if h.dtype != k_cache.dtype or not h.is_contiguous() or h.numel() < blocks.numel() * per_block:
            raise PAError(f"pa_swap_blocks: {name} must be a contiguous {k_cache.dtype} tensor of at least "
                          f"{blocks.numel()} x {per_block} elements")
    _check(lib.pa_swap_blocks(k_cache.data_ptr(), v_cache.data_ptr(), host_k.data_ptr(), host_v.data_ptr(),
                              blocks.data_ptr(), int(blocks.numel()), 1 if to_host else 0, hkv, d, bs, n_,
                              torch_dtype_code(k_cache.dtype), _stream(stream)))


def pa_prefill(out, q, k_cache, v_cache, block_tables, query_start, context_lens, max_query_len: int,
               max_context_len: int, scale: float, stream=None, workspace=None) -> None:
    """Causal attention of the chunks q[query_start[i]:query_start[i+1]] over
    their sequences' paged context (see pa_prefill in pa.h).  Tensors on the
    device; query_start / context_lens int32; workspace (uint8, device, at
    least pa_prefill_workspace_bytes(...) bytes) lets short chunks split
    their contexts."""
    n_, hkv, d, bs = _pool_dims(k_cache, v_cache)
    _check(lib.pa_prefill(out.data_ptr(), torch_dtype_code(out.dtype), q.data_ptr(), k_cache.data_ptr(),
                          v_cache.data_ptr(), torch_dtype_code(k_cache.dtype), block_tables.data_ptr(),
                          int(block_tables.shape[1]), query_start.data_ptr(), context_lens.data_ptr(),
                          int(max_query_len), int(max_context_len), int(context_lens.shape[0]), int(q.shape[1]), hkv,
                          d, bs, n_, float(scale), None if workspace is None else workspace.data_ptr(),
                          0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))


def pa_prefill_column_blocks(num_q_heads: int, num_kv_heads: int, max_query_len: int, num_seqs: int) -> int:
    """Column blocks per wave pa_prefill takes for this launch shape (see pa.h)."""
    return int(lib.pa_prefill_column_blocks(int(num_q_heads), int(num_kv_heads), int(max_query_len), int(num_seqs)))


def pa_prefill_workspace_bytes(max_query_len: int, max_context_len: int, num_seqs: int, num_q_heads: int,
                               num_kv_heads: int, head_dim: int) -> int:
    """Bytes of workspace pa_prefill's context split needs (0: no split)."""
    return int(lib.pa_prefill_workspace_bytes(int(max_query_len), int(max_context_len), int(num_seqs),
                                              int(num_q_heads), int(num_kv_heads), int(head_dim)))


def pa_step(bm: "BlockManager", seqs_i64: np.ndarray, stage_host, stage_dev, table_stride: int, k_cache, v_cache,
            k_new, v_new, q, out, scale: float, partition_size: int = 0, workspace=None, kernel: int = PA_KERNEL_AUTO,
            stream=None, pass_events=None, wg_weights: Optional[np.ndarray] = None, wave_times=None) -> int:
    """One decode step (see pa_step in pa.h); returns the longest context.
    ``seqs_i64`` is a contiguous int64 array; stage_host/stage_dev are int32
    tensors (pinned / device) of at least step_record_words(n, table_stride,
    Hkv) words;
    ``pass_events`` = (begin, end) torch CUDA events already created (recorded
    once), recorded around the decode pass; ``wg_weights`` (contiguous int32,
    pa_decode_stream_grid entries) sets the stream kernel's workgroup shares
    and ``wave_times`` (int32 tensor, pinned or device, 8 x grid) receives its
    wave start/end stamps."""
    n_, hkv, d, bs = _pool_dims(k_cache, v_cache)
    n = int(seqs_i64.shape[0])
    hq = int(q.shape[1])
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                          workspace.numel() * workspace.element_size())
    ev0, ev1 = (None, None) if pass_events is None else (pass_events[0].cuda_event, pass_events[1].cuda_event)
    max_ctx = ctypes.c_int32(0)
    words = min(stage_host.numel(), stage_dev.numel())
    _check(lib.pa_step(bm._h, seqs_i64.ctypes.data_as(_pi64), n, stage_host.data_ptr(), stage_dev.data_ptr(),
                       words, int(table_stride), k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                       q.data_ptr(), out.data_ptr(), torch_dtype_code(out.dtype), torch_dtype_code(k_cache.dtype),
                       hq, hkv, d, bs, n_, float(scale), int(partition_size), ws_ptr, ws_bytes, int(kernel),
                       _stream(stream), ev0, ev1, ctypes.byref(max_ctx),
                       None if wg_weights is None else wg_weights.ctypes.data_as(_pi32),
                       0 if wg_weights is None else int(wg_weights.shape[0]),
                       None if wave_times is None else wave_times.data_ptr()))
    return int(max_ctx.value)


def step_args(bm: "BlockManager", seqs_i64: np.ndarray, table_stride: int, k_cache, v_cache, k_new, v_new, q, out,
              scale: float, partition_size: int, workspace, kernel: int, stream, wg_weights=None) -> list:
    """pa_step's arguments as a list for ``step_call``, for callers that
    repeat one step shape: the step record (3, 4 and 5), the pass events (26,
    27) and the wave stamps (31) are set per call; entry 28 points at a
    c_int32 that receives the longest context.  ``seqs_i64`` and
    ``wg_weights`` must stay alive (and in place) while the list is used."""
    n_, hkv, d, bs = _pool_dims(k_cache, v_cache)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                          workspace.numel() * workspace.element_size())
    max_ctx = ctypes.c_int32(0)
    return [bm._h, seqs_i64.ctypes.data_as(_pi64), int(seqs_i64.shape[0]), None, None, 0, int(table_stride),
            k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), q.data_ptr(), out.data_ptr(),
            torch_dtype_code(out.dtype), torch_dtype_code(k_cache.dtype), int(q.shape[1]), hkv, d, bs, n_,
            float(scale), int(partition_size), ws_ptr, ws_bytes, int(kernel), _stream(stream), None, None,
            ctypes.pointer(max_ctx), None if wg_weights is None else wg_weights.ctypes.data_as(_pi32),
            0 if wg_weights is None else int(wg_weights.shape[0]), None]


def step_call(args: list) -> int:
    """pa_step on an argument list from ``step_args``; returns the longest
    context."""
    _check(lib.pa_step(*args))
    return int(args[28].contents.value)


def stream_class_finish(wave_times, grid: int, classes: int, out: np.ndarray) -> np.ndarray:
    """Mean finish time per workgroup class of a completed stream pass (see
    pa_stream_class_finish in pa.h) into ``out`` (float64, ``classes``)."""
    ptr = wave_times if isinstance(wave_times, int) else wave_times.data_ptr()
    _check(lib.pa_stream_class_finish(ptr, int(grid), int(classes), out.ctypes.data))
    return out


STEP_KV, STEP_PASS, STEP_MERGE, STEP_ALL = 1, 2, 4, 7


def pa_step_layer(stage_host, stage_dev, n: int, table_stride: int, k_cache, v_cache, k_new, v_new, q, out,
                  scale: float, partition_size: int = 0, workspace=None, kernel: int = PA_KERNEL_AUTO, stream=None,
                  phases: int = STEP_ALL, pass_events=None, wave_times=None) -> None:
    """The device part of the last pa_step again on its record, for another
    layer (see pa_step_layer in pa.h); ``phases`` from STEP_KV | STEP_PASS |
    STEP_MERGE."""
    n_, hkv, d, bs = _pool_dims(k_cache, v_cache)
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                          workspace.numel() * workspace.element_size())
    ev0, ev1 = (None, None) if pass_events is None else (pass_events[0].cuda_event, pass_events[1].cuda_event)
    nil = 0
    _check(lib.pa_step_layer(stage_host.data_ptr(), stage_dev.data_ptr(), int(n), int(table_stride),
                             k_cache.data_ptr(), v_cache.data_ptr(),
                             nil if k_new is None else k_new.data_ptr(), nil if v_new is None else v_new.data_ptr(),
                             q.data_ptr(), out.data_ptr(), torch_dtype_code(out.dtype),
                             torch_dtype_code(k_cache.dtype), int(q.shape[1]), hkv, d, bs, n_, float(scale),
                             int(partition_size), ws_ptr, ws_bytes, int(kernel), _stream(stream), int(phases), ev0, ev1,
                             None if wave_times is None else wave_times.data_ptr()))


def pa_decode_stream_grid(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int) -> int:
    """Workgroups of the stream kernel for this shape (0 when not used)."""
    return int(lib.pa_decode_stream_grid(num_seqs, num_q_heads, num_kv_heads, head_dim))


def pa_stream_plan(tile_prefix: np.ndarray, num_kv_heads: int, grid: int, weights: Optional[np.ndarray] = None):
    """The stream plan of pa_step for these tile counts: (wave starts [4 grid
    + 1], cut-item entries [ncut][8], wave list)."""
    pre = np.ascontiguousarray(tile_prefix, dtype=np.int32)
    n = pre.shape[0] - 1
    at = -(-(4 * grid + 1) // 4) * 4
    cap = at + 8 * n * num_kv_heads + 8 * grid
    out = np.zeros(cap, dtype=np.int32)
    ncut = ctypes.c_int32(0)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.int32)
    words = lib.pa_stream_plan(pre.ctypes.data_as(_pi32), n, num_kv_heads, grid,
                               None if w is None else w.ctypes.data_as(_pi32), out.ctypes.data_as(_pi32), cap,
                               ctypes.byref(ncut))
    if words < 0:
        raise PAError(1, "pa_stream_plan: bad arguments")
    k = int(ncut.value)
    return out[: 4 * grid + 1], out[at: at + 8 * k].reshape(k, 8), out[at + 8 * k: int(words)]


def step_record_words(max_seqs: int, table_stride: int, num_kv_heads: int) -> int:
    """Int32 words of a pa_step record for up to max_seqs sequences."""
    return int(lib.pa_step_record_words(max_seqs, table_stride, num_kv_heads))


def pa_check_tables(tables: np.ndarray, ctx_lens: np.ndarray, block_size: int, num_blocks: int) -> None:
    t = np.ascontiguousarray(tables, dtype=np.int32)
    c = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    _check(lib.pa_check_tables(t.ctypes.data_as(_pi32), t.shape[0], t.shape[1], c.ctypes.data_as(_pi32),
                               block_size, num_blocks))


# ------------------------------------------------------------ block manager
class BlockManager:
    """Host block manager (pa_bm_*): free list, refcounts, tables, COW."""

    def __init__(self, num_blocks: int, block_size: int, order: Optional[Sequence[int]] = None):
        self.block_size = block_size
        self.num_blocks = num_blocks
        arr = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
        self._h = lib.pa_bm_create(num_blocks, block_size, None if arr is None else arr.ctypes.data_as(_pi32))
        if not self._h:
            raise PAError(PA_ERR_INVALID, lib.pa_last_error().decode())

    def close(self):
        if getattr(self, "_h", None):
            lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_seq(self, seq: int, num_tokens: int) -> np.ndarray:
        out = np.empty(max(num_tokens, 0), dtype=np.int32)
        _check(lib.pa_bm_add_seq(self._h, int(seq), int(num_tokens), out.ctypes.data_as(_pi32)))
        return out

    def admit(self, seq: int, num_tokens: int, reserve_blocks: int = 0) -> np.ndarray:
        """add_seq only if reserve_blocks stay free afterwards (else OutOfBlocks)."""
        out = np.empty(max(num_tokens, 0), dtype=np.int32)
        _check(lib.pa_bm_admit(self._h, int(seq), int(num_tokens), int(reserve_blocks), out.ctypes.data_as(_pi32)))
        return out

    def swap_out(self, seq: int) -> np.ndarray:
        """Release the sequence's blocks, keeping its length; returns its table
        (copy the blocks out before they are reused)."""
        n = max(0, -(-max(self.seq_len(seq), 0) // self.block_size))
        out = np.empty(max(n, 1), dtype=np.int32)
        cnt = ctypes.c_int32(0)
        _check(lib.pa_bm_swap_out(self._h, int(seq), out.ctypes.data_as(_pi32), ctypes.byref(cnt)))
        return out[: cnt.value].copy()

    def swap_in(self, seq: int) -> np.ndarray:
        """Fresh blocks for a swapped-out sequence, in logical order."""
        n = max(0, -(-max(self.swapped_len(seq), 0) // self.block_size))
        out = np.empty(max(n, 1), dtype=np.int32)
        cnt = ctypes.c_int32(0)
        _check(lib.pa_bm_swap_in(self._h, int(seq), out.ctypes.data_as(_pi32), ctypes.byref(cnt)))
        return out[: cnt.value].copy()

    def swapped_len(self, seq: int) -> int:
        return int(lib.pa_bm_swapped_len(self._h, int(seq)))

    def add_seq_cached(self, seq: int, tokens) -> Tuple[np.ndarray, int]:
        """add_seq for a prompt given by its token ids, reusing cached full
        blocks of its prefix; returns (slots of all tokens, reused tokens)."""
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        out = np.empty(max(tok.size, 1), dtype=np.int32)
        hit = ctypes.c_int32(0)
        _check(lib.pa_bm_add_seq_cached(self._h, int(seq), tok.ctypes.data_as(_pi32), int(tok.size),
                                        out.ctypes.data_as(_pi32), ctypes.byref(hit)))
        return out[: tok.size].copy(), int(hit.value)

    def cache_stats(self) -> Tuple[int, int, int, int]:
        """(cached blocks, evictable blocks, reused blocks so far, looked-up blocks so far)"""
        out = np.zeros(4, dtype=np.int64)
        _check(lib.pa_bm_cache_stats(self._h, out.ctypes.data_as(_pi64)))
        return tuple(int(x) for x in out)

    def cache_clear(self) -> None:
        _check(lib.pa_bm_cache_clear(self._h))

    def occupancy(self) -> Tuple[int, int, int, int]:
        """(slots of held blocks, tokens, unused slots in last blocks, free slots)."""
        out = np.zeros(4, dtype=np.int64)
        _check(lib.pa_bm_occupancy(self._h, out.ctypes.data_as(_pi64)))
        return tuple(int(x) for x in out)

    def append_slots(self, seqs: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        slots = np.empty(len(s), dtype=np.int32)
        pairs = np.empty((len(s), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(lib.pa_bm_append_slots(self._h, s.ctypes.data_as(_pi64), len(s), slots.ctypes.data_as(_pi32),
                                      pairs.ctypes.data_as(_pi32), ctypes.byref(ncow)))
        return slots, pairs[: ncow.value].copy()

    def fork(self, parent: int, child: int) -> None:
        _check(lib.pa_bm_fork(self._h, int(parent), int(child)))

    def free_seq(self, seq: int) -> None:
        _check(lib.pa_bm_free_seq(self._h, int(seq)))

    def export(self, seqs: Sequence[int], stride: int, tables_out=None, ctx_out=None):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        tab = tables_out if tables_out is not None else np.empty((len(s), stride), dtype=np.int32)
        ctx = ctx_out if ctx_out is not None else np.empty(len(s), dtype=np.int32)
        _check(lib.pa_bm_export(self._h, s.ctypes.data_as(_pi64), len(s), int(stride), tab.ctypes.data_as(_pi32),
                                ctx.ctypes.data_as(_pi32)))
        return tab, ctx

    def num_free(self) -> int:
        return int(lib.pa_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(lib.pa_bm_refcount(self._h, int(block)))

    def seq_len(self, seq: int) -> int:
        return int(lib.pa_bm_seq_len(self._h, int(seq)))

    def shared_blocks(self, seq: int) -> int:
        """Blocks at the front of the sequence's table held elsewhere too
        (refcount above one); -1 if unknown."""
        return int(lib.pa_bm_shared_blocks(self._h, int(seq)))

    def num_seqs(self) -> int:
        return int(lib.pa_bm_num_seqs(self._h))

    def free_list(self) -> np.ndarray:
        """The free stack, next allocation first (evictable cached blocks not included)."""
        n = int(lib.pa_bm_num_free(self._h))      # an upper bound: it counts evictable blocks too
        out = np.empty(max(n, 1), dtype=np.int32)
        k = int(lib.pa_bm_free_list(self._h, out.ctypes.data_as(_pi32), n))
        return out[:k].copy()

    def stats(self) -> Tuple[int, int, int, int, int]:
        out = np.zeros(5, dtype=np.int64)
        _check(lib.pa_bm_stats(self._h, out.ctypes.data_as(_pi64)))
        return tuple(int(x) for x in out)
