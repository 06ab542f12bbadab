"""Python binding of libpa.so (argument marshalling only).

Every operation runs in the library's HIP kernels; this module only turns
torch tensors into device pointers, picks the stream, and maps status codes
to exceptions.  There is no fallback: if ``libpa.so`` has not been built,
loading it raises.

The functions carry the C names: :func:`pa_write_kv`, :func:`pa_decode`,
:func:`pa_copy_blocks`, :func:`pa_decode_workspace_bytes`.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_PARTITION_AUTO = -1          # pa_decode balances the split itself
DTYPE_CODE = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8_e4m3": PA_FP8_E4M3}
_TORCH_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
               torch.float8_e4m3fn: PA_FP8_E4M3}
_TORCH_STORAGE = {PA_F32: (torch.float32,), PA_F16: (torch.float16,),
                  PA_BF16: (torch.bfloat16, torch.int16, torch.uint16),
                  PA_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8)}
_ELEM = {PA_F32: 4, PA_F16: 2, PA_BF16: 2, PA_FP8_E4M3: 1}

EXPORTED = ("pa_write_kv", "pa_decode", "pa_decode_workspace_bytes", "pa_copy_blocks",
            "pa_status_string", "pa_last_error", "pa_version", "pa_time_next_decode",
            "pa_decode_status", "pa_set_wait_polls", "pa_decode_noalloc", "pa_swap_blocks",
            "pa_decode_window", "pa_prefill")
PA_NOALLOC_SCRATCH_BYTES = 32 << 20
PA_WS_CLEAN, PA_WS_MISPLACED, PA_WS_TIMED_OUT = 0, 1, 2


class PaError(RuntimeError):
    """A libpa call returned a non-zero status."""

    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail} ({name_of(status)})")
        self.status = status


class KvPool(ctypes.Structure):
    """Mirror of ``pa_kv_pool`` in include/pa.h."""
    _fields_ = [
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m paged_kv_cache_91_amd.build, or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
        pool_p = ctypes.POINTER(KvPool)
        L.pa_write_kv.argtypes = [vp, vp, i32, i32, vp, pool_p, vp]
        L.pa_write_kv.restype = ctypes.c_int
        L.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.pa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.pa_decode.argtypes = [vp, i32, i32, i32, pool_p, vp, i32, vp, ctypes.c_float, vp, i32,
                                vp, ctypes.c_size_t, vp]
        L.pa_decode.restype = ctypes.c_int
        L.pa_copy_blocks.argtypes = [pool_p, vp, i32, vp]
        L.pa_copy_blocks.restype = ctypes.c_int
        L.pa_status_string.argtypes = [ctypes.c_int]
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_last_error.argtypes = []
        L.pa_last_error.restype = ctypes.c_char_p
        L.pa_version.argtypes = []
        L.pa_version.restype = ctypes.c_int
        L.pa_time_next_decode.argtypes = [vp, vp]
        L.pa_time_next_decode.restype = ctypes.c_int
        L.pa_decode_status.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
        L.pa_decode_status.restype = ctypes.c_int
        L.pa_set_wait_polls.argtypes = [i32]
        L.pa_set_wait_polls.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = [vp, i32, i32, i32, pool_p, vp, i32, vp, ctypes.c_float, vp, i32, vp]
        L.pa_decode_noalloc.restype = ctypes.c_int
        L.pa_decode_window.argtypes = [vp, i32, i32, i32, pool_p, vp, i32, vp, i32, ctypes.c_float, vp, i32,
                                       vp, ctypes.c_size_t, vp]
        L.pa_decode_window.restype = ctypes.c_int
        L.pa_prefill.argtypes = [vp, i32, i32, i32, pool_p, i32, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp]
        L.pa_prefill.restype = ctypes.c_int
        L.pa_swap_blocks.argtypes = [pool_p, pool_p, vp, i32, vp]
        L.pa_swap_blocks.restype = ctypes.c_int
        _lib = L
    return _lib


def name_of(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(status: int, name: str) -> None:
    if status != 0:
        raise PaError(status, name, lib().pa_last_error().decode())


def _ptr(t: Optional[torch.Tensor], what: str, allow_none=False, pinned_ok=False) -> Optional[int]:
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{what} is required")
    if not t.is_cuda and not (pinned_ok and t.is_pinned()):
        raise ValueError(f"{what} must be a device tensor" + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _torch_stream(stream, device) -> torch.cuda.Stream:
    """The torch stream object for ``stream`` (None: the current stream)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def dtype_code(t: torch.Tensor, dtype: Optional[str] = None) -> int:
    """pa_dtype of a tensor; ``dtype`` names it when the storage is raw bits
    (int16/uint16 for bf16, uint8 for fp8)."""
    code = DTYPE_CODE[dtype] if dtype is not None else _TORCH_CODE.get(t.dtype)
    if code is None or t.dtype not in _TORCH_STORAGE[code]:
        raise ValueError(f"tensor dtype {t.dtype} cannot hold {dtype or 'that dtype'}")
    return code


def make_pool(k_pool: torch.Tensor, v_pool: torch.Tensor, dtype: Optional[str] = None,
              k_scale: float = 1.0, v_scale: float = 1.0, host: bool = False) -> KvPool:
    """Descriptor of caller-owned pools ``[num_blocks, Hkv, bs, D]``
    (``host``: a swap area in pinned host memory, for pa_swap_blocks)."""
    if k_pool.shape != v_pool.shape or k_pool.dim() != 4:
        raise ValueError("pools must be 4-D [num_blocks, num_kv_heads, block_size, head_dim] of equal shape")
    code = dtype_code(k_pool, dtype)
    if dtype_code(v_pool, dtype) != code:
        raise ValueError("K and V pools differ in dtype")
    n, h, bs, d = k_pool.shape
    return KvPool(_ptr(k_pool, "k_pool", pinned_ok=host), _ptr(v_pool, "v_pool", pinned_ok=host), n, h, bs, d,
                  code, float(k_scale), float(v_scale))


def pa_write_kv(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, pool: KvPool,
                src_dtype: Optional[str] = None, stream=None) -> None:
    """Cache write: rows ``[T, Hkv, D]`` to the slots in ``slot_mapping`` (int64 [T])."""
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    num_tokens = int(slot_mapping.numel())
    if k.shape != v.shape or (num_tokens and k.shape[0] != num_tokens):
        raise ValueError("k, v must be [num_tokens, num_kv_heads, head_dim]")
    if num_tokens and tuple(k.shape[1:]) != (pool.num_kv_heads, pool.head_dim):
        raise ValueError("k, v rows do not match the pool's heads / head_dim")
    code = dtype_code(k, src_dtype)
    _check(lib().pa_write_kv(_ptr(k, "k"), _ptr(v, "v"), code, num_tokens,
                             _ptr(slot_mapping, "slot_mapping"), ctypes.byref(pool), _stream(stream)),
           "pa_write_kv")


def pa_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                              max_blocks_per_seq: int, block_size: int, partition_size: int) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               max_blocks_per_seq, block_size, partition_size))


def new_workspace(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  max_blocks_per_seq: int, block_size: int, partition_size: int,
                  device="cuda") -> torch.Tensor:
    """Zero-filled split-KV workspace (its arrival counters must start at zero)."""
    n = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                  block_size, partition_size)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def pa_decode_window(q: torch.Tensor, pool: KvPool, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, window: int, scale: float,
                     out: Optional[torch.Tensor] = None, partition_size: int = 0,
                     workspace: Optional[torch.Tensor] = None, q_dtype: Optional[str] = None,
                     stream=None) -> torch.Tensor:
    """Paged decode under a sliding window of ``window`` positions (see
    :func:`pa_decode` for the other arguments)."""
    return pa_decode(q, pool, block_tables, context_lens, scale, out=out, partition_size=partition_size,
                     workspace=workspace, q_dtype=q_dtype, stream=stream, _window=int(window))


def pa_decode(q: torch.Tensor, pool: KvPool, block_tables: torch.Tensor,
              context_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
              partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
              q_dtype: Optional[str] = None, stream=None, _window: Optional[int] = None) -> torch.Tensor:
    """Paged decode attention; returns ``out`` ([S, Hq, D], q's dtype).

    ``workspace`` (split mode) is allocated zero-filled here when not given,
    on the stream the kernels run on (so the fill is ordered before them, and
    the memory is not handed out again before they end); pass one from
    :func:`new_workspace` to keep allocation out of a timed loop.
    """
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    s, hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, max_blocks], context_lens [S]")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    qcode = dtype_code(q, q_dtype)
    maxb = int(block_tables.shape[1])
    ws_ptr, ws_bytes, own_ws = None, 0, None
    if partition_size != 0:
        if workspace is None:
            own_ws = _torch_stream(stream, q.device)
            with torch.cuda.stream(own_ws):
                workspace = new_workspace(s, hq, pool.num_kv_heads, d, maxb, pool.block_size,
                                          partition_size, device=q.device)
        ws_ptr, ws_bytes = _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    if _window is None:
        _check(lib().pa_decode(_ptr(q, "q"), qcode, s, hq, ctypes.byref(pool), _ptr(block_tables, "block_tables"),
                               maxb, _ptr(context_lens, "context_lens"), float(scale), _ptr(out, "out"),
                               int(partition_size), ws_ptr, ws_bytes, _stream(stream)),
               "pa_decode")
    else:
        _check(lib().pa_decode_window(_ptr(q, "q"), qcode, s, hq, ctypes.byref(pool),
                                      _ptr(block_tables, "block_tables"), maxb, _ptr(context_lens, "context_lens"),
                                      _window, float(scale), _ptr(out, "out"), int(partition_size), ws_ptr,
                                      ws_bytes, _stream(stream)),
               "pa_decode_window")
    if own_ws is not None:
        workspace.record_stream(own_ws)
    return out


def pa_prefill(q: torch.Tensor, pool: KvPool, block_tables: torch.Tensor, context_lens: torch.Tensor,
               query_start: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
               window: int = 0, q_dtype: Optional[str] = None, stream=None) -> torch.Tensor:
    """Causal prefill: ``q`` ``[T, Hq, D]`` packed rows, ``query_start`` int32
    ``[S + 1]``; returns ``out`` ``[T, Hq, D]``."""
    if q.dim() != 3:
        raise ValueError("q must be [num_tokens, num_q_heads, head_dim]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or query_start.dtype != torch.int32:
        raise ValueError("block_tables, context_lens and query_start must be int32")
    s = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != s or query_start.shape != (s + 1,):
        raise ValueError("block_tables must be [S, max_blocks], query_start [S + 1]")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    t, hq, _ = q.shape
    _check(lib().pa_prefill(_ptr(q, "q"), dtype_code(q, q_dtype), t, hq, ctypes.byref(pool), s,
                            _ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
                            _ptr(context_lens, "context_lens"), _ptr(query_start, "query_start"), int(window),
                            float(scale), _ptr(out, "out"), _stream(stream)),
           "pa_prefill")
    return out


def pa_decode_noalloc(q: torch.Tensor, pool: KvPool, block_tables: torch.Tensor,
                      context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                      partition_size: int = 0, q_dtype: Optional[str] = None, stream=None) -> torch.Tensor:
    """pa_decode with the library's static scratch instead of a workspace;
    ``out`` is required (nothing is allocated)."""
    if q.dim() != 3 or out is None or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim] and out match it")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    s, hq, _ = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, max_blocks], context_lens [S]")
    _check(lib().pa_decode_noalloc(_ptr(q, "q"), dtype_code(q, q_dtype), s, hq, ctypes.byref(pool),
                                   _ptr(block_tables, "block_tables"), int(block_tables.shape[1]),
                                   _ptr(context_lens, "context_lens"), float(scale), _ptr(out, "out"),
                                   int(partition_size), _stream(stream)),
           "pa_decode_noalloc")
    return out


def pa_copy_blocks(pool: KvPool, src_dst_pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks for each (src, dst) row of an int64 ``[P, 2]`` tensor."""
    if src_dst_pairs.dtype != torch.int64 or (src_dst_pairs.numel() and src_dst_pairs.shape[-1] != 2):
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    num = int(src_dst_pairs.numel() // 2)
    _check(lib().pa_copy_blocks(ctypes.byref(pool), _ptr(src_dst_pairs, "src_dst_pairs") if num else None,
                                num, _stream(stream)),
           "pa_copy_blocks")


def pa_swap_blocks(src: KvPool, dst: KvPool, src_dst_pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks from pool pair ``src`` to ``dst`` (GPU pool and a
    pinned host swap area, either way) for each (src, dst) row of an int64
    ``[P, 2]`` tensor (device or pinned host)."""
    if src_dst_pairs.dtype != torch.int64 or (src_dst_pairs.numel() and src_dst_pairs.shape[-1] != 2):
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    num = int(src_dst_pairs.numel() // 2)
    _check(lib().pa_swap_blocks(ctypes.byref(src), ctypes.byref(dst),
                                _ptr(src_dst_pairs, "src_dst_pairs", pinned_ok=True) if num else None, num,
                                _stream(stream)),
           "pa_swap_blocks")


def pa_time_next_decode(start, stop) -> None:
    """Have the next pa_decode on this thread record ``start`` / ``stop`` as
    its kernels begin and end.  Each is an object whose ``cuda_event`` is a
    timing-enabled HIP event handle that exists (a torch.cuda.Event exists
    once it has been recorded)."""
    if (start is None) != (stop is None):
        raise ValueError("give both events or neither")
    _check(lib().pa_time_next_decode(None if start is None else start.cuda_event,
                                     None if stop is None else stop.cuda_event), "pa_time_next_decode")


def pa_decode_status(workspace: torch.Tensor, partition_size: int, stream=None) -> int:
    """Status word of a workspace (PA_WS_CLEAN / PA_WS_MISPLACED /
    PA_WS_TIMED_OUT); waits for ``stream`` to reach the read."""
    st = _torch_stream(stream, workspace.device)
    with torch.cuda.stream(st):
        out = torch.full((1,), -1, dtype=torch.int32, device=workspace.device)
    _check(lib().pa_decode_status(_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                  int(partition_size), _ptr(out, "status"), _stream(stream)),
           "pa_decode_status")
    st.synchronize()
    return int(out.item())


def pa_set_wait_polls(polls: int) -> None:
    """Test hook: poll bound of the balanced split's in-workgroup waits for
    this thread's later calls (0 restores the default)."""
    _check(lib().pa_set_wait_polls(int(polls)), "pa_set_wait_polls")
