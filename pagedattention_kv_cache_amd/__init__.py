"""Python binding of libpa.so, the MI355X paged KV-cache library (include/pa.h).

Argument marshalling only: torch tensors are turned into device pointers and
sizes, and the call goes to the C ABI on torch's current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If libpa.so is missing, :func:`lib` raises -- build it with
``python -m pagedattention_kv_cache_amd.build`` (or ``__graft_entry__.build()``).

    cache_write(k, v, slot_mapping, k_cache, v_cache)
    decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
           block_size, partition_size=0, workspace=None, flags=AUTO)

Cache tensors (tokens of a block in quads of four consecutive offsets):
``k_cache`` [num_blocks][num_kv_heads][block_size/4][head_dim/X][4][X] with
X = 16 bytes / element size (see :func:`key_cache_shape`), ``v_cache``
[num_blocks][num_kv_heads][block_size/4][head_dim][4].
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
AUTO, FORCE_VALU, FORCE_MFMA = 0, 1, 2
# waves per work item, OR-ed into flags (0 = library picks)
WAVES_1, WAVES_2, WAVES_4 = 4, 8, 12
WAVES_FLAG = {1: WAVES_1, 2: WAVES_2, 4: WAVES_4}
# one workgroup per possible (sequence, head, partition) item instead of the
# persistent grid over the items that hold tokens
NO_WORK_LIST = 16
# the items that hold tokens first, longest first (ordered on the device)
SORTED_GRID = 32
# a persistent grid walking the list of items that hold tokens
WORK_LIST = 48
GRID_NAMES = {NO_WORK_LIST: "grid", SORTED_GRID: "sorted", WORK_LIST: "work_list"}
# the workspace already holds the launch's item order (decode_order ran first)
ORDERED = 64
# torch.float8_e4m3fn: the OCP E4M3 KV-cache storage type (caches only)
_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3}

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pa status {status}: {message}")
        self.status = status


def key_chunk(dtype: torch.dtype) -> int:
    """X: elements per 16-byte chunk of the key cache layout."""
    return 16 // dtype.itemsize


def key_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                    dtype: torch.dtype) -> tuple:
    """[blocks][kv heads][block_size/4][head_dim/X][4][X]: tokens in quads of four."""
    X = key_chunk(dtype)
    return (num_blocks, num_kv_heads, block_size // 4, head_dim // X, 4, X)


def value_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int,
                      block_size: int) -> tuple:
    """[blocks][kv heads][block_size/4][head_dim][4]."""
    return (num_blocks, num_kv_heads, block_size // 4, head_dim, 4)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_blocks, num_kv_heads, block_size, head_dim) from validated caches."""
    _require(k_cache.dim() == 6 and v_cache.dim() == 5, "k_cache must be 6-D, v_cache 5-D")
    NB, H, nq, dx, four, X = k_cache.shape
    _require(X == key_chunk(k_cache.dtype) and four == 4,
             "k_cache must be [blocks][heads][block_size/4][head_dim/X][4][X]")
    d, bs = dx * X, nq * 4
    _require(tuple(v_cache.shape) == (NB, H, nq, d, 4), "v_cache shape does not match k_cache")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    return NB, H, bs, d


def lib() -> ctypes.CDLL:
    """Load libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library has not been built")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                 ctypes.c_size_t)
        L.pa_cache_write.restype = ctypes.c_int
        L.pa_cache_write.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i64, i32, i32, vp]
        dec_args = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32, i32, i32, i64, i32,
                    i32, i32, i32, vp, sz, u32, vp]
        for name in ("pa_decode", "pa_decode_partitions", "pa_decode_merge"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = dec_args
        f32 = ctypes.c_float
        dec8_args = [vp, vp, vp, vp, vp, vp, f32, f32, f32, i32, i32, i32, i32, i32, i32, i64, i32,
                     i32, i32, vp, sz, u32, vp]
        for name in ("pa_decode_fp8", "pa_decode_fp8_partitions"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = dec8_args
        decmq_args = [vp, vp, vp, vp, vp, vp, f32, f32, f32, i32, i32, i32, i32, i32, i32, i32,
                      i64, i32, i32, i32, i32, vp, sz, u32, vp]
        for name in ("pa_decode_mq", "pa_decode_mq_partitions", "pa_decode_mq_merge"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = decmq_args
        L.pa_check_tables.restype = ctypes.c_int
        L.pa_check_tables.argtypes = [vp, vp, i32, i32, i32, i64, vp, vp]
        L.pa_check_slots.restype = ctypes.c_int
        L.pa_check_slots.argtypes = [vp, i64, i64, i32, vp, vp]
        L.pa_decode_noalloc.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = dec_args[:18] + [u32, vp]
        step_args = [vp, vp, vp, i64, i64, i64] + dec_args
        L.pa_decode_order_fp8.restype = ctypes.c_int
        L.pa_decode_order_fp8.argtypes = [vp, vp, vp, i64, i64, i64, i32, f32, f32, vp, vp, vp, vp,
                                          vp, vp, f32, i32, i32, i32, i32, i32, i32, i64, i32,
                                          i32, i32, vp, sz, u32, vp]
        for name in ("pa_decode_step", "pa_decode_step_partitions", "pa_decode_order"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = step_args
        L.pa_decode_mq_kernel.restype = i32
        L.pa_decode_mq_kernel.argtypes = [i32, i32, i32, i32, i32, u32]
        L.pa_cache_write_fp8.restype = ctypes.c_int
        L.pa_cache_write_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i64, i32,
                                         i32, f32, f32, vp]
        L.pa_decode_partition_size.restype = i32
        L.pa_decode_partition_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, u32]
        L.pa_decode_partition_used.restype = i32
        L.pa_decode_partition_used.argtypes = [vp, sz, i32, i32, i32, i32, i32, i32, i32, u32, vp]
        L.pa_decode_workspace_size.restype = sz
        L.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, u32]
        L.pa_advance_step.restype = ctypes.c_int
        L.pa_advance_step.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]
        L.pa_decode_kernel.restype = i32
        L.pa_decode_kernel.argtypes = [i32, i32, i32, i32, u32]
        L.pa_decode_waves.restype = i32
        L.pa_decode_waves.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, u32]
        L.pa_decode_work_list.restype = i32
        L.pa_decode_work_list.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, u32]
        L.pa_decode_grid.restype = i32
        L.pa_decode_grid.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, u32]
        _declare_blocks(L)
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_status_string.argtypes = [i32]
        L.pa_abi_version.restype = i32
        L.pa_abi_version.argtypes = []
        _lib = L
    return _lib


def _declare_blocks(L, host_only: bool = False) -> None:
    """Argument types of the block-manager calls (host_only: only the pa_bm_*
    ones, for a library built from the host block manager alone)."""
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sigs = {
        "pa_bm_create": [i64, i32, i64, u32, vp],
        "pa_bm_add_sequence": [vp, i64, vp, i32, vp],
        "pa_bm_append": [vp, vp, vp, i32, vp, vp, vp],
        "pa_bm_fork": [vp, i64, i64],
        "pa_bm_free": [vp, i64],
        "pa_bm_mark_computed": [vp, i64],
        "pa_bm_slots": [vp, i64, i32, i32, vp],
        "pa_bm_block_tables": [vp, vp, i32, i32, vp, vp],
        "pa_bm_swap_out": [vp, i64, vp, vp],
        "pa_bm_swap_in": [vp, i64, vp, vp],
        "pa_bm_num_free_blocks": [vp, vp],
        "pa_bm_num_free_host_blocks": [vp, vp],
        "pa_bm_seq_info": [vp, i64, vp, vp],
        "pa_bm_ref_count": [vp, i32, vp],
        "pa_copy_blocks": [vp, vp, vp, i32, i64, i64, vp],
        "pa_swap_blocks": [vp, vp, vp, i32, i64, vp],
    }
    for name, args in sigs.items():
        if host_only and not name.startswith("pa_bm_"):
            continue
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = args
    L.pa_bm_destroy.restype = None
    L.pa_bm_destroy.argtypes = [vp]


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def _check(status: int) -> None:
    if status != PA_OK:
        raise PAError(status, status_string(status))


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise PAError(-3, f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device) -> int:
    """The current HIP stream of `device` (torch's raw handle query when it
    has one: a decode step makes several calls, and the Stream object costs
    microseconds each)."""
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None
                           else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise PAError(-2, msg)


def _decode_dims(out, q, k_cache, v_cache, block_tables, context_lens, block_size):
    """(B, Hq, d, NB, Hkv, bs, MB) of a decode call after the layout checks the
    C ABI cannot make (contiguity, cache layout, index dtypes).  Written out
    inline: a decode step makes several calls, each paying for these checks."""
    qs = q.shape
    if len(qs) != 3 or not q.is_contiguous():
        raise PAError(-2, "q must be contiguous [B][Hq][d]")
    if out.shape != qs or not out.is_contiguous():
        raise PAError(-2, "out must be contiguous [B][Hq][d]")
    B, Hq, d = qs
    ks = k_cache.shape
    if len(ks) != 6 or len(v_cache.shape) != 5:
        raise PAError(-2, "k_cache must be 6-D, v_cache 5-D")
    NB, Hkv, nq, dx, four, X = ks
    if four != 4 or X * k_cache.dtype.itemsize != 16:
        raise PAError(-2, "k_cache must be [blocks][heads][block_size/4][head_dim/X][4][X]")
    if v_cache.shape != (NB, Hkv, nq, dx * X, 4):
        raise PAError(-2, "v_cache shape does not match k_cache")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise PAError(-2, "caches must be contiguous")
    if nq * 4 != block_size or dx * X != d:
        raise PAError(-2, "cache shapes do not match block_size / head_dim")
    bts = block_tables.shape
    if (block_tables.dtype != torch.int32 or len(bts) != 2 or bts[0] != B
            or not block_tables.is_contiguous()):
        raise PAError(-2, "block_tables must be contiguous int32 [B][max_blocks]")
    if (context_lens.dtype != torch.int32 or context_lens.shape != (B,)
            or not context_lens.is_contiguous()):
        raise PAError(-2, "context_lens must be contiguous int32 [B]")
    return B, Hq, d, NB, Hkv, block_size, bts[1]


def cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Scatter k/v [T][Hkv][d] (token dim may be strided) into the caches."""
    _require(k.dim() == 3 and v.dim() == 3 and k.shape == v.shape, "k, v must be [T][Hkv][d]")
    T, H, d = k.shape
    NB, H2, bs, d2 = _cache_dims(k_cache, v_cache)
    _require((H2, d2) == (H, d), "cache shapes do not match k/v")
    for t in (k, v):
        _require(t.stride(2) == 1 and t.stride(1) == d, "heads of a token must be packed")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,)
             and slot_mapping.is_contiguous(), "slot_mapping must be contiguous int64 [T]")
    _require(k.dtype == v.dtype == k_cache.dtype == v_cache.dtype, "dtype mismatch")
    _check(lib().pa_cache_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                k_cache.data_ptr(), v_cache.data_ptr(), T, k.stride(0),
                                v.stride(0), H, d, NB, bs, _dt(k), _stream(k_cache.device)))


def cache_write_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                    v_scale: float) -> None:
    """Quantizing scatter of f32/f16/bf16 k/v [T][Hkv][d] into E4M3 caches
    (torch.float8_e4m3fn): element x is stored as e4m3(x / scale)."""
    _require(k.dim() == 3 and v.dim() == 3 and k.shape == v.shape, "k, v must be [T][Hkv][d]")
    T, H, d = k.shape
    NB, H2, bs, d2 = _cache_dims(k_cache, v_cache)
    _require((H2, d2) == (H, d), "cache shapes do not match k/v")
    for t in (k, v):
        _require(t.stride(2) == 1 and t.stride(1) == d, "heads of a token must be packed")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (T,)
             and slot_mapping.is_contiguous(), "slot_mapping must be contiguous int64 [T]")
    _require(k.dtype == v.dtype and k_cache.dtype == v_cache.dtype == torch.float8_e4m3fn,
             "E4M3 caches and k, v of one dtype")
    _check(lib().pa_cache_write_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                    k_cache.data_ptr(), v_cache.data_ptr(), T, k.stride(0),
                                    v.stride(0), H, d, NB, bs, _dt(k), float(k_scale),
                                    float(v_scale), _stream(k_cache.device)))


def advance_step(num_queries: int, block_size: int, input_tokens: torch.Tensor,
                 sampled_token_ids: torch.Tensor, input_positions: torch.Tensor,
                 seq_lens: torch.Tensor, slot_mapping: torch.Tensor,
                 block_tables: torch.Tensor) -> None:
    """Advance every sequence's decode state one step on the device (in place)."""
    B = input_tokens.shape[0]
    for t, dt in ((input_tokens, torch.int64), (input_positions, torch.int64),
                  (slot_mapping, torch.int64), (seq_lens, torch.int32)):
        _require(t.dtype == dt and t.shape == (B,) and t.is_contiguous(),
                 "state tensors: int64/int32 [num_seqs], contiguous")
    _require(sampled_token_ids.dtype == torch.int64 and sampled_token_ids.is_contiguous()
             and sampled_token_ids.numel() >= num_queries, "sampled_token_ids: int64 [num_queries]")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(),
             "block_tables must be contiguous int32 [num_seqs][max_blocks]")
    _check(lib().pa_advance_step(B, num_queries, block_size, input_tokens.data_ptr(),
                                 sampled_token_ids.data_ptr(), input_positions.data_ptr(),
                                 seq_lens.data_ptr(), slot_mapping.data_ptr(),
                                 block_tables.data_ptr(), block_tables.shape[1],
                                 _stream(input_tokens.device)))


def decode_partition_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          block_size: int, max_blocks_per_seq: int, kv_dtype: torch.dtype,
                          flags: int = AUTO) -> int:
    p = lib().pa_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, _DTYPE[kv_dtype], flags)
    _check(min(p, 0))
    return p


def decode_kernel(num_q_heads: int, num_kv_heads: int, q_dtype: torch.dtype,
                  kv_dtype: torch.dtype, flags: int = AUTO) -> str:
    """Which decode kernel family runs for these arguments: "valu" or "mfma"."""
    k = lib().pa_decode_kernel(num_q_heads, num_kv_heads, _DTYPE[q_dtype], _DTYPE[kv_dtype], flags)
    _check(min(k, 0))
    return {FORCE_VALU: "valu", FORCE_MFMA: "mfma"}[k]


def decode_waves(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, max_blocks_per_seq: int, partition_size: int,
                 q_dtype: torch.dtype, kv_dtype: torch.dtype, flags: int = AUTO) -> int:
    """Waves per (sequence, kv head, partition) work item that decode uses."""
    w = lib().pa_decode_waves(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                              max_blocks_per_seq, partition_size, _DTYPE[q_dtype],
                              _DTYPE[kv_dtype], flags)
    _check(min(w, 0))
    return w


def decode_work_list(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     block_size: int, max_blocks_per_seq: int, partition_size: int,
                     q_dtype: torch.dtype, kv_dtype: torch.dtype, flags: int = AUTO) -> bool:
    """Whether decode runs a persistent grid over the items that hold tokens."""
    r = lib().pa_decode_work_list(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                  max_blocks_per_seq, partition_size, _DTYPE[q_dtype],
                                  _DTYPE[kv_dtype], flags)
    _check(min(r, 0))
    return bool(r)


def decode_grid(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, max_blocks_per_seq: int, partition_size: int,
                q_dtype: torch.dtype, kv_dtype: torch.dtype, flags: int = AUTO) -> str:
    """The grid decode runs: "grid" (grid order), "sorted" or "work_list"."""
    r = lib().pa_decode_grid(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_size, _DTYPE[q_dtype],
                             _DTYPE[kv_dtype], flags)
    _check(min(r, 0))
    return GRID_NAMES[r]


def decode_partition_used(workspace: torch.Tensor, num_seqs: int, num_q_heads: int,
                          num_kv_heads: int, head_dim: int, block_size: int,
                          max_blocks_per_seq: int, kv_dtype: torch.dtype, flags: int = AUTO) -> int:
    """The partition the last partition_size = 0 decode on this workspace used
    (the device's refinement where there is one; waits for the stream)."""
    r = lib().pa_decode_partition_used(workspace.data_ptr(), workspace.nbytes, num_seqs,
                                       num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, _DTYPE[kv_dtype], flags,
                                       _stream(workspace.device))
    _check(min(r, 0))
    return r


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          block_size: int, max_blocks_per_seq: int, partition_size: int,
                          kv_dtype: torch.dtype, flags: int = AUTO) -> int:
    return lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          block_size, max_blocks_per_seq, partition_size,
                                          _DTYPE[kv_dtype], flags)


def _decode_call(fn_name, out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                 partition_size, workspace, flags, kv_scales=None):
    B, Hq, d, NB, Hkv, bs, MB = _decode_dims(out, q, k_cache, v_cache, block_tables,
                                             context_lens, block_size)
    if workspace is None and fn_name in ("pa_decode", "pa_decode_fp8"):
        # the one-call forms without a workspace: the binding allocates it (the
        # library checks every workspace it is given against the size it needs)
        need = decode_workspace_size(B, Hq, Hkv, d, bs, MB, partition_size, k_cache.dtype,
                                     flags)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    fn = getattr(_lib or lib(), fn_name)
    if kv_scales is not None:
        _check(fn(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                  block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
                  float(kv_scales[0]), float(kv_scales[1]), block_size, partition_size, B, Hq,
                  Hkv, d, NB, MB, _dt(q), _dt(out), ws_ptr, ws_bytes, flags, _stream(q.device)))
        return
    _check(fn(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
              block_tables.data_ptr(), context_lens.data_ptr(), float(scale), block_size,
              partition_size, B, Hq, Hkv, d, NB, MB, _dt(q), _dt(k_cache), _dt(out), ws_ptr,
              ws_bytes, flags, _stream(q.device)))


def decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
           block_size: int, partition_size: int = 0, workspace: torch.Tensor | None = None,
           flags: int = AUTO) -> None:
    """out[b][hq] = softmax(scale * q[b][hq] . K^T) V over the paged context of b.
    Allocates the workspace with torch when none (or too small a one) is given."""
    _decode_call("pa_decode", out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 block_size, partition_size, workspace, flags)


# bits of the status word pa_check_tables / pa_check_slots set
CHECK_CONTEXT_LEN, CHECK_BLOCK_ID, CHECK_SLOT = 1, 2, 4


def check_tables(block_tables: torch.Tensor, context_lens: torch.Tensor, num_blocks: int,
                 block_size: int, status: torch.Tensor) -> None:
    """OR CHECK_CONTEXT_LEN / CHECK_BLOCK_ID into status (a device int32 [1])
    where decode would cut a context length or clamp a block id."""
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.is_contiguous(), "block_tables must be contiguous int32 [B][MB]")
    B, MB = block_tables.shape
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (B,)
             and context_lens.is_contiguous(), "context_lens must be contiguous int32 [B]")
    _require(status.dtype == torch.int32 and status.numel() == 1 and status.is_cuda,
             "status must be a device int32 [1]")
    _check(lib().pa_check_tables(block_tables.data_ptr(), context_lens.data_ptr(), B, MB,
                                 block_size, num_blocks, status.data_ptr(),
                                 _stream(status.device)))


def check_slots(slot_mapping: torch.Tensor, num_blocks: int, block_size: int,
                status: torch.Tensor) -> None:
    """OR CHECK_SLOT into status (a device int32 [1]) where cache_write would
    drop a slot past the pool."""
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
             and slot_mapping.is_contiguous(), "slot_mapping must be contiguous int64 [T]")
    _require(status.dtype == torch.int32 and status.numel() == 1 and status.is_cuda,
             "status must be a device int32 [1]")
    _check(lib().pa_check_slots(slot_mapping.data_ptr(), slot_mapping.shape[0], num_blocks,
                                block_size, status.data_ptr(), _stream(status.device)))


# bytes of the library's static scratch behind decode_noalloc (PA_SCRATCH_BYTES)
SCRATCH_BYTES = 64 << 20


def decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, block_tables: torch.Tensor,
                   context_lens: torch.Tensor, scale: float, block_size: int,
                   partition_size: int = 0, flags: int = AUTO) -> None:
    """decode() with the library's static device scratch as its workspace:
    nothing is allocated, by the library or here (for callers that cannot
    allocate).  Raises PAError -9 when the workspace decode() would need
    exceeds SCRATCH_BYTES.  Calls that overlap on one GPU share the scratch
    and race."""
    _require(q.dim() == 3 and q.is_contiguous(), "q must be contiguous [B][Hq][d]")
    B, Hq, d = q.shape
    _require(out.shape == q.shape and out.is_contiguous(), "out must be contiguous [B][Hq][d]")
    NB, Hkv, bs, d2 = _cache_dims(k_cache, v_cache)
    _require(bs == block_size and d2 == d, "cache shapes do not match block_size / head_dim")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(),
             "block_tables must be contiguous int32 [B][max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (B,)
             and context_lens.is_contiguous(), "context_lens must be contiguous int32 [B]")
    _check(lib().pa_decode_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), block_size,
        partition_size, B, Hq, Hkv, d, NB, block_tables.shape[1], _dt(q), _dt(k_cache), _dt(out),
        flags, _stream(q.device)))


def decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                      partition_size=0, workspace=None, flags=AUTO) -> None:
    """Phase 1 of decode (attention per partition); needs the caller's workspace."""
    _decode_call("pa_decode_partitions", out, q, k_cache, v_cache, block_tables, context_lens,
                 scale, block_size, partition_size, workspace, flags)


def decode_merge(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                 partition_size=0, workspace=None, flags=AUTO) -> None:
    """Phase 2 of decode (log-sum-exp merge of the partitions)."""
    _decode_call("pa_decode_merge", out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 block_size, partition_size, workspace, flags)


def decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
               block_size, partition_size=0, workspace=None, flags=AUTO) -> None:
    """decode over E4M3 caches written with the scales k_scale / v_scale."""
    _require(k_cache.dtype == torch.float8_e4m3fn, "decode_fp8 needs E4M3 caches")
    _decode_call("pa_decode_fp8", out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 block_size, partition_size, workspace, flags, (k_scale, v_scale))


def decode_fp8_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                          v_scale, block_size, partition_size=0, workspace=None,
                          flags=AUTO) -> None:
    """Phase 1 of decode_fp8; decode_merge is phase 2 for every cache type."""
    _require(k_cache.dtype == torch.float8_e4m3fn, "decode_fp8 needs E4M3 caches")
    _decode_call("pa_decode_fp8_partitions", out, q, k_cache, v_cache, block_tables, context_lens,
                 scale, block_size, partition_size, workspace, flags, (k_scale, v_scale))


def _decode_step_call(fn_name, k, v, slot_mapping, out, q, k_cache, v_cache, block_tables,
                      context_lens, scale, block_size, partition_size, workspace, flags):
    B, Hq, d, NB, Hkv, bs, MB = _decode_dims(out, q, k_cache, v_cache, block_tables,
                                             context_lens, block_size)
    kshape = k.shape
    if len(kshape) != 3 or v.shape != kshape or kshape[1] != Hkv or kshape[2] != d:
        raise PAError(-2, "k, v must be [T][Hkv][d] matching the caches")
    T = kshape[0]
    if k.stride(2) != 1 or k.stride(1) != d or v.stride(2) != 1 or v.stride(1) != d:
        raise PAError(-2, "heads of a token must be packed")
    if (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,)
            or not slot_mapping.is_contiguous()):
        raise PAError(-2, "slot_mapping must be contiguous int64 [T]")
    if not (k.dtype == v.dtype == k_cache.dtype == v_cache.dtype):
        raise PAError(-2, "dtype mismatch")
    if workspace is None and fn_name == "pa_decode_step":
        need = decode_workspace_size(B, Hq, Hkv, d, bs, MB, partition_size, k_cache.dtype,
                                     flags)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _check(getattr(_lib or lib(), fn_name)(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), T, k.stride(0), v.stride(0),
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), block_size,
        partition_size, B, Hq, Hkv, d, NB, MB, _dt(q), _dt(k_cache), _dt(out), ws_ptr, ws_bytes,
        flags, _stream(q.device)))


def decode_step(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables, context_lens,
                scale, block_size, partition_size=0, workspace=None, flags=AUTO) -> None:
    """cache_write(k, v, slot_mapping, ...) then decode(out, q, ...) in as few launches as
    the grid allows (the write shares the launch that orders the decode's items)."""
    _decode_step_call("pa_decode_step", k, v, slot_mapping, out, q, k_cache, v_cache,
                      block_tables, context_lens, scale, block_size, partition_size, workspace,
                      flags)


def decode_order(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                 partition_size=0, workspace=None, flags=AUTO, k=None, v=None,
                 slot_mapping=None) -> None:
    """The launch before the decode kernel: the step's cache write of k, v at
    slot_mapping (when given) and, on the sorted grid, the item ordering into the
    workspace.  decode_partitions / decode (or the E4M3 forms) with the same
    arguments and flags | ORDERED then launch the decode kernel alone."""
    if k is not None:
        _decode_step_call("pa_decode_order", k, v, slot_mapping, out, q, k_cache, v_cache,
                          block_tables, context_lens, scale, block_size, partition_size,
                          workspace, flags)
        return
    B, Hq, d, NB, Hkv, bs, MB = _decode_dims(out, q, k_cache, v_cache, block_tables,
                                             context_lens, block_size)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode_order(
        None, None, None, 0, Hkv * d, Hkv * d, out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
        block_size, partition_size, B, Hq, Hkv, d, NB, MB, _dt(q), _dt(k_cache), _dt(out),
        ws_ptr, ws_bytes, flags, _stream(q.device)))


def decode_order_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                     v_scale, block_size, partition_size, workspace, flags, k, v,
                     slot_mapping) -> None:
    """decode_order for E4M3 caches: the quantizing write of k, v (f32 / f16 /
    bf16 rows) at slot_mapping with the caches' scales, and the item ordering,
    in one launch; decode_fp8_partitions with flags | ORDERED then launches the
    decode kernel alone."""
    B, Hq, d, NB, Hkv, bs, MB = _decode_dims(out, q, k_cache, v_cache, block_tables,
                                             context_lens, block_size)
    kshape = k.shape
    if len(kshape) != 3 or v.shape != kshape or kshape[1] != Hkv or kshape[2] != d:
        raise PAError(-2, "k, v must be [T][Hkv][d] matching the caches")
    T = kshape[0]
    if k.stride(2) != 1 or k.stride(1) != d or v.stride(2) != 1 or v.stride(1) != d:
        raise PAError(-2, "heads of a token must be packed")
    if (slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,)
            or not slot_mapping.is_contiguous()):
        raise PAError(-2, "slot_mapping must be contiguous int64 [T]")
    if k.dtype != v.dtype:
        raise PAError(-2, "dtype mismatch")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.nbytes if workspace is not None else 0
    _check((_lib or lib()).pa_decode_order_fp8(
        k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), T, k.stride(0), v.stride(0), _dt(k),
        float(k_scale), float(v_scale), out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
        block_size, partition_size, B, Hq, Hkv, d, NB, MB, _dt(q), _dt(out), ws_ptr, ws_bytes,
        flags, _stream(q.device)))


def decode_step_partitions(k, v, slot_mapping, out, q, k_cache, v_cache, block_tables,
                           context_lens, scale, block_size, partition_size=0, workspace=None,
                           flags=AUTO) -> None:
    """decode_step without the merge phase (decode_merge completes it)."""
    _decode_step_call("pa_decode_step_partitions", k, v, slot_mapping, out, q, k_cache, v_cache,
                      block_tables, context_lens, scale, block_size, partition_size, workspace,
                      flags)


def decode_mq_kernel(num_queries: int, num_q_heads: int, num_kv_heads: int,
                     q_dtype: torch.dtype, kv_dtype: torch.dtype, flags: int = AUTO) -> str:
    """Kernel family of a decode with num_queries query tokens per sequence."""
    k = lib().pa_decode_mq_kernel(num_queries, num_q_heads, num_kv_heads, _DTYPE[q_dtype],
                                  _DTYPE[kv_dtype], flags)
    _check(min(k, 0))
    return {FORCE_VALU: "valu", FORCE_MFMA: "mfma"}[k]


def _decode_mq_call(fn_name, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                    block_size, partition_size, workspace, flags, k_scale, v_scale):
    _require(q.dim() == 4 and q.is_contiguous(), "q must be contiguous [B][Q][Hq][d]")
    B, Q, Hq, d = q.shape
    _require(out.shape == q.shape and out.is_contiguous(), "out must be contiguous [B][Q][Hq][d]")
    NB, Hkv, bs, d2 = _cache_dims(k_cache, v_cache)
    _require(bs == block_size and d2 == d, "cache shapes do not match block_size / head_dim")
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2
             and block_tables.shape[0] == B and block_tables.is_contiguous(),
             "block_tables must be contiguous int32 [B][max_blocks]")
    _require(context_lens.dtype == torch.int32 and context_lens.shape == (B,)
             and context_lens.is_contiguous(), "context_lens must be contiguous int32 [B]")
    MB = block_tables.shape[1]
    if workspace is None and fn_name == "pa_decode_mq":
        need = decode_workspace_size(B * Q, Hq, Hkv, d, bs, MB, partition_size, k_cache.dtype,
                                     flags)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(lib(), fn_name)(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), float(k_scale),
        float(v_scale), block_size, partition_size, B, Q, Hq, Hkv, d, NB, MB, _dt(q),
        _dt(k_cache), _dt(out), ws_ptr, ws_bytes, flags, _stream(q.device)))


def decode_mq(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
              partition_size=0, workspace=None, flags=AUTO, k_scale=1.0, v_scale=1.0) -> None:
    """Decode of Q query tokens per sequence (q, out: [B][Q][Hq][d]): query i of sequence b
    sits at position context_lens[b] - Q + i and attends causally up to it."""
    _decode_mq_call("pa_decode_mq", out, q, k_cache, v_cache, block_tables, context_lens, scale,
                    block_size, partition_size, workspace, flags, k_scale, v_scale)


def decode_mq_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                         block_size, partition_size=0, workspace=None, flags=AUTO,
                         k_scale=1.0, v_scale=1.0) -> None:
    _decode_mq_call("pa_decode_mq_partitions", out, q, k_cache, v_cache, block_tables,
                    context_lens, scale, block_size, partition_size, workspace, flags, k_scale,
                    v_scale)


def decode_mq_merge(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                    partition_size=0, workspace=None, flags=AUTO) -> None:
    _decode_mq_call("pa_decode_mq_merge", out, q, k_cache, v_cache, block_tables, context_lens,
                    scale, block_size, partition_size, workspace, flags, 1.0, 1.0)


# ---------------------------------------------------------------- block management
# (include/pa_blocks.h: a host-side block manager and the device block copies)

PREFIX_CACHING = 1


def _np():
    import numpy
    return numpy


def _host_ptr(a) -> int:
    return a.ctypes.data


class BlockManager:
    """Host-side allocator of a paged cache's physical blocks (libpa.so): free list,
    reference-counted sharing with copy-on-write, prefix caching and host swap."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0,
                 prefix_caching: bool = False):
        h = ctypes.c_void_p()
        _check(lib().pa_bm_create(num_blocks, block_size, num_host_blocks,
                                  PREFIX_CACHING if prefix_caching else 0, ctypes.byref(h)))
        self._h = h
        self.block_size = block_size
        self.prefix_caching = prefix_caching

    def close(self) -> None:
        if self._h is not None and self._h.value:
            lib().pa_bm_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _ids(self, tokens, n):
        np = _np()
        if tokens is None:
            return None, None
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _require(t.shape == (n,), "tokens must hold one id per token")
        return t, _host_ptr(t)

    def add_sequence(self, seq_id: int, tokens=None, num_tokens: int | None = None) -> int:
        """New sequence; returns the number of leading tokens served by cached blocks."""
        n = len(tokens) if num_tokens is None else num_tokens
        t, tp = self._ids(tokens, n)
        cached = ctypes.c_int32(0)
        _check(lib().pa_bm_add_sequence(self._h, seq_id, tp, n, ctypes.byref(cached)))
        return cached.value

    def append(self, seq_ids, tokens=None):
        """One token per sequence: (slots int64 [n], copy-on-write pairs int32 [k][2])."""
        np = _np()
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        t, tp = self._ids(tokens, n)
        slots = np.empty(n, np.int64)
        copies = np.empty((max(n, 1), 2), np.int32)
        nc = ctypes.c_int32(0)
        _check(lib().pa_bm_append(self._h, _host_ptr(ids), tp, n, _host_ptr(slots),
                                  _host_ptr(copies), ctypes.byref(nc)))
        return slots, copies[: nc.value].copy()

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pa_bm_fork(self._h, parent, child))

    def free(self, seq_id: int) -> None:
        _check(lib().pa_bm_free(self._h, seq_id))

    def mark_computed(self, seq_id: int) -> None:
        _check(lib().pa_bm_mark_computed(self._h, seq_id))

    def slots(self, seq_id: int, start: int, n: int):
        np = _np()
        out = np.empty(n, np.int64)
        _check(lib().pa_bm_slots(self._h, seq_id, start, n, _host_ptr(out) if n else None))
        return out

    def block_tables(self, seq_ids, max_blocks_per_seq: int):
        """(block_tables int32 [n][max_blocks_per_seq] (-1 padded), context_lens int32 [n])."""
        np = _np()
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        bt = np.empty((n, max_blocks_per_seq), np.int32)
        lens = np.empty(n, np.int32)
        _check(lib().pa_bm_block_tables(self._h, _host_ptr(ids), n, max_blocks_per_seq,
                                        _host_ptr(bt), _host_ptr(lens)))
        return bt, lens

    def _swap(self, fn, seq_id: int):
        np = _np()
        length, _ = self.seq_info(seq_id)
        pairs = np.empty((max(1, -(-length // self.block_size)), 2), np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, seq_id, _host_ptr(pairs), ctypes.byref(n)))
        return pairs[: n.value].copy()

    def swap_out(self, seq_id: int):
        """(device block, host block) pairs to copy out."""
        return self._swap(lib().pa_bm_swap_out, seq_id)

    def swap_in(self, seq_id: int):
        """(host block, device block) pairs to copy in."""
        return self._swap(lib().pa_bm_swap_in, seq_id)

    @property
    def num_free_blocks(self) -> int:
        v = ctypes.c_int64(0)
        _check(lib().pa_bm_num_free_blocks(self._h, ctypes.byref(v)))
        return v.value

    @property
    def num_free_host_blocks(self) -> int:
        v = ctypes.c_int64(0)
        _check(lib().pa_bm_num_free_host_blocks(self._h, ctypes.byref(v)))
        return v.value

    def seq_info(self, seq_id: int):
        """(length, resident)."""
        n, r = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pa_bm_seq_info(self._h, seq_id, ctypes.byref(n), ctypes.byref(r)))
        return n.value, bool(r.value)

    def ref_count(self, block: int) -> int:
        v = ctypes.c_int32(0)
        _check(lib().pa_bm_ref_count(self._h, block, ctypes.byref(v)))
        return v.value


def _block_bytes(cache: torch.Tensor) -> int:
    return cache[0].numel() * cache.element_size()


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, pairs: torch.Tensor) -> None:
    """Copy-on-write on the device: block src -> dst of both caches for each row of pairs
    (a device int32 tensor [n][2])."""
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    _require(k_cache.shape[0] == v_cache.shape[0] and _block_bytes(k_cache) ==
             _block_bytes(v_cache), "caches must hold blocks of the same size")
    _require(pairs.dtype == torch.int32 and pairs.is_contiguous() and pairs.dim() == 2
             and pairs.shape[1] == 2 and pairs.device == k_cache.device,
             "pairs must be a contiguous int32 [n][2] tensor on the caches' device")
    _check(lib().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(),
                                pairs.shape[0], k_cache.shape[0], _block_bytes(k_cache),
                                _stream(k_cache.device)))


def swap_blocks(dst_pool: torch.Tensor, src_pool: torch.Tensor, pairs) -> None:
    """Block copies between a device cache and a pinned host pool of the same block layout
    (pairs: host int32 [n][2] of (src block, dst block)), on the device's current stream."""
    np = _np()
    _require(dst_pool.is_contiguous() and src_pool.is_contiguous(), "pools must be contiguous")
    _require(_block_bytes(dst_pool) == _block_bytes(src_pool) and dst_pool.dtype ==
             src_pool.dtype, "pools must hold blocks of the same layout")
    p = np.ascontiguousarray(pairs, dtype=np.int32)
    _require(p.ndim == 2 and p.shape[1] == 2, "pairs must be [n][2]")
    _require(bool((p[:, 0] < src_pool.shape[0]).all() and (p[:, 1] < dst_pool.shape[0]).all()),
             "block ids past the pools")
    dev = dst_pool.device if dst_pool.is_cuda else src_pool.device
    _require(dev.type == "cuda" and (dst_pool.is_pinned() or src_pool.is_pinned()),
             "one pool must be a device cache, the other pinned host memory")
    _check(lib().pa_swap_blocks(dst_pool.data_ptr(), src_pool.data_ptr(),
                                _host_ptr(p) if p.shape[0] else None, p.shape[0],
                                _block_bytes(dst_pool), _stream(dev)))
