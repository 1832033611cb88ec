"""fp64 CPU oracle for the paged KV-cache write and paged decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and
its Python binding) never imports this package.

The arithmetic lives in ``pa_oracle.c`` (plain C, double precision); this
module only builds it with gcc and marshals numpy arrays to it.  See the
header of ``pa_oracle.c`` for the passages each function follows and for the
pins that check it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16, FP8 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "fp8": FP8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}

ERRORS = {
    -1: "bad argument",
    -2: "slot out of range",
    -3: "block id out of range",
    -4: "context length out of range",
    -5: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into liboracle.so with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC,
               "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        c_void_p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.orc_cache_write.restype = ctypes.c_int
        L.orc_cache_write.argtypes = [c_void_p, c_void_p, c_void_p, i64, i64, i64, c_void_p,
                                      c_void_p, i32, i32, i64, i32, i32]
        L.orc_decode.restype = ctypes.c_int
        f32 = ctypes.c_float
        L.orc_decode.argtypes = [c_void_p, c_void_p, i32, c_void_p, c_void_p, i32, c_void_p,
                                 c_void_p, i32, i32, i32, i32, i64, i32, i32, f32, f32, f32,
                                 c_void_p, i64, i32]
        L.orc_decode_mq.restype = ctypes.c_int
        L.orc_decode_mq.argtypes = [c_void_p, c_void_p, i32, c_void_p, c_void_p, i32, c_void_p,
                                    c_void_p, i32, i32, i32, i32, i32, i64, i32, i32, f32, f32,
                                    f32, c_void_p, i64, i32]
        L.orc_cache_write_fp8.restype = ctypes.c_int
        L.orc_cache_write_fp8.argtypes = [c_void_p, c_void_p, c_void_p, i64, i64, i64, c_void_p,
                                          c_void_p, i32, i32, i64, i32, i32, f32, f32]
        L.orc_encode_fp8.restype = None
        L.orc_encode_fp8.argtypes = [c_void_p, i64, c_void_p]
        L.orc_advance_step.restype = ctypes.c_int
        L.orc_advance_step.argtypes = [i32, i32, i32, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, i32]
        L.orc_decode_bits.restype = None
        L.orc_decode_bits.argtypes = [c_void_p, i32, i64, c_void_p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(st: int) -> None:
    if st != 0:
        raise OracleError(f"oracle error {st}: {ERRORS.get(st, 'unknown')}")


def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
    """View an array holding the raw bits of `dtype` elements (uint16 for the
    16-bit types, float32/uint32 for f32) as a C-contiguous buffer."""
    a = np.ascontiguousarray(a)
    want = ELEM_BYTES[dtype]
    if a.dtype.itemsize != want:
        raise OracleError(f"array itemsize {a.dtype.itemsize} does not match dtype {dtype}")
    return a


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw element bits (uint8 for fp8, uint16 for f16/bf16, uint32 for f32)
    to float64."""
    bits = _raw(bits, dtype)
    out = np.empty(bits.size, dtype=np.float64)
    lib().orc_decode_bits(_ptr(bits), DTYPE_CODES[dtype], bits.size, _ptr(out))
    return out.reshape(bits.shape)


def cache_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray,
                v_cache: np.ndarray, dtype: str) -> None:
    """In-place ORC-W on host arrays of raw bits.

    k, v: [T][Hkv][d] (or [T][Hkv*d]); k_cache: [NB][Hkv][bs/4][d/X][4][X] with
    X = 16 / element bytes; v_cache: [NB][Hkv][bs/4][d][4]; slot_mapping: int64 [T]."""
    k = _raw(k, dtype)
    v = _raw(v, dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise OracleError("caches must be C-contiguous")
    NB, Hkv, nq, dx, four, X = k_cache.shape
    d, bs = dx * X, nq * 4
    if X != 16 // (4 if dtype == "f32" else 2) or four != 4:
        raise OracleError(f"k_cache shape {k_cache.shape} is not the quad layout of {dtype}")
    if v_cache.shape != (NB, Hkv, nq, d, 4):
        raise OracleError(f"v_cache shape {v_cache.shape} != {(NB, Hkv, nq, d, 4)}")
    T = slots.shape[0]
    if k.size != T * Hkv * d or v.size != T * Hkv * d:
        raise OracleError("k/v size does not match slot_mapping")
    _check(lib().orc_cache_write(_ptr(k), _ptr(v), _ptr(slots), T, Hkv * d, Hkv * d,
                                 _ptr(k_cache), _ptr(v_cache), Hkv, d, NB, bs,
                                 DTYPE_CODES[dtype]))


def encode_fp8(y: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 bit patterns (uint8): nearest, ties even, saturating."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().orc_encode_fp8(_ptr(y), y.size, _ptr(out))
    return out


def cache_write_fp8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                    k_cache: np.ndarray, v_cache: np.ndarray, src_dtype: str, k_scale: float,
                    v_scale: float) -> None:
    """In-place quantizing write into E4M3 caches (uint8 arrays):
    k_cache [NB][Hkv][bs/4][d/16][4][16], v_cache [NB][Hkv][bs/4][d][4]."""
    k = _raw(k, src_dtype)
    v = _raw(v, src_dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    if k_cache.dtype != np.uint8 or v_cache.dtype != np.uint8:
        raise OracleError("E4M3 caches are uint8 arrays")
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise OracleError("caches must be C-contiguous")
    NB, Hkv, nq, dx, four, X = k_cache.shape
    d, bs = dx * X, nq * 4
    if X != 16 or four != 4 or v_cache.shape != (NB, Hkv, nq, d, 4):
        raise OracleError("cache shapes are not the E4M3 quad layout")
    T = slots.shape[0]
    if k.size != T * Hkv * d or v.size != T * Hkv * d:
        raise OracleError("k/v size does not match slot_mapping")
    _check(lib().orc_cache_write_fp8(_ptr(k), _ptr(v), _ptr(slots), T, Hkv * d, Hkv * d,
                                     _ptr(k_cache), _ptr(v_cache), Hkv, d, NB, bs,
                                     DTYPE_CODES[src_dtype], float(k_scale), float(v_scale)))


def decode(q: np.ndarray, q_dtype: str, k_cache: np.ndarray, v_cache: np.ndarray,
           kv_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           rows: np.ndarray | None = None, threads: int = 1, k_scale: float = 1.0,
           v_scale: float = 1.0) -> np.ndarray:
    """ORC-D: float64 [B][Hq][d] attention output (rows not requested stay NaN).
    Cache elements are the stored values times k_scale / v_scale."""
    q = _raw(q, q_dtype)
    B, Hq, d = q.shape
    NB, Hkv, nq, dx, four, X = k_cache.shape
    bs = nq * 4
    if dx * X != d or four != 4 or v_cache.shape != (NB, Hkv, nq, d, 4):
        raise OracleError("cache shapes do not match q")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.shape[0] != B or cl.shape != (B,):
        raise OracleError("block_tables/context_lens do not match batch")
    MB = bt.shape[1]
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    _check(lib().orc_decode(_ptr(out), _ptr(q), DTYPE_CODES[q_dtype], _ptr(k_cache),
                            _ptr(v_cache), DTYPE_CODES[kv_dtype], _ptr(bt), _ptr(cl), B, Hq, Hkv,
                            d, NB, bs, MB, float(scale), float(k_scale), float(v_scale),
                            None if r is None else _ptr(r),
                            0 if r is None else r.size, int(threads)))
    return out


def decode_mq(q: np.ndarray, q_dtype: str, k_cache: np.ndarray, v_cache: np.ndarray,
              kv_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
              rows: np.ndarray | None = None, threads: int = 1, k_scale: float = 1.0,
              v_scale: float = 1.0) -> np.ndarray:
    """Multi-query decode: q [B][Q][Hq][d]; query i of sequence b sits at position
    context_lens[b] - Q + i and attends to positions 0 .. its own.  float64
    [B][Q][Hq][d] (rows = (b*Q + i)*Hq + hq not requested stay NaN)."""
    q = _raw(q, q_dtype)
    B, Q, Hq, d = q.shape
    NB, Hkv, nq, dx, four, X = k_cache.shape
    bs = nq * 4
    if dx * X != d or four != 4 or v_cache.shape != (NB, Hkv, nq, d, 4):
        raise OracleError("cache shapes do not match q")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.shape[0] != B or cl.shape != (B,):
        raise OracleError("block_tables/context_lens do not match batch")
    out = np.full((B, Q, Hq, d), np.nan, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    _check(lib().orc_decode_mq(_ptr(out), _ptr(q), DTYPE_CODES[q_dtype], _ptr(k_cache),
                               _ptr(v_cache), DTYPE_CODES[kv_dtype], _ptr(bt), _ptr(cl), B, Q, Hq,
                               Hkv, d, NB, bs, bt.shape[1], float(scale), float(k_scale),
                               float(v_scale), None if r is None else _ptr(r),
                               0 if r is None else r.size, int(threads)))
    return out


def advance_step(num_queries: int, block_size: int, input_tokens: np.ndarray,
                 sampled_token_ids: np.ndarray, input_positions: np.ndarray,
                 seq_lens: np.ndarray, slot_mapping: np.ndarray,
                 block_tables: np.ndarray) -> None:
    """In-place advance of host state arrays (int64 tokens/positions/slots,
    int32 lengths, int32 [B][MB] tables)."""
    arrs = [(input_tokens, np.int64), (input_positions, np.int64), (seq_lens, np.int32),
            (slot_mapping, np.int64)]
    for a, dt in arrs:
        if a.dtype != dt or not a.flags.c_contiguous:
            raise OracleError("state arrays must be contiguous int64 (int32 for seq_lens)")
    B = input_tokens.shape[0]
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sampled = np.ascontiguousarray(sampled_token_ids, dtype=np.int64)
    _check(lib().orc_advance_step(B, num_queries, block_size, _ptr(input_tokens), _ptr(sampled),
                                  _ptr(input_positions), _ptr(seq_lens), _ptr(slot_mapping),
                                  _ptr(bt), bt.shape[1]))
