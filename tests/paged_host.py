"""Host-side helpers for the tests: the oracle's view of a seeded workload.

Builds the oracle's own paged caches (numpy raw bits, NaN-poisoned) from the
same seeded inputs the GPU receives, and the contiguous float64 copies of each
sequence's K/V that the brute-force pin uses.  Nothing here reads GPU results.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from pagedattention_kv_cache_amd.workloads import POISON_BITS, Workload, raw_bits

_BITS_NP = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def key_chunk(dtype: str) -> int:
    """X: elements per 16-byte chunk of the key layout."""
    return {"f32": 4, "f16": 8, "bf16": 8, "fp8": 16}[dtype]


def key_pool_shape(NB: int, H: int, d: int, bs: int, dtype: str) -> tuple:
    X = key_chunk(dtype)
    return (NB, H, bs // 4, d // X, 4, X)


def value_pool_shape(NB: int, H: int, d: int, bs: int) -> tuple:
    return (NB, H, bs // 4, d, 4)


def poisoned_pool(wl: Workload, transposed: bool) -> np.ndarray:
    """Value pool [NB][Hkv][bs/4][d][4] (transposed=True) or key pool
    [NB][Hkv][bs/4][d/X][4][X], filled with the dtype's quiet NaN."""
    c = wl.cfg
    shape = (value_pool_shape(wl.num_blocks, c.num_kv_heads, c.head_dim, c.block_size)
             if transposed else
             key_pool_shape(wl.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.kv_dtype))
    return np.full(shape, POISON_BITS[c.kv_dtype], dtype=_BITS_NP[c.kv_dtype])


def abs_values(pool: np.ndarray, dtype: str) -> np.ndarray:
    """A raw-bit pool with every element's sign bit cleared (|x|; NaN stays NaN)."""
    top = {"f32": 0x80000000, "f16": 0x8000, "bf16": 0x8000, "fp8": 0x80}[dtype]
    return pool & pool.dtype.type(~top & (2 * top - 1))


def oracle_write(cfg, k: np.ndarray, v: np.ndarray, slots: np.ndarray, kc: np.ndarray,
                 vc: np.ndarray) -> None:
    """The oracle's cache write for the config's cache dtype (k, v raw bits)."""
    if cfg.kv_dtype == "fp8":
        oracle.cache_write_fp8(k, v, slots, kc, vc, cfg.dtype, *cfg.fp8_scales)
    else:
        oracle.cache_write(k, v, slots, kc, vc, cfg.dtype)


def oracle_decode(cfg, q: np.ndarray, kc: np.ndarray, vc: np.ndarray, block_tables, lens,
                  rows=None, threads: int = 8) -> np.ndarray:
    ks, vs = cfg.fp8_scales if cfg.kv_dtype == "fp8" else (1.0, 1.0)
    return oracle.decode(q, cfg.dtype, kc, vc, cfg.kv_dtype, block_tables, lens,
                         cfg.attn_scale(), rows=rows, threads=threads, k_scale=ks, v_scale=vs)


def key_rows(kc: np.ndarray, blk: int, off: int) -> np.ndarray:
    """The [Hkv][d] key rows of the token at (block, offset) of a key pool."""
    return kc[blk, :, off // 4, :, off % 4, :].reshape(kc.shape[1], -1)


def value_rows(vc: np.ndarray, blk: int, off: int) -> np.ndarray:
    """The [Hkv][d] value rows of the token at (block, offset) of a value pool."""
    return vc[blk, :, off // 4, :, off % 4]


def offset_major(pool: np.ndarray, key: bool) -> np.ndarray:
    """A pool viewed as [block][offset][...] (for per-slot comparisons)."""
    if key:  # [NB][H][bs/4][d/X][4][X] -> [NB][bs/4][4][H][d/X][X] -> [NB][bs][...]
        t = pool.transpose(0, 2, 4, 1, 3, 5)
    else:    # [NB][H][bs/4][d][4] -> [NB][bs/4][4][H][d]
        t = pool.transpose(0, 2, 4, 1, 3)
    return t.reshape(pool.shape[0], pool.shape[2] * 4, -1)


class OracleState:
    """The oracle's caches for a workload, advanced step by step like the GPU's."""

    def __init__(self, wl: Workload, seqs: list[int] | None = None):
        self.wl = wl
        c = wl.cfg
        self.kc = poisoned_pool(wl, transposed=False)
        self.vc = poisoned_pool(wl, transposed=True)
        self.q = wl.queries()
        self.step_k, self.step_v = wl.step_kv()
        for b in (range(c.num_seqs) if seqs is None else seqs):
            k, v = wl.prior_kv(b)
            if k.shape[0]:
                oracle_write(c, raw_bits(k), raw_bits(v), wl.prior_slots(b), self.kc, self.vc)
        self.steps_written = 0

    def write_step(self, step: int) -> None:
        c = self.wl.cfg
        oracle_write(c, raw_bits(self.step_k[step]), raw_bits(self.step_v[step]),
                     self.wl.step_slots(step), self.kc, self.vc)
        self.steps_written = step + 1

    def decode(self, step: int, rows: np.ndarray | None = None, threads: int = 8) -> np.ndarray:
        c = self.wl.cfg
        return oracle_decode(c, raw_bits(self.q[step]), self.kc, self.vc, self.wl.block_tables,
                             self.wl.context_lens(step), rows=rows, threads=threads)

    def decode_abs_values(self, step: int, rows: np.ndarray | None = None,
                          threads: int = 8) -> np.ndarray:
        """The oracle's decode with every value replaced by its magnitude:
        sum_t w_t |v_te| / sum_t w_t with the same softmax weights w_t.  Rounding
        errors of a weighted sum are bounded relative to this sum of magnitudes,
        so it is the denominator of the componentwise relative error."""
        c = self.wl.cfg
        return oracle_decode(c, raw_bits(self.q[step]), self.kc, abs_values(self.vc, c.kv_dtype),
                             self.wl.block_tables, self.wl.context_lens(step), rows=rows,
                             threads=threads)


def logical_kv(wl: Workload, b: int, step: int) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous float64 K, V [L][Hkv][d] of sequence b as attended at `step`
    (decoded by torch, not by the oracle)."""
    k, v = wl.prior_kv(b)
    sk, sv = wl.step_kv()
    k = torch.cat([k, sk[:step + 1, b]], 0)
    v = torch.cat([v, sv[:step + 1, b]], 0)
    return k.to(torch.float64).numpy(), v.to(torch.float64).numpy()
