"""Seeded synthetic decode batches (the five decode workloads and small variants).

This module only draws inputs: context lengths, a shuffled pool of physical
blocks, per-sequence block lists / block tables, the slot of every token, and
N(0,1) query/key/value values rounded to the storage dtype.  It holds none of
the attention or cache-write arithmetic; both the HIP path and the CPU oracle
consume what it returns.

Reproducibility: numpy ``Generator(PCG64)`` streams spawned from
``SeedSequence(seed)`` -- one each for lengths, block-pool permutation, queries
and per-step new tokens, plus one per sequence for its prior-token K/V, so any
single sequence can be regenerated without drawing the others.

Rounding to fp16/bf16 is round-to-nearest-even via torch's CPU conversion.

Slots follow the paged-KV convention of the "[core] Multi Step Scheduling"
pull request's advance_step review thread (slot mapping, block tables, block
size): the token at logical position ``pos`` of a sequence whose physical
blocks are ``blocks`` lives in slot ``blocks[pos // bs] * bs + pos % bs``.
Choosing slots is the scheduler's job; it is input preparation here.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Sequence

import numpy as np
import torch

# "fp8": OCP E4M3, a KV-cache storage type only (written from the 16-bit values
# with per-tensor scales)
DTYPE_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8": torch.float8_e4m3fn}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
# quiet-NaN bit patterns used to poison unused cache memory in parity runs
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}

# stream indices under SeedSequence(seed).spawn(...)
_S_LENGTHS, _S_POOL, _S_Q, _S_STEP, _S_SEQ, _S_SAMPLED, _S_MQ = range(7)
VOCAB = 128256  # token ids drawn for the "sampled" next tokens (a Llama-3-sized vocabulary)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # storage dtype of q, K, V: "f32" | "f16" | "bf16"
    block_size: int
    seed: int
    lengths: Callable[[np.random.Generator, int], np.ndarray]  # context at the first step
    steps: int = 1
    k_scale: float = 1.0
    partition_size: int = 0  # 0 = library default
    num_blocks: int | None = None  # None = ceil(1.25 * blocks needed)
    scale: float | None = None  # None = 1/sqrt(head_dim) rounded to fp32
    cache_dtype: str = ""  # "" = dtype; "fp8" = E4M3 caches written with fp8_scales
    fp8_scales: tuple = (1.0, 1.0)  # (k, v): cache element = stored value * scale

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def kv_dtype(self) -> str:
        """Storage dtype of the KV caches."""
        return self.cache_dtype or self.dtype

    def attn_scale(self) -> float:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        return float(np.float32(s))


def _fixed(values: Sequence[int]) -> Callable[[np.random.Generator, int], np.ndarray]:
    vals = np.asarray(values, dtype=np.int64)
    return lambda rng, n: vals.copy()


def _uniform(lo: int, hi: int):
    return lambda rng, n: rng.integers(lo, hi, size=n, endpoint=True)


def _skewed(lo: int, hi: int, long_len: int, long_index: int):
    def f(rng, n):
        short = rng.integers(lo, hi, size=n - 1, endpoint=True)
        return np.insert(short, long_index if long_index >= 0 else n - 1, long_len)
    return f


def _lognormal(median: float, sigma: float, lo: int, hi: int):
    def f(rng, n):
        x = np.exp(rng.normal(math.log(median), sigma, size=n))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return f


# The five decode workloads, numbered 1..5.  Number 1 (4 fp32 sequences of at
# most 200 tokens) is the small case the oracle finishes in seconds; number 4
# (256 Llama-3-8B-shaped GQA sequences, bf16) is the throughput workload.
WORKLOADS: dict[int, DecodeConfig] = {
    1: DecodeConfig("tiny-fp32", 4, 4, 4, 64, "f32", 16, seed=1,
                    lengths=_fixed([1, 17, 64, 200]), num_blocks=64),
    2: DecodeConfig("llama7b-mha-fp16", 64, 32, 32, 128, "f16", 16, seed=2,
                    lengths=_uniform(128, 2048)),
    3: DecodeConfig("llama13b-skew-fp16", 32, 40, 40, 128, "f16", 16, seed=3,
                    lengths=_skewed(16, 256, 4096, -1), partition_size=512),
    4: DecodeConfig("llama3-8b-gqa-bf16", 256, 32, 8, 128, "bf16", 16, seed=4,
                    lengths=_lognormal(1024.0, 1.0, 1, 8192), k_scale=0.5),
    5: DecodeConfig("llama3-70b-gqa-long-bf16", 64, 64, 8, 128, "bf16", 32, seed=5,
                    lengths=_uniform(4096, 32768), steps=8),
}


def config3_long_first() -> DecodeConfig:
    """The skewed 13B-shaped batch (number 3) with its 4096-token sequence at
    batch index 0 instead of the last index; the short sequences' lengths are
    the same draws."""
    return dataclasses.replace(WORKLOADS[3], name="llama13b-skew-long-first-fp16",
                               lengths=_skewed(16, 256, 4096, 0))


def fp8_variant(cfg: DecodeConfig, k_scale: float, v_scale: float) -> DecodeConfig:
    """The same workload with E4M3 caches: the 16-bit K/V are written with the
    per-tensor scales k_scale, v_scale (powers of two here, so x / scale is
    exact and only the E4M3 rounding quantizes)."""
    return dataclasses.replace(cfg, name=cfg.name.replace("-bf16", "") + "-fp8kv",
                               cache_dtype="fp8", fp8_scales=(k_scale, v_scale))


# E4M3-cache variants of the two GQA workloads (their KV are
# N(0, 0.5^2) / N(0, 1) keys and N(0, 1) values: with these scales every drawn
# value lands well inside the E4M3 range, the largest near 200).
FP8_WORKLOADS: dict[int, DecodeConfig] = {
    4: fp8_variant(WORKLOADS[4], 2.0 ** -6, 2.0 ** -5),
    5: fp8_variant(WORKLOADS[5], 2.0 ** -5, 2.0 ** -5),
}


def custom_config(name: str, lengths: Sequence[int], num_q_heads: int, num_kv_heads: int,
                  head_dim: int, dtype: str, block_size: int, seed: int, steps: int = 1,
                  k_scale: float = 1.0, partition_size: int = 0,
                  num_blocks: int | None = None, scale: float | None = None,
                  cache_dtype: str = "", fp8_scales: tuple = (1.0, 1.0)) -> DecodeConfig:
    return DecodeConfig(name, len(lengths), num_q_heads, num_kv_heads, head_dim, dtype,
                        block_size, seed, _fixed(lengths), steps, k_scale, partition_size,
                        num_blocks, scale, cache_dtype, fp8_scales)


def token_kv(tokens, positions, num_kv_heads: int, head_dim: int, dtype: str,
             seed: int) -> tuple[torch.Tensor, torch.Tensor]:
    """K, V rows [n][num_kv_heads][head_dim] (storage dtype) of the given tokens at the
    given positions: a seeded function of (token id, position) alone, so that sequences
    with equal token prefixes have equal KV there (what block sharing relies on)."""
    n = len(tokens)
    k = np.empty((n, num_kv_heads, head_dim), np.float32)
    v = np.empty_like(k)
    for i, (t, p) in enumerate(zip(tokens, positions)):
        rng = np.random.default_rng([seed, int(t), int(p)])
        kv = rng.standard_normal((2, num_kv_heads, head_dim), dtype=np.float32)
        k[i], v[i] = kv[0], kv[1]
    return round_to(k, dtype), round_to(v, dtype)


def round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU torch tensor of the storage dtype (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to(DTYPE_TORCH[dtype])


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """The raw element bits of a CPU tensor as a numpy array (uint8/uint16/uint32)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


class Workload:
    """All inputs of one decode workload, drawn from its seed.

    Step s (0-based, ``steps`` of them) appends one token per sequence at
    logical position ``L0 + s - 1`` and attends over ``L0 + s`` tokens, where
    ``L0`` is the drawn context length.  Positions ``0 .. L0 - 2`` are the
    prior context, written before the first step.
    """

    def __init__(self, cfg: DecodeConfig):
        self.cfg = cfg
        root = np.random.SeedSequence(cfg.seed)
        self._ss = root.spawn(7)
        n = cfg.num_seqs
        self._seq_ss = self._ss[_S_SEQ].spawn(n)
        rng_len = np.random.Generator(np.random.PCG64(self._ss[_S_LENGTHS]))
        L0 = np.asarray(cfg.lengths(rng_len, n), dtype=np.int64)
        if L0.shape != (n,) or (L0 < 1).any():
            raise ValueError("context lengths must be >= 1, one per sequence")
        self.lens0 = L0
        self.final_lens = L0 + cfg.steps - 1
        bs = cfg.block_size
        nblk = -(-self.final_lens // bs)
        need = int(nblk.sum())
        NB = cfg.num_blocks if cfg.num_blocks is not None else int(math.ceil(1.25 * need))
        if NB < need:
            raise ValueError(f"pool of {NB} blocks cannot hold {need}")
        self.num_blocks = NB
        rng_pool = np.random.Generator(np.random.PCG64(self._ss[_S_POOL]))
        perm = rng_pool.permutation(NB).astype(np.int64)
        self.block_lists = []
        off = 0
        for b in range(n):
            self.block_lists.append(perm[off:off + nblk[b]])
            off += nblk[b]
        self.max_blocks_per_seq = int(nblk.max()) if n else 1
        bt = np.full((n, self.max_blocks_per_seq), -1, dtype=np.int32)
        for b in range(n):
            bt[b, :nblk[b]] = self.block_lists[b]
        self.block_tables = bt

    # ---- sizes ---------------------------------------------------------
    @property
    def elem_bytes(self) -> int:
        """Bytes per KV cache element."""
        return DTYPE_BYTES[self.cfg.kv_dtype]

    def context_lens(self, step: int) -> np.ndarray:
        return (self.lens0 + step).astype(np.int32)

    def kv_bytes(self, step: int) -> int:
        """Algorithmic K+V bytes one decode step reads: each context element once."""
        c = self.cfg
        return int(self.context_lens(step).sum()) * c.num_kv_heads * c.head_dim * 2 * self.elem_bytes

    # ---- slots -----------------------------------------------------------
    def slots_for(self, b: int, positions: np.ndarray) -> np.ndarray:
        bs = self.cfg.block_size
        blocks = self.block_lists[b]
        positions = np.asarray(positions, dtype=np.int64)
        return blocks[positions // bs] * bs + positions % bs

    def prior_slots(self, b: int) -> np.ndarray:
        return self.slots_for(b, np.arange(self.lens0[b] - 1))

    def step_slots(self, step: int) -> np.ndarray:
        return np.array([self.slots_for(b, [self.lens0[b] - 1 + step])[0]
                         for b in range(self.cfg.num_seqs)], dtype=np.int64)

    # ---- values ----------------------------------------------------------
    def prior_kv(self, b: int) -> tuple[torch.Tensor, torch.Tensor]:
        """K, V of sequence b's prior positions: [L0_b - 1][Hkv][d] in the storage dtype."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(self._seq_ss[b]))
        shape = (int(self.lens0[b]) - 1, c.num_kv_heads, c.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if c.k_scale != 1.0:
            k *= np.float32(c.k_scale)
        return round_to(k, c.dtype), round_to(v, c.dtype)

    def queries(self) -> torch.Tensor:
        """q for every step: [steps][B][Hq][d] in the storage dtype."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(self._ss[_S_Q]))
        q = rng.standard_normal((c.steps, c.num_seqs, c.num_q_heads, c.head_dim), dtype=np.float32)
        return round_to(q, c.dtype)

    def multi_queries(self, num_queries: int) -> torch.Tensor:
        """q of a multi-query decode (several new tokens per sequence, e.g. draft tokens
        being verified): [B][num_queries][Hq][d] in the storage dtype."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(self._ss[_S_MQ]))
        shape = (c.num_seqs, num_queries, c.num_q_heads, c.head_dim)
        return round_to(rng.standard_normal(shape, dtype=np.float32), c.dtype)

    def step_kv(self) -> tuple[torch.Tensor, torch.Tensor]:
        """New-token K, V for every step: [steps][B][Hkv][d] in the storage dtype."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(self._ss[_S_STEP]))
        shape = (c.steps, c.num_seqs, c.num_kv_heads, c.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if c.k_scale != 1.0:
            k *= np.float32(c.k_scale)
        return round_to(k, c.dtype), round_to(v, c.dtype)

    def sampled_tokens(self) -> np.ndarray:
        """Token ids standing in for the sampler's output after each step:
        int64 [steps][B], uniform over the vocabulary."""
        c = self.cfg
        rng = np.random.Generator(np.random.PCG64(self._ss[_S_SAMPLED]))
        return rng.integers(0, VOCAB, size=(c.steps, c.num_seqs), dtype=np.int64)

    def initial_state(self) -> dict:
        """Per-sequence decode state before the first step: the input position
        of the first new token, the context length it is attended with and its
        slot."""
        pos = (self.lens0 - 1).astype(np.int64)
        return {"input_tokens": np.zeros(self.cfg.num_seqs, np.int64),
                "input_positions": pos,
                "seq_lens": self.lens0.astype(np.int32),
                "slot_mapping": self.step_slots(0)}

    def describe(self) -> dict:
        L = self.context_lens(self.cfg.steps - 1).astype(np.int64)
        bs = self.cfg.block_size
        used = int((-(-L // bs)).sum()) * bs
        return {
            "workload": self.cfg.name,
            "num_seqs": self.cfg.num_seqs,
            "num_q_heads": self.cfg.num_q_heads,
            "num_kv_heads": self.cfg.num_kv_heads,
            "head_dim": self.cfg.head_dim,
            "kv_dtype": self.cfg.kv_dtype,
            "block_size": bs,
            "num_blocks": self.num_blocks,
            "steps": self.cfg.steps,
            "ctx_mean": float(L.mean()),
            "ctx_p50": float(np.median(L)),
            "ctx_p99": float(np.percentile(L, 99)),
            "ctx_max": int(L.max()),
            "internal_fragmentation": 1.0 - float(L.sum()) / used,
        }
