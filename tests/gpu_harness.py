"""Runs a seeded workload through the HIP library (via the Python binding) and,
optionally, through the oracle in lockstep from the same host inputs.

The GPU side only ever receives the generator's inputs; the oracle builds its
own caches with its own cache write.  Nothing flows from the GPU into the
oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import DTYPE_TORCH, POISON_BITS, Workload, raw_bits


def _poison(shape, dtype: str, device) -> torch.Tensor:
    if dtype == "fp8":
        return torch.full(shape, POISON_BITS[dtype], dtype=torch.uint8,
                          device=device).view(torch.float8_e4m3fn)
    if dtype == "f32":
        bits = torch.full(shape, POISON_BITS[dtype], dtype=torch.int32, device=device)
        return bits.view(torch.float32)
    val = POISON_BITS[dtype] - (1 << 16 if POISON_BITS[dtype] >= 1 << 15 else 0)
    return torch.full(shape, val, dtype=torch.int16, device=device).view(DTYPE_TORCH[dtype])


class GpuState:
    """GPU caches + tables for a workload; cache writes and decodes via libpa."""

    def __init__(self, wl: Workload, device: str = "cuda", poison: bool = True,
                 oracle_state=None, seqs_for_oracle=None):
        self.wl = wl
        c = wl.cfg
        self.device = device
        kvd = c.kv_dtype
        shape_k = pa.key_cache_shape(wl.num_blocks, c.num_kv_heads, c.head_dim, c.block_size,
                                     DTYPE_TORCH[kvd])
        shape_v = pa.value_cache_shape(wl.num_blocks, c.num_kv_heads, c.head_dim, c.block_size)
        if poison:
            self.kc = _poison(shape_k, kvd, device)
            self.vc = _poison(shape_v, kvd, device)
        else:
            self.kc = torch.empty(shape_k, dtype=DTYPE_TORCH[kvd], device=device)
            self.vc = torch.empty(shape_v, dtype=DTYPE_TORCH[kvd], device=device)
        self.block_tables = torch.from_numpy(wl.block_tables).to(device)
        self.q = wl.queries().to(device)
        sk, sv = wl.step_kv()
        self.step_k = sk.to(device)
        self.step_v = sv.to(device)
        self.step_slots = [torch.from_numpy(wl.step_slots(s)).to(device) for s in range(c.steps)]
        self.ctx = [torch.from_numpy(wl.context_lens(s)).to(device) for s in range(c.steps)]
        self._fill_prior(oracle_state, seqs_for_oracle)

    def _fill_prior(self, oracle_state, seqs_for_oracle):
        from tests.paged_host import oracle_write  # only when an oracle state is being filled
        c = self.wl.cfg
        for b in range(c.num_seqs):
            k, v = self.wl.prior_kv(b)
            if k.shape[0] == 0:
                continue
            slots = self.wl.prior_slots(b)
            write_kv(c, k.to(self.device), v.to(self.device),
                     torch.from_numpy(slots).to(self.device), self.kc, self.vc)
            if oracle_state is not None and (seqs_for_oracle is None or b in seqs_for_oracle):
                oracle_write(c, raw_bits(k), raw_bits(v), slots, oracle_state.kc,
                             oracle_state.vc)

    def write_step(self, step: int) -> None:
        write_kv(self.wl.cfg, self.step_k[step], self.step_v[step], self.step_slots[step],
                 self.kc, self.vc)

    def decode(self, step: int, out_dtype: torch.dtype = torch.float32, partition_size=None,
               flags: int = pa.AUTO, q: torch.Tensor | None = None) -> torch.Tensor:
        c = self.wl.cfg
        qq = self.q[step] if q is None else q
        out = torch.empty(qq.shape, dtype=out_dtype, device=self.device)
        p = c.partition_size if partition_size is None else partition_size
        decode_kv(c, out, qq, self.kc, self.vc, self.block_tables, self.ctx[step], p, flags=flags)
        return out


def assert_rejected(call, out: torch.Tensor, status: int = -4) -> None:
    """An argument set the library does not serve (by default a kernel family
    forced onto dtypes or a column count it has no kernel for): the call
    raises PAError with `status` (-4, PA_ERR_UNSUPPORTED) before launching
    anything, so `out`, NaN-filled here, keeps its fill."""
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    try:
        call()
    except pa.PAError as e:
        assert e.status == status, f"status {e.status}, expected {status}"
    else:
        raise AssertionError("the library accepted an argument set it does not serve")
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "a rejected call wrote to out"


def write_kv(cfg, k, v, slots, kc, vc) -> None:
    """The library's cache write for the config's cache dtype."""
    if cfg.kv_dtype == "fp8":
        pa.cache_write_fp8(k, v, slots, kc, vc, *cfg.fp8_scales)
    else:
        pa.cache_write(k, v, slots, kc, vc)


def decode_kv(cfg, out, q, kc, vc, block_tables, lens, partition_size, workspace=None,
              flags=pa.AUTO, phase: str = "both") -> None:
    """The library's decode (or one phase of it) for the config's cache dtype."""
    args = (out, q, kc, vc, block_tables, lens, cfg.attn_scale())
    if cfg.kv_dtype == "fp8":
        fn = {"both": pa.decode_fp8, "partitions": pa.decode_fp8_partitions}.get(phase)
        if fn is not None:
            fn(*args, *cfg.fp8_scales, cfg.block_size, partition_size, workspace, flags)
            return
    else:
        fn = {"both": pa.decode, "partitions": pa.decode_partitions}.get(phase)
        if fn is not None:
            fn(*args, cfg.block_size, partition_size, workspace, flags)
            return
    pa.decode_merge(*args, cfg.block_size, partition_size, workspace, flags)


def oracle_state_empty(wl: Workload):
    """An OracleState-like holder whose prior context is filled by GpuState
    (from the same generated host tensors)."""
    from tests.paged_host import OracleState

    st = OracleState.__new__(OracleState)
    from tests.paged_host import poisoned_pool
    st.wl = wl
    st.kc = poisoned_pool(wl, transposed=False)
    st.vc = poisoned_pool(wl, transposed=True)
    st.q = wl.queries()
    st.step_k, st.step_v = wl.step_kv()
    st.steps_written = 0
    return st


def max_abs_err(gpu: torch.Tensor, ref: np.ndarray, rows: np.ndarray | None = None) -> float:
    g = gpu.float().cpu().numpy().astype(np.float64).reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    if rows is not None:
        g, r = g[rows], r[rows]
    return float(np.abs(g - r).max())


def rowwise_rel_err(gpu: torch.Tensor, ref: np.ndarray, rows: np.ndarray | None = None) -> float:
    """max over rows of max_e |gpu - ref| / max_e |ref| (normwise per row)."""
    g = gpu.float().cpu().numpy().astype(np.float64).reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    if rows is not None:
        g, r = g[rows], r[rows]
    return float((np.abs(g - r).max(axis=1) / np.abs(r).max(axis=1)).max())


def componentwise_rel_err(gpu: torch.Tensor, ref: np.ndarray, ref_abs: np.ndarray,
                          rows: np.ndarray | None = None) -> float:
    """max over elements of |gpu - ref| / ref_abs, where ref_abs is the oracle's
    decode over |V| (the same softmax weights on the values' magnitudes).  An
    element's rounding error in a weighted sum scales with the sum of the
    magnitudes, not with the (possibly cancelled) result, so this is the
    elementwise relative error with the denominator the arithmetic fixes."""
    g = gpu.float().cpu().numpy().astype(np.float64).reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    a = ref_abs.reshape(-1, ref_abs.shape[-1])
    if rows is not None:
        g, r, a = g[rows], r[rows], a[rows]
    return float((np.abs(g - r) / np.maximum(a, 1e-300)).max())
