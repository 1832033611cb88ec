"""GPU parity for multi-query decode (several new query tokens per sequence,
each attending causally up to its own position, as when a sequence's proposed
draft tokens are scored in one pass), through the C ABI, against the fp64
oracle's multi-query decode.

Bars as for single-query decode: 2e-3 max absolute error for 16-bit
attention, 1e-5 row-wise relative error for fp32; one query token per
sequence is bit-identical to the single-query entry point; queries whose
position falls before the sequence start give exact zero rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import (WORKLOADS, DTYPE_TORCH, FP8_WORKLOADS, Workload,
                                                   custom_config, raw_bits)
from tests.gpu_harness import (GpuState, assert_rejected, max_abs_err, oracle_state_empty,
                               rowwise_rel_err)

pytestmark = pytest.mark.gpu

TOL_ABS_HALF = 2e-3
TOL_REL_F32 = 1e-5
KERNELS = {"auto": pa.AUTO, "valu": pa.FORCE_VALU, "mfma": pa.FORCE_MFMA}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _scales(cfg):
    return cfg.fp8_scales if cfg.kv_dtype == "fp8" else (1.0, 1.0)


def _gpu_mq(gs: GpuState, q: torch.Tensor, lens: torch.Tensor, partition_size: int,
            flags: int, out_dtype=torch.float32, fn=None) -> torch.Tensor:
    c = gs.wl.cfg
    out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    (fn or pa.decode_mq)(out, q, gs.kc, gs.vc, gs.block_tables, lens, c.attn_scale(),
                         c.block_size, partition_size, None, flags, *_scales(c))
    return out


def _oracle_mq(st, q: torch.Tensor, lens: np.ndarray, rows=None, threads: int = 8):
    c = st.wl.cfg
    ks, vs = _scales(c)
    return oracle.decode_mq(raw_bits(q.cpu()), c.dtype, st.kc, st.vc, c.kv_dtype,
                            st.wl.block_tables, lens, c.attn_scale(), rows=rows,
                            threads=threads, k_scale=ks, v_scale=vs)


def _check(out: torch.Tensor, ref: np.ndarray, dtype: str, rows=None) -> float:
    if dtype == "f32":
        err = rowwise_rel_err(out, ref, rows)
        assert err <= TOL_REL_F32, f"rowwise relative error {err:.3e}"
    else:
        err = max_abs_err(out, ref, rows)
        assert err <= TOL_ABS_HALF, f"max abs error {err:.3e}"
    return err


def _states(cfg):
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    return wl, gs, st


def _supported(Q, cfg, kernel) -> bool:
    try:
        pa.decode_mq_kernel(Q, cfg.num_q_heads, cfg.num_kv_heads, DTYPE_TORCH[cfg.dtype],
                            DTYPE_TORCH[cfg.kv_dtype], KERNELS[kernel])
    except pa.PAError:
        return False
    return True


# ------------------------------------------------------------------ small cases

# (dtype, d, bs, Hq, Hkv, context lengths, query tokens per sequence)
MQ_CASES = [
    ("bf16", 128, 16, 32, 8, [4, 17, 300, 1029], 2),
    ("bf16", 128, 16, 32, 8, [5, 16, 33, 700], 3),
    ("bf16", 128, 16, 32, 8, [4, 64, 65, 1500], 4),
    ("bf16", 128, 16, 16, 4, [8, 100, 513], 5),
    ("bf16", 128, 32, 8, 1, [2, 63, 999], 2),
    ("bf16", 128, 32, 8, 1, [8, 31, 257], 8),
    ("bf16", 64, 8, 4, 2, [6, 9, 200], 6),
    ("bf16", 64, 64, 6, 3, [10, 65, 400], 10),
    ("f16", 64, 32, 4, 4, [5, 33, 450], 5),
    ("f16", 128, 16, 6, 2, [7, 16, 17, 600], 7),
    ("f16", 128, 16, 3, 1, [12, 40, 333], 12),
    ("f16", 128, 16, 2, 2, [16, 20, 301], 16),
    # two 16-column tiles over one K/V read: 24 or 32 (query, head) columns per item
    ("bf16", 128, 16, 32, 4, [4, 100, 1300, 2500], 4),
    ("bf16", 64, 16, 16, 2, [3, 50, 700], 3),
    ("f16", 128, 32, 16, 4, [6, 333, 1200], 6),
    ("bf16", 128, 16, 32, 8, [8, 64, 800, 1700], 8),
    ("f32", 128, 16, 8, 2, [4, 40, 129], 2),
    ("f32", 64, 8, 4, 4, [8, 9, 250], 8),
]


@pytest.mark.parametrize("case", MQ_CASES,
                         ids=lambda c: f"{c[0]}-d{c[1]}-bs{c[2]}-{c[3]}x{c[4]}-Q{c[6]}")
@pytest.mark.parametrize("partition", ["auto", "one-pass", "min"])
@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma"])
@pytest.mark.parametrize("waves", [0, 4])
def test_decode_mq_parity_small(case, partition, kernel, waves):
    dt, d, bs, hq, hkv, lens, Q = case
    cfg = custom_config(f"mq-{dt}", lens, hq, hkv, d, dt, bs, seed=sum(lens) + Q + d)
    max_ctx = -(-max(lens) // bs) * bs
    p = {"auto": 0, "one-pass": max_ctx, "min": max(bs, 16) * 2}[partition]
    if not _supported(Q, cfg, kernel):
        # no kernel of this family holds Q query tokens x the group: refused at the C ABI
        gs = GpuState(Workload(cfg))
        q = Workload(cfg).multi_queries(Q).cuda()
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        flags = KERNELS[kernel] | (pa.WAVES_FLAG[waves] if waves else 0)
        assert_rejected(lambda: pa.decode_mq(out, q, gs.kc, gs.vc, gs.block_tables, gs.ctx[0],
                                             cfg.attn_scale(), cfg.block_size, p, None, flags,
                                             *_scales(cfg)), out)
        return
    wl, gs, st = _states(cfg)
    _say(f"mq decode {dt} d={d} bs={bs} {hq}x{hkv} lens={lens} Q={Q} P={p} {kernel} "
         f"waves={waves}")
    q = wl.multi_queries(Q)
    flags = KERNELS[kernel] | (pa.WAVES_FLAG[waves] if waves else 0)
    out = _gpu_mq(gs, q.cuda(), gs.ctx[0], p, flags)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    _check(out, _oracle_mq(st, q, wl.context_lens(0)), dt)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("Q,hq", [(2, 16), (4, 16), (4, 32)])
def test_decode_mq_fp8_cache(kernel, Q, hq):
    cfg = custom_config("mq-fp8", [4, 100, 777, 1300], hq, 4, 128, "bf16", 16, seed=61 + Q,
                        cache_dtype="fp8", fp8_scales=(2.0 ** -5, 0.0371))
    wl, gs, st = _states(cfg)
    _say(f"mq fp8 decode Q={Q} {kernel}")
    q = wl.multi_queries(Q)
    out = _gpu_mq(gs, q.cuda(), gs.ctx[0], 0, KERNELS[kernel])
    torch.cuda.synchronize()
    _check(out, _oracle_mq(st, q, wl.context_lens(0)), "bf16")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_decode_mq_out_in_cache_dtype(dt):
    cfg = custom_config("mq-out", [9, 200, 901], 8, 2, 128, dt, 16, seed=83)
    wl, gs, st = _states(cfg)
    q = wl.multi_queries(4)
    out = _gpu_mq(gs, q.cuda(), gs.ctx[0], 0, pa.AUTO, out_dtype=q.dtype)
    torch.cuda.synchronize()
    ref = _oracle_mq(st, q, wl.context_lens(0))
    ulp = 2.0 ** (-10 if dt == "f16" else -7)
    err = np.abs(out.double().cpu().numpy() - ref)
    assert (err <= np.abs(ref) * ulp + TOL_ABS_HALF).all()


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("partition", [0, 32])
@pytest.mark.parametrize("waves", [1, 4])
def test_decode_mq_single_query_is_decode(kernel, partition, waves):
    """One query token per sequence runs the single-query decode: bit-identical."""
    cfg = custom_config("mq-q1", [1, 30, 500, 1025], 32, 8, 128, "bf16", 16, seed=5)
    wl, gs, _ = _states(cfg)
    flags = KERNELS[kernel] | pa.WAVES_FLAG[waves]
    q = gs.q[0]
    ref = gs.decode(0, partition_size=partition, flags=flags)
    out = _gpu_mq(gs, q.unsqueeze(1).contiguous(), gs.ctx[0], partition, flags)
    torch.cuda.synchronize()
    assert torch.equal(out.squeeze(1), ref)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_decode_mq_short_sequences_zero_rows(kernel):
    """Context shorter than the query count: the queries whose position is before the
    sequence start give zero rows; the last L queries are a multi-query decode of L
    tokens; an empty sequence is all zeros."""
    Q = 4
    lens = [0, 1, 2, 3, 4, 50]
    cfg = custom_config("mq-short", [max(n, 1) for n in lens], 8, 2, 64, "bf16", 16, seed=17)
    wl, gs, st = _states(cfg)
    q = wl.multi_queries(Q)
    ctx = np.array(lens, np.int32)
    out = _gpu_mq(gs, q.cuda(), torch.from_numpy(ctx).cuda(), 0, KERNELS[kernel])
    torch.cuda.synchronize()
    out = out.cpu()
    for b, L in enumerate(lens):
        keep = min(L, Q)
        assert torch.equal(out[b, : Q - keep], torch.zeros_like(out[b, : Q - keep])), f"seq {b}"
        if keep == 0:
            continue
        # the oracle over the same caches with this sequence's table alone
        ref = oracle.decode_mq(raw_bits(q[b: b + 1, Q - keep:].contiguous()), "bf16", st.kc,
                               st.vc, "bf16", wl.block_tables[b: b + 1],
                               np.array([L], np.int32), cfg.attn_scale())
        err = max_abs_err(out[b: b + 1, Q - keep:], ref)
        assert err <= TOL_ABS_HALF, f"seq {b}: {err:.3e}"


def test_decode_mq_phases_match_one_call():
    cfg = custom_config("mq-ph", [6, 300, 1200], 16, 4, 128, "bf16", 16, seed=29)
    wl, gs, _ = _states(cfg)
    Q = 3
    q = wl.multi_queries(Q).cuda()
    c = cfg
    p = 256
    need = pa.decode_workspace_size(c.num_seqs * Q, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                    c.block_size, gs.block_tables.shape[1], p, gs.kc.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    one = _gpu_mq(gs, q, gs.ctx[0], p, pa.AUTO)
    two = torch.empty_like(one)
    args = (two, q, gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), c.block_size, p,
            ws, pa.AUTO)
    pa.decode_mq_partitions(*args)
    pa.decode_mq_merge(*args)
    torch.cuda.synchronize()
    assert torch.equal(one, two)


# ------------------------------------------------------------------ full size

@pytest.mark.parametrize("cid,Q,fp8", [(4, 4, False), (4, 2, True), (5, 2, False), (5, 4, False),
                                        (4, 8, False)])
def test_full_workload_mq_parity(cid, Q, fp8):
    """The GQA workloads at full size with Q query tokens per sequence (library-picked
    launch): every (sequence, query, head) row against the oracle."""
    cfg = FP8_WORKLOADS[cid] if fp8 else WORKLOADS[cid]
    wl = Workload(cfg)
    assert int(wl.context_lens(0).min()) >= Q
    _say(f"full mq workload {cfg.name} Q={Q}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    q = wl.multi_queries(Q)
    out = _gpu_mq(gs, q.cuda(), gs.ctx[0], 0, pa.AUTO)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = max_abs_err(out, _oracle_mq(st, q, wl.context_lens(0), threads=16))
    _say(f"  err {err:.3e} rows all ({out.numel() // cfg.head_dim})")
    assert err <= TOL_ABS_HALF
