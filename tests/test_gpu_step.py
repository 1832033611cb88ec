"""GPU checks of pa_decode_step (the step's cache write + decode in as few
launches as the grid allows): bit-identical caches and outputs to
pa_cache_write followed by pa_decode, on every grid, and within tolerance of
the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import Workload, custom_config, raw_bits
from tests.gpu_harness import GpuState, max_abs_err, oracle_state_empty, rowwise_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    # dtype, Hq, Hkv, bs, lens, partition
    ("bf16", 32, 8, 16, [1, 17, 300, 1029, 2500, 4000], 1024),   # persistent sorted grid
    ("bf16", 32, 8, 16, [1, 17, 300, 1029, 2500, 4000], 256),    # sorted grid
    ("f16", 16, 16, 32, [5, 64, 700, 1500], 512),
    ("f32", 8, 2, 16, [3, 40, 129, 600], 128),
    ("bf16", 8, 2, 16, [7, 90, 200], 0),                         # one pass
]
GRIDS = {"auto": pa.AUTO, "grid": pa.NO_WORK_LIST, "list": pa.WORK_LIST}


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-bs{c[3]}-P{c[5]}")
@pytest.mark.parametrize("grid", list(GRIDS))
def test_step_equals_write_then_decode(case, grid):
    dt, hq, hkv, bs, lens, P = case
    cfg = custom_config(f"step-{dt}", lens, hq, hkv, 128, dt, bs, seed=sum(lens) + hq)
    wl = Workload(cfg)
    _say(f"step {dt} {hq}x{hkv} bs={bs} P={P} grid={grid}")
    st = oracle_state_empty(wl)
    g1 = GpuState(wl, oracle_state=st)
    g2 = GpuState(wl)
    st.write_step(0)
    flags = GRIDS[grid]
    a = torch.full(g1.q[0].shape, float("nan"), device="cuda")
    b = torch.full(g1.q[0].shape, float("nan"), device="cuda")
    pa.cache_write(g1.step_k[0], g1.step_v[0], g1.step_slots[0], g1.kc, g1.vc)
    pa.decode(a, g1.q[0], g1.kc, g1.vc, g1.block_tables, g1.ctx[0], cfg.attn_scale(), bs, P,
              flags=flags)
    pa.decode_step(g2.step_k[0], g2.step_v[0], g2.step_slots[0], b, g2.q[0], g2.kc, g2.vc,
                   g2.block_tables, g2.ctx[0], cfg.attn_scale(), bs, P, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(g1.kc.cpu()), raw_bits(g2.kc.cpu()))
    assert np.array_equal(raw_bits(g1.vc.cpu()), raw_bits(g2.vc.cpu()))
    assert torch.equal(a, b)
    ref = st.decode(0)
    err = rowwise_rel_err(b, ref) if dt == "f32" else max_abs_err(b, ref)
    assert err <= (1e-5 if dt == "f32" else 2e-3)


def test_step_phases_and_empty_batch():
    cfg = custom_config("step-ph", [9, 800, 3000], 16, 4, 128, "bf16", 16, seed=4)
    wl = Workload(cfg)
    g1, g2 = GpuState(wl), GpuState(wl)
    c = cfg
    P = 1024
    need = pa.decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                    c.block_size, wl.max_blocks_per_seq, P, g1.kc.dtype)
    ws = torch.full((need // 4,), float("nan"), device="cuda").view(torch.uint8)
    a = torch.empty(g1.q[0].shape, device="cuda")
    b = torch.empty_like(a)
    pa.decode_step(g1.step_k[0], g1.step_v[0], g1.step_slots[0], a, g1.q[0], g1.kc, g1.vc,
                   g1.block_tables, g1.ctx[0], c.attn_scale(), 16, P)
    args = (g2.step_k[0], g2.step_v[0], g2.step_slots[0], b, g2.q[0], g2.kc, g2.vc,
            g2.block_tables, g2.ctx[0], c.attn_scale(), 16, P, ws)
    pa.decode_step_partitions(*args)
    pa.decode_merge(b, g2.q[0], g2.kc, g2.vc, g2.block_tables, g2.ctx[0], c.attn_scale(), 16, P,
                    ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert np.array_equal(raw_bits(g1.kc.cpu()), raw_bits(g2.kc.cpu()))
    # no sequences to attend: the write still happens
    g3 = GpuState(wl)
    empty = torch.empty((0, c.num_q_heads, c.head_dim), device="cuda")
    pa.decode_step(g3.step_k[0], g3.step_v[0], g3.step_slots[0], empty,
                   g3.q[0][:0].contiguous(), g3.kc, g3.vc, g3.block_tables[:0].contiguous(),
                   g3.ctx[0][:0].contiguous(), c.attn_scale(), 16, P)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(g1.kc.cpu()), raw_bits(g3.kc.cpu()))
    assert np.array_equal(raw_bits(g1.vc.cpu()), raw_bits(g3.vc.cpu()))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-bs{c[3]}-P{c[5]}")
@pytest.mark.parametrize("grid", list(GRIDS))
def test_order_then_ordered_decode_equals_step(case, grid):
    """pa_decode_order (the step's write and, on the sorted grid, the item order)
    followed by pa_decode_partitions with PA_DECODE_ORDERED and the merge: the
    same caches and outputs as pa_decode_step, bit for bit, into NaN-filled
    outputs and workspace."""
    dt, hq, hkv, bs, lens, P = case
    cfg = custom_config(f"order-{dt}", lens, hq, hkv, 128, dt, bs, seed=sum(lens) + hq)
    wl = Workload(cfg)
    c = cfg
    _say(f"order {dt} {hq}x{hkv} bs={bs} P={P} grid={grid}")
    g1, g2 = GpuState(wl), GpuState(wl)
    flags = GRIDS[grid]
    a = torch.full(g1.q[0].shape, float("nan"), device="cuda")
    b = torch.full(g1.q[0].shape, float("nan"), device="cuda")
    pa.decode_step(g1.step_k[0], g1.step_v[0], g1.step_slots[0], a, g1.q[0], g1.kc, g1.vc,
                   g1.block_tables, g1.ctx[0], c.attn_scale(), bs, P, flags=flags)
    need = pa.decode_workspace_size(c.num_seqs, hq, hkv, 128, bs, wl.max_blocks_per_seq, P,
                                    g2.kc.dtype, flags)
    ws = torch.full((max(need, 256) // 4,), float("nan"), device="cuda").view(torch.uint8)
    dargs = (b, g2.q[0], g2.kc, g2.vc, g2.block_tables, g2.ctx[0], c.attn_scale(), bs, P, ws)
    pa.decode_order(*dargs, flags, k=g2.step_k[0], v=g2.step_v[0], slot_mapping=g2.step_slots[0])
    pa.decode_partitions(*dargs, flags | pa.ORDERED)
    pa.decode_merge(*dargs, flags)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(g1.kc.cpu()), raw_bits(g2.kc.cpu()))
    assert np.array_equal(raw_bits(g1.vc.cpu()), raw_bits(g2.vc.cpu()))
    assert torch.equal(a, b)


def test_order_then_ordered_decode_fp8_and_refusals():
    """E4M3 caches: pa_decode_order without a write, then the ordered decode,
    equals pa_decode_fp8.  The ordered flag is refused where no order can have
    been prepared: multi-query decodes, steps, the allocation-free decode."""
    from pagedattention_kv_cache_amd.workloads import FP8_WORKLOADS  # noqa: F401
    cfg = custom_config("order-fp8", [3, 700, 1500, 2600], 32, 8, 128, "bf16", 16, seed=12,
                        cache_dtype="fp8", fp8_scales=(2.0 ** -6, 2.0 ** -5))
    wl = Workload(cfg)
    c = cfg
    gs = GpuState(wl)
    gs.write_step(0)
    P = 1024
    ks, vs = c.fp8_scales
    a = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    b = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    pa.decode_fp8(a, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), ks, vs,
                  16, P)
    need = pa.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, wl.max_blocks_per_seq, P,
                                    gs.kc.dtype, pa.AUTO)
    ws = torch.full((need // 4,), float("nan"), device="cuda").view(torch.uint8)
    pa.decode_order(b, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), 16, P,
                    ws)
    pa.decode_fp8_partitions(b, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0],
                             c.attn_scale(), ks, vs, 16, P, ws, pa.ORDERED)
    pa.decode_merge(b, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), 16, P,
                    ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # refusals: nothing runs, out keeps its NaN fill
    q2 = wl.multi_queries(2).cuda()
    out2 = torch.full(q2.shape, float("nan"), device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.decode_mq(out2, q2, gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), 16, P,
                     None, pa.ORDERED, ks, vs)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.isnan(out2).all()


FP8_ORDER_CASES = [
    # lens, partition, grid flags
    ([3, 700, 1500, 2600], 1024, pa.AUTO),                       # sorted, counter deal
    ([3, 700, 1500, 2600, 90, 40], 256, pa.AUTO),                 # a step sorts (static deal)
    ([3, 700, 1500, 2600, 90, 40], 256, pa.WORK_LIST),            # the write on its own
    ([7, 90, 200], 0, pa.AUTO),                                   # one pass: the write alone
    ([int(x) for x in np.random.default_rng(3).integers(16, 257, 63)] + [8192], 0,
     pa.AUTO),                                                    # the device refines
]


@pytest.mark.parametrize("case", FP8_ORDER_CASES,
                         ids=lambda c: f"{len(c[0])}seqs-P{c[1]}-flags{c[2]}")
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_order_fp8_with_write_equals_write_then_decode(case, src):
    """pa_decode_order_fp8 (the quantizing write and the item order in one
    launch), then the ordered decode and the merge: caches and outputs
    bit-identical to pa_cache_write_fp8 followed by pa_decode_fp8, from the same
    prior caches; the source rows in f32 as well as the query dtype."""
    lens, P, flags = case
    cfg = custom_config("order-fp8-write", lens, 32, 8, 128, "bf16", 16, seed=14,
                        cache_dtype="fp8", fp8_scales=(2.0 ** -6, 2.0 ** -5))
    wl = Workload(cfg)
    c = cfg
    ks, vs = c.fp8_scales
    ref, got = GpuState(wl), GpuState(wl)
    k = ref.step_k[0].float() if src == "f32" else ref.step_k[0]
    v = ref.step_v[0].float() if src == "f32" else ref.step_v[0]
    _say(f"order_fp8 {len(lens)} seqs P={P} flags={flags} src={src}")
    MB = wl.max_blocks_per_seq
    a = torch.full(ref.q[0].shape, float("nan"), device="cuda")
    pa.cache_write_fp8(k, v, ref.step_slots[0], ref.kc, ref.vc, ks, vs)
    pa.decode_fp8(a, ref.q[0], ref.kc, ref.vc, ref.block_tables, ref.ctx[0], c.attn_scale(), ks,
                  vs, 16, P, None, flags)
    need = pa.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, MB, P, got.kc.dtype, flags)
    ws = torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device="cuda")
    b = torch.full(got.q[0].shape, float("nan"), device="cuda")
    args = (b, got.q[0], got.kc, got.vc, got.block_tables, got.ctx[0], c.attn_scale())
    pa.decode_order_fp8(*args, ks, vs, 16, P, ws, flags, k, v, got.step_slots[0])
    pa.decode_fp8_partitions(*args, ks, vs, 16, P, ws, flags | pa.ORDERED)
    pa.decode_merge(*args, 16, P, ws, flags)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(ref.kc.cpu()), raw_bits(got.kc.cpu())), "key caches differ"
    assert np.array_equal(raw_bits(ref.vc.cpu()), raw_bits(got.vc.cpu())), "value caches differ"
    assert torch.isfinite(b).all()
    assert torch.equal(a, b)
