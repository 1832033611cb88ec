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
