"""The opt-in id checks (pa_check_tables, pa_check_slots) on the GPU, and what
the hot kernels do with the out-of-contract ids the checks flag.

Every out-of-contract id used here is one the kernels' own guards keep in
bounds: block ids of a context are clamped into [0, num_blocks), context
lengths are cut to what the table addresses, slots past the pool are dropped
(all memory accesses stay inside the caches and tables)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import WORKLOADS, Workload, custom_config, raw_bits
from tests.gpu_harness import GpuState

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _word():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _tables_status(bt, ctx, NB, bs):
    w = _word()
    pa.check_tables(bt, ctx, NB, bs, w)
    torch.cuda.synchronize()
    return int(w.item())


def _slots_status(slots, NB, bs):
    w = _word()
    pa.check_slots(slots, NB, bs, w)
    torch.cuda.synchronize()
    return int(w.item())


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_clean_workloads_leave_the_word_zero(cid):
    """The five workloads' tables (-1 past each context), lengths and slots
    (prior context and every step) are within contract."""
    wl = Workload(WORKLOADS[cid])
    c = wl.cfg
    bt = torch.from_numpy(wl.block_tables).cuda()
    for s in range(c.steps):
        ctx = torch.from_numpy(wl.context_lens(s)).cuda()
        assert _tables_status(bt, ctx, wl.num_blocks, c.block_size) == 0
        assert _slots_status(torch.from_numpy(wl.step_slots(s)).cuda(), wl.num_blocks,
                             c.block_size) == 0
    prior = np.concatenate([wl.prior_slots(b) for b in range(min(c.num_seqs, 8))])
    assert _slots_status(torch.from_numpy(prior).cuda(), wl.num_blocks, c.block_size) == 0


def test_each_kind_of_violation_sets_exactly_its_bit():
    rng = np.random.default_rng(3)
    B, MB, bs, NB = 70, 9, 16, 200
    lens = rng.integers(1, MB * bs + 1, size=B).astype(np.int32)
    bt = np.full((B, MB), -1, np.int32)
    for b in range(B):
        n = -(-int(lens[b]) // bs)
        bt[b, :n] = rng.integers(0, NB, size=n)
    def run(bt_, lens_):
        return _tables_status(torch.from_numpy(bt_).cuda(), torch.from_numpy(lens_).cuda(), NB,
                              bs)
    assert run(bt, lens) == 0
    # entries past a context may hold anything
    bt2 = bt.copy()
    b = int(np.argmin(lens))
    bt2[b, -(-int(lens[b]) // bs):] = 10 ** 6
    assert run(bt2, lens) == 0
    # an entry inside a context outside the pool: high, and negative
    for bad in (NB, 10 ** 6, -1, -(2 ** 31)):
        bt3 = bt.copy()
        bt3[b, 0] = bad
        assert run(bt3, lens) == pa.CHECK_BLOCK_ID, bad
    # a context longer than the table addresses (its blocks are valid)
    bt4 = np.tile(np.arange(MB, dtype=np.int32), (B, 1))
    l4 = lens.copy()
    l4[5] = MB * bs + 1
    assert run(bt4, l4) == pa.CHECK_CONTEXT_LEN
    l4[5] = -3
    assert run(bt4, l4) == pa.CHECK_CONTEXT_LEN
    # both at once
    bt4[7, 0] = NB
    assert run(bt4, l4) == pa.CHECK_CONTEXT_LEN | pa.CHECK_BLOCK_ID
    # slots: negative is padding, the last slot is fine, one past the pool is not
    slots = torch.tensor([-1, 0, NB * bs - 1, 5], dtype=torch.int64, device="cuda")
    assert _slots_status(slots, NB, bs) == 0
    slots[3] = NB * bs
    assert _slots_status(slots, NB, bs) == pa.CHECK_SLOT
    # the word accumulates: a later clean check leaves earlier bits
    w = _word()
    pa.check_slots(slots, NB, bs, w)
    pa.check_slots(slots[:3].contiguous(), NB, bs, w)
    torch.cuda.synchronize()
    assert int(w.item()) == pa.CHECK_SLOT


@pytest.mark.parametrize("kernel", [pa.FORCE_VALU, pa.FORCE_MFMA])
@pytest.mark.parametrize("partition", [0, 32])
def test_decode_clamps_what_the_check_flags(kernel, partition):
    """A context block id past the pool is flagged, and the decode reads the
    pool's last block in its place: bit-identical to the table holding
    num_blocks - 1 there."""
    cfg = custom_config("clamp", [40, 100, 3], 8, 2, 128, "bf16", 16, seed=31)
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    NB = wl.num_blocks
    # the pool's last block (where the clamp lands) holds finite data: a copy of a used block
    src = int(gs.block_tables[0, 0])
    gs.kc[NB - 1] = gs.kc[src]
    gs.vc[NB - 1] = gs.vc[src]
    bad = gs.block_tables.clone()
    bad[1, 2] = NB + 5
    ref_tab = gs.block_tables.clone()
    ref_tab[1, 2] = NB - 1
    assert _tables_status(bad, gs.ctx[0], NB, 16) == pa.CHECK_BLOCK_ID
    outs = []
    for tab in (bad, ref_tab):
        out = torch.full(gs.q[0].shape, float("nan"), device="cuda")
        pa.decode(out, gs.q[0], gs.kc, gs.vc, tab, gs.ctx[0], cfg.attn_scale(), 16, partition,
                  flags=kernel)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0][[0, 2]], gs.decode(0, flags=kernel, partition_size=partition)[[0, 2]])


def test_cache_write_drops_what_the_check_flags():
    """A slot past the pool is flagged, and the write skips that token: the
    pools equal a write of the other tokens alone."""
    H, d, bs, NB, T = 2, 128, 16, 6, 5
    g = torch.Generator().manual_seed(9)
    k = torch.randn(T, H, d, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(T, H, d, generator=g).to(torch.bfloat16).cuda()
    slots = torch.tensor([3, NB * bs, 17, NB * bs + 40, 90], dtype=torch.int64, device="cuda")
    assert _slots_status(slots, NB, bs) == pa.CHECK_SLOT
    pools = []
    for sl, kk, vv in ((slots, k, v), (slots[[0, 2, 4]].contiguous(), k[[0, 2, 4]].contiguous(),
                                       v[[0, 2, 4]].contiguous())):
        kc = torch.zeros(pa.key_cache_shape(NB, H, d, bs, torch.bfloat16), dtype=torch.bfloat16,
                         device="cuda")
        vc = torch.zeros(pa.value_cache_shape(NB, H, d, bs), dtype=torch.bfloat16, device="cuda")
        pa.cache_write(kk, vv, sl, kc, vc)
        pools.append((kc, vc))
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(pools[0][0].cpu()), raw_bits(pools[1][0].cpu()))
    assert np.array_equal(raw_bits(pools[0][1].cpu()), raw_bits(pools[1][1].cpu()))
