"""The seeded input generator against the input recipe it states (CPU): the five decode
batches' shapes and length distributions, the shuffled block pool and its tables, the
slots of the prior context and of each step's new token, the value distributions and
the determinism of every stream."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from pagedattention_kv_cache_amd.workloads import (WORKLOADS, Workload, config3_long_first,
                                                   custom_config)

SHAPES = {  # sequences, q heads, kv heads, head_dim, dtype, block size, steps
    1: (4, 4, 4, 64, "f32", 16, 1),
    2: (64, 32, 32, 128, "f16", 16, 1),
    3: (32, 40, 40, 128, "f16", 16, 1),
    4: (256, 32, 8, 128, "bf16", 16, 1),
    5: (64, 64, 8, 128, "bf16", 32, 8),
}


@pytest.mark.parametrize("cid", sorted(SHAPES))
def test_shapes(cid):
    c = WORKLOADS[cid]
    assert (c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, c.dtype, c.block_size,
            c.steps) == SHAPES[cid]


def test_lengths():
    assert Workload(WORKLOADS[1]).lens0.tolist() == [1, 17, 64, 200]
    l2 = Workload(WORKLOADS[2]).lens0
    assert l2.min() >= 128 and l2.max() <= 2048
    l3 = Workload(WORKLOADS[3]).lens0
    assert l3[-1] == 4096 and l3[:-1].min() >= 16 and l3[:-1].max() <= 256
    assert WORKLOADS[3].partition_size == 512
    lf = Workload(config3_long_first()).lens0
    assert lf[0] == 4096 and (lf[1:] <= 256).all()
    l4 = Workload(WORKLOADS[4]).lens0
    assert l4.min() >= 1 and l4.max() <= 8192
    # log-lengths of a lognormal(ln 1024, 1): median near ln 1024, spread near 1 (256 draws;
    # the clip at 8192 only shortens the upper tail)
    assert abs(np.median(np.log(l4)) - math.log(1024)) < 0.25
    assert 0.8 < np.std(np.log(l4)) < 1.2
    l5 = Workload(WORKLOADS[5]).lens0
    assert l5.min() >= 4096 and l5.max() <= 32768


@pytest.mark.parametrize("cid", sorted(SHAPES))
def test_block_pool_and_tables(cid):
    """Each sequence owns ceil(L_final / bs) distinct blocks of a shuffled pool of
    ceil(1.25 x the blocks needed) (64 for the first batch), no block is shared, and the
    tables hold -1 past each sequence's last block."""
    wl = Workload(WORKLOADS[cid])
    c = wl.cfg
    nblk = -(-wl.final_lens // c.block_size)
    need = int(nblk.sum())
    assert wl.num_blocks == (64 if cid == 1 else math.ceil(1.25 * need))
    bt = wl.block_tables
    assert bt.dtype == np.int32 and bt.shape == (c.num_seqs, int(nblk.max()))
    used = []
    for b in range(c.num_seqs):
        row = bt[b]
        assert (row[:nblk[b]] >= 0).all() and (row[:nblk[b]] < wl.num_blocks).all()
        assert (row[nblk[b]:] == -1).all()
        used.append(row[:nblk[b]])
    used = np.concatenate(used)
    assert np.unique(used).size == used.size == need
    assert (wl.final_lens == wl.lens0 + c.steps - 1).all()


@pytest.mark.parametrize("cid", [1, 3, 5])
def test_slots(cid):
    """Slot of position p of sequence b: table[b][p // bs] * bs + p % bs; the prior context
    is positions 0 .. L0 - 2, step s writes position L0 - 1 + s."""
    wl = Workload(WORKLOADS[cid])
    c = wl.cfg
    bs = c.block_size
    for b in range(min(c.num_seqs, 6)):
        L0 = int(wl.lens0[b])
        pos = np.arange(L0 - 1)
        expect = wl.block_tables[b][pos // bs].astype(np.int64) * bs + pos % bs
        assert np.array_equal(wl.prior_slots(b), expect)
    for s in range(c.steps):
        slots = wl.step_slots(s)
        for b in range(c.num_seqs):
            p = int(wl.lens0[b]) - 1 + s
            assert slots[b] == int(wl.block_tables[b][p // bs]) * bs + p % bs
    assert np.unique(np.concatenate([wl.step_slots(s) for s in range(c.steps)])).size == \
        c.steps * c.num_seqs


def test_values():
    """q, K and V are N(0, 1) rounded to the storage dtype; the GQA batch's keys are
    scaled by 0.5 before rounding."""
    wl = Workload(WORKLOADS[4])
    q = wl.queries()
    assert q.dtype == torch.bfloat16 and q.shape == (1, 256, 32, 128)
    k, v = wl.prior_kv(int(np.argmax(wl.lens0)))
    assert k.dtype == v.dtype == torch.bfloat16
    assert abs(float(k.float().std()) - 0.5) < 0.01 and abs(float(v.float().std()) - 1.0) < 0.02
    assert abs(float(q.float().mean())) < 0.01 and abs(float(q.float().std()) - 1.0) < 0.01
    # rounding to bfloat16 is round-to-nearest-even of the fp32 draw
    cfg = custom_config("r", [300], 2, 2, 64, "bf16", 16, seed=5)
    k32 = np.random.Generator(np.random.PCG64(Workload(cfg)._seq_ss[0])).standard_normal(
        (299, 2, 64), dtype=np.float32)
    assert torch.equal(Workload(cfg).prior_kv(0)[0], torch.from_numpy(k32).to(torch.bfloat16))


def test_streams_are_deterministic_and_independent():
    a, b = Workload(WORKLOADS[2]), Workload(WORKLOADS[2])
    assert np.array_equal(a.block_tables, b.block_tables)
    assert torch.equal(a.queries(), b.queries())
    assert torch.equal(a.prior_kv(7)[0], b.prior_kv(7)[0])
    sk_a, sv_a = a.step_kv()
    assert torch.equal(sk_a, b.step_kv()[0]) and not torch.equal(sk_a, sv_a)
    # one sequence regenerates alone: its stream does not depend on the others
    assert torch.equal(a.prior_kv(7)[1], Workload(WORKLOADS[2]).prior_kv(7)[1])
    assert not torch.equal(a.prior_kv(7)[0][:50], a.prior_kv(8)[0][:50])
