"""GPU checks of block management: the copy-on-write block copy and the swap
copies (bit-exact against copies of the same bytes on the host), and the
whole protocol -- the host block manager handing out slots, sharing prompt
blocks through the prefix cache and forks, asking for copy-on-write copies --
driving cache writes and decode, against the fp64 oracle run on each
sequence's tokens laid out in blocks of its own.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import DTYPE_TORCH, POISON_BITS, raw_bits, token_kv
from tests.gpu_harness import max_abs_err

pytestmark = pytest.mark.gpu

TOL_ABS_HALF = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _random_caches(NB, H, d, bs, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    kshape = pa.key_cache_shape(NB, H, d, bs, dtype)
    vshape = pa.value_cache_shape(NB, H, d, bs)
    esz = torch.tensor([], dtype=dtype).element_size()
    bits = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[esz]
    lo, hi = {1: (0, 256), 2: (-(1 << 15), 1 << 15), 4: (-(1 << 31), 1 << 31)}[esz]
    kc = torch.randint(lo, hi, kshape, generator=g, dtype=torch.int64).to(bits).view(dtype)
    vc = torch.randint(lo, hi, vshape, generator=g, dtype=torch.int64).to(bits).view(dtype)
    return kc, vc


def _pairs(NB, n, seed):
    """n (src, dst) pairs: distinct destinations, none of them a source."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(NB)
    dst = perm[:n]
    src = rng.choice(perm[n:], size=n, replace=True)
    return np.stack([src, dst], 1).astype(np.int32)


def _host_copy(pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    out = pool.copy()
    for s, d in pairs:
        out[d] = pool[s]
    return out


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float8_e4m3fn])
@pytest.mark.parametrize("n", [1, 7, 300])
def test_copy_blocks_bit_exact(dtype, n):
    NB, H, d, bs = 700, 4, 128, 16
    kc, vc = _random_caches(NB, H, d, bs, dtype, seed=n)
    pairs = _pairs(NB, n, seed=n + 1)
    assert (pairs >= 0).all() and (pairs < NB).all()
    _say(f"copy_blocks {dtype} n={n}")
    kd, vd = kc.cuda(), vc.cuda()
    pa.copy_blocks(kd, vd, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(kd.cpu()), _host_copy(raw_bits(kc), pairs))
    assert np.array_equal(raw_bits(vd.cpu()), _host_copy(raw_bits(vc), pairs))


def test_copy_blocks_more_pairs_than_one_grid_row():
    """More pairs than the grid's second dimension holds (65535): the kernel loops."""
    NB, H, d, bs = 140_000, 1, 64, 4
    n = 70_000
    kc, vc = _random_caches(NB, H, d, bs, torch.float8_e4m3fn, seed=5)
    pairs = _pairs(NB, n, seed=6)
    _say(f"copy_blocks n={n}")
    kd, vd = kc.cuda(), vc.cuda()
    pa.copy_blocks(kd, vd, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(kd.cpu()), _host_copy(raw_bits(kc), pairs))
    assert np.array_equal(raw_bits(vd.cpu()), _host_copy(raw_bits(vc), pairs))


def test_swap_round_trip_bit_exact():
    NB, NH, H, d, bs = 64, 32, 2, 128, 16
    kc, vc = _random_caches(NB, H, d, bs, torch.bfloat16, seed=9)
    kd, vd = kc.cuda(), vc.cuda()
    kh = torch.empty((NH,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    vh = torch.empty((NH,) + tuple(vc.shape[1:]), dtype=vc.dtype, pin_memory=True)
    bm = pa.BlockManager(NB, bs, NH)
    bm.add_sequence(1, num_tokens=200)          # 13 blocks
    bm.add_sequence(2, num_tokens=50)
    bt, _ = bm.block_tables([1], 16)
    blocks = bt[0][bt[0] >= 0].astype(np.int64)
    want_k, want_v = raw_bits(kc)[blocks], raw_bits(vc)[blocks]
    _say("swap out / in")
    out = bm.swap_out(1)
    pa.swap_blocks(kh, kd, out)
    pa.swap_blocks(vh, vd, out)
    # another sequence takes the released blocks and overwrites them on the device
    bm.add_sequence(3, num_tokens=16 * 13)
    bt3, _ = bm.block_tables([3], 13)
    idx = torch.from_numpy(bt3[0].astype(np.int64)).cuda()
    kd.index_fill_(0, idx, 0)
    vd.index_fill_(0, idx, 0)
    bm.free(3)
    back = bm.swap_in(1)
    pa.swap_blocks(kd, kh, back)
    pa.swap_blocks(vd, vh, back)
    torch.cuda.synchronize()
    bt1, _ = bm.block_tables([1], 16)
    new_blocks = bt1[0][bt1[0] >= 0].astype(np.int64)
    assert np.array_equal(raw_bits(kd.cpu())[new_blocks], want_k)
    assert np.array_equal(raw_bits(vd.cpu())[new_blocks], want_v)


# ------------------------------------------------------------------ the protocol end to end

def _oracle_decode_logical(seqs_tokens, q, H, d, bs, dtype, seed, scale):
    """The oracle's decode over each sequence's own tokens, written by the oracle's cache
    write into blocks of its own (sequence i in blocks i*MB ..)."""
    B = len(seqs_tokens)
    MB = max(-(-len(t) // bs) for t in seqs_tokens)
    NB = B * MB
    kdt = DTYPE_TORCH[dtype]
    X = 16 // torch.tensor([], dtype=kdt).element_size()
    kc = np.full((NB, H, bs // 4, d // X, 4, X), POISON_BITS[dtype], np.uint16)
    vc = np.full((NB, H, bs // 4, d, 4), POISON_BITS[dtype], np.uint16)
    bt = np.full((B, MB), -1, np.int32)
    for i, toks in enumerate(seqs_tokens):
        L = len(toks)
        nb = -(-L // bs)
        bt[i, :nb] = np.arange(i * MB, i * MB + nb)
        pos = np.arange(L)
        k, v = token_kv(toks, pos, H, d, dtype, seed)
        slots = (bt[i, pos // bs].astype(np.int64) * bs + pos % bs)
        oracle.cache_write(raw_bits(k), raw_bits(v), slots, kc, vc, dtype)
    lens = np.array([len(t) for t in seqs_tokens], np.int32)
    return oracle.decode(raw_bits(q.cpu()), dtype, kc, vc, dtype, bt, lens, scale, threads=8)


@pytest.mark.parametrize("dtype,hq,hkv,bs", [("bf16", 16, 4, 16), ("f16", 8, 8, 8)])
def test_block_manager_drives_shared_decode(dtype, hq, hkv, bs):
    """Prefix-cache hits, forks with copy-on-write, and a fresh sequence, over several
    decode steps: every step's attention equals the oracle's on the logical sequences."""
    d, seed, NB = 128, 77, 256
    scale = float(np.float32(1.0 / np.sqrt(d)))
    kdt = DTYPE_TORCH[dtype]
    rng = np.random.default_rng(31)
    kc = torch.full(pa.key_cache_shape(NB, hkv, d, bs, kdt), float("nan"), dtype=kdt,
                    device="cuda")
    vc = torch.full(pa.value_cache_shape(NB, hkv, d, bs), float("nan"), dtype=kdt,
                    device="cuda")
    bm = pa.BlockManager(NB, bs, prefix_caching=True)
    sys_prompt = [int(t) for t in rng.integers(0, 1000, size=2 * bs + bs // 2)]
    prompts = {
        0: sys_prompt + [int(t) for t in rng.integers(0, 1000, size=30)],
        1: sys_prompt + [5, 6, 7],
        2: sys_prompt[:bs] + [int(t) for t in rng.integers(0, 1000, size=bs + 3)],
        3: [int(t) for t in rng.integers(0, 1000, size=5 * bs + 1)],
    }
    tokens: dict[int, list[int]] = {}
    hits = {}
    for sid, toks in prompts.items():
        cached = bm.add_sequence(sid, toks)
        hits[sid] = cached
        n = len(toks)
        if n > cached:
            slots = bm.slots(sid, cached, n - cached)
            k, v = token_kv(toks[cached:], range(cached, n), hkv, d, dtype, seed)
            pa.cache_write(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kc, vc)
        bm.mark_computed(sid)
        tokens[sid] = list(toks)
    assert hits == {0: 0, 1: 2 * bs, 2: bs, 3: 0}
    bm.fork(1, 4)          # a second sample of sequence 1: shares its partial last block
    bm.fork(0, 5)
    tokens[4] = list(tokens[1])
    tokens[5] = list(tokens[0])
    order = [0, 1, 2, 3, 4, 5]
    total_copies = 0
    for step in range(2 * bs + 3):
        new = [int(t) for t in rng.integers(0, 1000, size=len(order))]
        slots, copies = bm.append(order, new)
        total_copies += copies.shape[0]
        if copies.shape[0]:
            assert (copies >= 0).all() and (copies < NB).all()
            pa.copy_blocks(kc, vc, torch.from_numpy(copies).cuda())
        pos = [len(tokens[s]) for s in order]
        k = torch.empty((len(order), hkv, d), dtype=kdt)
        v = torch.empty_like(k)
        for i, (t, p) in enumerate(zip(new, pos)):
            ki, vi = token_kv([t], [p], hkv, d, dtype, seed)
            k[i], v[i] = ki[0], vi[0]
        pa.cache_write(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kc, vc)
        for s, t in zip(order, new):
            tokens[s].append(t)
        MB = max(-(-len(tokens[s]) // bs) for s in order)
        bt, lens = bm.block_tables(order, MB)
        assert (bt[bt >= 0] < NB).all()
        q = torch.randn(len(order), hq, d, generator=torch.Generator().manual_seed(step))
        q = q.to(kdt)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        pa.decode(out, q.cuda(), kc, vc, torch.from_numpy(bt).cuda(),
                  torch.from_numpy(lens).cuda(), scale, bs)
        torch.cuda.synchronize()
        ref = _oracle_decode_logical([tokens[s] for s in order], q, hkv, d, bs, dtype, seed,
                                     scale)
        err = max_abs_err(out, ref)
        assert err <= TOL_ABS_HALF, f"step {step}: max abs error {err:.3e}"
        if step % 8 == 0:
            for s in order:
                bm.mark_computed(s)
    # forks 4 (of 1) and 5 (of 0) each shared a partial last block: one copy each
    assert total_copies == 2
    _say(f"protocol {dtype}: hits {hits}, copies {total_copies}")
