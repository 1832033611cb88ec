"""Pins for the fp64 CPU oracle (CPU only).

Each test checks the oracle against something other than itself: numpy/torch
conversions, a hand-worked layout fixture, contiguous brute-force attention with
scipy's softmax, mpmath at 50 digits, and the invariants the pages fix
(exact attention regardless of paging -- "vLLM: Easy, Fast, and Cheap LLM
Serving with PagedAttention" thread, FlashAttention vs PagedAttention comments;
block-level storage -- "vLLM Project Update" talk, PagedAttention recap).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from pagedattention_kv_cache_amd.workloads import WORKLOADS, Workload, custom_config, raw_bits
from tests.paged_host import (OracleState, key_pool_shape, key_rows, logical_kv, offset_major,
                               poisoned_pool, value_pool_shape, value_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, scope="module")
def _built(oracle_lib):
    return oracle_lib


# ---------------------------------------------------------------- decoders

def test_f16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bits(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bits(bits, "bf16")
    ref_torch = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        ref_np = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref_np)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(np.isnan(ref_torch), nan)
    assert np.array_equal(got[~nan], ref_np[~nan])
    assert np.array_equal(got[~nan], ref_torch[~nan])


def test_f32_decoder_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x807FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000,
                        0xFF800000, 0x7FC00000, 0x3F800000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    got = oracle.decode_bits(bits, "f32")
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- cache write

def _read_layout_fixture():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "cache_write_layout.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            kind, *vals = line.split()
            if kind == "CASE":
                name, dtype, nb, h, bs, d, *slots = vals
                cur = dict(dtype=dtype, NB=int(nb), H=int(h), bs=int(bs), d=int(d),
                           slots=[int(x) for x in slots], K=[], V=[])
                cases.append(cur)
            else:
                cur[kind].append(tuple(int(x) for x in vals))
    return cases


def test_cache_write_hand_worked_layout():
    cases = _read_layout_fixture()
    assert [c["dtype"] for c in cases] == ["f32", "bf16"]
    for cs in cases:
        NB, H, bs, d, T = cs["NB"], cs["H"], cs["bs"], cs["d"], len(cs["slots"])
        X = 4 if cs["dtype"] == "f32" else 8
        i = np.arange(T)[:, None, None]
        h = np.arange(H)[None, :, None]
        e = np.arange(d)[None, None, :]
        k = (100 * i + 10 * h + e + 1).astype(np.float32)
        ek = np.zeros((NB, H, bs // 4, d // X, 4, X), np.float32)
        ev = np.zeros((NB, H, bs // 4, d, 4), np.float32)
        for blk, hh, quad, ch, row, lane, val in cs["K"]:
            ek[blk, hh, quad, ch, row, lane] = val
        for blk, hh, quad, ee, row, val in cs["V"]:
            ev[blk, hh, quad, ee, row] = val
        if cs["dtype"] == "f32":
            kb, vb = k.view(np.uint32), (-k).view(np.uint32)
            kc = np.zeros(ek.shape, np.uint32)
            vc = np.zeros(ev.shape, np.uint32)
            exp_k, exp_v = ek.view(np.uint32), ev.view(np.uint32)
        else:
            kb = raw_bits(torch.from_numpy(k).to(torch.bfloat16))
            vb = raw_bits(torch.from_numpy(-k).to(torch.bfloat16))
            kc = np.zeros(ek.shape, np.uint16)
            vc = np.zeros(ev.shape, np.uint16)
            exp_k = raw_bits(torch.from_numpy(ek).to(torch.bfloat16))
            exp_v = raw_bits(torch.from_numpy(ev).to(torch.bfloat16))
        oracle.cache_write(kb, vb, np.array(cs["slots"]), kc, vc, cs["dtype"])
        assert np.array_equal(kc, exp_k), cs["dtype"]
        assert np.array_equal(vc, exp_v), cs["dtype"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_cache_write_roundtrip_and_poison(dtype):
    """Writing a sequence through its slots and reading positions back through
    the block table returns the original rows bit-for-bit; every slot not
    written keeps its poison; negative slots are skipped."""
    cfg = custom_config("rt", [37, 5, 64], 2, 2, 8, dtype, 8, seed=11)
    wl = Workload(cfg)
    st = OracleState(wl)
    st.write_step(0)
    written = np.zeros((wl.num_blocks, cfg.block_size), bool)
    for b in range(cfg.num_seqs):
        k, v = wl.prior_kv(b)
        sk, sv = wl.step_kv()
        kb = raw_bits(torch.cat([k, sk[0, b:b + 1]]))
        vb = raw_bits(torch.cat([v, sv[0, b:b + 1]]))
        for pos in range(wl.lens0[b]):
            blk = wl.block_tables[b, pos // cfg.block_size]
            off = pos % cfg.block_size
            assert np.array_equal(key_rows(st.kc, blk, off), kb[pos])
            assert np.array_equal(value_rows(st.vc, blk, off), vb[pos])
            written[blk, off] = True
    # pools as [block][offset][...]: slots never written keep their poison
    kt, vt = offset_major(st.kc, True), offset_major(st.vc, False)
    assert np.array_equal(kt[~written], offset_major(poisoned_pool(wl, False), True)[~written])
    assert np.array_equal(vt[~written], offset_major(poisoned_pool(wl, True), False)[~written])
    # skip semantics: all-negative slots leave the pools untouched
    kc0, vc0 = st.kc.copy(), st.vc.copy()
    oracle.cache_write(raw_bits(st.step_k[0]), raw_bits(st.step_v[0]),
                       -np.ones(cfg.num_seqs, np.int64), st.kc, st.vc, dtype)
    assert np.array_equal(kc0, st.kc) and np.array_equal(vc0, st.vc)


def test_cache_write_rejects_out_of_range_slot():
    kc = np.zeros(key_pool_shape(2, 1, 4, 4, "f32"), np.float32)
    vc = np.zeros(value_pool_shape(2, 1, 4, 4), np.float32)
    k = np.ones((1, 1, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.cache_write(k.view(np.uint32), k.view(np.uint32), np.array([8]),
                           kc.view(np.uint32), vc.view(np.uint32), "f32")


# ---------------------------------------------------------------- decode

def _brute(wl: Workload, step: int) -> np.ndarray:
    """Contiguous attention with scipy's softmax on torch-decoded float64 values."""
    c = wl.cfg
    q = wl.queries()[step].to(torch.float64).numpy()
    out = np.empty((c.num_seqs, c.num_q_heads, c.head_dim))
    scale = np.float64(np.float32(c.attn_scale()))
    for b in range(c.num_seqs):
        K, V = logical_kv(wl, b, step)
        for hq in range(c.num_q_heads):
            hk = hq // c.group
            w = scipy.special.softmax(scale * (K[:, hk, :] @ q[b, hq]))
            out[b, hq] = w @ V[:, hk, :]
    return out


@pytest.mark.parametrize("dtype,d,bs,hq,hkv,lens,seed", [
    ("f32", 8, 4, 2, 2, [1, 5, 9], 21),
    ("f32", 64, 16, 4, 4, [1, 17, 64, 70], 22),
    ("f16", 8, 8, 4, 2, [3, 33, 70], 23),
    ("bf16", 64, 4, 4, 1, [2, 40, 64], 24),
    ("bf16", 8, 16, 8, 2, [16, 17, 48], 25),
    ("f16", 64, 4, 3, 3, [69], 26),
])
def test_decode_matches_brute_force(dtype, d, bs, hq, hkv, lens, seed):
    cfg = custom_config("bf", lens, hq, hkv, d, dtype, bs, seed=seed)
    wl = Workload(cfg)
    st = OracleState(wl)
    st.write_step(0)
    got = st.decode(0, threads=2)
    ref = _brute(wl, 0)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel <= 1e-12, rel


def test_decode_multistep_matches_brute_force():
    cfg = custom_config("ms", [5, 31, 16], 4, 2, 8, "bf16", 8, seed=27, steps=3)
    wl = Workload(cfg)
    st = OracleState(wl)
    for s in range(3):
        st.write_step(s)
        got = st.decode(s)
        ref = _brute(wl, s)
        assert np.abs(got - ref).max() / np.abs(ref).max() <= 1e-12


def _paged_from_logical(Ks, Vs, bs, perm_seed, nb_extra=3, dtype="f32"):
    """Page contiguous per-sequence K/V ([L][H][d] raw bits) into a NaN-poisoned
    pool with a random block permutation; return caches and block tables."""
    rng = np.random.default_rng(perm_seed)
    H, d = Ks[0].shape[1], Ks[0].shape[2]
    nblk = [-(-K.shape[0] // bs) for K in Ks]
    NB = sum(nblk) + nb_extra
    perm = rng.permutation(NB)
    bits = np.uint32 if dtype == "f32" else np.uint16
    from pagedattention_kv_cache_amd.workloads import POISON_BITS
    kc = np.full(key_pool_shape(NB, H, d, bs, dtype), POISON_BITS[dtype], bits)
    vc = np.full(value_pool_shape(NB, H, d, bs), POISON_BITS[dtype], bits)
    MB = max(nblk)
    bt = np.full((len(Ks), MB), -1, np.int32)
    off = 0
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        blocks = perm[off:off + nblk[b]]
        off += nblk[b]
        bt[b, :nblk[b]] = blocks
        pos = np.arange(K.shape[0])
        slots = blocks[pos // bs] * bs + pos % bs
        oracle.cache_write(K, V, slots, kc, vc, dtype)
    return kc, vc, bt


def _rand_f32(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_block_permutation_and_block_size_invariance():
    rng = np.random.default_rng(5)
    lens = [1, 7, 33, 64, 65]
    H, d, Hq = 2, 16, 4
    Ks = [_rand_f32(rng, (L, H, d)).view(np.uint32) for L in lens]
    Vs = [_rand_f32(rng, (L, H, d)).view(np.uint32) for L in lens]
    q = _rand_f32(rng, (len(lens), Hq, d)).view(np.uint32)
    cl = np.array(lens, np.int32)
    outs = []
    for bs, ps in [(4, 0), (4, 1), (8, 2), (8, 3), (16, 4), (16, 5), (32, 6), (64, 7)]:
        kc, vc, bt = _paged_from_logical(Ks, Vs, bs, ps)
        outs.append(oracle.decode(q, "f32", kc, vc, "f32", bt, cl, 0.25))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_context_length_one_returns_v_exactly():
    rng = np.random.default_rng(6)
    for dtype in ["f32", "f16", "bf16"]:
        K = [torch.from_numpy(_rand_f32(rng, (1, 2, 8))) for _ in range(3)]
        V = [torch.from_numpy(_rand_f32(rng, (1, 2, 8))) for _ in range(3)]
        if dtype != "f32":
            K = [k.to(getattr(torch, {"f16": "float16", "bf16": "bfloat16"}[dtype])) for k in K]
            V = [v.to(K[0].dtype) for v in V]
        kc, vc, bt = _paged_from_logical([raw_bits(k) for k in K], [raw_bits(v) for v in V], 4, 9,
                                         dtype=dtype)
        q = raw_bits(torch.from_numpy(_rand_f32(rng, (3, 4, 8))).to(K[0].dtype))
        out = oracle.decode(q, dtype, kc, vc, dtype, bt, np.ones(3, np.int32), 0.3)
        for b in range(3):
            for hq in range(4):
                assert np.array_equal(out[b, hq], V[b][0, hq // 2].to(torch.float64).numpy())


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(7)
    L, H, d = 300, 1, 16
    key = _rand_f32(rng, (1, H, d))
    K = np.repeat(key, L, axis=0).view(np.uint32)
    V = _rand_f32(rng, (L, H, d))
    kc, vc, bt = _paged_from_logical([K], [V.view(np.uint32)], 16, 1)
    q = _rand_f32(rng, (1, 2, d)).view(np.uint32)
    out = oracle.decode(q, "f32", kc, vc, "f32", bt, np.array([L], np.int32), 0.7)
    mean = V[:, 0, :].astype(np.float64).mean(axis=0)
    assert np.abs(out[0, 0] - mean).max() <= 1e-14
    assert np.abs(out[0, 1] - mean).max() <= 1e-14


def test_scale_zero_gives_mean_of_v():
    rng = np.random.default_rng(8)
    L, H, d = 77, 2, 8
    K = _rand_f32(rng, (L, H, d)).view(np.uint32)
    V = _rand_f32(rng, (L, H, d))
    kc, vc, bt = _paged_from_logical([K], [V.view(np.uint32)], 8, 2)
    q = _rand_f32(rng, (1, 2, d)).view(np.uint32)
    out = oracle.decode(q, "f32", kc, vc, "f32", bt, np.array([L], np.int32), 0.0)
    for h in range(2):
        assert np.abs(out[0, h] - V[:, h, :].astype(np.float64).mean(axis=0)).max() <= 1e-14


def test_one_hot_probe_returns_target_row():
    rng = np.random.default_rng(9)
    L, H, d = 50, 1, 16
    q = _rand_f32(rng, (1, 1, d))
    scale = 0.125
    c = np.float32(200.0 / (scale * float((q.astype(np.float64) ** 2).sum())) * 1.01)
    V = _rand_f32(rng, (L, H, d))
    for t in [0, 1, 15, 16, 31, 49]:
        K = np.zeros((L, H, d), np.float32)
        K[t, 0] = c * q[0, 0]
        kc, vc, bt = _paged_from_logical([K.view(np.uint32)], [V.view(np.uint32)], 16, t)
        out = oracle.decode(q.view(np.uint32), "f32", kc, vc, "f32", bt,
                            np.array([L], np.int32), scale)
        assert np.array_equal(out[0, 0], V[t, 0].astype(np.float64))


def test_gqa_equals_replicated_mha():
    rng = np.random.default_rng(10)
    lens, Hkv, g, d = [3, 40], 2, 4, 8
    Ks = [_rand_f32(rng, (L, Hkv, d)) for L in lens]
    Vs = [_rand_f32(rng, (L, Hkv, d)) for L in lens]
    q = _rand_f32(rng, (2, Hkv * g, d)).view(np.uint32)
    cl = np.array(lens, np.int32)
    kc, vc, bt = _paged_from_logical([k.view(np.uint32) for k in Ks], [v.view(np.uint32) for v in Vs],
                                     8, 3)
    gqa = oracle.decode(q, "f32", kc, vc, "f32", bt, cl, 0.5)
    Kr = [np.repeat(k, g, axis=1).view(np.uint32) for k in Ks]
    Vr = [np.repeat(v, g, axis=1).view(np.uint32) for v in Vs]
    kc2, vc2, bt2 = _paged_from_logical(Kr, Vr, 8, 4)
    mha = oracle.decode(q, "f32", kc2, vc2, "f32", bt2, cl, 0.5)
    assert np.array_equal(gqa, mha)


def test_two_token_closed_form():
    """L = 2: out = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1."""
    rng = np.random.default_rng(11)
    d = 8
    K = _rand_f32(rng, (2, 1, d))
    V = _rand_f32(rng, (2, 1, d))
    q = _rand_f32(rng, (1, 1, d))
    kc, vc, bt = _paged_from_logical([K.view(np.uint32)], [V.view(np.uint32)], 4, 0)
    out = oracle.decode(q.view(np.uint32), "f32", kc, vc, "f32", bt, np.array([2], np.int32), 0.9)
    # the library and the oracle take scale as fp32
    s = float(np.float32(0.9)) * (K[:, 0, :].astype(np.float64) @ q[0, 0].astype(np.float64))
    ref = (scipy.special.expit(s[0] - s[1]) * V[0, 0].astype(np.float64)
           + scipy.special.expit(s[1] - s[0]) * V[1, 0].astype(np.float64))
    assert np.abs(out[0, 0] - ref).max() <= 1e-15 * 8


def test_oracle_error_against_50_digit_reference():
    """The fp64 oracle's own error on a 4096-token row is far below the parity
    tolerances (1e-5 relative, 2e-3 absolute)."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    rng = np.random.default_rng(12)
    L, d = 4096, 16
    K = _rand_f32(rng, (L, 1, d))
    V = _rand_f32(rng, (L, 1, d))
    q = _rand_f32(rng, (1, 1, d))
    kc, vc, bt = _paged_from_logical([K.view(np.uint32)], [V.view(np.uint32)], 16, 1)
    out = oracle.decode(q.view(np.uint32), "f32", kc, vc, "f32", bt, np.array([L], np.int32), 0.25)
    mp = mpmath.mpf
    qs = [mp(float(x)) for x in q[0, 0]]
    s = [mp("0.25") * mpmath.fsum(qs[e] * mp(float(K[t, 0, e])) for e in range(d)) for t in range(L)]
    m = max(s)
    w = [mpmath.exp(x - m) for x in s]
    z = mpmath.fsum(w)
    ref = np.array([float(mpmath.fsum(w[t] * mp(float(V[t, 0, e])) for t in range(L)) / z)
                    for e in range(d)])
    assert np.abs(out[0, 0] - ref).max() / np.abs(ref).max() <= 1e-12


def test_threads_do_not_change_results():
    wl = Workload(custom_config("thr", [100, 3, 50, 64, 1], 8, 2, 16, "bf16", 16, seed=31))
    st = OracleState(wl)
    st.write_step(0)
    a = st.decode(0, threads=1)
    b = st.decode(0, threads=5)
    assert np.array_equal(a, b)
    rows = np.array([0, 9, 17, 39])
    c = st.decode(0, rows=rows, threads=3)
    flat_a = a.reshape(-1, a.shape[-1])
    flat_c = c.reshape(-1, c.shape[-1])
    assert np.array_equal(flat_c[rows], flat_a[rows])
    assert np.isnan(np.delete(flat_c, rows, axis=0)).all()


def test_decode_rejects_bad_inputs():
    wl = Workload(custom_config("bad", [4, 9], 2, 2, 8, "f32", 4, seed=1))
    st = OracleState(wl)
    st.write_step(0)
    c = wl.cfg
    q = raw_bits(st.q[0])
    with pytest.raises(oracle.OracleError):  # L = 0
        oracle.decode(q, "f32", st.kc, st.vc, "f32", wl.block_tables, np.array([0, 9], np.int32), 1.0)
    with pytest.raises(oracle.OracleError):  # L beyond the table
        oracle.decode(q, "f32", st.kc, st.vc, "f32", wl.block_tables,
                      np.array([4, 4 * wl.max_blocks_per_seq + 1], np.int32), 1.0)
    bt = wl.block_tables.copy()
    bt[1, 1] = -1
    with pytest.raises(oracle.OracleError):  # a block id of -1 inside the context
        oracle.decode(q, "f32", st.kc, st.vc, "f32", bt, wl.context_lens(0), 1.0)
    assert c.num_seqs == 2


def test_config1_end_to_end_against_brute_force():
    wl = Workload(WORKLOADS[1])
    st = OracleState(wl)
    st.write_step(0)
    got = st.decode(0)
    ref = _brute(wl, 0)
    assert np.abs(got - ref).max() / np.abs(ref).max() <= 1e-12
    # poisoned tail slots of the last blocks and unused blocks never leak
    assert np.isfinite(got).all()
    assert math.isclose(wl.cfg.attn_scale(), 0.125)


# ---------------------------------------------------------------- advance step

def test_advance_step_hand_worked():
    """block_size 16; tables: seq0 -> [7, 3], seq1 -> [5, -1], seq2 (padding)."""
    bt = np.array([[7, 3], [5, -1], [9, 9]], np.int32)
    tokens = np.array([11, 12, 13], np.int64)
    pos = np.array([14, 15, 2], np.int64)
    lens = np.array([15, 16, 3], np.int32)
    slots = np.array([0, 0, 0], np.int64)
    oracle.advance_step(2, 16, tokens, np.array([101, 102], np.int64), pos, lens, slots, bt)
    # seq0: position 15 -> block 7, offset 15 -> slot 127; seq1: position 16 ->
    # logical block 1 -> entry -1 -> slot -1; seq2 is padding
    assert tokens.tolist() == [101, 102, 13]
    assert pos.tolist() == [15, 16, 2]
    assert lens.tolist() == [16, 17, 3]
    assert slots.tolist() == [127, -1, -1]
    oracle.advance_step(2, 16, tokens, np.array([7, 8], np.int64), pos, lens, slots, bt)
    # seq0: position 16 -> logical block 1 -> block 3, offset 0 -> slot 48
    assert slots.tolist() == [48, -1, -1] and pos.tolist() == [16, 17, 2]


def test_advance_step_matches_generator_slots():
    """Stepping the oracle's state reproduces the generator's per-step slots and
    context lengths (two independent derivations of the same positions)."""
    wl = Workload(custom_config("adv", [1, 15, 16, 17, 31, 32, 200], 4, 2, 8, "bf16", 16,
                                seed=3, steps=8))
    st = wl.initial_state()
    sampled = wl.sampled_tokens()
    assert sampled.shape == (8, 7) and sampled.min() >= 0
    for s in range(8):
        assert np.array_equal(st["slot_mapping"], wl.step_slots(s))
        assert np.array_equal(st["seq_lens"], wl.context_lens(s))
        oracle.advance_step(7, 16, st["input_tokens"], sampled[s], st["input_positions"],
                            st["seq_lens"], st["slot_mapping"], wl.block_tables)
        assert np.array_equal(st["input_tokens"], sampled[s])

# ------------------------------------------------------------------ E4M3 (8-bit float) caches

def test_fp8_decoder_all_codes_match_torch():
    """All 256 E4M3 patterns decode to torch's float8_e4m3fn values (NaN where it has NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_bits(codes, "fp8")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_fp8_encoder_matches_torch_in_range():
    """Inside the finite range (|y| < 448) the encoder agrees with torch's conversion on
    random magnitudes over the whole exponent range and on every midpoint of the grid."""
    rng = np.random.default_rng(8)
    mag = np.exp2(rng.uniform(-13, np.log2(447.9), 100000)).astype(np.float32)
    y = mag * rng.choice(np.array([-1, 1], np.float32), mag.size)
    grid = np.unique(np.abs(oracle.decode_bits(np.arange(127, dtype=np.uint8), "fp8")))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids, grid.astype(np.float32)])
    y = y[np.abs(y) < 448]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8(y), ref)


@pytest.mark.parametrize("y,code", [
    (0.0, 0x00), (-0.0, 0x80), (448.0, 0x7E), (-448.0, 0xFE),
    (449.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (float("inf"), 0x7E), (float("-inf"), 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02),
    (7 * 2.0 ** -10, 0x04), (15 * 2.0 ** -10, 0x08), (1.0625, 0x38), (1.1875, 0x3A),
    (240.0, 0x77), (256.0, 0x78), (-0.001, 0x80 | 0x01),
])
def test_fp8_encoder_definition_cases(y, code):
    """Ties to even (normal and subnormal), the subnormal/normal boundary, signed zero and
    saturation of everything beyond 448, infinities included."""
    assert int(oracle.encode_fp8(np.array([y], np.float32))[0]) == code


def test_fp8_encoder_nan_keeps_sign():
    y = np.array([np.nan, -np.nan], np.float32)
    assert oracle.encode_fp8(y).tolist() == [0x7F, 0xFF]


def _fp8_fixture():
    rows = []
    scales = None
    for line in open(os.path.join(GOLDEN, "cache_write_fp8.txt")):
        f = line.split()
        if not f or f[0] == "#":
            continue
        if f[0] == "scales":
            scales = (float(f[1]), float(f[2]))
        else:
            rows.append((int(f[1]), float(f[2]), int(f[4], 16), float(f[5]), int(f[7], 16)))
    return scales, rows


def test_fp8_cache_write_hand_worked_fixture():
    (ks, vs), rows = _fp8_fixture()
    k = np.zeros((2, 1, 16), np.float32)
    v = np.zeros((2, 1, 16), np.float32)
    for e, kv, _, vv, _ in rows:
        k[0, 0, e] = kv
        v[0, 0, e] = vv
    k[1] = 7.0  # padding token (slot -1)
    v[1] = 7.0
    kb = raw_bits(torch.from_numpy(k).to(torch.bfloat16))
    vb = raw_bits(torch.from_numpy(v).to(torch.bfloat16))
    assert np.array_equal(torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).float().numpy(), k)
    kc = np.full((2, 1, 1, 1, 4, 16), 0x55, np.uint8)
    vc = np.full((2, 1, 1, 16, 4), 0x55, np.uint8)
    oracle.cache_write_fp8(kb, vb, np.array([6, -1], np.int64), kc, vc, "bf16", ks, vs)
    ek = np.full(128, 0x55, np.uint8)
    ev = np.full(128, 0x55, np.uint8)
    for e, _, kcode, _, vcode in rows:
        ek[96 + e] = kcode
        ev[66 + 4 * e] = vcode
    assert np.array_equal(kc.reshape(-1), ek)
    assert np.array_equal(vc.reshape(-1), ev)


def test_fp8_decode_equals_decode_of_dequantized_f32_caches():
    """Decoding E4M3 caches with scales equals decoding f32 caches that hold
    code value * scale (exact for power-of-two scales): same doubles, same result."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, d, bs, NB = 3, 4, 2, 32, 8, 20
    lens = np.array([1, 17, 40], np.int32)
    MB = 5
    bt = rng.permutation(NB)[:B * MB].reshape(B, MB).astype(np.int32)
    codes_k = rng.integers(0, 256, size=(NB, Hkv, bs // 4, d // 16, 4, 16), dtype=np.uint8)
    codes_v = rng.integers(0, 256, size=(NB, Hkv, bs // 4, d, 4), dtype=np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x3C  # no NaN patterns in the context
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x3C
    ks, vs = 0.25, 8.0
    fk = (oracle.decode_bits(codes_k, "fp8") * ks).astype(np.float32)
    fv = (oracle.decode_bits(codes_v, "fp8") * vs).astype(np.float32)
    kc32 = np.ascontiguousarray(fk.reshape(NB, Hkv, bs // 4, d // 16, 4, 4, 4)
                                .transpose(0, 1, 2, 3, 5, 4, 6)
                                .reshape(NB, Hkv, bs // 4, d // 4, 4, 4)).view(np.uint32)
    vc32 = np.ascontiguousarray(fv).view(np.uint32)
    q = raw_bits(torch.randn(B, Hq, d, generator=torch.Generator().manual_seed(3)))
    ref = oracle.decode(q, "f32", kc32, vc32, "f32", bt, lens, 0.125)
    got = oracle.decode(q, "f32", codes_k, codes_v, "fp8", bt, lens, 0.125, k_scale=ks, v_scale=vs)
    assert np.array_equal(got, ref)

# ------------------------------------------------------------------ multi-query decode

def _mq_case(seed, B, Q, Hq, Hkv, d, bs, lens, dtype="f32"):
    rng = np.random.default_rng(seed)
    MB = max(-(-L // bs) for L in lens) + 1
    NB = B * MB + 3
    perm = rng.permutation(NB)
    bt = np.full((B, MB), -1, np.int32)
    X = 16 // (4 if dtype == "f32" else 2)
    kc = np.zeros((NB, Hkv, bs // 4, d // X, 4, X), np.float32 if dtype == "f32" else np.uint16)
    vc = np.zeros((NB, Hkv, bs // 4, d, 4), kc.dtype)
    K, V = [], []
    for b, L in enumerate(lens):
        nb = -(-L // bs)
        bt[b, :nb] = perm[b * MB:b * MB + nb]
        k = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
        slots = bt[b, np.arange(L) // bs].astype(np.int64) * bs + np.arange(L) % bs
        oracle.cache_write(k.view(np.uint32), v.view(np.uint32), slots, kc.view(np.uint32),
                           vc.view(np.uint32), "f32")
        K.append(k.astype(np.float64))
        V.append(v.astype(np.float64))
    q = rng.standard_normal((B, Q, Hq, d)).astype(np.float32)
    return q, kc.view(np.uint32), vc.view(np.uint32), bt, np.array(lens, np.int32), K, V


@pytest.mark.parametrize("Q,Hq,Hkv", [(1, 4, 2), (3, 4, 2), (4, 2, 2), (7, 8, 1)])
def test_multi_query_decode_brute_force(Q, Hq, Hkv):
    """Query i of each sequence attends causally to positions 0 .. L - Q + i: contiguous
    numpy softmax per (sequence, query, head) on the same K/V."""
    lens = [Q, Q + 5, 37, 70]
    d, bs = 16, 8
    q, kc, vc, bt, cl, K, V = _mq_case(11 + Q, len(lens), Q, Hq, Hkv, d, bs, lens)
    scale = float(np.float32(0.37))
    got = oracle.decode_mq(q.view(np.uint32), "f32", kc, vc, "f32", bt, cl, scale)
    g = Hq // Hkv
    for b, L in enumerate(lens):
        for i in range(Q):
            n = L - Q + i + 1
            for hq in range(Hq):
                s = K[b][:n, hq // g] @ q[b, i, hq].astype(np.float64) * scale
                w = scipy.special.softmax(s)
                ref = w @ V[b][:n, hq // g]
                assert np.allclose(got[b, i, hq], ref, rtol=1e-12, atol=1e-12)


def test_multi_query_decode_equals_single_queries_on_truncated_contexts():
    """Row (b, i) of a Q-query decode is the single-query decode of sequence b with context
    length L - Q + i + 1 (the oracle's plain entry, bit for bit)."""
    Q, Hq, Hkv, d, bs = 4, 4, 2, 16, 8
    lens = [4, 9, 33]
    q, kc, vc, bt, cl, _, _ = _mq_case(5, len(lens), Q, Hq, Hkv, d, bs, lens)
    got = oracle.decode_mq(q.view(np.uint32), "f32", kc, vc, "f32", bt, cl, 0.25)
    for i in range(Q):
        single = oracle.decode(np.ascontiguousarray(q[:, i]).view(np.uint32), "f32", kc, vc,
                               "f32", bt, cl - Q + i + 1, 0.25)
        assert np.array_equal(got[:, i], single)


def test_multi_query_decode_rejects_contexts_shorter_than_the_queries():
    q, kc, vc, bt, cl, _, _ = _mq_case(6, 2, 3, 2, 2, 16, 8, [3, 10])
    with pytest.raises(oracle.OracleError):
        oracle.decode_mq(q[:, :3].copy().view(np.uint32)[:, :, :, :], "f32", kc, vc, "f32", bt,
                         np.array([2, 10], np.int32), 0.25)

