"""GPU parity for E4M3 (8-bit float) KV caches: the quantizing cache write and
decode over E4M3 caches, through the C ABI, against the fp64 oracle.

Bars: the quantizing write is bit-exact (whole NaN-poisoned pools compared,
every element's E4M3 code equal); decode is within 2e-3 max absolute error of
the oracle computing in fp64 on the same E4M3 codes and scales.  The GPU
widens every E4M3 value exactly (to fp32 on the vector ALUs, to bfloat16 on
the matrix cores: E4M3 values have at most 4 significant bits), so its
arithmetic is the 16-bit path's arithmetic on exact inputs and the 16-bit
tolerance applies unchanged.  Invariants (L = 1, one-hot probe) are
bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import (FP8_WORKLOADS, Workload, custom_config,
                                                   raw_bits)
from tests.gpu_harness import (GpuState, assert_rejected, decode_kv, max_abs_err,
                               oracle_state_empty)

pytestmark = pytest.mark.gpu

TOL_ABS = 2e-3
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


def _pools_equal(gs: GpuState, st) -> None:
    assert np.array_equal(raw_bits(gs.kc.cpu()), st.kc), "key pool differs from the oracle's"
    assert np.array_equal(raw_bits(gs.vc.cpu()), st.vc), "value pool differs from the oracle's"


# ------------------------------------------------------------------ quantizing write

@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bs", [8, 16, 64])
def test_cache_write_fp8_bit_exact(src, d, bs):
    """Scales that are not powers of two, so x / scale rounds: both sides must take the
    correctly rounded fp32 quotient and the same E4M3 rounding."""
    cfg = custom_config(f"cw8-{src}-{d}-{bs}", [1, bs - 1, bs, 3 * bs + 5], 2, 2, d, src, bs,
                        seed=300 + d + bs, steps=2, cache_dtype="fp8",
                        fp8_scales=(0.0137, 0.0291))
    wl = Workload(cfg)
    _say(f"fp8 cache write src={src} d={d} bs={bs}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    for s in range(cfg.steps):
        gs.write_step(s)
        st.write_step(s)
    torch.cuda.synchronize()
    _pools_equal(gs, st)


def test_cache_write_fp8_special_values():
    """Saturation (beyond 448, infinities), subnormal ties, signed zeros and NaN, from an
    fp32 source, through the whole quantizing path."""
    H, d, bs, NB = 1, 64, 16, 4
    specials = np.array([0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 1e30, np.inf, -np.inf, np.nan,
                         2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 15 * 2.0 ** -10,
                         1.0625, 1.1875, 240.0, 256.0, -0.001], np.float32)
    rng = np.random.default_rng(4)
    k = np.resize(specials, (3, H, d)).astype(np.float32)
    v = (rng.standard_normal((3, H, d)) * 300).astype(np.float32)
    slots = np.array([5, 17, 40], np.int64)
    kc_o = np.full((NB, H, bs // 4, d // 16, 4, 16), 0x7F, np.uint8)
    vc_o = np.full((NB, H, bs // 4, d, 4), 0x7F, np.uint8)
    oracle.cache_write_fp8(k.view(np.uint32), v.view(np.uint32), slots, kc_o, vc_o, "f32", 1.0,
                           0.5)
    kc = torch.full(kc_o.shape, 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    vc = torch.full(vc_o.shape, 0x7F, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    pa.cache_write_fp8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.from_numpy(slots).cuda(), kc, vc, 1.0, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(kc.cpu()), kc_o)
    assert np.array_equal(raw_bits(vc.cpu()), vc_o)


# ------------------------------------------------------------------ decode parity

SMALL = [
    # q dtype, d, bs, Hq, Hkv, lens
    ("bf16", 128, 16, 8, 2, [5, 16, 100, 1000, 1500]),
    ("bf16", 128, 32, 16, 2, [1, 64, 777, 2049]),
    ("bf16", 64, 64, 12, 4, [63, 64, 65, 700]),
    ("bf16", 128, 8, 7, 1, [9, 250, 600]),
    ("f16", 128, 16, 8, 8, [1, 15, 16, 17, 300, 513]),
    ("f16", 64, 32, 6, 2, [2, 31, 33, 400]),
    ("f32", 128, 16, 4, 2, [3, 40, 129]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"q{c[0]}-d{c[1]}-bs{c[2]}-{c[3]}x{c[4]}")
@pytest.mark.parametrize("partition", ["auto", "one-pass", "min"])
@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma"])
@pytest.mark.parametrize("waves", [0, 4])
def test_decode_fp8_parity_small(case, partition, kernel, waves):
    qd, d, bs, hq, hkv, lens = case
    max_ctx = -(-max(lens) // bs) * bs
    p = {"auto": 0, "one-pass": max_ctx, "min": max(bs, 16) * 2}[partition]
    cfg = custom_config(f"d8-{qd}", lens, hq, hkv, d, qd, bs, seed=sum(lens) + d + 7 * bs,
                        partition_size=p, cache_dtype="fp8", fp8_scales=(2.0 ** -5, 0.0371))
    wl = Workload(cfg)
    _say(f"fp8 decode {cfg.name} lens={lens} d={d} bs={bs} g={cfg.group} P={p} {kernel} "
         f"waves={waves}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    flags = KERNELS[kernel] | (pa.WAVES_FLAG[waves] if waves else 0)
    if kernel == "mfma" and qd != "bf16":
        # the matrix-core kernel takes E4M3 caches with bfloat16 queries only
        out = torch.empty(gs.q[0].shape, dtype=torch.float32, device="cuda")
        assert_rejected(lambda: decode_kv(cfg, out, gs.q[0], gs.kc, gs.vc, gs.block_tables,
                                          gs.ctx[0], p, flags=flags), out)
        return
    out = gs.decode(0, flags=flags)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = max_abs_err(out, st.decode(0))
    assert err <= TOL_ABS, f"max abs error {err:.3e}"
    _pools_equal(gs, st)


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_decode_fp8_out_in_query_dtype(qd):
    cfg = custom_config("d8-out", [7, 200, 901], 8, 2, 128, qd, 16, seed=78, cache_dtype="fp8",
                        fp8_scales=(2.0 ** -6, 2.0 ** -5))
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    ref = st.decode(0)
    out_h = gs.decode(0, out_dtype=gs.q.dtype)
    ulp = 2.0 ** (-10 if qd == "f16" else -7)
    err = np.abs(out_h.double().cpu().numpy() - ref)
    assert (err <= np.abs(ref) * ulp + TOL_ABS).all()


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("partition", [0, 16])
def test_decode_fp8_context_length_one_returns_v(kernel, partition):
    """L = 1: out = stored V * v_scale exactly (a power-of-two scale keeps it exact)."""
    vs = 2.0 ** -4
    cfg = custom_config("l1-fp8", [1] * 6, 8, 2, 128, "bf16", 16, seed=3, num_blocks=9,
                        cache_dtype="fp8", fp8_scales=(2.0 ** -5, vs))
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    out = gs.decode(0, partition_size=partition, flags=KERNELS[kernel])
    torch.cuda.synchronize()
    codes = oracle.encode_fp8((gs.step_v[0].float().cpu() / vs).numpy())
    expect = oracle.decode_bits(codes, "fp8") * vs  # [B][Hkv][d]
    expect = np.repeat(expect, cfg.group, axis=1).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), expect)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("partition", [0, 32, "one-pass"])
def test_decode_fp8_one_hot_probe_bit_exact(kernel, partition):
    """K = 0 except one target token whose stored key is large along q: every other
    weight underflows, so out == stored V[t*] * v_scale exactly, for every t*."""
    L, d, bs, H = 96, 64, 16, 1
    gen = torch.Generator().manual_seed(19)
    q = torch.randn(1, 1, d, generator=gen).to(torch.bfloat16)
    V = torch.randn(L, H, d, generator=gen)
    ks, vs = 1.0, 2.0 ** -3
    scale = 1.0 / 8.0
    NB = 12
    perm = torch.randperm(NB, generator=gen)[: L // bs].to(torch.int32)
    bt = perm.view(1, -1).cuda()
    pos = torch.arange(L)
    slots = (perm[pos // bs].to(torch.int64) * bs + pos % bs).cuda()
    p = {0: 0, 32: 32, "one-pass": L}[partition]
    qf = q.float()
    for t in [0, 1, 15, 16, 17, 47, 63, 64, 95]:
        K = torch.zeros(L, H, d)
        K[t, 0] = torch.sign(qf[0, 0]) * 448.0  # |score| = 448 * sum|q| * scale >> 200
        kc = torch.full(pa.key_cache_shape(NB, H, d, bs, torch.float8_e4m3fn), 0x7F,
                        dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        vc = torch.full(pa.value_cache_shape(NB, H, d, bs), 0x7F, dtype=torch.uint8,
                        device="cuda").view(torch.float8_e4m3fn)
        pa.cache_write_fp8(K.cuda(), V.cuda(), slots, kc, vc, ks, vs)
        out = torch.empty(1, 1, d, device="cuda")
        pa.decode_fp8(out, q.cuda(), kc, vc, bt, torch.tensor([L], dtype=torch.int32,
                                                               device="cuda"),
                      scale, ks, vs, bs, p, flags=KERNELS[kernel])
        torch.cuda.synchronize()
        expect = oracle.decode_bits(oracle.encode_fp8((V[t, 0] / vs).numpy()), "fp8") * vs
        assert np.array_equal(out[0, 0].cpu().numpy(), expect.astype(np.float32)), f"t*={t}"


def test_decode_fp8_rejected_by_plain_entry_points():
    cfg = custom_config("rej", [20], 8, 2, 128, "bf16", 16, seed=1, cache_dtype="fp8",
                        fp8_scales=(1.0, 1.0))
    wl = Workload(cfg)
    gs = GpuState(wl)
    out = torch.empty(gs.q[0].shape, device="cuda")
    with pytest.raises(pa.PAError):
        pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], 0.1, 16)


# ------------------------------------------------------------------ full size

@pytest.mark.parametrize("cid", [4, 5])
def test_full_workload_fp8_parity(cid):
    """The GQA workloads with E4M3 caches at full size, library-picked launch:
    every row of every step (8 steps of the long-context workload) against the
    oracle, and the whole pools bit for bit."""
    cfg = FP8_WORKLOADS[cid]
    wl = Workload(cfg)
    _say(f"full fp8 workload {cid} {cfg.name}: {wl.describe()}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    for s in range(cfg.steps):
        gs.write_step(s)
        st.write_step(s)
        out = gs.decode(s)
        err = max_abs_err(out, st.decode(s, threads=16))
        _say(f"  step {s}: err {err:.3e} rows all")
        assert err <= TOL_ABS
    torch.cuda.synchronize()
    _pools_equal(gs, st)
