"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars: the cache write is bit-exact (whole NaN-poisoned pools compared); decode
with fp32 KV is within 1e-5 relative error both rowwise (normwise per row) and
componentwise (each element against the oracle's sum of weighted value
magnitudes), decode with fp16/bf16 KV within 2e-3 max absolute error, against
the oracle in fp64 on the same rounded inputs.  Invariant checks (L = 1, one-hot probe, block
permutation) are bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import (WORKLOADS, Workload, config3_long_first,
                                                   custom_config, raw_bits)
from tests.gpu_harness import (GpuState, assert_rejected, componentwise_rel_err, decode_kv,
                               max_abs_err, oracle_state_empty, rowwise_rel_err, write_kv)
from tests.paged_host import OracleState, abs_values

pytestmark = pytest.mark.gpu

TOL_ABS_HALF = 2e-3
TOL_REL_F32 = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_decode(out: torch.Tensor, ref: np.ndarray, dtype: str, rows=None, ref_abs=None):
    """ref_abs (fp32 caches): the oracle's decode over |V|, the denominator of
    the componentwise relative error."""
    if dtype == "f32":
        err = rowwise_rel_err(out, ref, rows)
        assert err <= TOL_REL_F32, f"rowwise relative error {err:.3e}"
        if ref_abs is not None:
            cerr = componentwise_rel_err(out, ref, ref_abs, rows)
            assert cerr <= TOL_REL_F32, f"componentwise relative error {cerr:.3e}"
            err = max(err, cerr)
    else:
        err = max_abs_err(out, ref, rows)
        assert err <= TOL_ABS_HALF, f"max abs error {err:.3e}"
    return err


def _pools_equal(gs: GpuState, st) -> None:
    gk = raw_bits(gs.kc.cpu())
    gv = raw_bits(gs.vc.cpu())
    assert np.array_equal(gk, st.kc), "key pool differs from the oracle's"
    assert np.array_equal(gv, st.vc), "value pool differs from the oracle's"


def _run_small(cfg, flags=pa.AUTO, partition_size=None, out_dtype=torch.float32):
    wl = Workload(cfg)
    _say(f"case {cfg.name} lens={wl.lens0.tolist()} d={cfg.head_dim} bs={cfg.block_size} "
         f"g={cfg.group} dtype={cfg.dtype} P={partition_size} flags={flags}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    results = []
    for s in range(cfg.steps):
        gs.write_step(s)
        st.write_step(s)
        out = gs.decode(s, out_dtype=out_dtype, partition_size=partition_size, flags=flags)
        ref = st.decode(s)
        ref_abs = st.decode_abs_values(s) if cfg.kv_dtype == "f32" else None
        results.append((out, ref, ref_abs))
    torch.cuda.synchronize()
    return wl, gs, st, results


# ------------------------------------------------------------------ cache write

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_cache_write_bit_exact(dtype, d, bs):
    cfg = custom_config(f"cw-{dtype}-{d}-{bs}", [1, bs - 1, bs, bs + 1, 3 * bs + 5], 2, 2, d,
                        dtype, bs, seed=100 + d + bs, steps=2)
    wl = Workload(cfg)
    _say(f"cache write {dtype} d={d} bs={bs}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    for s in range(cfg.steps):
        gs.write_step(s)
        st.write_step(s)
    torch.cuda.synchronize()
    _pools_equal(gs, st)


def test_cache_write_strided_tokens_and_negative_slots():
    """k/v as column slices of a fused [T][3*H*d] projection output; slots < 0 skipped."""
    T, H, d, bs, NB = 37, 4, 128, 16, 12
    g = torch.Generator().manual_seed(5)
    qkv = torch.randn(T, 3 * H * d, generator=g).to(torch.bfloat16)
    k = qkv[:, H * d:2 * H * d].view(T, H, d)
    v = qkv[:, 2 * H * d:].view(T, H, d)
    slots = torch.randperm(NB * bs, generator=g)[:T].to(torch.int64)
    slots[::5] = -1
    kc_o = np.full(pa.key_cache_shape(NB, H, d, bs, torch.bfloat16), 0x7FC0, np.uint16)
    vc_o = np.full(pa.value_cache_shape(NB, H, d, bs), 0x7FC0, np.uint16)
    oracle.cache_write(raw_bits(k.contiguous()), raw_bits(v.contiguous()), slots.numpy(), kc_o,
                       vc_o, "bf16")
    # start from the same poisoned pools as the oracle
    kc = torch.full(pa.key_cache_shape(NB, H, d, bs, torch.bfloat16), 0x7FC0, dtype=torch.int16,
                    device="cuda").view(torch.bfloat16)
    vc = torch.full(pa.value_cache_shape(NB, H, d, bs), 0x7FC0, dtype=torch.int16,
                    device="cuda").view(torch.bfloat16)
    qkv_d = qkv.cuda()
    pa.cache_write(qkv_d[:, H * d:2 * H * d].view(T, H, d), qkv_d[:, 2 * H * d:].view(T, H, d),
                   slots.cuda(), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(raw_bits(kc.cpu()), kc_o)
    assert np.array_equal(raw_bits(vc.cpu()), vc_o)


# ------------------------------------------------------------------ decode parity

SMALL = [
    # dtype, d, bs, Hq, Hkv, lens
    ("f32", 64, 16, 4, 4, [1, 17, 64, 200]),
    ("f32", 128, 8, 4, 2, [3, 40, 129]),
    ("f16", 128, 16, 8, 8, [1, 15, 16, 17, 300, 513]),
    ("f16", 64, 32, 6, 2, [2, 31, 33, 400]),
    ("bf16", 128, 16, 8, 2, [5, 16, 100, 1000, 1500]),
    ("bf16", 128, 32, 16, 2, [1, 64, 777, 2049]),
    ("bf16", 64, 64, 12, 4, [63, 64, 65, 700]),
    ("bf16", 128, 8, 7, 1, [9, 250, 600]),
    ("f16", 128, 64, 16, 1, [1, 1000]),
    ("bf16", 128, 16, 32, 8, [1, 2, 1024, 3000]),
    # large groups (one kv head for many q heads): several items per kv head
    ("bf16", 128, 16, 64, 1, [1, 40, 700, 1500]),
    ("f16", 64, 32, 48, 2, [3, 33, 900]),
    ("f32", 64, 16, 32, 1, [5, 17, 300]),
]


KERNELS = {"auto": pa.AUTO, "valu": pa.FORCE_VALU, "mfma": pa.FORCE_MFMA}


def _check_rejected(cfg, partition_size, flags):
    """A kernel choice the library has no kernel for on these dtypes: the
    decode call is refused at the C ABI (PA_ERR_UNSUPPORTED), nothing runs."""
    gs = GpuState(Workload(cfg))
    out = torch.empty(gs.q[0].shape, dtype=torch.float32, device="cuda")
    assert_rejected(lambda: pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0],
                                      cfg.attn_scale(), cfg.block_size, partition_size,
                                      flags=flags), out)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-d{c[1]}-bs{c[2]}-{c[3]}x{c[4]}")
@pytest.mark.parametrize("partition", [0, "one-pass", "min"])
@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma"])
def test_decode_parity_small(case, partition, kernel):
    dtype, d, bs, hq, hkv, lens = case
    max_ctx = -(-max(lens) // bs) * bs
    p = {0: 0, "one-pass": max_ctx, "min": max(bs, 16) * 2}[partition]
    cfg = custom_config(f"dp-{dtype}", lens, hq, hkv, d, dtype, bs, seed=sum(lens) + d + bs,
                        partition_size=p)
    if kernel == "mfma" and dtype == "f32":  # the matrix-core kernel serves 16-bit caches only
        _check_rejected(cfg, p, KERNELS[kernel])
        return
    wl, gs, st, res = _run_small(cfg, flags=KERNELS[kernel])
    for out, ref, ref_abs in res:
        assert torch.isfinite(out).all()
        _check_decode(out, ref, dtype, ref_abs=ref_abs)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-d{c[1]}-bs{c[2]}-{c[3]}x{c[4]}")
@pytest.mark.parametrize("partition", ["one-pass", "min"])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("waves", [2, 4])
def test_decode_parity_split_waves(case, partition, kernel, waves):
    """Several waves per work item (tokens split between them, merged on chip)."""
    dtype, d, bs, hq, hkv, lens = case
    max_ctx = -(-max(lens) // bs) * bs
    p = {"one-pass": max_ctx, "min": max(bs, 16) * 2}[partition]
    cfg = custom_config(f"dw-{dtype}", lens, hq, hkv, d, dtype, bs, seed=sum(lens) + d + 5 * bs,
                        partition_size=p)
    if kernel == "mfma" and dtype == "f32":  # the matrix-core kernel serves 16-bit caches only
        _check_rejected(cfg, p, KERNELS[kernel] | pa.WAVES_FLAG[waves])
        return
    wl, gs, st, res = _run_small(cfg, flags=KERNELS[kernel] | pa.WAVES_FLAG[waves])
    for out, ref, ref_abs in res:
        assert torch.isfinite(out).all()
        _check_decode(out, ref, dtype, ref_abs=ref_abs)


def _decode_nan_prefilled(gs, wl, P, flags):
    """Decode into NaN-filled out and workspace (nothing left from earlier calls)."""
    c = wl.cfg
    kdt = gs.kc.dtype
    wsb = pa.decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                   c.block_size, wl.max_blocks_per_seq, P, kdt, flags)
    ws = torch.full((max(wsb, 256) // 4,), float("nan"), device="cuda")
    out = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(),
              c.block_size, P, ws.view(torch.uint8), flags)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kernel,dtype,hq,hkv", [("mfma", "bf16", 32, 8), ("valu", "f16", 16, 16)])
@pytest.mark.parametrize("waves", [1, 2, 4])
@pytest.mark.parametrize("P", [256, 768, 1024])
def test_grid_modes_agree_bit_for_bit(kernel, dtype, hq, hkv, waves, P):
    """More sequences than a wave has lanes, 11, 4 or 3 partitions: the persistent
    grid over the work list (several items per workgroup), the sorted grid (items
    ordered on the device, then dealt to a persistent grid in fixed snake rounds,
    or at 1024-token partitions from a counter) and the grid in its own order
    each compute every item exactly once --
    bit-identical to one another, into NaN-filled outputs and workspace -- and
    within tolerance of the oracle."""
    rng = np.random.default_rng(90 + waves)
    lens = rng.integers(1, 2600, size=300).tolist()
    lens[:3] = [1, 2600, 5]
    cfg = custom_config(f"gm-{kernel}", lens, hq, hkv, 128, dtype, 16, seed=123)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    flags = KERNELS[kernel] | pa.WAVES_FLAG[waves]
    modes = {}
    for mode in (pa.WORK_LIST, pa.SORTED_GRID, pa.NO_WORK_LIST):
        assert pa.decode_grid(cfg.num_seqs, hq, hkv, 128, 16, wl.max_blocks_per_seq, P,
                              gs.kc.dtype, gs.kc.dtype, flags | mode) == pa.GRID_NAMES[mode]
        modes[mode] = _decode_nan_prefilled(gs, wl, P, flags | mode)
    assert torch.isfinite(modes[pa.SORTED_GRID]).all()
    assert torch.equal(modes[pa.WORK_LIST], modes[pa.NO_WORK_LIST])
    assert torch.equal(modes[pa.SORTED_GRID], modes[pa.NO_WORK_LIST])
    _check_decode(modes[pa.SORTED_GRID], st.decode(0, threads=8), dtype)


def _device_partition(lens, num_kv_heads, p, cus):
    """The ordering kernel's refinement of the library's size p, as include/pa.h
    states it: kept where the longest context is at most twice the mean, else
    the largest of p / 2, p, 2p within a third of a compute unit's share of the
    token x kv-head work (2p only while the longest context spans two
    partitions and 2p <= 8192)."""
    total, lmax, B = sum(lens), max(lens), len(lens)
    if lmax <= 0 or lmax * B <= 2 * total:
        return p
    third = total * num_kv_heads // (3 * cus)
    q = p // 2
    if third >= p:
        q = p
    if third >= 2 * p and 4 * p <= lmax and 2 * p <= 8192:
        q = 2 * p
    return q


def _lognormal(n, seed):
    rng = np.random.default_rng(seed)
    return [int(min(8192, max(1, round(float(np.exp(rng.normal(np.log(1024), 1)))))))
            for _ in range(n)]


@pytest.mark.parametrize("case", ["skewed", "lognormal", "uniform"])
def test_device_refined_partition(case):
    """partition_size = 0 on the sorted grid from 2048 tokens: the ordering
    kernel refines the library's size from the actual lengths.  The result is
    bit-identical to the decode with that size passed explicitly, the same
    through the order / ordered-decode / merge phases, and within tolerance of
    the oracle.  Shapes: one 8192-token sequence among 63 short ones (refined
    down), 256 lognormal contexts up to 8192 (up, on a 256-CU device), 16
    equal 16k contexts (kept)."""
    rng = np.random.default_rng(21)
    lens = {"skewed": [int(x) for x in rng.integers(16, 257, 63)] + [8192],
            "lognormal": _lognormal(256, 4),
            "uniform": [16384] * 16}[case]
    cfg = custom_config(f"refine-{case}", lens, 32, 8, 128, "bf16", 16, seed=31)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    MB = wl.max_blocks_per_seq
    p = pa.decode_partition_size(cfg.num_seqs, 32, 8, 128, 16, MB, gs.kc.dtype)
    assert p >= 2048 and pa.decode_grid(cfg.num_seqs, 32, 8, 128, 16, MB, 0, gs.kc.dtype,
                                        gs.kc.dtype) == "sorted"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    want = _device_partition(lens, 8, p, cus)
    _say(f"refined partition {case}: host {p}, expected device pick {want} ({cus} CUs)")
    auto = _decode_nan_prefilled(gs, wl, 0, pa.AUTO)
    explicit = _decode_nan_prefilled(gs, wl, want, pa.AUTO)
    assert torch.isfinite(auto).all()
    assert torch.equal(auto, explicit), f"differs from the decode at {want}"
    # the same launch in phases: order (with the refinement), ordered decode, merge
    c = wl.cfg
    wsb = pa.decode_workspace_size(c.num_seqs, 32, 8, 128, 16, MB, 0, gs.kc.dtype)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    args = (out, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), 16, 0, ws)
    pa.decode_order(*args)
    pa.decode_partitions(*args, pa.ORDERED)
    pa.decode_merge(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, auto)
    assert pa.decode_partition_used(ws, c.num_seqs, 32, 8, 128, 16, MB, gs.kc.dtype) == want
    _check_decode(auto, st.decode(0, threads=16), "bf16")


def _order_of_workspace(ws: torch.Tensor, B: int, Hq: int, D: int, n_parts: int) -> np.ndarray:
    """The item order a sorted-grid decode leaves in its workspace.  Internal
    layout (not part of the C ABI): (m, l) per (sequence, q head, partition),
    then the partial outputs, each rounded up to 256 bytes, then the order of
    B * n_parts int32 entries."""
    def up(v):
        return (v + 255) // 256 * 256
    rows = B * Hq * n_parts
    off = up(rows * 2 * 4) + up(rows * D * 4)
    raw = ws.view(torch.uint8)[off:off + B * n_parts * 4].cpu().numpy()
    return raw.view(np.int32)


@pytest.mark.parametrize("P", [256, 1024])
def test_ordering_kernel_is_longest_first_over_every_item(P):
    """The ordering kernel's output, read back: every non-empty (sequence,
    partition) item exactly once, sizes (in 16-token chunks, capped at 1023)
    never increasing, then -1 for the unused entries.  Items of equal size may
    come in any order, so the check is on the multiset and the size sequence.
    Includes empty sequences (one item each, size 0, last among the items)."""
    rng = np.random.default_rng(77 + P)
    lens = rng.integers(1, 5000, size=200).tolist()
    lens[:4] = [1, 4999, 16, 17]
    cfg = custom_config(f"order-{P}", lens, 8, 2, 128, "bf16", 16, seed=5)
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    ctx_host = np.array(lens, dtype=np.int32)
    ctx_host[[7, 50]] = 0  # two empty sequences
    ctx = torch.from_numpy(ctx_host).cuda()
    flags = pa.FORCE_MFMA | pa.SORTED_GRID
    MB = wl.max_blocks_per_seq
    assert pa.decode_grid(cfg.num_seqs, 8, 2, 128, 16, MB, P, gs.kc.dtype, gs.kc.dtype,
                          flags) == pa.GRID_NAMES[pa.SORTED_GRID]
    wsb = pa.decode_workspace_size(cfg.num_seqs, 8, 2, 128, 16, MB, P, gs.kc.dtype, flags)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.empty(gs.q[0].shape, dtype=torch.float32, device="cuda")
    pa.decode_partitions(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, ctx, cfg.attn_scale(), 16,
                         P, ws, flags)
    torch.cuda.synchronize()
    n_parts = -(-MB * 16 // P)
    order = _order_of_workspace(ws, cfg.num_seqs, 8, 128, n_parts)

    def size_bin(L, p):
        return 0 if L == 0 else min((min(L - p * P, P) + 15) // 16, 1023)

    items = []
    for b, L in enumerate(ctx_host.tolist()):
        n = 1 if L == 0 else -(-L // P)
        items += [(b * n_parts + p, size_bin(L, p)) for p in range(n)]
    k = len(items)
    head = order[:k]
    assert sorted(head.tolist()) == sorted(e for e, _ in items), "items missing or repeated"
    bins = dict(items)
    sizes = [bins[e] for e in head.tolist()]
    assert all(x >= y for x, y in zip(sizes, sizes[1:])), "order is not longest first"
    assert (order[k:] == -1).all(), "unused entries are not -1"


def test_sorted_grid_with_empty_sequences():
    """Zero-length sequences are items too (their rows are zeroed), ordered last."""
    lens = [0, 700, 0, 1, 1500, 0]
    cfg = custom_config("sg-empty", [max(x, 1) for x in lens], 8, 2, 128, "bf16", 16, seed=8)
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    outs = []
    for mode in (pa.SORTED_GRID, pa.NO_WORK_LIST):
        out = torch.full(gs.q[0].shape, float("nan"), device="cuda")
        pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, ctx, cfg.attn_scale(), 16, 256,
                  flags=mode)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    for b, L in enumerate(lens):
        if L == 0:
            assert (outs[0][b] == 0).all()
        else:
            assert torch.isfinite(outs[0][b]).all()


def test_decode_multistep_parity():
    cfg = custom_config("ms", [1, 30, 31, 32, 500], 8, 2, 128, "bf16", 32, seed=9, steps=8)
    wl, gs, st, res = _run_small(cfg)
    for out, ref, _ in res:
        _check_decode(out, ref, "bf16")
    _pools_equal(gs, st)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_f32_query_and_half_output(dtype):
    cfg = custom_config("mix", [7, 200, 901], 8, 2, 128, dtype, 16, seed=77)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    # q in f32 (the same values as the half q, widened exactly)
    qf = gs.q[0].float()
    out_f = gs.decode(0, q=qf)
    ref = st.decode(0)
    _check_decode(out_f, ref, dtype)
    # out in the kv dtype: within one ulp of that dtype plus the half tolerance
    out_h = gs.decode(0, out_dtype=gs.kc.dtype)
    ulp = 2.0 ** (-10 if dtype == "f16" else -7)
    err = np.abs(out_h.double().cpu().numpy() - ref)
    assert (err <= np.abs(ref) * ulp + TOL_ABS_HALF).all()


# ------------------------------------------------------------------ invariants

def _single_token_state(dtype, d, bs, hq, hkv, n_seqs, seed):
    cfg = custom_config("l1", [1] * n_seqs, hq, hkv, d, dtype, bs, seed=seed, num_blocks=n_seqs + 3)
    return cfg, Workload(cfg)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("partition", [0, 16])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("waves", [1, 4])
def test_context_length_one_returns_v_bit_exact(dtype, partition, kernel, waves):
    cfg, wl = _single_token_state(dtype, 128, 16, 8, 2, 6, seed=3)
    if kernel == "mfma" and dtype == "f32":  # the matrix-core kernel serves 16-bit caches only
        _check_rejected(cfg, partition, KERNELS[kernel] | pa.WAVES_FLAG[waves])
        return
    gs = GpuState(wl)
    gs.write_step(0)
    out = gs.decode(0, partition_size=partition, flags=KERNELS[kernel] | pa.WAVES_FLAG[waves])
    torch.cuda.synchronize()
    v = gs.step_v[0].float()  # [B][Hkv][d]
    expect = v.repeat_interleave(cfg.group, dim=1)
    assert torch.equal(out, expect)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("partition", [0, 32, "one-pass"])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("waves", [1, 4])
def test_one_hot_probe_bit_exact(dtype, partition, kernel, waves):
    """K = 0 except one target token whose key is c*q (scale*c*|q|^2 >= 200):
    every other weight underflows, so out == V[t*] exactly, for every t*.  The
    matrix-core kernel on fp32 caches is refused instead (16-bit caches only)."""
    L, d, bs, H = 96, 64, 16, 1
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    gen = torch.Generator().manual_seed(17)
    q = torch.randn(1, 1, d, generator=gen).to(dt)
    V = torch.randn(L, H, d, generator=gen).to(dt)
    qf = q.float()
    scale = 1.0 / 8.0
    c = 260.0 / (scale * float((qf ** 2).sum()))
    NB = 12
    perm = torch.randperm(NB, generator=gen)[: L // bs].to(torch.int32)
    bt = perm.view(1, -1).cuda()
    pos = torch.arange(L)
    slots = (perm[pos // bs].to(torch.int64) * bs + pos % bs).cuda()
    p = {0: 0, 32: 32, "one-pass": L}[partition]
    for t in [0, 1, 15, 16, 17, 47, 63, 64, 95]:
        K = torch.zeros(L, H, d, dtype=dt)
        K[t, 0] = (qf[0, 0] * c).to(dt)
        kc = torch.full(pa.key_cache_shape(NB, H, d, bs, dt), float("nan"), dtype=dt, device="cuda")
        vc = torch.full(pa.value_cache_shape(NB, H, d, bs), float("nan"), dtype=dt, device="cuda")
        pa.cache_write(K.cuda(), V.cuda(), slots, kc, vc)
        out = torch.empty(1, 1, d, device="cuda")
        ctx = torch.tensor([L], dtype=torch.int32, device="cuda")
        flags = KERNELS[kernel] | pa.WAVES_FLAG[waves]
        if kernel == "mfma" and dtype == "f32":
            assert_rejected(lambda: pa.decode(out, q.cuda(), kc, vc, bt, ctx, scale, bs, p,
                                              flags=flags), out)
            return
        pa.decode(out, q.cuda(), kc, vc, bt, ctx, scale, bs, p, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(out[0, 0].cpu(), V[t, 0].float()), f"t*={t}"


def _uniform_weight_case(dtype: str, case: str, seed: int):
    """Sequences whose softmax weights are all equal: every key of a (sequence,
    kv head) is the same vector ("identical-keys"), or the scale is 0
    ("scale-0", random keys).  Returns the caches written by the library and by
    the oracle from the same tensors, and the decode arguments."""
    lens = [1, 17, 100, 300, 1000]
    hq, hkv, d, bs = 8, 2, 128, 16
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    gen = torch.Generator().manual_seed(seed)
    nblk = [-(-L // bs) for L in lens]
    NB = sum(nblk) + 7
    perm = torch.randperm(NB, generator=gen)
    MB = max(nblk)
    bt = torch.full((len(lens), MB), -1, dtype=torch.int32)
    kc = torch.full(pa.key_cache_shape(NB, hkv, d, bs, dt), float("nan"), dtype=dt, device="cuda")
    vc = torch.full(pa.value_cache_shape(NB, hkv, d, bs), float("nan"), dtype=dt, device="cuda")
    okc = np.full(kc.shape, POISON[dtype], dtype=raw_bits(torch.empty(0, dtype=dt)).dtype)
    ovc = np.full(vc.shape, POISON[dtype], dtype=okc.dtype)
    V_all, off = [], 0
    for b, L in enumerate(lens):
        blocks = perm[off:off + nblk[b]]
        off += nblk[b]
        bt[b, :nblk[b]] = blocks.to(torch.int32)
        pos = torch.arange(L)
        slots = blocks[pos // bs].to(torch.int64) * bs + pos % bs
        if case == "identical-keys":
            K = torch.randn(1, hkv, d, generator=gen).expand(L, hkv, d).to(dt).contiguous()
        else:
            K = torch.randn(L, hkv, d, generator=gen).to(dt)
        V = torch.randn(L, hkv, d, generator=gen).to(dt)
        V_all.append(V)
        pa.cache_write(K.cuda(), V.cuda(), slots.cuda(), kc, vc)
        oracle.cache_write(raw_bits(K), raw_bits(V), slots.numpy(), okc, ovc, dtype)
    q = torch.randn(len(lens), hq, d, generator=gen).to(dt)
    scale = 0.0 if case == "scale-0" else float(np.float32(1.0 / np.sqrt(d)))
    ctx = torch.tensor(lens, dtype=torch.int32)
    return dict(lens=lens, hq=hq, hkv=hkv, d=d, bs=bs, dt=dt, bt=bt, kc=kc, vc=vc, okc=okc,
                ovc=ovc, V=V_all, q=q, scale=scale, ctx=ctx)


POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("case", ["identical-keys", "scale-0"])
@pytest.mark.parametrize("partition", ["one-pass", 32, 256])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("waves", [1, 2, 4])
def test_uniform_weights_give_mean_of_v(dtype, case, partition, kernel, waves):
    """All scores of a row equal (identical keys, or scale 0): every weight is
    exactly 1, so out is the mean of V over the context -- exact attention
    whatever the paging.  After a wave's first chunk the running max never
    moves, so the lazy rescale is skipped on every later chunk, in both
    kernels, across the wave merge and the partition merge.  Checked against
    the oracle and against the fp64 mean of V, to the dtype's tolerance."""
    c = _uniform_weight_case(dtype, case, seed=61 if case == "scale-0" else 62)
    max_ctx = c["bt"].shape[1] * c["bs"]
    p = {"one-pass": max_ctx, 32: 32, 256: 256}[partition]
    out = torch.full((len(c["lens"]), c["hq"], c["d"]), float("nan"), device="cuda")
    call = lambda: pa.decode(out, c["q"].cuda(), c["kc"], c["vc"], c["bt"].cuda(),  # noqa: E731
                             c["ctx"].cuda(), c["scale"], c["bs"], p,
                             flags=KERNELS[kernel] | pa.WAVES_FLAG[waves])
    if kernel == "mfma" and dtype == "f32":  # the matrix-core kernel serves 16-bit caches only
        assert_rejected(call, out)
        return
    call()
    torch.cuda.synchronize()
    ref = oracle.decode(raw_bits(c["q"]), dtype, c["okc"], c["ovc"], dtype, c["bt"].numpy(),
                        c["ctx"].numpy(), c["scale"])
    g = c["hq"] // c["hkv"]
    mean = np.stack([V.double().numpy().mean(axis=0).repeat(g, axis=0) for V in c["V"]])
    if dtype == "f32":
        ref_abs = oracle.decode(raw_bits(c["q"]), dtype, c["okc"], abs_values(c["ovc"], dtype),
                                dtype, c["bt"].numpy(), c["ctx"].numpy(), c["scale"])
        _check_decode(out, ref, dtype, ref_abs=ref_abs)
        _check_decode(out, mean, dtype)
    else:
        _check_decode(out, ref, dtype)
        _check_decode(out, mean, dtype)
    assert np.abs(ref - mean).max() <= 1e-12 * max(1.0, np.abs(mean).max())


@pytest.mark.parametrize("dtype,scale", [("bf16", -0.0883883), ("bf16", 1.0), ("bf16", 8.0),
                                         ("f16", 8.0), ("f32", -0.0883883)])
@pytest.mark.parametrize("partition", [0, 32, "one-pass"])
@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_negative_and_sharp_scales(dtype, scale, partition, kernel):
    """The softmax scale is any real: negative (the weights favour the smallest
    scores) or large enough that each row's weights are nearly one-hot (score spreads
    of several hundred, most weights underflow, partition maxima far apart in the
    merge).  Within the dtype's tolerance of the oracle."""
    lens = [1, 31, 700, 2100]
    max_ctx = -(-max(lens) // 16) * 16
    p = {0: 0, 32: 32, "one-pass": max_ctx}[partition]
    cfg = custom_config(f"sc-{dtype}", lens, 8, 2, 128, dtype, 16, seed=71, partition_size=p,
                        scale=scale)
    if kernel == "mfma" and dtype == "f32":  # the matrix-core kernel serves 16-bit caches only
        _check_rejected(cfg, p, KERNELS[kernel])
        return
    wl, gs, st, res = _run_small(cfg, flags=KERNELS[kernel])
    for out, ref, ref_abs in res:
        assert torch.isfinite(out).all()
        _check_decode(out, ref, dtype, ref_abs=ref_abs)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_block_permutation_bit_identical(kernel):
    """Moving physical blocks (and remapping the table) does not change a bit."""
    cfg = custom_config("perm", [33, 300, 1000], 8, 2, 128, "bf16", 16, seed=44)
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    out1 = gs.decode(0, flags=KERNELS[kernel])
    NB = wl.num_blocks
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(1)).cuda()
    kc2 = torch.empty_like(gs.kc)
    vc2 = torch.empty_like(gs.vc)
    kc2[perm] = gs.kc
    vc2[perm] = gs.vc
    bt = gs.block_tables.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32)
    out2 = torch.empty_like(out1)
    pa.decode(out2, gs.q[0], kc2, vc2, bt2.contiguous(), gs.ctx[0], cfg.attn_scale(),
              cfg.block_size, 0, flags=KERNELS[kernel])
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_blocks_past_4_gib_of_the_pool(kernel, cache):
    """Each cache a little over 4 GiB, the sequences' blocks on both sides of the
    2 GiB and 4 GiB byte offsets and spread over the rest: addresses that need 64
    bits.  The step's write there equals the write into the small pool bit for bit,
    and the decode there equals the small pool's decode bit for bit (the block
    permutation invariant), which is itself within tolerance of the oracle."""
    fp8 = cache == "fp8"
    cfg = custom_config("far", [33, 300, 1000], 8, 2, 128, "bf16", 16, seed=48,
                        cache_dtype="fp8" if fp8 else "",
                        fp8_scales=(2.0 ** -6, 2.0 ** -5) if fp8 else (1.0, 1.0))
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    NB, bs = wl.num_blocks, cfg.block_size
    block_bytes = gs.kc[0].numel() * gs.kc.element_size()
    assert block_bytes == gs.vc[0].numel() * gs.vc.element_size()
    lo, edge = (1 << 31) // block_bytes, (1 << 32) // block_bytes
    nb_far = edge + 3 * NB
    spread = torch.randperm(3 * NB - 1, generator=torch.Generator().manual_seed(5))[: NB - 4]
    ids = torch.cat([torch.tensor([lo - 1, lo, edge - 1, edge]), edge + 1 + spread]).cuda()
    assert ids.unique().numel() == NB and int(ids.max()) < nb_far
    _say(f"far pool: {nb_far} blocks of {block_bytes} B per cache, cache {cache}, {kernel}")
    kf = torch.empty((nb_far,) + tuple(gs.kc.shape[1:]), dtype=gs.kc.dtype, device="cuda")
    vf = torch.empty((nb_far,) + tuple(gs.vc.shape[1:]), dtype=gs.vc.dtype, device="cuda")
    kf.view(torch.uint8)[ids] = gs.kc.view(torch.uint8)  # the prior context, moved
    vf.view(torch.uint8)[ids] = gs.vc.view(torch.uint8)

    slots = gs.step_slots[0].long()
    s0 = slots.clamp(min=0)
    far_slots = torch.where(slots >= 0, ids[s0 // bs] * bs + s0 % bs, slots)
    write_kv(cfg, gs.step_k[0], gs.step_v[0], far_slots, kf, vf)
    gs.write_step(0)
    st.write_step(0)
    torch.cuda.synchronize()
    _pools_equal(gs, st)
    assert torch.equal(kf.view(torch.uint8)[ids], gs.kc.view(torch.uint8))
    assert torch.equal(vf.view(torch.uint8)[ids], gs.vc.view(torch.uint8))

    bt = gs.block_tables.long()
    bt_far = torch.where(bt >= 0, ids[bt.clamp(min=0)], bt).to(torch.int32).contiguous()
    ref = st.decode(0)
    for p in (0, 256):
        out = gs.decode(0, partition_size=p, flags=KERNELS[kernel])
        out_far = torch.empty_like(out)
        decode_kv(cfg, out_far, gs.q[0], kf, vf, bt_far, gs.ctx[0], p, flags=KERNELS[kernel])
        torch.cuda.synchronize()
        assert torch.equal(out, out_far), f"partition {p}"
        _check_decode(out_far, ref, "bf16")
    del kf, vf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kernel,dtype,hq,hkv", [
    ("valu", "bf16", 32, 8), ("mfma", "bf16", 32, 8), ("valu", "f16", 16, 2),
    ("mfma", "f16", 16, 2), ("valu", "f32", 8, 2)])
@pytest.mark.parametrize("partition", [32, "one-pass"])
def test_gqa_equals_replicated_mha(kernel, dtype, hq, hkv, partition):
    """q head hq reads kv head hq / g: the same decode as an MHA batch whose caches hold
    every kv head g times over, bit for bit (a head's arithmetic does not depend on the
    other heads of its item), and within tolerance of the oracle."""
    cfg = custom_config(f"gqa-{dtype}", [1, 29, 300, 1100], hq, hkv, 128, dtype, 16, seed=81)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    p = wl.max_blocks_per_seq * cfg.block_size if partition == "one-pass" else partition
    flags = KERNELS[kernel] | pa.WAVES_2
    out = gs.decode(0, partition_size=p, flags=flags)
    g = hq // hkv
    kc_mha = gs.kc.repeat_interleave(g, dim=1).contiguous()
    vc_mha = gs.vc.repeat_interleave(g, dim=1).contiguous()
    out_mha = torch.empty_like(out)
    pa.decode(out_mha, gs.q[0], kc_mha, vc_mha, gs.block_tables, gs.ctx[0], cfg.attn_scale(),
              cfg.block_size, p, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out, out_mha)
    ref_abs = st.decode_abs_values(0) if dtype == "f32" else None
    _check_decode(out, st.decode(0), dtype, ref_abs=ref_abs)


@pytest.mark.parametrize("kernel,dtype", [("valu", "f32"), ("valu", "bf16"), ("mfma", "bf16"),
                                          ("mfma", "f16")])
@pytest.mark.parametrize("partition", [64, 1024])
def test_block_size_invariance(kernel, dtype, partition):
    """The same logical keys and values paged with blocks of 8, 16, 32 and 64 tokens
    (shuffled pools): the decode is bit-identical across block sizes (the arithmetic
    follows logical positions only) and within tolerance of the oracle."""
    lens = [5, 64, 333, 1000]
    hq, hkv, d = 8, 2, 128
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    gen = torch.Generator().manual_seed(91)
    K = [torch.randn(L, hkv, d, generator=gen).to(dt) for L in lens]
    V = [torch.randn(L, hkv, d, generator=gen).to(dt) for L in lens]
    q = torch.randn(len(lens), hq, d, generator=gen).to(dt)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    ctx = torch.tensor(lens, dtype=torch.int32)
    outs = {}
    for bs in (8, 16, 32, 64):
        nblk = [-(-L // bs) for L in lens]
        NB = sum(nblk) + 5
        perm = torch.randperm(NB, generator=torch.Generator().manual_seed(bs))
        bt = torch.full((len(lens), max(nblk)), -1, dtype=torch.int32)
        kc = torch.full(pa.key_cache_shape(NB, hkv, d, bs, dt), float("nan"), dtype=dt,
                        device="cuda")
        vc = torch.full(pa.value_cache_shape(NB, hkv, d, bs), float("nan"), dtype=dt,
                        device="cuda")
        okc = np.full(kc.shape, POISON[dtype], dtype=raw_bits(torch.empty(0, dtype=dt)).dtype)
        ovc = np.full(vc.shape, POISON[dtype], dtype=okc.dtype)
        off = 0
        for b, L in enumerate(lens):
            blocks = perm[off:off + nblk[b]]
            off += nblk[b]
            bt[b, :nblk[b]] = blocks.to(torch.int32)
            pos = torch.arange(L)
            slots = blocks[pos // bs].to(torch.int64) * bs + pos % bs
            pa.cache_write(K[b].cuda(), V[b].cuda(), slots.cuda(), kc, vc)
            oracle.cache_write(raw_bits(K[b]), raw_bits(V[b]), slots.numpy(), okc, ovc, dtype)
        out = torch.empty((len(lens), hq, d), dtype=torch.float32, device="cuda")
        # waves fixed: the library's pick follows the partition, which a one-pass launch
        # clamps to each table's width
        pa.decode(out, q.cuda(), kc, vc, bt.cuda(), ctx.cuda(), scale, bs, partition,
                  flags=KERNELS[kernel] | pa.WAVES_2)
        torch.cuda.synchronize()
        outs[bs] = out
        ref = oracle.decode(raw_bits(q), dtype, okc, ovc, dtype, bt.numpy(), ctx.numpy(), scale)
        ref_abs = (oracle.decode(raw_bits(q), dtype, okc, abs_values(ovc, dtype), dtype,
                                 bt.numpy(), ctx.numpy(), scale) if dtype == "f32" else None)
        _check_decode(out, ref, dtype, ref_abs=ref_abs)
    for bs in (16, 32, 64):
        assert torch.equal(outs[8], outs[bs]), f"block size {bs} differs from 8"


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_partition_sweep_within_tolerance(kernel):
    cfg = custom_config("sweep", [1, 100, 1000, 4000], 8, 2, 128, "bf16", 16, seed=45)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    ref = st.decode(0)
    for p in [16, 32, 48, 128, 256, 512, 1024, 4000, 4096]:
        out = gs.decode(0, partition_size=p, flags=KERNELS[kernel])
        _check_decode(out, ref, "bf16")


def test_zero_length_sequence_gives_zero_row_and_empty_batch_is_noop():
    cfg = custom_config("z", [5, 40], 4, 4, 64, "f16", 16, seed=46)
    wl = Workload(cfg)
    gs = GpuState(wl)
    gs.write_step(0)
    ctx = gs.ctx[0].clone()
    ctx[0] = 0
    out = torch.full((2, 4, 64), 7.0, device="cuda")
    pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, ctx, cfg.attn_scale(), 16, 0)
    torch.cuda.synchronize()
    assert torch.equal(out[0], torch.zeros_like(out[0]))
    assert torch.isfinite(out[1]).all()
    empty = torch.empty(0, 4, 64, device="cuda")
    pa.decode(empty, gs.q[0][:0], gs.kc, gs.vc, gs.block_tables[:0], ctx[:0],
              cfg.attn_scale(), 16, 0)


# ------------------------------------------------------------------ full-size workloads

FULL = dict(WORKLOADS)
# the skewed batch with its long sequence first instead of last (the first item
# of grid order, the last dispatched partition of the others)
FULL["3-long-first"] = config3_long_first()


@pytest.mark.parametrize("cid", [1, 2, 3, "3-long-first", 4, 5])
def test_full_workload_parity(cid):
    """Each decode workload at full size, in the launch configuration the
    benchmark times (library-picked or the workload's partition size,
    automatic kernel choice): every output row of every step against the
    oracle, and the whole pools bit for bit."""
    cfg = FULL[cid]
    wl = Workload(cfg)
    _say(f"full workload {cid} {cfg.name}: {wl.describe()}")
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    for s in range(cfg.steps):
        gs.write_step(s)
        st.write_step(s)
        out = gs.decode(s)
        ref = st.decode(s, threads=16)
        ref_abs = st.decode_abs_values(s, threads=16) if cfg.kv_dtype == "f32" else None
        err = _check_decode(out, ref, cfg.dtype, ref_abs=ref_abs)
        _say(f"  step {s}: err {err:.3e} rows all ({out.numel() // cfg.head_dim})")
    torch.cuda.synchronize()
    _pools_equal(gs, st)
