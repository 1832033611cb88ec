"""Host-side checks of libpa.so (CPU only; no kernel is ever launched here).

The library must load without a GPU, export every function include/pa.h
declares, and reject invalid arguments with the documented pa_status before
any HIP call.  The pointers passed are never dereferenced: every call here is
rejected by validation.  These tests are skipped where a GPU is visible so a
validation bug can never turn into a launch with fake pointers.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import pagedattention_kv_cache_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6
ECAP, ESEQ, ESCRATCH = -7, -8, -9
F32, F16, BF16 = 0, 1, 2
FAKE = 0x10000  # a 16-byte aligned non-null value; never dereferenced

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-validation tests use fake pointers; CPU only")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libpa.so every entry point raises: there is no fallback path."""
    monkeypatch.setattr(pa, "_lib", None)
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "libpa.so"))
    with pytest.raises(RuntimeError, match="has not been built"):
        pa.lib()
    with pytest.raises(RuntimeError, match="has not been built"):
        pa.decode_workspace_size(4, 32, 8, 128, 16, 64, 256, torch.bfloat16)


def test_library_loads_and_exports_header_symbols():
    L = pa.lib()
    names = _declared_functions()
    assert {"pa_cache_write", "pa_decode", "pa_decode_partitions", "pa_decode_merge",
            "pa_decode_workspace_size", "pa_decode_partition_size", "pa_decode_partition_used",
            "pa_decode_order_fp8", "pa_decode_kernel",
            "pa_decode_waves", "pa_decode_work_list",
            "pa_advance_step", "pa_status_string", "pa_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libpa.so does not export {n}"
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_library_exports_the_block_header():
    L = pa.lib()
    names = _declared_functions(os.path.join(ROOT, "include", "pa_blocks.h"))
    assert {"pa_bm_create", "pa_bm_append", "pa_bm_fork", "pa_bm_mark_computed",
            "pa_bm_swap_out", "pa_copy_blocks", "pa_swap_blocks"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libpa.so does not export {n}"


def test_probe_library_exports_its_header():
    probe = ctypes.CDLL(os.path.join(ROOT, "pagedattention_kv_cache_amd", "libpa_probe.so"))
    names = _declared_functions(os.path.join(ROOT, "include", "pa_probe.h"))
    assert names == ["pa_probe_stream_read"]
    for n in names:
        assert hasattr(probe, n)
    fn = probe.pa_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    assert fn(None, 1024, FAKE, 64, None) == -1  # invalid arguments: nothing launched
    assert fn(FAKE, 1000, FAKE, 64, None) == -1
    assert fn(FAKE, 1024, FAKE, 0, None) == -1


def test_status_strings_and_version():
    L = pa.lib()
    assert L.pa_abi_version() == 1
    fallback = pa.status_string(-99)
    assert fallback == "unknown pa_status"
    texts = [pa.status_string(st)
             for st in (OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EHIP, ECAP, ESEQ, ESCRATCH)]
    assert all(t and t != fallback for t in texts)
    assert len(set(texts)) == len(texts)


def _cw(**kw):
    args = dict(k=FAKE, v=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, T=4, ks=512, vs=512, H=4, d=128,
                NB=10, bs=16, dtype=BF16)
    args.update(kw)
    return pa.lib().pa_cache_write(args["k"], args["v"], args["slots"], args["kc"], args["vc"],
                                   args["T"], args["ks"], args["vs"], args["H"], args["d"],
                                   args["NB"], args["bs"], args["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), EDTYPE),
    (dict(T=-1), ESHAPE),
    (dict(H=0), ESHAPE),
    (dict(NB=0), ESHAPE),
    (dict(d=96), EUNSUP),
    (dict(bs=12), EUNSUP),
    (dict(bs=128), EUNSUP),
    (dict(ks=100), ESHAPE),
    (dict(vs=513), ESHAPE),
    (dict(k=None), ENULL),
    (dict(slots=None), ENULL),
    (dict(vc=None), ENULL),
    (dict(k=FAKE + 2), ESHAPE),
    (dict(kc=FAKE + 8), ESHAPE),
])
def test_cache_write_validation(kw, status):
    assert _cw(**kw) == status


def test_cache_write_zero_tokens_is_noop():
    assert _cw(T=0, k=None, v=None, slots=None, kc=None, vc=None) == OK


def _dec(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, bs=16, P=0, B=4,
             Hq=32, Hkv=8, d=128, NB=100, MB=64, qd=BF16, kvd=BF16, od=F32, ws=None, wsb=0,
             flags=pa.FORCE_VALU)
    a.update(kw)
    return pa.lib().pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"],
                              a["bs"], a["P"], a["B"], a["Hq"], a["Hkv"], a["d"], a["NB"], a["MB"],
                              a["qd"], a["kvd"], a["od"], a["ws"], a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE),
    (dict(Hq=0), ESHAPE),
    (dict(Hkv=0), ESHAPE),
    (dict(Hq=30), ESHAPE),
    (dict(MB=0), ESHAPE),
    (dict(NB=0), ESHAPE),
    (dict(d=96), EUNSUP),
    (dict(d=256), EUNSUP),
    (dict(bs=4), EUNSUP),
    (dict(bs=24), EUNSUP),
    (dict(kvd=5), EDTYPE),
    (dict(qd=F16), EDTYPE),
    (dict(od=F16), EDTYPE),
    (dict(od=9), EDTYPE),
    (dict(P=-16), ESHAPE),
    (dict(P=24), ESHAPE),
    (dict(flags=7), EUNSUP),
    (dict(flags=3), EUNSUP),               # both kernel bits
    (dict(flags=128), EUNSUP),             # unknown bit
    (dict(flags=pa.FORCE_MFMA, kvd=F32, qd=F32), EUNSUP),  # matrix cores: 16-bit caches only
    (dict(flags=pa.FORCE_MFMA, qd=F32), EUNSUP),           # ... queried in the same dtype
    (dict(out=None), ENULL),
    (dict(q=None), ENULL),
    (dict(bt=None), ENULL),
    (dict(cl=None), ENULL),
    (dict(kc=FAKE + 4), ESHAPE),
    (dict(ws=None, wsb=0), EWS),           # four partitions of 256 need a workspace
    (dict(ws=FAKE, wsb=1024), EWS),        # too small
    (dict(ws=FAKE + 8, wsb=1 << 30), EWS),  # misaligned
    (dict(P=16, MB=65536, ws=FAKE, wsb=1 << 40), ESHAPE),  # 65536 partitions of a sequence
])
def test_decode_validation(kw, status):
    assert _dec(**kw) == status


def test_decode_empty_batch_is_noop():
    assert _dec(B=0, out=None, q=None, bt=None, cl=None) == OK


def _dec_noalloc(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, bs=16, P=0, B=4,
             Hq=32, Hkv=8, d=128, NB=100, MB=64, qd=BF16, kvd=BF16, od=F32, flags=pa.FORCE_VALU)
    a.update(kw)
    return pa.lib().pa_decode_noalloc(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"],
                                      a["scale"], a["bs"], a["P"], a["B"], a["Hq"], a["Hkv"],
                                      a["d"], a["NB"], a["MB"], a["qd"], a["kvd"], a["od"],
                                      a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE),
    (dict(Hq=30), ESHAPE),
    (dict(d=96), EUNSUP),
    (dict(kvd=3), EDTYPE),                 # E4M3 caches: not through this entry point
    (dict(qd=F16), EDTYPE),
    (dict(out=None), ENULL),
    (dict(P=24), ESHAPE),
    (dict(flags=64), EUNSUP),             # ordered: no order can have been prepared
    (dict(flags=128), EUNSUP),
    # 2048 x 32 rows x 32 partitions of 256 tokens: a workspace of ~1 GB
    (dict(B=2048, MB=512, P=256), ESCRATCH),
])
def test_decode_noalloc_validation(kw, status):
    """Every argument is validated, and the scratch limit checked, before the
    static scratch is looked up or anything launched."""
    assert _dec_noalloc(**kw) == status


def test_decode_noalloc_empty_batch_is_noop():
    assert _dec_noalloc(B=0, out=None, q=None, bt=None, cl=None) == OK


def test_decode_noalloc_scratch_covers_the_full_size_workloads():
    """PA_SCRATCH_BYTES (64 MiB) holds the partition workspace of every
    full-size decode workload in the launch configuration the benchmark uses."""
    from pagedattention_kv_cache_amd.workloads import WORKLOADS, DTYPE_TORCH, Workload
    for cid, cfg in WORKLOADS.items():
        wl = Workload(cfg)
        need = pa.decode_workspace_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                        cfg.head_dim, cfg.block_size, wl.max_blocks_per_seq,
                                        cfg.partition_size, DTYPE_TORCH[cfg.kv_dtype], pa.AUTO)
        assert need <= pa.SCRATCH_BYTES, (cid, need)


def test_scratch_size_matches_the_header():
    m = re.search(r"#define PA_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == pa.SCRATCH_BYTES


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, -1, 4, 16, 10, FAKE), ESHAPE),
    ((FAKE, FAKE, 4, 0, 16, 10, FAKE), ESHAPE),
    ((FAKE, FAKE, 4, 4, 0, 10, FAKE), ESHAPE),
    ((FAKE, FAKE, 4, 4, 16, 0, FAKE), ESHAPE),
    ((None, FAKE, 4, 4, 16, 10, FAKE), ENULL),
    ((FAKE, None, 4, 4, 16, 10, FAKE), ENULL),
    ((FAKE, FAKE, 4, 4, 16, 10, None), ENULL),
    ((FAKE, FAKE, 4, 4, 16, 10, FAKE + 2), ESHAPE),   # status word misaligned
    ((None, None, 0, 4, 16, 10, None), OK),            # empty batch: nothing to check
])
def test_check_tables_validation(args, status):
    assert pa.lib().pa_check_tables(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, -1, 10, 16, FAKE), ESHAPE),
    ((FAKE, 4, 0, 16, FAKE), ESHAPE),
    ((FAKE, 4, 10, 0, FAKE), ESHAPE),
    ((None, 4, 10, 16, FAKE), ENULL),
    ((FAKE, 4, 10, 16, None), ENULL),
    ((FAKE, 4, 10, 16, FAKE + 1), ESHAPE),
    ((None, 0, 10, 16, None), OK),
])
def test_check_slots_validation(args, status):
    assert pa.lib().pa_check_slots(*args, None) == status


def test_kernel_family_policy():
    L = pa.lib()
    assert L.pa_decode_kernel(32, 8, BF16, BF16, 0) == pa.FORCE_MFMA   # GQA group of 4
    assert L.pa_decode_kernel(64, 8, BF16, BF16, 0) == pa.FORCE_MFMA
    assert L.pa_decode_kernel(32, 32, F16, F16, 0) == pa.FORCE_MFMA    # plain MHA: one column
    assert L.pa_decode_kernel(4, 4, F32, F32, 0) == pa.FORCE_VALU      # fp32 cache
    assert L.pa_decode_kernel(32, 8, F32, BF16, 0) == pa.FORCE_VALU    # fp32 queries
    assert L.pa_decode_kernel(32, 32, F16, F16, pa.FORCE_MFMA) == pa.FORCE_MFMA
    assert L.pa_decode_kernel(32, 8, BF16, BF16, pa.FORCE_VALU) == pa.FORCE_VALU
    assert L.pa_decode_kernel(32, 8, F32, F32, pa.FORCE_MFMA) == EUNSUP
    assert L.pa_decode_kernel(30, 8, BF16, BF16, 0) == ESHAPE
    assert L.pa_decode_kernel(32, 8, F16, BF16, 0) == EDTYPE


def test_waves_flags():
    L = pa.lib()
    args = (256, 32, 8, 128, 16, 512, 1024, BF16, BF16)
    for w, flag in pa.WAVES_FLAG.items():
        assert L.pa_decode_waves(*args, flag) == w
        assert L.pa_decode_waves(*args, flag | pa.FORCE_VALU) == w
    # library choice: 4 waves from 1024-token partitions, 2 from 256, else 1
    assert L.pa_decode_waves(*args, 0) == 4                                     # 1024 tokens
    assert L.pa_decode_waves(*args[:6], 4096, BF16, BF16, 0) == 4
    assert L.pa_decode_waves(*args[:6], 1008, BF16, BF16, 0) == 2
    assert L.pa_decode_waves(*args[:6], 512, BF16, BF16, 0) == 2
    assert L.pa_decode_waves(*args[:6], 256, BF16, BF16, 0) == 2
    assert L.pa_decode_waves(*args[:6], 384, BF16, BF16, 0) == 2
    assert L.pa_decode_waves(*args[:6], 128, BF16, BF16, 0) == 1
    assert L.pa_decode_waves(4, 4, 4, 64, 16, 13, 0, F32, F32, 0) == 1          # one pass of 208
    assert L.pa_decode_waves(*args, 128) == EUNSUP
    assert L.pa_decode_waves(*args[:6], 24, BF16, BF16, 0) == ESHAPE  # not a block multiple
    assert L.pa_decode_waves(*args[:7], F16, BF16, pa.WAVES_2) == EDTYPE
    # grid: the sorted grid for partitions of 1024+ tokens whose order fits
    # (num_seqs * partitions <= 65536); below 1024 tokens the work list for
    # batches of up to 64 sequences (where it fits in LDS), else the sorted grid
    G, S, W = pa.NO_WORK_LIST, pa.SORTED_GRID, pa.WORK_LIST
    assert L.pa_decode_grid(*args, 0) == S                                      # 8 of 1024
    assert L.pa_decode_grid(*args[:6], 512, BF16, BF16, 0) == S                 # 256 sequences
    assert L.pa_decode_grid(64, 32, 8, 128, 16, 512, 512, BF16, BF16, 0) == W   # 64 sequences
    assert L.pa_decode_grid(65, 32, 8, 128, 16, 512, 512, BF16, BF16, 0) == S
    assert L.pa_decode_grid(64, 32, 8, 128, 16, 512, 1024, BF16, BF16, 0) == S
    assert L.pa_decode_grid(32, 40, 40, 128, 16, 256, 512, F16, F16, 0) == W    # skewed batch
    assert L.pa_decode_work_list(32, 40, 40, 128, 16, 256, 512, F16, F16, 0) == 1
    # a step's launches sort wherever the order fits (PA_DECODE_ORDERED asks for them)
    assert L.pa_decode_grid(32, 40, 40, 128, 16, 256, 512, F16, F16, pa.ORDERED) == S
    assert L.pa_decode_work_list(32, 40, 40, 128, 16, 256, 512, F16, F16, pa.ORDERED) == 0
    assert L.pa_decode_grid(32, 40, 40, 128, 16, 256, 512, F16, F16, pa.ORDERED | W) == W
    # the workspace covers the step's order too
    ws_step = L.pa_decode_workspace_size(32, 40, 40, 128, 16, 256, 512, F16, 0)
    ws_list = L.pa_decode_workspace_size(32, 40, 40, 128, 16, 256, 512, F16, W)
    assert ws_step == ws_list + -(-32 * 8 * 4 // 256) * 256 + 256
    assert L.pa_decode_grid(*args[:6], 2048, BF16, BF16, 0) == S                # 4 partitions
    assert L.pa_decode_grid(*args[:6], 8192, BF16, BF16, 0) == G                # one pass
    assert L.pa_decode_grid(*args[:6], 8192, BF16, BF16, W) == G
    assert L.pa_decode_grid(*args, G) == G and L.pa_decode_grid(*args, W) == W
    assert L.pa_decode_grid(*args, S | pa.FORCE_VALU) == S
    assert L.pa_decode_grid(4096, 32, 8, 128, 16, 512, 256, BF16, BF16, 0) == G  # order too big
    assert L.pa_decode_grid(4096, 32, 8, 128, 16, 512, 256, BF16, BF16, W) == G  # list too
    assert L.pa_decode_grid(1000, 32, 8, 128, 16, 512, 256, BF16, BF16, W) == W
    assert L.pa_decode_work_list(*args, 0) == 0
    assert L.pa_decode_work_list(*args, W) == 1
    assert L.pa_decode_work_list(*args[:6], 8192, BF16, BF16, W) == 0           # one pass
    assert L.pa_decode_work_list(*args, 128) == EUNSUP
    assert L.pa_decode_grid(*args, 128) == EUNSUP
    # the waves bits leave the kernel family alone
    assert L.pa_decode_kernel(32, 8, BF16, BF16, pa.WAVES_4) == pa.FORCE_MFMA
    assert L.pa_decode_kernel(32, 8, BF16, BF16, pa.WAVES_4 | pa.FORCE_VALU) == pa.FORCE_VALU


def test_partition_policy_and_workspace_size():
    L = pa.lib()
    # one pass when the longest context fits one partition: no workspace
    assert L.pa_decode_partition_size(4, 4, 4, 64, 16, 13, F32, 0) == 208
    assert L.pa_decode_workspace_size(4, 4, 4, 64, 16, 13, 0, F32, 0) == 0
    # about a quarter of the longest context, a power of two in [1024, 8192] ...
    assert L.pa_decode_partition_size(64, 32, 32, 128, 16, 128, F16, 0) == 1024    # 2048 max
    assert L.pa_decode_partition_size(32, 40, 40, 128, 16, 256, F16, 0) == 1024    # 4096 max
    assert L.pa_decode_partition_size(256, 32, 8, 128, 16, 512, BF16, 0) == 2048   # 8192 max
    assert L.pa_decode_partition_size(64, 64, 8, 128, 32, 1025, BF16, 0) == 8192   # 32800 max
    assert L.pa_decode_partition_size(16, 8, 8, 128, 16, 100000, BF16, 0) == 8192  # capped
    # ... halved (down to 512) until sequences x kv heads x partitions >= 256
    assert L.pa_decode_partition_size(1, 64, 8, 128, 16, 2048, BF16, 0) == 1024    # 1 x 32k
    assert L.pa_decode_partition_size(4, 64, 8, 128, 16, 2048, BF16, 0) == 4096    # 4 x 32k
    assert L.pa_decode_partition_size(1, 64, 8, 128, 16, 256, BF16, 0) == 512      # 1 x 4k
    assert L.pa_decode_partition_size(4, 8, 8, 128, 16, 40, BF16, 0) == 512        # 640 max
    assert L.pa_decode_partition_size(4, 8, 8, 128, 16, 30, BF16, 0) == 480        # one pass
    # workspace = (m, l) and a head_dim vector per (seq, q head, partition), 256-B aligned
    B, Hq, d, MB, bs, P = 256, 32, 128, 512, 16, 512
    n_part = MB * bs // P
    rows = B * Hq * n_part
    expect = -(-rows * 8 // 256) * 256 + -(-rows * d * 4 // 256) * 256
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, P, BF16, pa.NO_WORK_LIST) == expect
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, P, BF16, pa.WORK_LIST) == expect
    # the sorted grid (the library's choice here) adds its order, an int per (seq,
    # partition), and a 256-byte counter
    order = -(-B * n_part * 4 // 256) * 256 + 256
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, P, BF16, 0) == expect + order
    # the library's own size on the sorted grid from 2048 tokens: the device may
    # halve it, so the workspace covers the half (here 2048 -> 1024)
    assert L.pa_decode_partition_size(B, Hq, 8, d, bs, MB, BF16, 0) == 2048
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 0, BF16, 0) == \
        L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 1024, BF16, 0)
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 0, BF16, 0) > \
        L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 2048, BF16, 0)
    # below 2048 tokens, or off the sorted grid, the size is the one picked
    assert L.pa_decode_partition_size(64, 32, 32, 128, 16, 128, F16, 0) == 1024
    assert L.pa_decode_workspace_size(64, 32, 32, 128, 16, 128, 0, F16, 0) == \
        L.pa_decode_workspace_size(64, 32, 32, 128, 16, 128, 1024, F16, 0)
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 0, BF16, pa.NO_WORK_LIST) == \
        L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 2048, BF16, pa.NO_WORK_LIST)
    # one pass: none
    assert L.pa_decode_workspace_size(4, 8, 8, 128, 16, 30, 0, BF16, 0) == 0
    # the partition a launch used: no device copy where nothing is refined (the
    # host's pick); a refining shape needs its workspace
    used = L.pa_decode_partition_used
    assert used(None, 0, 64, 32, 32, 128, 16, 128, F16, 0, None) == 1024
    assert used(None, 0, B, Hq, 8, d, bs, MB, BF16, 0, None) == EWS
    assert used(None, 0, B, 30, 8, d, bs, MB, BF16, 0, None) == ESHAPE
    # forced partition sizes must be multiples of the block size; invalid -> 0
    assert L.pa_decode_workspace_size(B, Hq, 8, d, bs, MB, 24, BF16, 0) == 0
    assert L.pa_decode_partition_size(4, 3, 2, 128, 16, 8, BF16, 0) == ESHAPE


def _adv(**kw):
    a = dict(B=8, nq=6, bs=16, tok=FAKE, samp=FAKE, pos=FAKE, lens=FAKE, slots=FAKE, bt=FAKE, MB=4)
    a.update(kw)
    return pa.lib().pa_advance_step(a["B"], a["nq"], a["bs"], a["tok"], a["samp"], a["pos"],
                                    a["lens"], a["slots"], a["bt"], a["MB"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), ESHAPE),
    (dict(nq=-1), ESHAPE),
    (dict(nq=9), ESHAPE),
    (dict(MB=0), ESHAPE),
    (dict(bs=0), ESHAPE),
    (dict(tok=None), ENULL),
    (dict(samp=None), ENULL),
    (dict(slots=None), ENULL),
    (dict(bt=None), ENULL),
])
def test_advance_step_validation(kw, status):
    assert _adv(**kw) == status


def test_advance_step_empty_is_noop():
    assert _adv(B=0, nq=0, tok=None, samp=None, pos=None, lens=None, slots=None, bt=None) == OK

# ------------------------------------------------------------------ E4M3 caches

FP8 = 3


def _cw8(**kw):
    args = dict(k=FAKE, v=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, T=4, ks=512, vs=512, H=4, d=128,
                NB=10, bs=16, src=BF16, kscale=0.5, vscale=0.25)
    args.update(kw)
    return pa.lib().pa_cache_write_fp8(args["k"], args["v"], args["slots"], args["kc"],
                                       args["vc"], args["T"], args["ks"], args["vs"], args["H"],
                                       args["d"], args["NB"], args["bs"], args["src"],
                                       args["kscale"], args["vscale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(src=FP8), EDTYPE),          # sources are f32 / f16 / bf16
    (dict(src=7), EDTYPE),
    (dict(kscale=0.0), ESHAPE),
    (dict(vscale=-1.0), ESHAPE),
    (dict(kscale=float("inf")), ESHAPE),
    (dict(vscale=float("nan")), ESHAPE),
    (dict(d=96), EUNSUP),
    (dict(bs=12), EUNSUP),
    (dict(ks=100), ESHAPE),
    (dict(k=None), ENULL),
    (dict(kc=FAKE + 8), ESHAPE),
])
def test_cache_write_fp8_validation(kw, status):
    assert _cw8(**kw) == status


def test_plain_cache_write_rejects_fp8_caches():
    assert _cw(dtype=FP8) == EDTYPE


def _dec8(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, kscale=0.5,
             vscale=0.25, bs=16, P=0, B=4, Hq=32, Hkv=8, d=128, NB=100, MB=64, qd=BF16, od=F32,
             ws=None, wsb=0, flags=pa.FORCE_VALU)
    a.update(kw)
    return pa.lib().pa_decode_fp8(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"],
                                  a["scale"], a["kscale"], a["vscale"], a["bs"], a["P"], a["B"],
                                  a["Hq"], a["Hkv"], a["d"], a["NB"], a["MB"], a["qd"], a["od"],
                                  a["ws"], a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qd=FP8), EDTYPE),                        # queries are f32 / f16 / bf16
    (dict(od=FP8), EDTYPE),
    (dict(qd=F16, od=BF16), EDTYPE),               # out: f32 or the query dtype
    (dict(kscale=0.0), ESHAPE),
    (dict(vscale=float("inf")), ESHAPE),
    (dict(flags=pa.FORCE_MFMA, qd=F16), EUNSUP),   # matrix cores: bfloat16 queries
    (dict(d=96), EUNSUP),
    (dict(ws=None, wsb=0, P=256), EWS),
    (dict(out=None), ENULL),
])
def test_decode_fp8_validation(kw, status):
    assert _dec8(**kw) == status


def test_decode_fp8_valid_argument_sets_pass_validation():
    """Argument sets that validate (B = 0 launches nothing)."""
    for kw in (dict(qd=F16, od=F16), dict(qd=F32), dict(qd=BF16, od=BF16, flags=pa.FORCE_MFMA)):
        assert _dec8(B=0, **kw) == OK


def test_plain_decode_rejects_fp8_caches():
    assert _dec(kvd=FP8) == EDTYPE


def test_fp8_kernel_family_policy():
    L = pa.lib()
    assert L.pa_decode_kernel(32, 8, BF16, FP8, 0) == pa.FORCE_MFMA   # GQA, bf16 queries
    assert L.pa_decode_kernel(32, 32, BF16, FP8, 0) == pa.FORCE_MFMA  # MHA
    assert L.pa_decode_kernel(32, 8, F16, FP8, 0) == pa.FORCE_VALU    # f16 queries
    assert L.pa_decode_kernel(32, 8, F32, FP8, 0) == pa.FORCE_VALU
    assert L.pa_decode_kernel(32, 8, F16, FP8, pa.FORCE_MFMA) == EUNSUP
    assert L.pa_decode_kernel(32, 8, FP8, FP8, 0) == EDTYPE
    # the workspace holds fp32 partials: it does not depend on the cache dtype
    assert L.pa_decode_workspace_size(4, 32, 8, 128, 16, 64, 256, FP8, 0) == \
        L.pa_decode_workspace_size(4, 32, 8, 128, 16, 64, 256, BF16, 0)



# ------------------------------------------------------------------ multi-query decode

def _decmq(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, kscale=1.0,
             vscale=1.0, bs=16, P=0, B=4, nq=4, Hq=32, Hkv=8, d=128, NB=100, MB=64, qd=BF16,
             kvd=BF16, od=F32, ws=None, wsb=0, flags=pa.FORCE_MFMA, fn="pa_decode_mq")
    a.update(kw)
    return getattr(pa.lib(), a["fn"])(
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"], a["kscale"],
        a["vscale"], a["bs"], a["P"], a["B"], a["nq"], a["Hq"], a["Hkv"], a["d"], a["NB"],
        a["MB"], a["qd"], a["kvd"], a["od"], a["ws"], a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(nq=0), ESHAPE),
    (dict(nq=17), ESHAPE),
    (dict(nq=9, Hq=8, Hkv=8), EUNSUP),            # 9 columns: no tile width, too many rows
    (dict(nq=5, Hq=8, Hkv=8, flags=pa.FORCE_VALU), OK),  # B = 0 below
    (dict(nq=16, Hq=16, Hkv=8, flags=pa.FORCE_VALU), EUNSUP),  # the vector ALUs hold 8 rows
    (dict(nq=3, flags=pa.FORCE_MFMA, qd=F32), EUNSUP),
    (dict(kscale=0.0), ESHAPE),
    (dict(Hq=30), ESHAPE),
    (dict(d=96), EUNSUP),
    (dict(out=None), ENULL),
    (dict(ws=None, wsb=0, P=256), EWS),
    (dict(fn="pa_decode_mq_partitions", ws=None, wsb=0, P=256), EWS),
    (dict(fn="pa_decode_mq_merge", ws=None, wsb=0, P=256), EWS),
])
def test_decode_mq_validation(kw, status):
    if status == OK:
        kw = dict(kw, B=0)
    assert _decmq(**kw) == status


def test_decode_mq_workspace_counts_query_rows():
    """The multi-query workspace is the single-query one of num_seqs * num_queries rows;
    a buffer 16 bytes short of it is rejected."""
    L = pa.lib()
    need = L.pa_decode_workspace_size(4 * 4, 32, 8, 128, 16, 64, 256, BF16, 0)
    assert need > L.pa_decode_workspace_size(4, 32, 8, 128, 16, 64, 256, BF16, 0)
    assert _decmq(P=256, ws=FAKE, wsb=need - 16) == EWS


def test_decode_mq_kernel_policy():
    L = pa.lib()
    k = L.pa_decode_mq_kernel
    assert k(1, 32, 8, BF16, BF16, 0) == L.pa_decode_kernel(32, 8, BF16, BF16, 0)
    assert k(2, 32, 32, F16, F16, 0) == pa.FORCE_MFMA     # MHA, 2 query tokens: 2 columns
    assert k(4, 32, 8, BF16, BF16, 0) == pa.FORCE_MFMA
    assert k(16, 8, 8, BF16, BF16, 0) == pa.FORCE_MFMA    # 16 columns of one head
    assert k(4, 64, 8, BF16, BF16, 0) == pa.FORCE_MFMA    # 32 columns: two tiles
    assert k(16, 16, 8, F16, F16, 0) == pa.FORCE_MFMA     # 16 queries x 2 heads
    assert k(16, 8, 8, BF16, BF16, pa.FORCE_VALU) == EUNSUP
    assert k(8, 8, 8, F32, F32, 0) == pa.FORCE_VALU       # fp32: vector ALUs, up to 8 rows
    assert k(10, 8, 8, F32, F32, 0) == EUNSUP
    for bad in (9, 11, 13, 14, 15):                      # no instantiated tile width
        assert k(bad, 8, 8, BF16, BF16, 0) == EUNSUP
    assert k(4, 32, 8, BF16, FP8, 0) == pa.FORCE_MFMA
    assert k(4, 32, 8, F16, FP8, 0) == pa.FORCE_VALU
    assert k(0, 32, 8, BF16, BF16, 0) == ESHAPE


# ------------------------------------------------------------------ block copies

@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), ESHAPE),
    (dict(nb=0), ESHAPE),
    (dict(bb=0), ESHAPE),
    (dict(bb=24), ESHAPE),                     # not a multiple of 16
    (dict(kc=None), ENULL),
    (dict(pairs=None), ENULL),
    (dict(kc=FAKE + 8), ESHAPE),
    (dict(n=0, kc=None, vc=None, pairs=None), OK),   # nothing to copy, nothing launched
])
def test_copy_blocks_validation(kw, status):
    a = dict(kc=FAKE, vc=FAKE, pairs=FAKE, n=3, nb=10, bb=4096)
    a.update(kw)
    assert pa.lib().pa_copy_blocks(a["kc"], a["vc"], a["pairs"], a["n"], a["nb"], a["bb"],
                                   None) == status


def test_swap_blocks_validation():
    L = pa.lib()
    bad = (ctypes.c_int32 * 4)(0, 1, -1, 2)
    assert L.pa_swap_blocks(FAKE, FAKE, bad, 2, 4096, None) == ESHAPE
    assert L.pa_swap_blocks(FAKE, FAKE, bad, -1, 4096, None) == ESHAPE
    assert L.pa_swap_blocks(FAKE, FAKE, bad, 1, 0, None) == ESHAPE
    assert L.pa_swap_blocks(None, FAKE, bad, 1, 4096, None) == ENULL
    assert L.pa_swap_blocks(None, None, None, 0, 4096, None) == OK


def test_block_manager_argument_validation():
    L = pa.lib()
    h = ctypes.c_void_p()
    assert L.pa_bm_create(0, 16, 0, 0, ctypes.byref(h)) == ESHAPE
    assert L.pa_bm_create(8, 0, 0, 0, ctypes.byref(h)) == ESHAPE
    assert L.pa_bm_create(8, 16, -1, 0, ctypes.byref(h)) == ESHAPE
    assert L.pa_bm_create(8, 16, 0, 2, ctypes.byref(h)) == ESHAPE
    assert L.pa_bm_create(8, 16, 0, 0, None) == ENULL
    assert L.pa_bm_create(8, 16, 0, 1, ctypes.byref(h)) == OK
    try:
        assert L.pa_bm_add_sequence(h, 1, None, 5, None) == ENULL  # caching needs the ids
        assert L.pa_bm_add_sequence(h, 1, None, -1, None) == ESHAPE
        assert L.pa_bm_add_sequence(None, 1, None, 0, None) == ENULL
        n = ctypes.c_int32(0)
        assert L.pa_bm_append(h, None, None, 0, None, None, ctypes.byref(n)) == OK
        assert L.pa_bm_append(h, None, None, 1, None, None, ctypes.byref(n)) == ENULL
        assert L.pa_bm_ref_count(h, 8, ctypes.byref(n)) == ESHAPE
        assert L.pa_bm_free(h, 42) == ESEQ
    finally:
        L.pa_bm_destroy(h)


# ------------------------------------------------------------------ decode step

def _step(**kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, T=4, ks=1024, vs=1024, out=FAKE, q=FAKE, kc=FAKE,
             vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, bs=16, P=0, B=4, Hq=32, Hkv=8, d=128, NB=100,
             MB=64, qd=BF16, kvd=BF16, od=F32, ws=None, wsb=0, flags=pa.FORCE_VALU,
             fn="pa_decode_step")
    a.update(kw)
    return getattr(pa.lib(), a["fn"])(
        a["k"], a["v"], a["slots"], a["T"], a["ks"], a["vs"], a["out"], a["q"], a["kc"], a["vc"],
        a["bt"], a["cl"], a["scale"], a["bs"], a["P"], a["B"], a["Hq"], a["Hkv"], a["d"],
        a["NB"], a["MB"], a["qd"], a["kvd"], a["od"], a["ws"], a["wsb"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kvd=FP8, qd=BF16), EDTYPE),          # E4M3 caches: write and decode separately
    (dict(ks=100), ESHAPE),                    # the write's arguments ...
    (dict(k=None), ENULL),
    (dict(T=-1), ESHAPE),
    (dict(Hq=30), ESHAPE),                     # ... and the decode's
    (dict(qd=F16), EDTYPE),
    (dict(ws=None, wsb=0, P=256), EWS),
    (dict(fn="pa_decode_step_partitions", ws=None, wsb=0, P=256), EWS),
    (dict(flags=64), EUNSUP),             # ordered: a step orders its items itself
    (dict(flags=128), EUNSUP),
    (dict(T=0, B=0, out=None, q=None, bt=None, cl=None), OK),   # nothing to do
])
def test_decode_step_validation(kw, status):
    assert _step(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(kvd=FP8, qd=BF16), EDTYPE),          # an E4M3 write needs its scales ...
    (dict(kvd=FP8, qd=BF16, T=0, ws=None, wsb=0, P=256), EWS),  # ... no write: decode checks
    (dict(T=-1), ESHAPE),
    (dict(k=None), ENULL),
    (dict(Hq=30), ESHAPE),
    (dict(ws=None, wsb=0, P=256), EWS),        # the order lives in the workspace
    (dict(flags=128), EUNSUP),
    (dict(T=0, B=0, out=None, q=None, bt=None, cl=None), OK),   # nothing to do
])
def test_decode_order_validation(kw, status):
    assert _step(fn="pa_decode_order", **kw) == status


def _order_fp8(**kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, T=4, ks=1024, vs=1024, src=BF16, ksc=0.25, vsc=0.5,
             out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.1, bs=16, P=0, B=4,
             Hq=32, Hkv=8, d=128, NB=100, MB=64, qd=BF16, od=F32, ws=None, wsb=0,
             flags=pa.FORCE_VALU)
    a.update(kw)
    return pa.lib().pa_decode_order_fp8(
        a["k"], a["v"], a["slots"], a["T"], a["ks"], a["vs"], a["src"], a["ksc"], a["vsc"],
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"], a["bs"], a["P"],
        a["B"], a["Hq"], a["Hkv"], a["d"], a["NB"], a["MB"], a["qd"], a["od"], a["ws"], a["wsb"],
        a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(src=FP8), EDTYPE),                   # the write's source: f32 / f16 / bf16
    (dict(ksc=0.0), ESHAPE),                   # scales must be positive and finite
    (dict(vsc=float("inf")), ESHAPE),
    (dict(ks=100), ESHAPE),
    (dict(k=None), ENULL),
    (dict(T=-1), ESHAPE),
    (dict(Hq=30), ESHAPE),                     # the decode's arguments
    (dict(qd=FP8), EDTYPE),                    # queries are f32, f16 or bf16
    (dict(ws=None, wsb=0, P=256), EWS),        # the order lives in the workspace
    (dict(flags=128), EUNSUP),
    (dict(T=0, B=0, out=None, q=None, bt=None, cl=None), OK),   # nothing to do
])
def test_decode_order_fp8_validation(kw, status):
    assert _order_fp8(**kw) == status


def test_ordered_flag_is_known_and_refused_for_multi_query():
    L = pa.lib()
    assert L.pa_decode_kernel(32, 8, BF16, BF16, pa.ORDERED) == pa.FORCE_MFMA
    assert L.pa_decode_workspace_size(4, 32, 8, 128, 16, 64, 256, BF16, pa.ORDERED) == \
        L.pa_decode_workspace_size(4, 32, 8, 128, 16, 64, 256, BF16, 0)
    f32 = 1.0
    st = L.pa_decode_mq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, f32, f32, 16, 0, 4, 2, 32, 8, 128,
                        100, 64, BF16, BF16, F32, None, 0, pa.ORDERED, None)
    assert st == EUNSUP
