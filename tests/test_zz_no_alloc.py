"""pa_decode_noalloc: the decode with the library's static device scratch as
its workspace, for callers that cannot allocate.  Its output must equal
pa_decode's (same kernels, caller-allocated workspace) bit for bit, call after
call on the same scratch, and stay within tolerance of the oracle; problems
whose workspace would exceed the scratch are refused before any launch."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import Workload, custom_config
from tests.gpu_harness import GpuState, max_abs_err, oracle_state_empty

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


def _case(name, lens, hq, hkv, dtype, bs, seed):
    cfg = custom_config(name, lens, hq, hkv, 128, dtype, bs, seed=seed)
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    return cfg, wl, gs, st


def _both(cfg, wl, gs, partition_size, flags=pa.AUTO):
    """(decode_noalloc output, decode output) on the same inputs, NaN-prefilled."""
    c = cfg
    args = (gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(), c.block_size,
            partition_size)
    out_n = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    pa.decode_noalloc(out_n, *args, flags)
    out_d = torch.full(gs.q[0].shape, float("nan"), device="cuda")
    pa.decode(out_d, *args, None, flags)
    torch.cuda.synchronize()
    return out_n, out_d


def test_noalloc_matches_decode_on_consecutive_calls():
    """Two calls in a row on one GPU's scratch, the second on a smaller batch
    (and a third that needs no workspace, then the first again): each equals
    pa_decode bit for bit and the oracle within 2e-3."""
    rng = np.random.default_rng(7)
    big_lens = np.clip(np.rint(np.exp(rng.normal(np.log(1024), 1.0, 200))), 1, 6000)
    big = _case("na-big", big_lens.astype(int).tolist(), 32, 8, "bf16", 16, seed=71)
    small = _case("na-small", [1, 17, 300, 513, 1500, 40], 40, 40, "f16", 16, seed=72)
    cases = [(big, 0), (small, 256), (small, 0), (big, 0)]
    for (cfg, wl, gs, st), p in cases:
        need = pa.decode_workspace_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, 128,
                                        cfg.block_size, wl.max_blocks_per_seq, p, gs.kc.dtype,
                                        pa.AUTO)
        _say(f"{cfg.name} partition {p}: workspace {need} of {pa.SCRATCH_BYTES} bytes")
        assert need <= pa.SCRATCH_BYTES
        out_n, out_d = _both(cfg, wl, gs, p)
        assert torch.isfinite(out_n).all()
        assert torch.equal(out_n, out_d), "decode_noalloc differs from decode"
        err = max_abs_err(out_n, st.decode(0, threads=16))
        _say(f"  err vs oracle {err:.3e}")
        assert err <= 2e-3


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    """A batch whose partition workspace would exceed PA_SCRATCH_BYTES is
    refused with PA_ERR_SCRATCH (-9) before anything runs: out keeps its fill."""
    B, hq, hkv, d, bs, MB = 2048, 32, 8, 128, 16, 512
    need = pa.decode_workspace_size(B, hq, hkv, d, bs, MB, 256, torch.bfloat16, pa.AUTO)
    assert need > pa.SCRATCH_BYTES
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, hq, d), float("nan"), device="cuda")
    kc = torch.zeros(pa.key_cache_shape(8, hkv, d, bs, torch.bfloat16), dtype=torch.bfloat16,
                     device="cuda")
    vc = torch.zeros(pa.value_cache_shape(8, hkv, d, bs), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, MB, dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(out, q, kc, vc, bt, ctx, 0.1, bs, 256)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
