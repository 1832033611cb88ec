"""GPU parity at the library's size limits, through the C ABI, against the fp64 oracle.

- The most partitions one sequence may have: 65535 blocks of 16 tokens (1,048,560
  positions) in 16-token partitions, so 65535 partial results per row to merge,
  next to a 5-token sequence; also the same context in one pass (one workgroup
  streaming a million positions) and at the library's own partition size.
- More sequences in one batch (70,000) than one grid dimension holds (65,535),
  each split into up to three partitions, so the merge steps over the batch.

Both kernel families, every output row against the oracle (2e-3 max absolute error
with 16-bit caches, fp32 accumulation, the oracle in fp64 on the same rounded inputs).
"""
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

TOL_ABS_HALF = 2e-3
KERNELS = {"valu": pa.FORCE_VALU, "mfma": pa.FORCE_MFMA}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _state(cfg):
    wl = Workload(cfg)
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    gs.write_step(0)
    st.write_step(0)
    return wl, gs, st.decode(0, threads=8)


def test_most_partitions_per_sequence():
    cfg = custom_config("max-parts", [65535 * 16, 5], 8, 1, 128, "bf16", 16, seed=61)
    wl, gs, ref = _state(cfg)
    assert wl.max_blocks_per_seq == 65535
    one_pass = wl.max_blocks_per_seq * cfg.block_size
    for kernel, flags in KERNELS.items():
        for p in (16, one_pass, 0):
            _say(f"1,048,560 + 5 positions, partition {p}, {kernel}")
            out = gs.decode(0, partition_size=p, flags=flags)
            torch.cuda.synchronize()
            err = max_abs_err(out, ref)
            assert err <= TOL_ABS_HALF, f"partition {p}, {kernel}: max abs error {err:.3e}"


def test_batch_beyond_one_grid_dimension():
    lens = np.random.default_rng(7).integers(1, 49, size=70000).tolist()
    lens[-1] = 48  # the last sequence, past the first 65535, has three partitions of 16
    cfg = custom_config("wide-batch", lens, 2, 1, 64, "f16", 16, seed=62)
    wl, gs, ref = _state(cfg)
    for kernel, flags in KERNELS.items():
        for p in (16, 32):
            _say(f"70,000 sequences, partition {p}, {kernel}")
            assert pa.decode_grid(cfg.num_seqs, 2, 1, 64, 16, wl.max_blocks_per_seq, p,
                                  gs.kc.dtype, gs.kc.dtype, flags) == "grid"
            out = gs.decode(0, partition_size=p, flags=flags)
            torch.cuda.synchronize()
            err = max_abs_err(out, ref)
            assert err <= TOL_ABS_HALF, f"partition {p}, {kernel}: max abs error {err:.3e}"
