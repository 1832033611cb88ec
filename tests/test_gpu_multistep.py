"""GPU: the device advance step and an 8-step decode loop captured in a HIP graph.

pa_advance_step is compared bit-exactly with the oracle's advance step; the
captured loop (cache write -> decode -> advance, eight times) is replayed
several times, each replay checked bit-exactly against the eager run of the
same calls and, within tolerance, against the oracle stepping in lockstep.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import pagedattention_kv_cache_amd as pa
from pagedattention_kv_cache_amd.workloads import Workload, custom_config, raw_bits
from tests.gpu_harness import GpuState, max_abs_err, oracle_state_empty

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    oracle.build(force=False)


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_advance_step_matches_oracle(bs):
    rng = np.random.default_rng(bs)
    B, nq, MB = 37, 30, 6
    bt = rng.integers(0, 1000, size=(B, MB)).astype(np.int32)
    bt[rng.random((B, MB)) < 0.15] = -1  # blocks not allocated yet
    pos = rng.integers(0, MB * bs + 3, size=B).astype(np.int64)  # some step past the table
    pos[:6] = np.arange(6) * bs + bs - 1  # next position starts a new block
    state = {
        "input_tokens": rng.integers(0, 1000, size=B).astype(np.int64),
        "input_positions": pos,
        "seq_lens": (pos + 1).astype(np.int32),
        "slot_mapping": rng.integers(0, 1000, size=B).astype(np.int64),
    }
    sampled = rng.integers(0, 128256, size=nq).astype(np.int64)
    dev = {k: torch.from_numpy(v.copy()).cuda() for k, v in state.items()}
    pa.advance_step(nq, bs, dev["input_tokens"], torch.from_numpy(sampled).cuda(),
                    dev["input_positions"], dev["seq_lens"], dev["slot_mapping"],
                    torch.from_numpy(bt).cuda())
    oracle.advance_step(nq, bs, state["input_tokens"], sampled, state["input_positions"],
                        state["seq_lens"], state["slot_mapping"], bt)
    torch.cuda.synchronize()
    for k in state:
        assert np.array_equal(dev[k].cpu().numpy(), state[k]), k


def _device_state(wl: Workload):
    st = wl.initial_state()
    return {k: torch.from_numpy(v.copy()).cuda() for k, v in st.items()}


def _run_steps(gs: GpuState, wl: Workload, state, outs, sampled, ws, flags):
    c = wl.cfg
    for s in range(c.steps):
        pa.cache_write(gs.step_k[s], gs.step_v[s], state["slot_mapping"], gs.kc, gs.vc)
        pa.decode(outs[s], gs.q[s], gs.kc, gs.vc, gs.block_tables, state["seq_lens"],
                  c.attn_scale(), c.block_size, c.partition_size, ws, flags)
        pa.advance_step(c.num_seqs, c.block_size, state["input_tokens"], sampled[s],
                        state["input_positions"], state["seq_lens"], state["slot_mapping"],
                        gs.block_tables)


@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_multistep_graph_replays_match_eager_and_oracle(kernel):
    flags = {"auto": pa.AUTO, "valu": pa.FORCE_VALU}[kernel]
    cfg = custom_config("ms-graph", [1, 31, 32, 33, 500, 1000], 8, 2, 128, "bf16", 32,
                        seed=61, steps=8, partition_size=256)
    wl = Workload(cfg)
    c = cfg
    st = oracle_state_empty(wl)
    gs = GpuState(wl, oracle_state=st)
    torch.cuda.synchronize()
    kc0, vc0 = gs.kc.clone(), gs.vc.clone()
    sampled = torch.from_numpy(wl.sampled_tokens()).cuda()
    ws_bytes = pa.decode_workspace_size(c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                        c.block_size, wl.max_blocks_per_seq, c.partition_size,
                                        torch.bfloat16, flags)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    # eager reference run
    state = _device_state(wl)
    eager_out = [torch.empty(gs.q[0].shape, device="cuda") for _ in range(c.steps)]
    _run_steps(gs, wl, state, eager_out, sampled, ws, flags)
    torch.cuda.synchronize()
    eager_state = {k: v.clone() for k, v in state.items()}
    eager_k, eager_v = gs.kc.clone(), gs.vc.clone()

    # the oracle steps through the same eight steps with its own advance
    ost = wl.initial_state()
    samp = wl.sampled_tokens()
    for s in range(c.steps):
        oracle.cache_write(raw_bits(st.step_k[s]), raw_bits(st.step_v[s]), ost["slot_mapping"],
                           st.kc, st.vc, c.dtype)
        ref = oracle.decode(raw_bits(st.q[s]), c.dtype, st.kc, st.vc, c.dtype, wl.block_tables,
                            ost["seq_lens"], c.attn_scale(), threads=4)
        assert max_abs_err(eager_out[s], ref) <= 2e-3, f"step {s}"
        oracle.advance_step(c.num_seqs, c.block_size, ost["input_tokens"], samp[s],
                            ost["input_positions"], ost["seq_lens"], ost["slot_mapping"],
                            wl.block_tables)
    assert np.array_equal(raw_bits(eager_k.cpu()), st.kc)
    assert np.array_equal(raw_bits(eager_v.cpu()), st.vc)
    for k in ost:
        assert np.array_equal(eager_state[k].cpu().numpy(), ost[k]), k

    # capture the same eight steps once, replay three times from the initial state
    gs.kc.copy_(kc0)
    gs.vc.copy_(vc0)
    state = _device_state(wl)
    graph_out = [torch.empty(gs.q[0].shape, device="cuda") for _ in range(c.steps)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run_steps(gs, wl, state, graph_out, sampled, ws, flags)
    init = _device_state(wl)
    for rep in range(3):
        gs.kc.copy_(kc0)  # eager work between replays
        gs.vc.copy_(vc0)
        for k in state:
            state[k].copy_(init[k])
        for o in graph_out:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(c.steps):
            assert torch.equal(graph_out[s], eager_out[s]), f"replay {rep} step {s}"
        # raw bits: the pools hold NaN poison, which never compares equal as floats
        assert torch.equal(gs.kc.view(torch.int16), eager_k.view(torch.int16)), f"replay {rep}"
        assert torch.equal(gs.vc.view(torch.int16), eager_v.view(torch.int16)), f"replay {rep}"
        for k in state:
            assert torch.equal(state[k], eager_state[k]), f"replay {rep} {k}"


@pytest.mark.parametrize("lens_seed,n_seqs,partition", [(5, 6, 256), (6, 80, 256), (7, 40, 1024)])
def test_one_step_graph_replays_match_eager(lens_seed, n_seqs, partition):
    """One decode step (cache write, then decode with its partition merge)
    captured in a HIP graph and replayed three times, with eager work in
    between: every replay bit-identical to the eager run.  The three cases
    take the three deals of a partitioned launch: the LDS work list (6
    sequences, 256-token partitions), the sorted order dealt in fixed rounds
    (80 sequences, 256) and dealt from the counter (1024)."""
    rng = np.random.default_rng(lens_seed)
    lens = rng.integers(1, 3000, size=n_seqs).tolist()
    cfg = custom_config(f"g1-{n_seqs}-{partition}", lens, 8, 2, 128, "bf16", 16,
                        seed=70 + lens_seed, partition_size=partition)
    wl = Workload(cfg)
    c = cfg
    gs = GpuState(wl)
    B, MB = c.num_seqs, wl.max_blocks_per_seq
    want = {256: pa.WORK_LIST if n_seqs <= 64 else pa.SORTED_GRID, 1024: pa.SORTED_GRID}[partition]
    assert pa.decode_grid(B, 8, 2, 128, 16, MB, partition, torch.bfloat16, torch.bfloat16,
                          pa.AUTO) == pa.GRID_NAMES[want]
    ws_bytes = pa.decode_workspace_size(B, 8, 2, 128, 16, MB, partition, torch.bfloat16, pa.AUTO)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    slots = torch.from_numpy(wl.step_slots(0)).cuda()
    torch.cuda.synchronize()
    kc0, vc0 = gs.kc.clone(), gs.vc.clone()

    def step(out):
        pa.cache_write(gs.step_k[0], gs.step_v[0], slots, gs.kc, gs.vc)
        pa.decode(out, gs.q[0], gs.kc, gs.vc, gs.block_tables, gs.ctx[0], c.attn_scale(),
                  c.block_size, partition, ws)

    eager = torch.empty(gs.q[0].shape, device="cuda")
    step(eager)
    torch.cuda.synchronize()
    assert torch.isfinite(eager).all()
    graph_out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graph_out)
    for rep in range(3):
        gs.kc.copy_(kc0)  # eager work between replays
        gs.vc.copy_(vc0)
        graph_out.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graph_out, eager), f"replay {rep}"
