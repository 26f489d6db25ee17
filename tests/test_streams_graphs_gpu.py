"""The entry points on caller streams and inside HIP graphs.

Every device entry point only enqueues kernels on the stream it is given (no
allocation, no memset, no synchronisation), so it can run on any stream and
be captured into a HIP graph. Checked against eager runs on the null stream
and against the oracle.
"""

import gc

import numpy as np
import pytest
import torch

from datagen import workloads as W
from oracle import fsdp_oracle as O
from shard_cases import Case, assert_bits, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sharded_flatparameter_flatten_amd as fsdp  # noqa: E402

HPD = fsdp.AdamWHparams(**W.ADAMW)
DEV = "cuda"


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _state(case):
    u = fsdp.Unit(case.shapes, case.F, case.rank)
    flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], case.F)
    p = torch.from_numpy(flat.view(np.float32)[u.shard_begin:u.shard_begin + u.S].copy()).to(DEV)
    m = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    v = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    return u, p, m, v, w


def _bits(x):
    x = np.asarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


def test_side_stream_matches_oracle():
    case = Case(W.shapes(W.TINY), 4, 2, config=11)
    grads = case.device_grads(1)
    u, p, m, v, w = _state(case)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1)       # current stream = side
    side.synchronize()
    want = case.oracle_full(1)[-1]
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(to_np(got)[:u.shard_valid]), _bits(exp), name)


def test_two_units_on_two_streams_concurrently():
    cases = [Case(W.shapes(W.TINY), 4, 0, config=12), Case([(4096, 33), (17,)], 8, 5, config=13)]
    inputs = [(c.device_grads(1),) + _state(c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (grads, u, p, m, v, w), s in zip(inputs, streams):
        fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1, stream=s)
    for s in streams:
        s.synchronize()
    for c, (grads, u, p, m, v, w) in zip(cases, inputs):
        want = c.oracle_full(1)[-1]
        for got, exp in zip((p, m, v, w), want):
            assert_bits(_bits(to_np(got)[:u.shard_valid]), _bits(exp), "two streams")


def test_graph_captured_step_replays_like_eager():
    """Capture fused step + gather once; replay 3 times with eager work between."""
    shapes, F, rank = W.shapes(W.TINY), 4, 1
    case = Case(shapes, F, rank, config=14)
    grads = case.device_grads(1)
    units = [fsdp.Unit(shapes, F, r) for r in range(F)]
    u = units[rank]
    _, p0, m0, v0, _ = _state(case)
    shards = [torch.empty(u.S, dtype=torch.bfloat16, device=DEV) for _ in range(F)]
    for k, s in enumerate(shards):
        s.view(torch.int16).copy_(torch.arange(u.S, device=DEV, dtype=torch.int16) * (k + 3))

    # eager reference: three steps from the same start, t fixed at 2
    pe, me, ve = p0.clone(), m0.clone(), v0.clone()
    she = [s.clone() for s in shards]
    oute = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    eager = []
    for _ in range(3):
        fsdp.reduce_adamw_shard(u, grads, pe, me, ve, she[rank], HPD, 2)
        fsdp.cast_unflatten(u, she, oute)
        torch.cuda.synchronize()
        eager.append([to_np(x).copy() for x in (pe, me, ve, she[rank])] +
                     [to_np(o).copy() for o in oute])

    pg, mg, vg = p0.clone(), m0.clone(), v0.clone()
    shg = [s.clone() for s in shards]
    outg = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        graph.capture_begin()
        fsdp.reduce_adamw_shard(u, grads, pg, mg, vg, shg[rank], HPD, 2)
        fsdp.cast_unflatten(u, shg, outg)
        graph.capture_end()
    torch.cuda.synchronize()
    # capture records without running: state must be untouched
    assert torch.equal(pg.view(torch.int32), p0.view(torch.int32))
    scratch = torch.empty(1 << 20, device=DEV)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = [to_np(x).copy() for x in (pg, mg, vg, shg[rank])] + [to_np(o).copy() for o in outg]
        for a, b in zip(got, eager[rep]):
            assert_bits(_bits(a), _bits(b), f"replay {rep}")
        scratch.normal_()                  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_graph_captured_capped_launches_replay_like_eager():
    """Launches long enough to run with the occupancy cap (at least 8192 workgroups:
    9M-element units through the single-unit fused kernels, with 1 row, with 8 rows
    (the staged one-tile kernel) and with 11 rows (the run-time fold in it), and 30
    units of 300K through the batched kernel) captured into a graph: every replay
    equals eager."""
    bigs = [Case([(4096, 2200)], 1, 0, n_grads=ng, config=15 + 40 * j)   # 8800 tiles each
            for j, ng in enumerate((1, 8, 11))]
    mids = [Case([(600, 500)], 1, 0, config=16 + j) for j in range(30)]   # 30 x 293 tiles
    cases = bigs + mids
    nb = len(bigs)
    units = [fsdp.Unit(c.shapes, c.F, c.rank) for c in cases]
    grads = [c.device_grads(1) for c in cases]
    start = [_state(c)[1:4] for c in cases]
    torch.cuda.synchronize()

    def state_copy():
        return [tuple(x.clone() for x in s) + (torch.empty(u.S, dtype=torch.bfloat16, device=DEV),)
                for s, u in zip(start, units)]

    def step(st):
        for j in range(nb):
            p, m, v, w = st[j]
            fsdp.reduce_adamw_shard(units[j], grads[j], p, m, v, w, HPD, 3)
        fsdp.reduce_adamw_units([(u, g) + tuple(s) for u, g, s in zip(units[nb:], grads[nb:], st[nb:])],
                                HPD, 3)

    eager_st = state_copy()
    eager = []
    for _ in range(3):
        step(eager_st)
        torch.cuda.synchronize()
        eager.append([to_np(x).copy() for s in eager_st for x in s])
    graph_st = state_copy()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        graph.capture_begin()
        step(graph_st)
        graph.capture_end()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device=DEV)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = [to_np(x).copy() for s in graph_st for x in s]
        for a, b in zip(got, eager[rep]):
            assert_bits(_bits(a), _bits(b), f"replay {rep}")
        scratch.normal_()
        torch.cuda.synchronize()
