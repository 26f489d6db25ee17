"""Seeded random units against the oracle, every element, bit for bit.

Each case draws its unit and call from a seeded generator: 1 to 4 tensors of 1
or 2 dimensions (from a single element to a few hundred thousand; a third of
the units hold 1M-3M elements), the sharding factor, the rank, the fold (flat
over n_grads rows, hybrid sharding over R replica groups, or bf16 partial
sums), where each gradient row's window sits (on an 8-byte boundary at a
random 8-byte step past a 256-byte one, or 2-6 bytes past one, all rows alike
or each its own), whether the fp32 state sits 4 bytes off 16-byte alignment,
the bf16 emission, and the fused or the unfused entry points. One optimizer step runs on the GPU from a flattened
master and zero m and v; master, m, v and the emitted parameter are compared
with the oracle on every element of the rank's window, and the bytes past the
window must be untouched. The draws reach the vector path (with and without
tiles in XCD runs: launches of 64 tiles or more whose windows start off a
128-byte line), the shifted-row path, the scalar path, ragged tails, ranks
holding only pad, and compile-time and run-time row counts.
"""

import numpy as np
import pytest
import torch

from conftest import gpu_available
from shard_cases import FP32_SENTINEL, HP, Case, to_np
from oracle import fsdp_oracle as O

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import sharded_flatparameter_flatten_amd as fsdp  # noqa: E402

N_CASES = 160


def draw(i):
    """The unit, the fold and the buffer placement of case i."""
    rng = np.random.default_rng(9000 + i)
    shapes = []
    big = rng.random() < 0.3          # a unit of 1M-3M elements: launches of 64+ tiles
    for _ in range(int(rng.integers(1, 5))):
        n = int(np.exp(rng.uniform(np.log(250_000) if big else 0,
                                   np.log(800_000 if big else 400_000))))
        if rng.random() < 0.5 and n > 8:
            a = int(rng.integers(1, 64))
            shapes.append((a, max(1, n // a)))
        else:
            shapes.append((n,))
    U = sum(int(np.prod(s)) for s in shapes)
    F = int(rng.choice([1, 2, 4] if big else [1, 2, 3, 4, 5, 7, 8, 11, 13, 16]))
    rank = int(rng.integers(0, F))
    fold = str(rng.choice(["flat", "flat", "hybrid", "bf16acc"]))
    replicas, bf16acc = 1, fold == "bf16acc"
    if fold == "hybrid":
        replicas = int(rng.integers(2, 1 + max(2, min(4, 64 // F))))
        n_grads = replicas * F
    else:
        n_grads = int(rng.choice([F, F, int(rng.integers(1, 13)), 16, 24]))
    n_grads = max(1, min(n_grads, 64))
    if replicas > 1 and n_grads != replicas * F:
        replicas = 1
    # keep the host oracle quick: at most about 8M row elements
    while U * n_grads > 8_000_000 and n_grads > 1:
        n_grads = max(1, n_grads // 2)
        replicas = 1
    # where each row's window sits: on an 8-byte boundary at a random 8-byte step past
    # a 256-byte one (the vector path; off a 128-byte line unless the step is a
    # multiple of 16), 2-6 bytes past one (the same for every row, or each its own)
    begin = rank * (-(-U // F))
    align = int((-begin) % 4)
    kind = str(rng.choice(["aligned", "aligned", "same", "mixed"]))
    if kind == "aligned":
        offs = [align + 4 * int(rng.integers(0, 30))] * n_grads
    elif kind == "same":
        offs = [int(rng.integers(0, 4))] * n_grads
    else:
        offs = [int(x) for x in rng.integers(0, 4, n_grads)]
    return dict(shapes=shapes, U=U, F=F, rank=rank, replicas=replicas, bf16acc=bf16acc,
                n_grads=n_grads, row_offs=offs, state_off=int(rng.random() < 0.15),
                emit=bool(rng.random() < 0.7), fused=bool(rng.random() < 0.7))


def run_case(d, i):
    case = Case(d["shapes"], d["F"], d["rank"], n_grads=d["n_grads"], config=600 + i,
                replicas=d["replicas"], bf16acc=d["bf16acc"])
    u = fsdp.Unit(case.shapes, case.F, case.rank)
    L = case.L
    n, S, U = L.shard_valid, L.S, L.U
    # gradient rows: U-element views starting row_offs[k] elements past a 256-byte boundary
    bufs = [torch.empty(U + 128, dtype=torch.bfloat16, device="cuda") for _ in range(d["n_grads"])]
    rows = [b[o:o + U] for b, o in zip(bufs, d["row_offs"])]
    case.device_grads(1, out=rows)
    # state: S elements (plus a sentinel tail) at state_off elements past 16-byte alignment
    o = d["state_off"]
    slabs = [torch.full((S + 64,), 0, dtype=torch.int32, device="cuda") for _ in range(3)]
    p, m, v = (sl.view(torch.float32)[o:o + S] for sl in slabs)
    flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], case.F)
    p.copy_(torch.from_numpy(flat.view(np.float32)[L.shard_begin:L.shard_begin + S].copy()))
    m.zero_()
    v.zero_()
    for sl in slabs:
        sl[o + n:].fill_(FP32_SENTINEL)   # past the window: must stay
    w = torch.empty(S, dtype=torch.bfloat16, device="cuda") if d["emit"] else None
    hp = fsdp.AdamWHparams(**HP.__dict__)
    if d["fused"]:
        if d["bf16acc"]:
            fsdp.reduce_adamw_shard_bf16acc(u, rows, p, m, v, w, hp, 1)
        elif d["replicas"] > 1:
            fsdp.reduce_adamw_shard_hybrid(u, d["replicas"], rows, p, m, v, w, hp, 1)
        else:
            fsdp.reduce_adamw_shard(u, rows, p, m, v, w, hp, 1)
    else:
        g = torch.empty(S, dtype=torch.float32, device="cuda")
        if d["bf16acc"]:
            fsdp.reduce_shard_bf16acc(u, rows, g)
        elif d["replicas"] > 1:
            fsdp.reduce_shard_hybrid(u, d["replicas"], rows, g)
        else:
            fsdp.reduce_shard(u, rows, g)
        fsdp.adamw_shard(u, g, p, m, v, w, hp, 1)
    torch.cuda.synchronize()
    return case, (p, m, v, w), slabs


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_unit_every_element(i):
    d = draw(i)
    case, (p, m, v, w), slabs = run_case(d, i)
    n, o = case.L.shard_valid, d["state_off"]
    what = (f"case {i}: U={d['U']} F={d['F']} rank={d['rank']} n_grads={d['n_grads']} "
            f"replicas={d['replicas']} bf16acc={d['bf16acc']} rows+{d['row_offs'][:4]} "
            f"state+{o} emit={d['emit']} fused={d['fused']}")
    print(what, flush=True)
    for sl, name in zip(slabs, ("master", "exp_avg", "exp_avg_sq")):
        tail = to_np(sl)[o + n:]
        assert (tail.view(np.uint32) == FP32_SENTINEL).all(), f"{what}: {name} written past the window"
    if n == 0:
        return
    want = case.oracle_full(1, emit=d["emit"])[-1]
    got = [to_np(p)[:n].view(np.uint32), to_np(m)[:n].view(np.uint32), to_np(v)[:n].view(np.uint32)]
    for g_, w_, name in zip(got, want[:3], ("master", "exp_avg", "exp_avg_sq")):
        bad = np.flatnonzero(g_ != np.asarray(w_).view(np.uint32))
        assert bad.size == 0, f"{what}: {name}: {bad.size} elements differ, first {bad[:5].tolist()}"
    if d["emit"]:
        gw = to_np(w)[:n]
        bad = np.flatnonzero(gw != np.asarray(want[3]))
        assert bad.size == 0, f"{what}: bf16 param: {bad.size} elements differ, first {bad[:5].tolist()}"
