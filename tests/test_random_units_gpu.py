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


# ---------------------------------------------------------------------------
# the copies: flatten/pad windows and unflatten, random units and placements
# ---------------------------------------------------------------------------

N_COPY_CASES = 64


def draw_copy(i):
    rng = np.random.default_rng(19000 + i)
    shapes = []
    for _ in range(int(rng.integers(1, 9))):
        n = int(np.exp(rng.uniform(0, np.log(300_000))))
        shapes.append((n,) if rng.random() < 0.6 or n < 4 else (int(rng.integers(1, 9)), n // 4 + 1))
    F = int(rng.choice([1, 2, 3, 4, 7, 8, 13, 16]))
    U = sum(int(np.prod(s)) for s in shapes)
    S = -(-U // F)
    begin = int(rng.integers(0, F * S))
    length = int(rng.integers(0, F * S - begin + 1))
    return dict(shapes=shapes, F=F, rank=int(rng.integers(0, F)), begin=begin, length=length,
                dtype=str(rng.choice(["f32", "bf16"])), out=str(rng.choice(["f32", "bf16"])),
                src_off=int(rng.integers(0, 8)), dst_off=int(rng.integers(0, 8)))


def host_tensor_bits(rng_seed, shape, dtype):
    rng = np.random.default_rng(rng_seed)
    n = int(np.prod(shape))
    if dtype == "f32":
        return rng.standard_normal(n).astype(np.float32).view(np.uint32)
    return (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def to_dev(bits, off):
    """bits as a device tensor starting `off` elements into a larger buffer."""
    tdtype = torch.int32 if bits.dtype == np.uint32 else torch.int16
    fdtype = torch.float32 if bits.dtype == np.uint32 else torch.bfloat16
    buf = torch.zeros(bits.size + 16, dtype=tdtype, device="cuda")
    buf[off:off + bits.size] = torch.from_numpy(bits.view(np.int32 if bits.dtype == np.uint32
                                                          else np.int16)).cuda()
    return buf.view(fdtype)[off:off + bits.size]


@pytest.mark.parametrize("i", range(N_COPY_CASES))
def test_random_copies_every_element(i):
    """flatten_pad of a random window of the padded flat buffer (tensors and the
    destination at random element offsets), and unflatten of the F shards into
    per-tensor outputs (fp32 or bf16 on each side), against the oracle, bit for bit,
    with the bytes around each destination untouched."""
    d = draw_copy(i)
    u = fsdp.Unit(d["shapes"], d["F"], d["rank"])
    L = O.unit_layout(d["shapes"], d["F"], d["rank"])
    what = f"copy case {i}: {d}"
    print(what, flush=True)
    # flatten_pad: window [begin, begin + length) of the padded flat buffer
    host = [host_tensor_bits(29000 + 31 * i + j, s, d["dtype"]) for j, s in enumerate(d["shapes"])]
    dev = [to_dev(h, (d["src_off"] + j) % 8) for j, h in enumerate(host)]
    want = O.flatten_pad(host, d["F"], d["begin"], d["length"])
    sent = 0x7FC00001 if d["dtype"] == "f32" else 0x7FC1
    dst_bits = np.full(d["length"] + 16, sent, dtype=np.uint32 if d["dtype"] == "f32" else np.uint16)
    dst_buf = to_dev(dst_bits, 0)
    dst = dst_buf[d["dst_off"]:d["dst_off"] + d["length"]]
    fsdp.flatten_pad(u, dev, dst, begin=d["begin"], length=d["length"])
    torch.cuda.synchronize()
    got = to_np(dst_buf)
    got = got.view(np.uint32) if got.dtype == np.float32 else got
    o = d["dst_off"]
    assert (got[:o] == sent).all() and (got[o + d["length"]:] == sent).all(), f"{what}: flatten guards"
    bad = np.flatnonzero(got[o:o + d["length"]] != want)
    assert bad.size == 0, f"{what}: flatten: {bad.size} differ, first {bad[:5].tolist()}"
    # unflatten: the F shards of the whole padded buffer into per-tensor outputs
    full = O.flatten_pad(host, d["F"])
    S = L.S
    shards = [to_dev(full[k * S:(k + 1) * S].copy(), (d["src_off"] + k) % 8) for k in range(d["F"])]
    want_t = O.unflatten([full[k * S:(k + 1) * S].view(np.float32) if d["dtype"] == "f32"
                          else full[k * S:(k + 1) * S] for k in range(d["F"])], L, d["shapes"],
                         out=d["out"])
    osent = 0x7FC00001 if d["out"] == "f32" else 0x7FC1
    outs, bufs = [], []
    for j, s in enumerate(d["shapes"]):
        n = int(np.prod(s))
        b = to_dev(np.full(n + 16, osent, dtype=np.uint32 if d["out"] == "f32" else np.uint16), 0)
        oo = (d["dst_off"] + 3 * j) % 8
        outs.append(b[oo:oo + n])
        bufs.append((b, oo, n))
    fsdp.unflatten(u, shards, outs)
    torch.cuda.synchronize()
    for j, ((b, oo, n), w_) in enumerate(zip(bufs, want_t)):
        g = to_np(b)
        g = g.view(np.uint32) if g.dtype == np.float32 else g
        wb = np.asarray(w_).reshape(-1)
        wb = wb.view(np.uint32) if wb.dtype == np.float32 else wb
        assert (g[:oo] == osent).all() and (g[oo + n:] == osent).all(), f"{what}: tensor {j} guards"
        bad = np.flatnonzero(g[oo:oo + n] != wb)
        assert bad.size == 0, f"{what}: unflatten tensor {j}: {bad.size} differ, first {bad[:5].tolist()}"


# ---------------------------------------------------------------------------
# the batched many-unit step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("i", range(8))
def test_random_unit_lists_every_element(i):
    """fsdp_reduce_adamw_units over a random list of units (small ones batched,
    larger ones launched alone; rows and state at random placements), against the
    oracle unit by unit, every element."""
    rng = np.random.default_rng(39000 + i)
    F = int(rng.choice([2, 4, 8]))
    n_grads = int(rng.choice([F, max(1, F // 2), 8]))
    steps, cases = [], []
    for j in range(int(rng.integers(2, 12))):
        big = rng.random() < 0.2
        n = int(np.exp(rng.uniform(np.log(4_000_000) if big else 0,
                                   np.log(9_000_000 if big else 300_000))))
        shapes = [(n,)] if rng.random() < 0.5 else [(max(1, n // 3),), (max(1, n - n // 3),)]
        case = Case(shapes, F, int(rng.integers(0, F)), n_grads=n_grads, config=700 + 16 * i + j)
        u = fsdp.Unit(case.shapes, F, case.rank)
        L = case.L
        roff = int(rng.integers(0, 4))
        rows = [torch.empty(L.U + 8, dtype=torch.bfloat16, device="cuda")[roff:roff + L.U]
                for _ in range(n_grads)]
        case.device_grads(1, out=rows)
        flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], F)
        p = torch.from_numpy(flat.view(np.float32)[L.shard_begin:L.shard_begin + L.S].copy()).cuda()
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        w = torch.empty(L.S, dtype=torch.bfloat16, device="cuda") if rng.random() < 0.7 else None
        steps.append((u, rows, p, m, v, w))
        cases.append(case)
    fsdp.reduce_adamw_units(steps, fsdp.AdamWHparams(**HP.__dict__), 1)
    torch.cuda.synchronize()
    for j, (case, (u, rows, p, m, v, w)) in enumerate(zip(cases, steps)):
        n = case.L.shard_valid
        if n == 0:
            continue
        want = case.oracle_full(1, emit=w is not None)[-1]
        for got, exp, name in zip((p, m, v), want[:3], ("master", "exp_avg", "exp_avg_sq")):
            bad = np.flatnonzero(to_np(got)[:n].view(np.uint32) != np.asarray(exp).view(np.uint32))
            assert bad.size == 0, f"list {i} unit {j} (U={case.L.U}): {name}: {bad.size} differ"
        if w is not None:
            bad = np.flatnonzero(to_np(w)[:n] != np.asarray(want[3]))
            assert bad.size == 0, f"list {i} unit {j}: bf16 param: {bad.size} differ"
