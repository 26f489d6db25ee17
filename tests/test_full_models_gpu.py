"""GPU parity on whole-model rank shards: every unit of the model, in order.

* Llama-7B-shaped rank shard: 32 block units + the root unit (untied
  embedding, final norm, lm_head), F=8, rank 0, ~842M params;
* Llama-70B-shaped rank shard: 80 GQA block units + root, F=8, rank 0,
  ~8.62B params (~138 GB of persistent state resident in HBM).
One fused reduce + AdamW + bf16 step per unit on one stream. Every element of
the named units and of the root unit (for the 7B shard through the per-unit
calls: of every unit) is checked against the oracle (run on host copies of
the generator's device fills, which are spot-checked against its host form
first), and sampled indices of every unit (with the oracle's inputs
regenerated on the host). Persistent bytes allocated equal
16 * sum(S) per the pages' budget.
"""

import gc

import numpy as np
import pytest
import torch

import datagen
from datagen import workloads as W
from oracle import fsdp_oracle as O
from shard_cases import HP, ModelShard, assert_bf16_ulp, assert_bits, assert_rel, gather, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sharded_flatparameter_flatten_amd as fsdp  # noqa: E402

HPD = fsdp.AdamWHparams(**W.ADAMW)


def check_every_element(ms, i, p_before, what, row_cache):
    """Unit i's window after the step against the oracle on every element. The
    oracle's inputs are host copies of the device fills (the rank window of
    each gradient row and the master before the step), each spot-checked
    against the host generator. row_cache keeps the host copies of rows that
    several units share."""
    L = ms.L[i]
    lo, n = L.shard_begin, L.shard_valid
    key = (id(ms.grads(i)), lo, n)
    if key not in row_cache:
        row_cache.clear()
        row_cache[key] = [to_np(g[lo:lo + n]) for g in ms.grads(i)]
    rows = row_cache[key]
    loc = ms.sample(i, 4096, seed=1000 + i)
    want_in = ms.inputs_at(i, loc)
    for k in (0, ms.F - 1):
        assert_bits(rows[k][loc], want_in[1][k], f"{what} row {k} fill")
    assert_bits(p_before[loc].view(np.uint32), want_in[0].view(np.uint32), f"{what} master fill")
    z = np.zeros(n, np.float32)
    want = O.reduce_adamw_shard(rows, O.unit_layout([(n,)], 1, 0), p_before, z, z.copy(), HP,
                                1, grad_scale=1.0 / ms.F, emit_bf16=True)
    assert_rel(to_np(ms.window(ms.p, i))[:n], want[0], what=what + " master (every element)")
    assert_rel(to_np(ms.window(ms.m, i))[:n], want[1], what=what + " exp_avg (every element)")
    assert_rel(to_np(ms.window(ms.v, i))[:n], want[2], what=what + " exp_avg_sq (every element)")
    assert_bf16_ulp(to_np(ms.window(ms.w, i))[:n], want[3], what=what + " bf16 (every element)")


def run_model(name, full_units, sparse_n, multi=False):
    wl = W.WORKLOADS[name]
    ms = ModelShard(wl["units"], wl["F"], wl["rank"], wl["config"])
    units = [fsdp.Unit(W.shapes(u), wl["F"], wl["rank"]) for u in wl["units"]]
    assert [u.S for u in units] == [L.S for L in ms.L]
    n_units = len(units)
    full_units = set(full_units) | {n_units - 1}
    torch.cuda.synchronize()
    p_before = {i: to_np(ms.window(ms.p, i))[:units[i].shard_valid] for i in sorted(full_units)}
    if multi:
        fsdp.reduce_adamw_units([(u, ms.grads(i), ms.window(ms.p, i), ms.window(ms.m, i),
                                  ms.window(ms.v, i), ms.window(ms.w, i))
                                 for i, u in enumerate(units)], HPD, 1)
    else:
        for i, u in enumerate(units):
            fsdp.reduce_adamw_shard(u, ms.grads(i), ms.window(ms.p, i), ms.window(ms.m, i),
                                    ms.window(ms.v, i), ms.window(ms.w, i), HPD, 1)
    torch.cuda.synchronize()
    row_cache = {}
    for i in range(n_units):
        what = f"{name} unit {i}"
        if i in full_units:
            check_every_element(ms, i, p_before.pop(i), what, row_cache)
            print(f"{what}: every element of {units[i].shard_valid:,} checked", flush=True)
        loc = ms.sample(i, sparse_n, seed=i)
        want = ms.oracle_sampled(i, loc)
        assert_rel(gather(ms.window(ms.p, i), loc), want[0], what=what + " master")
        assert_rel(gather(ms.window(ms.m, i), loc), want[1], what=what + " exp_avg")
        assert_rel(gather(ms.window(ms.v, i), loc), want[2], what=what + " exp_avg_sq")
        assert_bf16_ulp(gather(ms.window(ms.w, i), loc), want[3], what=what + " bf16")
    persistent = sum(u.persistent_bytes for u in units)
    assert ms.persistent_bytes() == persistent
    print(f"{name}: {n_units} units, {ms.total:,} shard params, persistent {persistent:,} B",
          flush=True)
    del ms
    gc.collect()
    torch.cuda.empty_cache()
    return persistent


@pytest.mark.parametrize("multi", [False, True])
def test_full_7b_rank_shard_every_unit(multi):
    """Per-unit calls: every element of every unit (842M shard elements); the batched
    entry point: every element of the named units, sampled indices of the rest."""
    full = set(range(33)) if not multi else {0, 15, 31}
    assert run_model("full7b", full, 4096, multi) == 13_476_831_232


def test_full_70b_rank_shard_every_unit():
    free, total = torch.cuda.mem_get_info()
    if free < 170 * 2**30:
        pytest.skip(f"needs ~160 GB free HBM, {free / 2**30:.0f} GiB free")
    assert run_model("full70b", {0, 40, 79}, 2048, multi=True) == 137_953_296_384


@pytest.mark.parametrize("ng", [4, 8, 12])
def test_multi_unit_step_equals_per_unit_calls(ng):
    """Mixed list: aligned units (batched), shifted-row units, ng > 8 (one launch each)."""
    from shard_cases import Case, assert_bits, to_np
    specs = [([(300, 77)], 4, 1), ([(1000, 3), (17,)], 7, 1), ([(64, 64)], 2, 0),
             ([(5,)], 8, 6), ([(2048 * 5 + 3,)], 3, 2)] * 7          # 35 units: > one batch
    cases = [Case(sh, F, r, n_grads=ng, config=20 + j) for j, (sh, F, r) in enumerate(specs)]
    ins = []
    for j, c in enumerate(cases):
        u = fsdp.Unit(c.shapes, c.F, c.rank)
        p0 = torch.empty(u.S, dtype=torch.float32, device="cuda")
        datagen.fill_normal_f32_(p0, c.master_seed, j, W.MASTER_SIGMA)
        ins.append((u, c.device_grads(1), p0))
    outs = {}
    for mode in ("per_unit", "multi"):
        st = [(u, g, p0.clone(), torch.zeros_like(p0), torch.zeros_like(p0),
               torch.empty(u.S, dtype=torch.bfloat16, device="cuda")) for u, g, p0 in ins]
        if mode == "multi":
            fsdp.reduce_adamw_units(st, HPD, 3)
        else:
            for s_ in st:
                fsdp.reduce_adamw_shard(*s_, HPD, 3)
        torch.cuda.synchronize()
        outs[mode] = [[to_np(x)[:s_[0].shard_valid].copy() for x in s_[2:]] for s_ in st]
    for a, b in zip(outs["per_unit"], outs["multi"]):
        for x, y in zip(a, b):
            assert_bits(x.view(np.uint32) if x.dtype == np.float32 else x,
                        y.view(np.uint32) if y.dtype == np.float32 else y, "multi vs per-unit")
