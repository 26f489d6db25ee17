"""Full-state-dict export / resume (fsdp_unflatten with fp32, fsdp_flatten_pad with fp32).

[Glossary, "Debugging FSDP" -> Checkpoint/Resume]: a full state dict gathers
the sharded state into whole tensors. Export: the F fp32 shards of master,
exp_avg and exp_avg_sq -> per-tensor fp32 tensors. Resume: per-tensor fp32
tensors -> this rank's shard window (pad = +0). Checked against the oracle
and as a bitwise round trip at full size.
"""

import gc

import numpy as np
import pytest
import torch

import datagen
from datagen import workloads as W
from oracle import fsdp_oracle as O
from shard_cases import Case, assert_bits, to_np

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import sharded_flatparameter_flatten_amd as fsdp  # noqa: E402

DEV = "cuda"
HPD = fsdp.AdamWHparams(**W.ADAMW)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _bits(x):
    x = np.asarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


@pytest.mark.parametrize("src,dst", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"),
                                     ("bf16", "bf16")])
@pytest.mark.parametrize("shapes,F", [(W.shapes(W.TINY), 4), ([(1000, 3), (17,), (5, 5)], 7),
                                      ([(3,)], 8)])
@pytest.mark.parametrize("offset", [0, 1])
def test_unflatten_dtype_pairs_bit_exact(src, dst, shapes, F, offset):
    """offset = 1 puts every shard and output one element past an aligned address."""
    u = fsdp.Unit(shapes, F, 0)
    rng = np.random.default_rng(F + offset)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    if src == "f32":
        host = [(rng.standard_normal(u.S) * 0.02).astype(np.float32) for _ in range(F)]
        dev = [torch.zeros(u.S + offset, dtype=torch.float32, device=DEV) for _ in range(F)]
        for d, h in zip(dev, host):
            d[offset:].copy_(torch.from_numpy(h))
    else:
        host = [rng.integers(0, 1 << 16, u.S, dtype=np.uint64).astype(np.uint16) for _ in range(F)]
        dev = [torch.zeros(u.S + offset, dtype=torch.bfloat16, device=DEV) for _ in range(F)]
        for d, h in zip(dev, host):
            d[offset:].view(torch.int16).copy_(torch.from_numpy(h.view(np.int16)))
    shards = [d[offset:] for d in dev]
    big = [torch.empty(O.numel(s) + offset, dtype=tdt[dst], device=DEV) for s in shapes]
    outs = [b[offset:].view(s) for b, s in zip(big, shapes)]
    fsdp.unflatten(u, shards, outs)
    torch.cuda.synchronize()
    want = O.unflatten(host, O.unit_layout(shapes, F, 0), shapes, out=dst)
    for o, wnt in zip(outs, want):
        got = to_np(o)
        if dst == "f32" and src == "bf16":
            nan = np.isnan(wnt)
            assert_bits(_bits(got[~nan]), _bits(wnt[~nan]), "widen")
            assert np.all(np.isnan(got[nan]))
        else:
            assert_bits(_bits(got), _bits(wnt), f"{src}->{dst}")


def test_full_size_state_dict_export_resume_round_trip():
    """7B block at F=8: step every rank, export master/m/v to whole fp32 tensors,
    resume them into fresh shards: bitwise identical shards, pad +0."""
    shapes, F = W.shapes(W.BLK7), 8
    units = [fsdp.Unit(shapes, F, r) for r in range(F)]
    U, S = units[0].U, units[0].S
    grads = [torch.empty(U, dtype=torch.bfloat16, device=DEV) for _ in range(F)]
    for k in range(F):
        datagen.fill_bf16_(grads[k], datagen.seed_for(15, 1, 1), k, W.GRAD_SIGMA)
    state = []
    for r, u in enumerate(units):
        p = torch.empty(S, dtype=torch.float32, device=DEV)
        datagen.fill_normal_f32_(p, datagen.seed_for(15, 0), r, W.MASTER_SIGMA)
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        fsdp.reduce_adamw_shard(u, grads, p, m, v, None, HPD, 1)
        state.append((p, m, v))
    del grads
    for kind in range(3):
        shards = [st[kind] for st in state]
        whole = [torch.empty(s, dtype=torch.float32, device=DEV) for s in shapes]
        fsdp.unflatten(units[0], shards, whole)                 # export
        for r, u in enumerate(units):
            back = torch.empty(S, dtype=torch.float32, device=DEV)
            fsdp.flatten_pad(u, whole, back)                    # resume
            assert torch.equal(back.view(torch.int32), shards[r].view(torch.int32)), (kind, r)
        # the export equals the shards concatenated and split at the tensor offsets
        flat = torch.cat(shards)[:U]
        for t, off, n in zip(whole, units[0].offsets, units[0].numels):
            assert torch.equal(t.reshape(-1).view(torch.int32), flat[off:off + n].view(torch.int32))
        del whole
