"""Host-side checks of libfsdpshard.so (no GPU needed, no kernel launched).

* the library loads and exports every function include/fsdp_shard.h declares;
* the C indexer agrees with the oracle's on every config and on brute force;
* argument validation returns the documented status before enqueuing work
  (each case below fails a check that runs before any HIP call).
"""

import ctypes
import os
import re

import numpy as np
import pytest

from datagen import workloads as W
from oracle import fsdp_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsdp_shard.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsdp_\w+)\s*\(", text)))


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 12
    raw = ctypes.CDLL(lib.library_path())
    for n in names:
        assert hasattr(raw, n), n
    assert lib.abi_version() == 1


def _check_unit(shapes, F, rank, lib):
    u = lib.Unit(shapes, F, rank)
    L = O.unit_layout(shapes, F, rank)
    assert (u.U, u.S, u.padded, u.pad, u.shard_begin, u.shard_valid, u.persistent_bytes) == \
        (L.U, L.S, L.padded, L.pad, L.shard_begin, L.shard_valid, L.persistent_bytes)
    assert u.offsets == list(L.offsets[:-1]) and u.numels == list(L.numels)
    return u


@pytest.mark.parametrize("name", ["tiny", "blk7", "full7b", "full70b"])
def test_indexer_matches_oracle_on_workloads(lib, name):
    wl = W.WORKLOADS[name]
    for unit in {id(u): u for u in wl["units"]}.values():
        for r in range(wl["F"]):
            _check_unit(W.shapes(unit), wl["F"], r, lib)


def test_indexer_sweep_and_padded_factors(lib):
    wl = W.WORKLOADS["sweep"]
    for F in wl["Fs"] + wl["padded_Fs"]:
        for r in (0, F - 1):
            _check_unit(W.shapes(W.BLK7), F, r, lib)


def test_indexer_brute_force(lib):
    rng = np.random.default_rng(0)
    for _ in range(300):
        T = int(rng.integers(1, 6))
        shapes = [tuple(int(d) for d in rng.integers(0, 7, int(rng.integers(0, 3))))
                  for _ in range(T)]
        if sum(O.numel(s) for s in shapes) == 0:
            shapes.append((1,))
        F = int(rng.integers(1, 17))
        _check_unit(shapes, F, int(rng.integers(0, F)), lib)


def test_tensor_count_limit(lib):
    """FSDP_MAX_TENSORS tensors (ragged, some empty) index like the oracle;
    one more is rejected; so are more than 16 dimensions."""
    rng = np.random.default_rng(5)
    sizes = rng.integers(0, 9, 65536)
    sizes[0] = 3
    shapes = [(int(n),) for n in sizes]
    for F, r in ((8, 0), (8, 7), (13, 6)):
        _check_unit(shapes, F, r, lib)
    with pytest.raises(lib.FsdpError) as e:
        lib.Unit(shapes + [(1,)], 8, 0)
    assert e.value.status == 1
    lib.Unit([tuple([1] * 16)], 2, 0)
    with pytest.raises(lib.FsdpError) as e:
        lib.Unit([tuple([1] * 17)], 2, 0)
    assert e.value.status == 1


def test_config_totals_closed_form(lib):
    # one rank's persistent bytes for the 7B and 70B shapes at F=8
    blk7, root7 = lib.Unit(W.shapes(W.BLK7), 8, 0), lib.Unit(W.shapes(W.ROOT7), 8, 0)
    assert 32 * blk7.persistent_bytes + root7.persistent_bytes == 13_476_831_232
    blk70, root70 = lib.Unit(W.shapes(W.BLK70), 8, 0), lib.Unit(W.shapes(W.ROOT70), 8, 0)
    assert 80 * blk70.persistent_bytes + root70.persistent_bytes == 137_953_296_384
    assert blk7.U == 202_383_360 and blk70.U == 855_654_400


def test_fingerprint_matches_across_ranks_and_catches_reordering(lib):
    shapes = W.shapes(W.BLK7)
    fps = {lib.Unit(shapes, 8, r).fingerprint for r in range(8)}
    assert len(fps) == 1
    permuted = shapes[1:] + shapes[:1]
    assert lib.Unit(permuted, 8, 0).fingerprint not in fps
    assert lib.Unit(shapes, 4, 0).fingerprint not in fps


@pytest.mark.parametrize("F,rank,shapes,status", [
    (0, 0, [(4,)], 1), (65, 0, [(4,)], 1), (4, 4, [(4,)], 1), (4, -1, [(4,)], 1),
    (2, 0, [(0,)], 2), (2, 0, [(-1, 3)], 1), (2, 0, [(1 << 40, 1 << 30)], 2),
])
def test_unit_create_rejects_bad_arguments(lib, F, rank, shapes, status):
    with pytest.raises(lib.FsdpError) as e:
        lib.Unit(shapes, F, rank)
    assert e.value.status == status


def _raw(lib):
    return lib._lib


def _hp(lib, **kw):
    base = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                grad_scale=0.125, step=1)
    base.update(kw)
    return lib._Hparams(**base)


FAKE = 1 << 40     # a 16-byte aligned address never dereferenced: validation fails first


def test_step_entry_points_validate_before_launch(lib):
    u = lib.Unit([(4096,)], 8, 3)
    raw = _raw(lib)
    S = u.S
    grads = [FAKE + k * (1 << 20) for k in range(8)]
    arr = lib._ptr_array(grads)
    p, m, v = FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    # n_grads out of range
    assert raw.fsdp_reduce_adamw_shard(u.handle, 0, arr, p, m, v, None,
                                       ctypes.byref(_hp(lib)), None) == 1
    assert raw.fsdp_reduce_adamw_shard(u.handle, 65, arr, p, m, v, None,
                                       ctypes.byref(_hp(lib)), None) == 1
    # bad hyper-parameters
    for bad in (dict(step=0), dict(beta1=1.0), dict(eps=0.0), dict(lr=float("nan")),
                dict(grad_scale=float("inf"))):
        assert raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, p, m, v, None,
                                           ctypes.byref(_hp(lib, **bad)), None) == 1, bad
    # null state pointer, misaligned state pointer
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, None, m, v, None,
                                       ctypes.byref(_hp(lib)), None) == 1
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, p + 2, m, v, None,
                                       ctypes.byref(_hp(lib)), None) == 1
    # master overlapping exp_avg; output overlapping a gradient row's window
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, p, p + 4 * (S - 1), v, None,
                                       ctypes.byref(_hp(lib)), None) == 3
    win3 = grads[3] + 2 * u.shard_begin
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, win3, m, v, None,
                                       ctypes.byref(_hp(lib)), None) == 3
    assert raw.fsdp_reduce_shard(u.handle, 8, arr, 0.125, win3 + 4, None) == 3
    assert "overlaps grads[3]" in raw.fsdp_last_error().decode()
    assert raw.fsdp_reduce_shard(u.handle, 8, arr, float("nan"), p, None) == 1
    # unfused AdamW: grad overlapping the bf16 output
    assert raw.fsdp_adamw_shard(u.handle, p, m, v, FAKE + (4 << 30), p + 8,
                                ctypes.byref(_hp(lib)), None) == 3


def test_flatten_and_unflatten_validate_before_launch(lib):
    u = lib.Unit([(100,), (28,)], 4, 0)
    raw = _raw(lib)
    ts = lib._ptr_array([FAKE, FAKE + (1 << 20)])
    # window outside the padded buffer; unsupported dtype; overlap
    assert raw.fsdp_flatten_pad(u.handle, 0, ts, 100, 29, FAKE + (2 << 20), None) == 2
    assert raw.fsdp_flatten_pad(u.handle, 7, ts, 0, 32, FAKE + (2 << 20), None) == 4
    assert raw.fsdp_flatten_pad(u.handle, 0, ts, 0, 32, FAKE + 16, None) == 3
    shards = lib._ptr_array([FAKE + k * 4096 for k in range(4)])
    outs = lib._ptr_array([FAKE + (1 << 22), FAKE + (1 << 22) + 100])   # tensors 0, 1 overlap
    assert raw.fsdp_cast_unflatten(u.handle, 1, shards, outs, None) == 3
    outs2 = lib._ptr_array([FAKE + 4096, FAKE + (1 << 22)])             # output over shard 1
    assert raw.fsdp_cast_unflatten(u.handle, 0, shards, outs2, None) == 3
    assert "overlaps" in raw.fsdp_last_error().decode()
    assert raw.fsdp_cast_unflatten(u.handle, 3, shards, outs2, None) == 4


def test_status_strings(lib):
    raw = _raw(lib)
    assert raw.fsdp_status_string(0) == b"ok"
    assert raw.fsdp_status_string(3) == b"overlapping buffers"


def test_multi_unit_step_validates_across_units(lib):
    raw = _raw(lib)
    u = lib.Unit([(4096,)], 8, 1)
    rows0 = lib._ptr_array([FAKE + k * (1 << 20) for k in range(8)])
    rows1 = lib._ptr_array([FAKE + (64 << 20) + k * (1 << 20) for k in range(8)])
    base = FAKE + (1 << 30)

    def step(rows, off):
        return lib._UnitStep(u.handle.value, ctypes.cast(rows, ctypes.POINTER(ctypes.c_void_p)),
                             base + off, base + off + (1 << 20), base + off + (2 << 20), None)

    hp = ctypes.byref(_hp(lib))
    arr = (lib._UnitStep * 2)(step(rows0, 0), step(rows1, 0))      # unit 1 master on unit 0's
    assert raw.fsdp_reduce_adamw_units(2, arr, 8, hp, None) == 3
    assert "unit 1 master overlaps unit 0 master" in raw.fsdp_last_error().decode()
    arr = (lib._UnitStep * 2)(step(rows0, 0), step(rows0, 16 << 20))   # rows may be shared
    arr[1].unit = None
    assert raw.fsdp_reduce_adamw_units(2, arr, 8, hp, None) == 1
    assert raw.fsdp_reduce_adamw_units(0, None, 8, hp, None) == 0
    assert raw.fsdp_reduce_adamw_units(-1, None, 8, hp, None) == 1
    arr = (lib._UnitStep * 1)(step(rows0, 0))
    assert raw.fsdp_reduce_adamw_units(1, arr, 0, hp, None) == 1


def test_hybrid_entry_points_validate_before_launch(lib):
    raw = _raw(lib)
    u = lib.Unit([(4096,)], 8, 2)
    rows = lib._ptr_array([FAKE + k * (1 << 20) for k in range(64)])
    p, m, v = FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    hp = ctypes.byref(_hp(lib))
    assert raw.fsdp_reduce_adamw_shard_hybrid(u.handle, 9, rows, p, m, v, None, hp, None) == 1
    assert "replicas * F" in raw.fsdp_last_error().decode()
    assert raw.fsdp_reduce_adamw_shard_hybrid(u.handle, 0, rows, p, m, v, None, hp, None) == 1
    assert raw.fsdp_reduce_shard_hybrid(u.handle, 2, rows, float("nan"), p, None) == 1
    win = FAKE + 5 * (1 << 20) + 2 * u.shard_begin
    assert raw.fsdp_reduce_shard_hybrid(u.handle, 2, rows, 0.0625, win, None) == 3


def test_empty_window_needs_no_buffers(lib):
    """A rank whose window holds only pad (shard_valid 0): the step calls check their
    counts and hyper-parameters and return ok without touching their buffers."""
    raw = _raw(lib)
    u = lib.Unit([(5,)], 8, 6)
    assert u.shard_valid == 0
    hp = ctypes.byref(_hp(lib))
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, None, None, None, None, None, hp, None) == 0
    assert raw.fsdp_reduce_shard(u.handle, 8, None, 0.125, None, None) == 0
    assert raw.fsdp_adamw_shard(u.handle, None, None, None, None, None, hp, None) == 0
    assert raw.fsdp_reduce_adamw_shard_bf16acc(u.handle, 8, None, None, None, None, None, hp,
                                               None) == 0
    assert raw.fsdp_reduce_adamw_shard_hybrid(u.handle, 2, None, None, None, None, None, hp,
                                              None) == 0
    # counts and hyper-parameters are still checked
    assert raw.fsdp_reduce_adamw_shard(u.handle, 0, None, None, None, None, None, hp, None) == 1
    assert raw.fsdp_reduce_adamw_shard(u.handle, 8, None, None, None, None, None,
                                       ctypes.byref(_hp(lib, step=0)), None) == 1
    assert raw.fsdp_reduce_adamw_shard_hybrid(u.handle, 9, None, None, None, None, None, hp,
                                              None) == 1
    arr = (lib._UnitStep * 1)(lib._UnitStep(u.handle.value, None, None, None, None, None))
    assert raw.fsdp_reduce_adamw_units(1, arr, 8, hp, None) == 0


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="needs a HIP runtime with no usable device (the CPU container)")
def test_pending_runtime_error_is_reported_before_any_launch(lib):
    """Without a usable device the HIP runtime holds an error from its start-up; a call
    with valid arguments reports it as pending (FSDP_ERR_HIP) and launches nothing."""
    raw = _raw(lib)
    u = lib.Unit([(4096,)], 8, 3)
    arr = lib._ptr_array([FAKE + k * (1 << 20) for k in range(8)])
    p, m, v = FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    hp = ctypes.byref(_hp(lib))
    for call in (lambda: raw.fsdp_reduce_adamw_shard(u.handle, 8, arr, p, m, v, None, hp, None),
                 lambda: raw.fsdp_reduce_shard(u.handle, 8, arr, 0.125, p, None),
                 lambda: raw.fsdp_flatten_pad(u.handle, 0, lib._ptr_array([FAKE]), 0, 512, p,
                                              None)):
        assert call() == 5
        msg = raw.fsdp_last_error().decode()
        assert "pending" in msg and "nothing was enqueued" in msg, msg
