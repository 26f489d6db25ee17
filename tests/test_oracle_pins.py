"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a number the pages print
(tests/golden/, with its citation), a closed form, a textbook bound, a library
routine (numpy concatenation, torch's bf16 cast, torch.optim.AdamW in float64)
or brute force on tiny inputs. The mutation tests at the end plant a
plausible mistake in a copy of an oracle step and check that a pin catches it.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
from oracle import fsdp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24          # unit roundoff of binary32


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def ulp32(x):
    """Spacing of binary32 numbers at |x| (float64 in, float64 out)."""
    x = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def rng_bf16(seed, n, sigma=1e-3, stream=0):
    return datagen.bf16_bits_host(seed, stream, np.arange(n), sigma)


# ----------------------------------------------------------------------------
# indexer
# ----------------------------------------------------------------------------

def test_layout_brute_force_small():
    for U in range(1, 65):
        for F in range(1, 17):
            windows = []
            for r in range(F):
                L = O.unit_layout([(U,)], F, r)
                assert L.F * L.S >= U > L.F * (L.S - 1)
                assert 0 <= L.pad < F
                assert L.padded == F * L.S
                assert L.shard_begin == r * L.S
                windows.append((L.shard_begin, L.shard_valid))
            assert sum(v for _, v in windows) == U
            covered = []
            for b, v in windows:
                covered.extend(range(b, b + v))
            assert covered == list(range(U))   # contiguous, in rank order


def test_layout_offsets_are_prefix_sums_of_shapes():
    shapes = [(256, 1024), (1024,), (1024, 256), (256,)]
    L = O.unit_layout(shapes, 4, 1)
    assert L.offsets == (0, 262144, 263168, 525312, 525568)
    assert L.U == 525568 and L.S == 131392 and L.pad == 0
    assert (L.shard_begin, L.shard_valid) == (131392, 131392)


def test_sharding_factor_table():
    g = golden("sharding_factor_table.json")
    for case in g["cases"]:
        for r in range(case["F"]):
            L = O.unit_layout([(case["U"],)], case["F"], r)
            assert L.S == case["shard_len"]
    one = O.unit_layout([(1000,)], 1, 0)
    assert one.shard_valid == one.U        # F = 1: the rank holds the whole unit


def test_bytes_per_param_breakdown():
    g = golden("bytes_per_param.json")
    parts = (g["low_precision_weight"] + g["low_precision_grad"] + g["fp32_master"]
             + g["adam_momentum"] + g["adam_variance"])
    assert parts == g["total"] == 16
    assert O.persistent_bytes(1) == g["total"]


def test_worked_example_7b_on_8_gpus():
    g = golden("worked_example_7b_8gpu.json")
    P, N = g["params"], g["ranks"]
    whole = O.unit_layout([(P,)], N, 0)
    assert whole.persistent_bytes == g["fsdp_persistent_bytes_per_gpu"]
    ddp = O.unit_layout([(P,)], 1, 0)
    assert ddp.persistent_bytes == g["ddp_state_bytes_per_gpu"]
    assert abs(P / g["blocks"] - g["unit_params_approx"]) <= g["unit_params_approx_tolerance"]


# ----------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------

def _structured_fp32_bits():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF], dtype=np.uint32)
    rng = np.random.default_rng(7)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, 8, dtype=np.uint32)])
    structured = (hi[:, None] | lows[None, :]).reshape(-1)
    rand = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([structured, rand])


def test_bf16_rne_matches_torch_cast():
    bits = _structured_fp32_bits()
    x = bits.view(np.float32)
    ours = O.bf16_round_nearest_even(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)
    assert np.all((ref[nan] & 0x7F80) == 0x7F80)     # torch also returns a NaN there


def test_bf16_rne_matches_torch_cast_on_every_fp32_pattern():
    """All 2^32 fp32 bit patterns: the oracle's rounding equals torch's CPU cast
    on every non-NaN input, and both give a NaN for every NaN input."""
    import multiprocessing as mp
    import os
    from concurrent.futures import ProcessPoolExecutor

    import bf16_sweep

    chunk = 1 << 25
    starts = list(range(0, 1 << 32, chunk))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(bf16_sweep.check_range, starts, [chunk] * len(starts)))
    bad = sum(r[0] for r in res)
    firsts = [hex(r[1]) for r in res if r[1] is not None][:3]
    assert bad == 0, f"{bad} patterns differ, first {firsts}"
    assert sum(r[2] for r in res) == 0


def test_bf16_rne_ties_and_overflow_closed_forms():
    halfway_past_max = np.array([0x7F7F8000], dtype=np.uint32).view(np.float32)[0]
    f = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, np.finfo(np.float32).max, -0.0,
                  2.0 ** -133, halfway_past_max], dtype=np.float32)
    out = O.bf16_round_nearest_even(f)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    assert out[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to even -> 1+2^-6 (0x3F82)
    assert out[1] == 0x3F82
    # fp32 max lies more than half a bf16 step above the largest finite bf16 -> +inf
    assert out[2] == 0x7F80
    # exactly halfway between the largest finite bf16 (odd last bit) and 2^128 -> +inf
    assert out[5] == 0x7F80
    assert out[3] == 0x8000
    # a subnormal fp32 keeps its high half
    assert out[4] == (np.float32(2.0 ** -133).view(np.uint32) >> 16)


# ----------------------------------------------------------------------------
# flatten / pad / unflatten
# ----------------------------------------------------------------------------

def _random_unit(rng, T):
    shapes = []
    for _ in range(T):
        nd = int(rng.integers(0, 3))
        shapes.append(tuple(int(rng.integers(1, 9)) for _ in range(nd)) or (int(rng.integers(1, 40)),))
    return shapes


def test_flatten_f1_equals_concatenation():
    rng = np.random.default_rng(1)
    shapes = _random_unit(rng, 6)
    ts = [rng.integers(0, 1 << 16, O.numel(s), dtype=np.uint64).astype(np.uint16).reshape(s)
          for s in shapes]
    assert np.array_equal(O.flatten_pad(ts, 1), np.concatenate([t.reshape(-1) for t in ts]))


def test_flatten_pad_is_zero_and_windows_tile():
    rng = np.random.default_rng(2)
    for F in (1, 2, 3, 5, 8, 13, 64):
        shapes = _random_unit(rng, 5)
        ts = [rng.integers(1, 1 << 32, O.numel(s), dtype=np.uint64).astype(np.uint32)
              for s in shapes]
        U = sum(t.size for t in ts)
        flat = O.flatten_pad(ts, F)
        S = -(-U // F)
        assert flat.size == F * S
        assert np.all(flat[U:] == 0)
        joined = np.concatenate([O.flatten_pad(ts, F, r * S, S) for r in range(F)])
        assert np.array_equal(joined, flat)


@pytest.mark.parametrize("F", [1, 2, 3, 4, 7, 8, 16, 64])
def test_flatten_unflatten_round_trip_is_identity(F):
    rng = np.random.default_rng(F)
    shapes = _random_unit(rng, 7)
    ts = [rng.integers(0, 1 << 16, O.numel(s), dtype=np.uint64).astype(np.uint16).reshape(s)
          for s in shapes]
    U = sum(t.size for t in ts)
    S = -(-U // F)
    shards = [O.flatten_pad(ts, F, r * S, S) for r in range(F)]
    L = O.unit_layout(shapes, F, 0)
    outs = O.cast_unflatten(shards, L, shapes)
    for a, b in zip(outs, ts):
        assert a.shape == b.shape and np.array_equal(a, b)


def test_unflatten_from_fp32_matches_torch_cast():
    rng = np.random.default_rng(3)
    shapes = [(33, 7), (5,), (17, 3), (1,)]
    F = 5
    ts = [rng.standard_normal(O.numel(s)).astype(np.float32) * np.float32(0.02) for s in shapes]
    ts[1][:] = np.array([np.inf, -np.inf, 0.0, -0.0, 3.4e38], dtype=np.float32)
    U = sum(t.size for t in ts)
    S = -(-U // F)
    flat = np.concatenate(ts)
    shards = [np.concatenate([flat, np.zeros(F * S - U, np.float32)])[r * S:(r + 1) * S]
              for r in range(F)]
    L = O.unit_layout(shapes, F, 0)
    outs = O.cast_unflatten(shards, L, shapes)
    for out, t, s in zip(outs, ts, shapes):
        ref = torch.from_numpy(t).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(out.reshape(-1), ref)
        assert out.shape == s


@pytest.mark.parametrize("F", [1, 3, 8])
def test_state_dict_export_resume_round_trip(F):
    """fp32 shards -> per-tensor fp32 (export) -> flatten into shards (resume): identity."""
    rng = np.random.default_rng(10 + F)
    shapes = [(37, 5), (11,), (64, 3)]
    U = sum(O.numel(s) for s in shapes)
    S = -(-U // F)
    flat = rng.standard_normal(F * S).astype(np.float32)
    flat[U:] = 0.0
    shards = [flat[r * S:(r + 1) * S].copy() for r in range(F)]
    L = O.unit_layout(shapes, F, 0)
    tensors = O.unflatten(shards, L, shapes, out="f32")
    # library pin: the export is the flat buffer split by numpy at the tensor offsets
    pieces = np.split(flat[:U], np.cumsum([O.numel(s) for s in shapes])[:-1])
    for t, piece, s in zip(tensors, pieces, shapes):
        assert t.shape == s and np.array_equal(t.reshape(-1).view(np.uint32), piece.view(np.uint32))
    back = [O.flatten_pad([t.view(np.uint32) for t in tensors], F, r * S, S).view(np.float32)
            for r in range(F)]
    for a, b in zip(back, shards):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_unflatten_bf16_to_f32_widens_exactly():
    rng = np.random.default_rng(12)
    shapes = [(9, 7), (5,)]
    L = O.unit_layout(shapes, 4, 0)
    shards = [rng.integers(0, 1 << 16, L.S, dtype=np.uint64).astype(np.uint16) for _ in range(4)]
    outs = O.unflatten(shards, L, shapes, out="f32")
    flat = np.concatenate(shards)[:L.U]
    ref = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.concatenate([o.reshape(-1) for o in outs])
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.all(np.isnan(got[nan]))


# ----------------------------------------------------------------------------
# reduce-scatter arithmetic
# ----------------------------------------------------------------------------

def test_reduce_two_buffers_is_one_rounding_of_the_exact_sum():
    n = 1 << 16
    a = rng_bf16(11, n, 1e-3, 0)
    b = rng_bf16(11, n, 1e-3, 1)
    b[:64] = rng_bf16(12, 64, 1e-9, 0)        # wide exponent gaps force rounding
    L = O.unit_layout([(n,)], 1, 0)
    got = O.reduce_shard([a, b], L, grad_scale=1.0)
    exact = O.bf16_widen(a).astype(np.float64) + O.bf16_widen(b).astype(np.float64)
    assert np.array_equal(got, exact.astype(np.float32))     # float64 sum of two bf16 is exact


def test_reduce_within_recursive_summation_bound_with_outliers():
    n_el, n = 1 << 15, 8
    seed, oseed = datagen.seed_for(3, 1), datagen.seed_for(3, 2)
    gs = [datagen.bf16_bits_host(seed, k, np.arange(n_el), 1e-3, outlier_seed=oseed)
          for k in range(n)]
    L = O.unit_layout([(n_el,)], 1, 0)
    got = O.reduce_shard(gs, L, grad_scale=1.0).astype(np.float64)
    vals = np.stack([O.bf16_widen(g).astype(np.float64) for g in gs])
    exact = vals.sum(axis=0)                  # exact: few terms of 8-bit significands
    gamma = (n - 1) * U32 / (1 - (n - 1) * U32)
    bound = gamma * np.abs(vals).sum(axis=0)
    assert np.all(np.abs(got - exact) <= bound)


def test_reduce_mean_is_exact_when_the_fold_is_exact():
    n_el, n = 1 << 15, 8
    gs = [rng_bf16(21, n_el, 1e-3, k) for k in range(n)]
    L = O.unit_layout([(n_el,)], 1, 0)
    got = O.reduce_shard(gs, L)               # default scale 1/8
    vals = np.stack([O.bf16_widen(g).astype(np.float64) for g in gs])
    partial = np.cumsum(vals, axis=0)
    exact_everywhere = np.all(partial.astype(np.float32).astype(np.float64) == partial, axis=0)
    assert exact_everywhere.mean() > 0.5
    want = (partial[-1] / 8.0).astype(np.float32)
    assert np.array_equal(got[exact_everywhere], want[exact_everywhere])


def test_reduce_single_buffer_is_identity_times_scale():
    g = rng_bf16(31, 4096)
    L = O.unit_layout([(4096,)], 1, 0)
    assert np.array_equal(O.reduce_shard([g], L), O.bf16_widen(g))
    half = O.reduce_shard([g], L, grad_scale=0.5).astype(np.float64)
    assert np.array_equal(half, O.bf16_widen(g).astype(np.float64) * 0.5)


@pytest.mark.parametrize("F", [2, 3, 4, 7, 8])
def test_reduce_shard_is_the_full_reduction_sliced(F):
    shapes = [(37, 11), (5,), (101,)]
    U = sum(O.numel(s) for s in shapes)
    gs = [rng_bf16(41, U, 1e-3, k) for k in range(F)]
    vals = np.stack([O.bf16_widen(g).astype(np.float64) for g in gs])
    exact_mean = vals.sum(axis=0) / F
    full = O.reduce_shard(gs, O.unit_layout(shapes, 1, 0))
    for r in range(F):
        L = O.unit_layout(shapes, F, r)
        got = O.reduce_shard(gs, L)
        lo, hi = L.shard_begin, L.shard_begin + L.shard_valid
        assert got.size == L.shard_valid
        assert np.array_equal(got, full[lo:hi])
        bound = 2 * F * U32 * np.abs(vals[:, lo:hi]).sum(axis=0) / F
        assert np.all(np.abs(got - exact_mean[lo:hi]) <= bound)


def test_reduce_brute_force_fractions_tiny():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 6))
        gs = [rng.integers(0, 1 << 16, 3, dtype=np.uint64).astype(np.uint16) for _ in range(n)]
        gs = [np.where(np.isfinite(O.bf16_widen(g)), g, np.uint16(0x3F80)).astype(np.uint16)
              for g in gs]
        L = O.unit_layout([(3,)], 1, 0)
        got = O.reduce_shard(gs, L, grad_scale=1.0)
        if not np.all(np.isfinite(got)):
            continue
        for e in range(3):
            terms = [Fraction(float(O.bf16_widen(g)[e])) for g in gs]
            exact = sum(terms, Fraction(0))
            mag = sum(abs(t) for t in terms)
            gamma = Fraction(n - 1) * Fraction(U32) / (1 - Fraction(n - 1) * Fraction(U32))
            assert abs(Fraction(float(got[e])) - exact) <= gamma * mag


def test_bf16acc_reduce_closed_forms():
    n = 1 << 14
    a, b = rng_bf16(121, n, 1e-3, 0), rng_bf16(121, n, 1e-3, 1)
    L = O.unit_layout([(n,)], 1, 0)
    # one row: the bf16 value itself, times the scale
    assert np.array_equal(O.reduce_shard_bf16acc([a], L), O.bf16_widen(a))
    # two rows: torch's bf16 rounding of the fp32 sum (itself one rounding of the exact sum)
    got = O.reduce_shard_bf16acc([a, b], L, grad_scale=1.0)
    s32 = (O.bf16_widen(a).astype(np.float64) + O.bf16_widen(b).astype(np.float64)).astype(np.float32)
    ref = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)


def _bf16acc_closed_form_3(a, b, c, gs):
    """Three rows with bf16 partials, by torch's bf16 cast (a library routine):
    bf16(fp32(bf16(fp32(a + b)) + c)) * fp32(gs), each fp32 add one rounding of
    the exact sum."""
    w = [O.bf16_widen(x).astype(np.float64) for x in (a, b, c)]
    to_bf16 = lambda f32: torch.from_numpy(f32).to(torch.bfloat16).float().numpy()
    s1 = to_bf16((w[0] + w[1]).astype(np.float32))
    s2 = to_bf16((s1.astype(np.float64) + w[2]).astype(np.float32))
    return (s2 * np.float32(gs)).astype(np.float32)


def _bf16acc_inputs(n=1 << 14):
    return [rng_bf16(131, n, 1e-3, k) for k in range(3)]


def test_bf16acc_reduce_three_rows_closed_form():
    a, b, c = _bf16acc_inputs()
    L = O.unit_layout([(a.size,)], 1, 0)
    got = O.reduce_shard_bf16acc([a, b, c], L, grad_scale=1.0 / 3)
    assert np.array_equal(got, _bf16acc_closed_form_3(a, b, c, 1.0 / 3))


def _mutant_round_once_at_end(rows, L, grad_scale):
    s32 = O.reduce_shard(rows, L, grad_scale=1.0)
    return O.bf16_widen(O.bf16_round_nearest_even(s32)) * np.float32(grad_scale)


def _mutant_scale_before_rounding(rows, L, grad_scale):
    acc = O.bf16_widen(rows[0][:L.shard_valid])
    for r in rows[1:-1]:
        acc = O.bf16_widen(O.bf16_round_nearest_even(acc + O.bf16_widen(r[:L.shard_valid])))
    last = (acc + O.bf16_widen(rows[-1][:L.shard_valid])) * np.float32(grad_scale)
    return O.bf16_widen(O.bf16_round_nearest_even(last))


@pytest.mark.parametrize("mutant", [_mutant_round_once_at_end, _mutant_scale_before_rounding])
def test_bf16acc_pin_has_teeth(mutant):
    """Plausible mistakes in the bf16-partials fold fail the three-row closed form."""
    a, b, c = _bf16acc_inputs()
    L = O.unit_layout([(a.size,)], 1, 0)
    assert not np.array_equal(mutant([a, b, c], L, 1.0 / 3), _bf16acc_closed_form_3(a, b, c, 1.0 / 3))


def test_bf16acc_reduce_within_bf16_summation_bound():
    n_el, n = 1 << 14, 8
    gs = [datagen.bf16_bits_host(datagen.seed_for(3, 1), k, np.arange(n_el), 1e-3,
                                 outlier_seed=datagen.seed_for(3, 2)) for k in range(n)]
    L = O.unit_layout([(n_el,)], 1, 0)
    got = O.reduce_shard_bf16acc(gs, L, grad_scale=1.0).astype(np.float64)
    vals = np.stack([O.bf16_widen(g).astype(np.float64) for g in gs])
    u = 2.0 ** -8 + U32 + 2.0 ** -8 * U32       # fp32 add then bf16 rounding, per step
    gamma = (n - 1) * u / (1 - (n - 1) * u)
    err = np.abs(got - vals.sum(axis=0))
    assert np.all(err <= gamma * np.abs(vals).sum(axis=0))
    # and it really is coarser than the fp32 reduction on these inputs
    fp32 = O.reduce_shard(gs, L, grad_scale=1.0).astype(np.float64)
    assert np.abs(fp32 - vals.sum(axis=0)).max() < err.max()


def test_hybrid_reduce_special_cases_reduce_to_the_flat_fold():
    shapes = [(777,)]
    rows8 = [rng_bf16(101, 777, 1e-3, k) for k in range(8)]
    # one replica group: the plain F-way reduction
    L8 = O.unit_layout(shapes, 8, 3)
    assert np.array_equal(O.reduce_shard_hybrid(rows8, L8, 1), O.reduce_shard(rows8, L8))
    # groups of one rank (F = 1): the plain fold over the R replicas
    L1 = O.unit_layout(shapes, 1, 0)
    assert np.array_equal(O.reduce_shard_hybrid(rows8, L1, 8), O.reduce_shard(rows8, L1))


def test_hybrid_reduce_two_by_two_closed_form():
    """R = 2 groups of F = 2: fl(fl(a+b) + fl(c+d)), each pair sum one rounding of the exact sum."""
    n = 1 << 14
    rows = [rng_bf16(111, n, 1e-3, k) for k in range(4)]
    rows[2][:128] = rng_bf16(112, 128, 1e-9, 0)            # wide exponent gaps: rounding happens
    L = O.unit_layout([(2 * n,)], 2, 0)                     # rank 0 of F = 2: elements [0, n)
    rows = [np.concatenate([r, r]) for r in rows]
    got = O.reduce_shard_hybrid(rows, L, 2, grad_scale=1.0)
    x = [O.bf16_widen(r[:n]).astype(np.float64) for r in rows]
    g0 = (x[0] + x[1]).astype(np.float32).astype(np.float64)   # exact pair sum, rounded once
    g1 = (x[2] + x[3]).astype(np.float32).astype(np.float64)
    want = (g0 + g1).astype(np.float32)
    assert np.array_equal(got, want)
    flat = O.reduce_shard(rows, O.unit_layout([(2 * n,)], 2, 0), grad_scale=1.0)
    assert not np.array_equal(got, flat)                    # the two trees round differently


def _hybrid_closed_form_3x2(rows, n, gs=1.0):
    """R = 3 groups of F = 2 (replica-major rows): ((p0 + p1) + p2) * fp32(gs) with
    each pair sum p_rho one rounding of the exact pair sum, folded in group order."""
    x = [O.bf16_widen(r[:n]).astype(np.float64) for r in rows]
    p = [(x[2 * j] + x[2 * j + 1]).astype(np.float32) for j in range(3)]
    acc = (p[0].astype(np.float64) + p[1]).astype(np.float32)
    acc = (acc.astype(np.float64) + p[2]).astype(np.float32)
    return (acc * np.float32(gs)).astype(np.float32)


def _hybrid_inputs_3x2(n=1 << 13):
    rows = [rng_bf16(121, n, 1e-3, k) for k in range(6)]
    rows[1][:256] = rng_bf16(122, 256, 1e-9, 0)            # rounding inside a pair
    rows[4][256:512] = rng_bf16(123, 256, 1e2, 0)          # a large group sum: order matters
    return [np.concatenate([r, r]) for r in rows], n


def test_hybrid_reduce_three_groups_closed_form():
    rows, n = _hybrid_inputs_3x2()
    L = O.unit_layout([(2 * n,)], 2, 0)
    got = O.reduce_shard_hybrid(rows, L, 3, grad_scale=1.0 / 6)
    assert np.array_equal(got, _hybrid_closed_form_3x2(rows, n, 1.0 / 6))


def _mutant_strided_groups(rows, L, R, grad_scale):
    F = len(rows) // R
    return O.reduce_shard_hybrid([rows[(k % R) * F + k // R] for k in range(len(rows))], L, R,
                                 grad_scale=grad_scale)


def _mutant_reversed_group_order(rows, L, R, grad_scale):
    F = len(rows) // R
    order = [rho * F + k for rho in reversed(range(R)) for k in range(F)]
    return O.reduce_shard_hybrid([rows[i] for i in order], L, R, grad_scale=grad_scale)


def _mutant_scale_per_group(rows, L, R, grad_scale):
    F = len(rows) // R
    parts = [O.reduce_shard(rows[rho * F:(rho + 1) * F], L, grad_scale=grad_scale)
             for rho in range(R)]
    acc = parts[0]
    for q in parts[1:]:
        acc = acc + q
    return acc


@pytest.mark.parametrize("mutant", [_mutant_strided_groups, _mutant_reversed_group_order,
                                    _mutant_scale_per_group])
def test_hybrid_pin_has_teeth(mutant):
    """Plausible mistakes in the two-level fold fail the three-group closed form."""
    rows, n = _hybrid_inputs_3x2()
    L = O.unit_layout([(2 * n,)], 2, 0)
    want = _hybrid_closed_form_3x2(rows, n, 1.0 / 6)      # the default scale for 6 rows
    assert not np.array_equal(mutant(rows, L, 3, 1.0 / 6), want)


def test_hybrid_reduce_within_summation_bound():
    n, R, F = 1 << 13, 4, 4
    rows = [datagen.bf16_bits_host(datagen.seed_for(3, 1), k, np.arange(n * F), 1e-3,
                                   outlier_seed=datagen.seed_for(3, 2)) for k in range(R * F)]
    L = O.unit_layout([(n * F,)], F, 1)
    got = O.reduce_shard_hybrid(rows, L, R, grad_scale=1.0).astype(np.float64)
    vals = np.stack([O.bf16_widen(r[n:2 * n]).astype(np.float64) for r in rows])
    depth = (F - 1) + (R - 1)
    gamma = depth * U32 / (1 - depth * U32)
    assert np.all(np.abs(got - vals.sum(axis=0)) <= gamma * np.abs(vals).sum(axis=0))


# ----------------------------------------------------------------------------
# AdamW
# ----------------------------------------------------------------------------

HP = O.AdamW(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _adam_inputs(n, seed=51):
    p = datagen.normal_f32_host(seed, 0, np.arange(n), 0.02)
    g = O.bf16_widen(datagen.bf16_bits_host(seed, 1, np.arange(n), 1e-3))
    g = g.copy()
    g[:n // 16] *= np.float32(1e-5)           # gradients near eps scale
    g[n // 16:n // 8] = 0.0
    return p, g


def test_adamw_scalars_are_rounded_once_from_double():
    c = O.adamw_scalars(HP, 1)
    assert c["omb1"] == np.float32(0.1)
    assert c["omb1"] != np.float32(1.0) - np.float32(0.9)
    assert c["bc2"] == np.float32(1.0 - 0.999)


def test_adamw_first_step_closed_form():
    p, g = _adam_inputs(1 << 14)
    z = np.zeros_like(p)
    p1, m1, v1 = O.adamw_step(g, p, z, z, HP, 1)
    g64, p64 = g.astype(np.float64), p.astype(np.float64)
    # with m = v = 0 at t = 1 the bias corrections cancel exactly in real arithmetic
    m_exact = 0.1 * g64
    v_exact = 0.001 * g64 * g64
    p_exact = p64 - 1e-4 * (g64 / (np.abs(g64) + 1e-8) + 0.01 * p64)
    assert np.all(np.abs(m1 - m_exact) <= 2 * U32 * np.abs(m_exact) + 1e-45)
    assert np.all(np.abs(v1 - v_exact) <= 3 * U32 * np.abs(v_exact) + 1e-45)
    assert np.all(np.abs(p1 - p_exact) <= ulp32(p_exact) + 1e-4 * 16 * U32)


def test_adamw_zero_gradient_is_decoupled_decay_scaled_by_lr():
    p, _ = _adam_inputs(1 << 14)
    z = np.zeros_like(p)
    cur, m, v = p, z, z
    want = p.astype(np.float64)
    for t in (1, 2, 3):
        cur, m, v = O.adamw_step(z, cur, m, v, HP, t)
        want = want - 1e-4 * 0.01 * want
        assert np.all(m == 0) and np.all(v == 0)
        assert np.all(np.abs(cur - want) <= t * ulp32(want))
    # the other convention (decay not scaled by lr) would move p by 1e-2 relative
    assert np.all(np.abs(cur / p - 1.0) < 1e-5)


def _torch_adamw_reference(p, grads):
    """torch.optim.AdamW in float64 on CPU: the formula's library reference."""
    w = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([w], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False)
    states = []
    for g in grads:
        w.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
        st = opt.state[w]
        states.append((w.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
                       st["exp_avg_sq"].numpy().copy()))
    return states


def _check_against_torch(step_fn, p, grads):
    ref = _torch_adamw_reference(p, grads)
    cur, m, v = p, np.zeros_like(p), np.zeros_like(p)
    m_scale = np.zeros(p.size)
    for t, (g, (p_ref, m_ref, v_ref)) in enumerate(zip(grads, ref), start=1):
        cur, m, v = step_fn(g, cur, m, v, HP, t)
        m_scale = 0.9 * m_scale + 0.1 * np.abs(g.astype(np.float64))
        mh = m_ref / (1 - 0.9 ** t)
        u_ref = mh / (np.sqrt(v_ref / (1 - 0.999 ** t)) + 1e-8)
        assert np.all(np.abs(m - m_ref) <= 6 * t * U32 * m_scale + 1e-45), t
        assert np.all(np.abs(v - v_ref) <= 6 * t * U32 * v_ref + 1e-45), t
        tol = t * (2 * ulp32(p_ref) + 1e-4 * 32 * U32 * (np.abs(u_ref) + 0.01 * np.abs(p_ref)))
        assert np.all(np.abs(cur - p_ref) <= tol), t


def test_adamw_matches_torch_adamw_float64_three_steps():
    n = 1 << 14
    p, g1 = _adam_inputs(n, 61)
    grads = [g1]
    for s in (62, 63):
        grads.append(O.bf16_widen(datagen.bf16_bits_host(s, 1, np.arange(n), 1e-3)))
    _check_against_torch(O.adamw_step, p, grads)


@pytest.mark.parametrize("F", [2, 3, 8])
def test_sharded_adamw_concatenated_equals_unsharded(F):
    shapes = [(63, 5), (7,), (129,)]
    U = sum(O.numel(s) for s in shapes)
    gs = [rng_bf16(71, U, 1e-3, k) for k in range(F)]
    p = datagen.normal_f32_host(72, 0, np.arange(U), 0.02)
    z = np.zeros(U, np.float32)
    full = O.reduce_adamw_shard(gs, O.unit_layout(shapes, 1, 0), p, z, z, HP, 1,
                                grad_scale=1.0 / F, emit_bf16=True)
    parts = [[], [], [], []]
    for r in range(F):
        L = O.unit_layout(shapes, F, r)
        lo, hi = L.shard_begin, L.shard_begin + L.shard_valid
        out = O.reduce_adamw_shard(gs, L, p[lo:hi], z[lo:hi], z[lo:hi], HP, 1,
                                   emit_bf16=True)
        for acc, x in zip(parts, out):
            acc.append(x)
    for a, b in zip(parts, full):
        assert np.array_equal(np.concatenate(a), b)


def test_adamw_zero_state_stays_zero():
    z = np.zeros(64, np.float32)
    for t in (1, 2, 3):
        out = O.adamw_step(z, z, z, z, HP, t, emit_bf16=True)
        for x in out:
            assert np.all(x == 0) and not np.any(np.signbit(x.astype(np.float32)))


# ----------------------------------------------------------------------------
# the pins have teeth: planted mistakes (in oracle copies, on the CPU) fail them
# ----------------------------------------------------------------------------

def _mutant_eps_inside_sqrt(g, p, m, v, hp, t):
    c = O.adamw_scalars(hp, t)
    m2 = c["b1"] * m + c["omb1"] * g
    v2 = c["b2"] * v + c["omb2"] * (g * g)
    u = (m2 / c["bc1"]) / np.sqrt(v2 / c["bc2"] + c["eps"])
    return p - c["lr"] * (u + c["wd"] * p), m2, v2


def _mutant_no_bias_correction_v(g, p, m, v, hp, t):
    c = O.adamw_scalars(hp, t)
    m2 = c["b1"] * m + c["omb1"] * g
    v2 = c["b2"] * v + c["omb2"] * (g * g)
    u = (m2 / c["bc1"]) / (np.sqrt(v2) + c["eps"])
    return p - c["lr"] * (u + c["wd"] * p), m2, v2


def _mutant_old_moment(g, p, m, v, hp, t):
    c = O.adamw_scalars(hp, t)
    m2 = c["b1"] * m + c["omb1"] * g
    v2 = c["b2"] * v + c["omb2"] * (g * g)
    u = (np.where(t > 1, m, m2) / c["bc1"]) / (np.sqrt(v2 / c["bc2"]) + c["eps"])
    return p - c["lr"] * (u + c["wd"] * p), m2, v2


def _mutant_decay_unscaled(g, p, m, v, hp, t):
    c = O.adamw_scalars(hp, t)
    m2 = c["b1"] * m + c["omb1"] * g
    v2 = c["b2"] * v + c["omb2"] * (g * g)
    u = (m2 / c["bc1"]) / (np.sqrt(v2 / c["bc2"]) + c["eps"])
    return p - (c["lr"] * u + c["wd"] * p), m2, v2


@pytest.mark.parametrize("mutant", [_mutant_eps_inside_sqrt, _mutant_no_bias_correction_v,
                                    _mutant_old_moment, _mutant_decay_unscaled])
def test_planted_adamw_mistakes_fail_the_torch_pin(mutant):
    n = 1 << 12
    p, g1 = _adam_inputs(n, 81)
    grads = [g1] + [O.bf16_widen(datagen.bf16_bits_host(s, 1, np.arange(n), 1e-3))
                    for s in (82, 83)]
    with pytest.raises(AssertionError):
        _check_against_torch(mutant, p, grads)


def test_planted_reduce_mistake_fails_the_bound():
    n_el, n = 4096, 4
    gs = [rng_bf16(91, n_el, 1e-3, k) for k in range(n)]
    L = O.unit_layout([(n_el,)], 1, 0)
    dropped = O.reduce_shard(gs[:-1], L, grad_scale=1.0)      # one rank's buffer lost
    vals = np.stack([O.bf16_widen(g).astype(np.float64) for g in gs])
    exact = vals.sum(axis=0)
    bound = (n - 1) * U32 * np.abs(vals).sum(axis=0) * 1.01
    assert not np.all(np.abs(dropped - exact) <= bound)


def test_splitmix64_known_answer():
    # SplitMix64 seeded with 0 (Vigna's reference splitmix64.c): first three outputs
    out = datagen.splitmix64_host(0, np.arange(3))
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                     0x06C45D188009454F]


def test_generator_random_access_matches_sequential():
    seed = datagen.seed_for(0, 1)
    whole = datagen.bf16_bits_host(seed, 2, np.arange(10000), 1e-3)
    idx = np.array([0, 17, 4095, 9999])
    assert np.array_equal(datagen.bf16_bits_host(seed, 2, idx, 1e-3), whole[idx])
    x = datagen.normal_f32_host(seed, 3, np.arange(1 << 18), 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() / 0.02 - 1) < 0.01
    assert math.isclose(float(np.abs(x).max()) / 0.02, 2 * math.sqrt(3), rel_tol=0.05)
