"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (the stated tolerances for this path's numerics):
* flatten, pad, unflatten, indexing and bf16 copies: bit-exact;
* fp32 master, exp_avg, exp_avg_sq and the fp32 reduced gradient: relative
  error <= 1e-6 element-wise (the design target is bit equality; the tests
  report the bit-equal fraction);
* emitted bf16 parameters: <= 1 bf16 ulp.
Small units are compared on every element. The 7B block at F=8 is compared on
every element of every rank for one step (also with hybrid 2 x 8 rows and with
bf16 partial sums), and on every element of three ranks over two steps; the F
sweep on every element of every rank; full-size inputs also on sampled indices
against host-regenerated inputs; all in the launch configuration the bench
uses. Also here: the tensor-count limit, other
hyper-parameters and step numbers, and the fp32 -> bf16 rounding over all 2^32
fp32 patterns.
"""

import gc

import numpy as np
import pytest
import torch

import datagen
from datagen import workloads as W
from oracle import fsdp_oracle as O
from shard_cases import (BF16_SENTINEL, FP32_SENTINEL, HP, Case, assert_bf16_ulp, assert_bits,
                         assert_rel, gather, to_np)

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


def log(*a):
    print(*a, flush=True)


def run_rank(case: Case, steps: int, emit=True, fused=True, grads_buf=None, grads_ready=False):
    """Init the rank's shard with flatten_pad, then `steps` optimizer steps.

    ``grads_ready``: ``grads_buf`` already holds step 1's rows (one-step runs)."""
    u = fsdp.Unit(case.shapes, case.F, case.rank)
    masters = case.device_master_tensors()
    p = torch.empty(u.S, dtype=torch.float32, device=DEV)
    fsdp.flatten_pad(u, masters, p)
    del masters
    m = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    v = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV) if emit else None
    g32 = None if fused else torch.empty(u.S, dtype=torch.float32, device=DEV)
    for t in range(1, steps + 1):
        grads = grads_buf if grads_ready else case.device_grads(t, out=grads_buf)
        if fused:
            fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, t)
        else:
            fsdp.reduce_shard(u, grads, g32)
            fsdp.adamw_shard(u, g32, p, m, v, w, HPD, t)
    torch.cuda.synchronize()
    return u, p, m, v, w


def compare_full(case, got, want, emit=True):
    u, p, m, v, w = got
    n = u.shard_valid
    pw, mw, vw = want[:3]
    fr = [assert_rel(to_np(p)[:n], pw, what="master"),
          assert_rel(to_np(m)[:n], mw, what="exp_avg"),
          assert_rel(to_np(v)[:n], vw, what="exp_avg_sq")]
    if emit:
        fr.append(assert_bf16_ulp(to_np(w)[:n], want[3], what="bf16 param"))
    return fr


# ---------------------------------------------------------------------------
# generator twin
# ---------------------------------------------------------------------------

def test_device_generator_matches_host():
    seed, oseed = datagen.seed_for(9, 1), datagen.seed_for(9, 2)
    n = (1 << 24) + 123
    b = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    datagen.fill_bf16_(b, seed, 5, 1e-3, start=1000, outlier_seed=oseed)
    f = torch.empty(n, dtype=torch.float32, device=DEV)
    datagen.fill_normal_f32_(f, seed, 6, 0.02, start=77)
    idx = np.unique(np.concatenate([np.arange(4096), np.random.default_rng(0).integers(0, n, 1 << 16),
                                    n - 1 - np.arange(4096)]))
    assert_bits(gather(b, idx), datagen.bf16_bits_host(seed, 5, idx + 1000, 1e-3, oseed), "bf16")
    want = datagen.normal_f32_host(seed, 6, idx + 77, 0.02)
    assert_bits(gather(f, idx).view(np.uint32), want.view(np.uint32), "fp32")


# ---------------------------------------------------------------------------
# tiny unit (every element)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_fused_three_steps_every_element(rank):
    case = Case(W.shapes(W.TINY), 4, rank, config=0)
    log(f"tiny F=4 rank={rank}")
    got = run_rank(case, 3)
    want = case.oracle_full(3)[-1]
    fr = compare_full(case, got, want)
    log("bit-equal fractions master/m/v/w:", fr)


def test_tiny_unfused_matches_oracle_and_fused_bitwise():
    case = Case(W.shapes(W.TINY), 4, 1, config=0)
    fused = run_rank(case, 3)
    unfused = run_rank(case, 3, fused=False)
    for a, b, name in zip(fused[1:], unfused[1:], ["master", "exp_avg", "exp_avg_sq", "w"]):
        assert_bits(to_np(a), to_np(b), f"fused vs unfused {name}")
    compare_full(case, unfused, case.oracle_full(3)[-1])


def test_tiny_reduce_shard_every_element():
    case = Case(W.shapes(W.TINY), 4, 2, config=0)
    u = fsdp.Unit(case.shapes, 4, 2)
    grads = case.device_grads(1)
    out = torch.full((u.S + 64,), float("nan"), dtype=torch.float32, device=DEV)
    out.view(torch.int32).fill_(FP32_SENTINEL)
    fsdp.reduce_shard(u, grads, out)
    torch.cuda.synchronize()
    want = O.reduce_shard(case.host_grads(1), case.L)
    fr = assert_rel(to_np(out)[:u.shard_valid], want, what="reduced grad")
    assert np.all(to_np(out).view(np.uint32)[u.shard_valid:] == FP32_SENTINEL)
    log("reduce bit-equal fraction", fr)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_flatten_pad_windows_bit_exact(dtype):
    rng = np.random.default_rng(4)
    shapes = W.shapes(W.TINY)
    F = 4
    host = [rng.integers(0, 1 << 32, O.numel(s), dtype=np.uint64).astype(np.uint32) for s in shapes]
    if dtype == torch.bfloat16:
        host = [h.astype(np.uint16) for h in host]
        dev = [torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16) for h in host]
    else:
        dev = [torch.from_numpy(h.view(np.float32)).to(DEV) for h in host]
    u = fsdp.Unit(shapes, F, 0)
    windows = [(r * u.S, u.S) for r in range(F)] + [(0, u.padded), (3, 1001), (262141, 9),
                                                    (u.U - 5, 5), (1, 0)]
    for begin, length in windows:
        dst = torch.empty(max(length, 1), dtype=dtype, device=DEV)
        fsdp.flatten_pad(u, dev, dst, begin, length)
        torch.cuda.synchronize()
        want = O.flatten_pad(host, F, begin, length)
        assert_bits(to_np(dst)[:length].view(want.dtype), want, f"window {begin}+{length}")


@pytest.mark.parametrize("src", ["fp32", "bf16"])
def test_tiny_cast_unflatten_bit_exact(src):
    shapes = W.shapes(W.TINY)
    F = 4
    u = fsdp.Unit(shapes, F, 0)
    rng = np.random.default_rng(5)
    if src == "fp32":
        host = [(rng.standard_normal(u.S) * 0.02).astype(np.float32) for _ in range(F)]
        host[1][:6] = np.array([np.inf, -np.inf, np.nan, -0.0, 3.4e38, 1e-40], np.float32)
        dev = [torch.from_numpy(h).to(DEV) for h in host]
    else:
        host = [rng.integers(0, 1 << 16, u.S, dtype=np.uint64).astype(np.uint16) for _ in range(F)]
        dev = [torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16) for h in host]
    outs = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    fsdp.cast_unflatten(u, dev, outs)
    torch.cuda.synchronize()
    want = O.cast_unflatten(host, O.unit_layout(shapes, F, 0), shapes)
    for o, wnt, s in zip(outs, want, shapes):
        assert_bits(to_np(o).reshape(s), wnt, f"tensor {s}")


def test_fp32_to_bf16_cast_on_every_fp32_pattern():
    """The library's fp32 -> bf16 rounding (fsdp_cast_unflatten with fp32 shards,
    the same to_bf16 as the bf16 emission) on all 2^32 fp32 bit patterns, against
    torch's CPU cast, which the oracle's rounding equals on every pattern (the CPU
    pins). NaN inputs must give NaN (payloads are not pinned)."""
    chunk = 1 << 28
    u = fsdp.Unit([(chunk,)], 1, 0)
    out = torch.empty(chunk, dtype=torch.bfloat16, device=DEV)
    bad, first = 0, None
    for start in range(0, 1 << 32, chunk):
        src = torch.arange(start, start + chunk, dtype=torch.int64, device=DEV).to(torch.int32)
        src = src.view(torch.float32)
        fsdp.cast_unflatten(u, [src], [out])
        got = out.cpu().view(torch.int16).numpy().view(np.uint16)
        x = src.cpu()
        del src
        want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = torch.isnan(x).numpy()
        got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        mism = ((got != want) & ~nan) | (nan & ~got_nan)
        n = int(np.count_nonzero(mism))
        if n and first is None:
            first = hex(start + int(np.flatnonzero(mism)[0]))
        bad += n
    assert bad == 0, f"{bad} patterns round differently; first input bits {first}"


def test_round_trip_flatten_then_unflatten_is_identity():
    shapes = W.shapes(W.TINY) + [(7,), (3, 5)]
    for F in (1, 3, 4, 7, 64):
        rng = np.random.default_rng(F)
        host = [rng.integers(0, 1 << 16, O.numel(s), dtype=np.uint64).astype(np.uint16)
                for s in shapes]
        dev = [torch.from_numpy(h.view(np.int16)).to(DEV).view(torch.bfloat16) for h in host]
        units = [fsdp.Unit(shapes, F, r) for r in range(F)]
        shards = []
        for u in units:
            d = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
            fsdp.flatten_pad(u, dev, d)
            shards.append(d)
        outs = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
        fsdp.cast_unflatten(units[0], shards, outs)
        torch.cuda.synchronize()
        for o, h in zip(outs, host):
            assert_bits(to_np(o).reshape(-1), h, f"F={F}")


def test_max_tensor_count_flatten_and_gather_bit_exact():
    """FSDP_MAX_TENSORS ragged tensors (0..8 elements each, many empty, most
    not 16-byte aligned), views into one buffer: every rank's fp32 flatten/pad
    and the gather of the F shards back to bf16 tensors, against the oracle."""
    rng = np.random.default_rng(11)
    sizes = rng.integers(0, 9, 65536)
    sizes[0] = 3
    shapes = [(int(n),) for n in sizes]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    U, F = int(offs[-1]), 8
    host = (rng.standard_normal(U) * 0.02).astype(np.float32)
    src = torch.from_numpy(host).to(DEV)
    tensors = [src[offs[i]:offs[i + 1]] for i in range(sizes.size)]
    units = [fsdp.Unit(shapes, F, r) for r in range(F)]
    shards = []
    for u in units:
        d = torch.empty(u.S, dtype=torch.float32, device=DEV)
        fsdp.flatten_pad(u, tensors, d)
        shards.append(d)
    out = torch.empty(U, dtype=torch.bfloat16, device=DEV)
    outs = [out[offs[i]:offs[i + 1]] for i in range(sizes.size)]
    fsdp.cast_unflatten(units[0], shards, outs)
    torch.cuda.synchronize()
    L = O.unit_layout(shapes, F, 0)
    flat = O.flatten_pad([host[offs[i]:offs[i + 1]].view(np.uint32) for i in range(sizes.size)], F)
    S = L.S
    for r in range(F):
        assert_bits(to_np(shards[r]).view(np.uint32), flat[r * S:(r + 1) * S], f"shard {r}")
    want = O.cast_unflatten([flat.view(np.float32)[r * S:(r + 1) * S] for r in range(F)], L, shapes)
    assert_bits(to_np(out), np.concatenate([np.asarray(w).reshape(-1) for w in want]), "gather")


# ---------------------------------------------------------------------------
# ragged, padded, misaligned, many contributions (every element)
# ---------------------------------------------------------------------------

RAGGED = [
    ([(5,)], 8, None),                       # U < F: ranks 5..7 hold only pad
    ([(3, 7), (1,), (0,), (11,)], 3, None),  # S = 11, odd rank windows, empty tensor
    ([(1000, 3), (17,)], 7, None),           # S = 431: vector head peel and scalar path
    ([(4095,), (2049,)], 5, None),           # several tiles, ragged tail
    ([(300, 41)], 13, None),
    ([(2048 * 3 + 5,)], 2, 9),               # run-time n_grads path (9 rows)
    ([(5000,)], 4, 12),
    ([(4096, 3)], 64, 64),                   # F = 64, 64 rows
    ([(777,)], 1, 33),                       # F = 1 (the DDP point), 33 rows
]


@pytest.mark.parametrize("shapes,F,ng", RAGGED)
def test_ragged_units_every_rank_every_element(shapes, F, ng):
    for rank in range(F):
        case = Case(shapes, F, rank, n_grads=ng, config=5)
        got = run_rank(case, 2)
        if case.L.shard_valid == 0:
            continue
        want = case.oracle_full(2)[-1]
        compare_full(case, got, want)


def test_misaligned_buffers_take_the_scalar_path_and_match():
    case = Case([(333,), (64, 9)], 3, 1, config=6)
    u = fsdp.Unit(case.shapes, 3, 1)
    n = u.shard_valid
    big = [torch.empty(u.U + 3, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    grads = [b[1:1 + u.U] for b in big]                # 2-byte aligned, not 16
    case.device_grads(1, out=grads)
    flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], 3)
    p0 = flat.view(np.float32)[u.shard_begin:u.shard_begin + n]
    store = torch.zeros(4 * (u.S + 4), dtype=torch.float32, device=DEV)
    p = store[1:1 + u.S]
    m = store[u.S + 5:2 * u.S + 5]
    v = store[2 * u.S + 9:3 * u.S + 9]
    p[:n].copy_(torch.from_numpy(p0))
    wbig = torch.empty(u.S + 2, dtype=torch.bfloat16, device=DEV)
    w = wbig[1:1 + u.S]
    fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1)
    torch.cuda.synchronize()
    want = case.oracle_full(1)[-1]
    compare_full(case, (u, p, m, v, w), want)


def test_pad_slots_and_neighbours_are_never_touched():
    # last rank of a padded unit: slots [valid, S) of every output keep their sentinel
    shapes = [(1000, 3), (18,)]               # U = 3018, S = 432, rank 6 holds 426 + 6 pad
    case = Case(shapes, 7, 6, config=7)
    u = fsdp.Unit(shapes, 7, 6)
    assert u.shard_valid < u.S
    grads = case.device_grads(1)
    flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], 7)
    p = torch.from_numpy(flat.view(np.float32)[u.shard_begin:u.shard_begin + u.S].copy()).to(DEV)
    m = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    v = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    n = u.shard_valid
    for t in (p, m, v):
        t.view(torch.int32)[n:].fill_(FP32_SENTINEL)
    w.view(torch.int16)[:].fill_(BF16_SENTINEL)
    fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1)
    torch.cuda.synchronize()
    for t in (p, m, v):
        assert np.all(to_np(t).view(np.uint32)[n:] == FP32_SENTINEL)
    assert np.all(to_np(w)[n:] == BF16_SENTINEL)
    compare_full(case, (u, p, m, v, w), case.oracle_full(1)[-1])


# ---------------------------------------------------------------------------
# full-size 7B block at F = 8 (sampled indices) and the F sweep
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def blk7_grads():
    U = O.unit_layout(W.shapes(W.BLK7), 1, 0).U
    bufs = [torch.empty(U, dtype=torch.bfloat16, device=DEV) for _ in range(8)]
    yield bufs
    del bufs


@pytest.fixture(scope="module")
def sweep_grads():
    """64 rows of the sweep's step-1 gradients (outliers on); row k is rank k's."""
    case = Case(W.shapes(W.BLK7), 64, 0, config=3, outliers=True)
    bufs = case.device_grads(1)
    torch.cuda.synchronize()
    yield bufs
    del bufs


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_blk7_f8_two_steps(rank, blk7_grads):
    """Two fused steps (fresh gradients each step, so step 2 starts from non-zero
    m and v): every element after each step against the oracle on host copies
    of the device fills (spot-checked against the host generator), and sampled
    indices after step 2 against the oracle on host-regenerated inputs."""
    case = Case(W.shapes(W.BLK7), 8, rank, config=1)
    L = case.L
    lo, n = L.shard_begin, L.shard_valid
    log(f"blk7 F=8 rank={rank}")
    u = fsdp.Unit(case.shapes, 8, rank)
    masters = case.device_master_tensors()
    torch.cuda.synchronize()
    host_m = [to_np(t) for t in masters]
    spot = case.sample_indices(2048, seed=rank + 100)
    hp_ = np.concatenate(host_m)[lo + spot]
    assert_bits(hp_.view(np.uint32), case.host_master_at(lo + spot).view(np.uint32), "master fill")
    hp = O.flatten_pad([t.view(np.uint32) for t in host_m], 8).view(np.float32)[lo:lo + n].copy()
    del host_m
    p = torch.empty(u.S, dtype=torch.float32, device=DEV)
    fsdp.flatten_pad(u, masters, p)
    del masters
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    hm, hv = np.zeros(n, np.float32), np.zeros(n, np.float32)
    one = O.unit_layout([(n,)], 1, 0)
    for t in (1, 2):
        grads = case.device_grads(t, out=blk7_grads[:8])
        fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, t)
        torch.cuda.synchronize()
        rows = [to_np(g[lo:lo + n]) for g in grads]
        want_rows = case.host_grads_at(t, lo + spot)
        for k in (0, 7):
            assert_bits(rows[k][spot], want_rows[k], f"step {t} row {k} fill")
        want = O.reduce_adamw_shard(rows, one, hp, hm, hv, HP, t, grad_scale=1.0 / 8,
                                    emit_bf16=True)
        hp, hm, hv = want[:3]
        fr = compare_full(case, (u, p, m, v, w), want)
        log(f"step {t}: every element of {n:,}, bit-equal fractions {fr}")
        del rows
    loc = case.sample_indices()
    want = case.oracle_sampled(loc, 2)[-1]
    assert_rel(gather(p, loc), want[0], what="master")
    assert_rel(gather(m, loc), want[1], what="exp_avg")
    assert_rel(gather(v, loc), want[2], what="exp_avg_sq")
    assert_bf16_ulp(gather(w, loc), want[3], what="bf16 param")


def test_blk7_f8_fused_equals_unfused_full_shard(blk7_grads):
    case = Case(W.shapes(W.BLK7), 8, 5, config=1)
    a = run_rank(case, 1, grads_buf=blk7_grads[:8])
    b = run_rank(case, 1, fused=False, grads_buf=blk7_grads[:8])
    for x, y, name in zip(a[1:], b[1:], ["master", "exp_avg", "exp_avg_sq", "w"]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), name


def test_blk7_cast_unflatten_full_size():
    """The gather of 8 fp32 shards of the 7B block into its 9 bf16 tensors:
    sampled indices against the oracle's rounding of host-regenerated values,
    and every element against the oracle's unflatten of host copies of the
    shards."""
    shapes = W.shapes(W.BLK7)
    F = 8
    u = fsdp.Unit(shapes, F, 0)
    seed = datagen.seed_for(1, 3)
    shards = []
    for k in range(F):
        s = torch.empty(u.S, dtype=torch.float32, device=DEV)
        datagen.fill_normal_f32_(s, seed, k, 0.02)
        shards.append(s)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in shapes]
    fsdp.cast_unflatten(u, shards, outs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for i, (o, s) in enumerate(zip(outs, shapes)):
        n = o.numel()
        j = np.unique(np.concatenate([rng.integers(0, n, 4096), np.arange(min(n, 16)),
                                      n - 1 - np.arange(min(n, 16))]))
        g = u.offsets[i] + j
        k = g // u.S
        src = np.empty(j.size, np.float32)
        for kk in np.unique(k):
            sel = k == kk
            src[sel] = datagen.normal_f32_host(seed, int(kk), g[sel] - kk * u.S, 0.02)
        want = O.bf16_round_nearest_even(src)
        assert_bits(gather(o.reshape(-1), j), want, f"tensor {i}")
    want = O.unflatten([to_np(s_) for s_ in shards], O.unit_layout(shapes, F, 0), shapes,
                       out="bf16")
    for i, (o, e) in enumerate(zip(outs, want)):
        assert_bits(to_np(o).reshape(-1), np.asarray(e).reshape(-1), f"tensor {i} every element")


def test_blk7_f8_every_rank_every_element(blk7_grads):
    """The 7B block at F=8 in full: every rank's shard, every element, one
    fused step with bf16 emission, then the gather of the eight emitted shards
    into the nine tensors.

    Inputs are the seeded generator's device fills, spot-checked here against
    its host form; the expected values are the oracle's on host copies of
    those fills."""
    shapes, F = W.shapes(W.BLK7), 8
    case0 = Case(shapes, F, 0, config=1)
    grads = case0.device_grads(1, out=blk7_grads[:8])
    masters = case0.device_master_tensors()
    torch.cuda.synchronize()
    U = case0.L.U
    idx = np.unique(np.concatenate([np.random.default_rng(7).integers(0, U, 4096),
                                    np.arange(8), U - 1 - np.arange(8)]))
    for k in (0, F - 1):
        assert_bits(gather(grads[k], idx), case0.host_grads_at(1, idx)[k], f"row {k} fill")
    assert_bits(np.concatenate([to_np(t) for t in masters])[idx].view(np.uint32),
                case0.host_master_at(idx).view(np.uint32), "master fill")
    rows = [to_np(g) for g in grads]
    flat = O.flatten_pad([to_np(t).view(np.uint32) for t in masters], F).view(np.float32)
    emitted = []
    for rank in range(F):
        u = fsdp.Unit(shapes, F, rank)
        p = torch.empty(u.S, dtype=torch.float32, device=DEV)
        fsdp.flatten_pad(u, masters, p)
        m = torch.zeros(u.S, dtype=torch.float32, device=DEV)
        v = torch.zeros(u.S, dtype=torch.float32, device=DEV)
        w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
        fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1)
        torch.cuda.synchronize()
        L = O.unit_layout(shapes, F, rank)
        lo, hi = L.shard_begin, L.shard_begin + L.shard_valid
        z = np.zeros(L.shard_valid, np.float32)
        want = O.reduce_adamw_shard(rows, L, flat[lo:hi].copy(), z, z.copy(), HP, 1,
                                    grad_scale=1.0 / F, emit_bf16=True)
        fr = compare_full(Case(shapes, F, rank, config=1), (u, p, m, v, w), want)
        log(f"rank {rank}: bit-equal fractions {fr}")
        emitted.append(w)
        del p, m, v
    u = fsdp.Unit(shapes, F, 0)
    outs = [torch.empty(sh, dtype=torch.bfloat16, device=DEV) for sh in shapes]
    fsdp.cast_unflatten(u, emitted, outs)
    torch.cuda.synchronize()
    want = O.unflatten([to_np(w) for w in emitted], O.unit_layout(shapes, F, 0), shapes)
    for i, (o, e) in enumerate(zip(outs, want)):
        assert_bits(to_np(o).reshape(-1), np.asarray(e).reshape(-1), f"gathered tensor {i}")


@pytest.fixture(scope="module")
def sweep_master_host():
    """Host copy of the sweep's master tensors as the device twin fills them
    (the same for every F), spot-checked against the host generator."""
    case = Case(W.shapes(W.BLK7), 1, 0, config=3, outliers=True)
    masters = case.device_master_tensors()
    host = [to_np(t) for t in masters]
    del masters
    idx = np.unique(np.concatenate([np.random.default_rng(11).integers(0, case.L.U, 8192),
                                    np.arange(8), case.L.U - 1 - np.arange(8)]))
    flat = np.concatenate(host)
    assert_bits(flat[idx].view(np.uint32), case.host_master_at(idx).view(np.uint32),
                "sweep master fill")
    yield host
    del host, flat


@pytest.mark.parametrize("F", [1, 2, 4, 8, 16, 64, 7, 11, 13])
def test_blk7_sharding_factor_sweep_every_element(F, sweep_grads, sweep_master_host):
    """Every element of every rank of every sharding factor, one fused step with
    emission. The oracle runs on host copies of the device fills (rows
    spot-checked here, masters in the fixture)."""
    shapes = W.shapes(W.BLK7)
    flat = O.flatten_pad([t.view(np.uint32) for t in sweep_master_host], F).view(np.float32)
    for rank in range(F):
        case = Case(shapes, F, rank, config=3, outliers=True)
        L = case.L
        lo, n = L.shard_begin, L.shard_valid
        u, p, m, v, w = run_rank(case, 1, grads_buf=sweep_grads[:F], grads_ready=True)
        rows = [to_np(g[lo:lo + n]) for g in sweep_grads[:F]]
        loc = case.sample_indices(2048, seed=F * 64 + rank + 1)
        want_rows = case.host_grads_at(1, lo + loc)
        for k in {0, F - 1}:
            assert_bits(rows[k][loc], want_rows[k], f"F={F} rank={rank} row {k} fill")
        z = np.zeros(n, np.float32)
        want = O.reduce_adamw_shard(rows, O.unit_layout([(n,)], 1, 0), flat[lo:lo + n].copy(),
                                    z, z.copy(), HP, 1, grad_scale=1.0 / F, emit_bf16=True)
        fr = compare_full(case, (u, p, m, v, w), want)
        if rank in (0, F - 1):
            log(f"sweep F={F} rank={rank}: every element of {n:,}, bit-equal fractions {fr}")
        del p, m, v, w, rows, want


@pytest.mark.parametrize("F", [1, 2, 4, 8, 16, 64, 7, 11, 13])
def test_blk7_sharding_factor_sweep_with_outliers_sampled(F, sweep_grads):
    """Every rank of every sharding factor (ranks 0 and F-1 with more samples)."""
    for rank in range(F):
        case = Case(W.shapes(W.BLK7), F, rank, config=3, outliers=True)
        log(f"sweep F={F} rank={rank} S={case.L.S} valid={case.L.shard_valid}")
        u, p, m, v, w = run_rank(case, 1, grads_buf=sweep_grads[:F], grads_ready=True)
        n = 1 << 15 if rank in (0, F - 1) else (1 << 15) // F
        loc = case.sample_indices(n, seed=F * 64 + rank)
        want = case.oracle_sampled(loc, 1)[-1]
        assert_rel(gather(p, loc), want[0], what="master")
        assert_rel(gather(m, loc), want[1], what="exp_avg")
        assert_rel(gather(v, loc), want[2], what="exp_avg_sq")
        assert_bf16_ulp(gather(w, loc), want[3], what="bf16 param")
        del p, m, v, w


# ---------------------------------------------------------------------------
# hyper-parameters, step numbers and optimizer state other than the defaults
# ---------------------------------------------------------------------------

HP_CASES = [
    # lr, beta1, beta2, eps, weight_decay, grad_scale, step
    (3e-4, 0.8, 0.95, 1e-6, 0.1, 0.3, 1),
    (1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 12345),
    (1e-5, 0.0, 0.5, 1e-12, 0.5, 0.125, 7),
    (2e-2, 0.99, 0.9999, 1e-8, 0.01, 1.0 / 3, 1 << 20),
]


@pytest.mark.parametrize("case", HP_CASES)
@pytest.mark.parametrize("fused", [True, False])
def test_other_hyperparameters_and_steps_bit_equal(case, fused):
    """Fused and unfused steps from a non-zero optimizer state (m ~ N, v ~ |N|),
    at a given step number, against the oracle, bit for bit."""
    lr, b1, b2, eps, wd, gs, step = case
    shapes, F, rank = [(1000, 7), (33,)], 4, 1
    L = O.unit_layout(shapes, F, rank)
    n = L.shard_valid
    rng = np.random.default_rng(step)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    rows = [datagen.bf16_bits_host(datagen.seed_for(11, 1, 1), k, np.arange(L.U), 1e-3)
            for k in range(F)]
    u = fsdp.Unit(shapes, F, rank)
    dp, dm, dv = (torch.from_numpy(x.copy()).to(DEV) for x in (p, m, v))
    dw = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    dg = [torch.from_numpy(r.view(np.int16)).to(DEV).view(torch.bfloat16) for r in rows]
    hp = fsdp.AdamWHparams(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    if fused:
        fsdp.reduce_adamw_shard(u, dg, dp, dm, dv, dw, hp, step, grad_scale=gs)
    else:
        g32 = torch.empty(u.S, dtype=torch.float32, device=DEV)
        fsdp.reduce_shard(u, dg, g32, grad_scale=gs)
        fsdp.adamw_shard(u, g32, dp, dm, dv, dw, hp, step)
    torch.cuda.synchronize()
    ohp = O.AdamW(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    want = O.reduce_adamw_shard(rows, L, p, m, v, ohp, step, grad_scale=gs, emit_bf16=True)
    for got, exp, name in zip((dp, dm, dv, dw), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"{name} bits")


# ---------------------------------------------------------------------------
# design target: bit equality (stricter than the stated tolerances)
# ---------------------------------------------------------------------------

def _bits(x):
    x = np.asarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


@pytest.mark.parametrize("shapes,F,rank,ng", [
    (W.shapes(W.TINY), 4, 1, None), ([(1000, 3), (17,)], 7, 3, None), ([(5000,)], 4, 2, 12),
])
def test_fused_step_is_bit_equal_to_the_oracle(shapes, F, rank, ng):
    """Same binary32 op order, no contraction, correctly rounded div/sqrt on both sides."""
    case = Case(shapes, F, rank, n_grads=ng, config=8)
    u, p, m, v, w = run_rank(case, 3)
    n = u.shard_valid
    want = case.oracle_full(3)[-1]
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"{name} bits")


def test_blk7_f8_sampled_bit_equal(blk7_grads):
    case = Case(W.shapes(W.BLK7), 8, 2, config=1)
    u, p, m, v, w = run_rank(case, 2, grads_buf=blk7_grads[:8])
    loc = case.sample_indices()
    want = case.oracle_sampled(loc, 2)[-1]
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(gather(got, loc)), _bits(exp), f"{name} bits")


# ---------------------------------------------------------------------------
# gradient rows whose window is not 8-byte aligned (shifted-row vector path)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shift", [1, 2, 3, "mixed"])
@pytest.mark.parametrize("ng", [8, 9])
@pytest.mark.parametrize("fused", [True, False])
def test_shifted_rows_with_aligned_state(shift, ng, fused):
    """Rank 1 of F=4 with S = 5283 (odd): the rank window starts 6 bytes past an 8-byte
    boundary, and each row is further offset by `shift` elements ("mixed": row k by
    k mod 4, so the rows' windows sit at all four 2-byte offsets from 8-byte
    boundaries). 21 full 252-element runs and a ragged end; 8 rows (compile-time fold)
    and 9 (run-time fold ending in a partial chunk)."""
    shapes = [(3000, 7), (129,)]
    F, rank = 4, 1
    case = Case(shapes, F, rank, n_grads=ng, config=10)
    u = fsdp.Unit(shapes, F, rank)
    big = [torch.empty(u.U + 8, dtype=torch.bfloat16, device=DEV) for _ in range(ng)]
    offs = [k % 4 if shift == "mixed" else shift for k in range(ng)]
    grads = [b[o:o + u.U] for b, o in zip(big, offs)]   # 2*o bytes past a 512-byte boundary
    case.device_grads(1, out=grads)
    flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], F)
    n = u.shard_valid
    p = torch.from_numpy(flat.view(np.float32)[u.shard_begin:u.shard_begin + u.S].copy()).to(DEV)
    m = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    v = torch.zeros(u.S, dtype=torch.float32, device=DEV)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    if fused:
        fsdp.reduce_adamw_shard(u, grads, p, m, v, w, HPD, 1)
    else:
        g32 = torch.full((u.S,), float("nan"), dtype=torch.float32, device=DEV)
        fsdp.reduce_shard(u, grads, g32)
        torch.cuda.synchronize()
        want_g = O.reduce_shard(case.host_grads(1), case.L)
        assert_bits(to_np(g32)[:n].view(np.uint32), want_g.view(np.uint32), "reduced grad")
        fsdp.adamw_shard(u, g32, p, m, v, w, HPD, 1)
    torch.cuda.synchronize()
    want = case.oracle_full(1)[-1]
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"{name} bits")


# ---------------------------------------------------------------------------
# tiles visited in XCD runs: every element of a long launch, ragged
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ng", [3, 8, 16])
@pytest.mark.parametrize("offset", [12, 1], ids=["rows_off_line", "rows_shifted"])
@pytest.mark.parametrize("fused", [False, True])
def test_xcd_runs_cover_every_element(offset, fused, ng):
    """ng gradient rows whose windows start `offset` elements past a 128-byte line (12:
    8-byte aligned, the vector path; 1: 2 bytes off, the shifted path), over
    2^23 + 12345 elements: both paths visit their tiles in runs of 8 per XCD (with 8
    and 16 rows the fused vector path stages its loads in the general kernel). The
    launch has 32,817 one-wave tiles: 512 whole groups of 64 (8 runs of 8) and 49 tiles
    past them in the plain order, the last one ragged. Every element against the
    oracle, bit for bit."""
    n = (1 << 23) + 12345
    shapes, F, rank = [(n,)], 1, 0
    u = fsdp.Unit(shapes, F, rank)
    L = O.unit_layout(shapes, F, rank)
    seed = datagen.seed_for(46, 1, 1)
    bufs = [torch.empty(n + 64, dtype=torch.bfloat16, device=DEV) for _ in range(ng)]
    rows = [b[offset:offset + n] for b in bufs]
    for k, r in enumerate(rows):
        datagen.fill_bf16_(r, seed, k, W.GRAD_SIGMA)
    host = [to_np(r) for r in rows]
    if not fused:
        out = torch.empty(n, dtype=torch.float32, device=DEV)
        fsdp.reduce_shard(u, rows, out)
        torch.cuda.synchronize()
        assert_bits(to_np(out).view(np.uint32), O.reduce_shard(host, L).view(np.uint32),
                    f"reduce, rows {offset} elements off a line")
        return
    p = torch.empty(n, dtype=torch.float32, device=DEV)
    datagen.fill_normal_f32_(p, datagen.seed_for(46, 0), 0, W.MASTER_SIGMA)
    m = torch.empty(n, dtype=torch.float32, device=DEV)
    datagen.fill_normal_f32_(m, datagen.seed_for(46, 0), 1, 1e-4)
    v = torch.empty(n, dtype=torch.float32, device=DEV)
    datagen.fill_normal_f32_(v, datagen.seed_for(46, 0), 2, 1e-6)
    v.abs_()
    p0, m0, v0 = to_np(p).copy(), to_np(m).copy(), to_np(v).copy()
    w = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    fsdp.reduce_adamw_shard(u, rows, p, m, v, w, HPD, 3)
    torch.cuda.synchronize()
    want = O.reduce_adamw_shard(host, L, p0, m0, v0, HP, 3, emit_bf16=True)
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(to_np(got)), _bits(exp), f"fused {name}, rows {offset} elements off a line")


# ---------------------------------------------------------------------------
# the one-tile kernel of the staged fused step: every element, ragged end
# ---------------------------------------------------------------------------

ONE_TILE_CASES = [
    # name, unit F, replicas, rows, bf16 partials, emit
    ("flat8", 1, 1, 8, False, True),
    ("flat8_no_emit", 1, 1, 8, False, False),
    ("flat16", 1, 1, 16, False, True),
    ("hybrid_2x4", 4, 2, 8, False, True),
    ("hybrid_3x8", 8, 3, 24, False, True),
    ("hybrid_4x8", 8, 4, 32, False, True),
    ("bf16acc8", 1, 1, 8, True, True),
    ("bf16acc16", 1, 1, 16, True, True),
    ("runtime11", 1, 1, 11, False, True),
]


@pytest.mark.parametrize("name,F,R,ng,bacc,emit", ONE_TILE_CASES, ids=[c[0] for c in ONE_TILE_CASES])
def test_one_tile_kernel_ragged_end_every_element(name, F, R, ng, bacc, emit):
    """The staged fused step in its one-tile kernel (one-wave workgroups, every window
    on a 128-byte line, 2^23 + 131 elements): the last tile holds 32 whole lanes and a
    3-element scalar tail. Every element against the oracle, bit for bit, from a
    non-zero optimizer state at step 3, with NaN guards after every output window."""
    n = (1 << 23) + 131
    u = fsdp.Unit([(F * n,)], F, 0)
    L = O.unit_layout([(F * n,)], F, 0)
    assert u.shard_valid == n and u.shard_begin == 0
    seed = datagen.seed_for(47, 1, 1)
    rows = [torch.empty(F * n, dtype=torch.bfloat16, device=DEV) for _ in range(ng)]
    for k, r in enumerate(rows):                  # rank 0 reads [0, n) of each row
        datagen.fill_bf16_(r[:n], seed, k, W.GRAD_SIGMA)
    host = [to_np(r[:n]) for r in rows]
    G = 64

    def guarded(dtype, bits):
        buf = torch.empty(n + G, dtype=dtype, device=DEV)
        buf.view(torch.int32 if dtype == torch.float32 else torch.int16).fill_(bits)
        return buf

    pb, mb, vb = (guarded(torch.float32, FP32_SENTINEL) for _ in range(3))
    sseed = datagen.seed_for(47, 0)
    datagen.fill_normal_f32_(pb[:n], sseed, 0, W.MASTER_SIGMA)
    datagen.fill_normal_f32_(mb[:n], sseed, 1, 1e-4)
    datagen.fill_normal_f32_(vb[:n], sseed, 2, 1e-6)
    vb[:n].abs_()
    p0, m0, v0 = (to_np(b[:n]).copy() for b in (pb, mb, vb))
    wb = guarded(torch.bfloat16, BF16_SENTINEL) if emit else None
    w = wb[:n] if emit else None
    if R > 1:
        fsdp.reduce_adamw_shard_hybrid(u, R, rows, pb[:n], mb[:n], vb[:n], w, HPD, 3)
        want = O.reduce_adamw_shard_hybrid(host, L, R, p0, m0, v0, HP, 3, emit_bf16=emit)
    elif bacc:
        fsdp.reduce_adamw_shard_bf16acc(u, rows, pb[:n], mb[:n], vb[:n], w, HPD, 3)
        want = O.reduce_adamw_shard_bf16acc(host, L, p0, m0, v0, HP, 3, emit_bf16=emit)
    else:
        fsdp.reduce_adamw_shard(u, rows, pb[:n], mb[:n], vb[:n], w, HPD, 3)
        want = O.reduce_adamw_shard(host, L, p0, m0, v0, HP, 3, emit_bf16=emit)
    torch.cuda.synchronize()
    outs = [(pb, "master", FP32_SENTINEL), (mb, "exp_avg", FP32_SENTINEL),
            (vb, "exp_avg_sq", FP32_SENTINEL)] + ([(wb, "w", BF16_SENTINEL)] if emit else [])
    for (buf, nm, sent), exp in zip(outs, want):
        got = to_np(buf)
        assert_bits(_bits(got[:n]), _bits(exp), f"{name} {nm}")
        tail = got[n:].view(np.uint32) if got.dtype == np.float32 else got[n:]
        assert (tail == sent).all(), f"{name} {nm}: guard after the window"


# ---------------------------------------------------------------------------
# hybrid sharding (HSDP): R replica groups of F ranks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,F", [(2, 2), (2, 4), (3, 4), (2, 8), (3, 8), (4, 8), (8, 8)])   # 8 x 8: 64 rows
def test_hybrid_fused_every_rank_every_element(R, F):
    shapes = [(1000, 7), (33,)]
    for rank in range(F):
        case = Case(shapes, F, rank, config=30, replicas=R)
        u = fsdp.Unit(shapes, F, rank)
        grads = case.device_grads(1)
        flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], F)
        p = torch.from_numpy(flat.view(np.float32)[u.shard_begin:u.shard_begin + u.S].copy()).to(DEV)
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
        fsdp.reduce_adamw_shard_hybrid(u, R, grads, p, m, v, w, HPD, 1)
        torch.cuda.synchronize()
        want = case.oracle_full(1)[-1]
        n = u.shard_valid
        for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
            assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"R={R} F={F} r={rank} {name}")


@pytest.mark.parametrize("R,F,rank", [(2, 4, 1), (3, 7, 3),      # F=7: odd S, scalar path
                                      (2, 8, 5)])                 # compile-time 2 x 8 fold
def test_hybrid_reduce_shard_every_element(R, F, rank):
    shapes = [(2049,), (7, 9)]
    case = Case(shapes, F, rank, config=31, replicas=R)
    u = fsdp.Unit(shapes, F, rank)
    grads = case.device_grads(1)
    out = torch.empty(u.S, dtype=torch.float32, device=DEV)
    fsdp.reduce_shard_hybrid(u, R, grads, out)
    torch.cuda.synchronize()
    want = O.reduce_shard_hybrid(case.host_grads(1), case.L, R)
    assert_bits(to_np(out)[:u.shard_valid].view(np.uint32), want.view(np.uint32), "hybrid reduce")


def blk7_every_rank_every_element(config, step_fn, **case_kw):
    """One fused step of the 7B block at F=8 on every rank, compared with the
    oracle on every element. The oracle runs on host copies of the device
    fills (gradient rows and master tensors), spot-checked against the host
    generator first; step_fn(u, grads, p, m, v, w) calls the library."""
    shapes, F = W.shapes(W.BLK7), 8
    case0 = Case(shapes, F, 0, config=config, **case_kw)
    grads = case0.device_grads(1)
    masters = case0.device_master_tensors()
    torch.cuda.synchronize()
    U = case0.L.U
    idx = np.unique(np.concatenate([np.random.default_rng(config).integers(0, U, 4096),
                                    np.arange(8), U - 1 - np.arange(8)]))
    want_rows = case0.host_grads_at(1, idx)
    for k in (0, len(grads) - 1):
        assert_bits(gather(grads[k], idx), want_rows[k], f"row {k} fill")
    host_m = [to_np(t) for t in masters]
    assert_bits(np.concatenate(host_m)[idx].view(np.uint32),
                case0.host_master_at(idx).view(np.uint32), "master fill")
    rows = [to_np(g) for g in grads]
    flat = O.flatten_pad([t.view(np.uint32) for t in host_m], F).view(np.float32)
    del host_m
    for rank in range(F):
        case = Case(shapes, F, rank, config=config, **case_kw)
        u = fsdp.Unit(shapes, F, rank)
        p = torch.empty(u.S, dtype=torch.float32, device=DEV)
        fsdp.flatten_pad(u, masters, p)
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
        step_fn(u, grads, p, m, v, w)
        torch.cuda.synchronize()
        lo, n = u.shard_begin, u.shard_valid
        z = np.zeros(n, np.float32)
        want = case._step(rows, case.L, flat[lo:lo + n].copy(), z, z.copy(), 1, True)
        for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
            assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"blk7 rank {rank} {name}")
        log(f"blk7 F=8 rank {rank}: every element of {n:,} bit-equal")
        del p, m, v, w, want


def test_hybrid_blk7_two_groups_of_8_every_rank_every_element():
    blk7_every_rank_every_element(
        32, lambda u, g, p, m, v, w: fsdp.reduce_adamw_shard_hybrid(u, 2, g, p, m, v, w, HPD, 1),
        replicas=2)


# ---------------------------------------------------------------------------
# reduce dtype bf16: bf16 partial sums
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shapes,F,ng", [([(1000, 7), (33,)], 4, 4), ([(1000, 7), (33,)], 8, 8),
                                         ([(5000,)], 4, 12), ([(1000, 3), (17,)], 7, 7),
                                         ([(1000, 7), (33,)], 8, 16),
                                         ([(1000, 7), (33,)], 8, 64)])     # the row limit
def test_bf16acc_fused_every_rank_every_element(shapes, F, ng):
    for rank in range(F):
        case = Case(shapes, F, rank, n_grads=ng, config=40, outliers=True, bf16acc=True)
        u = fsdp.Unit(shapes, F, rank)
        grads = case.device_grads(1)
        flat = O.flatten_pad([t.view(np.uint32) for t in case.host_master_tensors()], F)
        p = torch.from_numpy(flat.view(np.float32)[u.shard_begin:u.shard_begin + u.S].copy()).to(DEV)
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
        fsdp.reduce_adamw_shard_bf16acc(u, grads, p, m, v, w, HPD, 1)
        torch.cuda.synchronize()
        want = case.oracle_full(1)[-1]
        n = u.shard_valid
        for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
            assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"bf16acc F={F} r={rank} {name}")


@pytest.mark.parametrize("ng", [4, 8, 16])       # 8 and 16: the compile-time folds
def test_bf16acc_reduce_shard_every_element_and_coarser_than_fp32(ng):
    shapes, F, rank = [(4096, 5)], 4, 2
    case = Case(shapes, F, rank, n_grads=ng, config=41, outliers=True, bf16acc=True)
    u = fsdp.Unit(shapes, F, rank)
    grads = case.device_grads(1)
    out = torch.empty(u.S, dtype=torch.float32, device=DEV)
    fsdp.reduce_shard_bf16acc(u, grads, out)
    torch.cuda.synchronize()
    host = case.host_grads(1)
    want = O.reduce_shard_bf16acc(host, case.L)
    assert_bits(to_np(out).view(np.uint32), want.view(np.uint32), "bf16acc reduce")
    assert not np.array_equal(want, O.reduce_shard(host, case.L))


def test_bf16acc_blk7_every_rank_every_element():
    blk7_every_rank_every_element(
        42, lambda u, g, p, m, v, w: fsdp.reduce_adamw_shard_bf16acc(u, g, p, m, v, w, HPD, 1),
        outliers=True, bf16acc=True)


@pytest.mark.parametrize("n_grads", [8, 11, 24])
def test_unfused_long_launch(n_grads):
    """fsdp_reduce_shard then fsdp_adamw_shard on a 202,383,360-element shard (the 7B
    block at F=1): 8 gradient rows (a compile-time fold in one-wave workgroups, 16
    per CU for this reduce, 11 for the AdamW), 11 and 24 rows (a run-time count
    folded in chunks of 8; the 11-row fold ends in a partial chunk); two steps. Every
    element of the reduced gradient and of the state after each step against the
    oracle on host copies of the device fills (spot-checked against the host
    generator), and sampled indices against host-regenerated inputs."""
    case = Case(W.shapes(W.BLK7), 1, 0, n_grads=n_grads, config=44)
    u = fsdp.Unit(case.shapes, 1, 0)
    L = case.L
    n = u.shard_valid
    assert n >= 1 << 25
    masters = case.device_master_tensors()
    spot = case.sample_indices(4096, seed=n_grads)
    torch.cuda.synchronize()
    host_m = [to_np(t) for t in masters]
    assert_bits(np.concatenate(host_m)[spot].view(np.uint32),
                case.host_master_at(spot).view(np.uint32), "master fill")
    hp = O.flatten_pad([t.view(np.uint32) for t in host_m], 1).view(np.float32)[:n].copy()
    hm, hv = np.zeros(n, np.float32), np.zeros(n, np.float32)
    del host_m
    p = torch.empty(u.S, dtype=torch.float32, device=DEV)
    fsdp.flatten_pad(u, masters, p)
    del masters
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    w = torch.empty(u.S, dtype=torch.bfloat16, device=DEV)
    g32 = torch.empty(u.S, dtype=torch.float32, device=DEV)
    grads = None
    for t in (1, 2):
        grads = case.device_grads(t, out=grads)
        fsdp.reduce_shard(u, grads, g32)
        fsdp.adamw_shard(u, g32, p, m, v, w, HPD, t)
        torch.cuda.synchronize()
        rows = [to_np(g) for g in grads]
        want_rows = case.host_grads_at(t, spot)
        for k in (0, n_grads - 1):
            assert_bits(rows[k][spot], want_rows[k], f"step {t} row {k} fill")
        gw = O.reduce_shard(rows, L)
        del rows
        assert_bits(to_np(g32)[:n].view(np.uint32), gw.view(np.uint32), f"step {t} reduced gradient")
        want = O.adamw_step(gw, hp, hm, hv, HP, t, True)
        hp, hm, hv = want[:3]
        for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
            assert_bits(_bits(to_np(got)[:n]), _bits(exp), f"unfused F=1 {n_grads} rows step {t} {name}")
        log(f"{n_grads} rows step {t}: every element of {n:,} bit-equal")
    torch.cuda.synchronize()
    loc = case.sample_indices()
    want = case.oracle_sampled(loc, 2)[-1]
    for got, exp, name in zip((p, m, v, w), want, ("master", "exp_avg", "exp_avg_sq", "w")):
        assert_bits(_bits(gather(got, loc)), _bits(exp), f"unfused F=1 {n_grads} rows {name}")


def test_sharded_steps_concatenated_equal_the_ddp_step():
    """[NOTE-003, "Key results"]: F = 1 is plain data parallelism. All 8 ranks' F=8 shard
    steps, concatenated, equal the F=1 step over the same 8 gradient rows, bitwise."""
    shapes = W.shapes(W.BLK7)
    rows = Case(shapes, 8, 0, config=43).device_grads(1)
    ddp = fsdp.Unit(shapes, 1, 0)
    masters = Case(shapes, 8, 0, config=43).device_master_tensors()
    full = [torch.empty(ddp.S, dtype=torch.float32, device=DEV)]
    fsdp.flatten_pad(ddp, masters, full[0])
    full += [torch.zeros_like(full[0]), torch.zeros_like(full[0]),
             torch.empty(ddp.S, dtype=torch.bfloat16, device=DEV)]
    shards = []
    for r in range(8):
        u = fsdp.Unit(shapes, 8, r)
        st = [full[0][u.shard_begin:u.shard_begin + u.S].clone()]
        st += [torch.zeros_like(st[0]), torch.zeros_like(st[0]),
               torch.empty(u.S, dtype=torch.bfloat16, device=DEV)]
        fsdp.reduce_adamw_shard(u, rows, *st, HPD, 1)
        shards.append(st)
    fsdp.reduce_adamw_shard(ddp, rows, *full, HPD, 1)
    torch.cuda.synchronize()
    for j in range(4):
        cat = torch.cat([s[j] for s in shards])[:ddp.U]
        a = cat.view(torch.int16 if cat.dtype == torch.bfloat16 else torch.int32)
        b = full[j].view(torch.int16 if full[j].dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(a, b), j
