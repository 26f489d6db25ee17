"""GPU parity on IEEE special values in the step kernels.

The reductions and the optimizer run in fp32 ([Glossary, "FSDP Implementation
(PyTorch)" -> Mixed Precision]); the library's readings are binary32 round to
nearest even per operation, denormals kept (no flush to zero), -0.0 kept by a
left fold that starts from rank 0's value, and NaN results compared as NaN
(payloads are not fixed by the pages). These tests plant -0.0, subnormal bf16
and fp32 values, values near the largest finite ones (so that g*g and sums
overflow to infinity), +-infinity and NaN (quiet and signalling patterns) in
the gradient rows and in master, m and v, and compare every output element with
the oracle: bit-equal, or NaN on both sides.

Paths covered: the vector path (aligned windows, with and without a ragged
tail), the shifted-row path (a rank window r*S with S odd), the scalar path
(fp32 state not 16-byte aligned), long fused launches (a 25M-element shard
with 8 rows in one-wave workgroups, and 11 and 64 rows folded in chunks of 8
at run time; sampled), the compile-time grouped folds (hybrid
sharding, bf16 partial sums) and a run-time row count; entry points: fused
with and without the bf16 emission, and the unfused reduce + AdamW pair. The
run-time fold starts from -0.0 rather than from rank 0's value; -0.0 is the
exact identity of IEEE addition, so the sums are the same, and the planted
-0.0 rows check that.
"""

import zlib

import numpy as np
import pytest
import torch

from conftest import gpu_available
from shard_cases import HP, to_np
from oracle import fsdp_oracle as O
import datagen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

BF16_SPECIAL = np.array([
    0x0000, 0x8000,                  # +0, -0
    0x0001, 0x8001, 0x007F, 0x807F,  # subnormals (smallest, largest)
    0x0080, 0x8080,                  # smallest normals
    0x7F7F, 0xFF7F, 0x7F00,          # largest finite, and a value whose square overflows
    0x7F80, 0xFF80,                  # +-inf
    0x7FC0, 0xFFC1, 0x7F81,          # quiet NaNs, a signalling NaN pattern
    0x3F80, 0xBF80,                  # +-1
], dtype=np.uint16)

F32_SPECIAL = np.array([
    0x00000000, 0x80000000,          # +0, -0
    0x00000001, 0x80000001,          # smallest subnormals
    0x007FFFFF, 0x807FFFFF,          # largest subnormals
    0x00800000,                      # smallest normal
    0x7F7FFFFF, 0xFF7FFFFF,          # largest finite
    0x7F800000, 0xFF800000,          # +-inf
    0x7FC00000, 0xFFC00001, 0x7FA00000,   # NaNs (quiet, quiet with payload, signalling pattern)
    0x3F800000, 0x1E3CE508,          # 1, ~1e-20 (squares to a subnormal)
], dtype=np.uint32)


def is_nan32(b):
    b = np.asarray(b, dtype=np.uint32)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)


def is_nan16(b):
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def assert_f32_parity(got, want, what):
    g = np.asarray(got, dtype=np.float32).view(np.uint32)
    w = np.asarray(want, dtype=np.float32).view(np.uint32)
    ok = (g == w) | (is_nan32(g) & is_nan32(w))
    if not ok.all():
        bad = np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements differ; first at "
                             f"{bad.tolist()}: got {[hex(x) for x in g[bad]]} "
                             f"want {[hex(x) for x in w[bad]]}")


def assert_bf16_parity(got, want, what):
    g = np.asarray(got, dtype=np.uint16)
    w = np.asarray(want, dtype=np.uint16)
    ok = (g == w) | (is_nan16(g) & is_nan16(w))
    if not ok.all():
        bad = np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements differ; first at "
                             f"{bad.tolist()}: got {[hex(x) for x in g[bad]]} "
                             f"want {[hex(x) for x in w[bad]]}")


# ---------------------------------------------------------------------------
# inputs: normal draws with specials planted, plus fixed structured columns
# ---------------------------------------------------------------------------

def planted_rows(n_rows, n, seed):
    """n_rows bf16 rows of n elements: normal draws, ~35% replaced by specials, and
    structured columns at the start: all rows -0.0; +inf against -inf; every row
    the largest finite value (the sum overflows); one row largest, the rest 0
    (g*g overflows); every row the smallest subnormal; mixed-sign subnormals."""
    rng = np.random.default_rng(seed)
    rows = []
    for k in range(n_rows):
        r = datagen.bf16_bits_host(datagen.seed_for(9, 1, seed), k, np.arange(n), 1e-3)
        mask = rng.random(n) < 0.35
        r[mask] = rng.choice(BF16_SPECIAL, int(mask.sum()))
        rows.append(r)
    cols = [
        [0x8000] * n_rows,
        [0x7F80, 0xFF80] + [0x0000] * (n_rows - 2),
        [0x7F7F] * n_rows,
        [0x7F7F] + [0x0000] * (n_rows - 1),
        [0x0001] * n_rows,
        [0x0001 if k % 2 == 0 else 0x8001 for k in range(n_rows)],
        [0x8000] + [0x0000] * (n_rows - 1),
        [0x0000] + [0x8000] * (n_rows - 1),
    ]
    for j, col in enumerate(cols):
        if j < n:
            for k in range(n_rows):
                rows[k][j] = col[k]
    return rows


def planted_state(n, seed):
    """fp32 master, m, v: normal draws with ~25% replaced by specials."""
    rng = np.random.default_rng(seed + 1)
    out = []
    for kind, sigma in ((0, 0.02), (1, 1e-4), (2, 1e-6)):
        x = datagen.normal_f32_host(datagen.seed_for(9, 0, seed), kind, np.arange(n), sigma)
        if kind == 2:
            x = np.abs(x)
        mask = rng.random(n) < 0.25
        x.view(np.uint32)[mask] = rng.choice(F32_SPECIAL, int(mask.sum()))
        out.append(x.astype(np.float32))
    return out


def dev_u16(a, lead=0, extra=0):
    """A bf16 device tensor holding the bits of `a` at element offset `lead` of a
    larger allocation (returns the view)."""
    t = torch.zeros(lead + a.size + extra, dtype=torch.int16)
    t[lead:lead + a.size] = torch.from_numpy(a.view(np.int16))
    return t.cuda().view(torch.bfloat16)[lead:lead + a.size]


def dev_f32(a, lead=0):
    t = torch.zeros(lead + a.size, dtype=torch.float32)
    t[lead:] = torch.from_numpy(a)
    return t.cuda()[lead:]


def full_rows(L, rows_win, n_rows):
    """U-long rows holding `rows_win` in this rank's window (zeros elsewhere)."""
    out = []
    for k in range(n_rows):
        r = np.zeros(L.U, np.uint16)
        r[L.shard_begin:L.shard_begin + L.shard_valid] = rows_win[k]
        out.append(r)
    return out


# ---------------------------------------------------------------------------
# small whole-shard cases
# ---------------------------------------------------------------------------

# (name, F, S, U, rank, n_rows, replicas, bf16acc, state_lead): the window start
# r*S and the state alignment pick the path.
CASES = [
    ("vector", 4, 4100, 4 * 4100, 1, 4, 1, False, 0),
    ("vector_tail", 4, 4100, 4 * 4100 - 2, 3, 4, 1, False, 0),
    ("vector_8rows", 8, 2052, 8 * 2052, 5, 8, 1, False, 0),
    ("shifted", 4, 4097, 4 * 4097, 1, 4, 1, False, 0),
    ("shifted_8rows", 8, 2049, 8 * 2049 - 5, 3, 8, 1, False, 0),
    ("scalar_state", 4, 4100, 4 * 4100, 2, 4, 1, False, 1),
    ("runtime_rows_11", 4, 4100, 4 * 4100, 1, 11, 1, False, 0),
    ("hybrid_2x4", 4, 4100, 4 * 4100, 1, 8, 2, False, 0),
    ("hybrid_3x8", 8, 2052, 8 * 2052, 5, 24, 3, False, 0),
    ("bf16acc_8", 8, 2052, 8 * 2052, 2, 8, 1, True, 0),
    ("bf16acc_runtime_5", 4, 4100, 4 * 4100, 1, 5, 1, True, 0),
]


def _oracle_step(rows_full, L, p, m, v, step, replicas, bf16acc, emit):
    gs = 1.0 / len(rows_full)
    with np.errstate(all="ignore"):
        if bf16acc:
            return O.reduce_adamw_shard_bf16acc(rows_full, L, p, m, v, HP, step, gs, emit)
        if replicas > 1:
            return O.reduce_adamw_shard_hybrid(rows_full, L, replicas, p, m, v, HP, step, gs,
                                               emit)
        return O.reduce_adamw_shard(rows_full, L, p, m, v, HP, step, gs, emit)


def _lib_step(lib, u, rows, p, m, v, w, step, replicas, bf16acc):
    hp = lib.AdamWHparams(**HP.__dict__)
    if bf16acc:
        lib.reduce_adamw_shard_bf16acc(u, rows, p, m, v, w, hp, step)
    elif replicas > 1:
        lib.reduce_adamw_shard_hybrid(u, replicas, rows, p, m, v, w, hp, step)
    else:
        lib.reduce_adamw_shard(u, rows, p, m, v, w, hp, step)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("emit", [True, False], ids=["emit", "no_emit"])
def test_fused_special_values(lib, case, emit):
    name, F, S, U, rank, n_rows, replicas, bf16acc, lead = case
    shapes = [(U,)]
    L = O.unit_layout(shapes, F, rank)
    assert L.S == S
    n = L.shard_valid
    u = lib.Unit(shapes, F, rank)
    rows_win = planted_rows(n_rows, n, seed=zlib.crc32(name.encode()) % 1000)
    rows_full = full_rows(L, rows_win, n_rows)
    p0, m0, v0 = planted_state(n, seed=len(name))
    rows_dev = [dev_u16(r) for r in rows_full]
    p, m, v = dev_f32(p0, lead), dev_f32(m0, lead), dev_f32(v0, lead)
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda") if emit else None
    want_p, want_m, want_v = p0, m0, v0
    for step in (1, 2):
        _lib_step(lib, u, rows_dev, p, m, v, w, step, replicas, bf16acc)
        res = _oracle_step(rows_full, L, want_p, want_m, want_v, step, replicas, bf16acc, emit)
        want_p, want_m, want_v = res[:3]
        torch.cuda.synchronize()
        assert_f32_parity(to_np(p), want_p, f"{name} master, step {step}")
        assert_f32_parity(to_np(m), want_m, f"{name} exp_avg, step {step}")
        assert_f32_parity(to_np(v), want_v, f"{name} exp_avg_sq, step {step}")
        if emit:
            assert_bf16_parity(to_np(w), res[3], f"{name} bf16 parameter, step {step}")


@pytest.mark.parametrize("case", [c for c in CASES if c[6] == 1 and not c[7]],
                         ids=[c[0] for c in CASES if c[6] == 1 and not c[7]])
def test_unfused_special_values(lib, case):
    """reduce_shard, then adamw_shard on its fp32 output (a special-laden g)."""
    name, F, S, U, rank, n_rows, replicas, bf16acc, lead = case
    shapes = [(U,)]
    L = O.unit_layout(shapes, F, rank)
    n = L.shard_valid
    u = lib.Unit(shapes, F, rank)
    rows_win = planted_rows(n_rows, n, seed=zlib.crc32(name.encode()) % 1000 + 7)
    rows_full = full_rows(L, rows_win, n_rows)
    p0, m0, v0 = planted_state(n, seed=len(name) + 3)
    rows_dev = [dev_u16(r) for r in rows_full]
    g = torch.empty(n + lead, dtype=torch.float32, device="cuda")[lead:]
    lib.reduce_shard(u, rows_dev, g)
    with np.errstate(all="ignore"):
        want_g = O.reduce_shard(rows_full, L, 1.0 / n_rows)
    torch.cuda.synchronize()
    assert_f32_parity(to_np(g), want_g, f"{name} reduced gradient")
    p, m, v = dev_f32(p0, lead), dev_f32(m0, lead), dev_f32(v0, lead)
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    lib.adamw_shard(u, g, p, m, v, w, lib.AdamWHparams(**HP.__dict__), 3)
    with np.errstate(all="ignore"):
        wp, wm, wv, ww = O.adamw_step(want_g, p0, m0, v0, HP, 3, emit_bf16=True)
    torch.cuda.synchronize()
    assert_f32_parity(to_np(p), wp, f"{name} master")
    assert_f32_parity(to_np(m), wm, f"{name} exp_avg")
    assert_f32_parity(to_np(v), wv, f"{name} exp_avg_sq")
    assert_bf16_parity(to_np(w), ww, f"{name} bf16 parameter")


# ---------------------------------------------------------------------------
# a full-size launch: the one-wave-workgroup shape of long fused launches
# ---------------------------------------------------------------------------

LONG_CASES = [
    # F, S, rank, row stride: 8 rows over the 7B block's shard at F = 8 (the staged
    # compile-time fold in one-wave workgroups, its one-tile kernel); 11 rows and 64 rows,
    # folded in chunks of 8 at run time (for 11 rows the last chunk is partial), with the
    # rows packed S elements apart (windows off 8 bytes: the shifted path) and, for 11
    # rows, on 128-byte lines (the vector path's one-tile kernel, a ragged last tile)
    (8, 25297920, 3, "packed"),
    (11, (1 << 23) + 5, 4, "packed"),
    (11, (1 << 23) + 5, 0, "lines"),
    (64, (1 << 22) + 7, 5, "packed"),
]


@pytest.mark.parametrize("F,S,rank,stride", LONG_CASES,
                         ids=[f"rows{c[0]}_{c[3]}" for c in LONG_CASES])
def test_fused_special_values_long_launch(lib, F, S, rank, stride):
    """F rows over an S-element shard (rank `rank` of F): normal draws in HBM with
    specials planted at 2^17 random positions and in one contiguous run that spans
    several workgroup tiles; those positions and the run are compared with the
    oracle element by element. Row k is the U-element view of one arena that
    starts at element k*Sr (Sr = S, or S rounded up to a multiple of 64), so the
    rank windows of the rows are disjoint (the views overlap outside them, where
    the step reads nothing)."""
    n_rows = F
    shapes = [(F * S,)]
    L = O.unit_layout(shapes, F, rank)
    u = lib.Unit(shapes, F, rank)
    n = L.shard_valid
    rng = np.random.default_rng(11 + F)
    run = np.arange(123456, 123456 + 3000, dtype=np.int64)
    pos = np.unique(np.concatenate([rng.integers(0, n, 1 << 17), run, [0, n - 1]]))
    gseed, mseed = datagen.seed_for(9, 1, 77), datagen.seed_for(9, 0, 77)
    Sr = S if stride == "packed" else -(-S // 64) * 64
    arena = torch.empty((n_rows - 1) * Sr + L.U, dtype=torch.bfloat16, device="cuda")
    rows_dev, rows_at = [], []
    for k in range(n_rows):
        r = arena[k * Sr:k * Sr + L.U]        # window: arena[kSr + begin, kSr + begin + S)
        datagen.fill_bf16_(r[L.shard_begin:L.shard_begin + n], gseed, k, 1e-3,
                           start=L.shard_begin)
        at = datagen.bf16_bits_host(gseed, k, L.shard_begin + pos, 1e-3)
        planted = rng.choice(BF16_SPECIAL, pos.size)
        sel = rng.random(pos.size) < 0.5
        at[sel] = planted[sel]
        idx = torch.from_numpy(L.shard_begin + pos).cuda()
        r.view(torch.int16)[idx] = torch.from_numpy(at.view(np.int16)).cuda()
        rows_dev.append(r)
        rows_at.append(at)
    state, state_at = [], []
    for kind, sigma in ((0, 0.02), (1, 1e-4), (2, 1e-6)):
        t = torch.empty(n, dtype=torch.float32, device="cuda")
        datagen.fill_normal_f32_(t, mseed, kind, sigma)
        if kind == 2:
            t.abs_()
        at = datagen.normal_f32_host(mseed, kind, pos, sigma)
        if kind == 2:
            at = np.abs(at)
        sel = rng.random(pos.size) < 0.3
        at.view(np.uint32)[sel] = rng.choice(F32_SPECIAL, int(sel.sum()))
        t.view(torch.int32)[torch.from_numpy(pos).cuda()] = torch.from_numpy(
            at.view(np.int32)).cuda()
        state.append(t)
        state_at.append(at.astype(np.float32))
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    lib.reduce_adamw_shard(u, rows_dev, *state, w, lib.AdamWHparams(**HP.__dict__), 1)
    one = O.unit_layout([(pos.size,)], 1, 0)
    with np.errstate(all="ignore"):
        wp, wm, wv, ww = O.reduce_adamw_shard(rows_at, one, *state_at, HP, 1,
                                              grad_scale=1.0 / n_rows, emit_bf16=True)
    torch.cuda.synchronize()
    idx = torch.from_numpy(pos).cuda()
    assert_f32_parity(to_np(state[0][idx]), wp, "master")
    assert_f32_parity(to_np(state[1][idx]), wm, "exp_avg")
    assert_f32_parity(to_np(state[2][idx]), wv, "exp_avg_sq")
    assert_bf16_parity(to_np(w[idx]), ww, "bf16 parameter")
    # the planted inputs did produce NaN and infinite results
    assert is_nan32(wp.view(np.uint32)).any() and np.isinf(wv).any()
