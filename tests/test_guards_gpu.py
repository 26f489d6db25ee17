"""Guard sentinels around every output window, for every entry point and path.

[FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: a rank
updates only its own slice. The library's contract is that a call writes
exactly its output windows: no byte before or after them, and (for the step
kernels) no shard position at or past shard_valid. Each test allocates every
output inside a larger buffer whose other elements hold a NaN pattern that no
kernel produces (fp32 0x7FC00001, bf16 0x7FC1), passes the window as the
output, and checks that the guards are unchanged bit for bit and that the
window itself was written.

Covered: flatten_pad (fp32 and bf16 windows, aligned and odd offsets, the
zero-pad segment), reduce_shard, adamw_shard, the fused step (vector, shifted
and scalar paths, a ragged tail, the one-wave-workgroup shape of long
launches), the batched many-unit step, hybrid sharding, bf16 partial sums, and
cast_unflatten / unflatten into views packed in one buffer with guards between
the tensors.
"""

import numpy as np
import pytest
import torch

from conftest import gpu_available
from shard_cases import HP, FP32_SENTINEL, BF16_SENTINEL
from oracle import fsdp_oracle as O
import datagen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

G = 96       # guard elements on each side of a window


class Guarded:
    """A window of n elements at element offset `lead` of a buffer of
    lead + n + tail elements; everything outside the window holds the sentinel."""

    def __init__(self, n, dtype, lead=G, tail=G, fill_window=True):
        self.n, self.lead, self.tail, self.dtype = n, lead, tail, dtype
        if dtype == torch.float32:
            self.buf = torch.full((lead + n + tail,), FP32_SENTINEL, dtype=torch.int32,
                                  device="cuda").view(torch.float32)
            self.bits = self.buf.view(torch.int32)
            self.sentinel = FP32_SENTINEL
        else:
            self.buf = torch.full((lead + n + tail,), BF16_SENTINEL, dtype=torch.int16,
                                  device="cuda").view(torch.bfloat16)
            self.bits = self.buf.view(torch.int16)
            self.sentinel = BF16_SENTINEL
        self.win = self.buf[lead:lead + n]

    def check(self, what, written=True):
        torch.cuda.synchronize()
        b = self.bits.cpu().numpy()
        before, after = b[:self.lead], b[self.lead + self.n:]
        assert (before == self.sentinel).all(), \
            f"{what}: {int((before != self.sentinel).sum())} guard elements before the window changed"
        assert (after == self.sentinel).all(), \
            f"{what}: {int((after != self.sentinel).sum())} guard elements after the window changed"
        if written:
            w = b[self.lead:self.lead + self.n]
            assert not (w == self.sentinel).any(), \
                f"{what}: {int((w == self.sentinel).sum())} window elements were not written"


def hp(lib):
    return lib.AdamWHparams(**HP.__dict__)


def rows_for(u, n_rows, seed=5):
    rows = []
    for k in range(n_rows):
        r = torch.zeros(u.U, dtype=torch.bfloat16, device="cuda")
        datagen.fill_bf16_(r[u.shard_begin:u.shard_begin + u.shard_valid], seed, k, 1e-3,
                           start=u.shard_begin)
        rows.append(r)
    return rows


def state_for(n, lead=G):
    """Guarded master (normal draws), m and v (zeros) windows of n fp32 elements."""
    p, m, v = (Guarded(n, torch.float32, lead=lead) for _ in range(3))
    datagen.fill_normal_f32_(p.win, 3, 0, 0.02)
    m.win.zero_()
    v.win.zero_()
    return p, m, v


# unit shapes picking the paths: (name, shapes, F, rank, state lead)
STEP_CASES = [
    ("vector", [(4 * 4100,)], 4, 1, G),
    ("vector_tail", [(4 * 4100 - 2,)], 4, 3, G),
    ("pad_rank", [(5,)], 8, 4, G),                        # the last rank with data
    ("empty_rank", [(5,)], 8, 6, G),                      # a rank holding only pad
    ("shifted", [(4 * 4097,)], 4, 1, G),
    ("scalar_state", [(4 * 4100,)], 4, 2, G + 1),
    ("tiny_unit", [(256, 1024), (1024,), (1024, 256), (256,)], 4, 1, G),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
@pytest.mark.parametrize("n_rows", [4, 11])
def test_fused_step_guards(lib, case, n_rows):
    name, shapes, F, rank, lead = case
    u = lib.Unit(shapes, F, rank)
    n = u.shard_valid
    rows = rows_for(u, n_rows)
    p, m, v = state_for(n, lead)
    w = Guarded(n, torch.bfloat16, lead=lead)
    lib.reduce_adamw_shard(u, rows, p.win, m.win, v.win, w.win, hp(lib), 1)
    for t, nm in ((p, "master"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "bf16 parameter")):
        t.check(f"{name} {nm}")


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_reduce_and_adamw_guards(lib, case):
    name, shapes, F, rank, lead = case
    u = lib.Unit(shapes, F, rank)
    n = u.shard_valid
    rows = rows_for(u, F)
    g = Guarded(n, torch.float32, lead=lead)
    lib.reduce_shard(u, rows, g.win)
    g.check(f"{name} reduce out")
    p, m, v = state_for(n, lead)
    w = Guarded(n, torch.bfloat16, lead=lead)
    lib.adamw_shard(u, g.win, p.win, m.win, v.win, w.win, hp(lib), 1)
    for t, nm in ((p, "master"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "bf16 parameter")):
        t.check(f"{name} adamw {nm}")


@pytest.mark.parametrize("kind", ["hybrid_2x4", "hybrid_3x8", "bf16acc_8", "bf16acc_6"])
def test_grouped_fold_guards(lib, kind):
    F, R = (8, 3) if kind == "hybrid_3x8" else (4, 2)
    u = lib.Unit([(F * 4100 - 2,)], F, F - 1)
    n = u.shard_valid
    rows = rows_for(u, {"hybrid_2x4": 8, "hybrid_3x8": 24, "bf16acc_8": 8, "bf16acc_6": 6}[kind])
    p, m, v = state_for(n)
    w = Guarded(n, torch.bfloat16)
    if kind.startswith("hybrid"):
        lib.reduce_adamw_shard_hybrid(u, R, rows, p.win, m.win, v.win, w.win, hp(lib), 1)
        g = Guarded(n, torch.float32)
        lib.reduce_shard_hybrid(u, R, rows, g.win)
    else:
        lib.reduce_adamw_shard_bf16acc(u, rows, p.win, m.win, v.win, w.win, hp(lib), 1)
        g = Guarded(n, torch.float32)
        lib.reduce_shard_bf16acc(u, rows, g.win)
    for t, nm in ((p, "master"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "bf16 parameter"),
                  (g, "reduce out")):
        t.check(f"{kind} {nm}")


LONG_GUARD_CASES = [
    # name, F, S, rank, row stride: 8 rows over 2^24 + 3 elements (a ragged last tile) in
    # one-wave workgroups, with every row's window on a 128-byte line (rank 0, rows a
    # multiple of 64 elements apart: the one-tile kernel of the staged step) and at a
    # 6-byte offset (rank 1: the shifted-row path); 11 rows folded in chunks of 8 at run
    # time over 2^23 + 5 elements (ending in a partial chunk), with the rows on lines and
    # packed S elements apart (windows 2 bytes off: the shifted path); 64 rows over
    # 2^22 + 7 elements
    ("vector_rows", 8, (1 << 24) + 3, 0, "lines"),
    ("shifted_rows", 8, (1 << 24) + 3, 1, "lines"),
    ("chunked_rows11", 11, (1 << 23) + 5, 0, "lines"),
    ("chunked_rows11_packed", 11, (1 << 23) + 5, 0, "packed"),
    ("chunked_rows64", 64, (1 << 22) + 7, 0, "lines"),
    ("chunked_rows64_packed", 64, (1 << 22) + 7, 0, "packed"),
]


@pytest.mark.parametrize("name,F,S,rank,stride", LONG_GUARD_CASES,
                         ids=[c[0] for c in LONG_GUARD_CASES])
def test_long_launch_guards(lib, name, F, S, rank, stride):
    """Long launches, fused and reduce: the guards around the windows and the
    elements at both ends. Row k is the U-element view of one arena that starts at
    element k*Sr (disjoint rank windows), Sr = S ("packed") or S rounded up to a
    multiple of 64 ("lines")."""
    u = lib.Unit([(F * S,)], F, rank)
    n = u.shard_valid
    Sr = S if stride == "packed" else -(-S // 64) * 64
    arena = torch.zeros((F - 1) * Sr + u.U, dtype=torch.bfloat16, device="cuda")
    rows = []
    for k in range(F):
        r = arena[k * Sr:k * Sr + u.U]
        datagen.fill_bf16_(r[u.shard_begin:u.shard_begin + n], 5, k, 1e-3, start=u.shard_begin)
        rows.append(r)
    starts = [r.data_ptr() + 2 * u.shard_begin for r in rows]
    assert n == S
    if name == "shifted_rows" or stride == "packed":
        assert any(a % 8 for a in starts)             # the shifted-row path
    else:
        assert all(a % 128 == 0 for a in starts)      # the vector path, tiles in plain order
    p, m, v = state_for(n)                              # windows 384 bytes in: on a line
    w = Guarded(n, torch.bfloat16, lead=128)            # 256 bytes in: on a line
    lib.reduce_adamw_shard(u, rows, p.win, m.win, v.win, w.win, hp(lib), 1)
    out = Guarded(n, torch.float32)
    lib.reduce_shard(u, rows, out.win)
    torch.cuda.synchronize()
    for t, nm in ((p, "master"), (m, "exp_avg"), (v, "exp_avg_sq"), (w, "bf16 parameter"),
                  (out, "reduce out")):
        b = t.bits
        assert (b[:t.lead].cpu().numpy() == t.sentinel).all(), f"{nm}: guard before"
        assert (b[t.lead + n:].cpu().numpy() == t.sentinel).all(), f"{nm}: guard after"
        ends = torch.cat([b[t.lead:t.lead + 4096], b[t.lead + n - 4096:t.lead + n]])
        assert not (ends.cpu().numpy() == t.sentinel).any(), f"{nm}: window ends not written"


def test_batched_units_guards(lib):
    """fsdp_reduce_adamw_units over units whose state windows share one slab, with
    guards between the windows (the batched kernel for the aligned ones, the
    single-unit kernels for a misaligned one)."""
    shapes = [[(4096, 33)], [(1000, 7)], [(131072,)], [(5, 3)], [(64, 64), (64,)]]
    F = 4
    units = [lib.Unit(s, F, 1) for s in shapes]
    starts, pos = [], G
    for i, u in enumerate(units):
        if i == 3:
            pos += 1                      # a window that is not 16-byte aligned
        starts.append(pos)
        pos += u.shard_valid + G
        pos = (pos + 3) // 4 * 4
    total = pos
    slabs = {}
    for name, dt, sent in (("p", torch.int32, FP32_SENTINEL), ("m", torch.int32, FP32_SENTINEL),
                           ("v", torch.int32, FP32_SENTINEL), ("w", torch.int16, BF16_SENTINEL)):
        slabs[name] = torch.full((total,), sent, dtype=dt, device="cuda")
    wins = []
    for u, a in zip(units, starts):
        n = u.shard_valid
        p = slabs["p"].view(torch.float32)[a:a + n]
        datagen.fill_normal_f32_(p, 3, a, 0.02)
        m = slabs["m"].view(torch.float32)[a:a + n]
        v = slabs["v"].view(torch.float32)[a:a + n]
        m.zero_()
        v.zero_()
        w = slabs["w"].view(torch.bfloat16)[a:a + n]
        wins.append((u, rows_for(u, F, seed=a), p, m, v, w))
    lib.reduce_adamw_units(wins, hp(lib), 1)
    torch.cuda.synchronize()
    inside = np.zeros(total, bool)
    for u, a in zip(units, starts):
        inside[a:a + u.shard_valid] = True
    for name, sent in (("p", FP32_SENTINEL), ("m", FP32_SENTINEL), ("v", FP32_SENTINEL),
                       ("w", BF16_SENTINEL)):
        b = slabs[name].cpu().numpy()
        assert (b[~inside] == sent).all(), f"{name}: {int((b[~inside] != sent).sum())} guards changed"
        assert not (b[inside] == sent).any(), f"{name}: window elements not written"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("window", ["shard", "odd_begin", "into_pad"])
def test_flatten_pad_guards(lib, dtype, window):
    shapes = [(256, 1024), (1024,), (1024, 256), (255,)]
    F = 4
    u = lib.Unit(shapes, F, 1)
    ts = [torch.randn(int(np.prod(s)), device="cuda").to(dtype) for s in shapes]
    if window == "shard":
        begin, length = u.shard_begin, u.S
    elif window == "odd_begin":
        begin, length = 1001, 70001
    else:
        begin, length = u.padded - 3000, 3000       # ends in the zero pad
    d = Guarded(length, dtype, lead=G + (1 if window == "odd_begin" else 0))
    lib.flatten_pad(u, ts, d.win, begin=begin, length=length)
    d.check(f"flatten_pad {window}")
    if window == "into_pad":
        tail = d.win[-u.pad:].float().cpu().numpy()
        assert u.pad > 0 and (tail == 0).all() and not np.signbit(tail).any()


@pytest.mark.parametrize("src", [torch.float32, torch.bfloat16], ids=["from_f32", "from_bf16"])
@pytest.mark.parametrize("dst", [torch.float32, torch.bfloat16], ids=["to_f32", "to_bf16"])
def test_unflatten_guards_between_packed_views(lib, src, dst):
    """Outputs are views into one buffer with G sentinel elements before, between
    and after them; one of them starts at an odd element offset."""
    shapes = [(256, 1024), (1024,), (1024, 256), (255,)]
    F = 4
    u = lib.Unit(shapes, F, 0)
    shards = [torch.randn(u.S, device="cuda").to(src) for _ in range(F)]
    numels = [int(np.prod(s)) for s in shapes]
    offs, pos = [], G
    for i, nel in enumerate(numels):
        if i == 2:
            pos += 1
        offs.append(pos)
        pos += nel + G
    total = pos
    sent = FP32_SENTINEL if dst == torch.float32 else BF16_SENTINEL
    idt = torch.int32 if dst == torch.float32 else torch.int16
    buf = torch.full((total,), sent, dtype=idt, device="cuda")
    outs = [buf.view(dst)[a:a + nel].view(s) for a, nel, s in zip(offs, numels, shapes)]
    if dst == torch.bfloat16:
        lib.cast_unflatten(u, shards, outs)
    else:
        lib.unflatten(u, shards, outs)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    inside = np.zeros(total, bool)
    for a, nel in zip(offs, numels):
        inside[a:a + nel] = True
    assert (b[~inside] == sent).all(), f"{int((b[~inside] != sent).sum())} guards changed"
    assert not (b[inside] == sent).any()
