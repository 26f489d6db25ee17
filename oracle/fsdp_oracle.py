"""CPU oracle for one rank's share of the sharded FlatParameter lifecycle.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never does, and this module never imports the HIP library: the two
share no code.

Plain, slow, obviously-correct numpy. Every floating-point step is one IEEE-754
binary32 operation (numpy float32 ufuncs are correctly rounded, never fused),
so the order of operations written here *is* the definition the GPU path is
checked against. Integer and bit work is exact.

Pages cited (page title, then section):

* [FSDP-math]  the aicassindra "transformer math" page on FSDP
  (``tm_fsdp_math``);
* [NOTE-003]   "NOTE-003: PyTorch FSDP" (anthology-of-the-sota note);
* [Glossary]   the chipfoundryservices glossary entry
  "fully sharded data parallel fsdp".

The pages name Adam and its fp32 momentum and variance but print no update
rule; the step below follows Kingma & Ba, "Adam" (ICLR 2015), Algorithm 1
(bias-corrected moments, eps added outside the square root) with decoupled
weight decay from Loshchilov & Hutter, "Decoupled Weight Decay
Regularization" (ICLR 2019), Algorithm 2, taking the schedule multiplier to be
the learning rate (decay applied as lr * wd * p).

Parity status of each function (see the pins in tests/test_oracle_pins.py):
``unit_layout``, ``flatten_pad``, ``reduce_shard``, ``adamw_step``,
``bf16_round_nearest_even``, ``unflatten`` (bf16 and fp32 outputs), ``cast_unflatten``,
``reduce_shard_hybrid``, ``reduce_shard_bf16acc``, ``persistent_bytes`` are
pinned. Parity unpinned: the choice of one binary32 op order among the
mathematically equal ones (fixed by this file), and NaN payloads other than the
canonical quiet NaN.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------
# Unit indexer
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class UnitLayout:
    numels: tuple          # element count of each tensor, in unit order
    offsets: tuple         # start of each tensor in the flat buffer (+ U at the end)
    U: int                 # params in the unit
    F: int                 # sharding factor
    rank: int
    S: int                 # shard length = ceil(U / F)
    padded: int            # F * S
    pad: int               # padded - U
    shard_begin: int       # rank * S
    shard_valid: int       # real (non-pad) elements in this rank's shard
    persistent_bytes: int  # 16 * S


def numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def unit_layout(shapes, F: int, rank: int) -> UnitLayout:
    """Offsets, shard length and this rank's window for one FSDP unit.

    [FSDP-math, "The sharding unit: FlatParameter and the wrapping policy"]:
    the unit's parameters are flattened into one 1-D buffer that is split
    evenly over the ranks, each rank keeping one contiguous slice.
    [NOTE-003, "Key results" (table of F)]: F is the number of ranks the
    parameters are sharded over; F = 1 is plain data parallelism.
    Reading: tensors laid end to end in the given order, each row-major; the
    buffer is padded at its end to the next multiple of F; rank r owns
    [r*S, (r+1)*S).
    """
    if F < 1 or not (0 <= rank < F):
        raise ValueError("need F >= 1 and 0 <= rank < F")
    numels = tuple(numel(s) for s in shapes)
    offsets = [0]
    for n in numels:
        offsets.append(offsets[-1] + n)
    U = offsets[-1]
    S = -(-U // F)
    padded = F * S
    begin = rank * S
    valid = max(0, min(S, U - begin))
    return UnitLayout(numels, tuple(offsets), U, F, rank, S, padded, padded - U,
                      begin, valid, persistent_bytes(S))


def persistent_bytes(S: int) -> int:
    """Bytes of state one rank keeps for one unit between steps.

    [FSDP-math, "Why FSDP exists: the redundancy in plain data parallelism"]:
    per parameter a 2-byte low-precision weight, a 2-byte gradient, a 4-byte
    fp32 master copy and two 4-byte Adam moments, 16 bytes in all.
    [FSDP-math, "Per-unit memory and communication, in numbers"]: sharded,
    that budget is paid on 1/N of the parameters. Per unit: 16 * S.
    """
    return (2 + 2 + 4 + 4 + 4) * S


# ----------------------------------------------------------------------------
# bf16 helpers (bit level)
# ----------------------------------------------------------------------------

def bf16_widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: the bf16 bits are the fp32 high half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round_nearest_even(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    [Glossary, "FSDP Implementation (PyTorch)" -> Mixed Precision]: parameters
    are kept in bf16 for compute and communication.
    Definition used: of the two bf16 values that bracket x (drop the low 16
    bits = toward zero; or one bf16 step further from zero), take the nearer;
    on a tie take the one whose last kept bit is 0. A step past the largest
    finite value carries into the exponent and gives infinity. NaN maps to
    the canonical quiet NaN 0x7FC0 (reading; the pages are silent).
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    toward_zero = bits >> np.uint32(16)
    dropped = bits & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    last_kept_odd = (toward_zero & np.uint32(1)) == np.uint32(1)
    away = (dropped > half) | ((dropped == half) & last_kept_odd)
    out = toward_zero + away.astype(np.uint32)
    out = np.where(np.isnan(x), np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------
# flatten / pad
# ----------------------------------------------------------------------------

def flatten_pad(tensors, F: int, begin: int = 0, length: int | None = None) -> np.ndarray:
    """The padded flat buffer of a unit (raw bits), or the window [begin, begin+length).

    [FSDP-math, "The sharding unit: FlatParameter and the wrapping policy"]:
    the unit's tensors become one flat 1-D buffer. Reading: end to end in
    order, then zeros up to F * S (the pad is the value +0.0).
    Works on bit patterns (uint16 for 2-byte, uint32 for 4-byte elements).
    """
    parts = [np.asarray(t).reshape(-1) for t in tensors]
    dtype = parts[0].dtype
    U = sum(p.size for p in parts)
    S = -(-U // F)
    flat = np.zeros(F * S, dtype=dtype)
    pos = 0
    for p in parts:
        flat[pos:pos + p.size] = p
        pos += p.size
    if length is None:
        length = F * S - begin
    if begin < 0 or begin + length > F * S:
        raise ValueError("window outside the padded buffer")
    return flat[begin:begin + length].copy()


# ----------------------------------------------------------------------------
# reduce-scatter arithmetic
# ----------------------------------------------------------------------------

def reduce_shard(grads, layout: UnitLayout, grad_scale: float | None = None) -> np.ndarray:
    """This rank's slice of the sum (scaled to a mean) of the ranks' gradients.

    [FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: the
    collective sums the full gradients over ranks (the data-parallel average)
    and leaves each rank only the slice matching its own parameter slice.
    [Glossary, "FSDP Implementation (PyTorch)" -> Mixed Precision]:
    reductions run in fp32.

    ``grads``: one uint16 bf16 array of length U per contributing rank.
    Reading: each bf16 is widened exactly to fp32; the sum is a left fold in
    rank order starting from rank 0's value; the mean is that sum times
    fp32(grad_scale), grad_scale defaulting to 1/len(grads) computed in
    double. Returns fp32 of length ``shard_valid``.
    """
    n = len(grads)
    if n < 1:
        raise ValueError("need at least one gradient buffer")
    if grad_scale is None:
        grad_scale = 1.0 / n
    gs = np.float32(grad_scale)
    lo = layout.shard_begin
    hi = lo + layout.shard_valid
    acc = bf16_widen(grads[0][lo:hi])
    for k in range(1, n):
        acc = acc + bf16_widen(grads[k][lo:hi])
    return acc * gs


def reduce_shard_bf16acc(grads, layout: UnitLayout, grad_scale: float | None = None) -> np.ndarray:
    """The reduce-scatter arithmetic with bf16 partial sums (reduce dtype bf16).

    [NOTE-003, "Recommendations"] (R3): mixed precision for communication
    volume as much as for memory; [Glossary, "FSDP Implementation (PyTorch)"
    -> Mixed Precision]: the reduce dtype is a choice (fp32 there). Reading of
    a reduce-scatter that keeps its partials in bf16: a left fold in rank
    order where every addition is one binary32 addition of the two bf16
    values followed by rounding the partial to bf16 (nearest even); the final
    bf16 sum is widened and multiplied by fp32(grad_scale). Numerics pinned by
    closed forms and the summation bound with bf16's unit roundoff, not by
    parity with the fp32 reduction.
    """
    n = len(grads)
    if n < 1:
        raise ValueError("need at least one gradient buffer")
    if grad_scale is None:
        grad_scale = 1.0 / n
    gs = np.float32(grad_scale)
    lo = layout.shard_begin
    hi = lo + layout.shard_valid
    partial = np.asarray(grads[0][lo:hi], dtype=np.uint16)
    for k in range(1, n):
        total = bf16_widen(partial) + bf16_widen(grads[k][lo:hi])
        partial = bf16_round_nearest_even(total)
    return bf16_widen(partial) * gs


def reduce_adamw_shard_bf16acc(grads, layout: UnitLayout, p, m, v, hp, step: int,
                               grad_scale: float | None = None, emit_bf16: bool = False):
    """The bf16-partials reduction followed by ``adamw_step`` on its fp32 result."""
    g = reduce_shard_bf16acc(grads, layout, grad_scale)
    return adamw_step(g, p, m, v, hp, step, emit_bf16)


def reduce_shard_hybrid(grads, layout: UnitLayout, replicas: int,
                        grad_scale: float | None = None) -> np.ndarray:
    """Hybrid sharding: this rank's slice of the gradient summed over R groups of F ranks.

    [NOTE-003, "Concepts"]: hybrid sharding shards within a group and
    replicates across groups. [Glossary, "Hybrid Sharding"]: gradients are
    all-reduced across the replica groups (data-parallel style) and sharded
    within a group. Reading: ``grads`` holds R*F rows, replica-major (row
    rho*F + f is rank f of group rho, F = layout.F); each group first sums its
    F rows in rank order (the reduce-scatter inside the group, a left fold
    from rank 0's value), then the R group sums are added in group order (the
    all-reduce across groups, again a left fold), then scaled by
    fp32(grad_scale), default 1/(R*F) computed in double.
    """
    F = layout.F
    if replicas < 1 or len(grads) != replicas * F:
        raise ValueError("need replicas * F gradient rows")
    if grad_scale is None:
        grad_scale = 1.0 / (replicas * F)
    gs = np.float32(grad_scale)
    lo = layout.shard_begin
    hi = lo + layout.shard_valid
    total = None
    for rho in range(replicas):
        group = bf16_widen(grads[rho * F][lo:hi])
        for f in range(1, F):
            group = group + bf16_widen(grads[rho * F + f][lo:hi])
        total = group if total is None else total + group
    return total * gs


def reduce_adamw_shard_hybrid(grads, layout: UnitLayout, replicas: int, p, m, v, hp, step: int,
                              grad_scale: float | None = None, emit_bf16: bool = False):
    """The hybrid reduction followed by ``adamw_step`` on its fp32 result."""
    g = reduce_shard_hybrid(grads, layout, replicas, grad_scale)
    return adamw_step(g, p, m, v, hp, step, emit_bf16)


# ----------------------------------------------------------------------------
# AdamW on the local slice
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_scalars(hp: AdamW, step: int) -> dict:
    """fp32 scalars of step ``step`` (1-based), each computed in double and rounded once."""
    if step < 1:
        raise ValueError("step is 1-based")
    f = np.float32
    return dict(
        b1=f(hp.beta1), omb1=f(1.0 - hp.beta1),
        b2=f(hp.beta2), omb2=f(1.0 - hp.beta2),
        bc1=f(1.0 - hp.beta1 ** step), bc2=f(1.0 - hp.beta2 ** step),
        lr=f(hp.lr), eps=f(hp.eps), wd=f(hp.weight_decay),
    )


def adamw_step(g, p, m, v, hp: AdamW, step: int, emit_bf16: bool = False):
    """One AdamW step on fp32 master ``p`` and moments ``m``, ``v``; returns new arrays.

    [FSDP-math, "The backward cycle: all-gather, grads, reduce-scatter"]: after
    the reduce-scatter the optimizer updates the local slice in place.
    [Glossary, "FSDP Sharding Strategy" -> Optimizer State Sharding]: each rank
    keeps momentum and variance only for its own slice, with no communication.
    [FSDP-math, "Why FSDP exists: ..."]: master, momentum and variance are fp32.

    Steps (Adam, Algorithm 1; decoupled decay, AdamW Algorithm 2), one binary32
    op per line:
        m' = beta1*m + (1-beta1)*g
        v' = beta2*v + (1-beta2)*g*g
        m_hat = m' / (1 - beta1^t)
        v_hat = v' / (1 - beta2^t)
        u  = m_hat / (sqrt(v_hat) + eps)
        p' = p - lr * (u + wd * p)
    ``emit_bf16`` also returns the bf16 bits of p' (the parameter the next
    all-gather ships, [NOTE-003, "Key components"]: mixed precision for
    parameters and communication).
    """
    c = adamw_scalars(hp, step)
    g = np.asarray(g, dtype=np.float32)
    p = np.asarray(p, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)

    first_old = c["b1"] * m
    first_new = c["omb1"] * g
    m_new = first_old + first_new

    g_sq = g * g
    second_old = c["b2"] * v
    second_new = c["omb2"] * g_sq
    v_new = second_old + second_new

    m_hat = m_new / c["bc1"]
    v_hat = v_new / c["bc2"]
    root = np.sqrt(v_hat)
    denom = root + c["eps"]
    u = m_hat / denom

    decay = c["wd"] * p
    direction = u + decay
    delta = c["lr"] * direction
    p_new = p - delta

    out = (p_new, m_new, v_new)
    if emit_bf16:
        out = out + (bf16_round_nearest_even(p_new),)
    return out


def reduce_adamw_shard(grads, layout: UnitLayout, p, m, v, hp: AdamW, step: int,
                       grad_scale: float | None = None, emit_bf16: bool = False):
    """The fused step: ``reduce_shard`` then ``adamw_step`` on its fp32 result."""
    g = reduce_shard(grads, layout, grad_scale)
    return adamw_step(g, p, m, v, hp, step, emit_bf16)


# ----------------------------------------------------------------------------
# all-gather arithmetic + unflatten
# ----------------------------------------------------------------------------

def unflatten(shards, layout: UnitLayout, shapes, out: str = "bf16"):
    """Per-tensor outputs from the F rank shards of a unit.

    [FSDP-math, "The forward cycle: all-gather, compute, reshard"]: every rank
    contributes its slice and each ends with the unit's full weights, which
    the module then uses as ordinary per-tensor parameters.
    [Glossary, "Debugging FSDP" -> Checkpoint/Resume]: a full state dict
    gathers the sharded state back into whole tensors (here in fp32 for the
    master weights and the Adam moments).

    ``shards``: F arrays of S elements each (fp32 values, or uint16 bf16
    bits). Global element g of the unit lives in shard g // S at position
    g % S; pad slots are never read. ``out``: "bf16" (fp32 sources rounded to
    nearest even, bf16 sources copied bit for bit) or "f32" (fp32 sources
    copied bit for bit, bf16 sources widened exactly).
    Returns a list of arrays shaped like ``shapes`` (uint16 bits or float32).
    """
    S = layout.S
    outs = []
    for i, shape in enumerate(shapes):
        off = layout.offsets[i]
        g = np.arange(off, off + layout.numels[i], dtype=np.int64)
        k = g // S
        local = g - k * S
        src_dtype = np.asarray(shards[0]).dtype
        vals = np.empty(g.size, dtype=src_dtype)
        for shard_id in np.unique(k):
            sel = k == shard_id
            vals[sel] = np.asarray(shards[int(shard_id)])[local[sel]]
        if src_dtype not in (np.float32, np.uint16):
            raise TypeError("shards must be float32 values or uint16 bf16 bits")
        if out == "bf16":
            res = bf16_round_nearest_even(vals) if src_dtype == np.float32 else vals
        elif out == "f32":
            res = vals if src_dtype == np.float32 else bf16_widen(vals)
        else:
            raise ValueError("out must be 'bf16' or 'f32'")
        outs.append(res.reshape(tuple(shape)))
    return outs


def cast_unflatten(shards, layout: UnitLayout, shapes):
    """The all-gather arithmetic: ``unflatten`` into bf16 parameters."""
    return unflatten(shards, layout, shapes, out="bf16")
