"""Test cases for the GPU parity tests: device inputs and oracle expectations.

Inputs come from ``datagen`` (the host generator for the oracle, its device
twin to fill HBM). Expected values come only from ``oracle``, evaluated on
host-generated inputs, either on whole (small) units or on sampled indices of
full-size units: every step of the path is elementwise in the shard index, so
a sampled index's whole multi-step trajectory can be recomputed on its own.
The every-element checks of full-size units feed the oracle host copies of the
device twin's fills instead (regenerating billions of values on the host takes
minutes), after spot-checking those fills against the host generator.
"""

from __future__ import annotations

import os

import numpy as np
import torch

import datagen
from datagen import workloads as W
from oracle import fsdp_oracle as O

FP32_SENTINEL = 0x7FC00001      # a NaN bit pattern no kernel produces
BF16_SENTINEL = 0x7FC1

HP = O.AdamW(**W.ADAMW)


class Case:
    """One rank's shard of one unit: shapes, F, rank, contributions, seeds.

    ``replicas`` > 1 is hybrid sharding: replicas*F rows, replica-major."""

    def __init__(self, shapes, F, rank, n_grads=None, config=0, outliers=False,
                 grad_sigma=W.GRAD_SIGMA, master_sigma=W.MASTER_SIGMA, replicas=1,
                 bf16acc=False):
        self.shapes = [tuple(s) for s in shapes]
        self.F, self.rank = F, rank
        self.replicas = replicas
        self.bf16acc = bf16acc
        self.n_grads = F * replicas if n_grads is None else n_grads
        self.L = O.unit_layout(self.shapes, F, rank)
        self.config = config
        self.outliers = outliers
        self.grad_sigma, self.master_sigma = grad_sigma, master_sigma
        self.master_seed = datagen.seed_for(config, datagen.KIND_MASTER)

    def grad_seed(self, step):
        return datagen.seed_for(self.config, datagen.KIND_GRAD, step)

    def outlier_seed(self, step):
        return datagen.seed_for(self.config, datagen.KIND_OUTLIER, step) if self.outliers else None

    # ---------------- host inputs -------------------------------------------
    def host_master_tensors(self):
        return [datagen.normal_f32_host(self.master_seed, i, np.arange(n), self.master_sigma)
                for i, n in enumerate(self.L.numels)]

    def host_grads(self, step):
        idx = np.arange(self.L.U)
        return [datagen.bf16_bits_host(self.grad_seed(step), k, idx, self.grad_sigma,
                                       self.outlier_seed(step)) for k in range(self.n_grads)]

    def host_master_at(self, g):
        """Generated master values at flat indices g (tensor lookup by offsets)."""
        offs = np.asarray(self.L.offsets, dtype=np.int64)
        tid = np.searchsorted(offs, g, side="right") - 1
        out = np.empty(g.size, np.float32)
        for i in np.unique(tid):
            sel = tid == i
            out[sel] = datagen.normal_f32_host(self.master_seed, int(i), g[sel] - offs[i],
                                               self.master_sigma)
        return out

    def host_grads_at(self, step, g):
        return [datagen.bf16_bits_host(self.grad_seed(step), k, g, self.grad_sigma,
                                       self.outlier_seed(step)) for k in range(self.n_grads)]

    # ---------------- device inputs -----------------------------------------
    def device_master_tensors(self, device="cuda"):
        ts = []
        for i, n in enumerate(self.L.numels):
            t = torch.empty(n, dtype=torch.float32, device=device)
            datagen.fill_normal_f32_(t, self.master_seed, i, self.master_sigma)
            ts.append(t)
        return ts

    def device_grads(self, step, device="cuda", out=None):
        out = out or [torch.empty(self.L.U, dtype=torch.bfloat16, device=device)
                      for _ in range(self.n_grads)]
        for k in range(self.n_grads):
            datagen.fill_bf16_(out[k], self.grad_seed(step), k, self.grad_sigma,
                               outlier_seed=self.outlier_seed(step))
        return out

    # ---------------- oracle expectations -----------------------------------
    def oracle_full(self, steps, emit=True):
        """Whole-shard oracle trajectory: list of (p, m, v, w) after each step."""
        L = self.L
        lo, hi = L.shard_begin, L.shard_begin + L.shard_valid
        flat = O.flatten_pad([t.view(np.uint32) for t in self.host_master_tensors()], self.F)
        p = flat.view(np.float32)[lo:hi].copy()
        m = np.zeros_like(p)
        v = np.zeros_like(p)
        out = []
        for t in range(1, steps + 1):
            res = self._step(self.host_grads(t), L, p, m, v, t, emit)
            p, m, v = res[:3]
            out.append(res)
        return out

    def _step(self, rows, L, p, m, v, t, emit):
        if self.bf16acc:
            return O.reduce_adamw_shard_bf16acc(rows, L, p, m, v, HP, t,
                                                grad_scale=1.0 / self.n_grads, emit_bf16=emit)
        if self.replicas > 1:
            return O.reduce_adamw_shard_hybrid(rows, L, self.replicas, p, m, v, HP, t,
                                               grad_scale=1.0 / self.n_grads, emit_bf16=emit)
        return O.reduce_adamw_shard(rows, L, p, m, v, HP, t, grad_scale=1.0 / self.n_grads,
                                    emit_bf16=emit)

    def oracle_sampled(self, loc, steps, emit=True):
        """Oracle trajectory at local shard indices ``loc`` only."""
        g = self.L.shard_begin + np.asarray(loc, dtype=np.int64)
        # a layout of the sampled elements only: F kept (the hybrid groups rows by F),
        # rank 0 of a unit whose shard is exactly the sample
        one = O.unit_layout([(g.size * self.F,)], self.F, 0)
        p = self.host_master_at(g)
        m = np.zeros_like(p)
        v = np.zeros_like(p)
        out = []
        for t in range(1, steps + 1):
            rows = [np.concatenate([r, np.zeros(g.size * (self.F - 1), np.uint16)])
                    for r in self.host_grads_at(t, g)]
            res = self._step(rows, one, p, m, v, t, emit)
            p, m, v = res[:3]
            out.append(res)
        return out

    def sample_indices(self, n=1 << 16, seed=0):
        """Random local indices plus both ends and every tensor boundary in the window."""
        valid = self.L.shard_valid
        if valid <= n:
            return np.arange(valid, dtype=np.int64)
        rng = np.random.default_rng(seed)
        pts = [rng.integers(0, valid, n), np.arange(16), valid - 1 - np.arange(16)]
        for off in self.L.offsets:
            rel = off - self.L.shard_begin
            pts.append(np.arange(rel - 9, rel + 9))
        s = np.unique(np.concatenate(pts))
        return s[(s >= 0) & (s < valid)].astype(np.int64)


# ---------------- comparison helpers -------------------------------------------

def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    return to_np(t[torch.from_numpy(idx).to(t.device)])


# FSDP_STRICT_BITS=1 turns the tolerance checks below into bit equality (the
# design target), to confirm that every compared element is bit-equal.
STRICT = os.environ.get("FSDP_STRICT_BITS", "0") == "1"


def assert_rel(got, want, tol=1e-6, what=""):
    """Element-wise relative error <= tol (exact where the expected value is 0)."""
    if STRICT:
        tol = 0.0
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, what
    same = got.view(np.uint32) == want.view(np.uint32)
    g64, w64 = got.astype(np.float64), want.astype(np.float64)
    err = np.abs(g64 - w64)
    ok = same if STRICT else same | (err <= tol * np.abs(w64))
    if not ok.all():
        bad = np.flatnonzero(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements beyond rel {tol}; first "
                             f"at {bad.tolist()}: got {got[bad].tolist()} want {want[bad].tolist()}")
    return float(same.mean())


def bf16_ordinal(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_bf16_ulp(got, want, ulps=1, what=""):
    if STRICT:
        ulps = 0
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    d = np.abs(bf16_ordinal(got) - bf16_ordinal(want))
    if not (d <= ulps).all():
        bad = np.flatnonzero(d > ulps)[:5]
        raise AssertionError(f"{what}: {int((d > ulps).sum())} bf16 values beyond {ulps} ulp; "
                             f"first at {bad.tolist()}")
    return float((got == want).mean())


def assert_bits(got, want, what=""):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, what
    neq = got != want
    if neq.any():
        bad = np.flatnonzero(neq)[:5]
        raise AssertionError(f"{what}: {int(neq.sum())} elements differ; first at {bad.tolist()}")


class ModelShard:
    """One rank's persistent shard of a whole model: every unit's fp32 master,
    exp_avg, exp_avg_sq, bf16 parameter and bf16 gradient slot, carved from
    one slab per kind (unit u at the prefix sum of the shard lengths).

    Inputs: unit u's master comes from tensor streams 256*u + i; all block
    units share one generated set of gradient rows (streams k) and the root
    unit has its own (streams 100 + k). Both sides regenerate any element.
    """

    def __init__(self, units, F, rank, config, device="cuda"):
        self.units = units
        self.F, self.rank, self.config = F, rank, config
        self.L = [O.unit_layout(W.shapes(u), F, rank) for u in units]
        self.starts = np.concatenate([[0], np.cumsum([L.S for L in self.L])]).astype(np.int64)
        total = int(self.starts[-1])
        self.total = total
        self.master_seed = datagen.seed_for(config, datagen.KIND_MASTER)
        self.grad_seed = datagen.seed_for(config, datagen.KIND_GRAD, 1)
        self.p = torch.empty(total, dtype=torch.float32, device=device)
        self.m = torch.zeros(total, dtype=torch.float32, device=device)
        self.v = torch.zeros(total, dtype=torch.float32, device=device)
        self.w = torch.empty(total, dtype=torch.bfloat16, device=device)
        self.gslot = torch.zeros(total, dtype=torch.bfloat16, device=device)
        for u, L in enumerate(self.L):
            self._fill_master(u, L)
        ublk = max(L.U for L, unit in zip(self.L, units) if unit is not units[-1])
        self.block_grads = [torch.empty(ublk, dtype=torch.bfloat16, device=device)
                            for _ in range(F)]
        for k in range(F):
            datagen.fill_bf16_(self.block_grads[k], self.grad_seed, k, W.GRAD_SIGMA)
        self.root_grads = [torch.empty(self.L[-1].U, dtype=torch.bfloat16, device=device)
                           for _ in range(F)]
        for k in range(F):
            datagen.fill_bf16_(self.root_grads[k], self.grad_seed, 100 + k, W.GRAD_SIGMA)

    def _fill_master(self, u, L):
        lo, hi = L.shard_begin, L.shard_begin + L.shard_valid
        base = int(self.starts[u])
        for i in range(len(L.numels)):
            a, b = max(lo, L.offsets[i]), min(hi, L.offsets[i + 1])
            if a >= b:
                continue
            dst = self.p[base + a - lo: base + b - lo]
            datagen.fill_normal_f32_(dst, self.master_seed, 256 * u + i, W.MASTER_SIGMA,
                                     start=a - L.offsets[i])

    def window(self, t, u):
        b = int(self.starts[u])
        return t[b:b + self.L[u].S]

    def grads(self, u):
        return self.root_grads if u == len(self.L) - 1 else self.block_grads

    def persistent_bytes(self):
        return sum(t.numel() * t.element_size() for t in (self.p, self.m, self.v, self.w,
                                                          self.gslot))

    def inputs_at(self, u, loc):
        """Unit u's master and gradient-row values at local shard indices loc,
        regenerated on the host: (master fp32, [bf16 bits of row k])."""
        L = self.L[u]
        g = L.shard_begin + np.asarray(loc, dtype=np.int64)
        offs = np.asarray(L.offsets, dtype=np.int64)
        tid = np.searchsorted(offs, g, side="right") - 1
        p = np.empty(g.size, np.float32)
        for i in np.unique(tid):
            sel = tid == i
            p[sel] = datagen.normal_f32_host(self.master_seed, 256 * u + int(i), g[sel] - offs[i],
                                             W.MASTER_SIGMA)
        base = 100 if u == len(self.L) - 1 else 0
        rows = [datagen.bf16_bits_host(self.grad_seed, base + k, g, W.GRAD_SIGMA)
                for k in range(self.F)]
        return p, rows

    def oracle_sampled(self, u, loc):
        """Oracle's first step of unit u at local shard indices loc."""
        p, rows = self.inputs_at(u, loc)
        g = np.asarray(loc, dtype=np.int64)
        z = np.zeros_like(p)
        one = O.unit_layout([(g.size,)], 1, 0)
        return O.reduce_adamw_shard(rows, one, p, z, z, HP, 1, grad_scale=1.0 / self.F,
                                    emit_bf16=True)

    def sample(self, u, n, seed):
        L = self.L[u]
        rng = np.random.default_rng(seed)
        pts = [rng.integers(0, L.shard_valid, n), np.arange(8), L.shard_valid - 1 - np.arange(8)]
        for off in L.offsets:
            rel = off - L.shard_begin
            pts.append(np.arange(rel - 5, rel + 5))
        s = np.unique(np.concatenate(pts))
        return s[(s >= 0) & (s < L.shard_valid)].astype(np.int64)
