"""Seeded synthetic inputs for the FlatParameter shard-step tests and bench.

This module only draws random numbers. It holds none of the arithmetic of the
method under test (no reduction, no optimizer step, no rounding to bf16): the
oracle under ``oracle/`` and the HIP library under
``sharded_flatparameter_flatten_amd/`` both consume what it produces, and
neither imports the other.

Every draw is a pure function of ``(seed, stream, index)``, so any element of
any buffer can be regenerated on the host without generating the rest of it.
That is what lets full-size GPU runs be checked on sampled indices.

Generator (host and device give bit-identical results):

* ``splitmix64(key, i)``: the SplitMix64 output function of Steele, Lea and
  Flood ("Fast splittable pseudorandom number generators", OOPSLA 2014), in
  the form Vigna publishes as ``splitmix64.c``, evaluated at Weyl-sequence
  position ``i + 1`` of a per-(seed, stream) key.
* ``normal_f32``: an Irwin-Hall(4) approximation of N(0, sigma): the four
  16-bit fields of one SplitMix64 word are summed exactly, centred
  (|centred| < 2**18, so the int -> fp32 conversion is exact) and multiplied
  once, in fp32, by ``fp32(sigma / std(IH4))``.
* ``bf16_bits``: the high 16 bits of a ``normal_f32`` draw, i.e. the fp32
  value truncated toward zero to bf16 (a draw, not a rounding step of the
  method), optionally after an fp32 outlier multiply.
* ``outlier_mask``: a second, independent SplitMix64 stream; an element is
  an outlier when the word's top 24 bits are below floor(0.01 * 2**24).

The device twin uses torch int64 tensor ops only (two's-complement wrap on
multiply, logical shifts written as arithmetic shift + mask), so the bench and
the GPU tests can fill multi-GB buffers in HBM without host round trips.
"""

from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# std of the sum of four independent discrete uniforms on {0, ..., 65535}
IH4_CENTRE = 4 * 65535 // 2          # 131070
IH4_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
OUTLIER_THRESHOLD_24 = int(0.01 * (1 << 24))   # 167772
OUTLIER_FACTOR = 1000.0

SEED_BASE = 0xF5D90000
KIND_MASTER, KIND_GRAD, KIND_OUTLIER = 0, 1, 2


def seed_for(config: int, kind: int, step: int = 0) -> int:
    """Seed of one input family: config id, kind (master/grad/outlier), step."""
    return SEED_BASE + 256 * config + 16 * kind + step


# ----------------------------------------------------------------------------
# host (numpy, uint64 arithmetic wraps modulo 2**64 by definition)
# ----------------------------------------------------------------------------

def _mix64_py(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """Key of one (seed, stream) sequence: the mixed pair, as a 64-bit int."""
    return _mix64_py(((seed & 0xFFFFFFFF) << 32) ^ (stream & 0xFFFFFFFF) ^ GAMMA)


def splitmix64_host(key: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
        z = z ^ (z >> np.uint64(31))
    return z


def _scale_f32(sigma: float) -> np.float32:
    return np.float32(sigma / IH4_STD)


def normal_f32_host(seed: int, stream: int, idx, sigma: float) -> np.ndarray:
    z = splitmix64_host(stream_key(seed, stream), idx)
    m16 = np.uint64(0xFFFF)
    s = ((z & m16) + ((z >> np.uint64(16)) & m16)
         + ((z >> np.uint64(32)) & m16) + (z >> np.uint64(48)))
    centred = s.astype(np.int64) - IH4_CENTRE
    return centred.astype(np.float32) * _scale_f32(sigma)


def outlier_mask_host(seed: int, stream: int, idx) -> np.ndarray:
    z = splitmix64_host(stream_key(seed, stream), idx)
    return (z >> np.uint64(40)) < np.uint64(OUTLIER_THRESHOLD_24)


def bf16_bits_host(seed: int, stream: int, idx, sigma: float,
                   outlier_seed: int | None = None) -> np.ndarray:
    """uint16 bit patterns of bf16 draws (fp32 draw truncated to its high half)."""
    x = normal_f32_host(seed, stream, idx, sigma)
    if outlier_seed is not None:
        mask = outlier_mask_host(outlier_seed, stream, idx)
        x = np.where(mask, x * np.float32(OUTLIER_FACTOR), x).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# device twin (torch int64; only used to fill large buffers in HBM)
# ----------------------------------------------------------------------------

def _s64(u: int) -> int:
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _lsr(t, k: int):
    import torch  # noqa: F401  (torch tensor method use only)
    return (t >> k) & ((1 << (64 - k)) - 1)


def _splitmix64_dev(key: int, idx):
    z = idx + 1
    z = z * _s64(GAMMA) + _s64(key)
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


def _normal_f32_dev_chunk(seed, stream, start, n, sigma, device):
    import torch
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    z = _splitmix64_dev(stream_key(seed, stream), idx)
    s = (z & 0xFFFF) + ((z >> 16) & 0xFFFF) + ((z >> 32) & 0xFFFF) + _lsr(z, 48)
    scale = torch.tensor(float(_scale_f32(sigma)), dtype=torch.float32, device=device)
    return (s - IH4_CENTRE).to(torch.float32) * scale


def fill_normal_f32_(out, seed: int, stream: int, sigma: float, start: int = 0,
                     chunk: int = 1 << 24):
    """Fill a 1-D fp32 device tensor with draws for indices [start, start+numel)."""
    n = out.numel()
    for c in range(0, n, chunk):
        m = min(chunk, n - c)
        out[c:c + m].copy_(_normal_f32_dev_chunk(seed, stream, start + c, m, sigma,
                                                 out.device))
    return out


def fill_bf16_(out, seed: int, stream: int, sigma: float, start: int = 0,
               outlier_seed: int | None = None, chunk: int = 1 << 24):
    """Fill a 1-D bf16 device tensor with draws for indices [start, start+numel)."""
    import torch
    n = out.numel()
    bits_view = out.view(torch.int16)
    for c in range(0, n, chunk):
        m = min(chunk, n - c)
        x = _normal_f32_dev_chunk(seed, stream, start + c, m, sigma, out.device)
        if outlier_seed is not None:
            idx = torch.arange(start + c, start + c + m, dtype=torch.int64,
                               device=out.device)
            z = _splitmix64_dev(stream_key(outlier_seed, stream), idx)
            mask = _lsr(z, 40) < OUTLIER_THRESHOLD_24
            big = x * torch.tensor(OUTLIER_FACTOR, dtype=torch.float32, device=out.device)
            x = torch.where(mask, big, x)
        hi = (x.view(torch.int32) >> 16).to(torch.int16)
        bits_view[c:c + m].copy_(hi)
    return out
