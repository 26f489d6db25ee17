"""Device binary32 square root and division against the host's IEEE-754 results.

The AdamW update computes two divisions by the bias corrections, one square
root and one division by the denominator per element, each required to be a
correctly rounded binary32 operation (the same op sequence as the oracle). A
1-ulp error there rarely reaches the updated parameter (lr * u is small next
to p), so the end-to-end parity tests pin these operations only weakly. Here
the two operations, compiled by the same compiler with the library's flags
(tests/probes/fp32_ops_probe.hip; the library's gfx950 code uses the same
instruction sequences), are compared bit for bit with x86 SSE results
(numpy's float32 sqrt and division, correctly rounded by IEEE 754):
* square root over all 2^32 input bit patterns;
* division over random bit-pattern pairs (every exponent range, subnormals,
  infinities, NaNs), operands in the AdamW update's ranges, and an edge-case
  cross product.
NaN results compare as NaN (payloads are not pinned).
"""

import ctypes
import importlib.util
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

_spec = importlib.util.spec_from_file_location(
    "fsdp_fp32_probe_build",
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "build.py"))
probe_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(probe_build)

CHUNK = 1 << 28


@pytest.fixture(scope="module")
def probe():
    path = probe_build.path()
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.probe_sqrt_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.probe_sqrt_range.restype = ctypes.c_int
    lib.probe_div.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
    lib.probe_div.restype = ctypes.c_int
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _mismatch(got, want):
    same = got.view(np.uint32) == want.view(np.uint32)
    return ~(same | (np.isnan(got) & np.isnan(want)))


def test_sqrt_every_fp32_bit_pattern(probe):
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    bad, first = 0, None
    for base in range(0, 1 << 32, CHUNK):
        assert probe.probe_sqrt_range(base, CHUNK, ctypes.c_void_p(out.data_ptr()), _stream()) == 0
        got = out.cpu().numpy()
        x = np.arange(base, base + CHUNK, dtype=np.uint64).astype(np.uint32).view(np.float32)
        with np.errstate(invalid="ignore"):
            want = np.sqrt(x)
        bad_here = _mismatch(got, want)
        n = int(np.count_nonzero(bad_here))
        if n and first is None:
            i = int(np.flatnonzero(bad_here)[0])
            first = (hex(base + i), got[i], want[i])
        bad += n
        del got, x, want, bad_here
    assert bad == 0, f"{bad} sqrt results differ; first input {first}"


def _edge_values():
    f = np.float32
    fi = np.finfo(np.float32)
    bits = [0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x00400000,
            0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000, 0x3F800001,
            0x3F7FFFFF, 0x40000000, 0x3F000000, 0x40400000, 0x3EAAAAAB, 0x33D6BF95,
            0x322BCC77, 0x38D1B717, 0x3DCCCCCD, 0x3A83126F, 0x1E3CE508, 0x60AD78EC,
            0x0CAC5E40, 0x72F71C41, 0x7E967699, 0x01000000]
    v = np.array(bits, dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, -v, np.array([fi.tiny, fi.max, fi.eps, 1 / f(3), f(0.999)],
                                        dtype=np.float32)])
    return v.astype(np.float32)


def _run_div(probe, a, b):
    da = torch.from_numpy(a).cuda()
    db = torch.from_numpy(b).cuda()
    out = torch.empty_like(da)
    assert probe.probe_div(ctypes.c_void_p(da.data_ptr()), ctypes.c_void_p(db.data_ptr()),
                           ctypes.c_void_p(out.data_ptr()), a.size, _stream()) == 0
    got = out.cpu().numpy()
    with np.errstate(all="ignore"):
        want = a / b
    bad = _mismatch(got, want)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{int(bad.sum())} quotients differ; first "
                             f"{a[i]!r}/{b[i]!r}: got {got[i]!r} want {want[i]!r}")


def test_div_random_bit_patterns(probe):
    rng = np.random.default_rng(2024)
    n = 1 << 26
    a = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    b = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    _run_div(probe, a, b)


def test_div_same_binade_and_adamw_ranges(probe):
    """Quotients near 1 (hard rounding cases) and the update's operand ranges:
    moments over bias corrections, and m_hat over sqrt(v_hat) + eps."""
    rng = np.random.default_rng(7)
    n = 1 << 24
    mant = lambda k: rng.integers(0, 1 << 23, k, dtype=np.uint32)
    a = (np.uint32(0x3F800000) | mant(n)).view(np.float32)
    b = (np.uint32(0x3F800000) | mant(n)).view(np.float32)
    _run_div(probe, a, b)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = (np.float32(0.1) * g).astype(np.float32)
    bc = (1.0 - 0.9 ** rng.integers(1, 10000, n)).astype(np.float32)
    _run_div(probe, m, bc)
    den = (np.sqrt(np.abs(g) * np.float32(0.03)) + np.float32(1e-8)).astype(np.float32)
    _run_div(probe, m, den)


def test_div_edge_cross_product(probe):
    e = _edge_values()
    a = np.repeat(e, e.size)
    b = np.tile(e, e.size)
    _run_div(probe, a, b)
