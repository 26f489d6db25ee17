"""Python binding of libfsdpshard.so (argument marshalling only).

Every step of the path runs in the HIP library; this module only turns torch
tensors into device pointers, picks the current HIP stream, and turns status
codes into exceptions. torch is imported first so that the library binds to
the HIP runtime torch has already loaded.

Names follow the C ABI in include/fsdp_shard.h:

* ``Unit(shapes, F, rank)``                 -> fsdp_unit_create / query / tensor
* ``flatten_pad(unit, tensors, dst, ...)``  -> fsdp_flatten_pad
* ``reduce_shard(unit, grads, out, ...)``   -> fsdp_reduce_shard
* ``adamw_shard(unit, grad, master, exp_avg, exp_avg_sq, param_out, hp)``
                                            -> fsdp_adamw_shard
* ``reduce_adamw_shard(unit, grads, master, exp_avg, exp_avg_sq, param_out, hp)``
                                            -> fsdp_reduce_adamw_shard
* ``reduce_adamw_units(steps, hp, step)``   -> fsdp_reduce_adamw_units
* ``reduce_shard_hybrid`` / ``reduce_adamw_shard_hybrid`` -> the hybrid-sharding forms
* ``reduce_shard_bf16acc`` / ``reduce_adamw_shard_bf16acc`` -> bf16 partial sums
* ``cast_unflatten(unit, shards, outs)``    -> fsdp_cast_unflatten (bf16 outputs)
* ``unflatten(unit, shards, outs)``         -> fsdp_unflatten (dtypes from the tensors)
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "FsdpError", "Unit", "AdamWHparams", "flatten_pad", "reduce_shard", "adamw_shard",
    "reduce_adamw_shard", "reduce_adamw_units", "UnitsStep", "cast_unflatten", "unflatten",
    "reduce_shard_hybrid", "reduce_adamw_shard_hybrid", "reduce_shard_bf16acc",
    "reduce_adamw_shard_bf16acc", "abi_version", "library_path",
    "F32", "BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfsdpshard.so"
F32, BF16 = 0, 1
MAX_RANKS = 64

_c_void_p_p = ctypes.POINTER(ctypes.c_void_p)


class FsdpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class _UnitInfo(ctypes.Structure):
    _fields_ = [("U", ctypes.c_int64), ("S", ctypes.c_int64), ("padded", ctypes.c_int64),
                ("pad", ctypes.c_int64), ("shard_begin", ctypes.c_int64),
                ("shard_valid", ctypes.c_int64), ("persistent_bytes", ctypes.c_int64),
                ("F", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("n_tensors", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("fingerprint", ctypes.c_uint64)]


class _UnitStep(ctypes.Structure):
    _fields_ = [("unit", ctypes.c_void_p), ("grads", ctypes.POINTER(ctypes.c_void_p)),
                ("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("param_bf16_out", ctypes.c_void_p)]


class _Hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("step", ctypes.c_int64)]


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python sharded_flatparameter_flatten_amd/build.py) first")
    lib = ctypes.CDLL(path)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "fsdp_abi_version": (i32, []),
        "fsdp_status_string": (ctypes.c_char_p, [st]),
        "fsdp_last_error": (ctypes.c_char_p, []),
        "fsdp_unit_create": (st, [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i64),
                                  ctypes.POINTER(vp)]),
        "fsdp_unit_destroy": (st, [vp]),
        "fsdp_unit_query": (st, [vp, ctypes.POINTER(_UnitInfo)]),
        "fsdp_unit_tensor": (st, [vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "fsdp_flatten_pad": (st, [vp, st, _c_void_p_p, i64, i64, vp, vp]),
        "fsdp_reduce_shard": (st, [vp, i32, _c_void_p_p, ctypes.c_double, vp, vp]),
        "fsdp_adamw_shard": (st, [vp, vp, vp, vp, vp, vp, ctypes.POINTER(_Hparams), vp]),
        "fsdp_reduce_adamw_shard": (st, [vp, i32, _c_void_p_p, vp, vp, vp, vp,
                                         ctypes.POINTER(_Hparams), vp]),
        "fsdp_cast_unflatten": (st, [vp, st, _c_void_p_p, _c_void_p_p, vp]),
        "fsdp_reduce_adamw_units": (st, [i32, ctypes.POINTER(_UnitStep), i32,
                                         ctypes.POINTER(_Hparams), vp]),
        "fsdp_unflatten": (st, [vp, st, st, _c_void_p_p, _c_void_p_p, vp]),
        "fsdp_reduce_shard_hybrid": (st, [vp, i32, _c_void_p_p, ctypes.c_double, vp, vp]),
        "fsdp_reduce_shard_bf16acc": (st, [vp, i32, _c_void_p_p, ctypes.c_double, vp, vp]),
        "fsdp_reduce_adamw_shard_bf16acc": (st, [vp, i32, _c_void_p_p, vp, vp, vp, vp,
                                                 ctypes.POINTER(_Hparams), vp]),
        "fsdp_reduce_adamw_shard_hybrid": (st, [vp, i32, _c_void_p_p, vp, vp, vp, vp,
                                                ctypes.POINTER(_Hparams), vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.fsdp_abi_version())


def _check(status: int):
    if status != 0:
        msg = _lib.fsdp_last_error().decode() or _lib.fsdp_status_string(status).decode()
        raise FsdpError(status, msg)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _stream(stream, device=None):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, min_numel: int = 0) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


@dataclass
class AdamWHparams:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01

    def _c(self, step: int, grad_scale: float = 0.0) -> _Hparams:
        return _Hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                        grad_scale, int(step))


class Unit:
    """One FSDP unit (a list of tensor shapes) as seen by rank ``rank`` of ``F``."""

    def __init__(self, shapes, F: int, rank: int):
        shapes = [tuple(int(d) for d in s) for s in shapes]
        ndim = (ctypes.c_int32 * len(shapes))(*[len(s) for s in shapes])
        flat = [d for s in shapes for d in s]
        dims = (ctypes.c_int64 * max(1, len(flat)))(*flat)
        h = ctypes.c_void_p()
        _check(_lib.fsdp_unit_create(F, rank, len(shapes), ndim, dims, ctypes.byref(h)))
        self._h = h
        self.shapes = shapes
        info = _UnitInfo()
        _check(_lib.fsdp_unit_query(self._h, ctypes.byref(info)))
        for name, _ in _UnitInfo._fields_:
            if name != "reserved":
                setattr(self, name, int(getattr(info, name)))
        self.offsets, self.numels = [], []
        for i in range(len(shapes)):
            off, n = ctypes.c_int64(), ctypes.c_int64()
            _check(_lib.fsdp_unit_tensor(self._h, i, ctypes.byref(off), ctypes.byref(n)))
            self.offsets.append(off.value)
            self.numels.append(n.value)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.fsdp_unit_destroy(h)
            self._h = None


def flatten_pad(unit: Unit, tensors, dst: torch.Tensor, begin: int | None = None,
                length: int | None = None, stream=None):
    """dst[q] = padded_flat[begin + q]; defaults to this rank's shard window."""
    begin = unit.shard_begin if begin is None else int(begin)
    length = unit.S if length is None else int(length)
    dtype = dst.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("dst must be float32 or bfloat16")
    code = F32 if dtype == torch.float32 else BF16
    ptrs = [_dev(t, dtype, f"tensors[{i}]", n) for i, (t, n) in
            enumerate(zip(tensors, unit.numels))]
    if len(ptrs) != unit.n_tensors:
        raise ValueError(f"need {unit.n_tensors} tensors, got {len(ptrs)}")
    d = _dev(dst, dtype, "dst", length)
    _check(_lib.fsdp_flatten_pad(unit.handle, code, _ptr_array(ptrs), begin, length, d,
                                 _stream(stream, dst.device)))


def _grad_ptrs(unit: Unit, grads):
    if not 1 <= len(grads) <= MAX_RANKS:
        raise ValueError(f"need 1..{MAX_RANKS} gradient buffers, got {len(grads)}")
    return [_dev(g, torch.bfloat16, f"grads[{k}]", unit.U) for k, g in enumerate(grads)]


def reduce_shard(unit: Unit, grads, out: torch.Tensor, grad_scale: float | None = None,
                 stream=None):
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    o = _dev(out, torch.float32, "out", unit.shard_valid)
    _check(_lib.fsdp_reduce_shard(unit.handle, len(ptrs), _ptr_array(ptrs), gs, o,
                                  _stream(stream, out.device)))


def _state_ptrs(unit: Unit, master, exp_avg, exp_avg_sq, param_out):
    n = unit.shard_valid
    p = _dev(master, torch.float32, "master", n)
    m = _dev(exp_avg, torch.float32, "exp_avg", n)
    v = _dev(exp_avg_sq, torch.float32, "exp_avg_sq", n)
    w = None if param_out is None else _dev(param_out, torch.bfloat16, "param_out", n)
    return p, m, v, w


def adamw_shard(unit: Unit, grad, master, exp_avg, exp_avg_sq, param_out,
                hp: AdamWHparams, step: int, stream=None):
    g = _dev(grad, torch.float32, "grad", unit.shard_valid)
    p, m, v, w = _state_ptrs(unit, master, exp_avg, exp_avg_sq, param_out)
    c = hp._c(step)
    _check(_lib.fsdp_adamw_shard(unit.handle, g, p, m, v, w, ctypes.byref(c),
                                 _stream(stream, master.device)))


def reduce_adamw_shard(unit: Unit, grads, master, exp_avg, exp_avg_sq, param_out,
                       hp: AdamWHparams, step: int, grad_scale: float | None = None,
                       stream=None):
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    p, m, v, w = _state_ptrs(unit, master, exp_avg, exp_avg_sq, param_out)
    c = hp._c(step, gs)
    _check(_lib.fsdp_reduce_adamw_shard(unit.handle, len(ptrs), _ptr_array(ptrs), p, m, v, w,
                                        ctypes.byref(c), _stream(stream, master.device)))


def reduce_shard_bf16acc(unit: Unit, grads, out: torch.Tensor, grad_scale: float | None = None,
                         stream=None):
    """reduce_shard with bf16 partial sums (reduce dtype bf16)."""
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    o = _dev(out, torch.float32, "out", unit.shard_valid)
    _check(_lib.fsdp_reduce_shard_bf16acc(unit.handle, len(ptrs), _ptr_array(ptrs), gs, o,
                                          _stream(stream, out.device)))


def reduce_adamw_shard_bf16acc(unit: Unit, grads, master, exp_avg, exp_avg_sq, param_out,
                               hp: AdamWHparams, step: int, grad_scale: float | None = None,
                               stream=None):
    """reduce_adamw_shard with bf16 partial sums (reduce dtype bf16)."""
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    p, m, v, w = _state_ptrs(unit, master, exp_avg, exp_avg_sq, param_out)
    c = hp._c(step, gs)
    _check(_lib.fsdp_reduce_adamw_shard_bf16acc(unit.handle, len(ptrs), _ptr_array(ptrs),
                                                p, m, v, w, ctypes.byref(c),
                                                _stream(stream, master.device)))


def reduce_shard_hybrid(unit: Unit, replicas: int, grads, out: torch.Tensor,
                        grad_scale: float | None = None, stream=None):
    """Hybrid sharding: grads = replicas*F rows, replica-major."""
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    o = _dev(out, torch.float32, "out", unit.shard_valid)
    _check(_lib.fsdp_reduce_shard_hybrid(unit.handle, int(replicas), _ptr_array(ptrs), gs, o,
                                         _stream(stream, out.device)))


def reduce_adamw_shard_hybrid(unit: Unit, replicas: int, grads, master, exp_avg, exp_avg_sq,
                              param_out, hp: AdamWHparams, step: int,
                              grad_scale: float | None = None, stream=None):
    ptrs = _grad_ptrs(unit, grads)
    gs = 1.0 / len(grads) if grad_scale is None else float(grad_scale)
    p, m, v, w = _state_ptrs(unit, master, exp_avg, exp_avg_sq, param_out)
    c = hp._c(step, gs)
    _check(_lib.fsdp_reduce_adamw_shard_hybrid(unit.handle, int(replicas), _ptr_array(ptrs),
                                               p, m, v, w, ctypes.byref(c),
                                               _stream(stream, master.device)))


class UnitsStep:
    """A multi-unit optimizer step with its arguments marshalled once.

    ``steps``: sequence of (unit, grads, master, exp_avg, exp_avg_sq, param_out or None);
    every entry uses the same number of gradient rows. The tensors must stay
    alive (and at the same addresses) while the object is used; each call only
    fills in the hyper-parameters and the stream."""

    def __init__(self, steps):
        steps = list(steps)
        if not steps:
            raise ValueError("need at least one unit")
        self.n_grads = len(steps[0][1])
        self._keep = [steps]
        self._arr = (_UnitStep * len(steps))()
        for j, (unit, grads, master, exp_avg, exp_avg_sq, param_out) in enumerate(steps):
            if len(grads) != self.n_grads:
                raise ValueError("every unit needs the same number of gradient rows")
            rows = _ptr_array(_grad_ptrs(unit, grads))
            self._keep.append(rows)
            p, m, v, w = _state_ptrs(unit, master, exp_avg, exp_avg_sq, param_out)
            self._arr[j] = _UnitStep(unit.handle.value,
                                     ctypes.cast(rows, ctypes.POINTER(ctypes.c_void_p)), p, m, v, w)
        self.n_units = len(steps)
        self.device = steps[0][2].device

    def __call__(self, hp: AdamWHparams, step: int, grad_scale: float | None = None,
                 stream=None):
        gs = 1.0 / self.n_grads if grad_scale is None else float(grad_scale)
        c = hp._c(step, gs)
        _check(_lib.fsdp_reduce_adamw_units(self.n_units, self._arr, self.n_grads,
                                            ctypes.byref(c), _stream(stream, self.device)))


def reduce_adamw_units(steps, hp: AdamWHparams, step: int, grad_scale: float | None = None,
                       stream=None):
    """One optimizer step over many units (see UnitsStep for the argument layout)."""
    steps = list(steps)
    if steps:
        UnitsStep(steps)(hp, step, grad_scale, stream)


def unflatten(unit: Unit, shards, outs, stream=None):
    """Per-tensor outputs from the F shards; element types from the tensors (fp32/bf16)."""
    if len(shards) != unit.F:
        raise ValueError(f"need {unit.F} shards, got {len(shards)}")
    if len(outs) != unit.n_tensors:
        raise ValueError(f"need {unit.n_tensors} outputs, got {len(outs)}")
    sdtype, ddtype = shards[0].dtype, outs[0].dtype
    codes = {torch.float32: F32, torch.bfloat16: BF16}
    if sdtype not in codes or ddtype not in codes:
        raise TypeError("shards and outputs must be float32 or bfloat16")
    sp = []
    for k, s in enumerate(shards):
        valid = max(0, min(unit.S, unit.U - k * unit.S))
        sp.append(_dev(s, sdtype, f"shards[{k}]", valid))
    op = [_dev(o, ddtype, f"outs[{i}]", n) for i, (o, n) in enumerate(zip(outs, unit.numels))]
    _check(_lib.fsdp_unflatten(unit.handle, codes[sdtype], codes[ddtype], _ptr_array(sp),
                               _ptr_array(op), _stream(stream, outs[0].device)))


def cast_unflatten(unit: Unit, shards, outs, stream=None):
    """The all-gather arithmetic: F shards -> per-tensor bf16 parameters."""
    if outs and outs[0].dtype != torch.bfloat16:
        raise TypeError("cast_unflatten writes bf16 tensors; use unflatten for fp32 outputs")
    unflatten(unit, shards, outs, stream)
