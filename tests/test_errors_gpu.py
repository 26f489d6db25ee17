"""Error behaviour on a GPU: a HIP error left pending by earlier work.

The header promises that a device entry point checks the thread's HIP error
state before its first launch and, if an error from earlier work is pending,
returns FSDP_ERR_HIP, enqueues nothing and leaves that error for its owner.
The error is forced from the host with hipSetDevice on an ordinal that does
not exist (the runtime refuses it without touching the GPU); the call is made
through the raw C ABI so that no other runtime call runs in between.
"""

import ctypes

import numpy as np
import pytest
import torch

from conftest import gpu_available
from shard_cases import HP
import datagen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so.7")
    for name in ("hipPeekAtLastError", "hipGetLastError", "hipSetDevice"):
        getattr(hip, name).restype = ctypes.c_int
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    return hip


def test_pending_error_refuses_to_enqueue_and_is_left_in_place(lib):
    hip = hip_runtime()
    raw = lib._lib
    u = lib.Unit([(8 * 4096,)], 8, 2)
    rows = []
    for k in range(8):
        r = torch.zeros(u.U, dtype=torch.bfloat16, device="cuda")
        datagen.fill_bf16_(r, 5, k, 1e-3)
        rows.append(r)
    p = torch.empty(u.S, dtype=torch.float32, device="cuda")
    datagen.fill_normal_f32_(p, 3, 0, 0.02)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    torch.cuda.synchronize()
    before = [t.cpu().numpy().copy() for t in (p, m, v)]
    arr = lib._ptr_array([r.data_ptr() for r in rows])
    hp = lib.AdamWHparams(**HP.__dict__)._c(1, 1.0 / 8)
    stream = torch.cuda.current_stream().cuda_stream
    args = (u.handle, 8, arr, p.data_ptr(), m.data_ptr(), v.data_ptr(), None, ctypes.byref(hp),
            stream)
    assert hip.hipPeekAtLastError() == 0, "an error was pending before the test"

    assert hip.hipSetDevice(1 << 20) != 0                  # forced: no such device
    forced = hip.hipPeekAtLastError()
    if forced == 0:
        pytest.skip("this HIP runtime does not keep a refused call's status as the last error")
    status = raw.fsdp_reduce_adamw_shard(*args)
    msg = raw.fsdp_last_error().decode()
    still = hip.hipPeekAtLastError()
    cleared = hip.hipGetLastError()                        # the error's owner clears it
    assert status == 5 and "pending" in msg and "nothing was enqueued" in msg, (status, msg)
    assert still == forced and cleared == forced
    assert hip.hipPeekAtLastError() == 0

    torch.cuda.synchronize()
    after = [t.cpu().numpy() for t in (p, m, v)]
    for b, a, name in zip(before, after, ("master", "exp_avg", "exp_avg_sq")):
        assert np.array_equal(b.view(np.uint32), a.view(np.uint32)), f"{name} changed"

    assert raw.fsdp_reduce_adamw_shard(*args) == 0         # with the error cleared it runs
    torch.cuda.synchronize()
    assert not np.array_equal(before[0], p.cpu().numpy())
