"""A HIP error left pending by someone else's call is handed back, not swallowed.

Every entry point that launches work first looks at the calling thread's
pending HIP error: if an earlier, unrelated call left one, the entry point
returns ZS_ERR_HIP before enqueueing anything and leaves the error pending for
its owner; a clean thread's launches report only their own status. The error
is planted from the host (a device ordinal that does not exist), so no kernel
ever faults.
"""
import ctypes as C

import pytest
import torch

import fsdp_sharded_optimizer_flatparameter_amd as zs
from _gpu import device_rows

pytestmark = pytest.mark.gpu


def _hip():
    hip = C.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [C.c_int]
    hip.hipSetDevice.restype = C.c_int
    hip.hipPeekAtLastError.restype = C.c_int
    hip.hipGetLastError.restype = C.c_int
    return hip


def test_pending_error_is_returned_and_left_pending():
    hip = _hip()
    n = 4096
    th = device_rows(31, 1, n, "f32")[0]
    slot = torch.zeros(n, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0  # a clean thread to start from
    cur = torch.cuda.current_device()
    try:
        assert hip.hipSetDevice(1 << 20) != 0
        pending = hip.hipPeekAtLastError()
        if pending == 0:
            pytest.skip("this HIP runtime does not record a failed hipSetDevice as the last error")
        with pytest.raises(zs.ZsError) as e:
            zs.zs_cast_for_gather(th, slot)
        assert e.value.status == -100
        assert hip.hipPeekAtLastError() == pending  # still there for its owner
        assert hip.hipGetLastError() == pending     # which reads and clears it
    finally:
        hip.hipGetLastError()
        hip.hipSetDevice(cur)
    # nothing was enqueued by the refused call; a clean call then works
    assert torch.count_nonzero(slot.view(torch.int16)).item() == 0
    zs.zs_cast_for_gather(th, slot)
    torch.cuda.synchronize()
    assert torch.equal(slot, th.to(torch.bfloat16))
