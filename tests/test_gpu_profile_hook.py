"""The measurement hook m3_set_profile_events on the GPU.

With the hook set, the main scan kernel is launched with the caller's two
events attached, so that they are recorded as the kernel begins and ends.
The outputs must be bit for bit those of the same call without the hook, and
the events' span must be positive and no longer than the whole call's.
"""
import ctypes

import numpy as np
import pytest
import torch

from selective_state_space_mamba3_amd import _binding
from _gpu import gpu_mimo, gpu_siso, to_dev
from workloads import Dims, ssm_inputs

pytestmark = pytest.mark.gpu


def _hip():
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    return hip


CASES = [
    ("siso", Dims(2, 300, 4, 1, 64, 128, 32), 4100),
    ("mimo", Dims(2, 300, 4, 1, 64, 128, 32, R=4, has_output_norm=True), 4101),
]


@pytest.mark.parametrize("kind,d,seed", CASES, ids=[c[0] for c in CASES])
def test_profile_events_time_the_main_kernel(kind, d, seed):
    run = gpu_siso if kind == "siso" else gpu_mimo
    inp = to_dev(ssm_inputs(d, seed=seed))
    plain = run(inp, d).cpu().numpy()

    hip = _hip()
    lib = _binding.lib()
    lib.m3_set_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e0)) == 0
    assert hip.hipEventCreate(ctypes.byref(e1)) == 0
    try:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lib.m3_set_profile_events(e0, e1)
        try:
            a.record()
            hooked = run(inp, d)
            b.record()
            torch.cuda.synchronize()
        finally:
            lib.m3_set_profile_events(None, None)
        np.testing.assert_array_equal(hooked.cpu().numpy(), plain)
        kms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(kms), e0, e1) == 0
        call_ms = a.elapsed_time(b)
        assert 0.0 < kms.value <= call_ms * 1.05 + 0.01, (kms.value, call_ms)
        # with the hook off again, the next call leaves the events as they were
        run(inp, d)
        again = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(again), e0, e1) == 0
        assert again.value == kms.value
    finally:
        hip.hipEventDestroy(e0)
        hip.hipEventDestroy(e1)
