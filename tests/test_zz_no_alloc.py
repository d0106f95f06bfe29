"""m3_siso_fwd_noalloc: the allocation-free variant of m3_siso_fwd, called
through the C ABI, against m3_siso_fwd on the same inputs (the same kernels
run, so the outputs agree bit for bit, and both meet the oracle bar).  Two
calls in a row, the second on a smaller input, then the first again: the
shared scratch keeps the last call's contents and must not leak into the
next result."""

import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_mamba3_amd as m3
from selective_state_space_mamba3_amd import _binding as bd
from _gpu import OPS11, TOL, assert_parity, cfg_gpu, oracle_siso, to_dev
from workloads import Dims, ssm_inputs

pytestmark = pytest.mark.gpu


def _noalloc_c_call(inp_dev, d):
    """Call the entry point through ctypes with caller-owned buffers only."""
    cfg = cfg_gpu(d)
    out = torch.empty((d.B, d.L, d.H, d.P), dtype=torch.float32, device="cuda:0")
    L = m3.lib()
    ptrs = [ctypes.c_void_p(inp_dev[k].data_ptr()) for k in OPS11]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = L.m3_siso_fwd_noalloc(*ptrs, bd.c_ssm(cfg), ctypes.c_void_p(out.data_ptr()), stream)
    assert st == bd.M3_OK, m3.last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _reference(inp_dev, d):
    out = m3.m3_siso_fwd(*[inp_dev[k] for k in OPS11], cfg_gpu(d))
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # (dims, seed): the first spans several segments (the scratch holds their
    # summaries); the second is smaller (fewer heads, shorter, another A)
    (Dims(2, 700, 4, 1, 64, 128, 32), 7101),
    (Dims(1, 333, 3, 1, 64, 128, 16), 7102),
]


def test_noalloc_matches_siso_fwd_two_calls():
    print("[no-alloc] two calls, the second smaller", flush=True)
    results = []
    for d, seed in CASES + CASES[:1]:
        inp = ssm_inputs(d, seed=seed)
        di = to_dev(inp)
        with m3.scan_segments(0):
            assert m3.siso_fwd_workspace_bytes(cfg_gpu(d)) > 0
        got = _noalloc_c_call(di, d)
        ref = _reference(di, d)
        np.testing.assert_array_equal(got, ref)
        e = assert_parity(got, oracle_siso(inp, d), f"noalloc B{d.B} L{d.L} H{d.H} A{d.A}", tol=TOL)
        results.append(e["e"])
    assert len(results) == 3


def test_noalloc_forced_segments_and_binding():
    d = Dims(2, 260, 3, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=7103)
    di = to_dev(inp)
    with m3.scan_segments(7):
        got = m3.m3_siso_fwd_noalloc(*[di[k] for k in OPS11], cfg_gpu(d))
        ref = m3.m3_siso_fwd(*[di[k] for k in OPS11], cfg_gpu(d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
