"""GPU parity of m3_mimo_bwd against the float64 oracle's MIMO adjoints on
the same seeded inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from _gpu import MIMO4, OPS11, assert_parity, cfg_gpu, cfg_oracle, to_dev
from workloads import WORKLOADS, Dims, output_gradient, ssm_inputs

pytestmark = pytest.mark.gpu

OPS15 = OPS11 + MIMO4


def _gpu_bwd(inp_dev, dout_dev, d):
    g = m3.m3_mimo_bwd(dout_dev, *[inp_dev[k] for k in OPS15], cfg_gpu(d))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _angle_zero(got, ref, d):
    """One token: Q_0 . K_0 does not change under the shared rotation, so the
    angle gradient is exactly zero and both sides hold only the rounding
    residue of the rotation terms that cancel.  The check bounds that residue
    by the parity tolerance times the scale of the key adjoint d_b."""
    if not (d.L == 1 and d.A > 0):
        return False
    assert np.abs(ref["angle"]).max() <= 1e-12 * np.abs(ref["b"]).max()
    assert np.abs(got["angle"]).max() <= 1e-4 * np.abs(ref["b"]).max()
    return True


@pytest.mark.parametrize("d", [
    Dims(1, 40, 2, 1, 16, 32, 8, R=2, has_output_norm=True),
    Dims(2, 37, 4, 2, 16, 32, 8, R=3, has_z=False),                 # a padding rank, groups
    Dims(1, 70, 2, 1, 64, 128, 32, R=4, has_output_norm=True),      # the N=128 / P=64 / A=32 kernels
    Dims(1, 45, 2, 1, 64, 128, 32, R=3, has_output_norm=True),      # the same, a padding rank, ragged
    Dims(2, 37, 4, 2, 64, 128, 32, R=2, has_z=False),               # the same, groups, no z
    Dims(1, 20, 2, 1, 64, 128, 32, R=8, has_d=False),               # the same, eight ranks
    Dims(1, 33, 2, 1, 64, 128, 32, R=1, has_output_norm=True),      # the same, one rank
    Dims(2, 1, 2, 2, 64, 128, 32, R=4, has_output_norm=True),       # the same, a single token, one head per group
    Dims(1, 6, 2, 1, 64, 128, 32, R=8),                             # the same, one partial chunk of eight ranks
    Dims(1, 50, 2, 1, 32, 64, 16, R=1, has_output_norm=True),
    Dims(1, 21, 2, 2, 16, 16, 4, R=8, has_d=False),
    Dims(2, 30, 2, 1, 5, 6, 3, R=2, has_output_norm=True),          # odd sizes
    Dims(1, 45, 3, 0, 24, 40, 0, R=2),                              # no angles, one group per head
], ids=lambda d: f"B{d.B}L{d.L}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}R{d.R}{'n' if d.has_output_norm else ''}"
                 f"{'' if d.has_z else 'nz'}{'' if d.has_d else 'nd'}")
def test_mimo_bwd_matches_oracle(d):
    print(f"[case] mimo_bwd {d}", flush=True)
    inp = ssm_inputs(d, seed=9000 + d.L + d.R, mimo=True)
    dout = output_gradient(d, seed=9100 + d.L)
    got = _gpu_bwd(to_dev(inp), torch.from_numpy(dout).cuda(), d)
    ref = O.mimo_backward(dout, *[inp[k] for k in OPS15], cfg_oracle(d))
    for k in OPS15:
        if (k == "angle" and (d.A == 0 or _angle_zero(got, ref, d))) or (k == "norm_weight" and not d.has_output_norm):
            continue
        if (k in ("z", "mimo_z") and not d.has_z) or (k == "d" and not d.has_d):
            assert not np.any(got[k]), k
            continue
        assert_parity(got[k], ref[k], f"d_{k}")
    if not d.has_output_norm:
        assert not np.any(got["norm_weight"])


def test_mimo_bwd_is_deterministic():
    d = Dims(2, 60, 4, 2, 32, 64, 16, R=4, has_output_norm=True)
    print(f"[case] mimo_bwd twice {d}", flush=True)
    inp = to_dev(ssm_inputs(d, seed=9201, mimo=True))
    dout = torch.from_numpy(output_gradient(d, seed=9202)).cuda()
    a = _gpu_bwd(inp, dout, d)
    b = _gpu_bwd(inp, dout, d)
    for k in OPS15:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_mimo_bwd_unaligned_operands():
    """B, x and mimo_x 4 bytes off 16-byte alignment: the N=128 / P=64 / A=32
    geometry then runs on the general kernels, with the same results to the
    parity bound."""
    d = Dims(1, 30, 2, 1, 64, 128, 32, R=4, has_output_norm=True)
    print(f"[case] mimo_bwd unaligned {d}", flush=True)
    inp = ssm_inputs(d, seed=9301, mimo=True)
    dout = output_gradient(d, seed=9302)
    dev_inp = to_dev(inp)
    for k in ("b", "x", "mimo_x"):
        buf = torch.empty(inp[k].size + 1, dtype=torch.float32, device="cuda")
        dev_inp[k] = buf[1:].view(inp[k].shape)
        dev_inp[k].copy_(torch.from_numpy(inp[k]))
    got = _gpu_bwd(dev_inp, torch.from_numpy(dout).cuda(), d)
    ref = O.mimo_backward(dout, *[inp[k] for k in OPS15], cfg_oracle(d))
    for k in OPS15:
        assert_parity(got[k], ref[k], f"d_{k} (unaligned)")


def test_mimo_bwd_full_b8_l4096_r4_sampled():
    """The full mimo_b8_l4096_r4 geometry in one call; the oracle takes batch
    row 0 (all heads).  The batch-summed gradients are checked on a second
    full-size call whose upstream gradient is zero outside row 0."""
    w = WORKLOADS["mimo_b8_l4096_r4"]
    d = w.dims
    print(f"[case] mimo_bwd full {d}", flush=True)
    inp = ssm_inputs(d, seed=w.seed, dt_range=w.dt_range, mimo=True)
    dout = output_gradient(d, seed=w.seed)
    inp_dev = to_dev(inp)
    got = _gpu_bwd(inp_dev, torch.from_numpy(dout).cuda(), d)
    ref = O.mimo_backward(dout, *[inp[k] for k in OPS15], cfg_oracle(d), batches=[0])
    for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle"):
        assert_parity(got[k][:1], ref[k], f"d_{k} (batch row 0)")
    dout0 = dout.copy()
    dout0[1:] = 0.0
    got0 = _gpu_bwd(inp_dev, torch.from_numpy(dout0).cuda(), d)
    for k in ("c_bias", "b_bias", "d") + MIMO4:
        assert_parity(got0[k], ref[k], f"d_{k} (upstream gradient in row 0 only)")
