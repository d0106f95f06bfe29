"""GPU parity of m3_siso_bwd and m3_preprocess_bwd against the float64
oracle's adjoints on the same seeded inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from _gpu import OPS11, assert_parity, cfg_gpu, cfg_oracle, to_dev
from workloads import WORKLOADS, Dims, output_gradient, preprocess_inputs, preprocess_output_gradients, ssm_inputs

pytestmark = pytest.mark.gpu


def _gpu_bwd(inp_dev, dout_dev, d):
    g = m3.m3_siso_bwd(dout_dev, *[inp_dev[k] for k in OPS11], cfg_gpu(d))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _print_case(tag):
    print(f"[case] {tag}", flush=True)


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
    Dims(1, 64, 2, 1, 16, 16, 8),                    # two whole chunks
    Dims(2, 75, 4, 2, 16, 32, 8),                    # ragged last chunk, groups
    Dims(1, 33, 3, 0, 24, 40, 20, has_z=False),      # one head per group, N not a multiple of 16
    Dims(2, 50, 2, 1, 5, 6, 3, has_d=False),         # odd sizes
    Dims(1, 96, 2, 1, 64, 128, 32),                  # the N=128 / P=64 / A=32 geometry (its own kernels)
    Dims(1, 77, 4, 2, 64, 128, 32),                  # the same kernels, ragged last chunk, groups
    Dims(2, 45, 2, 1, 64, 128, 32, has_z=False, has_d=False),  # the same kernels without z and D
    Dims(1, 1, 2, 1, 64, 128, 32),                   # the same kernels, a single token
    Dims(3, 20, 2, 2, 64, 128, 32),                  # the same kernels, one partial chunk, one head per group
    Dims(1, 40, 2, 1, 32, 64, 0),                    # no rotary angles
    Dims(1, 70, 2, 1, 128, 128, 64),                 # the largest head_dim, state and angle count
    Dims(1, 31, 2, 2, 16, 32, 16, has_z=False, has_d=False),  # A = N/2, shorter than a chunk
], ids=lambda d: f"B{d.B}L{d.L}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}"
                 f"{'' if d.has_z else 'nz'}{'' if d.has_d else 'nd'}")
def test_siso_bwd_matches_oracle(d):
    _print_case(f"siso_bwd {d}")
    inp = ssm_inputs(d, seed=5000 + d.L, mimo=False)
    dout = output_gradient(d, seed=5100 + d.L)
    got = _gpu_bwd(to_dev(inp), torch.from_numpy(dout).cuda(), d)
    ref = O.siso_backward(dout, *[inp[k] for k in OPS11], cfg_oracle(d))
    for k in OPS11:
        if k == "angle" and (d.A == 0 or _angle_zero(got, ref, d)):
            continue
        assert_parity(got[k], ref[k], f"d_{k}")
    if not d.has_z:
        assert not np.any(got["z"])
    if not d.has_d:
        assert not np.any(got["d"])


def test_siso_bwd_is_deterministic():
    d = Dims(2, 100, 4, 2, 32, 64, 16)
    _print_case(f"siso_bwd twice {d}")
    inp = to_dev(ssm_inputs(d, seed=5201, mimo=False))
    dout = torch.from_numpy(output_gradient(d, seed=5202)).cuda()
    a = _gpu_bwd(inp, dout, d)
    b = _gpu_bwd(inp, dout, d)
    for k in OPS11:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def _offset_view(a: np.ndarray) -> torch.Tensor:
    """A device copy of ``a`` that starts 4 bytes into its allocation, so its
    rows are not 16-byte aligned."""
    buf = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
    v = buf[1:].view(a.shape)
    v.copy_(torch.from_numpy(a))
    return v


def test_siso_bwd_unaligned_operands():
    """B and x 4 bytes off 16-byte alignment: the N=128 / P=64 / A=32 geometry
    then runs on the general kernels, with the same results to the parity bound."""
    d = Dims(1, 70, 2, 1, 64, 128, 32)
    _print_case(f"siso_bwd unaligned {d}")
    inp = ssm_inputs(d, seed=5301, mimo=False)
    dout = output_gradient(d, seed=5302)
    dev_inp = to_dev(inp)
    dev_inp["b"] = _offset_view(inp["b"])
    dev_inp["x"] = _offset_view(inp["x"])
    got = _gpu_bwd(dev_inp, torch.from_numpy(dout).cuda(), d)
    aligned = _gpu_bwd(to_dev(inp), torch.from_numpy(dout).cuda(), d)
    ref = O.siso_backward(dout, *[inp[k] for k in OPS11], cfg_oracle(d))
    for k in OPS11:
        assert_parity(got[k], ref[k], f"d_{k} (unaligned)")
        assert_parity(aligned[k], ref[k], f"d_{k} (aligned)")


def test_siso_bwd_full_b4_l2048_sampled():
    """Full siso_b4_l2048 geometry in one call; the oracle takes batch row 0
    (all heads).  The batch-summed gradients are checked on a second full-size
    call whose upstream gradient is zero outside row 0."""
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    _print_case(f"siso_bwd full {d}")
    inp = ssm_inputs(d, seed=w.seed, mimo=False)
    dout = output_gradient(d, seed=w.seed)
    inp_dev = to_dev(inp)
    got = _gpu_bwd(inp_dev, torch.from_numpy(dout).cuda(), d)
    ref = O.siso_backward(dout, *[inp[k] for k in OPS11], cfg_oracle(d), batches=[0])
    for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle"):
        assert_parity(got[k][:1], ref[k], f"d_{k} (batch row 0)")
    dout0 = dout.copy()
    dout0[1:] = 0.0
    got0 = _gpu_bwd(inp_dev, torch.from_numpy(dout0).cuda(), d)
    for k in ("c_bias", "b_bias", "d"):
        assert_parity(got0[k], ref[k], f"d_{k} (upstream gradient in row 0 only)")


def _pre_cfgs(I, N, H, A, G, R=1):
    gcfg = m3.PreprocessConfig(I, N, H, A, G, R, 1e-5, 1e-3, 0.1, 1e-4)
    ocfg = O.PreprocessConfig(I, N, H, A, G, R, 1e-5, 1e-3, 0.1, 1e-4)
    return gcfg, ocfg


def _near_kinks(proj, bias, ocfg, margin=1e-5):
    """Masks of dt and A entries whose softplus lies within ``margin`` (relative)
    of the dt clamp bounds or the A floor: there float32 and float64 may take
    different branches, and both gradients would be correct."""
    I, M, H = ocfg.inner_size, ocfg.num_groups * ocfg.mimo_rank * ocfg.state_size, ocfg.num_heads
    o = 2 * I + 2 * M
    sp = O.softplus(proj[:, o:o + H].astype(np.float64) + bias.astype(np.float64)[None])
    sa = O.softplus(proj[:, o + H:o + 2 * H].astype(np.float64))
    lo, hi, fl = (float(np.float32(v)) for v in (ocfg.dt_min, ocfg.dt_max, ocfg.a_floor))
    near_dt = (np.abs(sp - lo) <= margin * lo) | (np.abs(sp - hi) <= margin * hi)
    near_a = np.abs(sa - fl) <= margin * fl
    return o, near_dt, near_a


def _off_kinks(proj, bias, ocfg):
    """Move the (rare) entries that sit on a kink off it by 2e-3 in the raw input."""
    for _ in range(4):
        o, near_dt, near_a = _near_kinks(proj, bias, ocfg)
        if not (near_dt.any() or near_a.any()):
            return proj
        H = ocfg.num_heads
        proj[:, o:o + H][near_dt] += np.float32(2e-3)
        proj[:, o + H:o + 2 * H][near_a] += np.float32(2e-3)
    raise AssertionError("could not move the seeded inputs off the clamp and floor boundaries")


@pytest.mark.parametrize("rows,I,N,H,A,G,R,missing", [
    (37, 48, 16, 3, 4, 2, 1, ()),
    (64, 64, 32, 4, 0, 1, 2, ("z", "adt")),
    (8192, 1536, 128, 24, 32, 1, 1, ()),           # the bench geometry, every row
    (50, 30, 12, 5, 6, 1, 1, ("x", "bh", "ch", "dt", "trap", "angle")),
])
def test_preprocess_bwd_matches_oracle(rows, I, N, H, A, G, R, missing):
    _print_case(f"preprocess_bwd rows={rows} I={I} N={N} H={H} A={A} G={G} R={R} missing={missing}")
    gcfg, ocfg = _pre_cfgs(I, N, H, A, G, R)
    pin = preprocess_inputs(rows, gcfg.width, H, seed=6000 + rows)
    proj, bias = pin["projected"], pin["dt_bias"]
    o = 2 * I + 2 * G * R * N
    proj[:, o + H:o + 2 * H] -= 9.0   # some A floors bind
    proj = _off_kinks(proj, bias, ocfg)
    grads = preprocess_output_gradients(rows, I, G * R * N, H, A, seed=6100 + rows, missing=missing)
    gdev = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in grads.items()}
    out = m3.m3_preprocess_bwd(torch.from_numpy(proj).cuda(), torch.from_numpy(bias).cuda(), gcfg, gdev)
    torch.cuda.synchronize()
    ref = O.preprocess_backward(proj, bias, grads, ocfg)
    got = out["projected"].cpu().numpy()
    # pass-through columns are bit-exact copies (or zeros)
    for name, lo, width in (("z", 0, I), ("x", I, I), ("trap", o + 2 * H, H), ("angle", o + 3 * H, A)):
        exp = np.zeros((rows, width), np.float32) if grads[name] is None else grads[name]
        np.testing.assert_array_equal(got[:, lo:lo + width], exp, err_msg=name)
    assert_parity(got, ref["projected"], "d_projected")
    assert_parity(out["dt_bias"].cpu().numpy(), ref["dt_bias"], "d_dt_bias")
