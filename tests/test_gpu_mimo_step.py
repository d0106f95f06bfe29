"""GPU parity of m3_mimo_step against the float64 oracle on seeded inputs."""

import numpy as np
import pytest
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from _gpu import MIMO4, OPS11, assert_parity, cfg_gpu, cfg_oracle, dev, gpu_mimo, to_dev
from workloads import WORKLOADS, Dims, mimo_decode_states, ssm_inputs, step_inputs

pytestmark = pytest.mark.gpu

STATE_KEYS = ("ssm_state", "angle_state", "k_state", "v_state")
OPS15 = OPS11 + MIMO4


def _gpu_step(tok_dev, states_dev, cfg):
    return m3.m3_mimo_step(*[tok_dev[k] for k in OPS15], *[states_dev[k] for k in STATE_KEYS], cfg)


@pytest.mark.parametrize("d", [
    Dims(3, 1, 4, 2, 16, 32, 8, R=2, has_output_norm=True),
    Dims(2, 1, 3, 0, 24, 48, 8, R=3, has_z=False),
    Dims(2, 1, 2, 1, 5, 6, 3, R=2),                  # odd sizes: generic kernel
    Dims(4, 1, 8, 1, 64, 128, 32, R=4, has_output_norm=True),
    Dims(2, 1, 2, 1, 64, 128, 16, R=8, has_d=False),
    Dims(1, 1, 2, 1, 64, 128, 0, R=1, has_output_norm=True),
    Dims(1, 1, 2, 1, 128, 128, 64, R=2),
    # N=128/P=64 kernel at the ranks whose LDS items do not fill whole thread rounds
    Dims(2, 1, 4, 2, 64, 128, 32, R=3, has_output_norm=True),
    Dims(1, 1, 3, 1, 64, 128, 64, R=5, has_z=False),
    Dims(1, 1, 2, 2, 64, 128, 8, R=6, has_output_norm=True, has_d=False),
    Dims(1, 1, 2, 1, 64, 128, 32, R=7),
], ids=lambda d: f"B{d.B}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}R{d.R}{'n' if d.has_output_norm else ''}")
def test_mimo_step_matches_oracle(d):
    st = mimo_decode_states(d, seed=3400 + d.P + d.R)
    tok = ssm_inputs(d, seed=3500 + d.N + d.R, mimo=True)
    sd = to_dev(st)
    out = _gpu_step(to_dev(tok), sd, cfg_gpu(d)).cpu().numpy()
    ref, ref_st = O.mimo_step(*[tok[k] for k in OPS15], *[st[k] for k in STATE_KEYS], cfg_oracle(d))
    assert_parity(out, ref, "mimo step out")
    for k in STATE_KEYS:
        if k == "v_state":
            xr = tok["x"][:, 0, :, None, :] * tok["mimo_x"][None]  # fp32 products, as the kernel forms them
            np.testing.assert_array_equal(sd[k].cpu().numpy(), xr)
        else:
            assert_parity(sd[k].cpu().numpy(), ref_st[k], f"mimo step {k}")


def test_mimo_steps_equal_mimo_scan_on_gpu():
    d = Dims(2, 40, 4, 2, 32, 64, 16, R=3, has_output_norm=True)
    inp = ssm_inputs(d, seed=3600)
    di = to_dev(inp)
    scan = gpu_mimo(di, d)
    d1 = Dims(d.B, 1, d.H, d.G, d.P, d.N, d.A, d.R, has_output_norm=True)
    zeros = {"ssm_state": torch.zeros(d.B, d.H, d.P, d.N, device=dev()),
             "angle_state": torch.zeros(d.B, d.H, d.A, device=dev()),
             "k_state": torch.zeros(d.B, d.H, d.R, d.N, device=dev()),
             "v_state": torch.zeros(d.B, d.H, d.R, d.P, device=dev())}
    outs = []
    for t in range(d.L):
        tok = {k: (v[:, t:t + 1].contiguous() if v.dim() >= 3 and v.shape[1] == d.L else v)
               for k, v in di.items()}
        outs.append(_gpu_step(tok, zeros, cfg_gpu(d1)))
    steps = torch.cat(outs, dim=1).cpu().numpy()
    assert_parity(steps, scan.cpu().numpy(), "mimo steps vs mimo scan (GPU)")
    assert_parity(steps, O.mimo_scan(*[inp[k] for k in OPS15], cfg_oracle(d)), "mimo steps vs oracle")


def test_mimo_step_rejection_leaves_states_untouched():
    d = Dims(2, 1, 2, 1, 16, 32, 8, R=2)
    st = to_dev(mimo_decode_states(d, seed=3700))
    before = {k: v.clone() for k, v in st.items()}
    tok = to_dev(ssm_inputs(d, seed=3701, mimo=True))
    from selective_state_space_mamba3_amd import _binding as bd
    bad = m3.SsmConfig(2, 1, 2, 1, 16, 32, 8, mimo_rank=9)  # rank above eight
    status = m3.lib().m3_mimo_step(*[tok[k].data_ptr() for k in OPS15],
                                   *[st[k].data_ptr() for k in STATE_KEYS], bd.c_ssm(bad),
                                   torch.empty(2, 1, 2, 16, device=dev()).data_ptr(), None)
    assert status == bd.M3_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    for k in STATE_KEYS:
        assert torch.equal(st[k], before[k])


def test_mimo_decode_b256_r4_full_geometry_sampled():
    """B256 H32 P64 N128 A32 R4 with the output norm: 64 consecutive steps with
    fresh seeded inputs.  Every step runs on the whole batch; the oracle
    follows three batch rows of all heads and checks outputs and states."""
    w = WORKLOADS["mimo_decode_b256_r4"]
    d = w.dims
    rows = np.array([0, 77, 255])
    st_np = mimo_decode_states(d, seed=w.seed)
    sd = to_dev(st_np)
    ref_st = {k: v[rows].astype(np.float64) for k, v in st_np.items()}
    sub = Dims(len(rows), 1, d.H, d.G, d.P, d.N, d.A, d.R, has_output_norm=True)
    cfg = cfg_gpu(d)
    worst = 0.0
    n_steps = 64
    for s in range(n_steps):
        tok = step_inputs(d, w.seed, s, mimo=True)
        out = _gpu_step(to_dev(tok), sd, cfg)
        tsub = {k: (v[rows] if v.ndim >= 3 and v.shape[0] == d.B else v) for k, v in tok.items()}
        ref, ref_st = O.mimo_step(*[tsub[k] for k in OPS15], *[ref_st[k] for k in STATE_KEYS],
                                  cfg_oracle(sub))
        if s % 16 == 0 or s == n_steps - 1:
            e = O.parity_error(out.cpu().numpy()[rows], ref)
            worst = max(worst, e["e"])
            print(f"[mimo decode] step {s}: sampled e={e['e']:.3e}", flush=True)
            assert e["e"] <= 1e-4, f"step {s}: {e}"
    print(f"[parity] mimo decode {n_steps} steps worst sampled e={worst:.3e}", flush=True)
    for k in STATE_KEYS:
        assert_parity(sd[k].cpu().numpy()[rows], ref_st[k], f"mimo decode final {k}")
