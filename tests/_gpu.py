"""Helpers shared by the GPU parity tests: run the HIP path through the
binding and the float64 oracle on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from workloads import Dims

TOL = 1e-4  # max |g - o| / max(|o|, rms(o)) for fp32 outputs

OPS11 = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")
MIMO4 = ("mimo_x", "mimo_z", "mimo_o", "norm_weight")


def dev():
    return torch.device("cuda:0")


def to_dev(inp: dict) -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev()) for k, v in inp.items()}


def cfg_gpu(d: Dims, **kw) -> m3.SsmConfig:
    base = dict(batch_size=d.B, sequence_length=d.L, num_heads=d.H, num_groups=d.G, head_dim=d.P,
                state_size=d.N, num_rope_angles=d.A, mimo_rank=d.R, has_z=d.has_z, has_d=d.has_d,
                has_output_norm=d.has_output_norm)
    base.update(kw)
    return m3.SsmConfig(**base)


def cfg_oracle(d: Dims, **kw) -> O.SsmConfig:
    base = dict(batch_size=d.B, sequence_length=d.L, num_heads=d.H, num_groups=d.G, head_dim=d.P,
                state_size=d.N, num_rope_angles=d.A, mimo_rank=d.R, has_z=d.has_z, has_d=d.has_d,
                has_output_norm=d.has_output_norm)
    base.update(kw)
    return O.SsmConfig(**base)


def gpu_siso(inp_dev: dict, d: Dims, **kw) -> torch.Tensor:
    out = m3.m3_siso_fwd(*[inp_dev[k] for k in OPS11], cfg_gpu(d), **kw)
    torch.cuda.synchronize()
    return out


def gpu_mimo(inp_dev: dict, d: Dims, **kw) -> torch.Tensor:
    out = m3.m3_mimo_fwd(*[inp_dev[k] for k in OPS11 + MIMO4], cfg_gpu(d), **kw)
    torch.cuda.synchronize()
    return out


def oracle_siso(inp: dict, d: Dims, heads=None, batches=None):
    sub, dd = _batch_subset(inp, d, batches)
    return O.siso_scan(*[sub[k] for k in OPS11], cfg_oracle(dd), heads=heads)


def oracle_mimo(inp: dict, d: Dims, heads=None, batches=None):
    sub, dd = _batch_subset(inp, d, batches)
    return O.mimo_scan(*[sub[k] for k in OPS11 + MIMO4], cfg_oracle(dd), heads=heads)


def _batch_subset(inp, d: Dims, batches):
    if batches is None:
        return inp, d
    bsel = np.asarray(batches)
    sub = {}
    for k, v in inp.items():
        if k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle"):
            sub[k] = v[bsel]
        else:
            sub[k] = v
    dd = Dims(len(bsel), d.L, d.H, d.G, d.P, d.N, d.A, d.R, d.has_z, d.has_d, d.has_output_norm)
    return sub, dd


def assert_parity(got, ref, what: str, tol: float = TOL):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    e = O.parity_error(got, ref)
    print(f"[parity] {what}: e={e['e']:.3e} max_abs={e['max_abs']:.3e} "
          f"normwise={e['normwise']:.3e} n_rel_over={e['n_rel_over']}", flush=True)
    assert e["nonfinite"] == 0, f"{what}: {e['nonfinite']} non-finite outputs"
    assert e["e"] <= tol, f"{what}: parity error {e['e']:.3e} > {tol}"
    return e
