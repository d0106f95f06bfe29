"""GPU checks of m3_siso_fwd_packed (preprocess and scan fused on the packed
rows): bit-identical to m3_preprocess followed by m3_siso_fwd when the packed
rows allow the same 16-byte loads (both calls then run the same kernel
variant), within 1e-5 of it otherwise, and within the parity bound of the
oracle's preprocess followed by its scan."""

import numpy as np
import pytest
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from _gpu import OPS11, assert_parity, cfg_gpu, cfg_oracle, dev
from workloads import WORKLOADS, Dims, packed_projection

pytestmark = pytest.mark.gpu

PRE_KEYS = (("x", "x"), ("z", "z"), ("b", "bh"), ("c", "ch"), ("adt", "adt"), ("dt", "dt"),
            ("trap", "trap"), ("angle", "angle"))


def _cfgs(d: Dims):
    G = d.groups
    gp = m3.PreprocessConfig(d.H * d.P, d.N, d.H, d.A, G, 1, 1e-5, 1e-3, 0.1, 1e-4)
    op = O.PreprocessConfig(d.H * d.P, d.N, d.H, d.A, G, 1, 1e-5, 1e-3, 0.1, 1e-4)
    return gp, op


def _shapes(d: Dims):
    B, L, H, P, N, A, G = d.B, d.L, d.H, d.P, d.N, d.A, d.groups
    return {"x": (B, L, H, P), "z": (B, L, H, P), "b": (B, L, G, N), "c": (B, L, G, N),
            "adt": (B, L, H), "dt": (B, L, H), "trap": (B, L, H), "angle": (B, L, A)}


def _same_variant(d: Dims) -> bool:
    """Packed rows with 16-byte x / z and angle columns (width, inner size and
    angle column offset multiples of 4), as the dense operands have."""
    I, M = d.H * d.P, d.groups * d.N
    W = 2 * I + 2 * M + 3 * d.H + d.A
    return W % 4 == 0 and I % 4 == 0 and (2 * I + 2 * M + 3 * d.H) % 4 == 0


@pytest.mark.parametrize("d", [
    Dims(2, 80, 4, 1, 16, 32, 8),
    Dims(1, 100, 3, 3, 24, 40, 4, has_z=False),     # one group per head, scalar-load layout
    Dims(2, 45, 4, 2, 32, 64, 0, has_d=False),       # no angles
    Dims(1, 300, 2, 1, 64, 128, 32),                 # N=128 / P=64, rows not 16-byte aligned
    Dims(1, 300, 4, 1, 64, 128, 32),                 # N=128 / P=64 variant on both paths, segments
], ids=lambda d: f"B{d.B}L{d.L}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}")
def test_packed_equals_preprocess_then_scan(d):
    print(f"[case] packed {d}", flush=True)
    gp, op = _cfgs(d)
    pk = packed_projection(d, seed=7000 + d.L)
    t = {k: torch.from_numpy(v).to(dev()) for k, v in pk.items()}
    fused = m3.m3_siso_fwd_packed(t["projected"], t["dt_bias"], t["c_bias"], t["b_bias"], t["d"], gp, cfg_gpu(d))
    outs = m3.m3_preprocess(t["projected"], t["dt_bias"], gp)
    shape = _shapes(d)
    gi = {k: outs[src].reshape(shape[k]) for k, src in PRE_KEYS}
    gi.update({k: t[k] for k in ("c_bias", "b_bias", "d")})
    twostep = m3.m3_siso_fwd(*[gi[k] for k in OPS11], cfg_gpu(d))
    torch.cuda.synchronize()
    if _same_variant(d):
        np.testing.assert_array_equal(fused.cpu().numpy(), twostep.cpu().numpy())
    else:
        # different kernel variants (the fixed-geometry one with its split-bf16
        # state update, fp32-level): they agree to fp32 rounding
        assert_parity(fused.cpu().numpy(), twostep.cpu().numpy().astype(np.float64), "packed vs two calls", tol=1e-5)
    ref = O.preprocess(pk["projected"], pk["dt_bias"], op)
    oi = {k: ref[src].reshape(shape[k]) for k, src in PRE_KEYS}
    oi.update({k: pk[k] for k in ("c_bias", "b_bias", "d")})
    want = O.siso_scan(*[oi[k] for k in OPS11], cfg_oracle(d))
    assert_parity(fused.cpu().numpy(), want, "packed preprocess -> scan vs oracle")


def test_packed_full_b4_l2048_sampled():
    """The bench geometry in one fused call: bit-identical to the two-call path,
    and heads 0 and 23 of every batch row against the oracle."""
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    print(f"[case] packed full {d}", flush=True)
    gp, op = _cfgs(d)
    pk = packed_projection(d, seed=w.seed)
    t = {k: torch.from_numpy(v).to(dev()) for k, v in pk.items()}
    fused = m3.m3_siso_fwd_packed(t["projected"], t["dt_bias"], t["c_bias"], t["b_bias"], t["d"], gp, cfg_gpu(d))
    outs = m3.m3_preprocess(t["projected"], t["dt_bias"], gp)
    shape = _shapes(d)
    gi = {k: outs[src].reshape(shape[k]) for k, src in PRE_KEYS}
    gi.update({k: t[k] for k in ("c_bias", "b_bias", "d")})
    twostep = m3.m3_siso_fwd(*[gi[k] for k in OPS11], cfg_gpu(d))
    torch.cuda.synchronize()
    got = fused.cpu().numpy()
    assert _same_variant(d)
    np.testing.assert_array_equal(got, twostep.cpu().numpy())
    ref = O.preprocess(pk["projected"], pk["dt_bias"], op)
    oi = {k: ref[src].reshape(shape[k]) for k, src in PRE_KEYS}
    oi.update({k: pk[k] for k in ("c_bias", "b_bias", "d")})
    heads = [0, d.H - 1]
    want = O.siso_scan(*[oi[k] for k in OPS11], cfg_oracle(d), heads=heads)
    assert_parity(got[:, :, heads], want, "packed full size, heads 0 and 23")
