"""GPU parity of m3_siso_fwd against the float64 oracle on seeded inputs."""

import os
import time

import numpy as np
import pytest
import torch

import selective_state_space_mamba3_amd as m3
from _gpu import assert_parity, gpu_siso, oracle_siso, to_dev
from oracle_pool import oracle_heads, pool_size
from workloads import WORKLOADS, Dims, ssm_inputs

pytestmark = pytest.mark.gpu

SMALL = [
    # (name, dims, seed, dt_range)
    ("siso_tiny_B1_L64_H2_P16_N16_A8", WORKLOADS["siso_tiny"].dims, 1000, (1e-3, 0.1)),
    ("X1_B2_L67_H4_G2_P24_N48_A8", Dims(2, 67, 4, 2, 24, 48, 8), 2001, (1e-3, 0.1)),
    ("X2_G0_H3_A0_noz", Dims(2, 45, 3, 0, 16, 32, 0, has_z=False), 2002, (1e-3, 0.1)),
    ("X3_N32_A16_nod", Dims(1, 99, 2, 1, 32, 32, 16, has_d=False), 2003, (1e-3, 0.1)),
    ("X4_P128_N128_L130", Dims(2, 130, 2, 1, 128, 128, 32), 2004, (1e-3, 0.1)),
    ("odd_P5_N6_A3_L33", Dims(1, 33, 2, 2, 5, 6, 3), 2005, (1e-3, 0.1)),
    ("P64_N128_L1", Dims(3, 1, 5, 1, 64, 128, 32), 2006, (1e-3, 0.1)),
    ("P64_N128_L257_ragged", Dims(2, 257, 6, 3, 64, 128, 32), 2007, (1e-3, 0.1)),
    ("P48_N80_A40_L100", Dims(1, 100, 4, 4, 48, 80, 40), 2008, (1e-3, 0.1)),
    ("P16_N128_A64_L70_flags_off", Dims(2, 70, 2, 1, 16, 128, 64, has_z=False, has_d=False), 2009,
     (1e-3, 0.1)),
    ("P64_N128_A16_L150_G2_noz", Dims(2, 150, 4, 2, 64, 128, 16, has_z=False), 2011, (1e-3, 0.1)),
    ("P64_N128_A0_L97_nod", Dims(1, 97, 3, 1, 64, 128, 0, has_d=False), 2012, (1e-3, 0.1)),
    ("P64_N128_A16_L31_flags_off", Dims(2, 31, 2, 1, 64, 128, 16, has_z=False, has_d=False), 2013,
     (1e-3, 0.1)),
    ("P64_N128_A8_L70", Dims(1, 70, 2, 1, 64, 128, 8), 2014, (1e-3, 0.1)),
]


@pytest.mark.parametrize("name,d,seed,dtr", SMALL, ids=[s[0] for s in SMALL])
def test_siso_small(name, d, seed, dtr):
    inp = ssm_inputs(d, seed=seed, dt_range=dtr)
    got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), name)


@pytest.mark.parametrize("sign", [+1, -1])
def test_siso_trap_extremes(sign):
    d = Dims(2, 90, 3, 1, 32, 64, 16)
    inp = ssm_inputs(d, seed=2010 + sign)
    inp["trap"][:] = 40.0 * sign
    got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), f"X6_trap_{sign * 40}")


@pytest.mark.parametrize("nseg", [1, 3])
def test_siso_wide_dynamic_range(nseg):
    """x spread over eight decades per token and fast decay (dt up to 0.2):
    the head-geometry kernels split their state-update operands into bf16
    heads and remainders, whose error is relative to each product, so the
    bar holds at any mix of scales."""
    d = Dims(2, 300, 3, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=2030, dt_range=(1e-3, 0.2))
    rng = np.random.default_rng(2031)
    inp["x"] = (inp["x"] * 10.0 ** rng.uniform(-4.0, 4.0, size=(d.B, d.L, 1, 1))).astype(np.float32)
    with m3.scan_segments(nseg):
        got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), f"wide_range_segments_{nseg}")


@pytest.mark.parametrize("nseg", [1, 2, 3, 7])
def test_siso_forced_segments(nseg):
    # the same answer whatever the number of sequence segments
    d = Dims(2, 300, 3, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=2020)
    with m3.scan_segments(nseg):
        got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), f"segments_{nseg}")


@pytest.mark.parametrize("nseg", [4, 10])
def test_siso_forced_segments_a16(nseg):
    d = Dims(2, 300, 3, 1, 64, 128, 16, has_z=False)
    inp = ssm_inputs(d, seed=2021)
    with m3.scan_segments(nseg):
        got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), f"segments_a16_{nseg}")


def test_siso_sixty_four_segments():
    # one 32-token chunk per segment: the entry state composes up to 63 summaries
    d = Dims(1, 2048, 2, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=2022)
    with m3.scan_segments(64):
        got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), "segments_64")


def test_siso_register_fold_limit():
    # 128 one-chunk segments: the last folds 127 summaries, next to the
    # register fold's limit of 128
    d = Dims(1, 4096, 2, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=2024, dt_range=(1e-3, 0.01))
    with m3.scan_segments(128):
        got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), "segments_128")


def test_siso_few_chains_long_sequence_automatic_plan():
    # two chains over 16384 tokens: the automatic plan would take 128 segments
    # and is held at 65 (the last segment folds 64 summaries)
    d = Dims(1, 16384, 2, 1, 64, 128, 32)
    inp = ssm_inputs(d, seed=2023, dt_range=(1e-3, 0.01))
    cfg = m3.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A)
    with m3.scan_segments(65):
        capped = m3.siso_fwd_workspace_bytes(cfg)
    assert m3.siso_fwd_workspace_bytes(cfg) == capped
    got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_siso(inp, d), "few chains, 65 segments")


def test_siso_deterministic():
    d = Dims(2, 200, 4, 1, 64, 128, 32)
    inp = to_dev(ssm_inputs(d, seed=2030))
    a = gpu_siso(inp, d).cpu().numpy()
    b = gpu_siso(inp, d).cpu().numpy()
    np.testing.assert_array_equal(a, b)


def test_siso_does_not_touch_inputs():
    d = Dims(1, 50, 2, 1, 16, 32, 8)
    inp = ssm_inputs(d, seed=2040)
    di = to_dev(inp)
    gpu_siso(di, d)
    for k, v in inp.items():
        np.testing.assert_array_equal(di[k].cpu().numpy(), v)


def test_siso_full_b4_l2048_all_heads():
    """The 1.3B-class layer B4 L2048 H24 P64 N128 A32: every output element
    against the oracle (all 24 heads, the oracle sharded over host cores)."""
    w = WORKLOADS["siso_b4_l2048"]
    d = w.dims
    inp = ssm_inputs(d, seed=w.seed, dt_range=w.dt_range)
    got = gpu_siso(to_dev(inp), d).cpu().numpy()
    assert got.shape == (4, 2048, 24, 64)
    assert np.isfinite(got).all()
    t0 = time.time()
    ref = oracle_heads("siso_b4_l2048")
    print(f"[oracle] siso_b4_l2048 all heads on {pool_size(d.H)} processes: {time.time() - t0:.1f} s", flush=True)
    assert_parity(got, ref, "siso_b4_l2048 all heads")


def test_siso_full_long_l65536_all_heads():
    """B1 L65536 H32 with dt in [1e-3, 0.01]: every head over the whole
    sequence (the oracle sharded over host cores)."""
    w = WORKLOADS["siso_long_l65536"]
    d = w.dims
    inp = ssm_inputs(d, seed=w.seed, dt_range=w.dt_range)
    got = gpu_siso(to_dev(inp), d).cpu().numpy()
    del inp
    assert np.isfinite(got).all()
    t0 = time.time()
    ref = oracle_heads("siso_long_l65536")
    print(f"[oracle] siso_long_l65536 all heads on {pool_size(d.H)} processes: {time.time() - t0:.1f} s",
          flush=True)
    assert_parity(got, ref, "siso_long_l65536 all heads")
