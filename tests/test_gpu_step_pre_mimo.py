"""GPU parity of m3_siso_step, m3_preprocess and m3_mimo_fwd against the oracle."""

import time

import numpy as np
import pytest
import torch

import oracle as O
import selective_state_space_mamba3_amd as m3
from _gpu import (OPS11, assert_parity, cfg_gpu, cfg_oracle, dev, gpu_mimo, gpu_siso, oracle_mimo,
                  to_dev)
from oracle_pool import DecodeOracle, oracle_heads, pool_size
from workloads import WORKLOADS, Dims, decode_states, preprocess_inputs, ssm_inputs, step_inputs

pytestmark = pytest.mark.gpu

STATE_KEYS = ("ssm_state", "angle_state", "k_state", "v_state")


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------

def _gpu_step(tok_dev, states_dev, d1):
    out = m3.m3_siso_step(*[tok_dev[k] for k in OPS11], *[states_dev[k] for k in STATE_KEYS], d1)
    return out


@pytest.mark.parametrize("d", [
    Dims(3, 1, 4, 2, 16, 32, 8),
    Dims(2, 1, 3, 0, 24, 48, 8, has_z=False),
    Dims(2, 1, 2, 1, 5, 6, 3),      # odd sizes: scalar state path
    Dims(4, 1, 8, 1, 64, 128, 32),
    Dims(2, 1, 4, 2, 64, 128, 16, has_z=False),
    Dims(1, 1, 3, 1, 64, 128, 0, has_d=False),
    Dims(1, 1, 2, 1, 128, 128, 64, has_d=False),
], ids=lambda d: f"B{d.B}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}")
def test_step_matches_oracle(d):
    st = decode_states(d, seed=3000 + d.P)
    tok = ssm_inputs(d, seed=3100 + d.N)
    sd = to_dev(st)
    out = _gpu_step(to_dev(tok), sd, cfg_gpu(d)).cpu().numpy()
    ref, ref_st = O.siso_step(*[tok[k] for k in OPS11], *[st[k] for k in STATE_KEYS], cfg_oracle(d))
    assert_parity(out, ref, "step out")
    for k in STATE_KEYS:
        if k == "v_state":
            np.testing.assert_array_equal(sd[k].cpu().numpy(), tok["x"][:, 0])
        else:
            assert_parity(sd[k].cpu().numpy(), ref_st[k], f"step {k}")


def test_steps_equal_scan_on_gpu():
    d = Dims(2, 75, 4, 2, 32, 64, 16)
    inp = ssm_inputs(d, seed=3200)
    di = to_dev(inp)
    scan = gpu_siso(di, d)
    d1 = Dims(d.B, 1, d.H, d.G, d.P, d.N, d.A)
    zeros = {"ssm_state": torch.zeros(d.B, d.H, d.P, d.N, device=dev()),
             "angle_state": torch.zeros(d.B, d.H, d.A, device=dev()),
             "k_state": torch.zeros(d.B, d.H, d.N, device=dev()),
             "v_state": torch.zeros(d.B, d.H, d.P, device=dev())}
    outs = []
    for t in range(d.L):
        tok = {k: (v[:, t:t + 1].contiguous() if v.dim() >= 3 and v.shape[1] == d.L else v)
               for k, v in di.items()}
        outs.append(_gpu_step(tok, zeros, cfg_gpu(d1)))
    steps = torch.cat(outs, dim=1).cpu().numpy()
    # both are fp32 paths; compare each against the other with the same metric
    assert_parity(steps, scan.cpu().numpy(), "steps vs scan (GPU)")
    assert_parity(steps, O.siso_scan(*[inp[k] for k in OPS11], cfg_oracle(d)), "steps vs oracle")


def test_step_rejection_leaves_states_untouched():
    d = Dims(2, 1, 2, 1, 16, 32, 8)
    st = to_dev(decode_states(d, seed=3300))
    before = {k: v.clone() for k, v in st.items()}
    tok = to_dev(ssm_inputs(d, seed=3301))
    bad = m3.SsmConfig(2, 1, 2, 1, 16, 32, 8, mimo_rank=2)  # rank must be one
    from selective_state_space_mamba3_amd import _binding as bd
    status = m3.lib().m3_siso_step(*[tok[k].data_ptr() for k in OPS11],
                                   *[st[k].data_ptr() for k in STATE_KEYS], bd.c_ssm(bad),
                                   torch.empty(2, 1, 2, 16, device=dev()).data_ptr(), None)
    assert status == bd.M3_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    for k in STATE_KEYS:
        assert torch.equal(st[k], before[k])


def _decode_rows(w, n=16):
    """Seeded batch rows followed through every step: the first and last row
    and n - 2 others."""
    rng = np.random.default_rng([w.seed, 16])
    mid = np.sort(rng.choice(np.arange(1, w.dims.B - 1), size=n - 2, replace=False))
    return np.concatenate([[0], mid, [w.dims.B - 1]])


def test_decode_b256_full_geometry_1024_steps():
    """B256 H32 P64 N128 A32: 1024 consecutive steps with fresh seeded inputs.
    The whole batch is compared with the oracle at each of the first 16
    steps; 16 seeded rows (all heads) are followed through all 1024 steps,
    every step's output compared, and their final states checked.  The
    oracle runs in a process pool while the GPU steps."""
    w = WORKLOADS["decode_b256"]
    d = w.dims
    full_steps = 16
    rows = _decode_rows(w)
    groups = [rows[i:i + 2] for i in range(0, len(rows), 2)]
    t0 = time.time()
    with DecodeOracle("decode_b256", groups, full_steps) as orc:
        sd = to_dev(decode_states(d, seed=w.seed))
        rows_dev = torch.from_numpy(rows).to(dev())
        got_full, got_rows = [], []
        for s in range(w.steps):
            out = _gpu_step(to_dev(step_inputs(d, w.seed, s)), sd, cfg_gpu(d))
            if s < full_steps:
                got_full.append(out.cpu().numpy())
            got_rows.append(out.index_select(0, rows_dev).cpu().numpy())
        final = {k: sd[k].index_select(0, rows_dev).cpu().numpy() for k in STATE_KEYS}
        t_gpu = time.time() - t0
        ref_full, ref_groups = orc.results()
    print(f"[decode] GPU 1024 steps {t_gpu:.1f} s, oracle done at {time.time() - t0:.1f} s", flush=True)
    for s in range(full_steps):
        assert_parity(got_full[s], ref_full[s], f"decode step {s}, whole batch")
    ref_rows = np.concatenate([g[0] for g in ref_groups], axis=1)  # [steps, rows, 1, H, P]
    worst = 0.0
    for s in range(w.steps):
        e = O.parity_error(got_rows[s], ref_rows[s])["e"]
        worst = max(worst, e)
        assert e <= 1e-4, f"decode step {s}, rows {rows.tolist()}: e={e:.3e}"
    print(f"[parity] decode 1024 steps x {len(rows)} rows worst e={worst:.3e}", flush=True)
    for k in STATE_KEYS:
        ref_k = np.concatenate([g[1][k] for g in ref_groups], axis=0)
        assert_parity(final[k], ref_k, f"decode final {k}")


@pytest.mark.parametrize("centre", [1.0e4, -3.0e4, 2.5e6])
def test_decode_large_accumulated_angles(centre):
    """Angle states of large magnitude (|theta| > 8192, where float32 spacing
    reaches 1e-3): each of 12 steps is compared with the oracle run from the
    GPU's own states of the step before, and the stored angle must be the
    float32 rounding of the exact theta."""
    d = Dims(8, 1, 4, 1, 64, 128, 32)
    st = decode_states(d, seed=3400)
    st["angle_state"] = (np.float32(centre) + st["angle_state"]).astype(np.float32)
    st["angle_state"][1::2] *= np.float32(-1.0)
    sd = to_dev(st)
    for s in range(12):
        tok = step_inputs(d, 3401, s)
        before = {k: v.cpu().numpy() for k, v in sd.items()}
        out = _gpu_step(to_dev(tok), sd, cfg_gpu(d)).cpu().numpy()
        ref, ref_st = O.siso_step(*[tok[k] for k in OPS11], *[before[k] for k in STATE_KEYS], cfg_oracle(d))
        assert_parity(out, ref, f"large-angle step {s} out")
        np.testing.assert_array_equal(sd["angle_state"].cpu().numpy(), ref_st["angle_state"].astype(np.float32))
        assert_parity(sd["ssm_state"].cpu().numpy(), ref_st["ssm_state"], f"large-angle step {s} ssm_state")


# ---------------------------------------------------------------------------
# preprocess
# ---------------------------------------------------------------------------

def _pre_cfgs(I, N, H, A, G, R):
    kw = dict(inner_size=I, state_size=N, num_heads=H, num_rope_angles=A, num_groups=G, mimo_rank=R,
              epsilon=1e-5, dt_min=1e-3, dt_max=0.1, a_floor=1e-4)
    return m3.PreprocessConfig(**kw), O.PreprocessConfig(**kw)


@pytest.mark.parametrize("rows,I,N,H,A,G,R", [
    (37, 12, 8, 3, 2, 2, 2),       # odd widths: scalar copies
    (64, 64, 16, 4, 8, 1, 1),
    (8192, 1536, 128, 24, 32, 1, 1),  # the B4 L2048 H24 layer's packed projection
    (300, 256, 128, 8, 32, 1, 4),     # MIMO rank 4
])
def test_preprocess_matches_oracle(rows, I, N, H, A, G, R):
    gcfg, ocfg = _pre_cfgs(I, N, H, A, G, R)
    pin = preprocess_inputs(rows, gcfg.width, H, seed=4000 + rows)
    pin["projected"] *= 3.0  # push dt/A through both clamps
    outs = m3.m3_preprocess(torch.from_numpy(pin["projected"]).to(dev()),
                            torch.from_numpy(pin["dt_bias"]).to(dev()), gcfg)
    torch.cuda.synchronize()
    ref = O.preprocess(pin["projected"], pin["dt_bias"], ocfg)
    for k in ("x", "z", "trap", "angle"):
        np.testing.assert_array_equal(outs[k].cpu().numpy(), ref[k].astype(np.float32))
    for k in ("bh", "ch", "dt", "adt"):
        assert_parity(outs[k].cpu().numpy(), ref[k], f"preprocess {k}")
    dtv = outs["dt"].cpu().numpy()
    assert dtv.min() >= np.float32(1e-3) and dtv.max() <= np.float32(0.1)


def test_preprocess_then_scan_end_to_end():
    B, L, H, P, N, A = 2, 80, 4, 16, 32, 8
    gcfg, ocfg = _pre_cfgs(H * P, N, H, A, 1, 1)
    pin = preprocess_inputs(B * L, gcfg.width, H, seed=4100)
    outs = m3.m3_preprocess(torch.from_numpy(pin["projected"]).to(dev()),
                            torch.from_numpy(pin["dt_bias"]).to(dev()), gcfg)
    ref = O.preprocess(pin["projected"], pin["dt_bias"], ocfg)
    d = Dims(B, L, H, 1, P, N, A)
    rng = np.random.default_rng(4101)
    extra = {"c_bias": (0.02 * rng.standard_normal((H, N))).astype(np.float32),
             "b_bias": (0.02 * rng.standard_normal((H, N))).astype(np.float32),
             "d": rng.standard_normal(H).astype(np.float32)}
    shape = {"x": (B, L, H, P), "z": (B, L, H, P), "b": (B, L, 1, N), "c": (B, L, 1, N),
             "adt": (B, L, H), "dt": (B, L, H), "trap": (B, L, H), "angle": (B, L, A)}
    gi = {k: outs[src].reshape(shape[k]) for k, src in
          (("x", "x"), ("z", "z"), ("b", "bh"), ("c", "ch"), ("adt", "adt"), ("dt", "dt"),
           ("trap", "trap"), ("angle", "angle"))}
    gi.update(to_dev(extra))
    got = gpu_siso(gi, d).cpu().numpy()
    oi = {k: ref[src].reshape(shape[k]) for k, src in
          (("x", "x"), ("z", "z"), ("b", "bh"), ("c", "ch"), ("adt", "adt"), ("dt", "dt"),
           ("trap", "trap"), ("angle", "angle"))}
    oi.update(extra)
    want = O.siso_scan(*[oi[k] for k in OPS11], cfg_oracle(d))
    assert_parity(got, want, "preprocess -> siso end to end")


# ---------------------------------------------------------------------------
# MIMO
# ---------------------------------------------------------------------------

MIMO_SMALL = [
    ("R2_G2_H4_nonorm", Dims(2, 70, 4, 2, 32, 64, 16, R=2), 5001),
    ("R2_G2_H4_norm", Dims(2, 70, 4, 2, 32, 64, 16, R=2, has_output_norm=True), 5002),
    ("R8_H2_norm", Dims(1, 40, 2, 1, 16, 32, 8, R=8, has_output_norm=True), 5003),
    ("R3_odd_P24_N40", Dims(2, 35, 3, 1, 24, 40, 4, R=3, has_output_norm=True), 5004),
    ("R4_P64_N128_L100", Dims(2, 100, 2, 1, 64, 128, 32, R=4, has_output_norm=True), 5005),
    ("R1_noz_nod", Dims(1, 50, 2, 2, 16, 16, 8, R=1, has_z=False, has_d=False), 5006),
    ("R5_many_segments", Dims(1, 200, 1, 1, 32, 64, 16, R=5, has_output_norm=True), 5007),
    ("R6_G2_H2", Dims(2, 77, 2, 2, 16, 48, 8, R=6), 5008),
    ("R7_P128_N128_A64", Dims(1, 60, 1, 1, 128, 128, 64, R=7, has_output_norm=True), 5009),
    # the head-geometry kernels at every rank stride (1, 2, 4 via rank 3, 8),
    # long enough for sequence segments, so both passes of each run
    ("R1_P64_N128_A32_L200", Dims(1, 200, 2, 1, 64, 128, 32, R=1, has_output_norm=True), 5010),
    ("R2_P64_N128_A32_L160_nonorm", Dims(2, 160, 2, 1, 64, 128, 32, R=2), 5011),
    ("R3_P64_N128_A16_L150", Dims(1, 150, 3, 1, 64, 128, 16, R=3, has_output_norm=True), 5012),
    ("R8_P64_N128_A32_L96", Dims(1, 96, 2, 1, 64, 128, 32, R=8, has_output_norm=True), 5013),
]


@pytest.mark.parametrize("name,d,seed", MIMO_SMALL, ids=[m[0] for m in MIMO_SMALL])
def test_mimo_small(name, d, seed):
    inp = ssm_inputs(d, seed=seed, mimo=True)
    got = gpu_mimo(to_dev(inp), d).cpu().numpy()
    assert_parity(got, oracle_mimo(inp, d), name)


def test_mimo_rank_one_equals_siso_on_gpu():
    d = Dims(2, 90, 4, 2, 32, 64, 16, R=1)
    inp = ssm_inputs(d, seed=5100, mimo=True)
    for k in ("mimo_x", "mimo_z", "mimo_o"):
        inp[k][:] = 1.0
    m_out = gpu_mimo(to_dev(inp), d).cpu().numpy()
    s_inp = dict(inp)
    s_inp["c_bias"] = inp["c_bias"][:, 0].copy()
    s_inp["b_bias"] = inp["b_bias"][:, 0].copy()
    s_out = gpu_siso(to_dev(s_inp), d).cpu().numpy()
    assert_parity(m_out, s_out, "MIMO(R=1) vs SISO on GPU")


def test_mimo_full_b8_l4096_r4_all_heads():
    """B8 L4096 H32 P64 N128 A32 R4 with output norm: every head, every batch
    row (the oracle sharded over host cores)."""
    w = WORKLOADS["mimo_b8_l4096_r4"]
    d = w.dims
    inp = ssm_inputs(d, seed=w.seed, mimo=True)
    got = gpu_mimo(to_dev(inp), d).cpu().numpy()
    del inp
    assert np.isfinite(got).all()
    t0 = time.time()
    ref = oracle_heads("mimo_b8_l4096_r4")
    print(f"[oracle] mimo_b8_l4096_r4 all heads on {pool_size(d.H)} processes: {time.time() - t0:.1f} s",
          flush=True)
    assert_parity(got, ref, "mimo_b8_l4096_r4 all heads")
