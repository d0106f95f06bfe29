"""Pins for the float64 oracle, each against something other than the oracle.

* brute force: the materialised L x L quadratic form built with explicit
  loops, products of decays and complex-number rotation;
* reductions: lambda = 1 and lambda = 0 turn the recurrence into a plain
  exponential-decay filter, checked with scipy.signal.lfilter;
* closed forms: constant inputs give a geometric series, with and without
  a constant rotary angular velocity;
* structure: decode steps continue a scan; MIMO with rank one is SISO;
  MIMO pre-gate outputs superpose SISO runs over rank pairs; flags; head
  permutation and group sharing; A = 0 equals angle = 0;
* preprocess: bit-exact copies, the RMS identity, softplus against
  numpy.logaddexp, clamp and floor bounds.
"""

import cmath
import math

import numpy as np
import pytest
from scipy.signal import lfilter

import oracle as O
from workloads import Dims, decode_states, ssm_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cfg(d: Dims, **kw) -> O.SsmConfig:
    base = dict(batch_size=d.B, sequence_length=d.L, num_heads=d.H, num_groups=d.G,
                head_dim=d.P, state_size=d.N, num_rope_angles=d.A, mimo_rank=d.R,
                has_z=d.has_z, has_d=d.has_d, has_output_norm=d.has_output_norm)
    base.update(kw)
    return O.SsmConfig(**base)


def _siso(inp, cfg, **kw):
    return O.siso_scan(inp["c"], inp["b"], inp["x"], inp["z"], inp["adt"], inp["dt"], inp["trap"],
                       inp["angle"], inp["c_bias"], inp["b_bias"], inp["d"], cfg, **kw)


def _mimo(inp, cfg):
    return O.mimo_scan(inp["c"], inp["b"], inp["x"], inp["z"], inp["adt"], inp["dt"], inp["trap"],
                       inp["angle"], inp["c_bias"], inp["b_bias"], inp["d"], inp["mimo_x"],
                       inp["mimo_z"], inp["mimo_o"], inp["norm_weight"], cfg)


def _lg(u):
    return 1.0 / (1.0 + math.exp(-u))


# ---------------------------------------------------------------------------
# Brute-force quadratic form
# ---------------------------------------------------------------------------

def _brute_quadratic(inp, d: Dims):
    """y[b,t,h,:] = sum_{s<=t} W[t,s] (Q_t . K_s) x_s  (+ D x_t) (* silu z_t).

    W[t,t] = lam_t dt_t and, for s < t,
    W[t,s] = (prod_{r=s+1..t} exp(adt_r)) * (lam_s dt_s + (1 - lam_{s+1}) dt_{s+1}).
    Rotations are done on complex pairs q_a = v_a + i v_{a+A} times e^{i theta_a}.
    """
    B, L, H, G, P, N, A = d.B, d.L, d.H, d.groups, d.P, d.N, d.A
    f = lambda k: np.asarray(inp[k], dtype=np.float64)
    c, b, x, z = f("c"), f("b"), f("x"), f("z")
    adt, dt, trap, ang = f("adt"), f("dt"), f("trap"), f("angle")
    cb, bb, D = f("c_bias"), f("b_bias"), f("d")
    out = np.zeros((B, L, H, P))
    for bi in range(B):
        for h in range(H):
            g = h // (H // G)
            theta = [[sum(dt[bi, s, h] * ang[bi, s, a] for s in range(t + 1)) for a in range(A)]
                     for t in range(L)]

            def rot(v, t):
                w = list(v)
                for a in range(A):
                    zc = complex(v[a], v[a + A]) * cmath.exp(1j * theta[t][a])
                    w[a], w[a + A] = zc.real, zc.imag
                return w

            Qs = [rot(c[bi, t, g] + cb[h], t) for t in range(L)]
            Ks = [rot(b[bi, t, g] + bb[h], t) for t in range(L)]
            lam = [_lg(trap[bi, t, h]) for t in range(L)]
            for t in range(L):
                y = np.zeros(P)
                for s in range(t + 1):
                    if s == t:
                        w = lam[t] * dt[bi, t, h]
                    else:
                        decay = 1.0
                        for r in range(s + 1, t + 1):
                            decay *= math.exp(adt[bi, r, h])
                        w = decay * (lam[s] * dt[bi, s, h] + (1.0 - lam[s + 1]) * dt[bi, s + 1, h])
                    qk = sum(Qs[t][n] * Ks[s][n] for n in range(N))
                    y += w * qk * x[bi, s, h]
                if d.has_d:
                    y += D[h] * x[bi, t, h]
                if d.has_z:
                    zz = z[bi, t, h]
                    y *= zz / (1.0 + np.exp(-zz))
                out[bi, t, h] = y
    return out


@pytest.mark.parametrize("d,seed", [
    (Dims(1, 12, 2, 1, 5, 8, 3), 11),
    (Dims(2, 9, 4, 2, 3, 6, 2, has_z=False), 12),
    (Dims(1, 7, 3, 0, 4, 4, 2, has_d=False), 13),
    (Dims(1, 10, 2, 2, 2, 5, 0), 14),
])
def test_recurrence_matches_brute_quadratic(d, seed):
    inp = ssm_inputs(d, seed=seed)
    # widen the angle so the rotation is far from the identity
    inp["angle"] = (inp["angle"] * 10.0).astype(np.float32)
    got = _siso(inp, _cfg(d))
    ref = _brute_quadratic(inp, d)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


# ---------------------------------------------------------------------------
# lambda = 1 / lambda = 0 reductions to a plain exponential-decay filter
# ---------------------------------------------------------------------------

def _plain_filter_output(alpha, u_in, C, Bv):
    """h_t = alpha h_{t-1} + u_t[p] B_t[n]  via lfilter per (p, n); y_t = h_t C_t."""
    L, P = u_in.shape
    N = Bv.shape[1]
    y = np.zeros((L, P))
    for p in range(P):
        for n in range(N):
            series = lfilter([1.0], [1.0, -alpha], u_in[:, p] * Bv[:, n])
            y[:, p] += series * C[:, n]
    return y


@pytest.mark.parametrize("lam_sign", [+1, -1])
def test_trap_extremes_reduce_to_plain_scan(lam_sign):
    d = Dims(2, 40, 3, 1, 4, 6, 3)
    inp = ssm_inputs(d, seed=21)
    inp["trap"][:] = 40.0 * lam_sign
    inp["angle"][:] = 0.0
    inp["c_bias"][:] = 0.0
    inp["b_bias"][:] = 0.0
    adt_h = np.array([-0.3, -0.05, -1.2], dtype=np.float32)
    inp["adt"][:] = adt_h[None, None, :]
    got = _siso(inp, _cfg(d))
    f = lambda k: np.asarray(inp[k], dtype=np.float64)
    x, z, dt, c, b, D = f("x"), f("z"), f("dt"), f("c"), f("b"), f("d")
    for bi in range(d.B):
        for h in range(d.H):
            alpha = math.exp(float(adt_h[h]))
            if lam_sign > 0:  # h_t = a h_{t-1} + dt_t x_t B_t
                u = dt[bi, :, h, None] * x[bi, :, h]
                Bv = b[bi, :, 0]
            else:  # h_t = a h_{t-1} + a dt_t x_{t-1} B_{t-1}
                u = np.zeros_like(x[bi, :, h])
                u[1:] = alpha * dt[bi, 1:, h, None] * x[bi, :-1, h]
                Bv = np.zeros_like(b[bi, :, 0])
                Bv[1:] = b[bi, :-1, 0]
            y = _plain_filter_output(alpha, u, c[bi, :, 0], Bv)
            y = y + D[h] * x[bi, :, h]
            zz = z[bi, :, h]
            y = y * zz / (1.0 + np.exp(-zz))
            np.testing.assert_allclose(got[bi, :, h], y, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms under constant inputs
# ---------------------------------------------------------------------------

def _constant_inputs(d: Dims, seed: int, omega):
    rng = np.random.default_rng(seed)
    B, L, H, P, N, A = d.B, d.L, d.H, d.P, d.N, d.A
    inp = {
        "x": np.broadcast_to(rng.standard_normal((1, 1, H, P)), (B, L, H, P)),
        "z": np.broadcast_to(rng.standard_normal((1, 1, H, P)), (B, L, H, P)),
        "c": np.broadcast_to(rng.standard_normal((1, 1, 1, N)), (B, L, 1, N)),
        "b": np.broadcast_to(rng.standard_normal((1, 1, 1, N)), (B, L, 1, N)),
        "dt": np.broadcast_to(rng.uniform(0.01, 0.1, (1, 1, H)), (B, L, H)),
        "adt": np.broadcast_to(-rng.uniform(0.01, 0.5, (1, 1, H)), (B, L, H)),
        "trap": np.broadcast_to(rng.standard_normal((1, 1, H)), (B, L, H)),
        "angle": np.broadcast_to(np.asarray(omega, dtype=np.float64).reshape(1, 1, A), (B, L, A)),
        "c_bias": 0.02 * rng.standard_normal((H, N)),
        "b_bias": 0.02 * rng.standard_normal((H, N)),
        "d": rng.standard_normal(H),
    }
    return {k: np.array(v, dtype=np.float64) for k, v in inp.items()}


def _closed_form(inp, d: Dims):
    B, L, H, P, N, A = d.B, d.L, d.H, d.P, d.N, d.A
    out = np.zeros((B, L, H, P))
    for h in range(H):
        dt = inp["dt"][0, 0, h]
        al = math.exp(inp["adt"][0, 0, h])
        lam = _lg(inp["trap"][0, 0, h])
        gam = lam * dt
        cc = gam + (1.0 - lam) * dt
        q = inp["c"][0, 0, 0] + inp["c_bias"][h]
        k = inp["b"][0, 0, 0] + inp["b_bias"][h]
        x = inp["x"][0, 0, h]
        zz = inp["z"][0, 0, h]
        gate = zz / (1.0 + np.exp(-zz))
        for t in range(L):
            coef = 0.0
            for a in range(A):
                w = al * cmath.exp(-1j * dt * inp["angle"][0, 0, a])
                geo = gam + cc * w * (1.0 - w ** t) / (1.0 - w)
                qa = complex(q[a], q[a + A])
                ka = complex(k[a], k[a + A])
                coef += (qa.conjugate() * ka * geo).real
            plain = gam * al ** t + (gam + (1.0 - lam) * dt * al) * (1.0 - al ** t) / (1.0 - al)
            coef += float(np.dot(q[2 * A:], k[2 * A:])) * plain
            out[:, t, h] = (coef * x + inp["d"][h] * x) * gate
    return out


@pytest.mark.parametrize("omega", [
    [0.0, 0.0, 0.0, 0.0],
    [0.7, -1.3, 2.0, 0.05],
])
def test_constant_input_closed_form(omega):
    d = Dims(2, 50, 3, 1, 5, 11, 4)
    inp = _constant_inputs(d, 31, omega)
    got = _siso(inp, _cfg(d))
    ref = _closed_form(inp, d)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Decode steps continue a scan
# ---------------------------------------------------------------------------

def test_steps_continue_a_scan():
    d = Dims(2, 30, 4, 2, 6, 8, 3)
    inp = ssm_inputs(d, seed=41)
    cfg = _cfg(d)
    full = _siso(inp, cfg)
    L1 = 17
    part = {k: (v[:, :L1] if v.ndim >= 3 and v.shape[1] == d.L else v) for k, v in inp.items()}
    _, st = O.siso_scan(*[part[k] for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle",
                                             "c_bias", "b_bias", "d")],
                        _cfg(d, sequence_length=L1), return_states=True)
    cfg1 = _cfg(d, sequence_length=1)
    for t in range(L1, d.L):
        tok = {k: (v[:, t:t + 1] if v.ndim >= 3 and v.shape[1] == d.L else v) for k, v in inp.items()}
        y, st = O.siso_step(*[tok[k] for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle",
                                                "c_bias", "b_bias", "d")],
                            st["ssm_state"], st["angle_state"], st["k_state"], st["v_state"], cfg1)
        np.testing.assert_allclose(y[:, 0], full[:, t], rtol=1e-12, atol=1e-13)
    # the stored previous value is the last token's x, bit for bit
    np.testing.assert_array_equal(st["v_state"], inp["x"][:, -1].astype(np.float64))


# ---------------------------------------------------------------------------
# MIMO structure
# ---------------------------------------------------------------------------

def test_mimo_rank_one_is_siso():
    d = Dims(2, 33, 4, 2, 6, 10, 4, R=1)
    inp = ssm_inputs(d, seed=51, mimo=True)
    inp["mimo_x"][:] = 1.0
    inp["mimo_z"][:] = 1.0
    inp["mimo_o"][:] = 1.0
    cfg = _cfg(d)
    m = _mimo(inp, cfg)
    s_inp = dict(inp)
    s_inp["c_bias"] = inp["c_bias"][:, 0]
    s_inp["b_bias"] = inp["b_bias"][:, 0]
    s = _siso(s_inp, cfg)
    np.testing.assert_allclose(m, s, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("R,G,norm", [(2, 2, False), (3, 1, True), (2, 2, True)])
def test_mimo_superposes_siso_over_rank_pairs(R, G, norm):
    d = Dims(2, 21, 4, G, 5, 8, 3, R=R, has_output_norm=norm)
    inp = ssm_inputs(d, seed=52 + R, mimo=True)
    cfg = _cfg(d)
    got = _mimo(inp, cfg)
    # pre-gate Y_r = sum_r' SISO-core(C rows of rank r, B rows of rank r', x * mimo_x[r'])
    core_cfg = _cfg(d, mimo_rank=1, has_z=False, has_d=False, has_output_norm=False)
    f = lambda k: np.asarray(inp[k], dtype=np.float64)
    x, z = f("x"), f("z")
    Y = np.zeros((d.B, d.L, d.H, R, d.P))
    for r in range(R):
        for rp in range(R):
            s_inp = dict(inp)
            s_inp["c"] = f("c")[:, :, r * G:(r + 1) * G]
            s_inp["b"] = f("b")[:, :, rp * G:(rp + 1) * G]
            s_inp["x"] = x * f("mimo_x")[None, None, :, rp, :]
            s_inp["c_bias"] = f("c_bias")[:, r]
            s_inp["b_bias"] = f("b_bias")[:, rp]
            Y[:, :, :, r] += _siso(s_inp, core_cfg)
    Xr = x[:, :, :, None, :] * f("mimo_x")[None, None]
    Y = Y + f("d")[None, None, :, None, None] * Xr
    Zr = z[:, :, :, None, :] * f("mimo_z")[None, None]
    Y = Y * Zr / (1.0 + np.exp(-Zr))
    if norm:
        Y = Y / np.sqrt(np.mean(Y ** 2, axis=-1, keepdims=True) + 1e-5) * f("norm_weight")[None, None, :, None, :]
    ref = np.sum(f("mimo_o")[None, None] * Y, axis=3)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


MIMO15 = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d",
          "mimo_x", "mimo_z", "mimo_o", "norm_weight")


def test_mimo_steps_from_zero_states_equal_the_scan():
    d = Dims(2, 12, 4, 2, 5, 8, 3, R=3, has_output_norm=True)
    inp = ssm_inputs(d, seed=53, mimo=True)
    full = _mimo(inp, _cfg(d))
    cfg1 = _cfg(d, sequence_length=1)
    st = {"ssm_state": np.zeros((d.B, d.H, d.P, d.N)), "angle_state": np.zeros((d.B, d.H, d.A)),
          "k_state": np.zeros((d.B, d.H, d.R, d.N)), "v_state": np.zeros((d.B, d.H, d.R, d.P))}
    for t in range(d.L):
        tok = {k: (v[:, t:t + 1] if v.ndim >= 3 and v.shape[1] == d.L else v) for k, v in inp.items()}
        y, st = O.mimo_step(*[tok[k] for k in MIMO15], st["ssm_state"], st["angle_state"],
                            st["k_state"], st["v_state"], cfg1)
        np.testing.assert_allclose(y[:, 0], full[:, t], rtol=1e-12, atol=1e-13)
    # the stored previous values are the last token's x * mimo_x per rank
    xr = inp["x"][:, -1, :, None, :].astype(np.float64) * inp["mimo_x"][None].astype(np.float64)
    np.testing.assert_array_equal(st["v_state"], xr)


def test_mimo_step_rank_one_is_siso_step():
    d = Dims(3, 1, 4, 2, 6, 10, 4, R=1)
    inp = ssm_inputs(d, seed=54, mimo=True)
    for k in ("mimo_x", "mimo_z", "mimo_o"):
        inp[k][:] = 1.0
    st = decode_states(d, seed=55)
    cfg = _cfg(d)
    y_m, st_m = O.mimo_step(*[inp[k] for k in MIMO15], st["ssm_state"], st["angle_state"],
                            st["k_state"][:, :, None], st["v_state"][:, :, None], cfg)
    s_inp = dict(inp)
    s_inp["c_bias"] = inp["c_bias"][:, 0]
    s_inp["b_bias"] = inp["b_bias"][:, 0]
    y_s, st_s = O.siso_step(*[s_inp[k] for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle",
                                                  "c_bias", "b_bias", "d")],
                            st["ssm_state"], st["angle_state"], st["k_state"], st["v_state"], cfg)
    np.testing.assert_allclose(y_m, y_s, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st_m["ssm_state"], st_s["ssm_state"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st_m["k_state"][:, :, 0], st_s["k_state"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(st_m["v_state"][:, :, 0], st_s["v_state"])
    np.testing.assert_array_equal(st_m["angle_state"], st_s["angle_state"])


# ---------------------------------------------------------------------------
# Flags and invariances
# ---------------------------------------------------------------------------

def test_flags():
    d = Dims(1, 25, 3, 1, 4, 8, 2)
    inp = ssm_inputs(d, seed=61)
    on = _siso(inp, _cfg(d))
    no_z = _siso(inp, _cfg(d, has_z=False))
    zz = inp["z"].astype(np.float64)
    np.testing.assert_allclose(on, no_z * zz / (1.0 + np.exp(-zz)), rtol=1e-12, atol=1e-14)
    no_d = _siso(inp, _cfg(d, has_d=False))
    inp2 = dict(inp)
    inp2["d"] = inp["d"] * 7.0
    np.testing.assert_array_equal(no_d, _siso(inp2, _cfg(d, has_d=False)))
    zero = dict(inp)
    for k in ("c", "b", "c_bias", "b_bias"):
        zero[k] = np.zeros_like(inp[k])
    y0 = _siso(zero, _cfg(d))
    x = inp["x"].astype(np.float64)
    np.testing.assert_allclose(y0, inp["d"].astype(np.float64)[None, None, :, None] * x * zz / (1.0 + np.exp(-zz)),
                               rtol=1e-14, atol=1e-15)


def test_head_permutation_and_group_sharing():
    d = Dims(2, 19, 4, 0, 5, 6, 2)  # one group per head
    inp = ssm_inputs(d, seed=71)
    base = _siso(inp, _cfg(d))
    perm = np.array([2, 0, 3, 1])
    pin = dict(inp)
    for k in ("x", "z"):
        pin[k] = inp[k][:, :, perm]
    for k in ("adt", "dt", "trap"):
        pin[k] = inp[k][:, :, perm]
    for k in ("c", "b"):
        pin[k] = inp[k][:, :, perm]
    for k in ("c_bias", "b_bias", "d"):
        pin[k] = inp[k][perm]
    np.testing.assert_array_equal(_siso(pin, _cfg(d)), base[:, :, perm])
    # two heads of one group with identical per-head inputs give identical outputs
    d2 = Dims(1, 15, 4, 2, 3, 6, 2)
    i2 = ssm_inputs(d2, seed=72)
    for k in ("x", "z", "adt", "dt", "trap"):
        i2[k][:, :, 1] = i2[k][:, :, 0]
    for k in ("c_bias", "b_bias", "d"):
        i2[k][1] = i2[k][0]
    y = _siso(i2, _cfg(d2))
    np.testing.assert_array_equal(y[:, :, 1], y[:, :, 0])
    assert not np.allclose(y[:, :, 2], y[:, :, 0])


def test_no_angles_equals_zero_angle():
    d = Dims(1, 20, 2, 1, 4, 8, 3)
    inp = ssm_inputs(d, seed=81)
    zero = dict(inp)
    zero["angle"] = np.zeros_like(inp["angle"])
    y_zero = _siso(zero, _cfg(d))
    noa = dict(inp)
    noa["angle"] = np.zeros((d.B, d.L, 0), dtype=np.float32)
    y_noa = _siso(noa, _cfg(d, num_rope_angles=0))
    np.testing.assert_allclose(y_noa, y_zero, rtol=0, atol=0)


def test_rotation_preserves_norm_and_passes_tail():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((7, 16))
    th = rng.uniform(-4, 4, (7, 5))
    w = O.rotate(v, th, 5)
    np.testing.assert_allclose(np.linalg.norm(w, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-14)
    np.testing.assert_array_equal(w[:, 10:], v[:, 10:])
    # a quarter turn maps (1, 0) -> (0, 1) in pair (a, a + A)
    e = np.zeros(4)
    e[0] = 1.0
    np.testing.assert_allclose(O.rotate(e, np.array([math.pi / 2, 0.0]), 2), [0, 0, 1, 0], atol=1e-16)


# ---------------------------------------------------------------------------
# Preprocess
# ---------------------------------------------------------------------------

def _pcfg(**kw):
    base = dict(inner_size=12, state_size=8, num_heads=3, num_rope_angles=2, num_groups=2,
                mimo_rank=2, epsilon=1e-5, dt_min=1e-3, dt_max=0.1, a_floor=1e-4)
    base.update(kw)
    return O.PreprocessConfig(**base)


def test_preprocess_transforms():
    cfg = _pcfg()
    W = O.preprocess_width(cfg)
    assert W == 2 * 12 + 2 * 2 * 2 * 8 + 3 * 3 + 2
    rng = np.random.default_rng(91)
    rows = 37
    proj = (3.0 * rng.standard_normal((rows, W))).astype(np.float32)
    proj[0, 2 * 12:2 * 12 + 8] = 0.0  # an all-zero B row
    dtb = rng.standard_normal(3).astype(np.float32)
    out = O.preprocess(proj, dtb, cfg)
    I, M, H = 12, 32, 3
    np.testing.assert_array_equal(out["z"], proj[:, :I])
    np.testing.assert_array_equal(out["x"], proj[:, I:2 * I])
    off = 2 * I + 2 * M + 2 * H
    np.testing.assert_array_equal(out["trap"], proj[:, off:off + H])
    np.testing.assert_array_equal(out["angle"], proj[:, off + H:])
    eps = float(np.float32(1e-5))
    for name, start in (("bh", 2 * I), ("ch", 2 * I + M)):
        raw = proj[:, start:start + M].astype(np.float64).reshape(rows, 4, 8)
        ms = np.mean(raw ** 2, axis=-1)
        got = out[name].reshape(rows, 4, 8)
        np.testing.assert_allclose(np.mean(got ** 2, axis=-1), ms / (ms + eps), rtol=1e-12, atol=1e-300)
        # direction unchanged: got is a positive multiple of raw
        np.testing.assert_allclose(got * np.sqrt(ms + eps)[..., None], raw, rtol=1e-12, atol=1e-300)
    dt_raw = proj[:, 2 * I + 2 * M:2 * I + 2 * M + H].astype(np.float64)
    sp = np.logaddexp(0.0, dt_raw + dtb.astype(np.float64))
    lo, hi = float(np.float32(1e-3)), float(np.float32(0.1))
    np.testing.assert_allclose(out["dt"], np.minimum(np.maximum(sp, lo), hi), rtol=1e-14)
    assert np.all(out["dt"] >= lo) and np.all(out["dt"] <= hi)
    assert np.any(out["dt"] == lo) and np.any(out["dt"] == hi) and np.any((out["dt"] > lo) & (out["dt"] < hi))
    a_raw = proj[:, 2 * I + 2 * M + H:2 * I + 2 * M + 2 * H].astype(np.float64)
    mag = np.maximum(np.logaddexp(0.0, a_raw), float(np.float32(1e-4)))
    np.testing.assert_allclose(out["adt"], -mag * out["dt"], rtol=1e-14)
    assert np.all(out["adt"] <= -float(np.float32(1e-4)) * out["dt"] * (1 - 1e-15))


def test_preprocess_floor_binds():
    cfg = _pcfg(a_floor=0.5)
    W = O.preprocess_width(cfg)
    proj = np.full((2, W), -30.0, dtype=np.float32)  # softplus(-30) ~ 1e-13 < floor
    out = O.preprocess(proj, np.zeros(3, np.float32), cfg)
    np.testing.assert_allclose(out["adt"], -0.5 * out["dt"], rtol=1e-15)
    np.testing.assert_allclose(out["dt"], float(np.float32(1e-3)))


def test_softplus_and_sigmoid_reference_values():
    u = np.array([-800.0, -30.0, -1.0, 0.0, 1e-8, 2.5, 40.0, 800.0])
    np.testing.assert_allclose(O.softplus(u), np.logaddexp(0.0, u), rtol=1e-15, atol=1e-300)
    assert O.softplus(np.array([0.0]))[0] == math.log(2.0)
    from scipy.special import expit
    np.testing.assert_allclose(O.sigmoid(u), expit(u), rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------------------
# Parity metric
# ---------------------------------------------------------------------------

def test_parity_metric():
    ref = np.array([1.0, -2.0, 0.0, 1e-9])
    rms = math.sqrt(np.mean(ref ** 2))
    e = O.parity_error(ref + np.array([0, 2e-4, 0, 1e-5]), ref)
    assert math.isclose(e["e"], max(1e-4, 1e-5 / rms), rel_tol=1e-9)
    bad = O.parity_error(np.array([np.nan, 0, 0, 0]), ref)
    assert bad["nonfinite"] == 1 and bad["e"] == float("inf")
    with pytest.raises(ValueError):
        O.parity_error(np.zeros(3), np.zeros(4))
