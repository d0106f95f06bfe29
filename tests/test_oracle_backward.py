"""Pins for the oracle's adjoints, each against the forward oracle itself
differentiated numerically, or against a closed form.

* central finite differences in float64 of L = sum(dout * mamba3_siso(...))
  along a seeded random direction, separately for each of the eleven
  operands, over several geometries and flag combinations;
* every element of every gradient by finite differences on a tiny case;
* a one-token closed form;
* the block size of the recompute and batch-row selection do not change
  the result;
* preprocess: directional and element-wise finite differences through the
  forward preprocess, missing output gradients as zeros, and zero gradients
  where the dt clamp or the A floor binds.
"""

import numpy as np
import pytest

import oracle as O
from workloads import Dims, output_gradient, preprocess_inputs, preprocess_output_gradients, ssm_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

OPS = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")


def _cfg(d: Dims) -> O.SsmConfig:
    return O.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A, 1, d.has_z, d.has_d, False)


def _inputs64(d: Dims, seed: int) -> dict:
    return {k: v.astype(np.float64) for k, v in ssm_inputs(d, seed=seed, mimo=False).items()}


def _loss(inp: dict, dout, cfg) -> float:
    y = O.siso_scan(*[inp[k] for k in OPS], cfg)
    return float(np.sum(dout * y))


def _fd_dir(inp, dout, cfg, name, v, eps):
    plus = dict(inp)
    minus = dict(inp)
    plus[name] = inp[name] + eps * v
    minus[name] = inp[name] - eps * v
    return (_loss(plus, dout, cfg) - _loss(minus, dout, cfg)) / (2 * eps)


CASES = [
    Dims(2, 9, 4, 2, 3, 6, 2),
    Dims(1, 11, 3, 1, 4, 8, 3, has_z=False),
    Dims(2, 7, 2, 0, 5, 4, 2, has_d=False),
    Dims(1, 10, 2, 1, 3, 5, 0),
    Dims(1, 6, 4, 1, 2, 4, 2, has_z=False, has_d=False),
]


@pytest.mark.parametrize("d", CASES, ids=lambda d: f"B{d.B}L{d.L}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}"
                         f"{'' if d.has_z else 'nz'}{'' if d.has_d else 'nd'}")
def test_siso_backward_matches_directional_finite_differences(d):
    cfg = _cfg(d)
    inp = _inputs64(d, seed=700 + d.L)
    dout = output_gradient(d, seed=710 + d.L).astype(np.float64)
    grads = O.siso_backward(dout, *[inp[k] for k in OPS], cfg, block=4)
    rng = np.random.default_rng(720 + d.L)
    for name in OPS:
        v = rng.standard_normal(inp[name].shape)
        fd = _fd_dir(inp, dout, cfg, name, v, eps=1e-5)
        an = float(np.sum(grads[name] * v))
        scale = max(abs(fd), abs(an), 1e-3)
        assert abs(fd - an) <= 1e-6 * scale, (name, fd, an)
    if not d.has_z:
        assert not np.any(grads["z"])
    if not d.has_d:
        assert not np.any(grads["d"])


def test_siso_backward_every_element_on_a_tiny_case():
    d = Dims(1, 5, 2, 1, 2, 4, 1)
    cfg = _cfg(d)
    inp = _inputs64(d, seed=731)
    dout = output_gradient(d, seed=732).astype(np.float64)
    grads = O.siso_backward(dout, *[inp[k] for k in OPS], cfg, block=2)
    for name in OPS:
        g = grads[name]
        assert g.shape == inp[name].shape, name
        for idx in np.ndindex(*g.shape):
            e = np.zeros_like(inp[name])
            e[idx] = 1.0
            fd = _fd_dir(inp, dout, cfg, name, e, eps=1e-5)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def test_siso_backward_one_token_closed_form():
    # One token from a zero state: h = gamma x K^T, y = gamma (K.Q) x + D x, out = y silu(z).
    d = Dims(1, 1, 1, 1, 3, 4, 1)
    cfg = _cfg(d)
    inp = _inputs64(d, seed=741)
    dout = output_gradient(d, seed=742).astype(np.float64)
    g = O.siso_backward(dout, *[inp[k] for k in OPS], cfg)
    x, z, go = inp["x"][0, 0, 0], inp["z"][0, 0, 0], dout[0, 0, 0]
    dt, trap, D = inp["dt"][0, 0, 0], inp["trap"][0, 0, 0], inp["d"][0]
    lam = 1.0 / (1.0 + np.exp(-trap))
    th = dt * inp["angle"][0, 0, 0]
    rot = np.array([[np.cos(th), -np.sin(th)], [np.sin(th), np.cos(th)]])

    def rotv(v):
        w = v.copy()
        w[[0, 1]] = rot @ v[[0, 1]]
        return w
    K = rotv(inp["b"][0, 0, 0] + inp["b_bias"][0])
    Q = rotv(inp["c"][0, 0, 0] + inp["c_bias"][0])
    qk = float(K @ Q)
    sz = z / (1.0 + np.exp(-z))
    gy = go * sz
    np.testing.assert_allclose(g["x"][0, 0, 0], (lam * dt * qk + D) * gy, rtol=1e-12)
    np.testing.assert_allclose(g["d"][0], float(gy @ x), rtol=1e-12)
    np.testing.assert_allclose(g["adt"][0, 0, 0], 0.0, atol=1e-15)   # no earlier state to decay
    np.testing.assert_allclose(g["trap"][0, 0, 0], lam * (1 - lam) * dt * qk * float(gy @ x), rtol=1e-12)
    # y depends on theta only through K.Q, which a common rotation leaves unchanged
    np.testing.assert_allclose(g["angle"][0, 0], 0.0, atol=1e-13)
    # dK = gamma (x.gy) Q, turned back by -theta onto B + b_bias
    np.testing.assert_allclose(g["b_bias"][0], lam * dt * float(gy @ x) * np.concatenate([rot.T @ Q[[0, 1]], Q[2:]]),
                               rtol=1e-12)
    np.testing.assert_allclose(g["c"][0, 0, 0], lam * dt * float(gy @ x) * np.concatenate([rot.T @ K[[0, 1]], K[2:]]),
                               rtol=1e-12)


def test_siso_backward_block_and_row_selection_invariance():
    d = Dims(3, 13, 2, 1, 3, 4, 2)
    cfg = _cfg(d)
    inp = _inputs64(d, seed=751)
    dout = output_gradient(d, seed=752).astype(np.float64)
    a = O.siso_backward(dout, *[inp[k] for k in OPS], cfg, block=64)
    b = O.siso_backward(dout, *[inp[k] for k in OPS], cfg, block=3)
    for k in OPS:
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-13, err_msg=k)
    one = O.siso_backward(dout, *[inp[k] for k in OPS], cfg, batches=[1])
    for k in ("c", "b", "x", "z", "adt", "dt", "trap", "angle"):
        np.testing.assert_allclose(one[k][0], a[k][1], rtol=1e-12, atol=1e-13, err_msg=k)
    parts = [O.siso_backward(dout, *[inp[k] for k in OPS], cfg, batches=[r]) for r in range(d.B)]
    for k in ("c_bias", "b_bias", "d"):
        np.testing.assert_allclose(sum(p[k] for p in parts), a[k], rtol=1e-11, atol=1e-13, err_msg=k)


# ---------------------------------------------------------------------------
# Preprocess
# ---------------------------------------------------------------------------

def _pcfg(I, N, H, A, G, R=1):
    return O.PreprocessConfig(I, N, H, A, G, R, 1e-5, 1e-3, 0.1, 1e-4)


def _pre_loss(proj, bias, gr, cfg):
    out = O.preprocess(proj, bias, cfg)
    return sum(float(np.sum(out[k] * gr[k])) for k in O.PREPROCESS_OUTPUTS if gr.get(k) is not None)


def _far_from_kinks(proj, bias, cfg, margin=1e-3):
    """Mask of dt / A columns whose softplus is not within ``margin`` (relative) of a bound."""
    I, M, H = cfg.inner_size, cfg.num_groups * cfg.mimo_rank * cfg.state_size, cfg.num_heads
    o_dt = 2 * I + 2 * M
    sp_dt = O.softplus(proj[:, o_dt:o_dt + H] + bias[None])
    sp_a = O.softplus(proj[:, o_dt + H:o_dt + 2 * H])
    ok_dt = (np.abs(sp_dt - cfg.dt_min) > margin * cfg.dt_min) & (np.abs(sp_dt - cfg.dt_max) > margin * cfg.dt_max)
    ok_a = np.abs(sp_a - cfg.a_floor) > margin * cfg.a_floor
    return o_dt, ok_dt, ok_a


@pytest.mark.parametrize("missing", [(), ("z", "angle"), ("x", "bh", "adt")])
def test_preprocess_backward_matches_directional_finite_differences(missing):
    I, N, H, A, G = 6, 8, 3, 2, 2
    cfg = _pcfg(I, N, H, A, G)
    W = O.preprocess_width(cfg)
    rows = 40
    pin = preprocess_inputs(rows, W, H, seed=761)
    proj = pin["projected"].astype(np.float64)
    o_dt = 2 * I + 2 * G * N
    proj[:, o_dt + H:o_dt + 2 * H] -= 9.0          # about a third of the A floors bind
    bias = pin["dt_bias"].astype(np.float64)
    gr = preprocess_output_gradients(rows, I, G * N, H, A, seed=762, missing=missing)
    got = O.preprocess_backward(proj, bias, gr, cfg)
    o_dt, ok_dt, ok_a = _far_from_kinks(proj, bias, cfg)
    assert (~ok_a).sum() == 0 and (~ok_dt).sum() == 0, "seeded inputs sit on a kink"
    sp_dt = O.softplus(proj[:, o_dt:o_dt + H] + bias[None])
    sp_a = O.softplus(proj[:, o_dt + H:o_dt + 2 * H])
    assert np.any(sp_dt < cfg.dt_min) and np.any(sp_dt > cfg.dt_max) and np.any(sp_a < cfg.a_floor)
    rng = np.random.default_rng(763)
    for which in ("projected", "dt_bias"):
        v = rng.standard_normal(proj.shape if which == "projected" else bias.shape)
        eps = 1e-6
        if which == "projected":
            fd = (_pre_loss(proj + eps * v, bias, gr, cfg) - _pre_loss(proj - eps * v, bias, gr, cfg)) / (2 * eps)
        else:
            fd = (_pre_loss(proj, bias + eps * v, gr, cfg) - _pre_loss(proj, bias - eps * v, gr, cfg)) / (2 * eps)
        an = float(np.sum(got[which] * v))
        assert abs(fd - an) <= 1e-6 * max(abs(fd), 1.0), (which, fd, an)
    # clamped dt and floor-bound A columns pass no gradient
    d_dt_cols = got["projected"][:, o_dt:o_dt + H]
    d_a_cols = got["projected"][:, o_dt + H:o_dt + 2 * H]
    assert not np.any(d_dt_cols[(sp_dt < cfg.dt_min) | (sp_dt > cfg.dt_max)])
    assert not np.any(d_a_cols[sp_a < cfg.a_floor])
    np.testing.assert_allclose(got["dt_bias"], d_dt_cols.sum(axis=0), rtol=1e-14, atol=0)
    # copies pass their gradients through unchanged; missing ones are zero
    for k, lo in (("z", 0), ("x", I)):
        ref = np.zeros((rows, I)) if gr[k] is None else gr[k]
        np.testing.assert_array_equal(got["projected"][:, lo:lo + I], ref)


def test_preprocess_backward_every_element_on_a_tiny_case():
    I, N, H, A, G = 2, 4, 2, 1, 1
    cfg = _pcfg(I, N, H, A, G)
    W = O.preprocess_width(cfg)
    rows = 3
    pin = preprocess_inputs(rows, W, H, seed=771)
    proj = pin["projected"].astype(np.float64)
    bias = pin["dt_bias"].astype(np.float64)
    o_dt, ok_dt, ok_a = _far_from_kinks(proj, bias, cfg)
    assert ok_dt.all() and ok_a.all()
    gr = preprocess_output_gradients(rows, I, G * N, H, A, seed=772)
    got = O.preprocess_backward(proj, bias, gr, cfg)
    eps = 1e-6
    for idx in np.ndindex(*proj.shape):
        e = np.zeros_like(proj)
        e[idx] = eps
        fd = (_pre_loss(proj + e, bias, gr, cfg) - _pre_loss(proj - e, bias, gr, cfg)) / (2 * eps)
        assert abs(fd - got["projected"][idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, got["projected"][idx])


# ---------------------------------------------------------------------------
# MIMO
# ---------------------------------------------------------------------------

MOPS = OPS + ("mimo_x", "mimo_z", "mimo_o", "norm_weight")


def _mcfg(d: Dims) -> O.SsmConfig:
    return O.SsmConfig(d.B, d.L, d.H, d.G, d.P, d.N, d.A, d.R, d.has_z, d.has_d, d.has_output_norm)


def _mloss(inp: dict, dout, cfg) -> float:
    return float(np.sum(dout * O.mimo_scan(*[inp[k] for k in MOPS], cfg)))


MCASES = [
    Dims(2, 7, 2, 1, 3, 6, 2, R=2, has_output_norm=True),
    Dims(1, 9, 4, 2, 4, 4, 1, R=3, has_z=False),
    Dims(1, 6, 2, 0, 5, 8, 3, R=2, has_d=False, has_output_norm=True),
    Dims(2, 5, 3, 1, 2, 4, 0, R=1, has_output_norm=True),
    Dims(1, 8, 2, 2, 3, 4, 2, R=4, has_z=False, has_d=False),
]


@pytest.mark.parametrize("d", MCASES, ids=lambda d: f"B{d.B}L{d.L}H{d.H}G{d.G}P{d.P}N{d.N}A{d.A}R{d.R}"
                         f"{'n' if d.has_output_norm else ''}{'' if d.has_z else 'nz'}{'' if d.has_d else 'nd'}")
def test_mimo_backward_matches_directional_finite_differences(d):
    cfg = _mcfg(d)
    inp = {k: v.astype(np.float64) for k, v in ssm_inputs(d, seed=800 + d.L, mimo=True).items()}
    dout = output_gradient(d, seed=810 + d.L).astype(np.float64)
    grads = O.mimo_backward(dout, *[inp[k] for k in MOPS], cfg, block=3)
    rng = np.random.default_rng(820 + d.L)
    for name in MOPS:
        v = rng.standard_normal(inp[name].shape)
        plus, minus = dict(inp), dict(inp)
        plus[name] = inp[name] + 1e-5 * v
        minus[name] = inp[name] - 1e-5 * v
        fd = (_mloss(plus, dout, cfg) - _mloss(minus, dout, cfg)) / 2e-5
        an = float(np.sum(grads[name] * v))
        assert abs(fd - an) <= 1e-6 * max(abs(fd), abs(an), 1e-3), (name, fd, an)
    if not d.has_output_norm:
        assert not np.any(grads["norm_weight"])
    if not d.has_z:
        assert not np.any(grads["z"]) and not np.any(grads["mimo_z"])


def test_mimo_backward_every_element_on_a_tiny_case():
    d = Dims(1, 3, 2, 1, 2, 4, 1, R=2, has_output_norm=True)
    cfg = _mcfg(d)
    inp = {k: v.astype(np.float64) for k, v in ssm_inputs(d, seed=831, mimo=True).items()}
    dout = output_gradient(d, seed=832).astype(np.float64)
    g = O.mimo_backward(dout, *[inp[k] for k in MOPS], cfg)
    for name in MOPS:
        assert g[name].shape == inp[name].shape, name
        for idx in np.ndindex(*g[name].shape):
            plus, minus = dict(inp), dict(inp)
            e = np.zeros_like(inp[name])
            e[idx] = 1e-6   # the norm over P = 2 curves strongly: a smaller step keeps the truncation error down
            plus[name] = inp[name] + e
            minus[name] = inp[name] - e
            fd = (_mloss(plus, dout, cfg) - _mloss(minus, dout, cfg)) / 2e-6
            assert abs(fd - g[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[name][idx])


def test_mimo_backward_rank_one_is_siso_backward():
    d = Dims(2, 11, 4, 2, 3, 6, 2, R=1)
    inp = ssm_inputs(d, seed=841, mimo=True)
    H, P = d.H, d.P
    inp["mimo_x"] = np.ones((H, 1, P), np.float32)
    inp["mimo_z"] = np.ones((H, 1, P), np.float32)
    inp["mimo_o"] = np.ones((H, 1, P), np.float32)
    inp = {k: v.astype(np.float64) for k, v in inp.items()}
    dout = output_gradient(d, seed=842).astype(np.float64)
    gm = O.mimo_backward(dout, *[inp[k] for k in MOPS], _mcfg(d))
    sin = dict(inp)
    sin["c_bias"], sin["b_bias"] = inp["c_bias"][:, 0], inp["b_bias"][:, 0]
    gs = O.siso_backward(dout, *[sin[k] for k in OPS], _cfg(d))
    for k in OPS:
        np.testing.assert_allclose(gm[k].reshape(gs[k].shape), gs[k], rtol=1e-10, atol=1e-12, err_msg=k)
    # with unit weights the MIMO weight gradients are the SISO sums they multiply
    np.testing.assert_allclose(gm["mimo_x"][:, 0], np.sum(gs["x"] * inp["x"], axis=(0, 1)), rtol=1e-10, atol=1e-12)
