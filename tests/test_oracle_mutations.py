"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of ``oracle/m3_oracle.py``
(a dropped term, a wrong sign or index, a swapped order, a transposed
operand) and runs ``tests/test_oracle.py`` against that copy in a fresh
process; mistakes in the adjoints of ``oracle/m3_backward.py`` run
``tests/test_oracle_backward.py``.  The pins must fail for every planted
mistake.  Runs on the CPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

# name -> (text in the oracle, planted replacement), or a list of such pairs
MUTATIONS = {
    "beta_without_decay": ("beta = (1.0 - lam) * dt_t * alpha", "beta = (1.0 - lam) * dt_t"),
    "theta_without_dt": ("theta = theta + dt_t[:, :, None] * ang_t[:, None, :]",
                         "theta = theta + ang_t[:, None, :]"),
    # K and Q rotated by the angle before this token's increment.
    "theta_exclusive_prefix": [
        ("    theta = theta + dt_t[:, :, None] * ang_t[:, None, :]\n",
         "    theta_new = theta + dt_t[:, :, None] * ang_t[:, None, :]\n"),
        ("    return y, h, theta, K, Xt.copy()", "    return y, h, theta_new, K, Xt.copy()")],
    "rotation_sign": ("out[..., :A] = lo * cos - hi * sin", "out[..., :A] = lo * cos + hi * sin"),
    "bias_after_rotation": ("K = rotate(Bt + bb[None], theta, A)", "K = rotate(Bt, theta, A) + bb[None]"),
    "gamma_uses_one_minus_lambda": ("gamma = lam * dt_t\n", "gamma = (1.0 - lam) * dt_t\n"),
    "previous_token_term_dropped": (
        "+ beta[..., None, None] * v_prev[..., :, None] * k_prev[..., None, :]\n", "\n"),
    "gate_before_skip": (
        "    if cfg.has_d:\n        y = y + D[None, :, None] * Xt\n    if cfg.has_z:\n        y = y * silu(Zt)",
        "    if cfg.has_z:\n        y = y * silu(Zt)\n    if cfg.has_d:\n        y = y + D[None, :, None] * Xt"),
    "group_of_head_modulo": ("grp = hs // (H // G)", "grp = hs % G"),
    "mimo_row_order_transposed": ("rows = np.arange(R)[None, :] * G + grp[:, None]",
                                  "rows = grp[:, None] * R + np.arange(R)[None, :]"),
    "mimo_norm_without_eps": ("Y = Y / np.sqrt(ms + MIMO_NORM_EPS)", "Y = Y / np.sqrt(ms)"),
    "preprocess_x_z_swapped": (
        "z = P[:, off:off + I]; off += I\n    x = P[:, off:off + I]; off += I",
        "x = P[:, off:off + I]; off += I\n    z = P[:, off:off + I]; off += I"),
    "preprocess_eps_outside_sqrt": (
        "return (v / np.sqrt(ms + float(np.float32(cfg.epsilon)))).reshape(rows, M)",
        "return (v / (np.sqrt(ms) + float(np.float32(cfg.epsilon)))).reshape(rows, M)"),
    "preprocess_no_a_floor": ("adt = -a_mag * dt", "adt = -softplus(a_raw) * dt"),
    "mimo_step_ignores_previous_keys": ("_f64(k_state)[:, hs], _f64(v_state)[:, hs])",
                                        "0.0 * _f64(k_state)[:, hs], _f64(v_state)[:, hs])"),
    "step_keeps_unrotated_key": ("return y, h, theta, K, Xt.copy()",
                                 "return y, h, theta, Bt + bb[None], Xt.copy()"),
}

# mistakes planted in the adjoints (oracle/m3_backward.py), caught by tests/test_oracle_backward.py
BACKWARD_MUTATIONS = {
    "bwd_previous_token_value_dropped": ("dX[:, t - 1] += beta[:, t, :, None] * hk1", "pass"),
    "bwd_carry_without_decay": ("carry = alpha[:, t, :, None, None] * hbar", "carry = hbar"),
    "bwd_query_gradient_from_previous_state": (
        'dQ[:, t] += np.einsum("bhpn,bhp->bhn", h_t, gy)', 'dQ[:, t] += np.einsum("bhpn,bhp->bhn", h_prev, gy)'),
    "bwd_unrotate_with_plus_theta": ("dKraw = rotate(dK, -theta, A)", "dKraw = rotate(dK, theta, A)"),
    "bwd_theta_sign": ("dQ[..., A:2 * A] * Qm[..., :A] - dQ[..., :A] * Qm[..., A:2 * A])",
                       "dQ[..., :A] * Qm[..., A:2 * A] - dQ[..., A:2 * A] * Qm[..., :A])"),
    "bwd_theta_forward_cumsum": ("tail = np.flip(np.cumsum(np.flip(d_theta, axis=1), axis=1), axis=1)",
                                 "tail = np.cumsum(d_theta, axis=1)"),
    "bwd_dt_without_beta_path": ("d_dt = d_gamma * lam + d_beta * (1.0 - lam) * alpha", "d_dt = d_gamma * lam"),
    "bwd_gate_derivative_without_product_term": ("return s * (1.0 + u * (1.0 - s))", "return s"),
    "bwd_rms_without_projection": ("return (r * (gy - y * np.mean(gy * y, axis=-1, keepdims=True))).reshape(rows, M)",
                                   "return (r * gy).reshape(rows, M)"),
    "bwd_clamp_passes_gradient": ("d_u = np.where(dt_pass, g_dt * sigmoid(u), 0.0)", "d_u = g_dt * sigmoid(u)"),
    "bwd_a_without_softplus_slope": ("d_a = np.where(a_pass, -dt * g[\"adt\"] * sigmoid(a_raw), 0.0)",
                                     "d_a = np.where(a_pass, -dt * g[\"adt\"], 0.0)"),
    "bwd_dt_ignores_adt": ("g_dt = g[\"dt\"] - a_mag * g[\"adt\"]", "g_dt = g[\"dt\"]"),
    "mimo_bwd_norm_without_projection": ("g3 = rinv * (gn - yn * np.mean(gn * yn, axis=-1, keepdims=True))",
                                         "g3 = rinv * gn"),
    "mimo_bwd_gate_without_mimo_z": ("dZ[:, t] += np.sum(du * MZ[None], axis=2)", "dZ[:, t] += np.sum(du, axis=2)"),
    "mimo_bwd_x_weights_ignored": ("dX = np.sum(dXR * MX[None, None], axis=3)", "dX = np.sum(dXR, axis=3)"),
    "mimo_bwd_mimo_o_before_norm": ("dMO += np.sum(g * y4, axis=0)", "dMO += np.sum(g * y3, axis=0)"),
    "mimo_bwd_theta_half": ("dQ[..., A:2 * A] * Qm[..., :A] - dQ[..., :A] * Qm[..., A:2 * A], axis=3)",
                            "dQ[..., A:2 * A] * Qm[..., :A] - dQ[..., :A] * Qm[..., A:2 * A], axis=3) * 0.5"),
    "mimo_bwd_bc_rows_transposed": ("bc_rows = np.arange(R)[None, :] * G + grp[:, None]              # [H, R]",
                                    "bc_rows = grp[:, None] * R + np.arange(R)[None, :]              # [H, R]"),
}


def _run_planted(tmp_path, module, edits, test_file, name):
    src_path = os.path.join(ORACLE, module)
    with open(src_path) as f:
        src = f.read()
    for old, new in edits if isinstance(edits, list) else [edits]:
        assert src.count(old) >= 1, f"mutation site of {name!r} not found in the oracle"
        src = src.replace(old, new, 1)
    dst = tmp_path / "oracle"
    shutil.copytree(ORACLE, dst, ignore=shutil.ignore_patterns("__pycache__"))
    (dst / module).write_text(src)
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}{os.pathsep}{ROOT}")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", test_file)],
        env=env, cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin failed with the mistake {name!r} planted:\n{r.stdout[-2000:]}"
    # The failure must come from an assertion, not from the copy failing to import.
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    _run_planted(tmp_path, "m3_backward.py", BACKWARD_MUTATIONS[name], "test_oracle_backward.py", name)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src_path = os.path.join(ORACLE, "m3_oracle.py")
    with open(src_path) as f:
        src = f.read()
    edits = MUTATIONS[name]
    for old, new in edits if isinstance(edits, list) else [edits]:
        assert src.count(old) >= 1, f"mutation site of {name!r} not found in the oracle"
        src = src.replace(old, new, 1)
    dst = tmp_path / "oracle"
    shutil.copytree(ORACLE, dst, ignore=shutil.ignore_patterns("__pycache__"))
    (dst / "m3_oracle.py").write_text(src)
    env = dict(os.environ, PYTHONPATH=f"{tmp_path}{os.pathsep}{ROOT}")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle.py")],
        env=env, cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin failed with the mistake {name!r} planted:\n{r.stdout[-2000:]}"
    # The failure must come from an assertion, not from the copy failing to import.
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
