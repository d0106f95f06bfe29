"""Plain, slow float64 CPU oracle of the Mamba-3 selective-state forward path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's ``cpu_baseline`` leg may import this module.  The GPU product path
never calls it, shares no code with it and must fail loudly when its HIP
library is missing.

Sources (the oarust 0.8.6 source page ``src/rs/ml/matrix/mamba3.rs`` and the
``ml::matrix`` API index page):

* ``Mamba3PreprocessConfig`` / ``Mamba3PreprocessResult`` docs and
  ``PreprocessGeometry::resolve`` (packed width, bounds) -> :func:`preprocess`.
* ``SsmConfig`` docs, ``Geometry::resolve`` and the ``mamba3_siso`` docs
  (operand order and layouts) -> :func:`siso_scan`.
* ``mamba3_siso_step`` docs (four recurrent states, their layouts)
  -> :func:`siso_step`.
* ``MimoGeometry::resolve`` and the ``mamba3_mimo`` docs -> :func:`mimo_scan`.
* ``mamba3_mimo_step`` docs and ``dispatch_mamba3_mimo_step`` (four states:
  ssm [B,H,P,N], angle [B,H,A], per-rank keys [B,H,R,N] and values
  [B,H,R,P]) -> :func:`mimo_step`.

The pages print no formula of the recurrence.  The definition used here is
read off the docstrings, the operand shapes and the intermediates that the
backward dispatches name (``c_rot``, ``b_rot``, ``theta``, ``qk``, ``decay``,
``gamma``, ``scale``, ``h_previous``).  For each token t of one (batch, head):

    theta_t = theta_{t-1} + dt_t * angle_t              (cumulative angle)
    alpha_t = exp(adt_t)                                (decay)
    lam_t   = sigmoid(trap_t)                           (raw trapezoidal gate)
    gamma_t = lam_t * dt_t
    beta_t  = (1 - lam_t) * dt_t * alpha_t
    K_t     = rot(B_t + b_bias, theta_t)
    Q_t     = rot(C_t + c_bias, theta_t)
    h_t     = alpha_t h_{t-1} + beta_t x_{t-1} K_{t-1}^T + gamma_t x_t K_t^T
    y_t     = h_t Q_t  (+ D x_t)  (* silu(z_t))

with a zero state, zero previous key and zero previous value before the
first token.  rot() turns the split-half pairs (a, a+A), a < A, of the
state axis by +theta_a; coordinates n >= 2A pass through.

Pinned by tests/test_oracle.py: a brute-force materialised quadratic form,
the lambda = 1 and lambda = 0 reductions to a plain exponential-decay scan
(checked with scipy.signal.lfilter), closed forms under constant inputs with
and without rotation, MIMO rank-superposition, flag and invariance checks,
and the preprocess transforms against numpy's logaddexp and the RMS
identity.  Parity against any external Mamba-3 implementation is unpinned:
the conventions listed above are readings of the pages, not printed values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MIMO_NORM_EPS = 1.0e-5  # the MIMO output-norm epsilon the MIMO push constants hard-code


@dataclass(frozen=True)
class SsmConfig:
    """Mirror of ``SsmConfig`` (mamba3.rs): explicit scan geometry and flags."""

    batch_size: int
    sequence_length: int
    num_heads: int
    num_groups: int  # zero means one group per head
    head_dim: int
    state_size: int
    num_rope_angles: int
    mimo_rank: int = 1
    has_z: bool = True
    has_d: bool = True
    has_output_norm: bool = False

    @property
    def groups(self) -> int:
        return self.num_heads if self.num_groups == 0 else self.num_groups


@dataclass(frozen=True)
class PreprocessConfig:
    """Mirror of ``Mamba3PreprocessConfig`` (mamba3.rs)."""

    inner_size: int
    state_size: int
    num_heads: int
    num_rope_angles: int
    num_groups: int
    mimo_rank: int
    epsilon: float
    dt_min: float
    dt_max: float
    a_floor: float


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def softplus(u):
    """Overflow-safe softplus, log(1 + e^u) (``softplus`` entry of the ml::matrix index)."""
    u = _f64(u)
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def sigmoid(u):
    """Logistic function 1 / (1 + e^-u) (``sigmoid`` entry of the ml::matrix index)."""
    u = _f64(u)
    out = np.empty_like(u)
    pos = u >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-u[pos]))
    e = np.exp(u[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(u):
    """z * sigmoid(z) (``silu`` entry of the ml::matrix index)."""
    u = _f64(u)
    return u * sigmoid(u)


# ---------------------------------------------------------------------------
# Preprocess
# ---------------------------------------------------------------------------

def preprocess_width(cfg: PreprocessConfig) -> int:
    """Packed row width 2I + 2GRN + 3H + A (``mamba3_preprocess`` docs)."""
    return (2 * cfg.inner_size + 2 * cfg.num_groups * cfg.mimo_rank * cfg.state_size
            + 3 * cfg.num_heads + cfg.num_rope_angles)


def preprocess(projected, dt_bias, cfg: PreprocessConfig) -> dict:
    """Split and transform one packed projection (``mamba3_preprocess``).

    Column order z | x | B | C | dt | A | trap | angle, the order in which the
    preprocess dispatch binds its outputs (z before x).  B and C rows of
    ``state_size`` values are RMS-normalised without a weight; dt is
    softplus(raw + dt_bias[h]) clamped to [dt_min, dt_max] inclusive; adt is
    -max(softplus(A_raw), a_floor) * dt ("negative A-times-dt log decays",
    "positive floor for the magnitude of the negative A token"); trap and
    angle are passed through raw.
    """
    P = _f64(projected)
    rows, width = P.shape
    I, N, H, A = cfg.inner_size, cfg.state_size, cfg.num_heads, cfg.num_rope_angles
    M = cfg.num_groups * cfg.mimo_rank * N
    if width != preprocess_width(cfg):
        raise ValueError("projected width does not match the configuration")
    off = 0
    z = P[:, off:off + I]; off += I
    x = P[:, off:off + I]; off += I
    b_raw = P[:, off:off + M]; off += M
    c_raw = P[:, off:off + M]; off += M
    dt_raw = P[:, off:off + H]; off += H
    a_raw = P[:, off:off + H]; off += H
    trap = P[:, off:off + H]; off += H
    angle = P[:, off:off + A]; off += A

    def rms_rows(v):
        v = v.reshape(rows, -1, N)
        ms = np.mean(v * v, axis=-1, keepdims=True)
        return (v / np.sqrt(ms + float(np.float32(cfg.epsilon)))).reshape(rows, M)

    dt = np.clip(softplus(dt_raw + _f64(dt_bias)[None, :]),
                 float(np.float32(cfg.dt_min)), float(np.float32(cfg.dt_max)))
    a_mag = np.maximum(softplus(a_raw), float(np.float32(cfg.a_floor)))
    adt = -a_mag * dt
    return {
        "x": x.copy(), "z": z.copy(), "bh": rms_rows(b_raw), "ch": rms_rows(c_raw),
        "dt": dt, "adt": adt, "trap": trap.copy(), "angle": angle.copy(),
    }


# ---------------------------------------------------------------------------
# Scan helpers
# ---------------------------------------------------------------------------

def rotate(v, theta, num_angles: int):
    """Turn split-half pairs (a, a + A) of the last axis by +theta[..., a].

    ``v`` has the state axis last; ``theta`` has ``num_angles`` entries last
    and broadcasts against ``v``'s leading axes.  Coordinates n >= 2A are
    unchanged.  The split-half pairing is the library's ``rope`` convention.
    """
    A = num_angles
    out = v.copy()
    if A == 0:
        return out
    lo = v[..., :A]
    hi = v[..., A:2 * A]
    cos = np.cos(theta)
    sin = np.sin(theta)
    out[..., :A] = lo * cos - hi * sin
    out[..., A:2 * A] = lo * sin + hi * cos
    return out


def _head_selection(cfg: SsmConfig, heads):
    H = cfg.num_heads
    G = cfg.groups
    hs = np.arange(H) if heads is None else np.asarray(heads, dtype=np.int64)
    grp = hs // (H // G)  # heads h*H/G .. share group g
    return hs, grp


# ---------------------------------------------------------------------------
# SISO scan and decode step
# ---------------------------------------------------------------------------

def siso_scan(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, cfg: SsmConfig,
              heads=None, return_states: bool = False):
    """Mamba-3 SISO selective-state recurrence (``mamba3_siso``).

    Operands in the pages' order and layouts: C, B [B,L,G,N]; x, z [B,L,H,P];
    adt, dt, trap [B,L,H]; angle [B,L,A]; c_bias, b_bias [H,N]; D [H].
    Returns out [B,L,H',P] for the selected heads (all heads by default).
    With ``return_states`` also returns the four decode states after the
    last token, in the ``mamba3_siso_step`` layouts.
    """
    Bsz, L = cfg.batch_size, cfg.sequence_length
    P, N, A = cfg.head_dim, cfg.state_size, cfg.num_rope_angles
    hs, grp = _head_selection(cfg, heads)
    Hs = len(hs)
    Cm = _f64(c)[:, :, grp, :]
    Bm = _f64(b)[:, :, grp, :]
    X = _f64(x)[:, :, hs, :]
    Z = _f64(z)[:, :, hs, :]
    ADT = _f64(adt)[:, :, hs]
    DT = _f64(dt)[:, :, hs]
    TRAP = _f64(trap)[:, :, hs]
    ANG = _f64(angle)
    cb = _f64(c_bias)[hs]
    bb = _f64(b_bias)[hs]
    D = _f64(d)[hs]

    theta = np.zeros((Bsz, Hs, A))
    h = np.zeros((Bsz, Hs, P, N))
    k_prev = np.zeros((Bsz, Hs, N))
    v_prev = np.zeros((Bsz, Hs, P))
    out = np.zeros((Bsz, L, Hs, P))
    for t in range(L):
        y, h, theta, k_prev, v_prev = _siso_token(
            Cm[:, t], Bm[:, t], X[:, t], Z[:, t], ADT[:, t], DT[:, t], TRAP[:, t],
            ANG[:, t], cb, bb, D, cfg, h, theta, k_prev, v_prev)
        out[:, t] = y
    if return_states:
        return out, {"ssm_state": h, "angle_state": theta, "k_state": k_prev, "v_state": v_prev}
    return out


def _siso_token(Ct, Bt, Xt, Zt, adt_t, dt_t, trap_t, ang_t, cb, bb, D, cfg, h, theta, k_prev, v_prev):
    """One token of the SISO recurrence for all selected (batch, head) pairs.

    Shapes: Ct, Bt [B,Hs,N]; Xt, Zt [B,Hs,P]; scalars [B,Hs]; ang_t [B,A].
    """
    A = cfg.num_rope_angles
    theta = theta + dt_t[:, :, None] * ang_t[:, None, :]
    alpha = np.exp(adt_t)
    lam = sigmoid(trap_t)
    gamma = lam * dt_t
    beta = (1.0 - lam) * dt_t * alpha
    K = rotate(Bt + bb[None], theta, A)
    Q = rotate(Ct + cb[None], theta, A)
    h = (alpha[..., None, None] * h
         + beta[..., None, None] * v_prev[..., :, None] * k_prev[..., None, :]
         + gamma[..., None, None] * Xt[..., :, None] * K[..., None, :])
    y = np.einsum("bhpn,bhn->bhp", h, Q)
    if cfg.has_d:
        y = y + D[None, :, None] * Xt
    if cfg.has_z:
        y = y * silu(Zt)
    return y, h, theta, K, Xt.copy()


def siso_step(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
              ssm_state, angle_state, k_state, v_state, cfg: SsmConfig, heads=None):
    """One decode token (``mamba3_siso_step``), L == 1.

    States: ssm [B,H,P,N], cumulative angle [B,H,A], previous key [B,H,N]
    (the rotated, bias-added key of the previous token), previous value
    [B,H,P] (the previous token's x).  Returns (out [B,1,H',P], new_states);
    the inputs are not modified.
    """
    if cfg.sequence_length != 1:
        raise ValueError("siso_step requires sequence_length == 1")
    hs, grp = _head_selection(cfg, heads)
    y, h, theta, k, v = _siso_token(
        _f64(c)[:, 0][:, grp], _f64(b)[:, 0][:, grp], _f64(x)[:, 0][:, hs], _f64(z)[:, 0][:, hs],
        _f64(adt)[:, 0][:, hs], _f64(dt)[:, 0][:, hs], _f64(trap)[:, 0][:, hs], _f64(angle)[:, 0],
        _f64(c_bias)[hs], _f64(b_bias)[hs], _f64(d)[hs], cfg,
        _f64(ssm_state)[:, hs], _f64(angle_state)[:, hs], _f64(k_state)[:, hs], _f64(v_state)[:, hs])
    return y[:, None], {"ssm_state": h, "angle_state": theta, "k_state": k, "v_state": v}


# ---------------------------------------------------------------------------
# MIMO scan
# ---------------------------------------------------------------------------

def _mimo_inputs(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                 mimo_x, mimo_z, mimo_o, norm_weight, cfg: SsmConfig, heads):
    """float64 operands of the selected heads; B/C rows r*G + g per rank."""
    R, G = cfg.mimo_rank, cfg.groups
    hs, grp = _head_selection(cfg, heads)
    rows = np.arange(R)[None, :] * G + grp[:, None]  # [Hs, R]
    return dict(
        hs=hs, Cm=_f64(c)[:, :, rows, :], Bm=_f64(b)[:, :, rows, :],  # [B,L,Hs,R,N]
        X=_f64(x)[:, :, hs, :], Z=_f64(z)[:, :, hs, :], ADT=_f64(adt)[:, :, hs], DT=_f64(dt)[:, :, hs],
        TRAP=_f64(trap)[:, :, hs], ANG=_f64(angle),
        cb=_f64(c_bias)[hs], bb=_f64(b_bias)[hs], D=_f64(d)[hs],  # biases [Hs,R,N]
        MX=_f64(mimo_x)[hs], MZ=_f64(mimo_z)[hs], MO=_f64(mimo_o)[hs],  # [Hs,R,P]
        NW=_f64(norm_weight)[hs])  # [Hs,P]


def _mimo_token(m, t, cfg, h, theta, k_prev, v_prev):
    """One token t of the MIMO recurrence for all selected (batch, head) pairs;
    returns (out [B,Hs,P], h, theta, K [B,Hs,R,N], X_r [B,Hs,R,P])."""
    A = cfg.num_rope_angles
    DT, ADT = m["DT"][:, t], m["ADT"][:, t]
    theta = theta + DT[..., None] * m["ANG"][:, t, None, :]
    alpha = np.exp(ADT)
    lam = sigmoid(m["TRAP"][:, t])
    gamma = lam * DT
    beta = (1.0 - lam) * DT * alpha
    Xr = m["X"][:, t, :, None, :] * m["MX"][None]  # [B,Hs,R,P]
    K = rotate(m["Bm"][:, t] + m["bb"][None], theta[:, :, None, :], A)  # [B,Hs,R,N]
    Q = rotate(m["Cm"][:, t] + m["cb"][None], theta[:, :, None, :], A)
    h = (alpha[..., None, None] * h
         + beta[..., None, None] * np.einsum("bhrp,bhrn->bhpn", v_prev, k_prev)
         + gamma[..., None, None] * np.einsum("bhrp,bhrn->bhpn", Xr, K))
    Y = np.einsum("bhpn,bhrn->bhrp", h, Q)
    if cfg.has_d:
        Y = Y + m["D"][None, :, None, None] * Xr
    if cfg.has_z:
        Y = Y * silu(m["Z"][:, t, :, None, :] * m["MZ"][None])
    if cfg.has_output_norm:
        ms = np.mean(Y * Y, axis=-1, keepdims=True)
        Y = Y / np.sqrt(ms + MIMO_NORM_EPS) * m["NW"][None, :, None, :]
    out = np.einsum("hrp,bhrp->bhp", m["MO"], Y)
    return out, h, theta, K, Xr


def mimo_scan(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
              mimo_x, mimo_z, mimo_o, norm_weight, cfg: SsmConfig, heads=None):
    """Shared-state Mamba-3 MIMO scan (``mamba3_mimo``).

    C, B [B,L,R*G,N] with row r*G + g for rank r of group g; biases [H,R,N];
    mimo_x, mimo_z, mimo_o [H,R,P]; norm_weight [H,P] (read only with
    has_output_norm).  Per rank r: X_r = x * mimo_x[h,r], K_r / Q_r from row
    r*G + g; one state per head fed by every rank; per-rank output
    Y_r = h Q_r (+ D X_r), gated by silu(z * mimo_z[h,r]), optionally
    RMS-normalised over P (eps 1e-5) and weighted by norm_weight[h];
    out = sum_r mimo_o[h,r] * Y_r.
    """
    Bsz, L = cfg.batch_size, cfg.sequence_length
    P, N, A, R = cfg.head_dim, cfg.state_size, cfg.num_rope_angles, cfg.mimo_rank
    m = _mimo_inputs(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     mimo_x, mimo_z, mimo_o, norm_weight, cfg, heads)
    Hs = len(m["hs"])
    theta = np.zeros((Bsz, Hs, A))
    h = np.zeros((Bsz, Hs, P, N))
    k_prev = np.zeros((Bsz, Hs, R, N))
    v_prev = np.zeros((Bsz, Hs, R, P))
    out = np.zeros((Bsz, L, Hs, P))
    for t in range(L):
        out[:, t], h, theta, k_prev, v_prev = _mimo_token(m, t, cfg, h, theta, k_prev, v_prev)
    return out


def mimo_step(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
              mimo_x, mimo_z, mimo_o, norm_weight,
              ssm_state, angle_state, k_state, v_state, cfg: SsmConfig, heads=None):
    """One MIMO decode token (``mamba3_mimo_step``), L == 1.

    States: ssm [B,H,P,N], cumulative angle [B,H,A], previous keys
    [B,H,R,N] (each rank's rotated, bias-added key of the previous token),
    previous values [B,H,R,P] (each rank's X_r of the previous token).
    Returns (out [B,1,H',P], new_states); the inputs are not modified.
    """
    if cfg.sequence_length != 1:
        raise ValueError("mimo_step requires sequence_length == 1")
    m = _mimo_inputs(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     mimo_x, mimo_z, mimo_o, norm_weight, cfg, heads)
    hs = m["hs"]
    y, h, theta, k, v = _mimo_token(m, 0, cfg, _f64(ssm_state)[:, hs], _f64(angle_state)[:, hs],
                                    _f64(k_state)[:, hs], _f64(v_state)[:, hs])
    return y[:, None], {"ssm_state": h, "angle_state": theta, "k_state": k, "v_state": v}


# ---------------------------------------------------------------------------
# Parity metric
# ---------------------------------------------------------------------------

def parity_error(got, ref) -> dict:
    """Max error normalised by max(|ref_i|, rms(ref)), plus diagnostics.

    Elementwise relative error is unbounded where an output cancels to near
    zero, so each element's error is scaled by the larger of its own
    magnitude and the root-mean-square of the whole reference tensor.
    """
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if g.shape != o.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {o.shape}")
    nonfinite = int(np.count_nonzero(~np.isfinite(g)))
    if g.size == 0:
        return {"e": 0.0, "max_abs": 0.0, "normwise": 0.0, "nonfinite": nonfinite, "n_rel_over": 0}
    diff = np.abs(g - o)
    rms = float(np.sqrt(np.mean(o * o)))
    denom = np.maximum(np.abs(o), rms)
    denom = np.where(denom > 0, denom, 1.0)
    e = float(np.max(diff / denom)) if nonfinite == 0 else float("inf")
    norm_o = float(np.linalg.norm(o))
    return {
        "e": e,
        "max_abs": float(np.max(diff)),
        "normwise": float(np.linalg.norm(g - o) / norm_o) if norm_o > 0 else float(np.linalg.norm(g - o)),
        "nonfinite": nonfinite,
        "n_rel_over": int(np.count_nonzero(diff > 1e-4 * np.abs(o))),
    }
