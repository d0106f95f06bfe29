"""Plain float64 CPU adjoints of the Mamba-3 SISO and MIMO scans and of the preprocess.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test
suite, the smoke check and the benchmark's ``cpu_baseline`` leg may import
it, and the GPU product path never calls it.

Sources (the oarust 0.8.6 source page ``src/rs/ml/matrix/mamba3.rs``):

* ``mamba3_siso_backward`` docs and ``SsmBackward``: eleven gradients, one
  per forward operand (C, B, x, z, adt, dt, trap, angle, c_bias, b_bias, D),
  each in its operand's layout -> :func:`siso_backward`.
* ``mamba3_mimo_backward`` docs and ``Mamba3MimoBackward``: fifteen gradients,
  the eleven of the SISO scan plus mimo_x, mimo_z, mimo_o and norm_weight
  -> :func:`mimo_backward`.
* ``mamba3_preprocess_backward`` docs and ``Mamba3PreprocessBackward``: the
  gradients of ``projected`` and ``dt_bias`` from the gradients of the
  preprocess outputs; an output without a gradient counts as zero (the
  autograd arm of the preprocess node fills zeros) -> :func:`preprocess_backward`.

The pages print no adjoint formulas.  A gradient is the derivative of the
forward that :mod:`oracle.m3_oracle` defines, so this module is that
forward's reverse-mode derivative written out token by token: the forward
recurrence is re-run, then a reverse sweep carries the adjoint of the state
h_t and turns it into the adjoints of every coefficient, key, query and
input, in the order the forward formed them.  Where the forward has a kink
(the dt clamp, the a_floor maximum) the gradient flows through the branch
whose value the forward returned, the unclamped one on a tie.

Pinned by tests/test_oracle_backward.py against central finite differences
of the forward oracle in float64 (directional derivatives for every operand
and element-wise checks on tiny cases) and against closed forms.
"""

from __future__ import annotations

import numpy as np

from .m3_oracle import PreprocessConfig, SsmConfig, _f64, preprocess_width, rotate, sigmoid, silu, softplus


def _dsilu(u):
    """d/du of u * sigmoid(u)."""
    s = sigmoid(u)
    return s * (1.0 + u * (1.0 - s))


def siso_backward(dout, c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, cfg: SsmConfig,
                  batches=None, block: int = 64) -> dict:
    """Gradients of sum(dout * mamba3_siso(...)) with respect to all eleven operands.

    Layouts as the forward operands: C, B [B,L,G,N]; x, z [B,L,H,P]; adt,
    dt, trap [B,L,H]; angle [B,L,A]; c_bias, b_bias [H,N]; D [H].  With
    ``batches`` only those batch rows are taken (every per-row gradient has
    the selected rows only, and the bias and D gradients sum over them).
    The reverse sweep re-runs the forward of ``block`` tokens at a time from
    a stored state instead of keeping every state.
    """
    L = cfg.sequence_length
    H, G = cfg.num_heads, cfg.groups
    P, N, A = cfg.head_dim, cfg.state_size, cfg.num_rope_angles
    rows = np.arange(cfg.batch_size) if batches is None else np.asarray(batches, dtype=np.int64)
    hs = np.arange(H)
    grp = hs // (H // G)
    Cm = _f64(c)[rows][:, :, grp, :]       # [B',L,H,N], each head's group row
    Bm = _f64(b)[rows][:, :, grp, :]
    X = _f64(x)[rows]                      # [B',L,H,P]
    Z = _f64(z)[rows]
    GO = _f64(dout)[rows]
    ADT = _f64(adt)[rows]                  # [B',L,H]
    DT = _f64(dt)[rows]
    TRAP = _f64(trap)[rows]
    ANG = _f64(angle)[rows]                # [B',L,A]
    cb = _f64(c_bias)
    bb = _f64(b_bias)
    D = _f64(d) if cfg.has_d else np.zeros(H)

    # forward coefficients of every token
    theta = np.cumsum(DT[..., None] * ANG[:, :, None, :], axis=1)   # [B',L,H,A]
    alpha = np.exp(ADT)
    lam = sigmoid(TRAP)
    gamma = lam * DT
    beta = (1.0 - lam) * DT * alpha
    K = rotate(Bm + bb[None, None], theta, A)                       # [B',L,H,N]
    Qm = rotate(Cm + cb[None, None], theta, A)

    def outer(v, k):
        return v[..., :, None] * k[..., None, :]

    def advance(h, t):
        h = alpha[:, t, :, None, None] * h + gamma[:, t, :, None, None] * outer(X[:, t], K[:, t])
        if t > 0:
            h = h + beta[:, t, :, None, None] * outer(X[:, t - 1], K[:, t - 1])
        return h

    # forward sweep: the state before each block
    nb = (L + block - 1) // block
    starts = []
    h = np.zeros((len(rows), H, P, N))
    for t in range(L):
        if t % block == 0:
            starts.append(h.copy())
        h = advance(h, t)

    dX = np.zeros_like(X)
    dZ = np.zeros_like(Z)
    dK = np.zeros_like(K)
    dQ = np.zeros_like(Qm)
    d_alpha = np.zeros_like(ADT)
    d_beta = np.zeros_like(ADT)
    d_gamma = np.zeros_like(ADT)
    dD = np.zeros(H)
    carry = np.zeros((len(rows), H, P, N))   # alpha_{t+1} times the adjoint of h_{t+1}
    for blk in reversed(range(nb)):
        t0, t1 = blk * block, min(L, (blk + 1) * block)
        hist = [starts[blk]]                   # hist[i] = h_{t0 + i - 1}
        for t in range(t0, t1):
            hist.append(advance(hist[-1], t))
        for t in reversed(range(t0, t1)):
            h_t, h_prev = hist[t - t0 + 1], hist[t - t0]
            y_ssm = np.einsum("bhpn,bhn->bhp", h_t, Qm[:, t])
            gy = GO[:, t]
            if cfg.has_z:
                y_pre = y_ssm + D[None, :, None] * X[:, t]
                dZ[:, t] = gy * y_pre * _dsilu(Z[:, t])
                gy = gy * silu(Z[:, t])
            if cfg.has_d:
                dD += np.sum(gy * X[:, t], axis=(0, 2))
                dX[:, t] += D[None, :, None] * gy
            hbar = carry + outer(gy, Qm[:, t])       # adjoint of h_t
            dQ[:, t] += np.einsum("bhpn,bhp->bhn", h_t, gy)
            d_alpha[:, t] = np.sum(hbar * h_prev, axis=(2, 3))
            hk = np.einsum("bhpn,bhn->bhp", hbar, K[:, t])
            d_gamma[:, t] = np.sum(X[:, t] * hk, axis=2)
            dX[:, t] += gamma[:, t, :, None] * hk
            dK[:, t] += gamma[:, t, :, None] * np.einsum("bhpn,bhp->bhn", hbar, X[:, t])
            if t > 0:
                hk1 = np.einsum("bhpn,bhn->bhp", hbar, K[:, t - 1])
                d_beta[:, t] = np.sum(X[:, t - 1] * hk1, axis=2)
                dX[:, t - 1] += beta[:, t, :, None] * hk1
                dK[:, t - 1] += beta[:, t, :, None] * np.einsum("bhpn,bhp->bhn", hbar, X[:, t - 1])
            carry = alpha[:, t, :, None, None] * hbar

    # scalar chain: alpha = e^adt, beta = (1 - lam) dt alpha, gamma = lam dt, lam = sigmoid(trap)
    d_adt = alpha * (d_alpha + d_beta * (1.0 - lam) * DT)
    d_lam = d_gamma * DT - d_beta * DT * alpha
    d_dt = d_gamma * lam + d_beta * (1.0 - lam) * alpha
    d_trap = d_lam * lam * (1.0 - lam)

    # rotation: K = rot(B + b_bias, theta), Q = rot(C + c_bias, theta), theta_t = sum_{s<=t} dt_s angle_s
    dKraw = rotate(dK, -theta, A)
    dQraw = rotate(dQ, -theta, A)
    d_angle = np.zeros_like(ANG)
    if A > 0:
        d_theta = (dK[..., A:2 * A] * K[..., :A] - dK[..., :A] * K[..., A:2 * A]
                   + dQ[..., A:2 * A] * Qm[..., :A] - dQ[..., :A] * Qm[..., A:2 * A])
        tail = np.flip(np.cumsum(np.flip(d_theta, axis=1), axis=1), axis=1)   # sum over s >= t
        d_dt = d_dt + np.sum(tail * ANG[:, :, None, :], axis=3)
        d_angle = np.sum(DT[..., None] * tail, axis=2)

    d_b = np.zeros((len(rows), L, G, N))
    d_c = np.zeros((len(rows), L, G, N))
    for h in range(H):
        d_b[:, :, grp[h]] += dKraw[:, :, h]
        d_c[:, :, grp[h]] += dQraw[:, :, h]
    return {
        "c": d_c, "b": d_b, "x": dX, "z": dZ, "adt": d_adt, "dt": d_dt, "trap": d_trap,
        "angle": d_angle, "c_bias": dQraw.sum(axis=(0, 1)), "b_bias": dKraw.sum(axis=(0, 1)),
        "d": dD if cfg.has_d else np.zeros(H),
    }


PREPROCESS_OUTPUTS = ("x", "z", "bh", "ch", "dt", "adt", "trap", "angle")


def preprocess_backward(projected, dt_bias, grads: dict, cfg: PreprocessConfig) -> dict:
    """Gradients of ``projected`` [rows, W] and ``dt_bias`` [H] (``mamba3_preprocess_backward``).

    ``grads`` maps preprocess output names (x, z, bh, ch, dt, adt, trap,
    angle) to their gradients; a missing name counts as zero.  Returns
    {"projected": [rows, W], "dt_bias": [H]}.
    """
    Pm = _f64(projected)
    rows, width = Pm.shape
    I, N, H, A = cfg.inner_size, cfg.state_size, cfg.num_heads, cfg.num_rope_angles
    M = cfg.num_groups * cfg.mimo_rank * N
    if width != preprocess_width(cfg):
        raise ValueError("projected width does not match the configuration")
    shapes = {"x": I, "z": I, "bh": M, "ch": M, "dt": H, "adt": H, "trap": H, "angle": A}
    g = {k: (_f64(grads[k]).reshape(rows, shapes[k]) if grads.get(k) is not None
             else np.zeros((rows, shapes[k]))) for k in PREPROCESS_OUTPUTS}
    o_b = 2 * I
    o_c = o_b + M
    o_dt = o_c + M
    o_a = o_dt + H
    b_raw = Pm[:, o_b:o_b + M]
    c_raw = Pm[:, o_c:o_c + M]
    u = Pm[:, o_dt:o_dt + H] + _f64(dt_bias)[None, :]
    a_raw = Pm[:, o_a:o_a + H]
    eps = float(np.float32(cfg.epsilon))
    lo, hi = float(np.float32(cfg.dt_min)), float(np.float32(cfg.dt_max))
    floor = float(np.float32(cfg.a_floor))

    def rms_backward(v, gy):
        # y = v r with r = (mean(v^2) + eps)^-1/2:  dv = r (gy - y mean(gy y))
        v = v.reshape(rows, -1, N)
        gy = gy.reshape(rows, -1, N)
        r = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
        y = v * r
        return (r * (gy - y * np.mean(gy * y, axis=-1, keepdims=True))).reshape(rows, M)

    sp_dt = softplus(u)
    dt = np.clip(sp_dt, lo, hi)
    dt_pass = (sp_dt >= lo) & (sp_dt <= hi)
    sp_a = softplus(a_raw)
    a_pass = sp_a >= floor
    a_mag = np.maximum(sp_a, floor)
    g_dt = g["dt"] - a_mag * g["adt"]                      # adt = -a_mag dt
    d_u = np.where(dt_pass, g_dt * sigmoid(u), 0.0)
    d_a = np.where(a_pass, -dt * g["adt"] * sigmoid(a_raw), 0.0)

    d_proj = np.concatenate([g["z"], g["x"], rms_backward(b_raw, g["bh"]), rms_backward(c_raw, g["ch"]),
                             d_u, d_a, g["trap"], g["angle"]], axis=1)
    return {"projected": d_proj, "dt_bias": d_u.sum(axis=0)}


def mimo_backward(dout, c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                  mimo_x, mimo_z, mimo_o, norm_weight, cfg: SsmConfig, batches=None, block: int = 64) -> dict:
    """Gradients of sum(dout * mamba3_mimo(...)) with respect to all fifteen operands.

    Layouts as the forward operands (``mamba3_mimo`` docs): C, B [B,L,R*G,N]
    with row r*G + g; x, z [B,L,H,P]; adt, dt, trap [B,L,H]; angle [B,L,A];
    c_bias, b_bias [H,R,N]; D [H]; mimo_x, mimo_z, mimo_o [H,R,P];
    norm_weight [H,P] (zero gradient without the norm).  ``batches`` and
    ``block`` as for :func:`siso_backward`.
    """
    from .m3_oracle import MIMO_NORM_EPS
    L = cfg.sequence_length
    H, G, R = cfg.num_heads, cfg.groups, cfg.mimo_rank
    P, N, A = cfg.head_dim, cfg.state_size, cfg.num_rope_angles
    rows = np.arange(cfg.batch_size) if batches is None else np.asarray(batches, dtype=np.int64)
    hs = np.arange(H)
    grp = hs // (H // G)
    bc_rows = np.arange(R)[None, :] * G + grp[:, None]              # [H, R]
    Cm = _f64(c)[rows][:, :, bc_rows, :]                             # [B',L,H,R,N]
    Bm = _f64(b)[rows][:, :, bc_rows, :]
    X = _f64(x)[rows]                                                # [B',L,H,P]
    Z = _f64(z)[rows]
    GO = _f64(dout)[rows]
    ADT = _f64(adt)[rows]
    DT = _f64(dt)[rows]
    TRAP = _f64(trap)[rows]
    ANG = _f64(angle)[rows]
    cb = _f64(c_bias)                                                # [H,R,N]
    bb = _f64(b_bias)
    D = _f64(d) if cfg.has_d else np.zeros(H)
    MX, MZ, MO = _f64(mimo_x), _f64(mimo_z), _f64(mimo_o)            # [H,R,P]
    NW = _f64(norm_weight)                                           # [H,P]

    theta = np.cumsum(DT[..., None] * ANG[:, :, None, :], axis=1)   # [B',L,H,A]
    th_r = theta[:, :, :, None, :]                                   # broadcast over ranks
    alpha = np.exp(ADT)
    lam = sigmoid(TRAP)
    gamma = lam * DT
    beta = (1.0 - lam) * DT * alpha
    K = rotate(Bm + bb[None, None], th_r, A)                         # [B',L,H,R,N]
    Qm = rotate(Cm + cb[None, None], th_r, A)
    XR = X[:, :, :, None, :] * MX[None, None]                        # [B',L,H,R,P]

    def rank_outer(v, k):                                            # sum_r v_r k_r^T
        return np.einsum("bhrp,bhrn->bhpn", v, k)

    def advance(h, t):
        h = alpha[:, t, :, None, None] * h + gamma[:, t, :, None, None] * rank_outer(XR[:, t], K[:, t])
        if t > 0:
            h = h + beta[:, t, :, None, None] * rank_outer(XR[:, t - 1], K[:, t - 1])
        return h

    nb = (L + block - 1) // block
    starts = []
    h = np.zeros((len(rows), H, P, N))
    for t in range(L):
        if t % block == 0:
            starts.append(h.copy())
        h = advance(h, t)

    dXR = np.zeros_like(XR)
    dZ = np.zeros_like(Z)
    dK = np.zeros_like(K)
    dQ = np.zeros_like(Qm)
    d_alpha = np.zeros_like(ADT)
    d_beta = np.zeros_like(ADT)
    d_gamma = np.zeros_like(ADT)
    dD = np.zeros(H)
    dMZ = np.zeros_like(MZ)
    dMO = np.zeros_like(MO)
    dNW = np.zeros_like(NW)
    carry = np.zeros((len(rows), H, P, N))
    for blk in reversed(range(nb)):
        t0, t1 = blk * block, min(L, (blk + 1) * block)
        hist = [starts[blk]]
        for t in range(t0, t1):
            hist.append(advance(hist[-1], t))
        for t in reversed(range(t0, t1)):
            h_t, h_prev = hist[t - t0 + 1], hist[t - t0]
            # forward epilogue of this token, stage by stage
            y1 = np.einsum("bhpn,bhrn->bhrp", h_t, Qm[:, t])           # [B',H,R,P]
            y2 = y1 + D[None, :, None, None] * XR[:, t]
            u = Z[:, t, :, None, :] * MZ[None]
            y3 = y2 * silu(u) if cfg.has_z else y2
            if cfg.has_output_norm:
                rinv = 1.0 / np.sqrt(np.mean(y3 * y3, axis=-1, keepdims=True) + MIMO_NORM_EPS)
                yn = y3 * rinv
                y4 = yn * NW[None, :, None, :]
            else:
                y4 = y3
            # out = sum_r mimo_o * y4
            g = GO[:, t][:, :, None, :]                                 # [B',H,1,P]
            dMO += np.sum(g * y4, axis=0)
            g4 = g * MO[None]
            if cfg.has_output_norm:
                dNW += np.sum(g4 * yn, axis=(0, 2))
                gn = g4 * NW[None, :, None, :]
                g3 = rinv * (gn - yn * np.mean(gn * yn, axis=-1, keepdims=True))
            else:
                g3 = g4
            if cfg.has_z:
                du = g3 * y2 * _dsilu(u)
                dZ[:, t] += np.sum(du * MZ[None], axis=2)
                dMZ += np.sum(du * Z[:, t, :, None, :], axis=0)
                g2 = g3 * silu(u)
            else:
                g2 = g3
            if cfg.has_d:
                dD += np.sum(g2 * XR[:, t], axis=(0, 2, 3))
                dXR[:, t] += D[None, :, None, None] * g2
            g1 = g2
            hbar = carry + np.einsum("bhrp,bhrn->bhpn", g1, Qm[:, t])    # adjoint of h_t
            dQ[:, t] += np.einsum("bhpn,bhrp->bhrn", h_t, g1)
            d_alpha[:, t] = np.sum(hbar * h_prev, axis=(2, 3))
            hk = np.einsum("bhpn,bhrn->bhrp", hbar, K[:, t])
            d_gamma[:, t] = np.sum(XR[:, t] * hk, axis=(2, 3))
            dXR[:, t] += gamma[:, t, :, None, None] * hk
            dK[:, t] += gamma[:, t, :, None, None] * np.einsum("bhpn,bhrp->bhrn", hbar, XR[:, t])
            if t > 0:
                hk1 = np.einsum("bhpn,bhrn->bhrp", hbar, K[:, t - 1])
                d_beta[:, t] = np.sum(XR[:, t - 1] * hk1, axis=(2, 3))
                dXR[:, t - 1] += beta[:, t, :, None, None] * hk1
                dK[:, t - 1] += beta[:, t, :, None, None] * np.einsum("bhpn,bhrp->bhrn", hbar, XR[:, t - 1])
            carry = alpha[:, t, :, None, None] * hbar

    d_adt = alpha * (d_alpha + d_beta * (1.0 - lam) * DT)
    d_lam = d_gamma * DT - d_beta * DT * alpha
    d_dt = d_gamma * lam + d_beta * (1.0 - lam) * alpha
    d_trap = d_lam * lam * (1.0 - lam)

    # X_r = x * mimo_x[h, r]
    dX = np.sum(dXR * MX[None, None], axis=3)
    dMX = np.sum(dXR * X[:, :, :, None, :], axis=(0, 1))

    # rotation, with one angle per head shared by the ranks
    dKraw = rotate(dK, -th_r, A)
    dQraw = rotate(dQ, -th_r, A)
    d_angle = np.zeros_like(ANG)
    if A > 0:
        d_theta = np.sum(dK[..., A:2 * A] * K[..., :A] - dK[..., :A] * K[..., A:2 * A]
                         + dQ[..., A:2 * A] * Qm[..., :A] - dQ[..., :A] * Qm[..., A:2 * A], axis=3)
        tail = np.flip(np.cumsum(np.flip(d_theta, axis=1), axis=1), axis=1)
        d_dt = d_dt + np.sum(tail * ANG[:, :, None, :], axis=3)
        d_angle = np.sum(DT[..., None] * tail, axis=2)

    d_b = np.zeros((len(rows), L, R * G, N))
    d_c = np.zeros((len(rows), L, R * G, N))
    for h in range(H):
        for r in range(R):
            d_b[:, :, bc_rows[h, r]] += dKraw[:, :, h, r]
            d_c[:, :, bc_rows[h, r]] += dQraw[:, :, h, r]
    return {
        "c": d_c, "b": d_b, "x": dX, "z": dZ, "adt": d_adt, "dt": d_dt, "trap": d_trap,
        "angle": d_angle, "c_bias": dQraw.sum(axis=(0, 1)), "b_bias": dKraw.sum(axis=(0, 1)),
        "d": dD if cfg.has_d else np.zeros(H), "mimo_x": dMX, "mimo_z": dMZ, "mimo_o": dMO,
        "norm_weight": dNW,
    }
