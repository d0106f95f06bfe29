"""Seeded synthetic inputs shaped like the Mamba-3 SsmConfig workloads.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random numbers and shapes their distributions; it computes none of the
scan's steps.  Every array it returns is float32 and C-contiguous, in the
operand layouts of the ``mamba3_siso`` / ``mamba3_mimo`` / ``mamba3_siso_step``
docs (mamba3.rs, oarust 0.8.6):

  c, b      [B, L, R*G, N]   standard normal rows rescaled to unit RMS
  x, z      [B, L, H, P]     standard normal
  dt        [B, L, H]        uniform on [dt_lo, dt_hi]
  adt       [B, L, H]        -A * dt with A uniform on [1, 16] per element
  trap      [B, L, H]        logistic of a standard normal
  angle     [B, L, A]        normal, standard deviation 0.1
  d         [H]              standard normal
  c_bias, b_bias [H, (R,) N] normal, standard deviation 0.02
  mimo_x/z/o [H, R, P]       normal, standard deviation 0.5 (variance 1/4)
  norm_weight [H, P]         1 + normal(0, 0.02)

Draw order is fixed (x, z, B, C, dt, A, trap, angle, D, c_bias, b_bias, MIMO
weights, states) so that one seed fixes every value.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

RMS_EPS = 1.0e-5


@dataclass(frozen=True)
class Dims:
    """Scan geometry: batch, length, heads, groups (0 => heads), head_dim, state, angles, rank."""

    B: int
    L: int
    H: int
    G: int
    P: int
    N: int
    A: int
    R: int = 1
    has_z: bool = True
    has_d: bool = True
    has_output_norm: bool = False

    @property
    def groups(self) -> int:
        return self.H if self.G == 0 else self.G


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "siso" | "mimo" | "step" | "mimo_step"
    dims: Dims
    dt_range: tuple = (1e-3, 0.1)
    seed: int = 0
    steps: int = 1
    extra: dict = field(default_factory=dict)


# The workloads: a tiny parity case, the 1.3B-class mixer layer, a long
# sequence, a rank-4 MIMO layer, batched single-token decode, and batched
# rank-4 MIMO decode.
WORKLOADS = {
    "siso_tiny": Workload("siso_tiny", "siso", Dims(1, 64, 2, 1, 16, 16, 8), seed=1000),
    "siso_b4_l2048": Workload("siso_b4_l2048", "siso", Dims(4, 2048, 24, 1, 64, 128, 32), seed=1001),
    "siso_long_l65536": Workload("siso_long_l65536", "siso", Dims(1, 65536, 32, 1, 64, 128, 32),
                                 dt_range=(1e-3, 0.01), seed=1002),
    "mimo_b8_l4096_r4": Workload("mimo_b8_l4096_r4", "mimo",
                                 Dims(8, 4096, 32, 1, 64, 128, 32, R=4, has_output_norm=True), seed=1003),
    "decode_b256": Workload("decode_b256", "step", Dims(256, 1, 32, 1, 64, 128, 32), seed=1004, steps=1024),
    # MIMO decode at the decode geometry with the MIMO workload's rank and norm
    "mimo_decode_b256_r4": Workload("mimo_decode_b256_r4", "mimo_step",
                                    Dims(256, 1, 32, 1, 64, 128, 32, R=4, has_output_norm=True),
                                    seed=1005, steps=256),
}


def _unit_rms_rows(raw: np.ndarray) -> np.ndarray:
    """Rescale each last-axis row to unit root-mean-square (input shaping)."""
    r64 = raw.astype(np.float64)
    scale = np.sqrt(np.mean(r64 * r64, axis=-1, keepdims=True) + RMS_EPS)
    return (r64 / scale).astype(np.float32)


def _logistic(v: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-v.astype(np.float64)))).astype(np.float32)


def ssm_inputs(d: Dims, seed: int, dt_range=(1e-3, 0.1), mimo: bool | None = None,
               overrides: dict | None = None) -> dict:
    """Seeded operands for one SISO or MIMO scan call."""
    rng = np.random.default_rng(seed)
    B, L, H, G, P, N, A, R = d.B, d.L, d.H, d.groups, d.P, d.N, d.A, d.R
    mimo = (R > 1 or d.has_output_norm) if mimo is None else mimo
    f32 = np.float32
    out = {}
    out["x"] = rng.standard_normal((B, L, H, P), dtype=f32)
    out["z"] = rng.standard_normal((B, L, H, P), dtype=f32)
    out["b"] = _unit_rms_rows(rng.standard_normal((B, L, R * G, N), dtype=f32))
    out["c"] = _unit_rms_rows(rng.standard_normal((B, L, R * G, N), dtype=f32))
    lo, hi = dt_range
    dt = (f32(lo) + f32(hi - lo) * rng.random((B, L, H), dtype=f32)).astype(f32)
    out["dt"] = dt
    a_mag = (f32(1.0) + f32(15.0) * rng.random((B, L, H), dtype=f32)).astype(f32)
    out["adt"] = (-a_mag * dt).astype(f32)
    out["trap"] = _logistic(rng.standard_normal((B, L, H), dtype=f32))
    out["angle"] = (f32(0.1) * rng.standard_normal((B, L, A), dtype=f32)).astype(f32)
    out["d"] = rng.standard_normal((H,), dtype=f32)
    bias_shape = (H, R, N) if mimo else (H, N)
    out["c_bias"] = (f32(0.02) * rng.standard_normal(bias_shape, dtype=f32)).astype(f32)
    out["b_bias"] = (f32(0.02) * rng.standard_normal(bias_shape, dtype=f32)).astype(f32)
    if mimo:
        out["mimo_x"] = (f32(0.5) * rng.standard_normal((H, R, P), dtype=f32)).astype(f32)
        out["mimo_z"] = (f32(0.5) * rng.standard_normal((H, R, P), dtype=f32)).astype(f32)
        out["mimo_o"] = (f32(0.5) * rng.standard_normal((H, R, P), dtype=f32)).astype(f32)
        out["norm_weight"] = (f32(1.0) + f32(0.02) * rng.standard_normal((H, P), dtype=f32)).astype(f32)
    if overrides:
        for k, v in overrides.items():
            out[k] = np.ascontiguousarray(np.broadcast_to(np.asarray(v, dtype=f32), out[k].shape))
    return {k: np.ascontiguousarray(v) for k, v in out.items()}


def decode_states(d: Dims, seed: int) -> dict:
    """Seeded recurrent states for ``mamba3_siso_step``.

    ssm_state ~ N(0,1) [B,H,P,N]; angle_state ~ U[-pi, pi] [B,H,A];
    k_state holds a unit-RMS B-like row [B,H,N] and v_state an x-like row
    [B,H,P], standing for the previous token's stored key and value.
    """
    rng = np.random.default_rng([seed, 0x5747])
    B, H, P, N, A = d.B, d.H, d.P, d.N, d.A
    f32 = np.float32
    st = {
        "ssm_state": rng.standard_normal((B, H, P, N), dtype=f32),
        "angle_state": (f32(-np.pi) + f32(2 * np.pi) * rng.random((B, H, A), dtype=f32)).astype(f32),
        "k_state": _unit_rms_rows(rng.standard_normal((B, H, N), dtype=f32)),
        "v_state": rng.standard_normal((B, H, P), dtype=f32),
    }
    return {k: np.ascontiguousarray(v) for k, v in st.items()}


def mimo_decode_states(d: Dims, seed: int) -> dict:
    """Seeded recurrent states for ``mamba3_mimo_step``: ssm_state ~ N(0,1)
    [B,H,P,N]; angle_state ~ U[-pi, pi] [B,H,A]; per rank r a unit-RMS key
    row k_state [B,H,R,N] and an x-like value row v_state [B,H,R,P]."""
    rng = np.random.default_rng([seed, 0x4D53])
    B, H, P, N, A, R = d.B, d.H, d.P, d.N, d.A, d.R
    f32 = np.float32
    st = {
        "ssm_state": rng.standard_normal((B, H, P, N), dtype=f32),
        "angle_state": (f32(-np.pi) + f32(2 * np.pi) * rng.random((B, H, A), dtype=f32)).astype(f32),
        "k_state": _unit_rms_rows(rng.standard_normal((B, H, R, N), dtype=f32)),
        "v_state": rng.standard_normal((B, H, R, P), dtype=f32),
    }
    return {k: np.ascontiguousarray(v) for k, v in st.items()}


def step_inputs(d: Dims, seed: int, step: int, dt_range=(1e-3, 0.1), mimo: bool = False) -> dict:
    """Fresh seeded L == 1 operands for decode step ``step`` (MIMO operands
    and [H,R,N] biases with ``mimo``)."""
    d1 = Dims(d.B, 1, d.H, d.G, d.P, d.N, d.A, d.R, d.has_z, d.has_d, d.has_output_norm)
    return ssm_inputs(d1, seed=np.random.SeedSequence([seed, step]).generate_state(1)[0],
                      dt_range=dt_range, mimo=mimo)


def preprocess_inputs(rows: int, width: int, heads: int, seed: int,
                      dt_lo: float = 1e-3, dt_hi: float = 0.1) -> dict:
    """Packed projections ~ N(0,1) [rows, width]; dt_bias [H] such that
    softplus(dt_bias) is log-uniform on [dt_lo, dt_hi]."""
    rng = np.random.default_rng(seed)
    projected = rng.standard_normal((rows, width), dtype=np.float32)
    target = np.exp(rng.uniform(np.log(dt_lo), np.log(dt_hi), size=heads))
    dt_bias = np.log(np.expm1(target)).astype(np.float32)  # inverse of log(1 + e^u)
    return {"projected": np.ascontiguousarray(projected), "dt_bias": dt_bias}


def _inverse_softplus(y: np.ndarray) -> np.ndarray:
    """u with log(1 + e^u) = y (input shaping for the packed projection)."""
    y64 = np.asarray(y, dtype=np.float64)
    return np.log(np.expm1(y64))


def packed_projection(d: Dims, seed: int, dt_range=(1e-3, 0.1)) -> dict:
    """A packed projection [B*L, 2I + 2GN + 3H + A] (I = H*P, rank one) whose
    preprocess outputs follow the scan-input recipe of this module: z, x ~ N(0,1);
    B, C standard normal (the preprocess RMS-normalises them); dt_raw such that
    softplus(dt_raw) is uniform on dt_range (dt_bias = 0); A_raw such that
    softplus(A_raw) is uniform on [1, 16]; trap = logistic(N(0,1)); angle ~ N(0, 0.1).
    Also returns dt_bias (zeros) and the scan parameters c_bias, b_bias, d."""
    rng = np.random.default_rng(seed)
    B, L, H, G, P, N, A = d.B, d.L, d.H, d.groups, d.P, d.N, d.A
    rows, I, M = B * L, H * P, G * N
    f32 = np.float32
    W = 2 * I + 2 * M + 3 * H + A
    proj = np.empty((rows, W), dtype=f32)
    off = 0
    proj[:, off:off + I] = rng.standard_normal((rows, I), dtype=f32); off += I      # z
    proj[:, off:off + I] = rng.standard_normal((rows, I), dtype=f32); off += I      # x
    proj[:, off:off + M] = rng.standard_normal((rows, M), dtype=f32); off += M      # B
    proj[:, off:off + M] = rng.standard_normal((rows, M), dtype=f32); off += M      # C
    lo, hi = dt_range
    proj[:, off:off + H] = _inverse_softplus(lo + (hi - lo) * rng.random((rows, H))); off += H
    proj[:, off:off + H] = _inverse_softplus(1.0 + 15.0 * rng.random((rows, H))); off += H
    proj[:, off:off + H] = _logistic(rng.standard_normal((rows, H), dtype=f32)); off += H
    proj[:, off:off + A] = f32(0.1) * rng.standard_normal((rows, A), dtype=f32); off += A
    assert off == W
    return {
        "projected": proj,
        "dt_bias": np.zeros(H, dtype=f32),
        "c_bias": (f32(0.02) * rng.standard_normal((H, N), dtype=f32)).astype(f32),
        "b_bias": (f32(0.02) * rng.standard_normal((H, N), dtype=f32)).astype(f32),
        "d": rng.standard_normal((H,), dtype=f32),
    }


def output_gradient(d: Dims, seed: int) -> np.ndarray:
    """Seeded upstream gradient ~ N(0,1) in the scan-output layout [B,L,H,P]."""
    rng = np.random.default_rng([seed, 0x4742])
    return np.ascontiguousarray(rng.standard_normal((d.B, d.L, d.H, d.P), dtype=np.float32))


def preprocess_output_gradients(rows: int, inner: int, bc_width: int, heads: int, angles: int,
                                seed: int, missing=()) -> dict:
    """Seeded gradients ~ N(0,1) of the eight preprocess outputs (x, z [rows, I];
    bh, ch [rows, GRN]; dt, adt, trap [rows, H]; angle [rows, A]); names in
    ``missing`` map to None (no gradient)."""
    rng = np.random.default_rng([seed, 0x5042])
    widths = {"x": inner, "z": inner, "bh": bc_width, "ch": bc_width, "dt": heads, "adt": heads,
              "trap": heads, "angle": angles}
    out = {}
    for k, w in widths.items():
        g = np.ascontiguousarray(rng.standard_normal((rows, w), dtype=np.float32))
        out[k] = None if k in missing else g
    return out
