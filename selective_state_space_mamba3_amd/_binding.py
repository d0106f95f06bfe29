"""ctypes binding of libm3.so: argument marshalling only.

Every function here checks dtype, device, contiguity and shape of the torch
tensors it is given (raw pointers cannot carry shapes), allocates outputs
and workspace with torch when the caller did not pass them, and calls the C
entry point of the same name on the current HIP stream.  No step of the
computation happens in Python, and nothing falls back to the CPU: if the
library is missing, :func:`lib` raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm3.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "m3.h")

M3_OK = 0
M3_ERR_INVALID_ARGUMENT = 1
M3_ERR_UNSUPPORTED = 2
M3_ERR_HIP = 3


@dataclass(frozen=True)
class SsmConfig:
    """Scan geometry and flags (mirror of the pages' SsmConfig)."""

    batch_size: int
    sequence_length: int
    num_heads: int
    num_groups: int
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
    """Preprocess geometry and bounds (mirror of Mamba3PreprocessConfig)."""

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

    @property
    def width(self) -> int:
        return (2 * self.inner_size + 2 * self.num_groups * self.mimo_rank * self.state_size
                + 3 * self.num_heads + self.num_rope_angles)


class _CSsm(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "batch_size", "sequence_length", "num_heads", "num_groups", "head_dim", "state_size",
        "num_rope_angles", "mimo_rank", "has_z", "has_d", "has_output_norm")]


class _CPre(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in (
        "inner_size", "state_size", "num_heads", "num_rope_angles", "num_groups", "mimo_rank")] + \
        [(n, ctypes.c_float) for n in ("epsilon", "dt_min", "dt_max", "a_floor")]


class M3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[m3 status {status}] {message}")
        self.status = status


_LIB = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libm3.so (built in-tree); raise loudly when it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m selective_state_space_mamba3_amd.build` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    L.m3_last_error.restype = ctypes.c_char_p
    L.m3_version.restype = ctypes.c_char_p
    L.m3_siso_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.m3_siso_fwd_workspace_bytes.argtypes = [_CSsm]
    L.m3_mimo_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.m3_mimo_fwd_workspace_bytes.argtypes = [_CSsm]
    L.m3_preprocess.restype = ctypes.c_int
    L.m3_preprocess.argtypes = [_P, _P, ctypes.c_uint32, _CPre] + [_P] * 8 + [_P]
    L.m3_siso_fwd.restype = ctypes.c_int
    L.m3_siso_fwd.argtypes = [_P] * 11 + [_CSsm, _P, _P, ctypes.c_size_t, _P]
    L.m3_mimo_fwd.restype = ctypes.c_int
    L.m3_mimo_fwd.argtypes = [_P] * 15 + [_CSsm, _P, _P, ctypes.c_size_t, _P]
    L.m3_siso_step.restype = ctypes.c_int
    L.m3_siso_step.argtypes = [_P] * 15 + [_CSsm, _P, _P]
    L.m3_mimo_step.restype = ctypes.c_int
    L.m3_mimo_step.argtypes = [_P] * 19 + [_CSsm, _P, _P]
    L.m3_siso_fwd_packed_workspace_bytes.restype = ctypes.c_size_t
    L.m3_siso_fwd_packed_workspace_bytes.argtypes = [_CPre, _CSsm]
    L.m3_siso_fwd_packed.restype = ctypes.c_int
    L.m3_siso_fwd_packed.argtypes = [_P] * 5 + [_CPre, _CSsm, _P, _P, ctypes.c_size_t, _P]
    L.m3_mimo_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.m3_mimo_bwd_workspace_bytes.argtypes = [_CSsm]
    L.m3_mimo_bwd.restype = ctypes.c_int
    L.m3_mimo_bwd.argtypes = [_P] * 16 + [_CSsm] + [_P] * 15 + [_P, ctypes.c_size_t, _P]
    L.m3_siso_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.m3_siso_bwd_workspace_bytes.argtypes = [_CSsm]
    L.m3_siso_bwd.restype = ctypes.c_int
    L.m3_siso_bwd.argtypes = [_P] * 12 + [_CSsm] + [_P] * 11 + [_P, ctypes.c_size_t, _P]
    L.m3_siso_fwd_noalloc.restype = ctypes.c_int
    L.m3_siso_fwd_noalloc.argtypes = [_P] * 11 + [_CSsm, _P, _P]
    L.m3_set_scan_segments.restype = None
    L.m3_set_scan_segments.argtypes = [ctypes.c_uint32]
    L.m3_preprocess_bwd.restype = ctypes.c_int
    L.m3_preprocess_bwd.argtypes = [_P, _P, ctypes.c_uint32, _CPre] + [_P] * 8 + [_P, _P, _P]
    _LIB = L
    return L


def set_scan_segments(segments: int) -> None:
    """Force the scan plan's segment count on this thread (0 = automatic)."""
    lib().m3_set_scan_segments(int(segments))


class scan_segments:
    """Context manager: run the scans inside it with a forced segment count."""

    def __init__(self, segments: int):
        self.segments = int(segments)

    def __enter__(self):
        set_scan_segments(self.segments)
        return self

    def __exit__(self, *exc):
        set_scan_segments(0)
        return False


def header_functions() -> list:
    """Names of the functions include/m3.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m3_[a-z0-9_]+)\s*\(", text)))


def last_error() -> str:
    return lib().m3_last_error().decode()


def _check(status: int):
    if status != M3_OK:
        raise M3Error(status, last_error())


def c_ssm(cfg: SsmConfig) -> _CSsm:
    return _CSsm(cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.num_groups, cfg.head_dim,
                 cfg.state_size, cfg.num_rope_angles, cfg.mimo_rank, int(cfg.has_z), int(cfg.has_d),
                 int(cfg.has_output_norm))


def c_pre(cfg: PreprocessConfig) -> _CPre:
    return _CPre(cfg.inner_size, cfg.state_size, cfg.num_heads, cfg.num_rope_angles, cfg.num_groups,
                 cfg.mimo_rank, cfg.epsilon, cfg.dt_min, cfg.dt_max, cfg.a_floor)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() if t.numel() > 0 else None


def _expect(name: str, t: torch.Tensor, shape, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _scan_shapes(cfg: SsmConfig, rows_bc: int, bias_shape):
    B, L, H, P, N, A = (cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.head_dim,
                        cfg.state_size, cfg.num_rope_angles)
    return {
        "c": (B, L, rows_bc, N), "b": (B, L, rows_bc, N), "x": (B, L, H, P), "z": (B, L, H, P),
        "adt": (B, L, H), "dt": (B, L, H), "trap": (B, L, H), "angle": (B, L, A),
        "c_bias": bias_shape, "b_bias": bias_shape, "d": (H,),
    }


_OPS11 = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")


def siso_fwd_workspace_bytes(cfg: SsmConfig) -> int:
    return int(lib().m3_siso_fwd_workspace_bytes(c_ssm(cfg)))


def mimo_fwd_workspace_bytes(cfg: SsmConfig) -> int:
    return int(lib().m3_mimo_fwd_workspace_bytes(c_ssm(cfg)))


def m3_siso_fwd(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, cfg: SsmConfig,
                out=None, workspace=None, stream=None) -> torch.Tensor:
    """SISO scan forward on the GPU; returns out [B, L, H, P]."""
    L_ = lib()
    dev = x.device
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    for k, shp in _scan_shapes(cfg, cfg.groups, (cfg.num_heads, cfg.state_size)).items():
        _expect(k, ops[k], shp, dev)
    oshape = (cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.head_dim)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _expect("out", out, oshape, dev)
    need = siso_fwd_workspace_bytes(cfg)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L_.m3_siso_fwd(*[_ptr(ops[k]) for k in _OPS11], c_ssm(cfg), _ptr(out),
                          _ptr(workspace), ws_bytes, _stream(dev, stream)))
    return out


def m3_siso_fwd_noalloc(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, cfg: SsmConfig,
                        out=None, stream=None) -> torch.Tensor:
    """m3_siso_fwd with the library's fixed scratch in place of a workspace
    (the C call allocates nothing); returns out [B, L, H, P]."""
    L_ = lib()
    dev = x.device
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    for k, shp in _scan_shapes(cfg, cfg.groups, (cfg.num_heads, cfg.state_size)).items():
        _expect(k, ops[k], shp, dev)
    oshape = (cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.head_dim)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _expect("out", out, oshape, dev)
    _check(L_.m3_siso_fwd_noalloc(*[_ptr(ops[k]) for k in _OPS11], c_ssm(cfg), _ptr(out),
                                  _stream(dev, stream)))
    return out


def m3_mimo_fwd(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, mimo_x, mimo_z, mimo_o,
                norm_weight, cfg: SsmConfig, out=None, workspace=None, stream=None) -> torch.Tensor:
    """MIMO scan forward on the GPU; returns out [B, L, H, P]."""
    L_ = lib()
    dev = x.device
    R = cfg.mimo_rank
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    for k, shp in _scan_shapes(cfg, R * cfg.groups, (cfg.num_heads, R, cfg.state_size)).items():
        _expect(k, ops[k], shp, dev)
    for k, t in (("mimo_x", mimo_x), ("mimo_z", mimo_z), ("mimo_o", mimo_o)):
        _expect(k, t, (cfg.num_heads, R, cfg.head_dim), dev)
    _expect("norm_weight", norm_weight, (cfg.num_heads, cfg.head_dim), dev)
    oshape = (cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.head_dim)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _expect("out", out, oshape, dev)
    need = mimo_fwd_workspace_bytes(cfg)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(L_.m3_mimo_fwd(*[_ptr(ops[k]) for k in _OPS11], _ptr(mimo_x), _ptr(mimo_z), _ptr(mimo_o),
                          _ptr(norm_weight), c_ssm(cfg), _ptr(out), _ptr(workspace), ws_bytes,
                          _stream(dev, stream)))
    return out


def m3_siso_step(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, ssm_state, angle_state,
                 k_state, v_state, cfg: SsmConfig, out=None, stream=None) -> torch.Tensor:
    """One SISO decode token; updates the four states in place, returns out [B, 1, H, P]."""
    L_ = lib()
    dev = x.device
    if cfg.sequence_length != 1:
        raise ValueError("m3_siso_step requires sequence_length == 1")
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    for k, shp in _scan_shapes(cfg, cfg.groups, (cfg.num_heads, cfg.state_size)).items():
        _expect(k, ops[k], shp, dev)
    B, H, P, N, A = cfg.batch_size, cfg.num_heads, cfg.head_dim, cfg.state_size, cfg.num_rope_angles
    _expect("ssm_state", ssm_state, (B, H, P, N), dev)
    _expect("angle_state", angle_state, (B, H, A), dev)
    _expect("k_state", k_state, (B, H, N), dev)
    _expect("v_state", v_state, (B, H, P), dev)
    oshape = (B, 1, H, P)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _expect("out", out, oshape, dev)
    _check(L_.m3_siso_step(*[_ptr(ops[k]) for k in _OPS11], _ptr(ssm_state), _ptr(angle_state),
                           _ptr(k_state), _ptr(v_state), c_ssm(cfg), _ptr(out), _stream(dev, stream)))
    return out


def m3_mimo_step(c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, mimo_x, mimo_z, mimo_o,
                 norm_weight, ssm_state, angle_state, k_state, v_state, cfg: SsmConfig, out=None,
                 stream=None) -> torch.Tensor:
    """One MIMO decode token; updates the four states in place, returns out [B, 1, H, P]."""
    L_ = lib()
    dev = x.device
    if cfg.sequence_length != 1:
        raise ValueError("m3_mimo_step requires sequence_length == 1")
    R = cfg.mimo_rank
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    for k, shp in _scan_shapes(cfg, R * cfg.groups, (cfg.num_heads, R, cfg.state_size)).items():
        _expect(k, ops[k], shp, dev)
    for k, t in (("mimo_x", mimo_x), ("mimo_z", mimo_z), ("mimo_o", mimo_o)):
        _expect(k, t, (cfg.num_heads, R, cfg.head_dim), dev)
    _expect("norm_weight", norm_weight, (cfg.num_heads, cfg.head_dim), dev)
    B, H, P, N, A = cfg.batch_size, cfg.num_heads, cfg.head_dim, cfg.state_size, cfg.num_rope_angles
    _expect("ssm_state", ssm_state, (B, H, P, N), dev)
    _expect("angle_state", angle_state, (B, H, A), dev)
    _expect("k_state", k_state, (B, H, R, N), dev)
    _expect("v_state", v_state, (B, H, R, P), dev)
    oshape = (B, 1, H, P)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=dev)
    _expect("out", out, oshape, dev)
    _check(L_.m3_mimo_step(*[_ptr(ops[k]) for k in _OPS11], _ptr(mimo_x), _ptr(mimo_z), _ptr(mimo_o),
                           _ptr(norm_weight), _ptr(ssm_state), _ptr(angle_state), _ptr(k_state),
                           _ptr(v_state), c_ssm(cfg), _ptr(out), _stream(dev, stream)))
    return out


_PRE_OUT = ("x", "z", "bh", "ch", "dt", "adt", "trap", "angle")


def m3_preprocess(projected, dt_bias, cfg: PreprocessConfig, outs: dict | None = None,
                  stream=None) -> dict:
    """Split and transform packed projections; returns the eight outputs."""
    L_ = lib()
    dev = projected.device
    rows = projected.shape[0] if projected.dim() == 2 else -1
    _expect("projected", projected, (rows, cfg.width), dev)
    _expect("dt_bias", dt_bias, (cfg.num_heads,), dev)
    M = cfg.num_groups * cfg.mimo_rank * cfg.state_size
    shapes = {"x": (rows, cfg.inner_size), "z": (rows, cfg.inner_size), "bh": (rows, M),
              "ch": (rows, M), "dt": (rows, cfg.num_heads), "adt": (rows, cfg.num_heads),
              "trap": (rows, cfg.num_heads), "angle": (rows, cfg.num_rope_angles)}
    outs = dict(outs or {})
    for k, shp in shapes.items():
        if k not in outs:
            outs[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        _expect(k, outs[k], shp, dev)
    _check(L_.m3_preprocess(_ptr(projected), _ptr(dt_bias), rows, c_pre(cfg),
                            *[_ptr(outs[k]) for k in _PRE_OUT], _stream(dev, stream)))
    return outs


def siso_bwd_workspace_bytes(cfg: SsmConfig) -> int:
    return int(lib().m3_siso_bwd_workspace_bytes(c_ssm(cfg)))


def m3_siso_bwd(dout, c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, cfg: SsmConfig,
                grads: dict | None = None, workspace=None, stream=None) -> dict:
    """SISO scan backward on the GPU; returns the eleven gradients by operand name."""
    L_ = lib()
    dev = x.device
    ops = dict(zip(_OPS11, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d)))
    shapes = _scan_shapes(cfg, cfg.groups, (cfg.num_heads, cfg.state_size))
    for k, shp in shapes.items():
        _expect(k, ops[k], shp, dev)
    _expect("dout", dout, shapes["x"], dev)
    grads = dict(grads or {})
    for k, shp in shapes.items():
        if k not in grads:
            grads[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        _expect("d_" + k, grads[k], shp, dev)
    need = siso_bwd_workspace_bytes(cfg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(L_.m3_siso_bwd(_ptr(dout), *[_ptr(ops[k]) for k in _OPS11], c_ssm(cfg),
                          *[_ptr(grads[k]) for k in _OPS11], _ptr(workspace), ws_bytes,
                          _stream(dev, stream)))
    return grads


def m3_preprocess_bwd(projected, dt_bias, cfg: PreprocessConfig, grads: dict, outs: dict | None = None,
                      stream=None) -> dict:
    """Preprocess backward; ``grads`` maps output names to gradients (missing or None = zero).
    Returns {"projected": d_projected [rows, W], "dt_bias": d_dt_bias [H]}."""
    L_ = lib()
    dev = projected.device
    rows = projected.shape[0] if projected.dim() == 2 else -1
    _expect("projected", projected, (rows, cfg.width), dev)
    _expect("dt_bias", dt_bias, (cfg.num_heads,), dev)
    M = cfg.num_groups * cfg.mimo_rank * cfg.state_size
    shapes = {"x": (rows, cfg.inner_size), "z": (rows, cfg.inner_size), "bh": (rows, M),
              "ch": (rows, M), "dt": (rows, cfg.num_heads), "adt": (rows, cfg.num_heads),
              "trap": (rows, cfg.num_heads), "angle": (rows, cfg.num_rope_angles)}
    for k in grads:
        if k not in shapes:
            raise ValueError(f"unknown preprocess output {k!r}")
    for k, shp in shapes.items():
        if grads.get(k) is not None:
            _expect("g_" + k, grads[k], shp, dev)
    outs = dict(outs or {})
    if "projected" not in outs:
        outs["projected"] = torch.empty((rows, cfg.width), dtype=torch.float32, device=dev)
    if "dt_bias" not in outs:
        outs["dt_bias"] = torch.empty((cfg.num_heads,), dtype=torch.float32, device=dev)
    _expect("d_projected", outs["projected"], (rows, cfg.width), dev)
    _expect("d_dt_bias", outs["dt_bias"], (cfg.num_heads,), dev)
    _check(L_.m3_preprocess_bwd(_ptr(projected), _ptr(dt_bias), rows, c_pre(cfg),
                                *[_ptr(grads.get(k)) for k in _PRE_OUT],
                                _ptr(outs["projected"]), _ptr(outs["dt_bias"]), _stream(dev, stream)))
    return outs


def siso_fwd_packed_workspace_bytes(pcfg: PreprocessConfig, cfg: SsmConfig) -> int:
    return int(lib().m3_siso_fwd_packed_workspace_bytes(c_pre(pcfg), c_ssm(cfg)))


def m3_siso_fwd_packed(projected, dt_bias, c_bias, b_bias, d, pcfg: PreprocessConfig, cfg: SsmConfig,
                       out=None, workspace=None, stream=None) -> torch.Tensor:
    """Preprocess + SISO scan on the packed rows [B*L, W]; returns out [B, L, H, P]."""
    L_ = lib()
    dev = projected.device
    B, L, H, P, N = cfg.batch_size, cfg.sequence_length, cfg.num_heads, cfg.head_dim, cfg.state_size
    _expect("projected", projected, (B * L, pcfg.width), dev)
    _expect("dt_bias", dt_bias, (H,), dev)
    _expect("c_bias", c_bias, (H, N), dev)
    _expect("b_bias", b_bias, (H, N), dev)
    _expect("d", d, (H,), dev)
    if out is None:
        out = torch.empty((B, L, H, P), dtype=torch.float32, device=dev)
    _expect("out", out, (B, L, H, P), dev)
    need = siso_fwd_packed_workspace_bytes(pcfg, cfg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(L_.m3_siso_fwd_packed(_ptr(projected), _ptr(dt_bias), _ptr(c_bias), _ptr(b_bias), _ptr(d),
                                 c_pre(pcfg), c_ssm(cfg), _ptr(out), _ptr(workspace), ws_bytes,
                                 _stream(dev, stream)))
    return out


_MIMO4 = ("mimo_x", "mimo_z", "mimo_o", "norm_weight")


def mimo_bwd_workspace_bytes(cfg: SsmConfig) -> int:
    return int(lib().m3_mimo_bwd_workspace_bytes(c_ssm(cfg)))


def m3_mimo_bwd(dout, c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d, mimo_x, mimo_z, mimo_o,
                norm_weight, cfg: SsmConfig, grads: dict | None = None, workspace=None, stream=None) -> dict:
    """MIMO scan backward on the GPU; returns the fifteen gradients by operand name."""
    L_ = lib()
    dev = x.device
    R = cfg.mimo_rank
    ops = dict(zip(_OPS11 + _MIMO4, (c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                                     mimo_x, mimo_z, mimo_o, norm_weight)))
    shapes = _scan_shapes(cfg, R * cfg.groups, (cfg.num_heads, R, cfg.state_size))
    for k in ("mimo_x", "mimo_z", "mimo_o"):
        shapes[k] = (cfg.num_heads, R, cfg.head_dim)
    shapes["norm_weight"] = (cfg.num_heads, cfg.head_dim)
    for k, shp in shapes.items():
        _expect(k, ops[k], shp, dev)
    _expect("dout", dout, shapes["x"], dev)
    grads = dict(grads or {})
    for k, shp in shapes.items():
        if k not in grads:
            grads[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        _expect("d_" + k, grads[k], shp, dev)
    need = mimo_bwd_workspace_bytes(cfg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    names = _OPS11 + _MIMO4
    _check(L_.m3_mimo_bwd(_ptr(dout), *[_ptr(ops[k]) for k in names], c_ssm(cfg),
                          *[_ptr(grads[k]) for k in names], _ptr(workspace), ws_bytes, _stream(dev, stream)))
    return grads
