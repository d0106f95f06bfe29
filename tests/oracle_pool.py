"""The float64 oracle sharded by head over a pool of host processes, for the
full-size parity cases.

Workers are fresh interpreters (the spawn start method): each regenerates
the workload's seeded inputs itself, so no large array crosses a pipe on the
way in, and none imports torch or the package.  Each worker's numeric
libraries are held to one thread; the pool has one worker per core, at most
sixteen.  A worker that cannot start breaks the pool with an error (no
respawning).
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle as O
from workloads import WORKLOADS, Dims, decode_states, ssm_inputs, step_inputs

OPS11 = ("c", "b", "x", "z", "adt", "dt", "trap", "angle", "c_bias", "b_bias", "d")
MIMO4 = ("mimo_x", "mimo_z", "mimo_o", "norm_weight")
STATE_KEYS = ("ssm_state", "angle_state", "k_state", "v_state")
_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "NUMEXPR_NUM_THREADS")

_STATE = {}


def _cfg(d) -> O.SsmConfig:
    return O.SsmConfig(batch_size=d.B, sequence_length=d.L, num_heads=d.H, num_groups=d.G, head_dim=d.P,
                       state_size=d.N, num_rope_angles=d.A, mimo_rank=d.R, has_z=d.has_z, has_d=d.has_d,
                       has_output_norm=d.has_output_norm)


def _init(name: str) -> None:
    w = WORKLOADS[name]
    _STATE["d"] = w.dims
    _STATE["mimo"] = w.kind == "mimo"
    _STATE["inp"] = ssm_inputs(w.dims, seed=w.seed, dt_range=w.dt_range, mimo=_STATE["mimo"])


def _one_head(h: int):
    inp, d = _STATE["inp"], _STATE["d"]
    if _STATE["mimo"]:
        out = O.mimo_scan(*[inp[k] for k in OPS11 + MIMO4], _cfg(d), heads=[h])
    else:
        out = O.siso_scan(*[inp[k] for k in OPS11], _cfg(d), heads=[h])
    return h, out


def pool_size(n_tasks: int) -> int:
    return max(1, min(16, os.cpu_count() or 1, n_tasks))


def oracle_heads(name: str, heads=None) -> np.ndarray:
    """The oracle's output of workload `name` for `heads` (all by default),
    stacked on the head axis in the order given."""
    w = WORKLOADS[name]
    heads = list(range(w.dims.H)) if heads is None else list(heads)
    saved = {k: os.environ.get(k) for k in _THREAD_VARS}
    for k in _THREAD_VARS:
        os.environ[k] = "1"  # inherited by the spawned workers
    try:
        with ProcessPoolExecutor(pool_size(len(heads)), mp_context=mp.get_context("spawn"), initializer=_init,
                                 initargs=(name,)) as pool:
            res = dict(pool.map(_one_head, heads))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return np.concatenate([res[h] for h in heads], axis=2)


def _decode_task(args):
    """Follow `rows` of a decode workload from its seeded states through
    `steps` steps; return the outputs [steps, rows, 1, H, P] and the final
    states of those rows."""
    name, rows, steps = args
    w = WORKLOADS[name]
    d = w.dims
    rows = np.asarray(rows)
    st = {k: v[rows].astype(np.float64) for k, v in decode_states(d, seed=w.seed).items()}
    sub = Dims(len(rows), 1, d.H, d.G, d.P, d.N, d.A)
    outs = []
    for s in range(steps):
        tok = step_inputs(d, w.seed, s)
        tok = {k: (v[rows] if v.ndim >= 3 else v) for k, v in tok.items()}
        y, st = O.siso_step(*[tok[k] for k in OPS11], *[st[k] for k in STATE_KEYS], _cfg(sub))
        outs.append(y)
    return np.stack(outs), st


class DecodeOracle:
    """The oracle's decode trajectories, computed in a process pool while the
    caller drives the GPU: every row of `row_groups` (a list of row lists)
    through all the workload's steps, and the whole batch through its first
    `full_steps` steps."""

    def __init__(self, name: str, row_groups, full_steps: int):
        w = WORKLOADS[name]
        self.tasks = [(name, list(range(w.dims.B)), full_steps)] + [(name, list(g), w.steps) for g in row_groups]

    def __enter__(self):
        self._saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        self.pool = ProcessPoolExecutor(pool_size(len(self.tasks)), mp_context=mp.get_context("spawn"))
        self.futures = [self.pool.submit(_decode_task, t) for t in self.tasks]
        return self

    def results(self):
        """(full-batch outputs [full_steps, B, 1, H, P], [(outputs, states) per row group])."""
        res = [f.result() for f in self.futures]
        return res[0][0], res[1:]

    def __exit__(self, *exc):
        self.pool.shutdown(wait=True, cancel_futures=True)
        for k, v in self._saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        return False
