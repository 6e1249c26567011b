"""CPU oracle for the sampler-level reductions: reconstructed timestep schedules,
the midpoint solver, limited-interval and adaptive guidance.

TEST INFRASTRUCTURE ONLY, like ``oracle.sampler`` (whose estimator, branch inputs
and guidance combine it reuses): only the test suite, the package's smoke check
and the benchmark's CPU-baseline leg may import it; the HIP library shares no
code with it. Plain float64 numpy, one request at a time.

Sources (VoiceHub "Diffusion and flow TTS optimization"):
  * section "Reduce a 50-step sampler before optimizing its kernels": the grid
    is rebuilt before the loop starts, keeps both endpoints and strict
    monotonicity, and has one of four shapes: a monotone subsequence of the
    native grid ("native"), linear between the endpoints ("uniform"), points
    concentrated near the noise end ("quadratic") or near the data end
    ("trailing");
  * table "Active families": the F5-TTS family samples with Euler or midpoint;
  * section "Guidance reduction": limited-interval guidance runs CFG only on a
    sub-interval of the trajectory (the configuration example uses 0.10 and
    0.70), adaptive guidance watches the conditional and unconditional branches
    converge and stops the unconditional lane only after a patience count
    (example: threshold 0.015, 4 warm-up steps, patience 2); guidance can only be
    narrowed, never enabled where the sampler did not ask for it, and each
    request's CFG lane is independent of the others.

The pages give no formulas for any of this. The readings (each listed in the
design notes of this repository) are:
  G1  the interval is on the sampling time t in [0, 1] (t = 0 noise, t = 1 data);
      an evaluation at time t is guided iff start <= t <= end;
  G2  an unguided evaluation runs the fully conditioned branch alone (the last
      branch: "cond", or "text+speaker" with three branches) and uses its
      velocity as is, i.e. the guidance equation at scale 1 (scales (1, 1));
  G3  adaptive metric of a request at an evaluation: sum |v_full - v_u| over the
      request's valid frames divided by sum |v_full| (relative L1 distance of the
      unconditional branch from the fully conditioned one; 0 when the
      denominator is 0);
  G4  adaptive state per request: steps k < warmup never count; from step
      `warmup` on, a step whose metric is below the threshold increments a
      counter and any other step resets it; when the counter reaches `patience`
      the request's unconditional lane stops for all later steps (its later
      evaluations are unguided, G2). With the midpoint solver only a step's
      first (left-endpoint) evaluation updates the state, and both evaluations
      of a step use the state the step started with;
  S1  schedules on S target steps, u_i = i / S: uniform t_i = u_i; quadratic
      t_i = u_i^2; trailing t_i = 1 - (1 - u_i)^2; native: t_i = n_i / N with
      n_i = round(i N / S) (half-way cases rounded up) on the native grid of N
      uniform steps, S <= N;
  M1  midpoint: x_{k+1} = x_k + dt_k v(t_k + dt_k / 2, x_k + (dt_k / 2) v(t_k, x_k)),
      both velocities guided per the policy at their own evaluation time.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Dict, Optional, Sequence, Tuple

import numpy as np

from oracle import sampler as O


# ---------------------------------------------------------------- schedules

def schedule(kind: str, n_steps: int, native_steps: Optional[int] = None) -> np.ndarray:
    """Time grid t_0 = 0 < t_1 < ... < t_S = 1 of S steps (reading S1)."""
    S = int(n_steps)
    if S <= 0:
        return np.zeros(1)
    u = np.arange(S + 1, dtype=np.float64) / S
    if kind == "uniform":
        t = u
    elif kind == "quadratic":
        t = u * u
    elif kind == "trailing":
        t = 1.0 - (1.0 - u) * (1.0 - u)
    elif kind == "native":
        N = int(native_steps if native_steps is not None else S)
        if N < S:
            raise ValueError(f"native grid of {N} steps cannot give {S} steps")
        idx = np.array([(2 * i * N + S) // (2 * S) for i in range(S + 1)])   # round(i N / S), halves up
        t = idx.astype(np.float64) / N
    else:
        raise ValueError(kind)
    return t


# ---------------------------------------------------------------- guidance policy

@dataclass(frozen=True)
class GuidancePolicy:
    mode: str = "full"                 # "full", "interval" or "adaptive"
    start: float = 0.0                 # interval mode: guided iff start <= t <= end (G1)
    end: float = 1.0
    threshold: float = 0.015           # adaptive mode (G3, G4)
    warmup: int = 4
    patience: int = 2


def in_interval(t: float, policy: GuidancePolicy) -> bool:
    return policy.start <= t <= policy.end


def adaptive_metric(v_full: np.ndarray, v_u: np.ndarray, valid: np.ndarray) -> float:
    """Relative L1 distance of the unconditional velocity from the fully conditioned one (G3)."""
    num = float(np.abs(v_full - v_u)[valid].sum())
    den = float(np.abs(v_full)[valid].sum())
    return num / den if den > 0 else 0.0


# ---------------------------------------------------------------- solver

def solve(x0_r: np.ndarray, grid: np.ndarray, velocity: Callable[[float, np.ndarray, bool], np.ndarray],
          scales: Sequence[float], nb: int, policy: GuidancePolicy, solver: str = "euler",
          valid: Optional[np.ndarray] = None):
    """One request through the whole sampler over ``grid``.

    ``velocity(t, x, guided)`` returns the stacked branch velocities [nb, ...]
    when ``guided``, else the fully conditioned branch alone [1, ...].
    Returns (x after the last step, per-step record). The record holds, per step,
    whether each evaluation was guided and the adaptive metric of the step's
    first evaluation (None when it was unguided).
    """
    x = np.asarray(x0_r, dtype=np.float64).copy()
    if valid is None:
        valid = np.ones(x.shape[:-1], dtype=bool)
    vmask = np.broadcast_to(valid[..., None], x.shape)
    lane_on = True          # adaptive: the unconditional lane still runs
    count = 0
    record = []

    def guided_at(t: float) -> bool:
        if nb == 1:
            return False
        if policy.mode == "full":
            return True
        if policy.mode == "interval":
            return in_interval(t, policy)
        if policy.mode == "adaptive":
            return lane_on
        raise ValueError(policy.mode)

    def combined(t: float, xx: np.ndarray, guided: bool):
        vs = velocity(t, xx, guided)
        if guided:
            return O.guidance_combine(vs, scales), vs
        return vs[0], vs

    for k in range(len(grid) - 1):
        t0, t1 = float(grid[k]), float(grid[k + 1])
        dt = t1 - t0
        g0 = guided_at(t0)
        v0, vs0 = combined(t0, x, g0)
        metric = adaptive_metric(vs0[-1], vs0[0], vmask) if g0 else None
        if solver == "euler":
            x = x + dt * v0
            rec = {"t": t0, "guided": (g0,), "metric": metric}
        elif solver == "midpoint":
            tm = t0 + 0.5 * dt
            gm = guided_at(tm)
            xm = x + (0.5 * dt) * v0
            vm, _ = combined(tm, xm, gm)
            x = x + dt * vm
            rec = {"t": t0, "guided": (g0, gm), "metric": metric}
        else:
            raise ValueError(solver)
        record.append(rec)
        if policy.mode == "adaptive" and nb > 1 and lane_on:
            if k >= policy.warmup:
                count = count + 1 if metric < policy.threshold else 0
                if count >= policy.patience:
                    lane_on = False
    return x, record


# ---------------------------------------------------------------- batched sampler

def sample_request(W64: Dict[str, np.ndarray], shape, x0_r, cond_r, spk_r, valid_r, grid: np.ndarray,
                   scales: Sequence[float], kinds: Sequence[str], policy: GuidancePolicy,
                   solver: str = "euler"):
    """All branches of one request through the sampler with the given grid, policy and solver."""
    cond_rows, spk_rows = [], []
    for kind in kinds:
        c, s = O.branch_inputs(kind, np.asarray(cond_r, np.float64),
                               None if spk_r is None else np.asarray(spk_r, np.float64))
        cond_rows.append(c)
        spk_rows.append(s)
    cond_rows = np.stack(cond_rows)
    spk_rows = None if spk_r is None else np.stack(spk_rows)
    nb = len(kinds)

    def velocity(t, x, guided):
        rows = slice(0, nb) if guided else slice(nb - 1, nb)
        n = nb if guided else 1
        x_rows = np.broadcast_to(x, (n,) + x.shape)
        valid_rows = np.broadcast_to(valid_r, (n,) + valid_r.shape)
        return O.estimator(W64, shape, x_rows, cond_rows[rows],
                           None if spk_rows is None else spk_rows[rows], t, valid_rows)

    return solve(x0_r, grid, velocity, scales, nb, policy, solver, valid=np.asarray(valid_r, bool))


_STATE = {}


def _init(W64, shape, grid, scales, kinds, policy, solver):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    _STATE.update(W64=W64, shape=shape, grid=grid, scales=scales, kinds=kinds, policy=policy, solver=solver)


def _task(args):
    x0_r, cond_r, spk_r, valid_r = args
    st = _STATE
    return sample_request(st["W64"], st["shape"], x0_r, cond_r, spk_r, valid_r, st["grid"], st["scales"],
                          st["kinds"], st["policy"], st["solver"])


def sample(weights: Dict[str, np.ndarray], shape, x0: np.ndarray, cond: np.ndarray,
           spk: Optional[np.ndarray], mask: Optional[np.ndarray], grid: np.ndarray,
           scales: Sequence[float], policy: GuidancePolicy = GuidancePolicy(), solver: str = "euler",
           kinds: Optional[Sequence[str]] = None, requests: Optional[Sequence[int]] = None,
           workers: int = 1) -> Tuple[np.ndarray, list]:
    """Batched sampler over ``grid``; returns (out [R', Tx, C] float64, per-request step records)."""
    kinds = tuple(kinds) if kinds is not None else O.default_kinds(shape)
    W64 = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
    R, Tx, _ = x0.shape
    valid = np.ones((R, Tx), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    idx = list(range(R)) if requests is None else list(requests)
    tasks = [(x0[r], cond[r], None if spk is None else spk[r], valid[r]) for r in idx]
    init = (W64, shape, np.asarray(grid, np.float64), tuple(scales), kinds, policy, solver)
    if workers <= 1 or len(tasks) <= 1:
        _init(*init)
        outs = [_task(a) for a in tasks]
    else:
        import concurrent.futures as cf
        import multiprocessing as mp
        with cf.ProcessPoolExecutor(max_workers=min(workers, len(tasks)), mp_context=mp.get_context("fork"),
                                    initializer=_init, initargs=init) as ex:
            outs = list(ex.map(_task, tasks))
    if not outs:
        return np.zeros((0,) + x0.shape[1:], dtype=np.float64), []
    return np.stack([o[0] for o in outs]), [o[1] for o in outs]
