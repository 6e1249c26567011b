"""CPU oracle for batched CFM / rectified-flow sampling with a DiT estimator.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module. The HIP library never
calls it, and it shares no code with the HIP library.

Plain, slow, float64 numpy. One request at a time: the branch rows of a request
are stacked along a leading batch axis and processed together; requests are
independent of each other, so a process pool over requests is allowed
(``sample(..., workers=n)``) and changes no result.

What is computed, and where it comes from:
  * VoiceHub "Diffusion and flow TTS optimization" (kadirnar.github.io/voicehub),
    "Active families" table: conditional flow matching / rectified flow sampled
    with classifier-free guidance and Euler steps.
  * same page, "Custom Triton and CUDA kernels": the estimator's repeated ops are
    adaptive-normalization modulation with residual gating, bias-GELU, and the
    guidance combine of the branch velocities fused with the Euler step.
  * same page, "Semantic-preserving and approximate changes" table: padded
    frames are fully masked and trimmed; packed CFG rows must equal separate
    calls with the same guidance equation.
  * vLLM-Omni TTS blog (shilu.ai), section "CFM/LocDiT decode-tail batching":
    the CFM estimator runs under CFG with two rows per request; many requests
    are batched into one estimator call.
The pages never write the estimator's equations. The readings used here
(time direction, embedding, adaLN layout, LN epsilon, GELU form, unconditional
branch, masks) are the plainest DiT/flow-matching ones and are listed one by one
in the design notes of this repository; each function below states its reading.
"""
from __future__ import annotations

import math
import os
from typing import Callable, Dict, Optional, Sequence

import numpy as np
from scipy.special import erf

LN_EPS = 1e-6          # LayerNorm epsilon (reading: DiT convention, no affine)
T_SCALE = 1000.0       # timestep argument scale of the sinusoidal embedding
T_BASE = 10000.0       # frequency base of the sinusoidal embedding


# ---------------------------------------------------------------- primitives

def timestep_grid(n_steps: int) -> np.ndarray:
    """Uniform grid t_k = k / S, k = 0..S; t = 0 is noise, t = 1 is data.

    Reading: the tiny benchmark case states "uniform Euler steps t_k = k/4";
    VoiceHub ("Reduce a 50-step sampler ...") keeps both endpoints and strict
    monotonicity of the grid.
    """
    return np.arange(n_steps + 1, dtype=np.float64) / float(n_steps)


def timestep_embedding(t: float, dim: int = 256) -> np.ndarray:
    """Sinusoidal embedding [cos(1000 t w_i) | sin(1000 t w_i)], w_i = 1e4^(-i/half)."""
    half = dim // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.exp(-math.log(T_BASE) * i / half)
    arg = T_SCALE * float(t) * omega
    return np.concatenate([np.cos(arg), np.sin(arg)])


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)) (VoiceHub's bias-GELU)."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b, W in [out, in] layout."""
    y = np.matmul(x, w.T)
    return y if b is None else y + b


def layer_norm(h: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis without affine: (h - mean) / sqrt(var + eps), biased var."""
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    return (h - mu) / np.sqrt(var + eps)


def modulate(u: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """adaLN modulation u * (1 + scale) + shift (VoiceHub: adaptive-normalization modulation)."""
    return u * (1.0 + scale) + shift


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     key_valid: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(hd) + key mask) v, non-causal, per batch row and head.

    q, k, v: [B, H, T, hd]; key_valid: [B, T] bool. Masked keys get probability
    0 (VoiceHub: padded values are fully masked). A row with no valid key gives
    an all-zero output (reading: the empty softmax contributes nothing).
    """
    B, H, Tq, hd = q.shape
    out = np.zeros((B, H, Tq, v.shape[-1]))
    for b in range(B):
        if not key_valid[b].any():
            continue
        bias = np.where(key_valid[b], 0.0, -np.inf)        # masked keys -> exp(-inf) = 0
        for h in range(H):
            s = np.matmul(q[b, h], k[b, h].T)
            s *= 1.0 / math.sqrt(hd)
            s += bias
            s -= s.max(axis=-1, keepdims=True)
            np.exp(s, out=s)
            s /= s.sum(axis=-1, keepdims=True)
            out[b, h] = np.matmul(s, v[b, h])
    return out


def guidance_combine(vs: np.ndarray, scales: Sequence[float]) -> np.ndarray:
    """Classifier-free guidance of the branch velocities vs[b].

    1 branch: v. 2 branches (uncond, cond): v_u + s (v_c - v_u).
    3 branches (uncond, text, text+speaker): v_u + s_t (v_t - v_u) + s_s (v_ts - v_t),
    the multi-condition form of the rectified-flow benchmark case (VoiceHub lists
    "independent text/speaker CFG" for its rectified-flow family).
    """
    nb = vs.shape[0]
    if nb == 1:
        return vs[0]
    if nb == 2:
        (s,) = scales
        return vs[0] + s * (vs[1] - vs[0])
    if nb == 3:
        st, ss = scales
        return vs[0] + st * (vs[1] - vs[0]) + ss * (vs[2] - vs[1])
    raise ValueError(nb)


# ---------------------------------------------------------------- estimator

def _f64(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}


def conditioning_vector(W: Dict[str, np.ndarray], t: float, spk_b: Optional[np.ndarray],
                        t_freq_dim: int) -> np.ndarray:
    """Global condition c = W2 SiLU(W1 e(t) + b1) + b2 (+ W_s spk + b_s when a speaker path exists)."""
    e = timestep_embedding(t, t_freq_dim)
    c = linear(silu(linear(e, W["t_embed.fc1.weight"], W["t_embed.fc1.bias"])),
               W["t_embed.fc2.weight"], W["t_embed.fc2.bias"])
    if "spk_proj.weight" in W:
        c = c + linear(spk_b, W["spk_proj.weight"], W["spk_proj.bias"])
    return c


def branch_inputs(kind: str, cond_r: np.ndarray, spk_r: Optional[np.ndarray]):
    """Condition inputs seen by one branch; an absent condition is zeroed.

    Reading: the unconditional branch is the same model with its condition
    input removed (set to zero); in the three-branch case the text branch also
    has its speaker vector zeroed.
    """
    has_cond = kind in ("cond", "cond_spk")
    has_spk = kind == "cond_spk"
    c = cond_r if has_cond else np.zeros_like(cond_r)
    s = None
    if spk_r is not None:
        s = spk_r if has_spk else np.zeros_like(spk_r)
    return c, s


def estimator(W: Dict[str, np.ndarray], shape, x_rows: np.ndarray, cond_rows: np.ndarray,
              spk_rows: Optional[np.ndarray], t: float, frame_valid: np.ndarray) -> np.ndarray:
    """DiT velocity for a stack of B rows (float64 weights).

    x_rows [B, Tx, C], cond_rows [B, Tc, Cc], spk_rows [B, spk] or None,
    frame_valid [B, Tx] bool. Returns v [B, Tx, C] with v = 0 on masked frames.
    """
    B, Tx, C = x_rows.shape
    d, H, L = shape.d_model, shape.n_heads, shape.n_layers
    hd = d // H

    # global condition per row -> SiLU once; shared by every adaLN projection
    cs = np.stack([conditioning_vector(W, t, None if spk_rows is None else spk_rows[b],
                                       shape.t_freq_dim) for b in range(B)])    # [B, d]
    sc = silu(cs)[:, None, :]                                                   # [B, 1, d]

    # input projection: channel concat [x | cond] per frame, or prefix frames
    if shape.cond_mode == "channel":
        seq = np.concatenate([x_rows, cond_rows], axis=-1)
        key_valid = frame_valid
        n_pre = 0
    else:
        seq = np.concatenate([cond_rows, x_rows], axis=1)
        n_pre = cond_rows.shape[1]
        key_valid = np.concatenate([np.ones((B, n_pre), dtype=bool), frame_valid], axis=1)
    h = linear(seq, W["in_proj.weight"], W["in_proj.bias"])                       # [B, T, d]
    T = h.shape[1]

    for l in range(L):
        p = f"blocks.{l}."
        mod = linear(sc, W[p + "ada.weight"], W[p + "ada.bias"])                 # [B, 1, 6d]
        sh1, sc1, g1, sh2, sc2, g2 = np.split(mod, 6, axis=-1)
        u = modulate(layer_norm(h), sh1, sc1)
        qkv = linear(u, W[p + "qkv.weight"], W[p + "qkv.bias"])                  # [B, T, 3d]
        q, k, v = np.split(qkv, 3, axis=-1)
        heads = lambda z: z.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        o = masked_attention(heads(q), heads(k), heads(v), key_valid)           # [B, H, T, hd]
        o = o.transpose(0, 2, 1, 3).reshape(B, T, d)
        h = h + g1 * linear(o, W[p + "proj.weight"], W[p + "proj.bias"])
        u = modulate(layer_norm(h), sh2, sc2)
        ff = gelu(linear(u, W[p + "fc1.weight"], W[p + "fc1.bias"]))
        h = h + g2 * linear(ff, W[p + "fc2.weight"], W[p + "fc2.bias"])

    fm = linear(sc, W["final.ada.weight"], W["final.ada.bias"])
    shf, scf = np.split(fm, 2, axis=-1)
    u = modulate(layer_norm(h), shf, scf)
    vel = linear(u, W["final.out.weight"], W["final.out.bias"])[:, n_pre:, :]    # [B, Tx, C]
    return np.where(frame_valid[:, :, None], vel, 0.0)


# ---------------------------------------------------------------- sampler

def euler_cfg(x0_r: np.ndarray, n_steps: int,
              branch_velocity: Callable[[float, np.ndarray], np.ndarray],
              scales: Sequence[float]) -> np.ndarray:
    """Explicit Euler over the uniform grid with guidance: x <- x + dt_k * combine(v_b(t_k, x)).

    ``branch_velocity(t, x)`` returns the stacked branch velocities [nb, ...].
    Reading: the velocity is evaluated at the left end t_k of each step.
    """
    t = timestep_grid(n_steps) if n_steps > 0 else np.zeros(1)
    x = np.asarray(x0_r, dtype=np.float64).copy()
    for k in range(n_steps):
        vs = branch_velocity(t[k], x)
        x = x + (t[k + 1] - t[k]) * guidance_combine(vs, scales)
    return x


def sample_request(W64: Dict[str, np.ndarray], shape, x0_r, cond_r, spk_r, valid_r,
                   n_steps: int, scales: Sequence[float], kinds: Sequence[str]) -> np.ndarray:
    """All branches of one request through the whole sampler; returns x after S steps [Tx, C]."""
    cond_rows, spk_rows = [], []
    for kind in kinds:
        c, s = branch_inputs(kind, np.asarray(cond_r, np.float64),
                             None if spk_r is None else np.asarray(spk_r, np.float64))
        cond_rows.append(c)
        spk_rows.append(s)
    cond_rows = np.stack(cond_rows)
    spk_rows = None if spk_r is None else np.stack(spk_rows)
    nb = len(kinds)
    valid_rows = np.broadcast_to(valid_r, (nb,) + valid_r.shape)

    def branch_velocity(t, x):
        x_rows = np.broadcast_to(x, (nb,) + x.shape)
        return estimator(W64, shape, x_rows, cond_rows, spk_rows, t, valid_rows)

    return euler_cfg(x0_r, n_steps, branch_velocity, scales)


def default_kinds(shape) -> tuple:
    """Branch order inside a request; rows are branch-major (row = b * R + r).

    2 branches: (uncond, cond) -- or (uncond, cond_spk) when a speaker input
    exists; 3 branches: (uncond, text, text+speaker); 1 branch: conditional.
    """
    nb, has_spk = shape.n_branches, shape.spk_dim > 0
    if nb == 1:
        return ("cond_spk",) if has_spk else ("cond",)
    if nb == 2:
        return ("uncond", "cond_spk") if has_spk else ("uncond", "cond")
    if nb == 3:
        return ("uncond", "cond", "cond_spk")
    raise ValueError(nb)


_WORKER_STATE = {}


def _worker_init(W64, shape, n_steps, scales, kinds):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    _WORKER_STATE.update(W64=W64, shape=shape, n_steps=n_steps, scales=scales, kinds=kinds)


def _request_task(args):
    x0_r, cond_r, spk_r, valid_r = args
    st = _WORKER_STATE
    return sample_request(st["W64"], st["shape"], x0_r, cond_r, spk_r, valid_r,
                          st["n_steps"], st["scales"], st["kinds"])


def sample(weights: Dict[str, np.ndarray], shape, x0: np.ndarray, cond: np.ndarray,
           spk: Optional[np.ndarray], mask: Optional[np.ndarray], n_steps: int,
           scales: Sequence[float], kinds: Optional[Sequence[str]] = None,
           requests: Optional[Sequence[int]] = None, workers: int = 1) -> np.ndarray:
    """Batched sampler: every request with all of its branches; returns out [R', Tx, C] float64.

    ``requests`` restricts the run to a subset of request indices (results are
    identical to the full run's rows, since requests never interact).
    ``workers`` > 1 runs requests in forked worker processes with one BLAS
    thread each; the weights reach the workers by inheritance, not by copy.
    """
    kinds = tuple(kinds) if kinds is not None else default_kinds(shape)
    W64 = _f64(weights)
    R, Tx, _ = x0.shape
    valid = np.ones((R, Tx), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    idx = list(range(R)) if requests is None else list(requests)
    tasks = [(x0[r], cond[r], None if spk is None else spk[r], valid[r]) for r in idx]
    init = (W64, shape, n_steps, tuple(scales), kinds)
    if workers <= 1 or len(tasks) <= 1:
        _WORKER_STATE.update(W64=W64, shape=shape, n_steps=n_steps, scales=tuple(scales), kinds=kinds)
        outs = [_request_task(a) for a in tasks]
    else:
        import concurrent.futures as cf
        import multiprocessing as mp
        with cf.ProcessPoolExecutor(max_workers=min(workers, len(tasks)),
                                    mp_context=mp.get_context("fork"),
                                    initializer=_worker_init, initargs=init) as ex:
            outs = list(ex.map(_request_task, tasks))
    if not outs:
        return np.zeros((0,) + x0.shape[1:], dtype=np.float64)
    return np.stack(outs)


def host_cores() -> int:
    return len(os.sched_getaffinity(0))
