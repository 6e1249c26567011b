"""CPU oracle for approximate block-residual caching (DBCache / first-block cache)
in the CFM sampler.

TEST INFRASTRUCTURE ONLY, like ``oracle.sampler`` (whose primitives it reuses):
only the test suite, the package's smoke check and the benchmark's CPU-baseline leg
may import it; the HIP library shares no code with it. Plain float64 numpy.

Source: VoiceHub "Diffusion and flow TTS optimization", section "Approximate
block-residual caching": the first Fn blocks always run and their output (the
probe) is compared with the previous probe by a normalised relative-L1 score; on
a step that must compute, the middle blocks run and their aggregate residual is
saved; on a cache hit they are skipped and the latest saved residual is added
(predictor "reuse"); the last Bn blocks always run. Warm-up steps always compute,
a limit on consecutive cached steps and an accumulated-error budget force
refreshes, and an explicit per-step mask can force computation. Packed CFG is one
lane.

Readings (the page gives the rules, not formulas; each is listed in the design
notes of this repository):
  C1  lane: one sampling call's packed batch (every request and CFG branch row of
      the call); the score is taken over all of its rows' valid frames, so one
      decision per estimator evaluation covers the whole batch;
  C2  score = sum |probe - probe_prev| / sum |probe_prev| over valid tokens, probe =
      hidden state after the first Fn blocks, probe_prev = the previous
      evaluation's probe (updated at every evaluation);
  C3  an evaluation computes when: it is forced by the mask, it is among the
      first `warmup` evaluations, no residual is saved yet, `max_cached` hits have
      been taken (when >= 0), `max_consecutive` hits in a row have been taken, the
      score is not below the threshold, or the accepted scores since the last
      computation plus this one exceed the budget; otherwise it is a hit;
  C4  a computing evaluation saves residual = (state after the middle blocks) -
      (state before them) and resets the consecutive count and the accumulated
      score; a hit adds the saved residual, increments both and adds its score;
  C5  every estimator evaluation is a cache step (Euler: one per solver step).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from oracle import sampler as O


@dataclass(frozen=True)
class CachePolicy:
    front: int = 1                 # Fn
    back: int = 1                  # Bn
    threshold: float = 0.05
    warmup: int = 3
    max_consecutive: int = 2
    max_cached: int = -1           # -1: unlimited
    budget: float = 0.12           # max accumulated relative error
    force: Tuple[bool, ...] = ()   # per-evaluation forced computation (missing entries: False)


def _block(W, l, shape, h, sc, heads_fn, key_valid):
    """One adaLN-Zero DiT block (the same arithmetic as the plain oracle's estimator)."""
    p = f"blocks.{l}."
    d, H = shape.d_model, shape.n_heads
    B, T, _ = h.shape
    mod = O.linear(sc, W[p + "ada.weight"], W[p + "ada.bias"])
    sh1, sc1, g1, sh2, sc2, g2 = np.split(mod, 6, axis=-1)
    u = O.modulate(O.layer_norm(h), sh1, sc1)
    qkv = O.linear(u, W[p + "qkv.weight"], W[p + "qkv.bias"])
    q, k, v = np.split(qkv, 3, axis=-1)
    o = O.masked_attention(heads_fn(q), heads_fn(k), heads_fn(v), key_valid)
    o = o.transpose(0, 2, 1, 3).reshape(B, T, d)
    h = h + g1 * O.linear(o, W[p + "proj.weight"], W[p + "proj.bias"])
    u = O.modulate(O.layer_norm(h), sh2, sc2)
    ff = O.gelu(O.linear(u, W[p + "fc1.weight"], W[p + "fc1.bias"]))
    return h + g2 * O.linear(ff, W[p + "fc2.weight"], W[p + "fc2.bias"])


class CacheState:
    """Per-lane state of the block-residual cache across the evaluations of one call."""

    def __init__(self, policy: CachePolicy):
        self.p = policy
        self.evals = 0
        self.probe_prev: Optional[np.ndarray] = None
        self.residual: Optional[np.ndarray] = None
        self.consecutive = 0
        self.hits = 0
        self.accumulated = 0.0
        self.log: List[dict] = []

    def decide(self, probe: np.ndarray, valid_tok: np.ndarray) -> Tuple[bool, float]:
        """(compute?, score) for this evaluation (readings C2, C3); updates probe_prev."""
        p, j = self.p, self.evals
        score = float("nan")
        if self.probe_prev is not None:
            diff = np.abs(probe - self.probe_prev)[valid_tok].sum()
            den = np.abs(self.probe_prev)[valid_tok].sum()
            score = float(diff / den) if den > 0 else 0.0
        self.probe_prev = probe.copy()
        forced = j < len(p.force) and bool(p.force[j])
        compute = (forced or j < p.warmup or self.residual is None
                   or (p.max_cached >= 0 and self.hits >= p.max_cached)
                   or self.consecutive >= p.max_consecutive
                   or not score < p.threshold
                   or self.accumulated + score > p.budget)
        return compute, score


def estimator_cached(W: Dict[str, np.ndarray], shape, x_rows, cond_rows, spk_rows, t: float,
                     frame_valid: np.ndarray, st: CacheState) -> np.ndarray:
    """Velocities of a stack of rows (the whole lane) with the block-residual cache."""
    B, Tx, C = x_rows.shape
    d, H, L = shape.d_model, shape.n_heads, shape.n_layers
    hd = d // H
    cs = np.stack([O.conditioning_vector(W, t, None if spk_rows is None else spk_rows[b], shape.t_freq_dim)
                   for b in range(B)])
    sc = O.silu(cs)[:, None, :]
    if shape.cond_mode == "channel":
        seq = np.concatenate([x_rows, cond_rows], axis=-1)
        key_valid = frame_valid
        n_pre = 0
    else:
        seq = np.concatenate([cond_rows, x_rows], axis=1)
        n_pre = cond_rows.shape[1]
        key_valid = np.concatenate([np.ones((B, n_pre), dtype=bool), frame_valid], axis=1)
    h = O.linear(seq, W["in_proj.weight"], W["in_proj.bias"])
    T = h.shape[1]
    heads = lambda z: z.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    p = st.p
    front, back = min(p.front, L), min(p.back, max(L - p.front, 0))
    for l in range(front):
        h = _block(W, l, shape, h, sc, heads, key_valid)
    if front + back < L:          # there are middle blocks to cache
        valid_tok = np.broadcast_to(key_valid[:, :, None], h.shape)
        compute, score = st.decide(h, valid_tok)
        if compute:
            h_in = h
            for l in range(front, L - back):
                h = _block(W, l, shape, h, sc, heads, key_valid)
            st.residual = h - h_in
            st.consecutive = 0
            st.accumulated = 0.0
        else:
            h = h + st.residual
            st.consecutive += 1
            st.hits += 1
            st.accumulated += score
        st.log.append({"eval": st.evals, "compute": compute, "score": score})
    for l in range(L - back, L):
        h = _block(W, l, shape, h, sc, heads, key_valid)
    st.evals += 1
    fm = O.linear(sc, W["final.ada.weight"], W["final.ada.bias"])
    shf, scf = np.split(fm, 2, axis=-1)
    u = O.modulate(O.layer_norm(h), shf, scf)
    vel = O.linear(u, W["final.out.weight"], W["final.out.bias"])[:, n_pre:, :]
    return np.where(frame_valid[:, :, None], vel, 0.0)


def sample(weights: Dict[str, np.ndarray], shape, x0: np.ndarray, cond: np.ndarray, spk: Optional[np.ndarray],
           mask: Optional[np.ndarray], n_steps: int, scales: Sequence[float], policy: CachePolicy,
           kinds: Optional[Sequence[str]] = None):
    """The whole batch as one cache lane, uniform Euler grid; returns (out [R, Tx, C], decision log)."""
    kinds = tuple(kinds) if kinds is not None else O.default_kinds(shape)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
    R, Tx, _ = x0.shape
    nb = len(kinds)
    valid = np.ones((R, Tx), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    # rows branch-major, row = b * R + r, as the batched library lays them out
    cond_rows, spk_rows = [], []
    for kind in kinds:
        for r in range(R):
            c, s_ = O.branch_inputs(kind, np.asarray(cond[r], np.float64),
                                    None if spk is None else np.asarray(spk[r], np.float64))
            cond_rows.append(c)
            spk_rows.append(s_)
    cond_rows = np.stack(cond_rows)
    spk_rows = None if spk is None else np.stack(spk_rows)
    valid_rows = np.concatenate([valid] * nb)
    st = CacheState(policy)
    t = O.timestep_grid(n_steps) if n_steps > 0 else np.zeros(1)
    x = np.asarray(x0, dtype=np.float64).copy()
    for k in range(n_steps):
        x_rows = np.concatenate([x] * nb)
        v = estimator_cached(W, shape, x_rows, cond_rows, spk_rows, t[k], valid_rows, st)
        vs = v.reshape(nb, R, Tx, -1)
        x = x + (t[k + 1] - t[k]) * O.guidance_combine(vs, scales)
    return x, st.log
