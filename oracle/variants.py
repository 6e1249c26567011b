"""CPU oracle for the DiT block variants of the CFM sampler: RMSNorm, the fused
gate-up SwiGLU MLP, rotary position embedding (RoPE) on the self-attention, and
cross-attention to condition keys/values that stay fixed over the steps.

TEST INFRASTRUCTURE ONLY, like ``oracle.sampler`` (whose pinned primitives it
reuses): only the test suite, the package's smoke check and the benchmark's
CPU-baseline leg may import it; the HIP library shares no code with it. Plain
float64 numpy.

Sources:
  * VoiceHub "Diffusion and flow TTS optimization", section "Custom Triton and
    CUDA kernels": RMSNorm and SwiGLU are among the repeated patterns of these
    estimators;
  * vLLM-Omni TTS blog, section "CFM/LocDiT decode-tail batching": the LocDiT
    runs a fused QKV projection and a fused gate-up MLP;
  * VoiceHub, "Recommended optimization boundaries" table, rows Echo and
    Irodori-TTS: the denoiser keeps condition (context) keys/values and RoPE
    caches across calls.
The pages name these parts and give no formulas; the readings (listed one by one
in the design notes of this repository):
  V1  RMSNorm(h) = h / sqrt(mean(h^2) + 1e-6) over the model width, no affine
      (the adaLN modulation supplies scale and shift, as for the LayerNorm);
      the block's two norms, the cross-attention norm and the final norm all
      follow the configured kind;
  V2  SwiGLU: the fused FC1 weight stacks the gate rows over the up rows
      ([2 f, d], bias [2 f]); act = SiLU(gate) * up, then FC2 [d, f];
  V3  RoPE (RoFormer, Su et al. 2021): feature pairs (2i, 2i+1) of every head of
      the self-attention queries and keys are rotated by the angle p * theta_i,
      theta_i = base^(-2i / head_dim), base 10000, p = the token's index in its
      row's sequence (prefix tokens first); values and the cross-attention are
      not rotated;
  V4  cross-attention sublayer between the self-attention and the MLP, without
      adaLN modulation or gate: h += W_o attn(W_q norm(h) + b_q, K, V) + b_o with
      [K | V] = W_kv ctx + b_kv over the row's context tokens, all of them valid;
      K and V depend only on the context, so they are computed once per call;
  V5  in the cross mode the condition input is the context [R, Tc, cond_dim]:
      the input projection sees the latent alone, the unconditional branch
      sees a zero context, and the sequence holds the generated frames only.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from oracle import sampler as O

NORM_EPS = O.LN_EPS


def rms_norm(h: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """V1: h / sqrt(mean(h^2) + eps) over the last axis."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def norm(kind: str, h: np.ndarray) -> np.ndarray:
    return rms_norm(h) if kind == "rms" else O.layer_norm(h)


def swiglu(z: np.ndarray) -> np.ndarray:
    """V2: z = [gate | up] along the last axis; SiLU(gate) * up."""
    f = z.shape[-1] // 2
    return O.silu(z[..., :f]) * z[..., f:]


def rope_angles(positions: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """V3: angle[p, i] = positions[p] * base^(-2 i / head_dim), i < head_dim / 2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    return np.asarray(positions, np.float64)[:, None] * theta[None, :]


def apply_rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotates pairs (2i, 2i+1) of the last axis of x [..., T, head_dim] by the
    angles of V3 for the T positions."""
    ang = rope_angles(positions, x.shape[-1], base)          # [T, hd/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def estimator(W: Dict[str, np.ndarray], shape, x_rows: np.ndarray, cond_rows: np.ndarray,
              spk_rows: Optional[np.ndarray], t: float, frame_valid: np.ndarray) -> np.ndarray:
    """DiT velocity of a stack of B rows with the configured block variants (float64).

    Same inputs and output as ``oracle.sampler.estimator``; with norm "layer",
    MLP "gelu", no RoPE and a channel or prefix condition it computes the same
    function. cond_rows is the context [B, Tc, cond_dim] in the cross mode.
    """
    B, Tx, C = x_rows.shape
    d, H, L = shape.d_model, shape.n_heads, shape.n_layers
    hd = d // H
    kind = shape.norm
    cs = np.stack([O.conditioning_vector(W, t, None if spk_rows is None else spk_rows[b], shape.t_freq_dim)
                   for b in range(B)])
    sc = O.silu(cs)[:, None, :]

    if shape.cond_mode == "channel":
        seq = np.concatenate([x_rows, cond_rows], axis=-1)
        key_valid, n_pre = frame_valid, 0
    elif shape.cond_mode == "prefix":
        seq = np.concatenate([cond_rows, x_rows], axis=1)
        n_pre = cond_rows.shape[1]
        key_valid = np.concatenate([np.ones((B, n_pre), dtype=bool), frame_valid], axis=1)
    else:   # cross (V5)
        seq = x_rows
        key_valid, n_pre = frame_valid, 0
    h = O.linear(seq, W["in_proj.weight"], W["in_proj.bias"])
    T = h.shape[1]
    pos = np.arange(T)
    heads = lambda z, n: z.reshape(B, n, H, hd).transpose(0, 2, 1, 3)

    for l in range(L):
        p = f"blocks.{l}."
        mod = O.linear(sc, W[p + "ada.weight"], W[p + "ada.bias"])
        sh1, sc1, g1, sh2, sc2, g2 = np.split(mod, 6, axis=-1)
        u = O.modulate(norm(kind, h), sh1, sc1)
        q, k, v = np.split(O.linear(u, W[p + "qkv.weight"], W[p + "qkv.bias"]), 3, axis=-1)
        q, k, v = heads(q, T), heads(k, T), heads(v, T)
        if shape.rope:
            q, k = apply_rope(q, pos, shape.rope_base), apply_rope(k, pos, shape.rope_base)
        o = O.masked_attention(q, k, v, key_valid).transpose(0, 2, 1, 3).reshape(B, T, d)
        h = h + g1 * O.linear(o, W[p + "proj.weight"], W[p + "proj.bias"])
        if shape.cond_mode == "cross":    # V4
            Tc = cond_rows.shape[1]
            kx, vx = np.split(O.linear(cond_rows, W[p + "xattn.kv.weight"], W[p + "xattn.kv.bias"]), 2, axis=-1)
            qx = O.linear(norm(kind, h), W[p + "xattn.q.weight"], W[p + "xattn.q.bias"])
            ox = O.masked_attention(heads(qx, T), heads(kx, Tc), heads(vx, Tc), np.ones((B, Tc), dtype=bool))
            ox = ox.transpose(0, 2, 1, 3).reshape(B, T, d)
            h = h + O.linear(ox, W[p + "xattn.out.weight"], W[p + "xattn.out.bias"])
        u = O.modulate(norm(kind, h), sh2, sc2)
        z = O.linear(u, W[p + "fc1.weight"], W[p + "fc1.bias"])
        ff = swiglu(z) if shape.mlp == "swiglu" else O.gelu(z)
        h = h + g2 * O.linear(ff, W[p + "fc2.weight"], W[p + "fc2.bias"])

    fm = O.linear(sc, W["final.ada.weight"], W["final.ada.bias"])
    shf, scf = np.split(fm, 2, axis=-1)
    u = O.modulate(norm(kind, h), shf, scf)
    vel = O.linear(u, W["final.out.weight"], W["final.out.bias"])[:, n_pre:, :]
    return np.where(frame_valid[:, :, None], vel, 0.0)


def sample(weights: Dict[str, np.ndarray], shape, x0: np.ndarray, cond: np.ndarray,
           spk: Optional[np.ndarray], mask: Optional[np.ndarray], n_steps: int,
           scales: Sequence[float], kinds: Optional[Sequence[str]] = None,
           requests: Optional[Sequence[int]] = None) -> np.ndarray:
    """Uniform-grid Euler sampler with guidance (``oracle.sampler.euler_cfg``) around
    the variant estimator, one request at a time; returns out [R', Tx, C] float64."""
    kinds = tuple(kinds) if kinds is not None else O.default_kinds(shape)
    W = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
    R, Tx, _ = x0.shape
    valid = np.ones((R, Tx), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    outs = []
    for r in (range(R) if requests is None else requests):
        conds, spks = [], []
        for kind in kinds:
            c, s_ = O.branch_inputs(kind, np.asarray(cond[r], np.float64),
                                    None if spk is None else np.asarray(spk[r], np.float64))
            conds.append(c)
            spks.append(s_)
        cond_rows = np.stack(conds)
        spk_rows = None if spk is None else np.stack(spks)
        nb = len(kinds)
        valid_rows = np.broadcast_to(valid[r], (nb, Tx))

        def branch_velocity(t, x):
            return estimator(W, shape, np.broadcast_to(x, (nb,) + x.shape), cond_rows, spk_rows, t, valid_rows)

        outs.append(O.euler_cfg(x0[r], n_steps, branch_velocity, scales))
    if not outs:
        return np.zeros((0,) + x0.shape[1:], dtype=np.float64)
    return np.stack(outs)
