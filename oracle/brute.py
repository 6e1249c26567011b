"""Brute-force CPU sampler in pure Python loops -- TEST INFRASTRUCTURE ONLY.

A second, independent statement of the same sampler as ``oracle.sampler``,
written with scalar loops and the ``math`` module only (no numpy, no shared
helpers), for tiny inputs. Its purpose is to catch a wrong index, a transposed
operand, a dropped term or a wrong sign in the vectorised oracle: the two are
compared end to end on a tiny workload.

Pages behind it: VoiceHub "Diffusion and flow TTS optimization" (active
families: CFM/RF with CFG and Euler; custom kernels: adaptive-norm modulation
and residual gating, bias-GELU, the guidance combine fused with the Euler step; padding fully
masked) and the vLLM-Omni TTS blog, "CFM/LocDiT decode-tail batching".

Conventions (same readings as the vectorised oracle, restated independently):
weights are [out][in]; uniform grid t_k = k/S from noise (0) to data (1);
e(t) = [cos(1000 t f_i)]_i ++ [sin(1000 t f_i)]_i with f_i = 10000^(-i/128);
c = W2 silu(W1 e + b1) + b2 (+ Ws spk + bs); per layer six modulation vectors
(shift1, scale1, gate1, shift2, scale2, gate2) from Wada silu(c) + bada;
LayerNorm without affine, biased variance, eps 1e-6; exact GELU; key-padding
mask; final (shift, scale) then output projection; masked frames give 0.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence


def _mat(a) -> List[List[float]]:
    return [[float(v) for v in row] for row in a]


def _vec(a) -> List[float]:
    return [float(v) for v in a]


def bf_linear(rows: List[List[float]], W: List[List[float]], b: Optional[List[float]]) -> List[List[float]]:
    out = []
    for x in rows:
        y = []
        for o in range(len(W)):
            acc = 0.0
            wo = W[o]
            for i in range(len(x)):
                acc += x[i] * wo[i]
            if b is not None:
                acc += b[o]
            y.append(acc)
        out.append(y)
    return out


def bf_silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def bf_gelu(z: float) -> float:
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def bf_layer_norm_row(x: List[float], eps: float = 1e-6) -> List[float]:
    n = len(x)
    mean = 0.0
    for v in x:
        mean += v
    mean /= n
    var = 0.0
    for v in x:
        var += (v - mean) * (v - mean)
    var /= n
    inv = 1.0 / math.sqrt(var + eps)
    return [(v - mean) * inv for v in x]


def bf_attention(q: List[List[float]], k: List[List[float]], v: List[List[float]],
                 key_valid: List[bool], n_heads: int) -> List[List[float]]:
    """Per head, per query: weights exp(s_j - max) over valid keys only, normalised."""
    T = len(q)
    d = len(q[0])
    hd = d // n_heads
    scale = 1.0 / math.sqrt(hd)
    out = [[0.0] * d for _ in range(T)]
    for h in range(n_heads):
        lo = h * hd
        for i in range(T):
            scores = []
            for j in range(T):
                if not key_valid[j]:
                    continue
                s = 0.0
                for e in range(hd):
                    s += q[i][lo + e] * k[j][lo + e]
                scores.append((j, s * scale))
            if not scores:
                continue
            mx = max(s for _, s in scores)
            ws = [(j, math.exp(s - mx)) for j, s in scores]
            z = sum(w for _, w in ws)
            for e in range(hd):
                acc = 0.0
                for j, w in ws:
                    acc += w * v[j][lo + e]
                out[i][lo + e] = acc / z
    return out


def bf_timestep_embedding(t: float, dim: int) -> List[float]:
    half = dim // 2
    cos_part, sin_part = [], []
    for i in range(half):
        f = 10000.0 ** (-i / half)
        cos_part.append(math.cos(1000.0 * t * f))
        sin_part.append(math.sin(1000.0 * t * f))
    return cos_part + sin_part


def bf_velocity(W: Dict[str, list], shape, x: List[List[float]], cond: List[List[float]],
                spk: Optional[List[float]], t: float, frame_valid: List[bool]) -> List[List[float]]:
    """One row of the DiT estimator; x [Tx][C], cond [Tc][Cc]. Returns v [Tx][C]."""
    d = shape.d_model
    e = bf_timestep_embedding(t, shape.t_freq_dim)
    hid = [bf_silu(z) for z in bf_linear([e], W["t_embed.fc1.weight"], W["t_embed.fc1.bias"])[0]]
    c = bf_linear([hid], W["t_embed.fc2.weight"], W["t_embed.fc2.bias"])[0]
    if "spk_proj.weight" in W:
        sp = bf_linear([spk], W["spk_proj.weight"], W["spk_proj.bias"])[0]
        c = [c[i] + sp[i] for i in range(d)]
    sc = [bf_silu(z) for z in c]

    if shape.cond_mode == "channel":
        tokens = [x[t_] + cond[t_] for t_ in range(len(x))]
        key_valid = list(frame_valid)
        n_pre = 0
    else:
        tokens = [list(r) for r in cond] + [list(r) for r in x]
        n_pre = len(cond)
        key_valid = [True] * n_pre + list(frame_valid)
    h = bf_linear(tokens, W["in_proj.weight"], W["in_proj.bias"])
    T = len(h)

    for l in range(shape.n_layers):
        p = f"blocks.{l}."
        m = bf_linear([sc], W[p + "ada.weight"], W[p + "ada.bias"])[0]
        shift1, scale1, gate1 = m[0:d], m[d:2 * d], m[2 * d:3 * d]
        shift2, scale2, gate2 = m[3 * d:4 * d], m[4 * d:5 * d], m[5 * d:6 * d]
        u = []
        for i in range(T):
            n = bf_layer_norm_row(h[i])
            u.append([n[j] * (1.0 + scale1[j]) + shift1[j] for j in range(d)])
        qkv = bf_linear(u, W[p + "qkv.weight"], W[p + "qkv.bias"])
        q = [r[0:d] for r in qkv]
        k = [r[d:2 * d] for r in qkv]
        v = [r[2 * d:3 * d] for r in qkv]
        o = bf_attention(q, k, v, key_valid, shape.n_heads)
        a = bf_linear(o, W[p + "proj.weight"], W[p + "proj.bias"])
        for i in range(T):
            for j in range(d):
                h[i][j] += gate1[j] * a[i][j]
        u = []
        for i in range(T):
            n = bf_layer_norm_row(h[i])
            u.append([n[j] * (1.0 + scale2[j]) + shift2[j] for j in range(d)])
        g = [[bf_gelu(z) for z in r] for r in bf_linear(u, W[p + "fc1.weight"], W[p + "fc1.bias"])]
        f = bf_linear(g, W[p + "fc2.weight"], W[p + "fc2.bias"])
        for i in range(T):
            for j in range(d):
                h[i][j] += gate2[j] * f[i][j]

    m = bf_linear([sc], W["final.ada.weight"], W["final.ada.bias"])[0]
    shift_f, scale_f = m[0:d], m[d:2 * d]
    u = []
    for i in range(n_pre, T):
        n = bf_layer_norm_row(h[i])
        u.append([n[j] * (1.0 + scale_f[j]) + shift_f[j] for j in range(d)])
    vel = bf_linear(u, W["final.out.weight"], W["final.out.bias"])
    C = len(vel[0])
    return [vel[i] if frame_valid[i] else [0.0] * C for i in range(len(vel))]


def bf_sample(weights, shape, x0, cond, spk, mask, n_steps: int, scales: Sequence[float]):
    """Whole sampler, request by request; returns nested lists [R][Tx][C]."""
    W = {}
    for name, a in weights.items():
        W[name] = _mat(a) if getattr(a, "ndim", 1) == 2 else _vec(a)
    R = len(x0)
    out = []
    nb = shape.n_branches
    for r in range(R):
        x = _mat(x0[r])
        cond_r = _mat(cond[r])
        zeros_cond = [[0.0] * len(cond_r[0]) for _ in cond_r]
        spk_r = None if spk is None else _vec(spk[r])
        zeros_spk = None if spk_r is None else [0.0] * len(spk_r)
        valid = [True] * len(x) if mask is None else [bool(m) for m in mask[r]]
        # branch inputs: b = 0 has no condition; b >= 1 has the condition;
        # the speaker vector is seen only by the last of three branches
        # (or by the conditional branch of a two-branch speaker model).
        branch_in = []
        for b in range(nb):
            cb = cond_r if (nb == 1 or b >= 1) else zeros_cond
            if spk_r is None:
                sb = None
            else:
                sb = spk_r if (b == nb - 1 and (nb == 1 or b >= 1)) else zeros_spk
            branch_in.append((cb, sb))
        for k in range(n_steps):
            t = k / n_steps
            dt = (k + 1) / n_steps - k / n_steps
            vs = [bf_velocity(W, shape, x, cb, sb, t, valid) for cb, sb in branch_in]
            for i in range(len(x)):
                for c in range(len(x[0])):
                    if nb == 1:
                        g = vs[0][i][c]
                    elif nb == 2:
                        g = vs[0][i][c] + scales[0] * (vs[1][i][c] - vs[0][i][c])
                    else:
                        g = (vs[0][i][c] + scales[0] * (vs[1][i][c] - vs[0][i][c])
                             + scales[1] * (vs[2][i][c] - vs[1][i][c]))
                    x[i][c] += dt * g
        out.append(x)
    return out
