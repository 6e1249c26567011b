"""Pins of the block-variant oracle (oracle/variants.py) on the CPU.

RMSNorm and SwiGLU against torch's own routines, RoPE against its complex-number
form and its defining property (scores depend on relative position only),
cross-attention against torch's scaled_dot_product_attention, and the whole
variant estimator against an independent torch twin written here from the same
readings (different library, different RoPE formulation, different head split).
With every variant off the variant estimator is the plain oracle's.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import sampler as O
from oracle import variants as V


def _tiny(**kw):
    return synth.workload("tiny_f32_variants").replace(**kw)


def test_rms_norm_matches_torch_and_closed_form():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((3, 5, 64)) * 2 + 0.5
    want = F.rms_norm(torch.from_numpy(h), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(V.rms_norm(h), want, rtol=1e-13, atol=1e-13)
    c = np.full((1, 64), -3.0)          # constant row c: sign(c) / sqrt(1 + eps / c^2)
    np.testing.assert_allclose(V.rms_norm(c), -1.0 / math.sqrt(1 + 1e-6 / 9.0), rtol=1e-15)
    y = V.rms_norm(h)                   # unit mean square (up to eps)
    np.testing.assert_allclose((y * y).mean(-1), 1.0, rtol=1e-5)
    assert not np.allclose(V.rms_norm(h), O.layer_norm(h), atol=1e-3)   # not the LayerNorm


def test_swiglu_matches_torch():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 7, 2 * 24)) * 3
    zt = torch.from_numpy(z)
    want = (F.silu(zt[..., :24]) * zt[..., 24:]).numpy()
    np.testing.assert_allclose(V.swiglu(z), want, rtol=1e-13, atol=1e-13)


def test_rope_complex_form_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    hd, T, base = 16, 11, 10000.0
    x = rng.standard_normal((2, 3, T, hd))
    pos = np.arange(T)
    got = V.apply_rope(x, pos, base)
    # complex form: z_i = x[2i] + j x[2i+1] times exp(j p base^(-2i/hd))
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([base ** (-2.0 * i / hd) for i in range(hd // 2)])
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    want = np.empty_like(x)
    want[..., 0::2], want[..., 1::2] = zr.real, zr.imag
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[..., 0, :], x[..., 0, :], rtol=0, atol=0)          # position 0
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    # first pair turns by exactly p radians, the last by p * base^(-(hd-2)/hd)
    a = V.rope_angles(pos, hd, base)
    np.testing.assert_allclose(a[:, 0], pos, rtol=0, atol=0)
    np.testing.assert_allclose(a[:, -1], pos * base ** (-(hd - 2) / hd), rtol=1e-15)
    # q(m) . k(n) after rotation depends on m - n only
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    def score(m, n):
        return float(V.apply_rope(q[None], np.array([m]), base)[0] @ V.apply_rope(k[None], np.array([n]), base)[0])
    for m, n, s in ((3, 1, 7), (0, 5, 12), (9, 9, 100)):
        assert abs(score(m, n) - score(m + s, n + s)) < 1e-10
    assert abs(score(3, 1) - score(1, 3)) > 1e-3


def test_cross_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((2, 4, 9, 16)), rng.standard_normal((2, 4, 13, 16)), rng.standard_normal((2, 4, 13, 16))
    got = O.masked_attention(q, k, v, np.ones((2, 13), bool))
    want = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_all_variants_off_is_the_plain_estimator():
    for name in ("tiny_f32", "locdit_tail"):
        s = synth.workload(name)
        if name == "locdit_tail":
            s = s.replace(n_layers=1, d_model=64, n_heads=4, ffn_dim=128, n_requests=2)
        W = {k: v.astype(np.float64) for k, v in synth.make_weights(s, 5).items()}
        I = synth.make_inputs(s, 6)
        x = np.stack([I["x0"][0]] * 2).astype(np.float64)
        c = np.stack([np.zeros_like(I["cond"][0]), I["cond"][0]]).astype(np.float64)
        fv = np.ones((2, s.n_frames), bool)
        fv[0, -3:] = False
        a = V.estimator(W, s, x, c, None, 0.3, fv)
        b = O.estimator(W, s, x, c, None, 0.3, fv)
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def _torch_twin(W, s, x_rows, ctx_rows, t, frame_valid):
    """Independent twin of the variant estimator in torch (float64) for small cases."""
    T_ = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    W = {k: T_(v) for k, v in W.items()}
    x, ctx, fv = T_(x_rows), T_(ctx_rows), torch.from_numpy(frame_valid)
    B, Tx, _ = x.shape
    d, H = s.d_model, s.n_heads
    hd = d // H
    half = s.t_freq_dim // 2
    freqs = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
    arg = 1000.0 * t * freqs
    e = torch.cat([torch.cos(arg), torch.sin(arg)])
    c = F.linear(F.silu(F.linear(e, W["t_embed.fc1.weight"], W["t_embed.fc1.bias"])),
                 W["t_embed.fc2.weight"], W["t_embed.fc2.bias"])
    sc = F.silu(c).expand(B, 1, d)
    nrm = (lambda h: F.rms_norm(h, (d,), eps=1e-6)) if s.norm == "rms" else (lambda h: F.layer_norm(h, (d,), eps=1e-6))
    h = F.linear(x, W["in_proj.weight"], W["in_proj.bias"])
    # RoPE through torch's complex numbers
    theta = s.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(Tx, hd // 2, dtype=torch.float64), torch.arange(Tx, dtype=torch.float64)[:, None] * theta)
    def rope(z):    # z [B, H, T, hd]
        zc = torch.view_as_complex(z.reshape(*z.shape[:-1], hd // 2, 2).contiguous())
        return torch.view_as_real(zc * rot).reshape(z.shape)
    split = lambda z: z.view(B, -1, H, hd).transpose(1, 2)
    merge = lambda z: z.transpose(1, 2).reshape(B, -1, d)
    kmask = fv[:, None, None, :]
    for l in range(s.n_layers):
        p = f"blocks.{l}."
        m = F.linear(sc, W[p + "ada.weight"], W[p + "ada.bias"]).chunk(6, dim=-1)
        u = nrm(h) * (1 + m[1]) + m[0]
        q, k, v = F.linear(u, W[p + "qkv.weight"], W[p + "qkv.bias"]).chunk(3, dim=-1)
        q, k, v = split(q), split(k), split(v)
        if s.rope:
            q, k = rope(q), rope(k)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=kmask)
        h = h + m[2] * F.linear(merge(o), W[p + "proj.weight"], W[p + "proj.bias"])
        kx, vx = F.linear(ctx, W[p + "xattn.kv.weight"], W[p + "xattn.kv.bias"]).chunk(2, dim=-1)
        qx = F.linear(nrm(h), W[p + "xattn.q.weight"], W[p + "xattn.q.bias"])
        ox = F.scaled_dot_product_attention(split(qx), split(kx), split(vx))
        h = h + F.linear(merge(ox), W[p + "xattn.out.weight"], W[p + "xattn.out.bias"])
        u = nrm(h) * (1 + m[4]) + m[3]
        g, up = F.linear(u, W[p + "fc1.weight"], W[p + "fc1.bias"]).chunk(2, dim=-1)
        h = h + m[5] * F.linear(F.silu(g) * up, W[p + "fc2.weight"], W[p + "fc2.bias"])
    mf = F.linear(sc, W["final.ada.weight"], W["final.ada.bias"]).chunk(2, dim=-1)
    vel = F.linear(nrm(h) * (1 + mf[1]) + mf[0], W["final.out.weight"], W["final.out.bias"])
    return torch.where(fv[:, :, None], vel, torch.zeros_like(vel)).numpy()


def test_variant_estimator_matches_independent_torch_twin():
    s = _tiny()
    W = {k: v.astype(np.float64) * 8 for k, v in synth.make_weights(s, 11).items()}   # larger weights: every term shows
    I = synth.make_inputs(s, 12)
    x = np.stack([I["x0"][0], I["x0"][1]]).astype(np.float64)
    ctx = np.stack([I["cond"][0], np.zeros_like(I["cond"][1])]).astype(np.float64)
    fv = np.ones((2, s.n_frames), bool)
    fv[1, 17:] = False
    got = V.estimator(W, s, x, ctx, None, 0.37, fv)
    want = _torch_twin(W, s, x, ctx, 0.37, fv)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
    # each variant matters: switching one off changes the result
    for off in (dict(norm="layer"), dict(rope=False)):
        assert np.abs(V.estimator(W, s.replace(**off), x, ctx, None, 0.37, fv) - got).max() > 1e-4


def test_rope_positions_are_row_local_and_masked_frames_do_not_leak():
    """Padded frames are keys nobody attends to: poisoning them changes no valid
    output; a request's result does not depend on the other requests."""
    s = _tiny(n_requests=2)
    W = synth.make_weights(s, 21)
    I = synth.make_inputs(s, 22)
    mask = np.ones((2, s.n_frames), np.uint8)
    mask[0, 15:] = 0
    a = V.sample(W, s, I["x0"], I["cond"], None, mask, 2, s.guidance)
    x0 = I["x0"].copy()
    x0[0, 15:] = 1e3
    b = V.sample(W, s, x0, I["cond"], None, mask, 2, s.guidance)
    np.testing.assert_allclose(a[0, :15], b[0, :15], rtol=1e-12, atol=1e-12)
    one = V.sample(W, s, I["x0"][1:], I["cond"][1:], None, mask[1:], 2, s.guidance)
    np.testing.assert_allclose(one[0], a[1], rtol=1e-12, atol=1e-12)


def test_cross_context_all_zero_for_the_unconditional_branch_only():
    """Guidance scale 1 gives the conditional branch's velocity alone: the sampler
    with s = 1 equals a one-branch run on the context; s = 0 one on a zero context."""
    s = _tiny(n_requests=1)
    W = synth.make_weights(s, 31)
    I = synth.make_inputs(s, 32)
    s1 = s.replace(n_branches=1, guidance=())
    full1 = V.sample(W, s, I["x0"], I["cond"], None, None, 3, (1.0,))
    cond_only = V.sample(W, s1, I["x0"], I["cond"], None, None, 3, ())
    np.testing.assert_allclose(full1, cond_only, rtol=1e-12, atol=1e-12)
    full0 = V.sample(W, s, I["x0"], I["cond"], None, None, 3, (0.0,))
    zero = V.sample(W, s1, I["x0"], np.zeros_like(I["cond"]), None, None, 3, ())
    np.testing.assert_allclose(full0, zero, rtol=1e-12, atol=1e-12)
    assert np.abs(full1 - full0).max() > 1e-4
