"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle (``oracle.sampler``) against one of:
  * a closed form (Euler on an analytic velocity field; left-endpoint grid);
  * the special cases of the guidance equation (scale 1 = conditional branch,
    scale 0 = unconditional branch, and the three-branch reductions);
  * an independent brute-force implementation in scalar Python loops
    (``oracle.brute``), component by component and end to end;
  * a library routine (torch CPU float64: scaled_dot_product_attention,
    layer_norm, gelu; math.erf);
  * invariants that the batching and masking rules of the pages imply
    (VoiceHub "Diffusion and flow TTS optimization", table "Semantic-preserving
    and approximate changes": packed CFG equals separate calls, padded frames
    fully masked and trimmed; empty shapes valid).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import brute as B
from oracle import sampler as O


def _rng(seed=0):
    return np.random.default_rng(seed)


def tiny_variant(**kw):
    base = synth.workload("tiny_f32")
    return base.replace(**kw)


# ------------------------------------------------------------ Euler + grid

@pytest.mark.parametrize("n_steps", [1, 3, 4, 7, 32])
@pytest.mark.parametrize("nb,scales", [(1, ()), (2, (2.0,)), (2, (-0.7,)), (3, (3.0, 1.5)), (3, (0.3, -2.0))])
def test_euler_reaches_x1_on_analytic_field(n_steps, nb, scales):
    rng = _rng(n_steps * 10 + nb)
    x0 = rng.standard_normal((17, 5))
    x1 = rng.standard_normal((17, 5))
    field = lambda t, x: np.stack([x1 - x0] * nb)
    x = O.euler_cfg(x0, n_steps, field, scales)
    np.testing.assert_allclose(x, x1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_steps", [1, 2, 5, 16])
def test_euler_evaluates_left_endpoint(n_steps):
    # v(t) = 2 t (x1 - x0): explicit Euler at t_k gives sum_k (1/S) 2 k/S = (S-1)/S.
    rng = _rng(n_steps)
    x0 = rng.standard_normal((4, 3))
    x1 = rng.standard_normal((4, 3))
    x = O.euler_cfg(x0, n_steps, lambda t, x: np.stack([2.0 * t * (x1 - x0)] * 2), (1.7,))
    np.testing.assert_allclose(x, x0 + (n_steps - 1) / n_steps * (x1 - x0), atol=1e-12)


def test_zero_steps_returns_x0():
    x0 = _rng(1).standard_normal((3, 2))
    np.testing.assert_array_equal(O.euler_cfg(x0, 0, None, (2.0,)), x0)


def test_grid_endpoints_and_monotone():
    for S in (1, 4, 10, 32, 40):
        t = O.timestep_grid(S)
        assert t[0] == 0.0 and t[-1] == 1.0
        assert np.all(np.diff(t) > 0)


# ------------------------------------------------------------ guidance

def test_guidance_combine_special_cases():
    rng = _rng(3)
    vu, vc, vt, vts = rng.standard_normal((4, 6, 5))
    np.testing.assert_allclose(O.guidance_combine(np.stack([vu, vc]), (1.0,)), vc, atol=1e-15)
    np.testing.assert_array_equal(O.guidance_combine(np.stack([vu, vc]), (0.0,)), vu)
    three = np.stack([vu, vt, vts])
    np.testing.assert_allclose(O.guidance_combine(three, (1.0, 1.0)), vts, atol=1e-15)
    np.testing.assert_allclose(O.guidance_combine(three, (1.0, 0.0)), vt, atol=1e-15)
    np.testing.assert_array_equal(O.guidance_combine(three, (0.0, 0.0)), vu)
    np.testing.assert_allclose(O.guidance_combine(three, (2.5, 2.5)),
                               O.guidance_combine(np.stack([vu, vts]), (2.5,)), atol=1e-14)


def _sample(shape, W, I, scales, kinds=None, mask=None):
    return O.sample(W, shape, I["x0"], I["cond"], I["spk"], I["mask"] if mask is None else mask,
                    shape.n_steps, scales, kinds=kinds)


def test_scale_one_is_conditional_branch_and_zero_is_unconditional():
    s = synth.workload("tiny_f32")
    W, I = synth.make_weights(s), synth.make_inputs(s)
    np.testing.assert_allclose(_sample(s, W, I, (1.0,)), _sample(s, W, I, (), kinds=("cond",)),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(_sample(s, W, I, (0.0,)), _sample(s, W, I, (), kinds=("uncond",)),
                               rtol=0, atol=1e-12)
    # and guidance actually matters at s = 2
    assert np.abs(_sample(s, W, I, (2.0,)) - _sample(s, W, I, (1.0,))).max() > 1e-3


def mini_three_branch():
    return synth.workload("multicond_rf").replace(
        n_layers=1, d_model=32, n_heads=2, ffn_dim=64, n_requests=2, n_frames=6,
        latent_dim=4, cond_dim=8, spk_dim=5, t_freq_dim=16, n_steps=2, dtype="f32")


def test_three_branch_reductions():
    s = mini_three_branch()
    W, I = synth.make_weights(s, 11), synth.make_inputs(s, 12)
    ref = lambda kinds: _sample(s, W, I, (), kinds=kinds)
    np.testing.assert_allclose(_sample(s, W, I, (1.0, 1.0)), ref(("cond_spk",)), atol=1e-12)
    np.testing.assert_allclose(_sample(s, W, I, (1.0, 0.0)), ref(("cond",)), atol=1e-12)
    np.testing.assert_allclose(_sample(s, W, I, (0.0, 0.0)), ref(("uncond",)), atol=1e-12)
    np.testing.assert_allclose(_sample(s, W, I, (1.8, 1.8)),
                               _sample(s, W, I, (1.8,), kinds=("uncond", "cond_spk")), atol=1e-12)


# ------------------------------------------------------------ components vs brute force / library

def test_attention_matches_brute_force_and_torch_sdpa():
    rng = _rng(5)
    T, H, hd = 9, 3, 4
    d = H * hd
    q, k, v = (rng.standard_normal((T, d)) * 2.0 for _ in range(3))
    masks = [np.ones(T, bool), np.array([1, 0, 1, 1, 0, 0, 1, 1, 0], bool),
             np.eye(T, dtype=bool)[4], np.zeros(T, bool)]
    for valid in masks:
        got = O.masked_attention(q.reshape(1, T, H, hd).transpose(0, 2, 1, 3),
                                 k.reshape(1, T, H, hd).transpose(0, 2, 1, 3),
                                 v.reshape(1, T, H, hd).transpose(0, 2, 1, 3),
                                 valid[None])[0].transpose(1, 0, 2).reshape(T, d)
        want = np.array(B.bf_attention(q.tolist(), k.tolist(), v.tolist(), list(valid), H))
        np.testing.assert_allclose(got, want, atol=1e-12)
        if valid.any():
            tq = torch.from_numpy(q.reshape(T, H, hd).transpose(1, 0, 2).copy())
            tk = torch.from_numpy(k.reshape(T, H, hd).transpose(1, 0, 2).copy())
            tv = torch.from_numpy(v.reshape(T, H, hd).transpose(1, 0, 2).copy())
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=torch.from_numpy(valid)[None, None, :].expand(H, T, T))
            np.testing.assert_allclose(got, ref.numpy().transpose(1, 0, 2).reshape(T, d), atol=1e-12)
        else:
            assert np.all(got == 0.0)


def test_attention_special_cases():
    rng = _rng(6)
    T, hd = 7, 5
    v = rng.standard_normal((1, 1, T, hd))
    valid = np.array([[1, 1, 0, 1, 0, 1, 1]], bool)
    # equal scores (zero queries) -> mean of the valid values
    q = np.zeros((1, 1, T, hd))
    k = rng.standard_normal((1, 1, T, hd))
    o = O.masked_attention(q, k, v, valid)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0][valid[0]].mean(0), (T, hd)), atol=1e-14)
    # one valid key -> exactly that value row
    one = np.zeros((1, T), bool)
    one[0, 3] = True
    o = O.masked_attention(rng.standard_normal((1, 1, T, hd)), k, v, one)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 3], (T, hd)), atol=1e-14)


def test_layer_norm_and_modulation():
    rng = _rng(7)
    h = rng.standard_normal((6, 33)) * 3 + 1.5
    ref = torch.nn.functional.layer_norm(torch.from_numpy(h), (33,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(h), ref, atol=1e-12)
    for i in range(6):
        np.testing.assert_allclose(O.layer_norm(h)[i], B.bf_layer_norm_row(h[i].tolist()), atol=1e-12)
    # output moments: mean 0 and variance var/(var + eps)
    u = O.layer_norm(h)
    var = h.var(axis=-1)
    np.testing.assert_allclose(u.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose(u.var(-1), var / (var + 1e-6), atol=1e-12)
    # constant row: LN gives 0, so the modulated output is the shift
    shift, scale = rng.standard_normal(33), rng.standard_normal(33)
    np.testing.assert_allclose(O.modulate(O.layer_norm(np.full((1, 33), 4.25)), shift, scale)[0], shift, atol=1e-12)


def test_gelu_and_silu():
    z = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(O.gelu(z), [B.bf_gelu(float(a)) for a in z], atol=1e-15)
    np.testing.assert_allclose(O.gelu(z), torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy(), atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), atol=1e-15)


def test_timestep_embedding():
    e0 = O.timestep_embedding(0.0, 256)
    np.testing.assert_array_equal(e0[:128], 1.0)
    np.testing.assert_array_equal(e0[128:], 0.0)
    for t in (0.25, 0.5, 0.975):
        np.testing.assert_allclose(O.timestep_embedding(t, 256), B.bf_timestep_embedding(t, 256), atol=1e-9)
        # first frequency is 1: cos(1000 t), sin(1000 t)
        e = O.timestep_embedding(t, 256)
        assert abs(e[0] - math.cos(1000 * t)) < 1e-12 and abs(e[128] - math.sin(1000 * t)) < 1e-12


def test_linear_matches_triple_loop():
    rng = _rng(8)
    x, w, b = rng.standard_normal((5, 7)), rng.standard_normal((3, 7)), rng.standard_normal(3)
    np.testing.assert_allclose(O.linear(x, w, b), B.bf_linear(x.tolist(), w.tolist(), b.tolist()), atol=1e-13)


# ------------------------------------------------------------ whole sampler vs brute force

def _brute_vs_oracle(s, wseed, iseed, mask=None, scales=None):
    W, I = synth.make_weights(s, wseed), synth.make_inputs(s, iseed)
    scales = s.guidance if scales is None else scales
    m = I["mask"] if mask is None else mask
    o1 = O.sample(W, s, I["x0"], I["cond"], I["spk"], m, s.n_steps, scales)
    o2 = np.array(B.bf_sample(W, s, I["x0"], I["cond"], I["spk"], m, s.n_steps, scales))
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    return o1, I


def test_brute_force_end_to_end_tiny_workload():
    s = synth.workload("tiny_f32")
    out, I = _brute_vs_oracle(s, None, None)
    assert np.abs(out - I["x0"]).max() > 0.05        # the estimator actually moves x


def test_brute_force_end_to_end_three_branch_masked():
    s = mini_three_branch()
    mask = np.ones((2, 6), np.uint8)
    mask[1, 4:] = 0
    _brute_vs_oracle(s, 21, 22, mask=mask)


def test_brute_force_end_to_end_prefix_mode():
    s = synth.workload("locdit_tail").replace(
        n_layers=2, d_model=32, n_heads=4, ffn_dim=64, n_requests=2, latent_dim=8,
        cond_dim=8, t_freq_dim=16, n_steps=3, dtype="f32")
    mask = np.array([[1, 1, 1, 1], [1, 0, 1, 0]], np.uint8)
    _brute_vs_oracle(s, 31, 32, mask=mask)


# ------------------------------------------------------------ batch-structure invariants

def small_channel(**kw):
    base = dict(n_layers=2, d_model=32, n_heads=4, ffn_dim=64, n_requests=4, n_frames=10,
                latent_dim=6, cond_dim=5, t_freq_dim=16, n_steps=3, dtype="f32")
    base.update(kw)
    return synth.workload("mel_dit").replace(**base)


def test_request_permutation_permutes_outputs():
    s = small_channel()
    W, I = synth.make_weights(s, 41), synth.make_inputs(s, 42)
    out = _sample(s, W, I, s.guidance)
    perm = np.array([2, 0, 3, 1])
    Ip = {k: (None if v is None else v[perm]) for k, v in I.items()}
    np.testing.assert_array_equal(_sample(s, W, Ip, s.guidance), out[perm])


def test_packed_branches_equal_separate_calls():
    s = small_channel(n_requests=1)
    W, I = synth.make_weights(s, 43), synth.make_inputs(s, 44)
    W64 = {k: v.astype(np.float64) for k, v in W.items()}
    x = I["x0"][0].astype(np.float64)
    c = I["cond"][0].astype(np.float64)
    valid = np.ones((1, s.n_frames), bool)
    rows = np.stack([np.zeros_like(c), c])
    packed = O.estimator(W64, s, np.stack([x, x]), rows, None, 0.375, np.repeat(valid, 2, 0))
    for b in range(2):
        one = O.estimator(W64, s, x[None], rows[b:b + 1], None, 0.375, valid)
        np.testing.assert_allclose(packed[b], one[0], atol=1e-12)


def test_padding_is_fully_masked_and_trimmed():
    s = small_channel(n_requests=1, n_frames=13)
    W, I = synth.make_weights(s, 45), synth.make_inputs(s, 46)
    n = 8
    mask = np.zeros((1, 13), np.uint8)
    mask[0, :n] = 1
    padded = O.sample(W, s, I["x0"], I["cond"], None, mask, s.n_steps, s.guidance)
    s_short = s.replace(n_frames=n)
    short = O.sample(W, s_short, I["x0"][:, :n], I["cond"][:, :n], None, None, s.n_steps, s.guidance)
    np.testing.assert_allclose(padded[:, :n], short, atol=1e-12)
    np.testing.assert_array_equal(padded[:, n:], I["x0"][:, n:])


def test_frame_permutation_equivariance():
    # no positional encoding: permuting frames (x, cond and mask together) permutes the output
    s = small_channel(n_requests=2)
    W, I = synth.make_weights(s, 47), synth.make_inputs(s, 48)
    mask = np.ones((2, 10), np.uint8)
    mask[1, [2, 7]] = 0
    out = O.sample(W, s, I["x0"], I["cond"], None, mask, s.n_steps, s.guidance)
    perm = _rng(9).permutation(10)
    outp = O.sample(W, s, I["x0"][:, perm], I["cond"][:, perm], None, mask[:, perm], s.n_steps, s.guidance)
    np.testing.assert_allclose(outp, out[:, perm], atol=1e-12)


def test_request_without_valid_frames_returns_x0():
    s = small_channel(n_requests=2)
    W, I = synth.make_weights(s, 49), synth.make_inputs(s, 50)
    mask = np.ones((2, 10), np.uint8)
    mask[0] = 0
    out = O.sample(W, s, I["x0"], I["cond"], None, mask, s.n_steps, s.guidance)
    assert np.all(np.isfinite(out))
    np.testing.assert_array_equal(out[0], I["x0"][0])
    assert np.abs(out[1] - I["x0"][1]).max() > 1e-3


def test_zero_requests_is_empty():
    s = small_channel(n_requests=0)
    W, I = synth.make_weights(s, 51), synth.make_inputs(s, 52)
    out = O.sample(W, s, I["x0"], I["cond"], None, None, s.n_steps, s.guidance)
    assert out.shape == (0, 10, 6)


def test_request_subset_and_worker_pool_match_full_run():
    s = small_channel(n_requests=3)
    W, I = synth.make_weights(s, 53), synth.make_inputs(s, 54)
    full = _sample(s, W, I, s.guidance)
    sub = O.sample(W, s, I["x0"], I["cond"], None, None, s.n_steps, s.guidance, requests=[2, 0])
    np.testing.assert_array_equal(sub, full[[2, 0]])
    pooled = O.sample(W, s, I["x0"], I["cond"], None, None, s.n_steps, s.guidance, workers=2)
    np.testing.assert_allclose(pooled, full, atol=1e-13)
