"""Pins of the block-residual cache oracle (oracle/cache.py) on the CPU.

VoiceHub "Diffusion and flow TTS optimization", section "Approximate block-residual
caching": forcing computation at every step must give the exact sampler; the
decision rules (warm-up, consecutive-hit limit, total-hit limit, accumulated-error
budget) fix the compute/hit schedule; a hit adds the saved middle-block residual.
"""
import numpy as np
import pytest

import synth
from oracle import cache as K
from oracle import sampler as O


def _case(n_layers=4, n_requests=2, n_steps=8, name="tiny_f32", **kw):
    s = synth.workload(name).replace(n_layers=n_layers, n_requests=n_requests, n_steps=n_steps, **kw)
    return s, synth.make_weights(s, 31), synth.make_inputs(s, 32)


def _exact(s, W, I):
    return O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance)


def _cached(s, W, I, **pol):
    return K.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance, K.CachePolicy(**pol))


def test_forced_computation_at_every_step_is_the_exact_sampler():
    s, W, I = _case()
    out, log = _cached(s, W, I, threshold=np.inf, force=(True,) * s.n_steps)
    np.testing.assert_allclose(out, _exact(s, W, I), rtol=1e-12, atol=1e-12)
    assert all(e["compute"] for e in log)


def test_zero_threshold_and_zero_budget_never_hit():
    """No score is below 0, and with a zero budget any positive score exceeds it."""
    s, W, I = _case()
    want = _exact(s, W, I)
    for pol in (dict(threshold=0.0), dict(threshold=np.inf, budget=0.0)):
        out, log = _cached(s, W, I, warmup=1, **pol)
        np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
        assert all(e["compute"] for e in log)


def test_no_middle_blocks_is_the_exact_sampler():
    s, W, I = _case(n_layers=2)
    out, log = _cached(s, W, I, front=1, back=1, threshold=np.inf, warmup=0)
    np.testing.assert_allclose(out, _exact(s, W, I), rtol=1e-12, atol=1e-12)
    assert log == []


def test_schedule_with_every_score_accepted():
    """Threshold and budget infinite: the first `warmup` evaluations compute, then at
    most `max_consecutive` hits follow each computation; `max_cached` caps the hits."""
    s, W, I = _case(n_steps=11)
    _, log = _cached(s, W, I, threshold=np.inf, budget=np.inf, warmup=3, max_consecutive=2)
    assert [e["compute"] for e in log] == [True, True, True, False, False, True, False, False, True, False, False]
    _, log = _cached(s, W, I, threshold=np.inf, budget=np.inf, warmup=1, max_consecutive=3, max_cached=2)
    assert [e["compute"] for e in log] == [True, False, False] + [True] * 8
    assert np.isnan(log[0]["score"]) and all(e["score"] >= 0 for e in log[1:])


def test_budget_accumulates_accepted_scores():
    """Hits accumulate their scores; a hit that would push the sum past the budget
    computes instead (and resets the sum)."""
    s, W, I = _case(n_steps=10)
    _, free = _cached(s, W, I, threshold=np.inf, budget=np.inf, warmup=1, max_consecutive=100)
    scores = [e["score"] for e in free]
    budget = 0.5 * (scores[1] + scores[2] + scores[3])
    _, log = _cached(s, W, I, threshold=np.inf, budget=budget, warmup=1, max_consecutive=100)
    acc, expect = 0.0, []
    for j, e in enumerate(log):
        if j < 1:
            expect.append(True)
            continue
        if acc + e["score"] > budget:
            expect.append(True)
            acc = 0.0
        else:
            expect.append(False)
            acc += e["score"]
    assert [e["compute"] for e in log] == expect and not all(expect[1:]) and any(expect[1:])


def test_identity_middle_blocks_make_hits_exact():
    """With every gate of the middle blocks zero (their adaLN-Zero gate rows and
    biases zeroed) the middle blocks are identities and their residual is zero, so
    the cached sampler must equal the exact one however many hits it takes."""
    s, W, I = _case(n_layers=5, n_steps=9)
    W = dict(W)
    d = s.d_model
    for l in (1, 2, 3):
        w = W[f"blocks.{l}.ada.weight"].copy()
        b = W[f"blocks.{l}.ada.bias"].copy()
        for g in (2, 5):                         # gate1, gate2 of (shift1, scale1, gate1, shift2, scale2, gate2)
            w[g * d:(g + 1) * d] = 0.0
            b[g * d:(g + 1) * d] = 0.0
        W[f"blocks.{l}.ada.weight"], W[f"blocks.{l}.ada.bias"] = w, b
    out, log = _cached(s, W, I, threshold=np.inf, budget=np.inf, warmup=1, max_consecutive=4)
    assert sum(not e["compute"] for e in log) >= 5
    np.testing.assert_allclose(out, _exact(s, W, I), rtol=1e-12, atol=1e-12)


def test_a_hit_adds_the_last_saved_residual():
    """On the schedule C C H: the second evaluation's middle residual is the one the
    third adds. Checked by running the third evaluation's front blocks by hand."""
    s, W, I = _case(n_layers=4, n_steps=3, n_requests=1)
    out, log = _cached(s, W, I, threshold=np.inf, budget=np.inf, warmup=2, max_consecutive=5)
    assert [e["compute"] for e in log] == [True, True, False]
    # a cache whose middle blocks always compute gives the same first two steps; at the
    # third the only difference is the middle residual, so the outputs must differ
    exact = _exact(s, W, I)
    assert np.abs(out - exact).max() > 0
    assert np.abs(out - exact).max() < 0.1 * np.abs(exact - I["x0"]).max()


def test_masked_three_branch_lane():
    """Masked frames do not enter the score; the lane covers every branch row."""
    s = synth.workload("multicond_rf").replace(n_layers=4, d_model=64, n_heads=4, ffn_dim=128, latent_dim=8,
                                               cond_dim=16, spk_dim=8, n_requests=2, n_frames=12, n_steps=6,
                                               varlen=(5, 12), dtype="f32")
    W, I = synth.make_weights(s, 41), synth.make_inputs(s, 42)
    out, log = _cached(s, W, I, threshold=np.inf, force=(True,) * 6)
    np.testing.assert_allclose(out, _exact(s, W, I), rtol=1e-12, atol=1e-12)
    # poison the masked frames' inputs: the decisions and valid outputs do not change
    I2 = dict(I, x0=np.where(I["mask"][..., None] > 0, I["x0"], 1e3).astype(np.float32))
    a, la = _cached(s, W, I, threshold=0.05, warmup=1)
    b, lb = _cached(s, W, I2, threshold=0.05, warmup=1)
    assert [e["compute"] for e in la] == [e["compute"] for e in lb]
    m = I["mask"].astype(bool)
    np.testing.assert_allclose(a[m], b[m], rtol=1e-12, atol=1e-12)
