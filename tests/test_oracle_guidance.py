"""Pins of the sampler-level oracle (oracle/guidance.py) against closed forms and the
plain sampler (CPU only).

VoiceHub "Diffusion and flow TTS optimization": section "Reduce a 50-step sampler
before optimizing its kernels" (rebuilt grids keep both endpoints and strict
monotonicity; native / uniform / quadratic / trailing shapes), table "Active
families" (Euler or midpoint), section "Guidance reduction" (limited-interval and
adaptive CFG, per-request lanes). Each test states what fixes the expected value.
"""
import numpy as np
import pytest

import synth
from oracle import guidance as G
from oracle import sampler as O


# ---------------------------------------------------------------- schedules

def test_schedules_closed_forms_for_four_steps():
    np.testing.assert_array_equal(G.schedule("uniform", 4), [0, 0.25, 0.5, 0.75, 1])
    np.testing.assert_array_equal(G.schedule("quadratic", 4), [0, 1 / 16, 1 / 4, 9 / 16, 1])
    np.testing.assert_array_equal(G.schedule("trailing", 4), [0, 7 / 16, 3 / 4, 15 / 16, 1])
    # 50-step native grid to 20 steps: indices round(2.5 i), halves up
    t = G.schedule("native", 20, native_steps=50)
    idx = np.rint(t * 50).astype(int)
    np.testing.assert_array_equal(t, idx / 50.0)                # every point is a native grid point
    assert list(idx[:6]) == [0, 3, 5, 8, 10, 13] and idx[-1] == 50


@pytest.mark.parametrize("kind", ["uniform", "quadratic", "trailing", "native"])
@pytest.mark.parametrize("S", [1, 2, 7, 20])
def test_schedules_keep_endpoints_and_strict_monotonicity(kind, S):
    t = G.schedule(kind, S, native_steps=50)
    assert len(t) == S + 1 and t[0] == 0.0 and t[-1] == 1.0
    assert np.all(np.diff(t) > 0)


def test_quadratic_concentrates_near_noise_and_trailing_near_data():
    q, tr = G.schedule("quadratic", 10), G.schedule("trailing", 10)
    assert np.diff(q)[0] < np.diff(q)[-1]       # small steps near t = 0 (noise)
    assert np.diff(tr)[0] > np.diff(tr)[-1]     # small steps near t = 1 (data)
    np.testing.assert_array_equal(G.schedule("native", 12, native_steps=12), G.schedule("uniform", 12))
    with pytest.raises(ValueError):
        G.schedule("native", 30, native_steps=20)


# ---------------------------------------------------------------- solvers on analytic fields

def _fields(seed=0, shape=(5, 3)):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape), rng.standard_normal(shape)


POLICIES = [G.GuidancePolicy(), G.GuidancePolicy("interval", 0.1, 0.7),
            G.GuidancePolicy("adaptive", threshold=1.0, warmup=1, patience=1)]


@pytest.mark.parametrize("solver", ["euler", "midpoint"])
@pytest.mark.parametrize("kind", ["uniform", "quadratic", "trailing", "native"])
@pytest.mark.parametrize("policy", POLICIES)
def test_constant_field_reaches_x1_on_any_grid(solver, kind, policy):
    """v_b = x1 - x0 for every branch: the guidance weights sum to one, so every
    evaluation's velocity is x1 - x0 and the sum of the steps is x1 - x0."""
    x0, x1 = _fields()
    vel = lambda t, x, guided: np.stack([x1 - x0] * (3 if guided else 1))
    x, _ = G.solve(x0, G.schedule(kind, 7, native_steps=50), vel, (3.0, 1.5), 3, policy, solver)
    np.testing.assert_allclose(x, x1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["uniform", "quadratic", "trailing"])
def test_midpoint_is_exact_for_velocity_linear_in_t_and_euler_is_not(kind):
    """x(t) = x0 + t^2 (x1 - x0) solves dx/dt = 2 t (x1 - x0). The midpoint rule
    integrates a velocity linear in t exactly on any grid (it evaluates at t_k + dt/2);
    Euler evaluates at t_k and falls short by sum dt_k^2 (x1 - x0)."""
    x0, x1 = _fields(1)
    vel = lambda t, x, guided: np.stack([2 * t * (x1 - x0)] * (2 if guided else 1))
    grid = G.schedule(kind, 5)
    xm, _ = G.solve(x0, grid, vel, (2.0,), 2, G.GuidancePolicy(), "midpoint")
    np.testing.assert_allclose(xm, x1, rtol=0, atol=1e-12)
    xe, _ = G.solve(x0, grid, vel, (2.0,), 2, G.GuidancePolicy(), "euler")
    np.testing.assert_allclose(xe, x1 - np.sum(np.diff(grid) ** 2) * (x1 - x0), rtol=0, atol=1e-12)


def _branch_constants(seed=2):
    rng = np.random.default_rng(seed)
    x0 = rng.standard_normal((4, 6))
    a = rng.standard_normal((4, 6))        # unconditional velocity
    b = rng.standard_normal((4, 6))        # conditional velocity
    return x0, a, b


def test_limited_interval_closed_form_euler():
    """Uniform 10-step grid, interval [0.10, 0.70] (the page's example): the steps at
    t = 0.1 .. 0.7 (both ends included) are guided, t = 0, 0.8, 0.9 run the
    conditional branch alone: x = x0 + 0.7 (a + s (b - a)) + 0.3 b."""
    x0, a, b = _branch_constants()
    s = 2.0
    vel = lambda t, x, guided: np.stack([a, b]) if guided else b[None]
    pol = G.GuidancePolicy("interval", 0.10, 0.70)
    x, rec = G.solve(x0, G.schedule("uniform", 10), vel, (s,), 2, pol, "euler")
    assert [r["guided"][0] for r in rec] == [False] + [True] * 7 + [False] * 2
    np.testing.assert_allclose(x, x0 + 0.7 * (a + s * (b - a)) + 0.3 * b, rtol=0, atol=1e-12)


def test_limited_interval_closed_form_midpoint():
    """Midpoint on the same grid: the midpoint evaluations sit at t = 0.05, 0.15, ...,
    0.95, of which 0.15 .. 0.65 (6 of them) are in [0.10, 0.70]; with velocities that
    do not depend on x only the midpoint evaluation enters x."""
    x0, a, b = _branch_constants(3)
    s = 2.5
    vel = lambda t, x, guided: np.stack([a, b]) if guided else b[None]
    pol = G.GuidancePolicy("interval", 0.10, 0.70)
    x, rec = G.solve(x0, G.schedule("uniform", 10), vel, (s,), 2, pol, "midpoint")
    assert [r["guided"][1] for r in rec] == [False] + [True] * 6 + [False] * 3
    np.testing.assert_allclose(x, x0 + 0.6 * (a + s * (b - a)) + 0.4 * b, rtol=0, atol=1e-12)


def test_adaptive_warmup_reset_and_patience():
    """A designed metric sequence (v_u = b (1 + m_k) gives metric m_k exactly):
    threshold 0.1, warm-up 4, patience 2. Steps 0-3 never count; step 4 counts 1,
    step 5 resets, steps 6 and 7 reach patience, so steps 8 and 9 are unguided."""
    x0, _, b = _branch_constants(4)
    m = [0.01, 0.01, 0.01, 0.01, 0.01, 0.5, 0.01, 0.01, 0.01, 0.01]
    grid = G.schedule("uniform", 10)
    step_of = lambda t: int(round(t * 10))
    vel = lambda t, x, guided: np.stack([b * (1 + m[step_of(t)]), b]) if guided else b[None]
    s = 3.0
    pol = G.GuidancePolicy("adaptive", threshold=0.1, warmup=4, patience=2)
    x, rec = G.solve(x0, grid, vel, (s,), 2, pol, "euler")
    assert [r["guided"][0] for r in rec] == [True] * 8 + [False] * 2
    np.testing.assert_allclose([r["metric"] for r in rec[:8]], m[:8], rtol=1e-12)
    guided_v = [b * (1 + m[k]) + s * (b - b * (1 + m[k])) for k in range(8)]
    np.testing.assert_allclose(x, x0 + 0.1 * (sum(guided_v) + 2 * b), rtol=0, atol=1e-12)


def test_adaptive_extremes():
    """Threshold 0: no metric is below it, guidance never stops (= full CFG).
    Threshold infinity: every counted step is below it, so the lane stops after
    exactly warm-up + patience guided steps."""
    x0, a, b = _branch_constants(5)
    vel = lambda t, x, guided: np.stack([a, b]) if guided else b[None]
    grid = G.schedule("uniform", 12)
    full, _ = G.solve(x0, grid, vel, (2.0,), 2, G.GuidancePolicy(), "euler")
    never, rec0 = G.solve(x0, grid, vel, (2.0,), 2, G.GuidancePolicy("adaptive", threshold=0.0), "euler")
    np.testing.assert_array_equal(never, full)
    assert all(r["guided"][0] for r in rec0)
    _, rec = G.solve(x0, grid, vel, (2.0,), 2, G.GuidancePolicy("adaptive", threshold=np.inf, warmup=3,
                                                                patience=4), "euler")
    assert [r["guided"][0] for r in rec] == [True] * 7 + [False] * 5


def test_adaptive_metric_definition():
    v_full = np.array([[1.0, -2.0], [3.0, 0.5]])
    v_u = np.array([[1.5, -2.0], [0.0, 0.5]])
    valid = np.array([[True, True], [False, False]])
    assert G.adaptive_metric(v_full, v_u, valid) == pytest.approx(0.5 / 3.0, rel=1e-15)
    assert G.adaptive_metric(np.zeros((2, 2)), v_u, valid) == 0.0


# ---------------------------------------------------------------- through the estimator

def _tiny(n_requests=3, n_steps=6):
    s = synth.workload("tiny_f32").replace(n_requests=n_requests, n_steps=n_steps)
    return s, synth.make_weights(s, 11), synth.make_inputs(s, 12)


def test_full_interval_and_uniform_grid_equal_the_plain_sampler():
    """Interval [0, 1] covers every evaluation: the plain CFG sampler, bit for bit."""
    s, W, I = _tiny()
    want = O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance)
    for pol in (G.GuidancePolicy(), G.GuidancePolicy("interval", 0.0, 1.0),
                G.GuidancePolicy("adaptive", threshold=0.0)):
        got, _ = G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], G.schedule("uniform", s.n_steps),
                          s.guidance, pol)
        np.testing.assert_array_equal(got, want)


def test_empty_interval_equals_the_conditional_branch_alone():
    s, W, I = _tiny()
    want = O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, (), kinds=("cond",))
    for start, end in ((0.6, 0.5), (1.5, 2.0)):
        got, rec = G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], G.schedule("uniform", s.n_steps),
                            s.guidance, G.GuidancePolicy("interval", start, end))
        np.testing.assert_array_equal(got, want)
        assert not any(r["guided"][0] for rr in rec for r in rr)


def test_guidance_lanes_are_per_request():
    """Adaptive guidance decides per request: permuting the requests permutes the
    outputs and the decisions, and a request alone decides as it does in the batch."""
    s, W, I = _tiny(n_requests=3, n_steps=8)
    grid = G.schedule("trailing", s.n_steps)
    pol = G.GuidancePolicy("adaptive", threshold=0.5, warmup=2, patience=1)
    a, ra = G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], grid, s.guidance, pol)
    perm = [2, 0, 1]
    b, rb = G.sample(W, s, I["x0"][perm], I["cond"][perm], None, None, grid, s.guidance, pol)
    np.testing.assert_array_equal(b, a[perm])
    one, r1 = G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], grid, s.guidance, pol, requests=[1])
    np.testing.assert_array_equal(one[0], a[1])
    assert [r["guided"] for r in r1[0]] == [r["guided"] for r in ra[1]]


def test_midpoint_through_the_estimator_uses_two_evaluations_per_step():
    """A midpoint step evaluates the estimator at t_k and at t_k + dt/2; counted
    through a wrapper of the estimator."""
    s, W, I = _tiny(n_requests=1, n_steps=3)
    calls = []
    real = O.estimator

    def counting(*a, **k):
        calls.append(a[5])
        return real(*a, **k)

    O.estimator = counting
    try:
        G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], G.schedule("uniform", 3), s.guidance,
                 G.GuidancePolicy(), "midpoint")
    finally:
        O.estimator = real
    np.testing.assert_allclose(calls, [0, 1 / 6, 1 / 3, 1 / 2, 2 / 3, 5 / 6], rtol=0, atol=1e-15)
