"""Block-residual cache (DBCache) of cfm_sample_ex on the GPU against the CPU oracle
(oracle/cache.py): VoiceHub "Diffusion and flow TTS optimization", section
"Approximate block-residual caching". The lane is the whole batch of a call.

Forcing computation at every step must give the exact sampler bit for bit. With
threshold and budget infinite the compute/hit schedule follows from the counts
alone (warm-up, consecutive-hit limit), so both sides take the same decisions and
the outputs are compared at the sampler's tolerance (relative L2 2e-2 bf16, 1e-4
fp32, on out and on the displacement). A threshold-driven case picks its threshold
from the oracle's own scores with a 2% margin on every score compared with it.
"""
import numpy as np
import pytest

import synth
from oracle import cache as K
from tests.helpers import TOL, config_for, dev, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


def _run(s, W, I, cache=None, sampler=None):
    import flow_matching_tts_amd as F
    if sampler is None:
        sampler = F.Sampler(config_for(s), W)
    hits = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    out = sampler.sample(dev(I["x0"]), dev(I["cond"]), mask=dev(I["mask"]), spk=dev(I["spk"]),
                         n_steps=s.n_steps, guidance=s.guidance, cache=cache, cache_hits=hits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(hits.cpu()[0]), sampler


def _oracle(s, W, I, **pol):
    return K.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance, K.CachePolicy(**pol))


def _valid(I, s):
    return np.ones((s.n_requests, s.n_frames), bool) if I["mask"] is None else I["mask"].astype(bool)


def _check(s, I, got, want):
    valid = _valid(I, s)
    err = rel_l2(got, want, valid)
    disp = rel_l2(got - I["x0"], want - I["x0"], valid)
    print(f"rel-L2 {err:.3e} (displacement {disp:.3e})")
    assert err <= TOL[s.dtype] and disp <= TOL[s.dtype], (err, disp)
    np.testing.assert_array_equal(got[~valid], I["x0"][~valid])


def _check_effect(s, W, I, got, want, smp):
    """The cache's own change to the result, (cached - exact), must be what the oracle's
    cache changes: otherwise a cache that never skipped (or skipped wrongly) could
    pass, its effect being below the sampler's tolerance."""
    import oracle.sampler as O
    plain, _, _ = _run(s, W, I, sampler=smp)
    exact = O.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], s.n_steps, s.guidance)
    valid = _valid(I, s)
    eff_o = (want - exact)[valid]
    eff_g = (got - plain)[valid]
    rel = np.linalg.norm(eff_g - eff_o) / np.linalg.norm(eff_o)
    print(f"cache effect {np.linalg.norm(eff_o) / np.linalg.norm(exact[valid]):.3e} of |out|, "
          f"reproduced to {rel:.3e}")
    assert np.linalg.norm(eff_o) > 10 * 1e-6 * np.linalg.norm(exact[valid])
    assert rel <= 0.25, rel


def _mel(**kw):
    return synth.workload("mel_dit").replace(n_layers=4, n_frames=300, n_requests=2, n_steps=8).replace(**kw)


COUNT_ONLY = dict(threshold=float("inf"), budget=float("inf"), warmup=2, max_consecutive=2)


def test_forced_computation_and_zero_threshold_equal_the_plain_sampler():
    s = _mel()
    W, I = synth.make_weights(s, 601), synth.make_inputs(s, 602)
    plain, h0, smp = _run(s, W, I)
    assert h0 == 0
    forced, h1, _ = _run(s, W, I, cache=dict(threshold=float("inf"), force=(True,) * s.n_steps), sampler=smp)
    np.testing.assert_array_equal(forced, plain)
    zero, h2, _ = _run(s, W, I, cache=dict(threshold=0.0, warmup=1), sampler=smp)
    np.testing.assert_array_equal(zero, plain)
    assert h1 == 0 and h2 == 0


@pytest.mark.parametrize("front,back", [(1, 1), (2, 1), (1, 0)])
def test_count_driven_schedule_matches_oracle(front, back):
    s = _mel()
    W, I = synth.make_weights(s, 611), synth.make_inputs(s, 612)
    pol = dict(COUNT_ONLY, front=front, back=back)
    got, hits, smp = _run(s, W, I, cache=pol)
    want, log = _oracle(s, W, I, **pol)
    assert hits == sum(not e["compute"] for e in log) == 4       # C C H H C H H C
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_threshold_driven_decisions_match_oracle():
    s = _mel(n_steps=10)
    W, I = synth.make_weights(s, 621), synth.make_inputs(s, 622)
    base = dict(warmup=1, max_consecutive=3, budget=float("inf"))
    _, free = _oracle(s, W, I, threshold=float("inf"), **base)
    scores = sorted(e["score"] for e in free[1:])
    best = None
    for th in [0.5 * (a + b) for a, b in zip(scores, scores[1:])]:
        want, log = _oracle(s, W, I, threshold=th, **base)
        used = [e["score"] for e in log if np.isfinite(e["score"])]
        if all(abs(x - th) > 0.02 * th for x in used):
            hits = sum(not e["compute"] for e in log)
            if 0 < hits < s.n_steps - 1 and (best is None or hits > best[2]):
                best = (th, want, hits)
    assert best is not None, "no threshold with a 2% margin"
    th, want, nh = best
    got, hits, smp = _run(s, W, I, cache=dict(base, threshold=th))
    print(f"threshold {th:.4g}: {nh} hits")
    assert hits == nh
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_cache_on_a_packed_three_branch_speaker_batch_matches_oracle():
    s = synth.workload("multicond_rf").replace(n_layers=4, n_frames=150, n_requests=3, n_steps=7, varlen=(30, 150))
    W, I = synth.make_weights(s, 631), synth.make_inputs(s, 632)
    got, hits, smp = _run(s, W, I, cache=COUNT_ONLY)
    want, log = _oracle(s, W, I, **COUNT_ONLY)
    assert hits == sum(not e["compute"] for e in log)
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_cache_on_the_fp32_path_matches_oracle():
    s = synth.workload("tiny_f32").replace(n_layers=4, n_requests=3, n_steps=8)
    W, I = synth.make_weights(s, 641), synth.make_inputs(s, 642)
    got, hits, smp = _run(s, W, I, cache=COUNT_ONLY)
    want, log = _oracle(s, W, I, **COUNT_ONLY)
    assert hits == sum(not e["compute"] for e in log) == 4
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_cache_on_the_prefix_layout_matches_oracle():
    s = synth.workload("locdit_tail").replace(n_requests=9, n_steps=8, n_layers=4)
    W, I = synth.make_weights(s, 651), synth.make_inputs(s, 652)
    got, hits, smp = _run(s, W, I, cache=COUNT_ONLY)
    want, log = _oracle(s, W, I, **COUNT_ONLY)
    assert hits == sum(not e["compute"] for e in log)
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_cache_at_full_locdit_tail_size_matches_oracle():
    """The LocDiT decode tail in its bench configuration (64 requests x CFG, 4 layers,
    10 steps): the count-driven schedule (C C H H C H H C H H) on the full batch."""
    s = synth.workload("locdit_tail")
    W, I = synth.make_weights(s), synth.make_inputs(s)
    got, hits, smp = _run(s, W, I, cache=COUNT_ONLY)
    want, log = _oracle(s, W, I, **COUNT_ONLY)
    assert hits == sum(not e["compute"] for e in log) == 6
    _check(s, I, got, want)
    _check_effect(s, W, I, got, want, smp)


def test_cache_options_are_validated():
    import flow_matching_tts_amd as F
    s = _mel()
    W, I = synth.make_weights(s, 661), synth.make_inputs(s, 662)
    smp = F.Sampler(config_for(s), W)
    for cache, extra in ((dict(front=0), {}), (dict(threshold=-1.0), {}), (dict(max_cached=-2), {}),
                         ({}, dict(guidance_mode="interval", interval=(0.0, 0.5)))):
        with pytest.raises(F.CfmError):
            smp.sample(dev(I["x0"]), dev(I["cond"]), n_steps=s.n_steps, guidance=s.guidance, cache=cache, **extra)
