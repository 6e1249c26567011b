"""Sampler-level options of cfm_sample_ex on the GPU against the CPU oracle
(oracle/guidance.py): reconstructed schedules, the midpoint solver, limited-interval
and adaptive guidance (VoiceHub "Diffusion and flow TTS optimization", sections
"Reduce a 50-step sampler before optimizing its kernels" and "Guidance
reduction"; table "Active families"). Same tolerances as the plain sampler:
relative L2 after all steps 1e-4 (fp32 path), 2e-2 (bf16 path), on out and on the
displacement out - x0.

Adaptive guidance decides with a threshold test on a metric the two sides compute
in different precisions (fp64 oracle, fp32 reductions of the bf16 path's
velocities). The tests pick thresholds from the oracle's own metrics with a
margin of 2% on every step that counts, so that both sides must take the same
decisions; the per-request number of guided evaluations is then compared exactly.
Some requests get a weakened condition (their branches then nearly agree), so
that lanes stop at different steps: each request decides on its own.

At full size (the bench configuration of the Mel DiT and variable-length
workloads) sampled requests are compared with stored oracle outputs written by
tests/golden/make_option_refs.py: adaptive guidance on the Mel DiT (every lane
stops after step 6, with the metric at least 5% from the threshold on every
counted step) and limited-interval guidance with the trailing schedule and the
midpoint solver on the packed variable-length batch.
"""
import hashlib
import os

import numpy as np
import pytest

import synth
from oracle import guidance as G
from tests.helpers import TOL, config_for, dev, rel_l2

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flow_matching_tts_amd as F
    F.load()


def _run(s, W, I, sampler=None, **opt):
    import flow_matching_tts_amd as F
    if sampler is None:
        per = 2 if opt.get("solver") == "midpoint" else 1
        sampler = F.Sampler(config_for(s, max_steps=per * s.n_steps), W)
    ge = torch.zeros(s.n_requests, dtype=torch.int32, device="cuda")
    out = sampler.sample(dev(I["x0"]), dev(I["cond"]), mask=dev(I["mask"]), spk=dev(I["spk"]),
                         n_steps=s.n_steps, guidance=s.guidance, guided_evals=ge, **opt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ge.cpu().numpy(), sampler


def _policy(opt):
    mode = opt.get("guidance_mode", "full")
    if mode == "interval":
        return G.GuidancePolicy("interval", *opt["interval"])
    if mode == "adaptive":
        th, wu, pa = opt["adaptive"]
        return G.GuidancePolicy("adaptive", threshold=th, warmup=wu, patience=pa)
    return G.GuidancePolicy()


def _oracle(s, W, I, requests=None, **opt):
    grid = G.schedule(opt.get("schedule", "uniform"), s.n_steps, opt.get("native_steps"))
    return G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], grid, s.guidance, _policy(opt),
                    opt.get("solver", "euler"), requests=requests, workers=min(4, s.n_requests))


def _guided_counts(records):
    return np.array([sum(sum(1 for g in r["guided"] if g) for r in rec) for rec in records])


def _valid(I, s):
    return np.ones((s.n_requests, s.n_frames), bool) if I["mask"] is None else I["mask"].astype(bool)


def _check(s, I, got, want, reqs=None):
    reqs = list(range(s.n_requests)) if reqs is None else reqs
    valid = _valid(I, s)[reqs]
    err = rel_l2(got[reqs], want, valid)
    disp = rel_l2(got[reqs] - I["x0"][reqs], want - I["x0"][reqs], valid)
    print(f"rel-L2 {err:.3e} (displacement {disp:.3e})")
    assert err <= TOL[s.dtype] and disp <= TOL[s.dtype], (err, disp)
    np.testing.assert_array_equal(got[~_valid(I, s)], I["x0"][~_valid(I, s)])


def _mel(**kw):
    s = synth.workload("mel_dit").replace(n_layers=2, n_frames=300, n_requests=2, n_steps=6)
    return s.replace(**kw)


@pytest.mark.parametrize("opt", [
    dict(schedule="quadratic"),
    dict(schedule="trailing", solver="midpoint"),
    dict(schedule="native", native_steps=16),
    dict(solver="midpoint"),
])
def test_schedules_and_midpoint_match_oracle(opt):
    s = _mel(n_steps=5)
    W, I = synth.make_weights(s, 501), synth.make_inputs(s, 502)
    got, ge, _ = _run(s, W, I, **opt)
    want, rec = _oracle(s, W, I, **opt)
    _check(s, I, got, want)
    np.testing.assert_array_equal(ge, _guided_counts(rec))


def test_limited_interval_matches_oracle():
    """Uniform 6-step grid, interval [0.10, 0.70]: steps at t = 1/6 .. 4/6 guided,
    t = 0 and 5/6 run the conditional rows alone."""
    s = _mel()
    W, I = synth.make_weights(s, 511), synth.make_inputs(s, 512)
    opt = dict(guidance_mode="interval", interval=(0.10, 0.70))
    got, ge, _ = _run(s, W, I, **opt)
    want, rec = _oracle(s, W, I, **opt)
    assert list(_guided_counts(rec)) == [4, 4]
    np.testing.assert_array_equal(ge, [4, 4])
    _check(s, I, got, want)


def test_full_interval_is_plain_cfg_and_empty_interval_is_the_conditional_branch():
    s = _mel()
    W, I = synth.make_weights(s, 521), synth.make_inputs(s, 522)
    plain, ge0, smp = _run(s, W, I)
    full, ge1, _ = _run(s, W, I, sampler=smp, guidance_mode="interval", interval=(0.0, 1.0))
    np.testing.assert_array_equal(full, plain)
    np.testing.assert_array_equal(ge1, ge0)
    empty, ge2, _ = _run(s, W, I, sampler=smp, guidance_mode="interval", interval=(0.6, 0.5))
    cond_only, _, _ = _run(s.replace(n_branches=1, guidance=()), W, I)
    np.testing.assert_allclose(empty, cond_only, rtol=0, atol=1e-6)
    np.testing.assert_array_equal(ge2, [0, 0])


def test_interval_on_the_prefix_layout_matches_oracle():
    """The LocDiT decode tail (condition frames before the patch frames): unguided
    steps run the conditional rows alone, which then carry the condition prefix."""
    s = synth.workload("locdit_tail").replace(n_requests=9, n_steps=5, n_layers=2)
    W, I = synth.make_weights(s, 531), synth.make_inputs(s, 532)
    opt = dict(guidance_mode="interval", interval=(0.2, 0.6), schedule="trailing")
    got, ge, _ = _run(s, W, I, **opt)
    want, rec = _oracle(s, W, I, **opt)
    np.testing.assert_array_equal(ge, _guided_counts(rec))
    _check(s, I, got, want)


def _pick_threshold(s, W, I, warmup, patience, requests, opt_extra=()):
    """A threshold such that every metric the adaptive oracle run compares with it
    (steps >= warmup, lanes still on) is at least 2% away from it (the two sides'
    metrics differ by about 1e-3 relative at the bf16 path's precision), chosen
    among the full-CFG metrics so that requests stop at different steps where
    possible (per-request lanes), else so that some lane stops."""
    _, rec_full = _oracle(s, W, I, requests=requests, **dict(opt_extra))
    per_step = [sorted(r["metric"] for r in col) for col in zip(*rec_full)][warmup:]
    cands = []
    for ms in per_step:                      # between requests' metrics at one step
        cands += [0.5 * (a + b) for a, b in zip(ms, ms[1:]) if b > 1.05 * a]
    allm = sorted(m for ms in per_step for m in ms)
    cands += [0.5 * (allm[0] + allm[-1]), allm[-1] * 1.5]
    cands = sorted(set(cands))
    if len(cands) > 8:
        cands = [cands[i] for i in np.linspace(0, len(cands) - 1, 8).round().astype(int)]
    best = None
    for th in cands:
        opt = dict(opt_extra, guidance_mode="adaptive", adaptive=(th, warmup, patience))
        want, rec = _oracle(s, W, I, requests=requests, **opt)
        used = [r["metric"] for rr in rec for k, r in enumerate(rr) if k >= warmup and r["metric"] is not None]
        if all(abs(m - th) > 0.02 * th for m in used):
            counts = _guided_counts(rec)
            score = (len(set(counts.tolist())), -int(counts.min()))
            if best is None or score > best[0]:
                best = (score, th, want, counts)
    assert best is not None, "no threshold with a 2% margin"
    return best[1], best[2], best[3]


def test_adaptive_guidance_matches_oracle():
    s = _mel(n_requests=4, n_steps=8)
    W, I = synth.make_weights(s, 541), synth.make_inputs(s, 542)
    I["cond"][0] *= 0.05
    I["cond"][2] *= 0.3
    th, want, counts = _pick_threshold(s, W, I, 2, 2, None)
    print(f"threshold {th:.4g}, guided evaluations per request {list(counts)}")
    assert counts.min() < s.n_steps and len(set(counts.tolist())) > 1   # lanes stop at different steps
    got, ge, _ = _run(s, W, I, guidance_mode="adaptive", adaptive=(th, 2, 2))
    np.testing.assert_array_equal(ge, counts)
    _check(s, I, got, want)


def test_adaptive_packed_three_branch_speaker_batch_matches_oracle():
    """Masked three-branch batch with the speaker branch: stopped lanes drop their
    unconditional and text rows from the packed layout step by step."""
    s = synth.workload("multicond_rf").replace(n_layers=2, n_frames=150, n_requests=4, n_steps=7,
                                               varlen=(40, 150))
    W, I = synth.make_weights(s, 551), synth.make_inputs(s, 552)
    I["cond"][1] *= 0.05
    I["spk"][1] *= 0.05
    th, want, counts = _pick_threshold(s, W, I, 1, 2, None, (("solver", "midpoint"),))
    print(f"threshold {th:.4g}, guided evaluations per request {list(counts)}")
    assert len(set(counts.tolist())) > 1
    got, ge, _ = _run(s, W, I, guidance_mode="adaptive", adaptive=(th, 1, 2), solver="midpoint")
    np.testing.assert_array_equal(ge, counts)
    _check(s, I, got, want)


def test_adaptive_fp32_path_matches_oracle():
    s = synth.workload("tiny_f32").replace(n_requests=3, n_steps=8)
    W, I = synth.make_weights(s, 561), synth.make_inputs(s, 562)
    th, want, counts = _pick_threshold(s, W, I, 2, 1, None)
    got, ge, _ = _run(s, W, I, guidance_mode="adaptive", adaptive=(th, 2, 1))
    np.testing.assert_array_equal(ge, counts)
    _check(s, I, got, want)


def test_adaptive_extremes_on_gpu():
    """Threshold 0 never stops (the plain sampler); threshold infinity stops every
    lane after warm-up + patience steps: the interval run that guides exactly those
    steps."""
    s = _mel()
    W, I = synth.make_weights(s, 571), synth.make_inputs(s, 572)
    plain, _, smp = _run(s, W, I)
    never, ge, _ = _run(s, W, I, sampler=smp, guidance_mode="adaptive", adaptive=(0.0, 2, 2))
    np.testing.assert_array_equal(never, plain)
    np.testing.assert_array_equal(ge, [6, 6])
    always, ge, _ = _run(s, W, I, sampler=smp, guidance_mode="adaptive", adaptive=(float("inf"), 1, 2))
    np.testing.assert_array_equal(ge, [3, 3])
    first3, _, _ = _run(s, W, I, sampler=smp, guidance_mode="interval", interval=(0.0, 0.4))
    np.testing.assert_allclose(always, first3, rtol=0, atol=1e-6)


def test_options_are_validated_before_any_work():
    import flow_matching_tts_amd as F
    s = _mel()
    W, I = synth.make_weights(s, 581), synth.make_inputs(s, 582)
    smp = F.Sampler(config_for(s), W)
    x0 = dev(I["x0"])
    ref = x0.clone()
    out = torch.full_like(x0, 7.0)
    for opt, code in ((dict(solver="midpoint"), "CAPACITY"),          # 12 evaluations > max_steps 6
                      (dict(schedule="native", native_steps=3), "VALUE"),
                      (dict(guidance_mode="adaptive", adaptive=(float("nan"), 1, 1)), "VALUE"),
                      (dict(guidance_mode="adaptive", adaptive=(0.1, 1, 0)), "VALUE"),
                      (dict(guidance_mode="interval", interval=(0.0, float("inf"))), "VALUE")):
        with pytest.raises((F.CfmError, ValueError)) as e:
            smp.sample(x0, dev(I["cond"]), n_steps=s.n_steps, guidance=s.guidance, out=out, **opt)
        assert code in str(e.value) or "capacity" in str(e.value), (opt, str(e.value))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.equal(x0, ref)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FULL_CASES = {
    "mel_dit_adaptive": ("mel_dit", dict(guidance_mode="adaptive", adaptive=(2.0, 4, 2))),
    "varlen_interval_midpoint": ("varlen_masked", dict(guidance_mode="interval", interval=(0.10, 0.70),
                                                       schedule="trailing", native_steps=64, solver="midpoint")),
}


@pytest.mark.parametrize("case", list(FULL_CASES))
def test_full_size_options_match_stored_oracle(case):
    path = os.path.join(GOLDEN, f"options_{case}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    z = np.load(path)
    h = hashlib.sha256()
    for f in ("guidance.py", "sampler.py"):
        with open(os.path.join(os.path.dirname(GOLDEN), "..", "oracle", f), "rb") as fh:
            h.update(fh.read())
    assert str(z["oracle_sha256"]) == h.hexdigest(), "stale oracle reference"
    name, opt = FULL_CASES[case]
    s = synth.workload(name)
    W, I = synth.make_weights(s), synth.make_inputs(s)
    got, ge, _ = _run(s, W, I, **opt)
    reqs, frames = list(z["requests"]), z["frames"]
    np.testing.assert_array_equal(ge[reqs], z["guided"])
    valid = _valid(I, s)[reqs][:, frames]
    g = got[reqs][:, frames, :]
    x0 = I["x0"][reqs][:, frames, :]
    err = rel_l2(g, z["out"], valid)
    disp = rel_l2(g - x0, z["out"] - x0, valid)
    print(f"{case}: full size, requests {reqs}, guided {ge[reqs].tolist()}: rel-L2 {err:.3e} "
          f"(displacement {disp:.3e})")
    assert err <= TOL[s.dtype] and disp <= TOL[s.dtype], (err, disp)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got[~_valid(I, s)], I["x0"][~_valid(I, s)])
