"""Writes the guidance oracle's outputs for sampled requests of full-size workloads
run with sampler options (oracle/guidance.py):

* ``mel_dit_adaptive``: the Mel DiT workload with adaptive guidance, threshold 2.0,
  warm-up 4, patience 2. On this random-weight model the metric of every counted
  step lies well below 2.0, so every request's unconditional lane stops after
  step 6; the writer checks that margin (5%) so the device, which computes the
  metric in fp32, must take the same decisions.
* ``varlen_interval_midpoint``: the variable-length masked batch with
  limited-interval guidance on [0.10, 0.70], the trailing subsequence of 64
  native steps and the midpoint solver (two evaluations per step).

Calls only ``oracle`` and the seeded generators in ``synth``; requests never
interact, so a subset is exact. Stores every 4th frame as float32, the number
of guided evaluations per stored request, and the sha256 of oracle/guidance.py
then oracle/sampler.py. Run from the repository root:

    python tests/golden/make_option_refs.py [case ...]
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import guidance as G  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
STRIDE = 4
MARGIN = 1.05

CASES = {
    "mel_dit_adaptive": dict(workload="mel_dit", requests=[0, 7],
                             options=dict(guidance_mode="adaptive", adaptive=(2.0, 4, 2))),
    "varlen_interval_midpoint": dict(workload="varlen_masked", requests=[2, 26],
                                     options=dict(guidance_mode="interval", interval=(0.10, 0.70),
                                                  schedule="trailing", native_steps=64, solver="midpoint")),
}


def oracle_hash() -> str:
    h = hashlib.sha256()
    for f in ("guidance.py", "sampler.py"):
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def policy_of(opt) -> G.GuidancePolicy:
    mode = opt.get("guidance_mode", "full")
    if mode == "interval":
        return G.GuidancePolicy("interval", *opt["interval"])
    if mode == "adaptive":
        th, wu, pa = opt["adaptive"]
        return G.GuidancePolicy("adaptive", threshold=th, warmup=wu, patience=pa)
    return G.GuidancePolicy()


def make(case: str) -> str:
    c = CASES[case]
    s = synth.workload(c["workload"])
    opt = c["options"]
    W, I = synth.make_weights(s), synth.make_inputs(s)
    grid = G.schedule(opt.get("schedule", "uniform"), s.n_steps, opt.get("native_steps"))
    policy = policy_of(opt)
    t0 = time.time()
    out, records = G.sample(W, s, I["x0"], I["cond"], I["spk"], I["mask"], grid, s.guidance, policy,
                            opt.get("solver", "euler"), requests=c["requests"], workers=len(c["requests"]))
    guided = np.array([sum(sum(1 for g in rec["guided"] if g) for rec in recs) for recs in records])
    if policy.mode == "adaptive":   # decisions far from the threshold on every counted step
        for recs in records:
            for k, rec in enumerate(recs):
                if k >= policy.warmup and rec["metric"] is not None:
                    m = rec["metric"]
                    assert m * MARGIN < policy.threshold or m > policy.threshold * MARGIN, (k, m)
    frames = np.arange(0, s.n_frames, STRIDE)
    path = os.path.join(HERE, f"options_{case}.npz")
    np.savez_compressed(path, out=out[:, frames, :].astype(np.float32), requests=np.array(c["requests"]),
                        frames=frames, guided=guided, oracle_sha256=np.array(oracle_hash()))
    print(f"{case}: requests {c['requests']}, guided evaluations {guided.tolist()}, "
          f"{time.time() - t0:.1f} s -> {path}", flush=True)
    return path


if __name__ == "__main__":
    for n in sys.argv[1:] or list(CASES):
        make(n)
